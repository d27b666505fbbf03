/*
 * specverify.h -- C ABI of libspecverify: batched verification of
 * speculative-decoding draft tokens against target logits on one AMD Instinct
 * MI355X (gfx950).
 *
 * The scheme is the one of "Accelerating Sonar through speculation"
 * (Perplexity; N. Licker, E. McKnight; 2025):
 *   - section "Speculative decoding": each prefix of the drafted tokens is
 *     scored and the longest prefix that passes acceptance is kept; n drafts
 *     yield up to n+1 tokens per step because the target's logits at the
 *     mismatch, or after the last draft, are sampled as well;
 *   - section "Target-Draft": acceptance compares the full draft and target
 *     probability distributions, and the target's extra logits row after the
 *     accepted drafts is sampled ("bonus" token);
 *   - section "EAGLE": for a tree of drafts the longest suitable root path is
 *     kept and one more target token is appended;
 *   - section "MTP": logits row i predicts token i+1, hence target row j
 *     scores draft j and row k follows the last draft;
 *   - sections "Inference with speculative decoding" and "MTP Schedule for a
 *     Single Token": the accepted lengths are what forces a device-to-host
 *     synchronisation, and a device kernel can place the next tokens without
 *     one -- so every result here stays in device memory and no call
 *     synchronises the host.
 * The acceptance rule (keep draft x with probability min(1, p(x)/q(x)); at
 * the first rejection draw from max(0, p - q) renormalised) is the
 * speculative sampling of Leviathan et al., "Fast Inference from
 * Transformers via Speculative Decoding", first in the pages' references.
 *
 * Conventions shared by every entry point
 *   - Array arguments are DEVICE pointers (hipMalloc memory, or a torch
 *     tensor's data_ptr()).  The caller owns every buffer; the library never
 *     allocates, frees, or copies between host and device.
 *   - Logit tensors are dense row-major; any alignment works, but rows that
 *     start on 16-byte boundaries (V * element size a multiple of 16 and a
 *     16-byte aligned base) take the vectorised path.
 *   - Calls are asynchronous on `stream` (NULL = the null stream) and never
 *     synchronise the host.  Outputs are valid once the stream has executed
 *     the call.
 *   - Argument errors are found on the host before any launch; the outputs are
 *     then untouched.  A failed launch returns SV_ERR_HIP.  Faults raised by
 *     a kernel surface at the caller's next synchronisation, as for any HIP
 *     call.
 *   - Not checked (preconditions): logits are finite; temperatures are
 *     finite and >= 0; uniforms lie in [0, 1); |l_v - max_w l_w| / T < 700
 *     within a row (no probability underflows to zero in double precision)
 *     and |l_v| / T < 10^6.  Draft token ids should lie in [0, V); an id
 *     outside that range is rejected (tau = 0), never used as an index.
 *   - The workspace must hold at least the number of bytes the matching
 *     sv_*_workspace_bytes() query returns and be 16-byte aligned.  It needs
 *     no initialisation.  Two calls in flight at the same time must not share
 *     one workspace.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SV_OK = 0,
    SV_ERR_INVALID_ARGUMENT = 1,    /* a null pointer, a negative size, an unknown dtype ... */
    SV_ERR_WORKSPACE_TOO_SMALL = 2, /* workspace_bytes below the matching query */
    SV_ERR_UNSUPPORTED = 3,         /* a size beyond the documented limits */
    SV_ERR_HIP = 4                  /* a HIP runtime call or kernel launch failed */
} sv_status;

typedef enum {
    SV_F32 = 0,  /* IEEE binary32 logits */
    SV_BF16 = 1  /* bfloat16 logits (upper half of a binary32) */
} sv_dtype;

/* Limits: k <= SV_MAX_DRAFTS draft tokens per sequence; N <= SV_MAX_TREE_NODES
 * tree nodes and max_depth <= 2^24 for the tree entry points; V <= SV_MAX_VOCAB.
 * Larger sizes return SV_ERR_UNSUPPORTED. */
#define SV_MAX_DRAFTS 64
#define SV_MAX_TREE_NODES 1024
#define SV_MAX_VOCAB (1 << 20)

/* Library version (major * 10000 + minor * 100 + patch). */
int sv_version(void);

/* Static text for a status code (never NULL). */
const char *sv_status_string(sv_status s);

/* Testing aid for the one-launch paths (the chain path of sv_verify_chain,
 * the two-phase greedy chain of sv_verify_greedy, the root rows and first
 * plan of sv_verify_tree): how many times a waiting workgroup reads the row
 * statistics that other workgroups of the same launch publish, before it
 * computes any still missing itself with the same arithmetic (the outputs
 * do not change).  Default 65536 (a bound far beyond any call's streaming);
 * 0 makes the waiting workgroups compute every statistic themselves; a
 * negative value restores the default.  Returns the previous value.
 * Applies to launches issued after it returns, from any thread. */
int sv_set_handoff_polls(int polls);

/* Workspace bytes for one call of the matching entry point with these sizes;
 * 0 when the sizes are invalid. */
size_t sv_chain_workspace_bytes(int B, int k, int V, sv_dtype dt);
size_t sv_greedy_workspace_bytes(int B, int k, int V, sv_dtype dt);
size_t sv_tree_workspace_bytes(int B, int N, int V, sv_dtype dt);
size_t sv_tree_sampled_workspace_bytes(int B, int N, int V, sv_dtype dt);

/*
 * Chain verification with sampling (sections "Speculative decoding" and
 * "Target-Draft" of the pages above).
 *
 * Sizes: B >= 0 sequences, 0 <= k <= SV_MAX_DRAFTS drafts each, vocabulary
 * 1 <= V <= SV_MAX_VOCAB.  B == 0 returns SV_OK without launching anything.
 * k == 0 is plain temperature sampling of target row 0.
 *
 *   draft_tokens  int32  [B][k]        drafted token ids (may be NULL if k == 0)
 *   draft_logits  dt     [B][k][V]     draft row i is the draft distribution that drew
 *                                      draft i (may be NULL if k == 0)
 *   target_logits dt     [B][k+1][V]   target row j scores draft j; row k is the bonus row
 *   temperature   fp32   [B]           T_b >= 0 scales sequence b's draft and target rows;
 *                                      T_b == 0 makes each row the one-hot distribution at
 *                                      its first (lowest-index) argmax
 *   uniforms      fp32   [B][k+1]      u[b][i] (i < k) tests draft i with "u < tau";
 *                                      u[b][k] drives the final draw
 *   accepted_len  int32  [B]      out  a_b = number of leading drafts accepted, 0..k
 *   emitted       int32  [B][k+1] out  drafts 0..a_b-1, then the final token, then -1
 *   accept_prob   fp32   [B][k]   out  optional (NULL to skip): tau_i = min(1, p_i/q_i)
 *                                      for every i < k (also past the first rejection)
 *
 * With P = softmax(logits / T_b) per row, p_i = P_target,i(x_i), q_i =
 * P_draft,i(x_i): draft i passes when u[b][i] < tau_i, a_b is the index of the
 * first failure (k if none).  The final token is drawn by inverse CDF over
 * ascending token ids with u[b][k]: from max(0, P_target,a - P_draft,a)
 * renormalised when a_b < k (from P_target,a if that residual is empty), from
 * P_target,k when a_b == k: y = min{ m : sum_{v<=m} w_v > u * sum_v w_v }.
 *
 * Without accept_prob, from k >= 6 and 128 MiB of draft and target rows
 * 0..k-1, the rows of positions max(1, k/4) and later are read only for the
 * sequences that accept all drafts before them.  The outputs are the same.
 * When the final draw takes at most 2048 workgroups and each row has at most
 * 8 G tiles of 8 KiB, G the largest power of two with 2k G <= 64 (k <= 32;
 * 512 tiles over the 2k rows when 2k is a power of two), the rows are
 * streamed and the draw made in one launch: each sequence's draw starts once its own rows are
 * streamed, waiting within a bound for their statistics
 * (sv_set_handoff_polls).  The statistics pass through the workspace tagged
 * with a 64-bit value unique to the call, so whatever the workspace held
 * before is never taken for them (unrelated bytes match a tag with
 * probability 2^-64); a call made while its stream is captured into a graph
 * clears them first instead, with one more launch.  The outputs are the same.
 */
sv_status sv_verify_chain(int B, int k, int V, sv_dtype dt,
                          const int32_t *draft_tokens, const void *draft_logits,
                          const void *target_logits, const float *temperature,
                          const float *uniforms, int32_t *accepted_len, int32_t *emitted,
                          float *accept_prob, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Bytes of the workspace that sv_verify_chain_static holds on each GPU. */
#define SV_STATIC_WORKSPACE_BYTES ((size_t)16 << 20)

/*
 * sv_verify_chain without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc).  It computes exactly what sv_verify_chain
 * computes, with the same arguments and outputs, and calls no allocating
 * routine: its workspace is a device array of SV_STATIC_WORKSPACE_BYTES
 * compiled into the library, one per GPU, held until the process ends.  The
 * first call on a device looks up that device's copy (hipGetSymbolAddress,
 * with the device current).
 *
 * Sizes whose workspace (sv_chain_workspace_bytes) exceeds
 * SV_STATIC_WORKSPACE_BYTES return SV_ERR_WORKSPACE_TOO_SMALL before any
 * launch; a failed symbol lookup returns SV_ERR_HIP.  The array needs no
 * clearing between calls (every call writes each byte it uses, and the
 * one-launch path tells its own statistics from earlier calls' by their
 * tag), but all calls on one GPU share it: calls that overlap on one GPU, on
 * different streams or from different host threads, race and give undefined
 * results.
 */
sv_status sv_verify_chain_static(int B, int k, int V, sv_dtype dt,
                                 const int32_t *draft_tokens, const void *draft_logits,
                                 const void *target_logits, const float *temperature,
                                 const float *uniforms, int32_t *accepted_len, int32_t *emitted,
                                 float *accept_prob, hipStream_t stream);

/*
 * Greedy chain verification (temperature 0; section "Speculative decoding").
 *
 *   draft_tokens  int32 [B][k]        (may be NULL if k == 0)
 *   target_logits dt    [B][k+1][V]
 *   accepted_len  int32 [B]      out  a_b = first i with x_i != g_i, else k, where g_j is
 *                                     the lowest-index argmax of target row j
 *   emitted       int32 [B][k+1] out  x_0..x_{a-1}, g_a, then -1
 *
 * When the target rows reach 256 MiB they are read in two phases: rows
 * 0..(k+1)/2-1 of every sequence, then the rest only for the sequences whose
 * drafts match in all of those rows.  When each row has at most 8 G tiles
 * of 8 KiB, G the largest power of two with G (k+1)/2 <= 64, both phases
 * run in one launch:
 * each second-phase workgroup waits within a bound for its sequence's
 * first-phase statistics (sv_set_handoff_polls), which pass through the
 * workspace tagged per call as in sv_verify_chain.
 */
sv_status sv_verify_greedy(int B, int k, int V, sv_dtype dt,
                           const int32_t *draft_tokens, const void *target_logits,
                           int32_t *accepted_len, int32_t *emitted,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Greedy static-tree verification, EAGLE-style (section "EAGLE").
 *
 *   node_tokens   int32 [B][N]   node 0 is the root (the last accepted token; its
 *                                own token is never matched)
 *   parent        int32 [N] when parent_stride == 0 (one tree shared by all
 *                                sequences), else [B][parent_stride], parent_stride >= N;
 *                                parent[i] in [0, i) for i >= 1, parent[0] ignored
 *   max_depth     >= 0, at least the depth of every node; width of the outputs is
 *                 max_depth + 1
 *   target_logits dt    [B][N][V] row n is the target's prediction after node n
 *   accepted_len  int32 [B]                out  depth d of the chosen node, or -1 when
 *                                               the parent array breaks the bounds above or
 *                                               a node is deeper than max_depth
 *   emitted       int32 [B][max_depth+1]   out  tokens of the path's nodes below the root,
 *                                               then the lowest-index argmax of the chosen
 *                                               node's row, then -1 (all -1 when invalid)
 *   accepted_nodes int32 [B][max_depth+1]  out  optional (NULL to skip): the path's node
 *                                               ids below the root, then -1
 *
 * Node i >= 1 is accepted when its parent is accepted and its token equals
 * the lowest-index argmax of its parent's row; the chosen node is the deepest
 * accepted node, the lowest index among equally deep ones.
 *
 * From 96 MiB of rows the root rows are read first, then only the rows of
 * nodes whose depth-1 ancestor is accepted (from 192 MiB and N >= 48: nodes
 * of depth 1-2 below an accepted depth-1 node, then deeper nodes below an
 * accepted depth-3 node).  The outputs are the same.  With at most 256
 * nodes, the root rows and the first choice of rows share one launch, the
 * root rows' statistics passing through the workspace tagged per call as in
 * sv_verify_chain.
 */
sv_status sv_verify_tree(int B, int N, int V, sv_dtype dt,
                         const int32_t *node_tokens, const int32_t *parent, int parent_stride,
                         int max_depth, const void *target_logits,
                         int32_t *accepted_len, int32_t *emitted, int32_t *accepted_nodes,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Sampled (stochastic) tree verification.  The pages (section "EAGLE") keep
 * the longest path of the draft tree that passes but give no rule for a
 * sampled tree; the rule is the multi-step speculative sampling of SpecInfer
 * (Miao et al., 2023), the one the EAGLE work uses.
 *
 *   node_tokens, parent, parent_stride, max_depth   as for sv_verify_tree;
 *                 the children of node n are expected to be independent draws
 *                 from node n's draft distribution (the output then follows the
 *                 target distribution)
 *   draft_logits  dt    [B][N][V]  row n: the draft distribution the children of n
 *                                  were drawn from (rows of leaves are not read)
 *   target_logits dt    [B][N][V]  row n: the target's prediction after node n (a
 *                                  leaf's row is read only if the walk ends there)
 *   temperature   f32   [B]        >= 0; 0 means one-hot rows at the lowest-index argmax
 *   uniforms      f32   [B][N]     in [0,1): u[b][i] tests node i >= 1, u[b][0] drives
 *                                  the final draw
 *   accepted_len, emitted, accepted_nodes   out, as for sv_verify_tree: the depth of
 *                 the last kept node (-1 for an invalid tree), the kept tokens then the
 *                 final token then -1, the kept node ids then -1
 *
 * From the root, the children of the current node n are tested in ascending
 * index order against a running distribution r that starts as P_target,n:
 * child i with token y is kept when u[b][i] < min(1, r(y) / P_draft,n(y)) and
 * the walk moves to it; a rejection replaces r by max(0, r - P_draft,n)
 * renormalised (by P_target,n itself if that is empty).  When no child is kept
 * (or n is a leaf) the final token is drawn from r by the inverse CDF over
 * ascending token ids with u[b][0].  Token ids outside [0,V) are rejected.
 * A streaming pass reads the target and draft rows of inner nodes; a leaf's
 * target row is read only when a walk ends at that leaf.  The walk then runs
 * in a fixed number of launches, several workgroups per sequence, each launch
 * testing siblings up to the next rejection and summing that rejection's
 * residual mass; a last one-workgroup-per-sequence pass draws the final token
 * or finishes any walk the launches did not complete.
 */
sv_status sv_verify_tree_sampled(int B, int N, int V, sv_dtype dt,
                                 const int32_t *node_tokens, const int32_t *parent, int parent_stride,
                                 int max_depth, const void *draft_logits, const void *target_logits,
                                 const float *temperature, const float *uniforms,
                                 int32_t *accepted_len, int32_t *emitted, int32_t *accepted_nodes,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Commit of one verification step on the device (section "MTP Schedule for
 * a Single Token": after acceptance a kernel places the next tokens, so the
 * host need not wait for the accepted lengths).
 *
 *   B             >= 0 sequences (0: no launch)
 *   width         >= 1 columns of `emitted` (k+1 for chain and greedy outputs,
 *                 max_depth+1 for tree outputs)
 *   accepted_len  int32 [B]         a_b as written by a verify call; a_b < 0 (an invalid
 *                                   tree) commits nothing
 *   emitted       int32 [B][width]  the step's tokens; the first a_b + 1 are committed
 *   seq_len       int32 [B]  in/out tokens already in each sequence's history; grows by
 *                                   the committed count
 *   history       int32 [B][history_stride] out  optional (NULL: no history, and no
 *                                   capacity limit): committed tokens are written at
 *                                   history[b][seq_len[b] + j], j = 0..a_b
 *   packed_offsets int32 [B+1] out  optional (NULL): exclusive prefix sum of the committed
 *                                   counts (where each sequence's new tokens start in a
 *                                   packed buffer), the total in [B]
 *   packed        int32 [>= B * width] out  optional (NULL): the committed tokens, packed
 *                                   in sequence order at packed_offsets
 *   status        int32 [B]   out  optional (NULL): 0 committed; 1 nothing committed because
 *                                   a_b >= width, seq_len[b] < 0, seq_len[b] + a_b + 1 >
 *                                   INT32_MAX or (with a history) seq_len[b] + a_b + 1 >
 *                                   history_stride; 2 nothing to commit (a_b < 0)
 *
 * The history and packed writes of different sequences never overlap; seq_len
 * is updated in place, so the call must not be repeated for the same step.
 * Limits: B <= 2^24.
 */
sv_status sv_commit_tokens(int B, int width, const int32_t *accepted_len, const int32_t *emitted,
                           int32_t *seq_len, int32_t *history, int history_stride,
                           int32_t *packed_offsets, int32_t *packed, int32_t *status,
                           hipStream_t stream);

/*
 * Kernel timing, for benchmarks.  Between sv_profile_begin() and
 * sv_profile_end() every entry point records a HIP event pair around each of
 * its kernel launches (host memory for at most max_launches launches is
 * reserved by sv_profile_begin; later launches are not timed).
 * sv_profile_end() waits for the recorded events and fills up to max_out
 * records, one per kernel name, returning how many it wrote (or -1 on error).
 * Not thread-safe; calls from several host threads must not overlap with it.
 */
typedef struct {
    char name[48];     /* kernel name */
    int launches;      /* timed launches */
    double total_ms;   /* sum of event-measured durations */
} sv_kernel_time;

sv_status sv_profile_begin(int max_launches);
int sv_profile_end(sv_kernel_time *out, int max_out);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
