// sv_greedy_tree.hpp -- sv_verify_greedy and sv_verify_tree: the streaming argmax and the
// per-sequence finalisers (part of sv_kernels.hpp).
#pragma once

#include "sv_tiles.hpp"

namespace sv {
// ---------------------------------------------------------------- argmax rows ---

// (max, lowest index) partials of every tile of `nrows` contiguous rows.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void argmax_rows_kernel(const void* __restrict__ logits, int64_t nrows,
                                                             int V, int nT, Partial* __restrict__ part) {
    const int64_t gw = global_wave();
    if (gw >= nrows * nT) return;
    const int64_t r = gw / nT;
    const int64_t tile = gw - r * nT;
    const ArgMax a = tile_argmax_any<DT, VEC, U>(logits, r * static_cast<int64_t>(V), V, tile);
    if (lane_id() == 0) part[gw] = Partial{a.val, a.idx};
}

// ---------------------------------------------------------------- greedy ---

// The argmax partials of rows j0 .. j0 + nrows - 1 of every sequence of a
// greedy chain (rows b * (k + 1) + j).  Rows after a sequence's first
// mismatch never reach its outputs, so the rows are streamed in two phases:
// CHECK = false streams rows 0 .. s - 1 of every sequence; CHECK = true
// streams rows s .. k only for sequences whose first s drafts all equal their
// rows' argmax, which wave 0 of each workgroup finds from the first phase's
// partials (G lanes per row, one round trip).  Each wave takes TPW tiles, a
// workgroup kWavesPerBlock * TPW consecutive ones (`groups` workgroups per
// row).  The one-dimensional grid (workgroup blk) runs over (sequence, row,
// group) with the group fastest: the dispatcher deals consecutive workgroups
// out to the XCDs in turn, so every sequence's work is spread over the XCDs
// and each gets an even share of the second phase however its sequences
// fall.  With SHARED both phases run in one launch (greedy_fused_kernel): the
// first also publishes its partials in tagged slots (slot row b * s + j), and
// the second's check reads them from there as they are published
// (await_slots, which needs all of a row's partials in one group_load).
template <int DT, bool VEC, int U, bool CHECK, int TPW, bool SHARED = false>
__device__ __forceinline__ void greedy_rows(const void* __restrict__ logits, const int32_t* __restrict__ tokens,
                                            int k, int V, int nT, int groups, int nrows, int j0,
                                            Partial* __restrict__ part, int64_t blk,
                                            TaggedPartial* __restrict__ slots = nullptr, int s_rows = 0,
                                            CallTag tag = {}, int polls = 0, Partial* s_q = nullptr) {
    const int per_seq = groups * nrows;
    const int64_t b = blk / per_seq;
    const int rem = static_cast<int>(blk - b * per_seq);
    const int z = rem / groups;
    const int group = rem - z * groups;
    const int rows = k + 1;
    if constexpr (CHECK) {
        __shared__ int s_go;
        if (threadIdx.x < kWave) {
            const int lane = lane_id();
            const int s = j0;  // rows 0 .. s - 1 were streamed by the first phase
            int G = kWave;
            while (G > 1 && G * s > kWave) G >>= 1;
            const int rho = lane / G;
            const bool valid = rho < s;
            const Partial* p = part + (b * rows + (valid ? rho : 0)) * static_cast<int64_t>(nT);
            Partial q[kBatch];
            if constexpr (SHARED)
                await_slots(slots + (b * s_rows + (valid ? rho : 0)) * static_cast<int64_t>(nT), valid, nT, G, tag,
                            polls, q, s_q, [&](int r, int64_t tile) {
                                const ArgMax a = tile_argmax_any<DT, VEC, U>(
                                    logits, (b * rows + r) * static_cast<int64_t>(V), V, tile);
                                return Partial{a.val, a.idx};
                            });
            else
                group_load(p, nT, G, valid, q);
            const int x = valid ? tokens[b * k + rho] : 0;
            int r;
            double sum;
            ArgMax am;
            group_reduce<false>(p, nT, G, valid, q, r, sum, am);
            const bool mismatch = __ballot(valid && (lane & (G - 1)) == 0 && x != am.idx) != 0;
            if (lane == 0) s_go = !mismatch;
        }
        __syncthreads();
        if (!s_go) return;
    }
    const int64_t row = b * rows + j0 + z;
    const int wave = threadIdx.x / kWave;
#pragma unroll 1
    for (int i = 0; i < TPW; ++i) {
        const int64_t tile = (static_cast<int64_t>(group) * TPW + i) * kWavesPerBlock + wave;
        if (tile >= nT) break;
        const ArgMax a = tile_argmax_any<DT, VEC, U>(logits, row * static_cast<int64_t>(V), V, tile);
        if (lane_id() == 0) {
            part[row * nT + tile] = Partial{a.val, a.idx};
            if constexpr (SHARED && !CHECK)
                store_partial_tagged(slots + (b * s_rows + j0 + z) * static_cast<int64_t>(nT) + tile,
                                     Partial{a.val, a.idx}, tag);
        }
    }
}

// The first phase (or the only one).
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void greedy_rows_kernel(const void* __restrict__ logits,
                                                             const int32_t* __restrict__ tokens, int k, int V,
                                                             int nT, int groups, int nrows, int j0,
                                                             Partial* __restrict__ part) {
    greedy_rows<DT, VEC, U, false, 1>(logits, tokens, k, V, nT, groups, nrows, j0, part, blockIdx.x);
}

// The second phase.
template <int DT, bool VEC, int U, int TPW>
__global__ __launch_bounds__(kBlock) void greedy_rows_rest_kernel(const void* __restrict__ logits,
                                                                  const int32_t* __restrict__ tokens, int k, int V,
                                                                  int nT, int groups, int nrows, int j0,
                                                                  Partial* __restrict__ part) {
    greedy_rows<DT, VEC, U, true, TPW>(logits, tokens, k, V, nT, groups, nrows, j0, part, blockIdx.x);
}

// Both phases in one launch: workgroups 0 .. p1_blocks - 1 stream rows
// 0 .. s - 1 of every sequence (groups1 workgroups per row) and publish their
// partials; the rest stream rows s .. k of the sequences whose first s
// drafts match, each checking its sequence as the partials arrive.  Every
// second-phase workgroup waits only on first-phase ones, which come first in
// the grid and wait on nothing.
template <int DT, bool VEC, int U, int TPW>
__global__ __launch_bounds__(kBlock) void greedy_fused_kernel(const void* __restrict__ logits,
                                                              const int32_t* __restrict__ tokens, int k, int V,
                                                              int nT, int s, int groups1, int groups2,
                                                              int64_t p1_blocks, TaggedPartial* __restrict__ slots,
                                                              CallTag tag, int polls, Partial* __restrict__ part) {
    if (blockIdx.x < p1_blocks) {
        greedy_rows<DT, VEC, U, false, 1, true>(logits, tokens, k, V, nT, groups1, s, 0, part, blockIdx.x, slots, s,
                                                tag);
        return;
    }
    __shared__ Partial s_q[kBatch * kWave];
    greedy_rows<DT, VEC, U, true, TPW, true>(logits, tokens, k, V, nT, groups2, k + 1 - s, s, part,
                                             blockIdx.x - p1_blocks, slots, s, tag, polls, s_q);
}

// One wave: the argmax g_j of each of the k + 1 rows of sequence b (partials
// rows_base[j * nT + t]) is combined by a group of G lanes (the first
// partials of every row and the draft tokens in flight together); the first
// position with x_j != g_j is the rejection, and g_a is the emitted target
// token.  s_g: k + 1 ints of LDS.
__device__ __forceinline__ void greedy_finish(const int32_t* __restrict__ tokens, int k, int nT,
                                              const Partial* rows_base, int64_t b, int* s_g,
                                              int32_t* __restrict__ accepted_len, int32_t* __restrict__ emitted) {
    const int lane = lane_id();
    const int rows = k + 1;
    int G = kWave;
    while (G > 1 && G * rows > kWave) G >>= 1;
    const int per_pass = kWave / G;
    Partial q[kBatch];
    group_load(rows_base + (lane / G < rows ? lane / G : 0) * static_cast<int64_t>(nT), nT, G, lane / G < rows, q);
    const int x = lane < k ? tokens[b * k + lane] : 0;
    for (int rho0 = 0; rho0 < rows; rho0 += per_pass) {
        const int rho = rho0 + lane / G;
        const bool valid = rho < rows;
        const Partial* p = rows_base + (valid ? rho : 0) * static_cast<int64_t>(nT);
        if (rho0 > 0) group_load(p, nT, G, valid, q);
        int r;
        double sum;
        ArgMax am;
        group_reduce<false>(p, nT, G, valid, q, r, sum, am);
        if (valid && (lane & (G - 1)) == 0) s_g[rho] = am.idx;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int g = lane < k ? s_g[lane] : -1;
    int a = first_lane(lane < k && x != g);
    if (a < 0) a = k;
    const int y = s_g[a];
    int32_t* out = emitted + b * (k + 1);
    for (int j = lane; j <= k; j += kWave) out[j] = j < a ? tokens[b * k + j] : (j == a ? y : -1);
    if (lane == 0) accepted_len[b] = a;
}

// One wave per sequence, from the streamed partials.  The partials of rows a
// second phase skipped hold stale values; they only yield g_j for j past a
// mismatch in the first phase's rows, which are never used.
__global__ __launch_bounds__(kWave) void greedy_finalize_kernel(const int32_t* __restrict__ tokens, int k,
                                                                int nT, const Partial* __restrict__ part,
                                                                int32_t* __restrict__ accepted_len,
                                                                int32_t* __restrict__ emitted) {
    __shared__ int s_g[SV_MAX_DRAFTS + 1];
    const int64_t b = blockIdx.x;
    greedy_finish(tokens, k, nT, part + b * (k + 1) * static_cast<int64_t>(nT), b, s_g, accepted_len, emitted);
}

// Small greedy chains in one launch: one workgroup per sequence streams the
// k + 1 rows' tiles (the tile argmax, partials to LDS) and its first wave
// finishes as greedy_finalize does (at most kSmallMaxParts tiles; the host
// sends at most one per wave).
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kSmallBlock) void greedy_small_kernel(const void* __restrict__ logits,
                                                                   const int32_t* __restrict__ tokens, int k, int V,
                                                                   int nT, int32_t* __restrict__ accepted_len,
                                                                   int32_t* __restrict__ emitted) {
    __shared__ Partial s_part[kSmallMaxParts];
    __shared__ int s_g[SV_MAX_DRAFTS + 1];
    const int64_t b = blockIdx.x;
    const int wave = threadIdx.x / kWave;
    for (int w = wave; w < (k + 1) * nT; w += kSmallWaves) {
        const int row = w / nT;
        const int tile = w - row * nT;
        const ArgMax a = tile_argmax_any<DT, VEC, U>(logits, (b * (k + 1) + row) * static_cast<int64_t>(V), V, tile);
        if (lane_id() == 0) s_part[w] = Partial{a.val, a.idx};
    }
    __syncthreads();
    if (threadIdx.x < kWave) greedy_finish(tokens, k, nT, s_part, b, s_g, accepted_len, emitted);
}

// ---------------------------------------------------------------- tree ---

// A node's row is needed only if the node is accepted, and a node can be
// accepted only if all its ancestors are.  Large trees are therefore
// streamed in phases by depth: the root rows first (tree_root_rows), then,
// each time after tree_plan has listed the nodes of the next depth range
// whose ancestor at the range's first depth is accepted, only their rows
// (tree_rows_rest).  tree_finalize is the same for every schedule: the
// partials of rows never streamed hold stale values, and they only yield g_p
// for nodes p that are not accepted, whose children fail their edge test
// whatever g_p is.

// Argmax partials of every sequence's root row (node 0 of N).
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void tree_root_rows_kernel(const void* __restrict__ logits, int N, int V,
                                                                int nT, int groups, Partial* __restrict__ part) {
    greedy_rows<DT, VEC, U, false, 1>(logits, nullptr, N - 1, V, nT, groups, 1, 0, part, blockIdx.x);
}

// The rows of one later phase, one workgroup per sequence and one thread per
// node: the nodes n with d_lo <= depth(n) <= d_hi whose ancestor at depth
// d_lo is accepted, listed in index order, and their number.  Earlier phases
// have streamed the rows of every node at depth < d_lo that may be accepted,
// so that ancestor's acceptance follows from their partials: the argmax of
// every row (G lanes per row; the root's alone when d_lo = 1), then depth and
// path acceptance by pointer jumping, then the ancestor at depth d_lo by
// pointer jumping.  A malformed tree lists nothing (tree_finalize reports it).
// With SHARED (d_lo = 1 only, in tree_root_plan_kernel) the root row's
// partials are read from the tagged slots that the same launch's first
// workgroups fill (await_slots, a missing one computed with their own
// tile_argmax_any); `logits` is only read then.
template <bool SHARED, int DT, bool VEC, int U>
__device__ __forceinline__ void tree_plan(const int32_t* __restrict__ node_tokens, const int32_t* __restrict__ parent,
                                          int parent_stride, int N, int nT, const Partial* __restrict__ part, int d_lo,
                                          int d_hi, int32_t* __restrict__ list, int32_t* __restrict__ count, int64_t b,
                                          const void* __restrict__ logits = nullptr, int V = 0,
                                          const TaggedPartial* __restrict__ slots = nullptr, CallTag tag = {},
                                          int polls = 0) {
    __shared__ int s_g[SV_MAX_TREE_NODES];
    __shared__ int s_tok[SV_MAX_TREE_NODES];
    __shared__ int s_anc[SV_MAX_TREE_NODES];
    __shared__ int s_len[SV_MAX_TREE_NODES];
    __shared__ int s_ok[SV_MAX_TREE_NODES];
    __shared__ int s_wave[SV_MAX_TREE_NODES / kWave];
    __shared__ int s_bad;
    const int n = threadIdx.x;
    const int lane = lane_id();
    const int nthreads = blockDim.x;
    if (n == 0) s_bad = 0;
    __syncthreads();
    const int rows = d_lo == 1 ? 1 : N;
    int G = kWave;
    while (G > 1 && G * rows > nthreads) G >>= 1;
    const int per_pass = nthreads / G;
    const Partial* rows_base = part + b * N * static_cast<int64_t>(nT);
    Partial q[kBatch];
    if constexpr (SHARED) {
        // one row, read by the lanes of wave 0 (G = 64); the other waves hold no
        // partial, so only wave 0 ever uses s_q
        __shared__ Partial s_q[kBatch * kWave];
        await_slots(slots + b * static_cast<int64_t>(nT), n / G < rows, nT, G, tag, polls, q, s_q,
                    [&](int, int64_t tile) {
                        const ArgMax a = tile_argmax_any<DT, VEC, U>(logits, b * N * static_cast<int64_t>(V), V, tile);
                        return Partial{a.val, a.idx};
                    });
    } else {
        group_load(rows_base + (n / G < rows ? n / G : 0) * static_cast<int64_t>(nT), nT, G, n / G < rows, q);
    }
    int p = 0;
    if (n < N) {
        s_tok[n] = node_tokens[b * N + n];
        p = n == 0 ? 0 : parent[b * static_cast<int64_t>(parent_stride) + n];
        if (n > 0 && (p < 0 || p >= n)) s_bad = 1;
    }
    for (int m0 = 0; m0 < rows; m0 += per_pass) {
        const int m = m0 + n / G;
        const bool valid = m < rows;
        const Partial* pr = rows_base + (valid ? m : 0) * static_cast<int64_t>(nT);
        if (m0 > 0) group_load(pr, nT, G, valid, q);
        int r;
        double sum;
        ArgMax am;
        group_reduce<false>(pr, nT, G, valid, q, r, sum, am);
        if (valid && (n & (G - 1)) == 0) s_g[m] = am.idx;
    }
    __syncthreads();
    if (s_bad) {
        if (n == 0) count[b] = 0;
        return;
    }
    // depth and path acceptance; with d_lo = 1 only the root's children are tested
    int anc = p, len = n == 0 ? 0 : 1;
    int ok = 1;
    if (n > 0 && n < N) ok = (d_lo == 1 && p != 0) ? 1 : (s_tok[n] == s_g[p]);
    if (n < N) {
        s_anc[n] = anc;
        s_len[n] = len;
        s_ok[n] = ok;
    }
    __syncthreads();
    for (int step = 1; step < N; step <<= 1) {
        int a2 = 0, l2 = 0, o2 = 1;
        if (n < N) {
            a2 = s_anc[anc];
            l2 = s_len[anc];
            o2 = s_ok[anc];
        }
        __syncthreads();
        if (n < N) {
            len += l2;
            ok &= o2;
            anc = a2;
            s_anc[n] = anc;
            s_len[n] = len;
            s_ok[n] = ok;
        }
        __syncthreads();
    }
    // the ancestor at depth d_lo: nodes no deeper are fixed points (s_anc is reused)
    int up = (n < N && len > d_lo) ? p : n;
    if (n < N) s_anc[n] = up;
    __syncthreads();
    for (int step = 1; step < N; step <<= 1) {
        const int u2 = n < N ? s_anc[up] : 0;
        __syncthreads();
        if (n < N) {
            up = u2;
            s_anc[n] = up;
        }
        __syncthreads();
    }
    const bool need = n > 0 && n < N && len >= d_lo && len <= d_hi && s_ok[up];
    const uint64_t m = __ballot(need);
    const int w = n / kWave;
    if (lane == 0) s_wave[w] = __popcll(m);
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += s_wave[i];
    if (need) list[b * N + base + __popcll(m & ((uint64_t(1) << lane) - 1))] = n;
    if (n == 0) {
        int total = 0;
        for (int i = 0; i < nthreads / kWave; ++i) total += s_wave[i];
        count[b] = total;
    }
}

__global__ __launch_bounds__(SV_MAX_TREE_NODES) void tree_plan_kernel(const int32_t* __restrict__ node_tokens,
                                                                      const int32_t* __restrict__ parent,
                                                                      int parent_stride, int N, int nT,
                                                                      const Partial* __restrict__ part, int d_lo,
                                                                      int d_hi, int32_t* __restrict__ list,
                                                                      int32_t* __restrict__ count) {
    tree_plan<false, SV_F32, false, 1>(node_tokens, parent, parent_stride, N, nT, part, d_lo, d_hi, list, count,
                                       blockIdx.x);
}

// The root rows and the first plan (d_lo = 1) in one launch, for trees of at
// most kBlock nodes: workgroups 0 .. root_blocks - 1 stream every sequence's
// root row as tree_root_rows_kernel does and publish its partials in tagged
// slots; workgroup root_blocks + b then lists sequence b's nodes as
// tree_plan_kernel does, reading the root's partials as they are published.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void tree_root_plan_kernel(const void* __restrict__ logits,
                                                                const int32_t* __restrict__ node_tokens,
                                                                const int32_t* __restrict__ parent,
                                                                int parent_stride, int N, int V, int nT, int groups,
                                                                int64_t root_blocks, TaggedPartial* __restrict__ slots,
                                                                CallTag tag, int polls, int d_hi,
                                                                Partial* __restrict__ part, int32_t* __restrict__ list,
                                                                int32_t* __restrict__ count) {
    if (blockIdx.x < root_blocks) {
        greedy_rows<DT, VEC, U, false, 1, true>(logits, nullptr, N - 1, V, nT, groups, 1, 0, part, blockIdx.x, slots,
                                                1, tag);
        return;
    }
    tree_plan<true, DT, VEC, U>(node_tokens, parent, parent_stride, N, nT, part, 1, d_hi, list, count,
                                blockIdx.x - root_blocks, logits, V, slots, tag, polls);
}

// Argmax partials of the listed rows: one workgroup per (sequence, list
// entry i, group of kWavesPerBlock tiles), the group fastest (consecutive
// workgroups go to different XCDs); entries past a sequence's count exit at
// once.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void tree_rows_rest_kernel(const void* __restrict__ logits, int N, int V,
                                                                int nT, int groups,
                                                                const int32_t* __restrict__ list,
                                                                const int32_t* __restrict__ count,
                                                                Partial* __restrict__ part) {
    const int64_t rest = blockIdx.x / groups;
    const int group = static_cast<int>(blockIdx.x - rest * groups);
    const int64_t b = rest / (N - 1);
    const int i = static_cast<int>(rest - b * (N - 1));
    const int cnt = count[b];
    const int node = list[b * N + i];
    if (i >= cnt) return;
    const int64_t tile = static_cast<int64_t>(group) * kWavesPerBlock + threadIdx.x / kWave;
    if (tile >= nT) return;
    const int64_t row = b * N + node;
    const ArgMax a = tile_argmax_any<DT, VEC, U>(logits, row * static_cast<int64_t>(V), V, tile);
    if (lane_id() == 0) part[row * nT + tile] = Partial{a.val, a.idx};
}

// One workgroup per sequence, one thread per node (N <= blockDim.x <= 1024).
// The argmax of each node's row is combined by a group of G lanes (G as large
// as the block allows; the first partials of every row, the tokens and the
// parent links in flight together).  Pointer jumping over the parent links
// gives every node its depth and whether every edge on its root path
// matches; the deepest accepted node (lowest index among equals) is chosen
// and its path written out.
__global__ __launch_bounds__(SV_MAX_TREE_NODES) void tree_finalize_kernel(
    const int32_t* __restrict__ node_tokens, const int32_t* __restrict__ parent, int parent_stride, int N,
    int max_depth, int nT, const Partial* __restrict__ part, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ emitted, int32_t* __restrict__ accepted_nodes) {
    __shared__ int s_g[SV_MAX_TREE_NODES];
    __shared__ int s_tok[SV_MAX_TREE_NODES];
    __shared__ int s_par[SV_MAX_TREE_NODES];
    __shared__ int s_anc[SV_MAX_TREE_NODES];
    __shared__ int s_len[SV_MAX_TREE_NODES];
    __shared__ int s_ok[SV_MAX_TREE_NODES];
    __shared__ int s_bad;
    __shared__ int s_best;
    const int64_t b = blockIdx.x;
    const int n = threadIdx.x;
    const int width = max_depth + 1;
    if (n == 0) {
        s_bad = 0;
        s_best = -1;
    }
    __syncthreads();
    const int32_t* par = parent + b * static_cast<int64_t>(parent_stride);
    const int nthreads = blockDim.x;
    int G = kWave;
    while (G > 1 && G * N > nthreads) G >>= 1;
    const int per_pass = nthreads / G;
    const Partial* rows_base = part + b * N * static_cast<int64_t>(nT);
    Partial q[kBatch];
    group_load(rows_base + (n / G < N ? n / G : 0) * static_cast<int64_t>(nT), nT, G, n / G < N, q);
    int p = 0;
    if (n < N) {
        s_tok[n] = node_tokens[b * N + n];
        p = n == 0 ? 0 : par[n];
        if (n > 0 && (p < 0 || p >= n)) s_bad = 1;
        s_par[n] = p;
    }
    for (int m0 = 0; m0 < N; m0 += per_pass) {
        const int m = m0 + n / G;
        const bool valid = m < N;
        const Partial* pr = rows_base + (valid ? m : 0) * static_cast<int64_t>(nT);
        if (m0 > 0) group_load(pr, nT, G, valid, q);
        int r;
        double sum;
        ArgMax am;
        group_reduce<false>(pr, nT, G, valid, q, r, sum, am);
        if (valid && (n & (G - 1)) == 0) s_g[m] = am.idx;
    }
    __syncthreads();
    int anc = 0, len = 0, ok = 0;
    if (!s_bad && n < N) {
        anc = p;
        len = n == 0 ? 0 : 1;
        ok = n == 0 ? 1 : (s_tok[n] == s_g[p]);
        s_anc[n] = anc;
        s_len[n] = len;
        s_ok[n] = ok;
    }
    __syncthreads();
    if (!s_bad) {
        for (int step = 1; step < N; step <<= 1) {
            int a2 = 0, l2 = 0, o2 = 1;
            if (n < N) {
                a2 = s_anc[anc];
                l2 = s_len[anc];
                o2 = s_ok[anc];
            }
            __syncthreads();
            if (n < N) {
                len += l2;
                ok &= o2;
                anc = a2;
                s_anc[n] = anc;
                s_len[n] = len;
                s_ok[n] = ok;
            }
            __syncthreads();
        }
        if (n < N && len > max_depth) s_bad = 1;
        if (n < N && ok) atomicMax(&s_best, (len << 16) | (0xffff - n));
    }
    __syncthreads();
    int32_t* out = emitted + b * width;
    int32_t* nodes = accepted_nodes ? accepted_nodes + b * width : nullptr;
    if (s_bad) {
        for (int j = n; j < width; j += blockDim.x) {
            out[j] = -1;
            if (nodes) nodes[j] = -1;
        }
        if (n == 0) accepted_len[b] = -1;
        return;
    }
    const int best = s_best;
    const int d = best >> 16;
    const int m = 0xffff - (best & 0xffff);
    for (int j = d + 1 + n; j < width; j += blockDim.x) {
        out[j] = -1;
        if (nodes) nodes[j] = -1;
    }
    if (n == 0) {
        int v = m;
        for (int j = d - 1; j >= 0; --j) {
            out[j] = s_tok[v];
            if (nodes) nodes[j] = v;
            v = s_par[v];
        }
        out[d] = s_g[m];
        if (nodes && d < width) {
            // slot d of accepted_nodes stays -1: it holds no node (the bonus token has none)
            nodes[d] = -1;
        }
        accepted_len[b] = d;
    }
}

}  // namespace sv
