/*
 * oracle.c -- plain fp64 CPU oracle for batched draft-token verification.
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library; the product path never
 * does.  It shares no source with the GPU library (no headers, helpers,
 * tables or constants): it is written to be read against the pages, not to
 * be fast.
 *
 * Source: "Accelerating Sonar through speculation" (Perplexity; N. Licker,
 * E. McKnight; 2025).
 *   - Section "Speculative decoding": every prefix of the draft is scored and
 *     the longest prefix that passes the acceptance threshold is kept; with n
 *     draft tokens one step yields up to n+1 tokens, because at the mismatch
 *     (or after the last draft) the target's own logits are sampled.
 *   - Section "Target-Draft": acceptance compares the full draft and target
 *     probability distributions; the target always emits one more logits row
 *     after the accepted drafts, and that row is sampled.
 *   - Section "EAGLE": a draft tree is scored, the longest suitable path is
 *     kept and one more target token is appended.
 *   - Section "MTP": logits row i predicts token i+1, so target row j scores
 *     draft token j and row k (after the last draft) is the bonus row.
 * The pages name the acceptance threshold but do not write it out.  The rule
 * used here is the speculative sampling of the first work in the pages'
 * references (Leviathan et al., "Fast Inference from Transformers via
 * Speculative Decoding"): keep draft x with probability min(1, p(x)/q(x));
 * at the first rejection draw from the normalised residual max(0, p - q).
 *
 * Readings taken where the pages are silent:
 *   R-temp   one temperature T_b per sequence scales its draft and target
 *            rows; T_b = 0 means the one-hot distribution at the first argmax.
 *   R-u      uniforms u[b][0..k-1] test the drafts with a strict "u < tau";
 *            u[b][k] drives whichever final sample is taken.
 *   R-cdf    the final sample is an inverse CDF over ascending token ids:
 *            y = min{ m : C_m > u * W } with C_m = sum_{v<=m} w_v, W = C_{V-1};
 *            if rounding leaves no such m, y = the last token with w_v > 0.
 *   R-q0     q(x) = 0 gives tau = 1 if p(x) > 0, else 0.
 *   R-W0     a residual of total mass 0 falls back to the target row itself.
 *   R-ties   every argmax is the lowest index among equal maxima.
 *   R-tree   a tree path starts at the root and may end at any node; the
 *            deepest fully accepted node wins, lowest index among equals.
 *   R-mss    sampled trees: the pages give no rule, so the multi-step
 *            speculative sampling of SpecInfer (Miao et al., 2023) -- the
 *            multi-round rule the EAGLE work applies to its trees -- is used;
 *            see svo_verify_tree_sampled.
 *   R-commit the device-side commit (section "MTP Schedule for a Single
 *            Token": a kernel places the next tokens, so the host need not
 *            read the accepted counts) appends a_b + 1 tokens to sequence b's
 *            history and advances its length; a row is refused whole when
 *            a_b < 0 (an invalid tree), a_b >= width, the length is negative,
 *            the new length would pass INT32_MAX or (with a history) its
 *            capacity; see svo_commit_tokens.
 *
 * Band flag (sequences with T_b > 0 only): set when a tested uniform lies
 * within band_eps of its threshold tau_i, or u[b][k] lies within band_eps of
 * either CDF boundary C_{y-1}/W or C_y/W of the token drawn.  Such decisions
 * may legitimately differ between this fp64 code and an fp32 implementation.
 *
 * Arithmetic is double precision throughout; logits are widened exactly
 * (bfloat16 -> float -> double).  dtype code 0 = float32, 1 = bfloat16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SVO_F32 0
#define SVO_BF16 1

/* Planted mistakes, used only by tests that check their own power. */
#define MUT_NONE 0
#define MUT_SAMPLE_TARGET_AT_MISMATCH 1 /* draw from p, not max(0,p-q)      */
#define MUT_RESIDUAL_SWAPPED 2          /* draw from max(0,q-p)             */
#define MUT_ROWS_SHIFTED 3              /* draft i scored by target row i+1 */
#define MUT_ACCEPT_INVERTED 4           /* accept when u > tau              */
#define MUT_ARGMAX_LAST 5               /* ties go to the highest index     */
#define MUT_TREE_TIE_HIGHEST 6          /* tree: equal depth -> highest idx */
#define MUT_TREE_STALE_RESIDUAL 7       /* sampled tree: later siblings tested
                                           against p, not the updated residual */
static int g_mutation = MUT_NONE;

void svo_set_mutation(int m) { g_mutation = m; }
int svo_version(void) { return 1; }

int svo_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void svo_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* One logit, widened exactly to double. */
static double logit_at(const void *base, int dtype, size_t idx) {
    if (dtype == SVO_BF16) {
        uint32_t w = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[idx];
}

/* First (or, under a planted mistake, last) index of the row maximum of the
 * raw logits. */
static int row_argmax(const void *base, int dtype, size_t off, int V) {
    int g = 0;
    double best = logit_at(base, dtype, off);
    for (int v = 1; v < V; ++v) {
        double x = logit_at(base, dtype, off + (size_t)v);
        if (x > best || (g_mutation == MUT_ARGMAX_LAST && x == best)) {
            best = x;
            g = v;
        }
    }
    return g;
}

/* The row's distribution over the vocabulary.  T > 0: P = softmax(l / T),
 * written as z = l / T, M = max z, S = sum_v exp(z_v - M) in ascending v,
 * P_v = exp(z_v - M) / S.  T == 0: one-hot at the first argmax. */
static void row_distribution(const void *base, int dtype, size_t off, int V, double T, double *P) {
    if (!(T > 0.0)) {
        int g = row_argmax(base, dtype, off, V);
        for (int v = 0; v < V; ++v) P[v] = 0.0;
        P[g] = 1.0;
        return;
    }
    double M = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double z = logit_at(base, dtype, off + (size_t)v) / T;
        if (z > M) M = z;
    }
    double S = 0.0;
    for (int v = 0; v < V; ++v) {
        double e = exp(logit_at(base, dtype, off + (size_t)v) / T - M);
        P[v] = e;
        S += e;
    }
    for (int v = 0; v < V; ++v) P[v] /= S;
}

/* log sum_v exp(l_v / T) = M + log S, the log-normaliser of one row. */
static double row_logz(const void *base, int dtype, size_t off, int V, double T) {
    double M = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double z = logit_at(base, dtype, off + (size_t)v) / T;
        if (z > M) M = z;
    }
    double S = 0.0;
    for (int v = 0; v < V; ++v) S += exp(logit_at(base, dtype, off + (size_t)v) / T - M);
    return M + log(S);
}

/* Threshold tau = min(1, p/q); q == 0 gives 1 when p > 0, else 0. */
static double threshold(double p, double q) {
    if (q > 0.0) {
        double r = p / q;
        return r < 1.0 ? r : 1.0;
    }
    return p > 0.0 ? 1.0 : 0.0;
}

/* Inverse CDF over ascending token ids: y = min{m : C_m > u W}.  Also
 * returns the CDF boundaries C_{y-1} and C_y. */
static int inverse_cdf(const double *w, int V, double W, double u, double *c_lo, double *c_hi) {
    double target = u * W, C = 0.0;
    for (int m = 0; m < V; ++m) {
        double prev = C;
        C += w[m];
        if (C > target) {
            *c_lo = prev;
            *c_hi = C;
            return m;
        }
    }
    /* Rounding left C_{V-1} <= u W: take the last token that has mass. */
    int y = V - 1;
    while (y > 0 && !(w[y] > 0.0)) --y;
    double prev = 0.0;
    for (int m = 0; m < y; ++m) prev += w[m];
    *c_lo = prev;
    *c_hi = prev + w[y];
    return y;
}

/*
 * Chain verification of B sequences, each with k draft tokens.
 *   draft_tokens  [B][k]        int32, token ids in [0, V)
 *   draft_logits  [B][k][V]     draft row i scored draft token i
 *   target_logits [B][k+1][V]   target row j scores draft j; row k is the bonus row
 *   temperature   [B]           >= 0
 *   uniforms      [B][k+1]      in [0, 1)
 * Outputs: accepted_len [B]; emitted [B][k+1] (accepted drafts, the final
 * sample, then -1); optional accept_prob [B][k] (tau_i for every i < k),
 * band [B] (flag described above) and final_mass [B] (W of the final sample).
 * Returns 0, or 1 on an invalid argument.
 */
int svo_verify_chain(int B, int k, int V, int dtype, const int32_t *draft_tokens,
                     const void *draft_logits, const void *target_logits,
                     const float *temperature, const float *uniforms,
                     int32_t *accepted_len, int32_t *emitted, double *accept_prob,
                     int32_t *band, double *final_mass, double band_eps) {
    if (B < 0 || k < 0 || V <= 0 || (dtype != SVO_F32 && dtype != SVO_BF16)) return 1;
    if (B == 0) return 0;
    if (!target_logits || !temperature || !uniforms || !accepted_len || !emitted) return 1;
    if (k > 0 && (!draft_tokens || !draft_logits)) return 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int b = 0; b < B; ++b) {
        double *Pt = (double *)malloc(sizeof(double) * (size_t)V);
        double *Pd = (double *)malloc(sizeof(double) * (size_t)V);
        double *w = (double *)malloc(sizeof(double) * (size_t)V);
        double *tau = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        if (!Pt || !Pd || !w || !tau) {
            bad = 1;
            free(Pt); free(Pd); free(w); free(tau);
            continue;
        }
        const double T = (double)temperature[b];
        const int32_t *x = draft_tokens ? draft_tokens + (size_t)b * k : NULL;
        const float *u = uniforms + (size_t)b * (k + 1);
        int32_t *out = emitted + (size_t)b * (k + 1);

        /* Acceptance test for every draft position (O2) and first rejection (O3). */
        int a = k;
        for (int i = 0; i < k; ++i) {
            int trow = (g_mutation == MUT_ROWS_SHIFTED) ? i + 1 : i;
            row_distribution(target_logits, dtype, ((size_t)b * (k + 1) + trow) * (size_t)V, V, T, Pt);
            row_distribution(draft_logits, dtype, ((size_t)b * k + i) * (size_t)V, V, T, Pd);
            int xi = x[i];
            if (xi < 0 || xi >= V) { bad = 1; xi = 0; }
            tau[i] = threshold(Pt[xi], Pd[xi]);
            int acc = (g_mutation == MUT_ACCEPT_INVERTED) ? ((double)u[i] > tau[i])
                                                         : ((double)u[i] < tau[i]);
            if (!acc && a == k) a = i;
        }

        /* Final distribution (O4): residual at the rejection row, else the bonus row. */
        double W = 0.0;
        if (a < k) {
            int trow = (g_mutation == MUT_ROWS_SHIFTED) ? a + 1 : a;
            row_distribution(target_logits, dtype, ((size_t)b * (k + 1) + trow) * (size_t)V, V, T, Pt);
            row_distribution(draft_logits, dtype, ((size_t)b * k + a) * (size_t)V, V, T, Pd);
            for (int v = 0; v < V; ++v) {
                double r;
                if (g_mutation == MUT_SAMPLE_TARGET_AT_MISMATCH) r = Pt[v];
                else if (g_mutation == MUT_RESIDUAL_SWAPPED) r = Pd[v] - Pt[v];
                else r = Pt[v] - Pd[v];
                w[v] = r > 0.0 ? r : 0.0;
                W += w[v];
            }
            if (W == 0.0) {
                for (int v = 0; v < V; ++v) { w[v] = Pt[v]; W += w[v]; }
            }
        } else {
            row_distribution(target_logits, dtype, ((size_t)b * (k + 1) + k) * (size_t)V, V, T, Pt);
            for (int v = 0; v < V; ++v) { w[v] = Pt[v]; W += w[v]; }
        }

        /* Inverse CDF (O5) and outputs (O6). */
        double c_lo = 0.0, c_hi = 0.0;
        int y = inverse_cdf(w, V, W, (double)u[k], &c_lo, &c_hi);
        accepted_len[b] = a;
        for (int i = 0; i < a; ++i) out[i] = x[i];
        out[a] = y;
        for (int j = a + 1; j <= k; ++j) out[j] = -1;
        if (accept_prob)
            for (int i = 0; i < k; ++i) accept_prob[(size_t)b * k + i] = tau[i];
        if (final_mass) final_mass[b] = W;
        if (band) {
            int f = 0;
            if (T > 0.0) {
                int last_tested = a < k ? a : k - 1;
                for (int i = 0; i <= last_tested; ++i)
                    if (fabs((double)u[i] - tau[i]) < band_eps) f = 1;
                if (fabs((double)u[k] - c_lo / W) < band_eps) f = 1;
                if (fabs((double)u[k] - c_hi / W) < band_eps) f = 1;
            }
            band[b] = f;
        }
        free(Pt); free(Pd); free(w); free(tau);
    }
    return bad;
}

/*
 * Greedy chain verification (temperature 0): g_j = first argmax of target row
 * j; a = first i with x_i != g_i, else k; emitted = x_0..x_{a-1}, g_a, -1...
 */
int svo_verify_greedy(int B, int k, int V, int dtype, const int32_t *draft_tokens,
                      const void *target_logits, int32_t *accepted_len, int32_t *emitted) {
    if (B < 0 || k < 0 || V <= 0 || (dtype != SVO_F32 && dtype != SVO_BF16)) return 1;
    if (B == 0) return 0;
    if (!target_logits || !accepted_len || !emitted || (k > 0 && !draft_tokens)) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const int32_t *x = draft_tokens ? draft_tokens + (size_t)b * k : NULL;
        int32_t *out = emitted + (size_t)b * (k + 1);
        int a = k, y = -1;
        for (int j = 0; j <= k; ++j) {
            int g = row_argmax(target_logits, dtype, ((size_t)b * (k + 1) + j) * (size_t)V, V);
            if (j == k || x[j] != g) {
                a = j;
                y = g;
                break;
            }
        }
        accepted_len[b] = a;
        for (int i = 0; i < a; ++i) out[i] = x[i];
        out[a] = y;
        for (int j = a + 1; j <= k; ++j) out[j] = -1;
    }
    return 0;
}

/*
 * Greedy static-tree verification (section "EAGLE").
 *   node_tokens   [B][N]   node 0 is the root (the last accepted token, never matched)
 *   parent        [N] when parent_stride == 0 (one tree for all sequences),
 *                 else [B][parent_stride] with parent_stride >= N;
 *                 parent[i] in [0, i) for i >= 1 (parent[0] is ignored)
 *   target_logits [B][N][V]   row n is the target's prediction after node n
 * Node i >= 1 is accepted when its parent is accepted and its token equals the
 * first argmax of the parent's row.  The deepest accepted node m (lowest index
 * among equal depths) is chosen; emitted = tokens of the path root -> m (root
 * excluded), then the first argmax of m's row, then -1.  accepted_nodes
 * (optional) lists the path's node ids, then -1.  A parent array that breaks
 * the bounds above, or a node deeper than max_depth, marks the sequence
 * invalid: accepted_len = -1 and every output slot -1.
 */
int svo_verify_tree(int B, int N, int V, int dtype, const int32_t *node_tokens,
                    const int32_t *parent, int parent_stride, int max_depth,
                    const void *target_logits, int32_t *accepted_len, int32_t *emitted,
                    int32_t *accepted_nodes) {
    if (B < 0 || N <= 0 || V <= 0 || max_depth < 0 || (dtype != SVO_F32 && dtype != SVO_BF16)) return 1;
    if (parent_stride != 0 && parent_stride < N) return 1;
    if (B == 0) return 0;
    if (!node_tokens || !parent || !target_logits || !accepted_len || !emitted) return 1;
    const int width = max_depth + 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * (size_t)parent_stride;
        const int32_t *tok = node_tokens + (size_t)b * N;
        int *g = (int *)malloc(sizeof(int) * (size_t)N);
        int *depth = (int *)malloc(sizeof(int) * (size_t)N);
        int *acc = (int *)malloc(sizeof(int) * (size_t)N);
        if (!g || !depth || !acc) {
            bad = 1;
            free(g); free(depth); free(acc);
            continue;
        }
        for (int n = 0; n < N; ++n)
            g[n] = row_argmax(target_logits, dtype, ((size_t)b * N + n) * (size_t)V, V);
        int valid = 1;
        depth[0] = 0;
        acc[0] = 1;
        for (int i = 1; i < N; ++i) {
            int p = par[i];
            if (p < 0 || p >= i) { valid = 0; depth[i] = 0; acc[i] = 0; continue; }
            depth[i] = depth[p] + 1;
            acc[i] = acc[p] && tok[i] == g[p];
            if (depth[i] > max_depth) valid = 0;
        }
        int32_t *out = emitted + (size_t)b * width;
        int32_t *nodes = accepted_nodes ? accepted_nodes + (size_t)b * width : NULL;
        for (int j = 0; j < width; ++j) {
            out[j] = -1;
            if (nodes) nodes[j] = -1;
        }
        if (!valid) {
            accepted_len[b] = -1;
        } else {
            int m = 0;
            for (int i = 1; i < N; ++i) {
                if (!acc[i]) continue;
                if (depth[i] > depth[m] || (g_mutation == MUT_TREE_TIE_HIGHEST && depth[i] == depth[m]))
                    m = i;
            }
            int d = depth[m];
            accepted_len[b] = d;
            int n = m;
            for (int j = d - 1; j >= 0; --j) {
                out[j] = tok[n];
                if (nodes) nodes[j] = n;
                n = par[n];
            }
            out[d] = g[m];
        }
        free(g); free(depth); free(acc);
    }
    return bad;
}

/*
 * Sampled (stochastic) tree verification: multi-step speculative sampling
 * (SpecInfer, Miao et al. 2023, the rule the EAGLE work uses for its draft
 * trees).
 *   node_tokens   [B][N]     node 0 is the root (its token is never tested)
 *   parent        as for svo_verify_tree
 *   draft_logits  [B][N][V]  row n: the draft distribution q_n from which the
 *                            children of node n were drawn (rows of leaves unused)
 *   target_logits [B][N][V]  row n: the target distribution p_n after node n
 *   temperature   [B]        >= 0 (0: one-hot at the first argmax)
 *   uniforms      [B][N]     u[b][i], i >= 1, tests node i; u[b][0] drives the
 *                            final draw
 * The walk starts at the root.  At node n the children are tested in
 * ascending index order against a running distribution r, which starts as
 * p_n: child i with token y is kept when u[b][i] < min(1, r(y) / q_n(y))
 * (the q = 0 rule as for chains), and the walk moves to it.  A rejection
 * replaces r by the normalised residual max(0, r - q_n) / Z, Z its total
 * mass; if Z is 0 (rounding), r falls back to p_n, as for chains.  When no
 * child is kept (or n is a leaf), the final token is drawn from r by the
 * inverse CDF with u[b][0].
 * Outputs as for svo_verify_tree: accepted_len = depth of the last kept node,
 * emitted = the kept tokens then the final token then -1, accepted_nodes the
 * kept node ids then -1; an invalid tree gives -1 everywhere.  band[b] (T > 0
 * only) flags a tested uniform within band_eps of its threshold or u[b][0]
 * within band_eps of a CDF boundary of the final token.  final_mass[b]
 * (optional) is the mass, in units of the target row, of the distribution the
 * final token is drawn from: the product of the masses Z of the residuals
 * formed at the node where the walk stopped (1 when none was: r = p).
 */
int svo_verify_tree_sampled(int B, int N, int V, int dtype, const int32_t *node_tokens,
                            const int32_t *parent, int parent_stride, int max_depth,
                            const void *draft_logits, const void *target_logits,
                            const float *temperature, const float *uniforms,
                            int32_t *accepted_len, int32_t *emitted, int32_t *accepted_nodes,
                            int32_t *band, double *final_mass, double band_eps) {
    if (B < 0 || N <= 0 || V <= 0 || max_depth < 0 || (dtype != SVO_F32 && dtype != SVO_BF16)) return 1;
    if (parent_stride != 0 && parent_stride < N) return 1;
    if (B == 0) return 0;
    if (!node_tokens || !parent || !draft_logits || !target_logits || !temperature || !uniforms ||
        !accepted_len || !emitted)
        return 1;
    const int width = max_depth + 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * (size_t)parent_stride;
        const int32_t *tok = node_tokens + (size_t)b * N;
        const float *u = uniforms + (size_t)b * N;
        const double T = (double)temperature[b];
        int32_t *out = emitted + (size_t)b * width;
        int32_t *nodes = accepted_nodes ? accepted_nodes + (size_t)b * width : NULL;
        for (int j = 0; j < width; ++j) {
            out[j] = -1;
            if (nodes) nodes[j] = -1;
        }
        int *depth = (int *)malloc(sizeof(int) * (size_t)N);
        double *P = (double *)malloc(sizeof(double) * (size_t)V);
        double *Q = (double *)malloc(sizeof(double) * (size_t)V);
        double *r = (double *)malloc(sizeof(double) * (size_t)V);
        if (!depth || !P || !Q || !r) {
            bad = 1;
            free(depth); free(P); free(Q); free(r);
            continue;
        }
        /* The same validity rule as the greedy tree. */
        int valid = 1;
        depth[0] = 0;
        for (int i = 1; i < N; ++i) {
            int p = par[i];
            if (p < 0 || p >= i) { valid = 0; depth[i] = 0; continue; }
            depth[i] = depth[p] + 1;
            if (depth[i] > max_depth) valid = 0;
        }
        int flag = 0;
        double mass = 1.0;
        if (!valid) {
            accepted_len[b] = -1;
        } else {
            int n = 0, d = 0;
            for (;;) {
                size_t trow = ((size_t)b * N + n) * (size_t)V;
                row_distribution(target_logits, dtype, trow, V, T, P);
                int has_children = 0;
                for (int i = n + 1; i < N; ++i)
                    if (par[i] == n) has_children = 1;
                if (has_children) row_distribution(draft_logits, dtype, trow, V, T, Q);
                /* the running distribution starts as the target row */
                for (int v = 0; v < V; ++v) r[v] = P[v];
                int rejected = 0;
                mass = 1.0;
                int next = -1;
                for (int i = n + 1; i < N && next < 0; ++i) {
                    if (par[i] != n) continue;
                    int y = tok[i];
                    if (y < 0 || y >= V) { bad = 1; y = 0; }
                    double ry = (g_mutation == MUT_TREE_STALE_RESIDUAL) ? P[y] : r[y];
                    double tau = threshold(ry, Q[y]);
                    if (T > 0.0 && fabs((double)u[i] - tau) < band_eps) flag = 1;
                    if ((double)u[i] < tau) {
                        next = i;
                        break;
                    }
                    /* rejected: r becomes the normalised residual max(0, r - q) */
                    rejected = 1;
                    double Z = 0.0;
                    for (int v = 0; v < V; ++v) {
                        double e = r[v] - Q[v];
                        r[v] = e > 0.0 ? e : 0.0;
                        Z += r[v];
                    }
                    mass *= Z;
                    if (Z == 0.0) {
                        mass = 1.0;
                        for (int v = 0; v < V; ++v) r[v] = P[v];
                    } else {
                        for (int v = 0; v < V; ++v) r[v] /= Z;
                    }
                }
                if (next >= 0) {
                    out[d] = tok[next];
                    if (nodes) nodes[d] = next;
                    ++d;
                    n = next;
                    continue;
                }
                /* No child kept: draw from r (p itself when nothing was rejected). */
                if (rejected && g_mutation == MUT_SAMPLE_TARGET_AT_MISMATCH)
                    for (int v = 0; v < V; ++v) r[v] = P[v];
                double W = 0.0;
                for (int v = 0; v < V; ++v) W += r[v];
                double c_lo = 0.0, c_hi = 0.0;
                int y = inverse_cdf(r, V, W, (double)u[0], &c_lo, &c_hi);
                if (T > 0.0 && (fabs((double)u[0] - c_lo / W) < band_eps ||
                                fabs((double)u[0] - c_hi / W) < band_eps))
                    flag = 1;
                out[d] = y;
                accepted_len[b] = d;
                break;
            }
        }
        if (band) band[b] = flag;
        if (final_mass) final_mass[b] = valid ? mass : 0.0;
        free(depth); free(P); free(Q); free(r);
    }
    return bad;
}

/* Debug export: log-normaliser log sum_v exp(l_v / T_r) of each row r
 * (rows contiguous, [nrows][V]); NaN for a row with T_r <= 0. */
int svo_row_logz(int nrows, int V, int dtype, const void *logits, const float *row_temperature,
                 double *logz) {
    if (nrows < 0 || V <= 0 || (dtype != SVO_F32 && dtype != SVO_BF16)) return 1;
    if (nrows == 0) return 0;
    if (!logits || !row_temperature || !logz) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        double T = (double)row_temperature[r];
        logz[r] = T > 0.0 ? row_logz(logits, dtype, (size_t)r * (size_t)V, V, T) : NAN;
    }
    return 0;
}

/* Debug export: first argmax of each row of raw logits [nrows][V]. */
int svo_row_argmax(int nrows, int V, int dtype, const void *logits, int32_t *out) {
    if (nrows < 0 || V <= 0 || (dtype != SVO_F32 && dtype != SVO_BF16)) return 1;
    if (nrows == 0) return 0;
    if (!logits || !out) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) out[r] = row_argmax(logits, dtype, (size_t)r * (size_t)V, V);
    return 0;
}

/*
 * Commit of one verification step (section "MTP Schedule for a Single
 * Token": once acceptance is known, the next tokens are placed without the
 * host).  For each sequence in order: the first a_b + 1 entries of its
 * emitted row are appended to its history at seq_len[b] and seq_len[b]
 * grows by that count; packed_offsets[b] is the number of tokens committed
 * by the sequences before b (the total in [B]) and packed holds the
 * committed tokens in that order.  status: 0 committed, 1 refused (the row
 * is too short for a_b + 1 tokens, the length is negative, the new length
 * would pass INT32_MAX, or the history would overflow), 2 nothing to commit
 * (a_b < 0).  history may be NULL (no history and no capacity limit).
 */
int svo_commit_tokens(int B, int width, const int32_t *accepted_len, const int32_t *emitted,
                      int32_t *seq_len, int32_t *history, int history_stride,
                      int32_t *packed_offsets, int32_t *packed, int32_t *status) {
    if (B < 0 || width < 1 || history_stride < 0) return 1;
    if (B == 0) return 0;
    if (!accepted_len || !emitted || !seq_len) return 1;
    int total = 0;
    for (int b = 0; b < B; ++b) {
        const int a = accepted_len[b];
        const int len = seq_len[b];
        int n = 0, st = 0;
        if (a < 0)
            st = 2;
        else if (a >= width || len < 0 || (long long)len + a + 1 > 2147483647LL ||
                 (history && (long long)len + a + 1 > (long long)history_stride))
            st = 1;
        else
            n = a + 1;
        if (packed_offsets) packed_offsets[b] = total;
        for (int j = 0; j < n; ++j) {
            const int32_t tok = emitted[(size_t)b * width + j];
            if (history) history[(size_t)b * history_stride + len + j] = tok;
            if (packed) packed[total + j] = tok;
        }
        seq_len[b] = len + n;
        total += n;
        if (status) status[b] = st;
    }
    if (packed_offsets) packed_offsets[B] = total;
    return 0;
}
