// sv_tree_sampled.hpp -- sv_verify_tree_sampled: the tree rowstats, the walk in rounds and
// the one-workgroup walk (part of sv_kernels.hpp).
#pragma once

#include "sv_chain.hpp"

namespace sv {
// ---------------------------------------------------------------- tree: sampled ---
//
// Multi-step speculative sampling over a draft tree (SpecInfer, Miao et al.
// 2023, the rule the EAGLE work applies to sampled trees; the pages, section
// "EAGLE", keep the longest path that passes).  At node n the children are
// tested in index order against a running distribution r that starts as the
// target row p_n; a rejection replaces r by the normalised residual
// max(0, r - q_n).  That residual after j rejections is max(0, p - c_j q) /
// Z(c_j), Z(c) = sum_v max(0, p_v - c q_v), c_0 = 0, c_{j+1} = c_j + Z(c_j)
// (an exact identity: max(0, max(0, a) / Z - q) = max(0, a - Z q) / Z for
// Z > 0), so a sibling's test needs only the scalars (c, Z) and each
// rejection one pass over the node's two rows.  The passes form each term
// relative to itself (residual_term, with kappa = log2(c S_t / S_d)), in
// units of the target row's reference, so Z(c) = M / S_t for the pass's sum M
// of the terms' positive parts.  The first rejection at a node has c = 1
// exactly; its pass also corrects the node's log2(S_t / S_d) (kappa_zeta).

// Rows 0 .. B*N-1 are target rows (b, n), rows B*N .. 2*B*N-1 draft rows.
// A leaf's rows are skipped: its draft row is never needed, and its target
// row only if a walk ends at the leaf, which then computes that row's
// statistics itself.
// The wave streaming tile 0 of inner node n's draft row also gathers, for
// every child i of n, the target and draft logits of row n at i's token into
// tg[b][i] and dg[b][i] (0 for a token outside [0, V)), so that the walk's
// sibling tests need no dependent loads.
// A wave streams TPW consecutive tiles of one row, so that its parent scan,
// a dependent load ahead of the tiles, is paid once per TPW tiles.
template <int DT, bool VEC, int U, int TPW>
__global__ __launch_bounds__(kBlock) void tree_rowstats_kernel(const void* __restrict__ target,
                                                               const void* __restrict__ draft,
                                                               const int32_t* __restrict__ parent, int parent_stride,
                                                               const int32_t* __restrict__ node_tokens,
                                                               const float* __restrict__ temperature, int B, int N,
                                                               int V, int nT, Partial* __restrict__ part,
                                                               float* __restrict__ tg, float* __restrict__ dg) {
    const int64_t gw = global_wave();
    const int64_t nbn = static_cast<int64_t>(B) * N;
    const int64_t wpr = (nT + TPW - 1) / TPW;  // waves per row
    if (gw >= 2 * nbn * wpr) return;
    const int64_t r = gw / wpr;
    const int64_t tw = gw - r * wpr;
    const bool is_target = r < nbn;
    const int64_t rr = is_target ? r : r - nbn;
    const int64_t b = rr / N;
    const int n = static_cast<int>(rr - b * N);
    {
        const int32_t* par = parent + b * static_cast<int64_t>(parent_stride);
        bool kid = false;
        for (int i = n + 1 + lane_id(); i < N; i += kWave) {
            const bool child = par[i] == n;
            kid |= child;
            if (!is_target && child && tw == 0) {
                const int y = node_tokens[b * N + i];
                const bool yok = static_cast<unsigned>(y) < static_cast<unsigned>(V);
                tg[b * N + i] = yok ? load_elem<DT>(target, rr * static_cast<int64_t>(V) + y) : 0.f;
                dg[b * N + i] = yok ? load_elem<DT>(draft, rr * static_cast<int64_t>(V) + y) : 0.f;
            }
        }
        if (!__ballot(kid)) return;
    }
    const void* base = is_target ? target : draft;
    const int64_t row_elem = rr * static_cast<int64_t>(V);
    const float T = temperature[b];
#pragma unroll 1
    for (int i = 0; i < TPW; ++i) {
        const int64_t tile = tw * TPW + i;
        if (tile >= nT) break;
        const Partial p = tile_is_full<VEC, U>(tile, V, Elem<DT>::per_vec)
                              ? rowstats_tile<DT, VEC, U, VEC>(base, row_elem, V, tile, T)
                              : rowstats_tile<DT, VEC, U, false>(base, row_elem, V, tile, T);
        if (lane_id() == 0) part[r * nT + tile] = p;
    }
}

// The statistics of a leaf's target row, which tree_rowstats skips, for a
// walk that ends at the leaf: one partial per segment (a segment is one
// vector per lane), segments seg0, seg0 + stride, ... into out[segment].
template <int DT, bool VEC>
__device__ __forceinline__ void leaf_row_partials(const void* target, int64_t b, int N, int n, int V, int64_t nseg,
                                                  float T, int64_t seg0, int64_t stride, Partial* out) {
    const int64_t row_elem = (b * N + n) * static_cast<int64_t>(V);
    for (int64_t g = seg0; g < nseg; g += stride) {
        const Partial p = tile_is_full<VEC, 1>(g, V, Elem<DT>::per_vec)
                              ? rowstats_tile<DT, VEC, 1, VEC>(target, row_elem, V, g, T)
                              : rowstats_tile<DT, VEC, 1, false>(target, row_elem, V, g, T);
        if (lane_id() == 0) out[g] = p;
    }
}

// One workgroup per sequence walks its tree; each thread holds kWalkSlots
// node slots (t, t + kWalkBlock, ...).
constexpr int kWalkBlock = 512;
constexpr int kWalkWaves = kWalkBlock / kWave;
constexpr int kWalkSlots = SV_MAX_TREE_NODES / kWalkBlock;
constexpr int kWalkMaxSegs = SV_MAX_VOCAB / (4 * 64);  // f32 rows have the most segments
constexpr int kWalkUnroll = 4;                          // segments in flight per wave

// Weights of segment g of the running distribution in units of the target
// row's reference (S_t times the distribution): p when the residual scale c
// is 0, else max(0, p - c q) by residual_term (s.kappa = log2(c S_t / S_d)).
template <int DT, bool VEC>
__device__ __forceinline__ void walk_weights(const void* draft, const void* target, int64_t row, int V, int64_t g,
                                             const SeqInfo& s, bool residual, float* w) {
    segment_weights<DT, VEC>(draft, target, row, row, V, g, s, residual, s.rt, w);
}

// One full segment's mass from its raw 16-byte vectors (the same arithmetic
// as walk_weights on an unmasked segment), and for a residual its sums E and
// X (residual_sums).
template <int DT, bool RESIDUAL>
__device__ __forceinline__ ResidualSums walk_sums_raw(const uint4& rt, const uint4& rd, const SeqInfo& s) {
    constexpr int VE = Elem<DT>::per_vec;
    float vt[VE];
    unpack<DT>(rt, vt);
    if constexpr (RESIDUAL) {
        float vd[VE];
        unpack<DT>(rd, vd);
        return residual_sums<DT, VE, true>(vt, vd, s);
    } else {
        float w[VE];
        bonus_weights<VE, true>(vt, s, s.rt, w);
        return ResidualSums{pairwise_sum<VE>(w), 0.f, 0.f, 0.f};
    }
}

// The same for a segment that may reach past the row's end (masked path).
template <int DT, bool VEC, bool RESIDUAL>
__device__ __forceinline__ ResidualSums walk_sums(const void* draft, const void* target, int64_t row, int V,
                                                  int64_t g, const SeqInfo& s) {
    constexpr int VE = Elem<DT>::per_vec;
    float vt[VE];
    load_tile<DT, VEC, 1, false>(target, row, V, g, lane_id(), vt);
    if constexpr (RESIDUAL) {
        float vd[VE];
        load_tile<DT, VEC, 1, false>(draft, row, V, g, lane_id(), vd);
        return residual_sums<DT, VE, false>(vt, vd, s);
    } else {
        float w[VE];
        bonus_weights<VE, false>(vt, s, s.rt, w);
        return ResidualSums{pairwise_sum<VE>(w), 0.f, 0.f, 0.f};
    }
}

// Totals of one walk pass in units of the target row's reference: M, the
// running distribution's mass (S_t Z(c) for a residual), and for a residual
// E, X and SW (see kappa_zeta).
struct PassSums {
    double m, ea, x, sw;
};

// Every thread of the workgroup: the mass of every segment of the running
// distribution into s_mass (and, for a residual, each segment's E into
// s_ea), and the totals (fp64, in a fixed order; X summed per wave, then over
// the waves) as the return value (identical in every thread).  Segments that lie wholly inside the row are
// read kWalkUnroll per wave at a time with straight-line 16-byte loads
// (indices clamped rather than branched on, so that all loads are in flight
// together); the row's tail takes the masked path.
template <int DT, bool VEC, bool RESIDUAL>
__device__ PassSums walk_masses(const void* draft, const void* target, int64_t row, int V, int64_t nseg,
                                const SeqInfo s, float* s_mass, float* s_ea, double* s_wx, PassSums* s_sum) {
    constexpr int VE = Elem<DT>::per_vec;
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int64_t nfull = VEC ? ((V + VE - 1) / VE) / 64 : 0;
    const char* tr = static_cast<const char*>(target) + row * Elem<DT>::bytes;
    const char* dr = static_cast<const char*>(draft) + row * Elem<DT>::bytes;
    double wx = 0.0, wsw = 0.0;  // this wave's shares of X and SW (the same in every lane)
    for (int64_t g0 = wave; g0 < nfull; g0 += kWalkWaves * kWalkUnroll) {
        uint4 rt[kWalkUnroll], rd[kWalkUnroll];
#pragma unroll
        for (int j = 0; j < kWalkUnroll; ++j) {
            const int64_t g = min<int64_t>(g0 + j * kWalkWaves, nfull - 1);
            rt[j] = *reinterpret_cast<const uint4*>(tr + (g * 64 + lane) * 16);
            if constexpr (RESIDUAL) rd[j] = *reinterpret_cast<const uint4*>(dr + (g * 64 + lane) * 16);
        }
#pragma unroll
        for (int j = 0; j < kWalkUnroll; ++j) {
            const int64_t g = g0 + j * kWalkWaves;
            ResidualSums r = walk_sums_raw<DT, RESIDUAL>(rt[j], rd[j], s);
            r.m = wave_sum(r.m);
            if constexpr (RESIDUAL) {
                r.ea = wave_sum(r.ea);
                r.x = wave_sum(r.x);
                r.sw = wave_sum(r.sw);
            }
            if (g < nfull) {
                wx += static_cast<double>(r.x);
                wsw += static_cast<double>(r.sw);
                if (lane == 0) {
                    s_mass[g] = r.m;
                    s_ea[g] = r.ea;
                }
            }
        }
    }
    for (int64_t g = nfull + wave; g < nseg; g += kWalkWaves) {
        ResidualSums r = walk_sums<DT, VEC, RESIDUAL>(draft, target, row, V, g, s);
        r.m = wave_sum(r.m);
        if constexpr (RESIDUAL) {
            r.ea = wave_sum(r.ea);
            r.x = wave_sum(r.x);
            r.sw = wave_sum(r.sw);
        }
        wx += static_cast<double>(r.x);
        wsw += static_cast<double>(r.sw);
        if (lane == 0) {
            s_mass[g] = r.m;
            s_ea[g] = r.ea;
        }
    }
    if (lane == 0) {
        s_wx[wave] = wx;
        s_wx[kWalkWaves + wave] = wsw;
    }
    __syncthreads();
    if (wave == 0) {
        const int64_t per = (nseg + kWave - 1) / kWave;
        const int64_t a = min<int64_t>(nseg, lane * per), e = min<int64_t>(nseg, a + per);
        double rm = 0.0, re = 0.0;
        for (int64_t g = a; g < e; ++g) {
            rm += static_cast<double>(s_mass[g]);
            re += static_cast<double>(s_ea[g]);
        }
        double rx = 0.0, rs = 0.0;
        for (int w = 0; w < kWalkWaves; ++w) {
            rx += s_wx[w];
            rs += s_wx[kWalkWaves + w];
        }
        const PassSums tot{__shfl(wave_inclusive_scan(rm), kWave - 1, kWave),
                           __shfl(wave_inclusive_scan(re), kWave - 1, kWave), rx, rs};
        if (lane == 0) *s_sum = tot;
    }
    __syncthreads();
    return *s_sum;
}

// Validity of a tree and the depth of every node (pointer jumping over the
// parent links), as for the greedy tree: BLOCK threads with
// SV_MAX_TREE_NODES / BLOCK node slots each.  Fills s_par (parent ids, -1 for
// the root) and returns whether the tree is invalid, in every thread.
template <int BLOCK>
__device__ bool walk_validate(const int32_t* __restrict__ par, int N, int max_depth, int* s_par, int* s_anc,
                              int* s_len, int* s_bad) {
    constexpr int kWalkSlots = SV_MAX_TREE_NODES / BLOCK;
    constexpr int kWalkBlock = BLOCK;
    const int t = threadIdx.x;
    if (t == 0) *s_bad = 0;
    __syncthreads();
    int anc[kWalkSlots], len[kWalkSlots];
#pragma unroll
    for (int q = 0; q < kWalkSlots; ++q) {
        const int i = t + q * kWalkBlock;
        anc[q] = 0;
        len[q] = 0;
        if (i < N) {
            const int p = i == 0 ? 0 : par[i];
            if (i > 0 && (p < 0 || p >= i)) *s_bad = 1;
            s_par[i] = i == 0 ? -1 : p;
            anc[q] = p;
            len[q] = i == 0 ? 0 : 1;
        }
    }
    __syncthreads();
    if (!*s_bad) {
#pragma unroll
        for (int q = 0; q < kWalkSlots; ++q) {
            const int i = t + q * kWalkBlock;
            if (i < N) {
                s_anc[i] = anc[q];
                s_len[i] = len[q];
            }
        }
        __syncthreads();
        for (int step = 1; step < N; step <<= 1) {
            int a2[kWalkSlots], l2[kWalkSlots];
#pragma unroll
            for (int q = 0; q < kWalkSlots; ++q) {
                const bool in = t + q * kWalkBlock < N;
                a2[q] = in ? s_anc[anc[q]] : 0;
                l2[q] = in ? s_len[anc[q]] : 0;
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < kWalkSlots; ++q) {
                const int i = t + q * kWalkBlock;
                if (i < N) {
                    len[q] += l2[q];
                    anc[q] = a2[q];
                    s_anc[i] = anc[q];
                    s_len[i] = len[q];
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int q = 0; q < kWalkSlots; ++q)
            if (t + q * kWalkBlock < N && len[q] > max_depth) *s_bad = 1;
    }
    __syncthreads();
    return *s_bad != 0;
}

// State of one sequence's walk between the round launches (double-buffered).
enum WalkPhase : int {
    kWalkEnter = 0,  // at the start of `node`: its statistics are still to be combined
    kWalkTest = 1,   // testing `node`'s children from rank kidx on (only inside a round)
    kWalkPass = 2,   // a rejection advanced c; the partial sums of Z(c) are in z
    kWalkPick = 3,   // the final distribution's segment masses are written; the pick remains
    kWalkDone = 4,
    kWalkStuck = 5,  // a case the rounds leave to the one-workgroup walk (an empty final residual)
    kWalkLeaf = 6    // at leaf `node`, whose target-row statistics the last round computed
};

// Normalisers of a node's target and draft rows, as the walk combines them
// from the row partials: reference exponent and sum of each softmax (at
// temperature 0 the two argmax indices).  A leaf's draft row is never
// streamed; its entries are rd = 0, sd = 1 and go unused.
struct alignas(8) NodeNorm {
    int rt, rd;
    double st, sd;
};

struct alignas(16) WalkState {
    int phase, node, depth, kidx;  // kidx: children of `node` already rejected
    int Rt, Rd;                    // node statistics (at temperature 0: the two argmaxes)
    int redone;                    // the pending pass at c = 1 was formed with the corrected K
    int pad;
    double St;                     // target row's normaliser in the reference Rt
    double K;                      // log2(S_t / S_d) in the reference Rt (corrected by the first pass)
    double c, Z;
};

// log2(S_t / S_d) of a node's two rows with both normalisers in the
// reference of the target row.
__device__ __forceinline__ double node_log_ratio(int Rt, int Rd, double St, double Sd) {
    return static_cast<double>(Rt - Rd) + (log2(St) - log2(Sd));
}

// The descriptor of a walk's weights at a node: the target row's reference
// and, for a residual (c > 0), kappa = log2(c S_t / S_d).
__device__ __forceinline__ SeqInfo walk_info(float T, int Rt, double St, double K, double c) {
    SeqInfo s{};
    temperature_scale(T > 0.f ? T : 1.f, s);
    s.rt = static_cast<float>(Rt);
    s.st = static_cast<float>(St);
    if (c > 0.0) set_kappa(s, K + log2(c));
    return s;
}

// The final draw of a walk that stopped at st.node, from the segment masses m
// of its final distribution (written by the last round): one wave.  Returns
// false, with y untouched, when the masses sum to zero (an empty residual).
template <int DT, bool VEC>
__device__ bool pick_from_masses(const void* draft, const void* target, int64_t b, int N, int V, float T,
                                 const WalkState& st, const float* m, float u, int& y) {
    constexpr int VE = Elem<DT>::per_vec;
    const int lane = lane_id();
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    const SeqInfo s = walk_info(T, st.Rt, st.St, st.K, st.c);
    const int64_t per = (nseg + kWave - 1) / kWave;
    const int64_t a0 = min<int64_t>(nseg, lane * per), a1 = min<int64_t>(nseg, a0 + per);
    const double W = __shfl(wave_inclusive_scan(run_sum(m, a0, a1, nseg)), kWave - 1, kWave);
    if (!(W > 0.0)) return false;
    const int64_t row = (b * N + st.node) * static_cast<int64_t>(V);
    y = pick_from_masses_f<DT, VEC>(draft, target, row, row, V, nseg, s, st.c > 0.0, m, static_cast<double>(u));
    return true;
}

// The walk's last launch, one workgroup per sequence.  It returns at once
// for a sequence the rounds finished, draws the final token of one whose
// last round wrote its final masses, and otherwise goes on from the state the
// last round left, on one CU: the pending rejection pass (formed here from
// the rows), the remaining children's tests and passes, the nodes below, and
// the final draw.  The paths the rounds wrote stay.  A final residual with no
// mass falls back to the node's target row.  With no state (state ==
// nullptr) it walks from the root and checks the tree itself.
template <int DT, bool VEC>
__global__ __launch_bounds__(kWalkBlock) void tree_sample_kernel(
    const int32_t* __restrict__ node_tokens, const int32_t* __restrict__ parent, int parent_stride, int N,
    int max_depth, const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, int B, int V, int nT,
    const Partial* __restrict__ part, const WalkState* __restrict__ state, const float* __restrict__ tsegs,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ emitted, int32_t* __restrict__ accepted_nodes) {
    constexpr int VE = Elem<DT>::per_vec;
    WalkState st{};
    bool from_p = false;  // the final residual at st.node was empty: draw from its target row
    if (state != nullptr) {
        st = state[blockIdx.x];
        if (st.phase == kWalkDone) return;  // finished by the rounds
        if (st.phase == kWalkPick) {
            // the rounds left only the final draw: its segment masses are written
            __shared__ int s_picked;
            const int64_t b = blockIdx.x;
            if (threadIdx.x < kWave) {
                const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
                int y = -1;
                const bool ok = pick_from_masses<DT, VEC>(draft, target, b, N, V, temperature[b], st,
                                                          tsegs + b * nseg, uniforms[b * N], y);
                if (lane_id() == 0) {
                    s_picked = ok;
                    if (ok) {
                        emitted[b * (max_depth + 1) + st.depth] = y;
                        accepted_len[b] = st.depth;
                    }
                }
            }
            __syncthreads();
            if (s_picked) return;
            from_p = true;
        }
        if (st.phase == kWalkStuck) from_p = true;
    }
    __shared__ int s_par[SV_MAX_TREE_NODES];
    __shared__ int s_anc[SV_MAX_TREE_NODES];
    __shared__ int s_len[SV_MAX_TREE_NODES];
    __shared__ uint64_t s_kids[SV_MAX_TREE_NODES / kWave];
    __shared__ float s_mass[kWalkMaxSegs];
    __shared__ float s_ea[kWalkMaxSegs];
    __shared__ double s_wx[2 * kWalkWaves];
    // the current node's children in index order: node id, uniform, and the
    // target and draft logits at the child's token
    __shared__ int s_cid[SV_MAX_TREE_NODES];
    __shared__ float s_cu[SV_MAX_TREE_NODES];
    __shared__ float s_clt[SV_MAX_TREE_NODES];
    __shared__ float s_cld[SV_MAX_TREE_NODES];
    __shared__ PassSums s_sum;
    __shared__ double s_norm[2];  // S_t, S_d of the current node
    __shared__ int s_ref[2];      // R_t, R_d (at temperature 0: the two argmaxes)
    __shared__ int s_bad, s_accept;
    __shared__ Partial s_lp[kWalkMaxSegs];  // a leaf's target-row statistics, per segment
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = lane_id();
    const int wave = t / kWave;
    const int width = max_depth + 1;
    const float T = temperature[b];
    const bool sampled = T > 0.f;
    int32_t* out = emitted + b * width;
    int32_t* nodes = accepted_nodes ? accepted_nodes + b * width : nullptr;

    // validity and depths (pointer jumping), as for the greedy tree; after the
    // rounds (which checked the tree) only the parent links are needed
    const bool bad = walk_validate<kWalkBlock>(parent + b * static_cast<int64_t>(parent_stride), N, max_depth, s_par,
                                               s_anc, s_len, &s_bad);
    if (state == nullptr) {
        for (int j = t; j < width; j += kWalkBlock) {
            out[j] = -1;
            if (nodes) nodes[j] = -1;
        }
        if (bad) {
            if (t == 0) accepted_len[b] = -1;
            return;
        }
    }

    const double cT = kLog2e / static_cast<double>(sampled ? T : 1.f);
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    const int nmask = (N + kWave - 1) / kWave;
    const int64_t nbn = static_cast<int64_t>(B) * N;
    // where the walk goes on: the state's node, with its statistics, c, Z and
    // the children already rejected when a pass is pending (or the final
    // residual was empty); entered afresh otherwise
    int n = st.node, d = st.depth;
    bool resumed = state != nullptr && (from_p || st.phase == kWalkPass);
    bool pending = resumed && !from_p;
    int Rt = st.Rt, Rd = st.Rd, k0 = st.kidx, redone = st.redone;
    double St = st.St, K = st.K, c = st.c, Z = st.Z;
    for (;;) {
        const int64_t row = (b * N + n) * static_cast<int64_t>(V);
        // children of n, and the statistics of its target and draft rows
#pragma unroll
        for (int q = 0; q < kWalkSlots; ++q) {
            const int i = t + q * kWalkBlock;
            const uint64_t km = __ballot(i < N && s_par[i] == n);
            if (lane == 0 && wave + q * kWalkWaves < nmask) s_kids[wave + q * kWalkWaves] = km;
        }
        __syncthreads();
        // every child reads its own token, uniform and the two logits at that token
        int nkids = 0;
        for (int m = 0; m < nmask; ++m) nkids += __popcll(s_kids[m]);
#pragma unroll
        for (int q = 0; q < kWalkSlots; ++q) {
            const int i = t + q * kWalkBlock;
            const int m = i / kWave;
            if (i < N && ((s_kids[m] >> (i % kWave)) & 1)) {
                int rank = __popcll(s_kids[m] & ((uint64_t{1} << (i % kWave)) - 1));
                for (int m2 = 0; m2 < m; ++m2) rank += __popcll(s_kids[m2]);
                const int y = node_tokens[b * N + i];
                const bool yok = static_cast<unsigned>(y) < static_cast<unsigned>(V);
                s_cid[rank] = yok ? i : -1 - i;  // an id outside [0, V) is rejected
                s_cu[rank] = uniforms[b * N + i];
                s_clt[rank] = yok ? load_elem<DT>(target, row + y) : 0.f;
                s_cld[rank] = yok ? load_elem<DT>(draft, row + y) : 0.f;
            }
        }
        if (!resumed) {
            // a leaf's target row was skipped by tree_rowstats: its statistics here
            const bool leaf = nkids == 0;
            if (leaf) {
                leaf_row_partials<DT, VEC>(target, b, N, n, V, nseg, T, wave, kWalkWaves, s_lp);
                __syncthreads();
            }
            if (wave == 0) {
                const bool is_draft = lane >= 32;
                const bool valid = !(leaf && is_draft);  // a leaf's draft row is never needed
                const Partial* pr = leaf ? s_lp : part + ((is_draft ? nbn : 0) + b * N + n) * nT;
                const int cnt = leaf ? static_cast<int>(nseg) : nT;
                Partial q[kBatch];
                group_load(pr, cnt, 32, valid, q);
                int r;
                double sum;
                ArgMax am;
                if (sampled) {
                    group_reduce<true>(pr, cnt, 32, valid, q, r, sum, am);
                } else {
                    group_reduce<false>(pr, cnt, 32, valid, q, r, sum, am);
                    r = am.idx;
                }
                if ((lane & 31) == 0) {
                    s_ref[is_draft] = r;
                    s_norm[is_draft] = sum;
                }
            }
            __syncthreads();
            Rt = s_ref[0];
            Rd = s_ref[1];
            St = s_norm[0];
            // log2(S_t / S_d), corrected by the first rejection's pass
            K = sampled && nkids > 0 ? node_log_ratio(Rt, Rd, St, s_norm[1]) : 0.0;
            c = 0.0;
            Z = 1.0;
            k0 = 0;
            redone = 0;
            __syncthreads();  // s_ref and s_norm are reused at the next node
        }
        resumed = false;
        // a rejection's pass at the advanced c: Z(c) = M / S_t from the segment
        // masses of max(0, p - c q) (left in s_mass for a final draw).  The
        // node's first (c = 1) corrects log2(S_t / S_d) and the masses to first
        // order, or forms them again with the corrected value, unless the
        // rounds already formed this pass again
        auto rejection_pass = [&]() {
            if (sampled) {
                PassSums ps = walk_masses<DT, VEC, true>(draft, target, row, V, nseg, walk_info(T, Rt, St, K, c),
                                                          s_mass, s_ea, s_wx, &s_sum);
                if (c == 1.0) {
                    const double zeta = kappa_zeta(ps.x, St);
                    K += zeta / kLn2;
                    const double Mc = ps.m - zeta * (ps.ea - ps.m);
                    if (redone || correction_trusted(zeta, ps.sw, Mc)) {
                        for (int64_t g = t; g < nseg; g += kWalkBlock) {
                            const double m = static_cast<double>(s_mass[g]);
                            s_mass[g] = static_cast<float>(fmax(0.0, m - zeta * (static_cast<double>(s_ea[g]) - m)));
                        }
                        __syncthreads();
                        if (wave == 0) {
                            const int64_t per = (nseg + kWave - 1) / kWave;
                            const int64_t a = min<int64_t>(nseg, lane * per), e = min<int64_t>(nseg, a + per);
                            double rm = 0.0;
                            for (int64_t g = a; g < e; ++g) rm += static_cast<double>(s_mass[g]);
                            rm = __shfl(wave_inclusive_scan(rm), kWave - 1, kWave);
                            if (lane == 0) s_sum.m = rm;
                        }
                        __syncthreads();
                        ps.m = s_sum.m;
                    } else {
                        ps = walk_masses<DT, VEC, true>(draft, target, row, V, nseg, walk_info(T, Rt, St, K, c),
                                                        s_mass, s_ea, s_wx, &s_sum);
                    }
                    redone = 0;
                }
                Z = ps.m / St;
            } else {
                Z = Rt != Rd ? 1.0 : fmax(0.0, 1.0 - c);
            }
            if (!(Z > 0.0)) {
                c = 0.0;
                Z = 1.0;
            }
        };
        int next = -1;
        if (from_p) {
            from_p = false;
            c = 0.0;
            Z = 1.0;
        } else {
            if (pending) {
                pending = false;
                rejection_pass();
            }
            for (int k = k0; k < nkids && next < 0; ++k) {
                if (t == 0) {
                    const int id = s_cid[k];
                    double tau = 0.0;
                    if (id >= 0) {
                        if (sampled) {
                            // p/q = exp2((l_t - l_d) c - log2(S_t / S_d))
                            const double lt = s_clt[k], ld = s_cld[k];
                            const double l2ratio = (lt - ld) * cT - K;
                            tau = fmin(1.0, fmax(0.0, exp2(l2ratio) - c) / Z);
                        } else {
                            const int y = node_tokens[b * N + id];
                            const double pv = y == Rt ? 1.0 : 0.0, qv = y == Rd ? 1.0 : 0.0;
                            const double rv = fmax(0.0, pv - c * qv) / Z;
                            tau = qv > 0.0 ? fmin(1.0, rv / qv) : (rv > 0.0 ? 1.0 : 0.0);
                        }
                    }
                    s_accept = static_cast<double>(s_cu[k]) < tau;
                }
                __syncthreads();
                if (s_accept) {
                    next = s_cid[k];
                } else {
                    // rejected: the residual becomes max(0, p - (c + Z) q) / Z(c + Z)
                    c += Z;
                    rejection_pass();
                }
                __syncthreads();
            }
        }
        if (next >= 0) {
            if (t == 0) {
                out[d] = node_tokens[b * N + next];
                if (nodes) nodes[d] = next;
            }
            ++d;
            n = next;
            continue;
        }
        // no child kept: the final token from max(0, p - c q) (p when c == 0)
        int y;
        if (!sampled) {
            y = Rt;  // one-hot p; with c > 0 the residual is p itself or empty (then p)
        } else {
            // a residual's segment masses are the last pass's (corrected at c = 1)
            const bool residual = c > 0.0;
            const SeqInfo s = walk_info(T, Rt, St, K, c);
            if (!residual) walk_masses<DT, VEC, false>(draft, target, row, V, nseg, s, s_mass, s_ea, s_wx, &s_sum);
            y = 0;
            if (wave == 0)
                y = pick_from_masses_f<DT, VEC>(draft, target, row, row, V, nseg, s, residual, s_mass,
                                                static_cast<double>(uniforms[b * N]));
        }
        if (t == 0) {
            out[d] = y;
            accepted_len[b] = d;
        }
        return;
    }
}

// The walk in rounds.  tree_sample runs each sequence's rejection passes on
// one CU, where a pass over two rows is VALU-bound (two exps and about ten
// more operations per element).  The rounds spread every pass over P
// workgroups per sequence and use the kernel boundaries between launches as
// the synchronisation: in every round each of a sequence's workgroups
// replays the same deterministic tests from the round's input state (the
// children's logits were gathered by tree_rowstats), up to the next
// rejection, and computes its slice of Z(c) = sum_v max(0, p - c q); one
// round later the slices are summed (in a fixed order) and the tests go on.
// When no child is kept, each workgroup writes its slice's segment masses of
// the final distribution and the next round's chunk 0 picks the token.
// Chunk 0 writes the outputs and the next state.  Round 0 also checks each
// tree (invalid trees give -1 outputs) and sets the outputs to -1.  When a
// sequence has at most one node per wave of its workgroups (N <= 4 P), round
// 0 also combines the normalisers of every node, one node per wave, so that
// from round 1 on a round reads all its inputs in one round trip and entering
// a child needs no dependent load; otherwise every entry combines the node's
// partials.  After the launched rounds, tree_sample draws the final token of
// a sequence whose last round wrote its final masses, and goes on with any
// other unfinished walk from the state its last round left.
//
// A walk needs one round per rejection pass, one per leaf it enters and one
// for its final draw's masses, then its pick: kWalkRounds rounds make up to
// seven of these, and the pick of a walk that needs all seven comes in
// tree_sample.  The number of passes depends on the outcome, which stays on
// the device, so the launches cannot follow it; a longer walk finishes on one
// CU in tree_sample.
constexpr int kRoundBlock = 256;
constexpr int kRoundWaves = kRoundBlock / kWave;
constexpr int kRoundSlots = SV_MAX_TREE_NODES / kRoundBlock;
constexpr int kWalkRounds = 7;

template <int DT, bool VEC>
__global__ __launch_bounds__(kRoundBlock) void tree_round_kernel(
    const int32_t* __restrict__ node_tokens, const int32_t* __restrict__ parent, int parent_stride, int N,
    int max_depth, const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, int B, int V, int nT,
    const Partial* __restrict__ part, const float* __restrict__ tg, const float* __restrict__ dg,
    const WalkState* __restrict__ st_in, WalkState* __restrict__ st_out, const double* __restrict__ z_in,
    double* __restrict__ z_out, float* __restrict__ tsegs, NodeNorm* __restrict__ norm,
    Partial* __restrict__ leafpart, int P, int first,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ emitted, int32_t* __restrict__ accepted_nodes) {
    constexpr int VE = Elem<DT>::per_vec;
    __shared__ int s_par[SV_MAX_TREE_NODES];
    __shared__ int s_anc[SV_MAX_TREE_NODES];
    __shared__ int s_len[SV_MAX_TREE_NODES];
    __shared__ int s_bad;
    __shared__ int s_tok[SV_MAX_TREE_NODES];
    __shared__ float s_u[SV_MAX_TREE_NODES];
    __shared__ float s_tg[SV_MAX_TREE_NODES];
    __shared__ float s_dg[SV_MAX_TREE_NODES];
    __shared__ uint64_t s_kids[SV_MAX_TREE_NODES / kWave];
    __shared__ double s_norm[2];
    __shared__ int s_ref[2];
    __shared__ double s_wsum[kRoundWaves][4];
    __shared__ double s_z[4];
    __shared__ int s_accept;
    const int64_t b = blockIdx.x / P;
    const int j = static_cast<int>(blockIdx.x - b * P);
    const int t = threadIdx.x;
    const int lane = lane_id();
    const int wave = t / kWave;
    const bool lead = j == 0;  // chunk 0 writes the outputs and the next state
    const int width = max_depth + 1;
    int32_t* out = emitted + b * width;
    int32_t* nodes = accepted_nodes ? accepted_nodes + b * width : nullptr;
    const int64_t nbn = static_cast<int64_t>(B) * N;
    const int32_t* par = parent + b * static_cast<int64_t>(parent_stride);
    // every input of the round first (none depends on another): the
    // sequence's temperature and walk state, the tree, the tokens, uniforms
    // and gathered logits of every node, the pending pass's partial sums and,
    // after round 0, the node normalisers
    const float T = temperature[b];
    WalkState st{};
    if (!first) st = st_in[b];
    int r_par[kRoundSlots], r_tok[kRoundSlots];
    float r_u[kRoundSlots], r_tg[kRoundSlots], r_dg[kRoundSlots];
    NodeNorm r_nrm[kRoundSlots];
    const bool cached = N <= kRoundWaves * P;  // node normalisers combined in round 0
#pragma unroll
    for (int q = 0; q < kRoundSlots; ++q) {
        const int i = t + q * kRoundBlock;
        if (i < N) {
            r_par[q] = i == 0 ? -1 : par[i];
            r_tok[q] = node_tokens[b * N + i];
            r_u[q] = uniforms[b * N + i];
            r_tg[q] = tg[b * N + i];
            r_dg[q] = dg[b * N + i];
            if (cached && !first) r_nrm[q] = norm[b * N + i];
        }
    }
    // the pending pass's slice sums M, E, X, SW (see walk_masses)
    double zz[4] = {0.0, 0.0, 0.0, 0.0};
    if (!first && wave == 0)
        for (int q = lane; q < P; q += kWave)
#pragma unroll
            for (int e = 0; e < 4; ++e) zz[e] += z_in[(b * P + q) * 4 + e];
    const bool sampled = T > 0.f;
    if (first) {
        // with the cache: node j + (3 - wave) P of this workgroup, if any, is
        // combined by this wave (lanes 0-31 the target row, 32-63 the draft
        // row), its partials in flight while the tree is checked
        const int i = j + (kRoundWaves - 1 - wave) * P;
        const bool mine = cached && i < N;
        const bool is_draft = lane >= 32;
        const Partial* rows = part + ((is_draft ? nbn : 0) + b * N + (mine ? i : 0)) * nT;
        Partial qv[kBatch];
        if (mine) group_load(rows, nT, 32, true, qv);
        const bool bad = walk_validate<kRoundBlock>(par, N, max_depth, s_par, s_anc, s_len, &s_bad);
        if (mine && !bad) {
            int r;
            double sum;
            ArgMax am;
            if (sampled) {
                group_reduce<true>(rows, nT, 32, true, qv, r, sum, am);
            } else {
                group_reduce<false>(rows, nT, 32, true, qv, r, sum, am);
                r = am.idx;
            }
            bool kid = false;
            for (int m = lane & 31; m < N; m += 32) kid |= s_par[m] == i;
            const bool inner = (__ballot(kid) >> 32) != 0;
            if (lane == 0) {
                norm[b * N + i].rt = r;
                norm[b * N + i].st = sum;
            } else if (lane == 32) {
                norm[b * N + i].rd = inner ? r : 0;
                norm[b * N + i].sd = inner ? sum : 1.0;
            }
        }
        if (lead) {
            for (int q = t; q < width; q += kRoundBlock) {
                out[q] = -1;
                if (nodes) nodes[q] = -1;
            }
        }
        __syncthreads();  // the -1s before any path write of this workgroup
        st.phase = bad ? kWalkDone : kWalkEnter;
        st.Z = 1.0;
        if (bad && lead && t == 0) accepted_len[b] = -1;
    }
    if (st.phase == kWalkDone || st.phase == kWalkStuck) {
        if (lead && t == 0) st_out[b] = st;
        return;
    }
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;

    if (st.phase == kWalkPick) {
        // the final distribution's masses were written last round: wave 0 of chunk 0 draws the token
        if (lead && wave == 0) {
            int y = -1;
            if (pick_from_masses<DT, VEC>(draft, target, b, N, V, T, st, tsegs + b * nseg,
                                          uniforms[b * N], y)) {
                if (lane == 0) {
                    out[st.depth] = y;
                    accepted_len[b] = st.depth;
                }
                st.phase = kWalkDone;
            } else {
                st.phase = kWalkStuck;  // an empty residual: the one-workgroup walk falls back to p
            }
            if (lane == 0) st_out[b] = st;
        }
        return;
    }

#pragma unroll
    for (int q = 0; q < kRoundSlots; ++q) {
        const int i = t + q * kRoundBlock;
        if (i < N) {
            if (!first) s_par[i] = r_par[q];  // round 0: filled by the tree check
            s_tok[i] = r_tok[q];
            s_u[i] = r_u[q];
            s_tg[i] = r_tg[q];
            s_dg[i] = r_dg[q];
        }
    }
    if (st.phase == kWalkPass && wave == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            zz[e] = wave_sum(zz[e]);
            if (lane == 0) s_z[e] = zz[e];
        }
    }
    __syncthreads();
    int n = st.node, d = st.depth, kidx = st.kidx, Rt = st.Rt, Rd = st.Rd, redone = st.redone;
    double St = st.St, K = st.K, c = st.c, Z = st.Z;
    int phase = st.phase;
    bool redo = false;  // form the pending pass again, with the corrected K, this round
    if (phase == kWalkPass) {
        double M = s_z[0];
        if (c == 1.0) {
            // the node's first rejection: correct log2(S_t / S_d) and, to first
            // order, the pass's mass; or, when that order is not trusted, form
            // the pass again with the corrected value (once)
            const double zeta = kappa_zeta(s_z[2], St);
            K += zeta / kLn2;
            M -= zeta * (s_z[1] - M);
            redo = !redone && !correction_trusted(zeta, s_z[3], M);
            redone = redo;
        }
        if (!redo) {
            Z = M / St;
            if (!(Z > 0.0)) {
                c = 0.0;
                Z = 1.0;
            }
            phase = kWalkTest;
        }
    }
    const double cT = kLog2e / static_cast<double>(sampled ? T : 1.f);
    const int nmask = (N + kWave - 1) / kWave;
    bool leaf_now = false;
    while (!redo) {
#pragma unroll
        for (int q = 0; q < kRoundSlots; ++q) {
            const int i = t + q * kRoundBlock;
            const uint64_t km = __ballot(i < N && s_par[i] == n);
            if (lane == 0 && wave + q * kRoundWaves < nmask) s_kids[wave + q * kRoundWaves] = km;
        }
        __syncthreads();
        int nkids = 0;
        for (int m = 0; m < nmask; ++m) nkids += __popcll(s_kids[m]);
        if (phase == kWalkEnter && nkids == 0) {
            // a leaf: tree_rowstats skipped its target row, whose statistics are
            // computed below, the combination follows next round
            phase = kWalkLeaf;
            leaf_now = true;
            break;
        }
        if (phase == kWalkEnter || phase == kWalkLeaf) {
            const bool leaf = phase == kWalkLeaf;
            if (cached && !first && !leaf) {
                // combined in round 0; the thread holding node n shares them
#pragma unroll
                for (int q = 0; q < kRoundSlots; ++q) {
                    if (t + q * kRoundBlock == n) {
                        s_ref[0] = r_nrm[q].rt;
                        s_ref[1] = r_nrm[q].rd;
                        s_norm[0] = r_nrm[q].st;
                        s_norm[1] = r_nrm[q].sd;
                    }
                }
            } else if (wave == 0) {
                const bool is_draft = lane >= 32;
                const bool valid = !(leaf && is_draft);  // a leaf's draft row is never needed
                const Partial* pr = leaf ? leafpart + b * nseg : part + ((is_draft ? nbn : 0) + b * N + n) * nT;
                const int cnt = leaf ? static_cast<int>(nseg) : nT;
                Partial qv[kBatch];
                group_load(pr, cnt, 32, valid, qv);
                int r;
                double sum;
                ArgMax am;
                if (sampled) {
                    group_reduce<true>(pr, cnt, 32, valid, qv, r, sum, am);
                } else {
                    group_reduce<false>(pr, cnt, 32, valid, qv, r, sum, am);
                    r = am.idx;
                }
                if ((lane & 31) == 0) {
                    s_ref[is_draft] = r;
                    s_norm[is_draft] = sum;
                }
            }
            __syncthreads();
            Rt = s_ref[0];
            Rd = s_ref[1];
            St = s_norm[0];
            // log2(S_t / S_d) (a leaf's draft row is never read: Rd = 0, S_d = 1)
            K = sampled ? node_log_ratio(Rt, Rd, St, s_norm[1]) : 0.0;
            c = 0.0;
            Z = 1.0;
            kidx = 0;
            redone = 0;
            phase = kWalkTest;
            __syncthreads();  // s_ref and s_norm are reused at the next node
        }
        int next = -1, rank = 0;
        bool pass = false;
        for (int m = 0; m < nmask && next < 0 && !pass; ++m) {
            uint64_t kids = s_kids[m];
            while (kids && next < 0 && !pass) {
                const int i = m * kWave + __builtin_ctzll(kids);
                kids &= kids - 1;
                if (rank++ < kidx) continue;  // rejected in an earlier round
                if (t == 0) {
                    const int y = s_tok[i];
                    double tau = 0.0;
                    if (static_cast<unsigned>(y) < static_cast<unsigned>(V)) {
                        if (sampled) {
                            // p/q = exp2((l_t - l_d) c - log2(S_t / S_d))
                            const double l2ratio =
                                (static_cast<double>(s_tg[i]) - static_cast<double>(s_dg[i])) * cT - K;
                            tau = fmin(1.0, fmax(0.0, exp2(l2ratio) - c) / Z);
                        } else {
                            const double pv = y == Rt ? 1.0 : 0.0, qv = y == Rd ? 1.0 : 0.0;
                            const double rv = fmax(0.0, pv - c * qv) / Z;
                            tau = qv > 0.0 ? fmin(1.0, rv / qv) : (rv > 0.0 ? 1.0 : 0.0);
                        }
                    }
                    s_accept = static_cast<double>(s_u[i]) < tau;
                }
                __syncthreads();
                const bool accepted = s_accept;
                __syncthreads();  // s_accept is reused by the next test
                if (accepted) {
                    next = i;
                } else {
                    // rejected: the residual becomes max(0, p - (c + Z) q) / Z(c + Z)
                    c += Z;
                    kidx = rank;
                    if (sampled) {
                        pass = true;
                    } else {
                        Z = Rt != Rd ? 1.0 : fmax(0.0, 1.0 - c);
                        if (!(Z > 0.0)) {
                            c = 0.0;
                            Z = 1.0;
                        }
                    }
                }
            }
        }
        if (next >= 0) {
            if (lead && t == 0) {
                out[d] = s_tok[next];
                if (nodes) nodes[d] = next;
            }
            ++d;
            n = next;
            phase = kWalkEnter;
            continue;
        }
        if (pass) {
            phase = kWalkPass;
        } else if (!sampled) {
            // one-hot p: the final token is its argmax
            if (lead && t == 0) {
                out[d] = Rt;
                accepted_len[b] = d;
            }
            phase = kWalkDone;
        } else {
            phase = kWalkPick;  // the masses are written below, the pick comes next round
        }
        break;
    }
    if (leaf_now) {
        // the sequence's workgroups compute the leaf's target-row statistics,
        // this one its share of the segments
        leaf_row_partials<DT, VEC>(target, b, N, n, V, nseg, T, static_cast<int64_t>(j) * kRoundWaves + wave,
                                   static_cast<int64_t>(P) * kRoundWaves, leafpart + b * nseg);
    }
    if (phase == kWalkPass || phase == kWalkPick) {
        // this workgroup's slice of the segments of node n's rows
        const int64_t row = (b * N + n) * static_cast<int64_t>(V);
        const SeqInfo s = walk_info(T, Rt, St, K, c);
        const bool residual = c > 0.0;
        const int64_t spc = (nseg + P - 1) / P;
        const int64_t g0 = j * spc, g1 = min<int64_t>(nseg, g0 + spc);
        double acc[4] = {0.0, 0.0, 0.0, 0.0};
        for (int64_t g = g0 + wave; g < g1; g += kRoundWaves) {
            const ResidualSums r = residual ? walk_sums<DT, VEC, true>(draft, target, row, V, g, s)
                                            : walk_sums<DT, VEC, false>(draft, target, row, V, g, s);
            const float m = wave_sum(r.m);
            if (phase == kWalkPick) {
                if (lane == 0) tsegs[b * nseg + g] = m;
            } else {
                acc[0] += static_cast<double>(m);
                acc[1] += static_cast<double>(wave_sum(r.ea));
                acc[2] += static_cast<double>(wave_sum(r.x));
                acc[3] += static_cast<double>(wave_sum(r.sw));
            }
        }
        if (phase == kWalkPass) {
            if (lane == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) s_wsum[wave][e] = acc[e];
            __syncthreads();
            if (t < 4) {
                double z = 0.0;
                for (int w = 0; w < kRoundWaves; ++w) z += s_wsum[w][t];
                z_out[(b * P + j) * 4 + t] = z;
            }
        }
    }
    if (lead && t == 0) {
        st.phase = phase;
        st.node = n;
        st.depth = d;
        st.kidx = kidx;
        st.Rt = Rt;
        st.Rd = Rd;
        st.St = St;
        st.K = K;
        st.redone = redone;
        st.c = c;
        st.Z = Z;
        st_out[b] = st;
    }
}

}  // namespace sv
