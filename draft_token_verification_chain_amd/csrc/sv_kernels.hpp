// sv_kernels.hpp -- gfx950 kernels of libspecverify.
//
// Pipeline of sv_verify_chain (one stream, no host synchronisation):
//   rowstats   streams the k target rows and k draft rows of every sequence
//              once; one wave64 per (row, tile) writes a softmax partial
//              (sum of exp2 against an integer reference) or, for rows at
//              temperature 0, the (max, lowest index) of the tile;
//   accept     one wave per sequence: combines the row partials, gathers the
//              2k logits at the draft tokens, forms tau_i in the log domain,
//              takes the first rejection with a ballot, writes the accepted
//              prefix and a descriptor of the final draw -- inside every
//              final_part workgroup for small draws, as its own kernel for
//              large ones, not at all without drafts;
//   final_part streams only the row(s) the final draw needs (target and draft
//              row a at a rejection, target row k after full acceptance) and
//              writes the residual mass of every 64-vector segment;
//   final_pick one wave per sequence: prefix over the segment masses, picks
//              the segment holding u * W and rescans only that segment to find
//              the token.
// sv_verify_greedy and sv_verify_tree use argmax_rows (the streaming argmax)
// followed by a per-sequence finaliser.  sv_verify_tree_sampled streams the
// tree's rows (tree_rowstats), then walks every tree in rounds of launches
// (tree_round), with a one-workgroup walk (tree_sample) for what the rounds
// leave.  sv_commit_tokens is one workgroup (commit_tokens).
//
// Scheme: "Accelerating Sonar through speculation" (Perplexity, 2025),
// sections "Speculative decoding", "Target-Draft" and "EAGLE"; acceptance
// and residual rule of Leviathan et al., first in that page's references;
// sampled trees: multi-step speculative sampling (SpecInfer, Miao et al.).
#pragma once

#include "sv_common.hpp"

namespace sv {

constexpr double kLog2e = 1.4426950408889634073599246810019;

enum FinalMode : int {
    kFinalDone = 0,      // nothing left to draw (temperature 0, rejection inside the draft)
    kFinalResidual = 1,  // draw from max(0, p - q) at the rejected position
    kFinalBonus = 2,     // draw from the target's row k (all drafts accepted)
    kFinalArgmax = 3     // temperature 0, all accepted: argmax of target row k
};

// What the final draw of one sequence needs.
struct SeqInfo {
    int mode;
    int a;         // accepted drafts; the final token goes to emitted[b][a]
    float rt;      // target row a: integer reference of its normaliser
    float inv_st;  //               1 / sum exp2(l c - rt)
    float rd;      // draft row a: the same
    float inv_sd;
    float c_hi;    // log2(e) / T as a double-float pair
    float c_lo;
    float u;       // u[b][k]
    int pad[3];
};

// log2 of a positive double with an exact exponent and an fp32 log2 of the
// mantissa in [0.5, 1): absolute error about 1.5e-7, far below the 1e-5 band
// within which acceptance decisions are allowed to differ.
__device__ __forceinline__ double log2_of_sum(double x) {
    int e;
    const double m = frexp(x, &e);
    return static_cast<double>(e) + static_cast<double>(log2f(static_cast<float>(m)));
}

__device__ __forceinline__ void temperature_scale(float T, float& c_hi, float& c_lo) {
    const double c = kLog2e / static_cast<double>(T);
    c_hi = static_cast<float>(c);
    c_lo = static_cast<float>(c - static_cast<double>(c_hi));
}

// ---------------------------------------------------------------- wave tiles ---

// Softmax partial of one tile whose logits are loaded: s = sum_v exp2(l_v c - r)
// with r = ceil(max l c) taken over the whole tile, so exp2 never exceeds ~1
// and never overflows.
template <int NE, bool FULL>
__device__ __forceinline__ Partial softmax_of_tile(const float* v, float c_hi, float c_lo) {
    float mx = v[0];
#pragma unroll
    for (int j = 1; j < NE; ++j) mx = fmaxf(mx, v[j]);
    mx = wave_max(mx);
    const float r = ceilf(mx * c_hi);
    float e[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) e[j] = exp_term<FULL>(v[j], c_hi, c_lo, r);
    const float s = wave_sum(pairwise_sum<NE>(e));
    return Partial{s, static_cast<int>(r)};
}

// (max, lowest index) of one tile whose logits are already loaded (masked
// elements hold -inf and never win).
template <int DT, int U>
__device__ __forceinline__ ArgMax argmax_of_tile(const float* v, int64_t tile) {
    constexpr int VE = Elem<DT>::per_vec;
    const int lane = lane_id();
    ArgMax a{-__builtin_inff(), kNoIndex};
    const int64_t v0 = tile * (64 * U) + lane;
#pragma unroll
    for (int i = 0; i < U; ++i) {
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const float x = v[i * VE + e];
            if (x > a.val) {
                a.val = x;
                a.idx = static_cast<int>((v0 + i * 64) * VE + e);
            }
        }
    }
    return wave_argmax(a);
}

// (max, lowest index) of one tile of raw logits.
template <int DT, bool VEC, int U, bool FULL>
__device__ __forceinline__ ArgMax tile_argmax(const void* base, int64_t row_elem, int V, int64_t tile) {
    float v[U * Elem<DT>::per_vec];
    load_tile<DT, VEC, U, FULL, true>(base, row_elem, V, tile, lane_id(), v);
    return argmax_of_tile<DT, U>(v, tile);
}

// Tile entry point that picks the unmasked path for tiles inside the row.
template <int DT, bool VEC, int U>
__device__ __forceinline__ ArgMax tile_argmax_any(const void* base, int64_t row_elem, int V, int64_t tile) {
    if (tile_is_full<VEC, U>(tile, V, Elem<DT>::per_vec))
        return tile_argmax<DT, VEC, U, VEC>(base, row_elem, V, tile);
    return tile_argmax<DT, VEC, U, false>(base, row_elem, V, tile);
}

// Partials are read kBatch at a time so that their loads are in flight
// together rather than one round trip each.
constexpr int kBatch = 8;

// Combine the nT argmax partials of one row (one lane, sequential).
__device__ inline ArgMax combine_argmax(const Partial* p, int nT) {
    ArgMax a{p[0].f, p[0].i};
    for (int t0 = 1; t0 < nT; t0 += kBatch) {
        Partial q[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) q[j] = (t0 + j < nT) ? p[t0 + j] : Partial{-__builtin_inff(), kNoIndex};
#pragma unroll
        for (int j = 0; j < kBatch; ++j) a = better(a, ArgMax{q[j].f, q[j].i});
    }
    return a;
}

// The same, with the whole wave striding over the tiles.
__device__ inline ArgMax wave_combine_argmax(const Partial* p, int nT) {
    ArgMax a{-__builtin_inff(), kNoIndex};
    for (int t = lane_id(); t < nT; t += kWave) a = better(a, ArgMax{p[t].f, p[t].i});
    return wave_argmax(a);
}

// Softmax partial merge: (r1, s1) + (r2, s2) over the larger reference.  The
// rescaling is by powers of two (exact) and the one rounded addition is
// commutative, so both lanes of a shuffle pair obtain identical bits.
constexpr int kNoRef = -(1 << 30);

__device__ __forceinline__ void merge_softmax(int& r, double& s, int r2, double s2) {
    const int R = max(r, r2);
    s = ldexp(s, r - R) + ldexp(s2, r2 - R);
    r = R;
}

// The rows of one sequence are combined by groups of G lanes (G a power of
// two): lane l works on row rho0 + l / G and reads that row's partials
// t = l % G + j G.  group_load issues the first kBatch of them (so the loads
// can be in flight before the caller knows how to combine them), and
// group_reduce merges them, reads any further ones and then merges across
// the group with a butterfly.
__device__ __forceinline__ void group_load(const Partial* p, int nT, int G, bool valid, Partial* q) {
    const int sl = lane_id() & (G - 1);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const int t = sl + j * G;
        q[j] = (valid && t < nT) ? p[t] : Partial{0.f, 0};
    }
}

template <bool SOFTMAX>
__device__ __forceinline__ void group_reduce(const Partial* p, int nT, int G, bool valid, const Partial* q, int& r,
                                             double& s, ArgMax& am) {
    const int sl = lane_id() & (G - 1);
    r = kNoRef;
    s = 0.0;
    am = ArgMax{-__builtin_inff(), kNoIndex};
    auto merge = [&](const Partial& x) {
        if constexpr (SOFTMAX)
            merge_softmax(r, s, x.i, static_cast<double>(x.f));
        else
            am = better(am, ArgMax{x.f, x.i});
    };
    if (valid) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (sl + j * G < nT) merge(q[j]);
        for (int t0 = sl + kBatch * G; t0 < nT; t0 += kBatch * G) {
            Partial qq[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int t = t0 + j * G;
                qq[j] = t < nT ? p[t] : Partial{0.f, 0};
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (t0 + j * G < nT) merge(qq[j]);
        }
    }
    for (int m = G >> 1; m >= 1; m >>= 1) {
        if constexpr (SOFTMAX) {
            const int r2 = __shfl_xor(r, m, kWave);
            const double s2 = __shfl_xor(s, m, kWave);
            merge_softmax(r, s, r2, s2);
        } else {
            am = better(am, ArgMax{__shfl_xor(am.val, m, kWave), __shfl_xor(am.idx, m, kWave)});
        }
    }
}

__device__ __forceinline__ int64_t global_wave() {
    return static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave;
}

// ---------------------------------------------------------------- chain: rowstats ---

// The partial of one tile of a row of sequence b: the tile's loads are issued
// before the temperature is known, which then selects softmax or argmax.
template <int DT, bool VEC, int U, bool FULL>
__device__ __forceinline__ Partial rowstats_tile(const void* base, int64_t row_elem, int V, int64_t tile, float T) {
    constexpr int NE = U * Elem<DT>::per_vec;
    float v[NE];
    load_tile<DT, VEC, U, FULL, true>(base, row_elem, V, tile, lane_id(), v);
    if (T > 0.f) {
        float c_hi, c_lo;
        temperature_scale(T, c_hi, c_lo);
        return softmax_of_tile<NE, FULL>(v, c_hi, c_lo);
    }
    const ArgMax a = argmax_of_tile<DT, U>(v, tile);
    return Partial{a.val, a.idx};
}

// Rows 0 .. B*k-1 are target rows (b, j < k); rows B*k .. 2*B*k-1 are draft
// rows (b, i).  The wave streaming tile 0 of a row also reads the row's logit
// at its draft token into gathered[r], so that the acceptance needs no
// dependent gather.  Draft rows of temperature-0 sequences are streamed too,
// and their partials go unused: deciding to skip them would put the
// temperature's load in front of every wave's tile loads.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void chain_rowstats_kernel(const void* __restrict__ target,
                                                                const void* __restrict__ draft,
                                                                const float* __restrict__ temperature,
                                                                const int32_t* __restrict__ tokens,
                                                                int B, int k, int V, int nT,
                                                                Partial* __restrict__ part,
                                                                float* __restrict__ gathered) {
    const int64_t gw = global_wave();
    const int64_t nbk = static_cast<int64_t>(B) * k;
    if (gw >= 2 * nbk * nT) return;
    const int64_t r = gw / nT;
    const int64_t tile = gw - r * nT;
    const bool is_target = r < nbk;
    const int64_t rr = is_target ? r : r - nbk;
    const int64_t b = rr / k;
    const void* base = is_target ? target : draft;
    const int64_t row_elem = (is_target ? (b * (k + 1) + (rr - b * k)) : rr) * static_cast<int64_t>(V);
    if (tile == 0) {
        const int x = tokens[rr];  // draft token scored by this row (rr = b * k + position)
        if (lane_id() == 0 && static_cast<unsigned>(x) < static_cast<unsigned>(V))
            gathered[r] = load_elem<DT>(base, row_elem + x);
    }
    const float T = temperature[b];
    const Partial p = tile_is_full<VEC, U>(tile, V, Elem<DT>::per_vec)
                          ? rowstats_tile<DT, VEC, U, VEC>(base, row_elem, V, tile, T)
                          : rowstats_tile<DT, VEC, U, false>(base, row_elem, V, tile, T);
    if (lane_id() == 0) part[r * nT + tile] = p;
}

// ---------------------------------------------------------------- chain: acceptance ---

// Acceptance of sequence b, computed by one wave (the first of its block):
// the row statistics from the streaming partials (G lanes per row, one
// round trip), the 2k logits at the draft tokens, tau_i in the log domain,
// the first rejection by ballot.  Writes the final draw's descriptor into
// *out and, when `publish`, accepted_len, the accepted prefix of emitted
// (the rest -1; the final token is written later) and accept_prob.
template <int DT>
__device__ __forceinline__ void accept_sequence(const int32_t* __restrict__ tokens,
                                                const float* __restrict__ temperature,
                                                const float* __restrict__ uniforms, int B, int k, int V, int nT,
                                                const Partial* __restrict__ part, const float* __restrict__ gathered,
                                                int64_t b, bool publish, int32_t* __restrict__ accepted_len,
                                                int32_t* __restrict__ emitted, float* __restrict__ accept_prob,
                                                int* s_r, double* s_s, SeqInfo* out) {
    const int lane = lane_id();
    const int64_t nbk = static_cast<int64_t>(B) * k;
    // every load first: none of them depends on another
    const int rows = 2 * k;  // target rows 0..k-1, then draft rows
    int G = kWave;
    while (G > 1 && G * rows > kWave) G >>= 1;
    const int per_pass = kWave / G;
    auto row_of = [&](int rho) -> int64_t { return rho < k ? b * k + rho : nbk + b * k + (rho - k); };
    Partial q[kBatch];
    const int rho_first = lane / G;
    group_load(part + (rho_first < rows ? row_of(rho_first) : 0) * nT, nT, G, rho_first < rows, q);
    const float T = temperature[b];
    const float uk = uniforms[b * (k + 1) + k];
    int x = 0;
    float ui = 0.f, lt = 0.f, ld = 0.f;
    if (lane < k) {
        x = tokens[b * k + lane];
        ui = uniforms[b * (k + 1) + lane];
        lt = gathered[b * k + lane];
        ld = gathered[nbk + b * k + lane];
    }
    const bool sampled = T > 0.f;
    const bool xok = static_cast<unsigned>(x) < static_cast<unsigned>(V);  // out-of-range ids are rejected
    // row statistics (at temperature 0 only the target rows' argmax matters)
    for (int rho0 = 0; rho0 < rows; rho0 += per_pass) {
        const int rho = rho0 + lane / G;
        const bool valid = rho < rows;
        const Partial* p = part + (valid ? row_of(rho) : 0) * nT;
        if (rho0 > 0) group_load(p, nT, G, valid, q);
        int r;
        double sum;
        ArgMax am;
        if (sampled) {
            group_reduce<true>(p, nT, G, valid, q, r, sum, am);
            if (valid && (lane & (G - 1)) == 0) {
                s_r[rho] = r;
                s_s[rho] = sum;
            }
        } else {
            group_reduce<false>(p, nT, G, valid, q, r, sum, am);
            if (valid && (lane & (G - 1)) == 0) s_r[rho] = am.idx;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    bool acc = true;
    double tau = 1.0;
    int g = -1;
    int rt = 0, rd = 0;
    double st = 1.0, sd = 1.0;
    if (lane < k) {
        if (!sampled) g = s_r[lane];
        if (!xok) {
            acc = false;
            tau = 0.0;
        } else if (sampled) {
            rt = s_r[lane];
            st = s_s[lane];
            rd = s_r[k + lane];
            sd = s_s[k + lane];
            const double c = kLog2e / static_cast<double>(T);
            // log2 p - log2 q with log2 p = l c - R - log2 S (the same for q)
            const double l2ratio = (static_cast<double>(lt) * c - rt - log2_of_sum(st)) -
                                   (static_cast<double>(ld) * c - rd - log2_of_sum(sd));
            // exp2 of a non-positive argument in fp32: relative error about 1e-7
            tau = static_cast<double>(exp2f(static_cast<float>(fmin(0.0, l2ratio))));
            acc = static_cast<double>(ui) < tau;
        } else {
            acc = (x == g);
            tau = acc ? 1.0 : 0.0;
        }
    }
    int a = first_lane(lane < k && !acc);
    if (a < 0) a = k;
    int32_t* em = emitted + b * (k + 1);
    if (publish) {
        if (accept_prob != nullptr && lane < k) accept_prob[b * k + lane] = static_cast<float>(tau);
        for (int j = lane; j <= k; j += kWave) em[j] = j < a ? tokens[b * k + j] : -1;
    }
    if (lane == (a < k ? a : 0)) {
        SeqInfo si{};
        si.a = a;
        temperature_scale(sampled ? T : 1.f, si.c_hi, si.c_lo);
        si.u = uk;
        if (!sampled) {
            if (a < k) {
                if (publish) em[a] = g;
                si.mode = kFinalDone;
            } else {
                si.mode = kFinalArgmax;
            }
        } else if (a < k) {
            si.mode = kFinalResidual;
            si.rt = static_cast<float>(rt);
            si.inv_st = static_cast<float>(1.0 / st);
            si.rd = static_cast<float>(rd);
            si.inv_sd = static_cast<float>(1.0 / sd);
        } else {
            si.mode = kFinalBonus;
        }
        *out = si;
    }
    if (publish && lane == 0) accepted_len[b] = a;
}

// One wave per sequence, kAccWaves sequences per workgroup: the acceptance
// of every sequence, its outputs and the descriptor of its final draw.
constexpr int kAccWaves = 4;

template <int DT>
__global__ __launch_bounds__(kAccWaves * kWave) void chain_accept_kernel(
    const int32_t* __restrict__ tokens, const float* __restrict__ temperature, const float* __restrict__ uniforms,
    int B, int k, int V, int nT, const Partial* __restrict__ part, const float* __restrict__ gathered,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ emitted, float* __restrict__ accept_prob,
    SeqInfo* __restrict__ info) {
    __shared__ int s_r[kAccWaves][2 * SV_MAX_DRAFTS];
    __shared__ double s_s[kAccWaves][2 * SV_MAX_DRAFTS];
    const int w = threadIdx.x / kWave;
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kAccWaves + w;
    if (b >= B) return;  // whole waves only; the kernel has no workgroup barrier
    accept_sequence<DT>(tokens, temperature, uniforms, B, k, V, nT, part, gathered, b, true, accepted_len, emitted,
                        accept_prob, s_r[w], s_s[w], info + b);
}

// ---------------------------------------------------------------- chain: final draw ---

// Weight of the final draw for the U*VE elements a lane holds.
//   residual: w = max(0, p - q), p = exp2(l_t c - rt) / S_t, q likewise;
//   bonus:    w = exp2(l c - ref), unnormalised (the draw is scale-free).
template <int NE, bool FULL>
__device__ __forceinline__ void residual_weights(const float* vt, const float* vd, const SeqInfo& s, float* w) {
#pragma unroll
    for (int j = 0; j < NE; ++j) {
        const float p = exp_term<FULL>(vt[j], s.c_hi, s.c_lo, s.rt) * s.inv_st;
        const float q = exp_term<FULL>(vd[j], s.c_hi, s.c_lo, s.rd) * s.inv_sd;
        w[j] = fmaxf(p - q, 0.f);
    }
}

template <int NE, bool FULL>
__device__ __forceinline__ void bonus_weights(const float* v, const SeqInfo& s, float ref, float* w) {
#pragma unroll
    for (int j = 0; j < NE; ++j) w[j] = exp_term<FULL>(v[j], s.c_hi, s.c_lo, ref);
}

// Weights of segment `seg` (one vector per lane) in the tile's scale.
template <int DT, bool VEC, bool FULL>
__device__ __forceinline__ void segment_weights_t(const void* draft, const void* target, int64_t trow,
                                                  int64_t drow, int V, int64_t seg, const SeqInfo& s,
                                                  bool residual, float ref, float* w) {
    constexpr int VE = Elem<DT>::per_vec;
    // a segment is tile seg/U's load seg%U, i.e. vectors 64*seg .. 64*seg+63
    float vt[VE];
    load_tile<DT, VEC, 1, FULL>(target, trow, V, seg, lane_id(), vt);
    if (residual) {
        float vd[VE];
        load_tile<DT, VEC, 1, FULL>(draft, drow, V, seg, lane_id(), vd);
        residual_weights<VE, FULL>(vt, vd, s, w);
    } else {
        bonus_weights<VE, FULL>(vt, s, ref, w);
    }
}

template <int DT, bool VEC>
__device__ __forceinline__ void segment_weights(const void* draft, const void* target, int64_t trow,
                                                int64_t drow, int V, int64_t seg, const SeqInfo& s,
                                                bool residual, float ref, float* w) {
    if (tile_is_full<VEC, 1>(seg, V, Elem<DT>::per_vec))
        segment_weights_t<DT, VEC, VEC>(draft, target, trow, drow, V, seg, s, residual, ref, w);
    else
        segment_weights_t<DT, VEC, false>(draft, target, trow, drow, V, seg, s, residual, ref, w);
}

// Inverse CDF inside one segment.  `P` is the mass before the segment and
// `scale` maps the segment's weights to the global scale (a power of two).
// Returns the token, or -1 when rounding leaves C <= target everywhere.
template <int DT>
__device__ __forceinline__ int pick_in_segment(const float* w, int64_t seg, double P, double scale,
                                               double target_mass) {
    constexpr int VE = Elem<DT>::per_vec;
    const int lane = lane_id();
    double lane_sum = 0.0;
#pragma unroll
    for (int e = 0; e < VE; ++e) lane_sum += static_cast<double>(w[e]) * scale;
    const double incl = wave_inclusive_scan(lane_sum);
    const double excl = __shfl_up(incl, 1, kWave);
    double C = P + (lane == 0 ? 0.0 : excl);
    int hit = -1;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        C += static_cast<double>(w[e]) * scale;
        if (hit < 0 && C > target_mass) hit = e;
    }
    const int fl = first_lane(hit >= 0);
    if (fl < 0) return -1;
    const int e = __shfl(hit, fl, kWave);
    return static_cast<int>((seg * 64 + fl) * VE + e);
}

// Last token of the segment whose weight is positive, or -1.
template <int DT>
__device__ __forceinline__ int last_positive_in_segment(const float* w, int64_t seg) {
    constexpr int VE = Elem<DT>::per_vec;
    int last = -1;
#pragma unroll
    for (int e = 0; e < VE; ++e)
        if (w[e] > 0.f) last = e;
    const uint64_t m = __ballot(last >= 0);
    if (!m) return -1;
    const int fl = 63 - __builtin_clzll(m);
    const int e = __shfl(last, fl, kWave);
    return static_cast<int>((seg * 64 + fl) * VE + e);
}

// The final draw of sequence b is spread over `nchunk` workgroups, each
// owning kSegPerChunk consecutive segments (a segment is the 64 vectors of
// one wave load).  A workgroup first needs the draw's descriptor, obtained
// in one of three ways (FinalAccept): with no drafts it is formed from the
// temperature alone, so the first loads are the row's; for a draw that fits
// in one round of resident workgroups every workgroup recomputes its
// sequence's acceptance (a few KB of partials: cheaper than another launch);
// for larger draws chain_accept_kernel has written it once per sequence.
// The workgroup then streams its chunk of the row(s) the draw needs and
// writes each segment's mass and reference exponent, or, at temperature 0,
// the chunk's argmax.
enum FinalAccept : int { kAcceptNone = 0, kAcceptInline = 1, kAcceptRead = 2 };

constexpr int kFinBlock = 256;
constexpr int kFinWaves = kFinBlock / kWave;
constexpr int kFinU = 4;  // segments per wave tile
constexpr int kSegPerChunk = kFinWaves * kFinU;  // segments per workgroup and tile round

template <int DT, bool VEC, bool FULL>
__device__ __forceinline__ void final_tile(const void* draft, const void* target, int64_t trow, int64_t drow,
                                           int V, int64_t tile, int64_t nseg, const SeqInfo& si, int mode,
                                           Partial* __restrict__ seg_out, ArgMax& best) {
    constexpr int VE = Elem<DT>::per_vec;
    constexpr int NE = kFinU * VE;
    const int lane = lane_id();
    float w[NE];  // the target's logits, then (in place) the weights
    load_tile<DT, VEC, kFinU, FULL>(target, trow, V, tile, lane, w);
    if (mode == kFinalArgmax) {
        best = better(best, argmax_of_tile<DT, kFinU>(w, tile));
        return;
    }
    float ref = 0.f;
    if (mode == kFinalResidual) {
        float vd[NE];
        load_tile<DT, VEC, kFinU, FULL>(draft, drow, V, tile, lane, vd);
        residual_weights<NE, FULL>(w, vd, si, w);
    } else {
        float mx = w[0];
#pragma unroll
        for (int j = 1; j < NE; ++j) mx = fmaxf(mx, w[j]);
        // a reference over the whole tile (which always holds an element of the row)
        ref = ceilf(wave_max(mx) * si.c_hi);
        bonus_weights<NE, FULL>(w, si, ref, w);
    }
    static_assert(kFinU == 4, "the four segment sums use one reduce-scatter");
    float a[kFinU];
#pragma unroll
    for (int i = 0; i < kFinU; ++i) a[i] = pairwise_sum<VE>(w + i * VE);
    int i_own;
    const float m = wave_sum4(a, i_own);
    const int64_t g = tile * kFinU + i_own;
    if (lane < kFinU && g < nseg) seg_out[g] = Partial{m, static_cast<int>(ref)};
}

template <int DT, bool VEC, int ACC>
__global__ __launch_bounds__(kFinBlock) void chain_final_part_kernel(
    const int32_t* __restrict__ tokens, const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, int B, int k, int V, int nT,
    const Partial* __restrict__ part, const float* __restrict__ gathered, int nchunk,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ emitted, float* __restrict__ accept_prob,
    SeqInfo* __restrict__ info, Partial* __restrict__ segs, Partial* __restrict__ chunkarg) {
    constexpr int VE = Elem<DT>::per_vec;
    __shared__ ArgMax s_arg[kFinWaves];
    const int64_t b = blockIdx.x / nchunk;
    const int c = static_cast<int>(blockIdx.x - b * nchunk);
    SeqInfo si;
    if constexpr (ACC == kAcceptInline) {
        __shared__ int s_r[2 * SV_MAX_DRAFTS];
        __shared__ double s_s[2 * SV_MAX_DRAFTS];
        __shared__ SeqInfo s_info;
        if (threadIdx.x < kWave)
            accept_sequence<DT>(tokens, temperature, uniforms, B, k, V, nT, part, gathered, b, c == 0, accepted_len,
                                emitted, accept_prob, s_r, s_s, &s_info);
        __syncthreads();
        si = s_info;
        if (c == 0 && threadIdx.x == 0) info[b] = si;
        if (si.mode == kFinalDone) return;
    } else if constexpr (ACC == kAcceptNone) {
        // k == 0: draw from target row 0 (its argmax at temperature 0)
        const float T = temperature[b];
        si = SeqInfo{};
        si.mode = T > 0.f ? kFinalBonus : kFinalArgmax;
        temperature_scale(T > 0.f ? T : 1.f, si.c_hi, si.c_lo);
        si.u = uniforms[b];
        if (c == 0 && threadIdx.x == 0) {
            info[b] = si;
            accepted_len[b] = 0;
        }
    } else {
        si = info[b];
        if (si.mode == kFinalDone) return;
    }
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    const int64_t trow = (b * (k + 1) + si.a) * static_cast<int64_t>(V);
    const int64_t drow = (b * k + si.a) * static_cast<int64_t>(V);
    const int wave = threadIdx.x / kWave;
    const int64_t tile = static_cast<int64_t>(c) * kFinWaves + wave;  // the workgroup's waves read adjacent tiles
    Partial* seg_out = segs + b * nseg;
    ArgMax best{-__builtin_inff(), kNoIndex};
    if (tile * kFinU < nseg) {
        if (tile_is_full<VEC, kFinU>(tile, V, VE))
            final_tile<DT, VEC, VEC>(draft, target, trow, drow, V, tile, nseg, si, si.mode, seg_out, best);
        else
            final_tile<DT, VEC, false>(draft, target, trow, drow, V, tile, nseg, si, si.mode, seg_out, best);
    }
    if (si.mode == kFinalArgmax) {
        if (lane_id() == 0) s_arg[wave] = best;
        __syncthreads();
        if (threadIdx.x == 0) {
            ArgMax r = s_arg[0];
            for (int w = 1; w < kFinWaves; ++w) r = better(r, s_arg[w]);
            chunkarg[b * nchunk + c] = Partial{r.val, r.idx};
        }
    }
}

// Slow path of the draw, one wave: inverse CDF of the target row's own
// distribution with two sequential sweeps over its segments.  Used only when
// the residual of a rejection has no mass at all (draft and target rows
// agree to rounding).
template <int DT, bool VEC>
__device__ int pick_from_target_row(const void* target, int64_t trow, int V, int64_t nseg, const SeqInfo& s) {
    constexpr int VE = Elem<DT>::per_vec;
    float w[VE];
    double W = 0.0;
    for (int64_t g = 0; g < nseg; ++g) {
        segment_weights<DT, VEC>(nullptr, target, trow, 0, V, g, s, false, s.rt, w);
        W += static_cast<double>(wave_sum(pairwise_sum<VE>(w)));
    }
    const double target_mass = static_cast<double>(s.u) * W;
    double P = 0.0;
    int last = -1;
    for (int64_t g = 0; g < nseg; ++g) {
        segment_weights<DT, VEC>(nullptr, target, trow, 0, V, g, s, false, s.rt, w);
        const double mass = static_cast<double>(wave_sum(pairwise_sum<VE>(w)));
        if (mass > 0.0) {
            const int y = pick_in_segment<DT>(w, g, P, 1.0, target_mass);
            if (y >= 0) return y;
            last = last_positive_in_segment<DT>(w, g);
        }
        P += mass;
    }
    return last;
}

// Select pass of the final draw: one wave per sequence.  Lane l owns a
// contiguous run of segments; a wave prefix over the run totals gives every
// segment's starting mass, the segment holding u * W is found with a ballot,
// and only that segment is read again to find the token.  The descriptor and
// the lane's first kSegRun segments are loaded together.
constexpr int kSegRun = 8;

template <int DT, bool VEC>
__global__ __launch_bounds__(kWave) void chain_final_pick_kernel(
    const void* __restrict__ draft, const void* __restrict__ target, int B, int k, int V, int nchunk,
    const SeqInfo* __restrict__ info, const Partial* __restrict__ segs, const Partial* __restrict__ chunkarg,
    int32_t* __restrict__ emitted) {
    constexpr int VE = Elem<DT>::per_vec;
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    const Partial* sg = segs + b * nseg;
    const int64_t per = (nseg + kWave - 1) / kWave;
    const int64_t g0 = min<int64_t>(nseg, lane * per), g1 = min<int64_t>(nseg, g0 + per);
    Partial first[kSegRun];
#pragma unroll
    for (int j = 0; j < kSegRun; ++j) first[j] = (g0 + j < g1) ? sg[g0 + j] : Partial{0.f, kNoRef};
    const SeqInfo s = info[b];
    if (s.mode == kFinalDone) return;
    int y;
    if (s.mode == kFinalArgmax) {
        y = wave_combine_argmax(chunkarg + b * nchunk, nchunk).idx;
    } else {
        const bool residual = s.mode == kFinalResidual;
        const int64_t trow = (b * (k + 1) + s.a) * static_cast<int64_t>(V);
        const int64_t drow = (b * k + s.a) * static_cast<int64_t>(V);
        const int64_t nwin = (per + kSegRun - 1) / kSegRun;
        // segment g of this lane's window w
        auto seg_at = [&](int64_t w, int j) -> Partial {
            const int64_t g = g0 + w * kSegRun + j;
            return w == 0 ? first[j] : (g < g1 ? sg[g] : Partial{0.f, kNoRef});
        };
        // global reference exponent (residual masses are absolute: reference 0)
        int R = 0;
        if (!residual) {
            R = kNoRef;
            for (int64_t w = 0; w < nwin; ++w)
#pragma unroll
                for (int j = 0; j < kSegRun; ++j) R = max(R, seg_at(w, j).i);
            R = wave_max(R);
        }
        // masses of this lane's window w in the global scale
        auto window = [&](int64_t w, double* mg) {
#pragma unroll
            for (int j = 0; j < kSegRun; ++j) {
                const Partial q = seg_at(w, j);
                const bool in = g0 + w * kSegRun + j < g1;
                mg[j] = !in ? 0.0 : residual ? static_cast<double>(q.f) : ldexp(static_cast<double>(q.f), q.i - R);
            }
        };
        double tot = 0.0;
        for (int64_t w = 0; w < nwin; ++w) {
            double mg[kSegRun];
            window(w, mg);
#pragma unroll
            for (int j = 0; j < kSegRun; ++j) tot += mg[j];
        }
        const double incl = wave_inclusive_scan(tot);
        const double W = __shfl(incl, kWave - 1, kWave);
        const double excl = __shfl_up(incl, 1, kWave);  // every lane shuffles
        double P = lane == 0 ? 0.0 : excl;
        if (!(W > 0.0)) {
            y = residual ? pick_from_target_row<DT, VEC>(target, trow, V, nseg, s) : 0;
        } else {
            const double target_mass = static_cast<double>(s.u) * W;
            int64_t found = -1, last_pos = -1;
            double Pfound = 0.0;
            for (int64_t w = 0; w < nwin; ++w) {
                double mg[kSegRun];
                window(w, mg);
#pragma unroll
                for (int j = 0; j < kSegRun; ++j) {
                    const int64_t g = g0 + w * kSegRun + j;
                    if (g >= g1) break;
                    if (found < 0 && P + mg[j] > target_mass) {
                        found = g;
                        Pfound = P;
                    }
                    if (mg[j] > 0.0) last_pos = g;
                    P += mg[j];
                }
            }
            int fl = first_lane(found >= 0);
            int64_t seg;
            double Ps;
            bool fallback = false;
            if (fl >= 0) {
                seg = __shfl(found, fl, kWave);
                Ps = __shfl(Pfound, fl, kWave);
            } else {
                // rounding put u * W at or past the total: the last segment with mass
                const uint64_t m = __ballot(last_pos >= 0);
                fl = m ? 63 - __builtin_clzll(m) : 0;
                seg = m ? __shfl(last_pos, fl, kWave) : 0;
                Ps = 0.0;
                fallback = true;
            }
            const int tref = residual ? 0 : sg[seg].i;
            const double scale = ldexp(1.0, tref - R);
            float w[VE];
            segment_weights<DT, VEC>(draft, target, trow, drow, V, seg, s, residual, static_cast<float>(tref), w);
            y = fallback ? -1 : pick_in_segment<DT>(w, seg, Ps, scale, target_mass);
            if (y < 0) y = last_positive_in_segment<DT>(w, seg);
        }
    }
    if (lane == 0) emitted[b * (k + 1) + s.a] = y;
}

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

// One wave per sequence: lane j combines row j's tiles into g_j; the first
// lane with x_j != g_j is the rejection; g_a is the emitted target token.
__global__ __launch_bounds__(kWave) void greedy_finalize_kernel(const int32_t* __restrict__ tokens, int k,
                                                                int nT, const Partial* __restrict__ part,
                                                                int32_t* __restrict__ accepted_len,
                                                                int32_t* __restrict__ emitted) {
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    int g = -1, x = 0;
    if (lane < k) {
        x = tokens[b * k + lane];
        g = combine_argmax(part + (b * (k + 1) + lane) * nT, nT).idx;
    }
    int a = first_lane(lane < k && x != g);
    int y;
    if (a < 0) {
        a = k;
        y = wave_combine_argmax(part + (b * (k + 1) + k) * nT, nT).idx;
    } else {
        y = __shfl(g, a, kWave);
    }
    int32_t* out = emitted + b * (k + 1);
    for (int j = lane; j <= k; j += kWave) out[j] = j < a ? tokens[b * k + j] : (j == a ? y : -1);
    if (lane == 0) accepted_len[b] = a;
}

// ---------------------------------------------------------------- tree ---

// One workgroup per sequence, one thread per node (N <= blockDim.x <= 1024).
// Pointer jumping over the parent links gives every node its depth and
// whether every edge on its root path matches; the deepest accepted node
// (lowest index among equals) is chosen and its path written out.
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
    int p = 0;
    if (n < N) {
        s_g[n] = combine_argmax(part + (b * N + n) * nT, nT).idx;
        s_tok[n] = node_tokens[b * N + n];
        p = n == 0 ? 0 : par[n];
        if (n > 0 && (p < 0 || p >= n)) s_bad = 1;
        s_par[n] = p;
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

// ---------------------------------------------------------------- tree: sampled ---
//
// Multi-step speculative sampling over a draft tree (SpecInfer, Miao et al.
// 2023, the rule the EAGLE work applies to sampled trees; the pages, section
// "EAGLE", keep the longest path that passes).  At node n the children are
// tested in index order against a running distribution r that starts as the
// target row p_n; a rejection replaces r by the normalised residual
// max(0, r - q_n).  That residual after j rejections is max(0, p - c_j q) /
// Z(c_j), Z(c) = sum_v max(0, p_v - c q_v), c_0 = 0, c_{j+1} = c_j + Z(c_j),
// so a sibling's test needs only the scalars (c, Z) and each rejection one
// pass over the node's two rows.

// Rows 0 .. B*N-1 are target rows (b, n), rows B*N .. 2*B*N-1 draft rows.
// The draft row of a leaf is never needed and is skipped.
// The wave streaming tile 0 of inner node n's draft row also gathers, for
// every child i of n, the target and draft logits of row n at i's token into
// tg[b][i] and dg[b][i] (0 for a token outside [0, V)), so that the walk's
// sibling tests need no dependent loads.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void tree_rowstats_kernel(const void* __restrict__ target,
                                                               const void* __restrict__ draft,
                                                               const int32_t* __restrict__ parent, int parent_stride,
                                                               const int32_t* __restrict__ node_tokens,
                                                               const float* __restrict__ temperature, int B, int N,
                                                               int V, int nT, Partial* __restrict__ part,
                                                               float* __restrict__ tg, float* __restrict__ dg) {
    const int64_t gw = global_wave();
    const int64_t nbn = static_cast<int64_t>(B) * N;
    if (gw >= 2 * nbn * nT) return;
    const int64_t r = gw / nT;
    const int64_t tile = gw - r * nT;
    const bool is_target = r < nbn;
    const int64_t rr = is_target ? r : r - nbn;
    const int64_t b = rr / N;
    const int n = static_cast<int>(rr - b * N);
    if (!is_target) {
        const int32_t* par = parent + b * static_cast<int64_t>(parent_stride);
        bool kid = false;
        for (int i = n + 1 + lane_id(); i < N; i += kWave) {
            const bool child = par[i] == n;
            kid |= child;
            if (child && tile == 0) {
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
    const Partial p = tile_is_full<VEC, U>(tile, V, Elem<DT>::per_vec)
                          ? rowstats_tile<DT, VEC, U, VEC>(base, row_elem, V, tile, T)
                          : rowstats_tile<DT, VEC, U, false>(base, row_elem, V, tile, T);
    if (lane_id() == 0) part[r * nT + tile] = p;
}

// One workgroup per sequence walks its tree; each thread holds kWalkSlots
// node slots (t, t + kWalkBlock, ...).
constexpr int kWalkBlock = 512;
constexpr int kWalkWaves = kWalkBlock / kWave;
constexpr int kWalkSlots = SV_MAX_TREE_NODES / kWalkBlock;
constexpr int kWalkMaxSegs = SV_MAX_VOCAB / (4 * 64);  // f32 rows have the most segments
constexpr int kWalkUnroll = 8;                          // segments in flight per wave

// Normalised weights of segment g of the running distribution: p when the
// residual scale c is 0, else max(0, p - c q) (s.inv_sd carries c / S_d).
template <int DT, bool VEC>
__device__ __forceinline__ void walk_weights(const void* draft, const void* target, int64_t row, int V, int64_t g,
                                             const SeqInfo& s, bool residual, float* w) {
    constexpr int VE = Elem<DT>::per_vec;
    segment_weights<DT, VEC>(draft, target, row, row, V, g, s, residual, s.rt, w);
    if (!residual) {
#pragma unroll
        for (int e = 0; e < VE; ++e) w[e] *= s.inv_st;
    }
}

// Weights of one full segment from its raw 16-byte vectors (the same
// arithmetic as walk_weights on an unmasked segment).
template <int DT, bool RESIDUAL>
__device__ __forceinline__ void walk_weights_raw(const uint4& rt, const uint4& rd, const SeqInfo& s, float* w) {
    constexpr int VE = Elem<DT>::per_vec;
    float vt[VE];
    unpack<DT>(rt, vt);
    if constexpr (RESIDUAL) {
        float vd[VE];
        unpack<DT>(rd, vd);
        residual_weights<VE, true>(vt, vd, s, w);
    } else {
        bonus_weights<VE, true>(vt, s, s.rt, w);
#pragma unroll
        for (int e = 0; e < VE; ++e) w[e] *= s.inv_st;
    }
}

// Every thread of the workgroup: the mass of every segment of the running
// distribution into s_mass, and their total (ascending order, fp64) as the
// return value (identical in every thread).  Segments that lie wholly inside
// the row are read kWalkUnroll per wave at a time with straight-line 16-byte
// loads (indices clamped rather than branched on, so that all loads are in
// flight together); the row's tail takes the masked path.
template <int DT, bool VEC, bool RESIDUAL>
__device__ double walk_masses(const void* draft, const void* target, int64_t row, int V, int64_t nseg,
                              const SeqInfo& s, float* s_mass, double* s_sum) {
    constexpr int VE = Elem<DT>::per_vec;
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int64_t nfull = VEC ? ((V + VE - 1) / VE) / 64 : 0;
    const char* tr = static_cast<const char*>(target) + row * Elem<DT>::bytes;
    const char* dr = static_cast<const char*>(draft) + row * Elem<DT>::bytes;
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
            float w[VE];
            walk_weights_raw<DT, RESIDUAL>(rt[j], rd[j], s, w);
            const float m = wave_sum(pairwise_sum<VE>(w));
            if (lane == 0 && g < nfull) s_mass[g] = m;
        }
    }
    for (int64_t g = nfull + wave; g < nseg; g += kWalkWaves) {
        float w[VE];
        walk_weights<DT, VEC>(draft, target, row, V, g, s, RESIDUAL, w);
        const float m = wave_sum(pairwise_sum<VE>(w));
        if (lane == 0) s_mass[g] = m;
    }
    __syncthreads();
    if (wave == 0) {
        const int64_t per = (nseg + kWave - 1) / kWave;
        const int64_t a = min<int64_t>(nseg, lane * per), e = min<int64_t>(nseg, a + per);
        double run = 0.0;
        for (int64_t g = a; g < e; ++g) run += static_cast<double>(s_mass[g]);
        const double tot = __shfl(wave_inclusive_scan(run), kWave - 1, kWave);
        if (lane == 0) *s_sum = tot;
    }
    __syncthreads();
    return *s_sum;
}

// Inverse CDF of the running distribution whose segment masses are in
// s_mass (wave 0; returns the token in every lane).
template <int DT, bool VEC>
__device__ int walk_pick(const void* draft, const void* target, int64_t row, int V, int64_t nseg, const SeqInfo& s,
                         bool residual, const float* s_mass, double W, double u) {
    const int lane = lane_id();
    const int64_t per = (nseg + kWave - 1) / kWave;
    const int64_t a = min<int64_t>(nseg, lane * per), e = min<int64_t>(nseg, a + per);
    double run = 0.0;
    for (int64_t g = a; g < e; ++g) run += static_cast<double>(s_mass[g]);
    const double incl = wave_inclusive_scan(run);
    const double excl = __shfl_up(incl, 1, kWave);  // every lane shuffles
    double P = lane == 0 ? 0.0 : excl;
    const double target_mass = u * W;
    int64_t found = -1, last_pos = -1;
    double Pfound = 0.0;
    for (int64_t g = a; g < e; ++g) {
        const double m = static_cast<double>(s_mass[g]);
        if (found < 0 && P + m > target_mass) {
            found = g;
            Pfound = P;
        }
        if (m > 0.0) last_pos = g;
        P += m;
    }
    int fl = first_lane(found >= 0);
    int64_t seg;
    double Ps = 0.0;
    bool fallback = false;
    if (fl >= 0) {
        seg = __shfl(found, fl, kWave);
        Ps = __shfl(Pfound, fl, kWave);
    } else {
        const uint64_t m = __ballot(last_pos >= 0);
        fl = m ? 63 - __builtin_clzll(m) : 0;
        seg = m ? __shfl(last_pos, fl, kWave) : 0;
        fallback = true;
    }
    float w[Elem<DT>::per_vec];
    walk_weights<DT, VEC>(draft, target, row, V, seg, s, residual, w);
    int y = fallback ? -1 : pick_in_segment<DT>(w, seg, Ps, 1.0, target_mass);
    if (y < 0) y = last_positive_in_segment<DT>(w, seg);
    return y;
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
    kWalkStuck = 5   // a case the rounds leave to the one-workgroup walk (an empty final residual)
};

struct alignas(16) WalkState {
    int phase, node, depth, kidx;  // kidx: children of `node` already rejected
    int Rt, Rd, pad0, pad1;        // node statistics (at temperature 0: the two argmaxes)
    double St, Sd, c, Z;
};

template <int DT, bool VEC>
__global__ __launch_bounds__(kWalkBlock) void tree_sample_kernel(
    const int32_t* __restrict__ node_tokens, const int32_t* __restrict__ parent, int parent_stride, int N,
    int max_depth, const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, int B, int V, int nT,
    const Partial* __restrict__ part, const WalkState* __restrict__ state, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ emitted, int32_t* __restrict__ accepted_nodes) {
    constexpr int VE = Elem<DT>::per_vec;
    if (state != nullptr && state[blockIdx.x].phase == kWalkDone) return;  // finished by the rounds
    __shared__ int s_par[SV_MAX_TREE_NODES];
    __shared__ int s_anc[SV_MAX_TREE_NODES];
    __shared__ int s_len[SV_MAX_TREE_NODES];
    __shared__ uint64_t s_kids[SV_MAX_TREE_NODES / kWave];
    __shared__ float s_mass[kWalkMaxSegs];
    // the current node's children in index order: node id, uniform, and the
    // target and draft logits at the child's token
    __shared__ int s_cid[SV_MAX_TREE_NODES];
    __shared__ float s_cu[SV_MAX_TREE_NODES];
    __shared__ float s_clt[SV_MAX_TREE_NODES];
    __shared__ float s_cld[SV_MAX_TREE_NODES];
    __shared__ double s_sum;
    __shared__ double s_norm[2];  // S_t, S_d of the current node
    __shared__ int s_ref[2];      // R_t, R_d (at temperature 0: the two argmaxes)
    __shared__ int s_bad, s_accept;
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = lane_id();
    const int wave = t / kWave;
    const int width = max_depth + 1;
    const float T = temperature[b];
    const bool sampled = T > 0.f;
    int32_t* out = emitted + b * width;
    int32_t* nodes = accepted_nodes ? accepted_nodes + b * width : nullptr;

    // validity and depths (pointer jumping), as for the greedy tree
    const bool bad = walk_validate<kWalkBlock>(parent + b * static_cast<int64_t>(parent_stride), N, max_depth, s_par,
                                               s_anc, s_len, &s_bad);
    for (int j = t; j < width; j += kWalkBlock) {
        out[j] = -1;
        if (nodes) nodes[j] = -1;
    }
    if (bad) {
        if (t == 0) accepted_len[b] = -1;
        return;
    }

    SeqInfo s{};
    temperature_scale(sampled ? T : 1.f, s.c_hi, s.c_lo);
    const double cT = kLog2e / static_cast<double>(sampled ? T : 1.f);
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    const int nmask = (N + kWave - 1) / kWave;
    const int64_t nbn = static_cast<int64_t>(B) * N;
    int n = 0, d = 0;
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
        if (wave == 0) {
            const bool is_draft = lane >= 32;
            const Partial* pr = part + ((is_draft ? nbn : 0) + b * N + n) * nT;
            Partial q[kBatch];
            group_load(pr, nT, 32, true, q);
            int r;
            double sum;
            ArgMax am;
            if (sampled) {
                group_reduce<true>(pr, nT, 32, true, q, r, sum, am);
            } else {
                group_reduce<false>(pr, nT, 32, true, q, r, sum, am);
                r = am.idx;
            }
            if ((lane & 31) == 0) {
                s_ref[is_draft] = r;
                s_norm[is_draft] = sum;
            }
        }
        __syncthreads();
        const int Rt = s_ref[0], Rd = s_ref[1];
        const double St = s_norm[0], Sd = s_norm[1];
        s.rt = static_cast<float>(Rt);
        s.inv_st = static_cast<float>(1.0 / St);
        s.rd = static_cast<float>(Rd);
        double c = 0.0, Z = 1.0;
        int next = -1;
        // log2 of the two normalisers' mantissas, once per node (thread 0 tests)
        const double lsum = t == 0 && sampled && nkids > 0 ? (Rt + log2(St)) - (Rd + log2(Sd)) : 0.0;
        for (int k = 0; k < nkids && next < 0; ++k) {
            if (t == 0) {
                const int id = s_cid[k];
                double tau = 0.0;
                if (id >= 0) {
                    if (sampled) {
                        // p/q = exp2((l_t - l_d) c - (R_t + log2 S_t) + (R_d + log2 S_d))
                        const double lt = s_clt[k], ld = s_cld[k];
                        const double l2ratio = (lt * cT - ld * cT) - lsum;
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
                if (sampled) {
                    s.inv_sd = static_cast<float>(c / Sd);
                    Z = walk_masses<DT, VEC, true>(draft, target, row, V, nseg, s, s_mass, &s_sum);
                } else {
                    Z = Rt != Rd ? 1.0 : fmax(0.0, 1.0 - c);
                }
                if (!(Z > 0.0)) {
                    c = 0.0;
                    Z = 1.0;
                }
            }
            __syncthreads();
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
            const bool residual = c > 0.0;
            double W = Z;
            if (!residual) W = walk_masses<DT, VEC, false>(draft, target, row, V, nseg, s, s_mass, &s_sum);
            y = 0;
            if (wave == 0)
                y = walk_pick<DT, VEC>(draft, target, row, V, nseg, s, residual, s_mass, W,
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
// tree (invalid trees give -1 outputs) and sets the outputs to -1.  A
// sequence not finished after the launched rounds is walked again from the
// start by tree_sample.
constexpr int kRoundBlock = 256;
constexpr int kRoundWaves = kRoundBlock / kWave;
constexpr int kRoundSlots = SV_MAX_TREE_NODES / kRoundBlock;
constexpr int kWalkRounds = 8;

template <int DT, bool VEC>
__global__ __launch_bounds__(kRoundBlock) void tree_round_kernel(
    const int32_t* __restrict__ node_tokens, const int32_t* __restrict__ parent, int parent_stride, int N,
    int max_depth, const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, int B, int V, int nT,
    const Partial* __restrict__ part, const float* __restrict__ tg, const float* __restrict__ dg,
    const WalkState* __restrict__ st_in, WalkState* __restrict__ st_out, const double* __restrict__ z_in,
    double* __restrict__ z_out, float* __restrict__ tsegs, int P, int first, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ emitted, int32_t* __restrict__ accepted_nodes) {
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
    __shared__ double s_wsum[kRoundWaves];
    __shared__ double s_z;
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
    WalkState st{};
    if (first) {
        const bool bad = walk_validate<kRoundBlock>(parent + b * static_cast<int64_t>(parent_stride), N, max_depth,
                                                    s_par, s_anc, s_len, &s_bad);
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
    } else {
        st = st_in[b];
    }
    if (st.phase == kWalkDone || st.phase == kWalkStuck) {
        if (lead && t == 0) st_out[b] = st;
        return;
    }
    const float T = temperature[b];
    const bool sampled = T > 0.f;
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    SeqInfo s{};
    temperature_scale(sampled ? T : 1.f, s.c_hi, s.c_lo);

    if (st.phase == kWalkPick) {
        // the final distribution's masses were written last round: wave 0 of chunk 0 draws the token
        if (lead && wave == 0) {
            const int64_t row = (b * N + st.node) * static_cast<int64_t>(V);
            s.rt = static_cast<float>(st.Rt);
            s.inv_st = static_cast<float>(1.0 / st.St);
            s.rd = static_cast<float>(st.Rd);
            s.inv_sd = static_cast<float>(st.c / st.Sd);
            const float* m = tsegs + b * nseg;
            const int64_t per = (nseg + kWave - 1) / kWave;
            const int64_t a0 = min<int64_t>(nseg, lane * per), a1 = min<int64_t>(nseg, a0 + per);
            double run = 0.0;
            for (int64_t g = a0; g < a1; ++g) run += static_cast<double>(m[g]);
            const double W = __shfl(wave_inclusive_scan(run), kWave - 1, kWave);
            if (W > 0.0) {
                const int y = walk_pick<DT, VEC>(draft, target, row, V, nseg, s, st.c > 0.0, m, W,
                                                 static_cast<double>(uniforms[b * N]));
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

    // the tree, the tokens, uniforms and gathered logits of every node, and
    // the partial sums of a pending pass
    const int32_t* par = parent + b * static_cast<int64_t>(parent_stride);
#pragma unroll
    for (int q = 0; q < kRoundSlots; ++q) {
        const int i = t + q * kRoundBlock;
        if (i < N) {
            s_par[i] = i == 0 ? -1 : par[i];
            s_tok[i] = node_tokens[b * N + i];
            s_u[i] = uniforms[b * N + i];
            s_tg[i] = tg[b * N + i];
            s_dg[i] = dg[b * N + i];
        }
    }
    if (st.phase == kWalkPass && wave == 0) {
        double zz = 0.0;
        for (int q = lane; q < P; q += kWave) zz += z_in[b * P + q];
        zz = wave_sum(zz);
        if (lane == 0) s_z = zz;
    }
    __syncthreads();
    int n = st.node, d = st.depth, kidx = st.kidx, Rt = st.Rt, Rd = st.Rd;
    double St = st.St, Sd = st.Sd, c = st.c, Z = st.Z;
    int phase = st.phase;
    if (phase == kWalkPass) {
        Z = s_z;
        if (!(Z > 0.0)) {
            c = 0.0;
            Z = 1.0;
        }
        phase = kWalkTest;
    }
    const double cT = kLog2e / static_cast<double>(sampled ? T : 1.f);
    const int nmask = (N + kWave - 1) / kWave;
    const int64_t nbn = static_cast<int64_t>(B) * N;
    for (;;) {
        if (phase == kWalkEnter) {
            if (wave == 0) {
                const bool is_draft = lane >= 32;
                const Partial* pr = part + ((is_draft ? nbn : 0) + b * N + n) * nT;
                Partial qv[kBatch];
                group_load(pr, nT, 32, true, qv);
                int r;
                double sum;
                ArgMax am;
                if (sampled) {
                    group_reduce<true>(pr, nT, 32, true, qv, r, sum, am);
                } else {
                    group_reduce<false>(pr, nT, 32, true, qv, r, sum, am);
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
            Sd = s_norm[1];
            c = 0.0;
            Z = 1.0;
            kidx = 0;
            phase = kWalkTest;
            __syncthreads();  // s_ref and s_norm are reused at the next node
        }
#pragma unroll
        for (int q = 0; q < kRoundSlots; ++q) {
            const int i = t + q * kRoundBlock;
            const uint64_t km = __ballot(i < N && s_par[i] == n);
            if (lane == 0 && wave + q * kRoundWaves < nmask) s_kids[wave + q * kRoundWaves] = km;
        }
        __syncthreads();
        const double lsum = t == 0 && sampled ? (Rt + log2(St)) - (Rd + log2(Sd)) : 0.0;
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
                            const double l2ratio = (static_cast<double>(s_tg[i]) * cT -
                                                    static_cast<double>(s_dg[i]) * cT) - lsum;
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
    if (phase == kWalkPass || phase == kWalkPick) {
        // this workgroup's slice of the segments of node n's rows
        const int64_t row = (b * N + n) * static_cast<int64_t>(V);
        s.rt = static_cast<float>(Rt);
        s.inv_st = static_cast<float>(1.0 / St);
        s.rd = static_cast<float>(Rd);
        s.inv_sd = static_cast<float>(c / Sd);
        const bool residual = c > 0.0;
        const int64_t spc = (nseg + P - 1) / P;
        const int64_t g0 = j * spc, g1 = min<int64_t>(nseg, g0 + spc);
        double acc = 0.0;
        for (int64_t g = g0 + wave; g < g1; g += kRoundWaves) {
            float w[VE];
            walk_weights<DT, VEC>(draft, target, row, V, g, s, residual, w);
            const float m = wave_sum(pairwise_sum<VE>(w));
            if (phase == kWalkPick) {
                if (lane == 0) tsegs[b * nseg + g] = m;
            } else {
                acc += static_cast<double>(m);
            }
        }
        if (phase == kWalkPass) {
            if (lane == 0) s_wsum[wave] = acc;
            __syncthreads();
            if (t == 0) {
                double z = 0.0;
                for (int w = 0; w < kRoundWaves; ++w) z += s_wsum[w];
                z_out[b * P + j] = z;
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
        st.Sd = Sd;
        st.c = c;
        st.Z = Z;
        st_out[b] = st;
    }
}

// ---------------------------------------------------------------- commit ---

// One workgroup: thread t handles sequences t, t + 1024, ... in rounds of
// 1024; an LDS scan of the committed counts gives the packed offsets (a
// running carry links the rounds).
constexpr int kCommitBlock = 1024;

__global__ __launch_bounds__(kCommitBlock) void commit_tokens_kernel(
    int B, int width, const int32_t* __restrict__ accepted_len, const int32_t* __restrict__ emitted,
    int32_t* __restrict__ seq_len, int32_t* __restrict__ history, int history_stride,
    int32_t* __restrict__ packed_offsets, int32_t* __restrict__ packed, int32_t* __restrict__ status) {
    __shared__ int s_wave[kCommitBlock / kWave];
    __shared__ int s_carry;
    const int t = threadIdx.x;
    const int lane = lane_id();
    const int wave = t / kWave;
    if (t == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < B; base += kCommitBlock) {
        const int b = base + t;
        int n = 0, st = 0, len = 0;
        if (b < B) {
            const int a = accepted_len[b];
            len = seq_len[b];
            if (a < 0) {
                st = 2;
            } else if (a + 1 > width || len < 0 ||
                       (history != nullptr &&
                        static_cast<int64_t>(len) + a + 1 > static_cast<int64_t>(history_stride))) {
                st = 1;
            } else {
                n = a + 1;
            }
        }
        // exclusive scan of n over the block
        int incl = n;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += y;
        }
        if (lane == kWave - 1) s_wave[wave] = incl;
        __syncthreads();
        int before = s_carry;
        for (int w = 0; w < wave; ++w) before += s_wave[w];
        const int excl = before + incl - n;
        if (b < B) {
            const int32_t* src = emitted + static_cast<int64_t>(b) * width;
            for (int j = 0; j < n; ++j) {
                const int32_t tok = src[j];
                if (history) history[static_cast<int64_t>(b) * history_stride + len + j] = tok;
                if (packed) packed[excl + j] = tok;
            }
            if (n > 0) seq_len[b] = len + n;
            if (packed_offsets) packed_offsets[b] = excl;
            if (status) status[b] = st;
        }
        __syncthreads();
        if (t == kCommitBlock - 1) s_carry = excl + n;
        __syncthreads();
    }
    if (t == 0 && packed_offsets) packed_offsets[B] = s_carry;
}

}  // namespace sv
