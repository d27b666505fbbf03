// sv_tiles.hpp -- descriptors shared by the kernels, wave-tile reductions and the
// combination of per-tile partials (part of sv_kernels.hpp).
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

// The argmax of a row from its nT partials, the whole wave striding over them.
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

}  // namespace sv
