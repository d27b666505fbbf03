// sv_common.hpp -- device helpers shared by the libspecverify kernels (gfx950).
//
// Row geometry.  A logits row of V elements is read as NV = ceil(V / VE)
// "vectors" of VE = 16 / sizeof(element) consecutive elements.  When every row
// starts on a 16-byte boundary (V * element size a multiple of 16 and a
// 16-byte aligned base) a vector is one 128-bit load; otherwise it is VE
// element loads masked against V.  A wave64 owns a *tile* of 64 * U
// consecutive vectors; lane l of the wave reads vectors tile*64U + i*64 + l
// for i < U, so each of the U load instructions of a wave touches 64
// consecutive 16-byte vectors (1 KiB, fully coalesced), and the 64 vectors
// touched by load i form a *segment* of 64 * VE consecutive tokens.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kNoIndex = 0x7fffffff;

template <int DT>
struct Elem;
template <>
struct Elem<SV_F32> {
    static constexpr int bytes = 4;
    static constexpr int per_vec = 4;
    static constexpr uint32_t neg_inf_word = 0xff800000u;  // -inf
};
template <>
struct Elem<SV_BF16> {
    static constexpr int bytes = 2;
    static constexpr int per_vec = 8;
    static constexpr uint32_t neg_inf_word = 0xff80ff80u;  // two bf16 -inf
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- loads ---

// The 16-byte vector vi of a row whose first element is at byte `row`
// (16-byte aligned).  Vectors past the row end (vi >= nv) read as -inf.
__device__ __forceinline__ uint4 load_vec_aligned(const char* row, int64_t vi, int64_t nv,
                                                  uint32_t neg_inf) {
    if (vi < nv) return *reinterpret_cast<const uint4*>(row + vi * 16);
    return make_uint4(neg_inf, neg_inf, neg_inf, neg_inf);
}

// Unpack a 16-byte vector into VE floats.
template <int DT>
__device__ __forceinline__ void unpack(const uint4 w, float* out);

template <>
__device__ __forceinline__ void unpack<SV_F32>(const uint4 w, float* out) {
    out[0] = __uint_as_float(w.x);
    out[1] = __uint_as_float(w.y);
    out[2] = __uint_as_float(w.z);
    out[3] = __uint_as_float(w.w);
}

// bfloat16 -> float is exact: the bf16 bits become the upper half of a binary32.
template <>
__device__ __forceinline__ void unpack<SV_BF16>(const uint4 w, float* out) {
    out[0] = __uint_as_float(w.x << 16);
    out[1] = __uint_as_float(w.x & 0xffff0000u);
    out[2] = __uint_as_float(w.y << 16);
    out[3] = __uint_as_float(w.y & 0xffff0000u);
    out[4] = __uint_as_float(w.z << 16);
    out[5] = __uint_as_float(w.z & 0xffff0000u);
    out[6] = __uint_as_float(w.w << 16);
    out[7] = __uint_as_float(w.w & 0xffff0000u);
}

// One element of a row, as float.
template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx);
template <>
__device__ __forceinline__ float load_elem<SV_F32>(const void* base, int64_t idx) {
    return static_cast<const float*>(base)[idx];
}
template <>
__device__ __forceinline__ float load_elem<SV_BF16>(const void* base, int64_t idx) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16);
}

// Vector vi of a row (element offset `row_elem` into `base`, V elements) as VE
// floats, with element loads masked against V: the path for rows that are not
// 16-byte aligned.
template <int DT>
__device__ __forceinline__ void load_vec_masked(const void* base, int64_t row_elem, int64_t vi,
                                                int V, float* out) {
    constexpr int VE = Elem<DT>::per_vec;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        const int64_t j = vi * VE + e;
        out[e] = (j < V) ? load_elem<DT>(base, row_elem + j) : -__builtin_inff();
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A 16-byte load marked non-temporal: the streaming passes read every logit
// exactly once, and the hint measurably raises their achieved bandwidth.
__device__ __forceinline__ uint4 load_nt(const char* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// U vectors of lane `lane` of tile `tile`, unpacked into U*VE floats.
// FULL (only with VEC): the whole tile lies inside the row, so the loads need
// no mask.  Otherwise elements past the row end read as -inf.  NT: load with
// the non-temporal hint (full tiles only).
template <int DT, bool VEC, int U, bool FULL = false, bool NT = false>
__device__ __forceinline__ void load_tile(const void* base, int64_t row_elem, int V, int64_t tile,
                                          int lane, float* v) {
    constexpr int VE = Elem<DT>::per_vec;
    const int64_t nv = (V + VE - 1) / VE;
    const int64_t v0 = tile * (64 * U) + lane;
    if constexpr (VEC) {
        const char* row = static_cast<const char*>(base) + row_elem * Elem<DT>::bytes;
        uint4 raw[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if constexpr (FULL && NT)
                raw[i] = load_nt(row + (v0 + i * 64) * 16);
            else if constexpr (FULL)
                raw[i] = *reinterpret_cast<const uint4*>(row + (v0 + i * 64) * 16);
            else
                raw[i] = load_vec_aligned(row, v0 + i * 64, nv, Elem<DT>::neg_inf_word);
        }
#pragma unroll
        for (int i = 0; i < U; ++i) unpack<DT>(raw[i], v + i * VE);
    } else {
        static_assert(!FULL, "element loads are always masked");
#pragma unroll
        for (int i = 0; i < U; ++i) load_vec_masked<DT>(base, row_elem, v0 + i * 64, V, v + i * VE);
    }
}

// Whether tile `tile` of U vectors per lane lies entirely inside a row of nv
// vectors (and may take the unmasked path).
template <bool VEC, int U>
__device__ __forceinline__ bool tile_is_full(int64_t tile, int V, int ve) {
    if constexpr (!VEC) return false;
    const int64_t nv = (V + ve - 1) / ve;
    return (tile + 1) * (64 * U) <= nv;
}

// ---------------------------------------------------------------- arithmetic ---

// Pairwise (tree) sum of N register values; N a power of two.
template <int N>
__device__ __forceinline__ float pairwise_sum(const float* x) {
    if constexpr (N == 1) {
        return x[0];
    } else {
        return pairwise_sum<N / 2>(x) + pairwise_sum<N / 2>(x + N / 2);
    }
}

// exp2(l * c - r) with c = c_hi + c_lo (a double-float split of log2(e) / T)
// and an integer-valued reference r: the product l * c_hi is exact inside the
// fma, so the argument carries about one rounding of its own (small) value.
// l must be finite (c_lo may be negative: -inf would give inf - inf).
__device__ __forceinline__ float scaled_exp2(float l, float c_hi, float c_lo, float r) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(l, c_lo, __builtin_fmaf(l, c_hi, -r)));
}

// The same term for a possibly masked element: masked (-inf) elements weigh 0.
template <bool FULL>
__device__ __forceinline__ float exp_term(float l, float c_hi, float c_lo, float r) {
    if constexpr (FULL) return scaled_exp2(l, c_hi, c_lo, r);
    return l == -__builtin_inff() ? 0.f : scaled_exp2(l, c_hi, c_lo, r);
}

// ---------------------------------------------------------------- wave64 reductions ---
//
// Reductions of 32-bit values use DPP row operations, which exchange registers
// without going through the LDS crossbar: quad permutes (lane ^ 1, lane ^ 2),
// half-row and row mirrors (which pair the groups of 4 and of 8 lanes once
// their values agree), then row_bcast15 / row_bcast31 to fold the four rows of
// 16 lanes into lane 63, read back as a wave-uniform value.  The order of the
// operations is fixed, so results are deterministic.

namespace dpp {
constexpr int kXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror
constexpr int kMirror = 0x140;      // row_mirror
constexpr int kBcast15 = 0x142;     // row_bcast:15 (rows 1 and 3 enabled below)
constexpr int kBcast31 = 0x143;     // row_bcast:31 (rows 2 and 3 enabled below)
constexpr int kRor4 = 0x124;        // row_ror:4
constexpr int kRor8 = 0x128;        // row_ror:8
}  // namespace dpp

// DPP move of v; lanes of rows outside ROW_MASK receive `identity`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_move(int identity, int v) {
    return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_move(float identity, float v) {
    return __int_as_float(dpp_move<CTRL, ROW_MASK>(__float_as_int(identity), __float_as_int(v)));
}

template <typename T, typename Op>
__device__ __forceinline__ T dpp_reduce(T v, T identity, Op op) {
    v = op(v, dpp_move<dpp::kXor1>(identity, v));
    v = op(v, dpp_move<dpp::kXor2>(identity, v));
    v = op(v, dpp_move<dpp::kHalfMirror>(identity, v));
    v = op(v, dpp_move<dpp::kMirror>(identity, v));
    v = op(v, dpp_move<dpp::kBcast15, 0xa>(identity, v));
    v = op(v, dpp_move<dpp::kBcast31, 0xc>(identity, v));
    return v;  // the reduction of all 64 lanes is in lane 63
}

__device__ __forceinline__ float lane63(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63)); }
__device__ __forceinline__ int lane63(int v) { return __builtin_amdgcn_readlane(v, 63); }

// Sum of the wave's values, returned to every lane.
__device__ __forceinline__ float wave_sum(float x) {
    return lane63(dpp_reduce(x, 0.f, [](float a, float b) { return a + b; }));
}

// Sums over the wave of four values per lane, as a reduce-scatter: two
// quad-permute steps leave each lane the sum over its quad of one of the four
// (index 2 * (lane & 1) + ((lane >> 1) & 1), returned in idx), two row
// rotations add the row's four quads and two shuffles the wave's four rows.
// Every lane ends with the total of its index; lanes 0..3 hold all four.
// About 20 operations instead of four full reductions.
__device__ __forceinline__ float wave_sum4(const float* a, int& idx) {
    const int lane = lane_id();
    const bool odd = lane & 1, hi = lane & 2;
    // lane ^ 1: even lanes keep values 0 and 1, odd lanes 2 and 3
    float k0 = odd ? a[2] : a[0], k1 = odd ? a[3] : a[1];
    k0 += dpp_move<dpp::kXor1>(0.f, odd ? a[0] : a[2]);
    k1 += dpp_move<dpp::kXor1>(0.f, odd ? a[1] : a[3]);
    // lane ^ 2: keep one of the two
    float keep = hi ? k1 : k0;
    keep += dpp_move<dpp::kXor2>(0.f, hi ? k0 : k1);
    keep += dpp_move<dpp::kRor4>(0.f, keep);
    keep += dpp_move<dpp::kRor8>(0.f, keep);
    keep += __shfl_xor(keep, 16, kWave);
    keep += __shfl_xor(keep, 32, kWave);
    idx = 2 * (odd ? 1 : 0) + (hi ? 1 : 0);
    return keep;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
    return lane63(dpp_reduce(x, -__builtin_inff(), [](float a, float b) { return fmaxf(a, b); }));
}

__device__ __forceinline__ int wave_max(int x) {
    return lane63(dpp_reduce(x, static_cast<int>(0x80000000), [](int a, int b) { return max(a, b); }));
}

// (value, index) maximum with ties resolved to the lowest index.
struct ArgMax {
    float val;
    int idx;
};

__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
    return (b.val > a.val || (b.val == a.val && b.idx < a.idx)) ? b : a;
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ ArgMax argmax_step(ArgMax a) {
    const ArgMax o{dpp_move<CTRL, ROW_MASK>(-__builtin_inff(), a.val), dpp_move<CTRL, ROW_MASK>(kNoIndex, a.idx)};
    return better(a, o);
}

// (max, lowest index) over the wave, returned to every lane.
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
    a = argmax_step<dpp::kXor1>(a);
    a = argmax_step<dpp::kXor2>(a);
    a = argmax_step<dpp::kHalfMirror>(a);
    a = argmax_step<dpp::kMirror>(a);
    a = argmax_step<dpp::kBcast15, 0xa>(a);
    a = argmax_step<dpp::kBcast31, 0xc>(a);
    return ArgMax{lane63(a.val), lane63(a.idx)};
}

// Inclusive prefix sum across the wave (Hillis-Steele, fixed order).
__device__ __forceinline__ double wave_inclusive_scan(double x) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const double y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    return x;
}

// Index of the lowest lane whose predicate holds, or -1.
__device__ __forceinline__ int first_lane(bool pred) {
    const uint64_t m = __ballot(pred);
    return m ? __builtin_ctzll(m) : -1;
}

// Per-(row, tile) partial result written by the streaming passes: softmax
// mode stores (s, r) with s = sum exp2(l c - r) over the tile and r an
// integer-valued reference; argmax mode stores (max value, lowest index).
struct Partial {
    float f;
    int i;
};

}  // namespace sv
