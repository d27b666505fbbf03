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
    float c_hi;    // log2(e) / T as a double-float pair
    float c_lo;
    float u;       // u[b][k]
    float st;      // sum exp2(l c - rt) of target row a (the residual's normaliser)
    int fast;      // residual of known large mass: the cheap form suffices (kFastResidualMass)
    double kappa;  // residual: log2(c S_t / S_d) with both rows' normalisers in the reference rt
    double cT;     // log2(e) / T
    float k_hi;    // kappa as a double-float pair
    float k_lo;
    int pad[2];
};
static_assert(sizeof(SeqInfo) == 64, "descriptor layout");

// A descriptor that every lane of the wave holds alike (read from LDS or
// memory at a uniform address), moved to scalar registers: the compiler
// cannot tell that an LDS value is uniform and would keep all sixteen words
// in vector registers.
__device__ __forceinline__ SeqInfo uniform_info(const SeqInfo& s) {
    SeqInfo u;
    const int* src = reinterpret_cast<const int*>(&s);
    int* dst = reinterpret_cast<int*>(&u);
#pragma unroll
    for (int i = 0; i < static_cast<int>(sizeof(SeqInfo) / sizeof(int)); ++i)
        dst[i] = __builtin_amdgcn_readfirstlane(src[i]);
    return u;
}

// The final draw's statistics of one segment: bonus draws store the mass
// sum exp2(l c - ref) and its integer reference; residual draws store, in
// units of the target row's reference, M = sum max(0, x), X = sum x,
// E = sum of e = exp2(l_t c - r_t) over the elements with x > 0 and SW =
// sum of e over the elements with |delta| < kSwitch, where x is the
// element's residual term (see residual_term).
struct alignas(16) SegMass {
    float m;
    union {
        int ref;   // bonus: reference exponent
        float ea;  // residual: E
    };
    float x;   // residual: X
    float sw;  // residual: SW
};
static_assert(sizeof(SegMass) == 16, "segment record layout");

__device__ __forceinline__ SegMass bonus_seg(float m, int ref) {
    SegMass s;
    s.m = m;
    s.ref = ref;
    s.x = 0.f;
    s.sw = 0.f;
    return s;
}

__device__ __forceinline__ SegMass residual_seg(float m, float ea, float x, float sw) {
    SegMass s;
    s.m = m;
    s.ea = ea;
    s.x = x;
    s.sw = sw;
    return s;
}

// ---------------------------------------------------------------- residual terms ---
//
// After a rejection the final draw samples w_v = max(0, p_v - c q_v): c = 1 in
// a chain, and the running residual of a sampled tree after j rejections at a
// node has this form with c = c_j.  When the draft nearly copies the target,
// p_v and c q_v nearly cancel.  Formed separately in fp32 they leave an
// absolute error of about 1e-7 p_v per term, which moves the draw's CDF
// boundaries C / W by about 1e-7 / W for a residual of total mass W.  So each
// term is formed with an error relative to itself instead.  In units of the
// target row's reference r_t,
//   x_v = e_t - e_q,  e_t = exp2(l_t c - r_t),  e_q = exp2(l_d c - r_t + kappa)
//       = e_t (1 - 2^delta_v),  delta_v = (l_d - l_t) c + kappa,
// kappa = log2(c S_t / S_d) with both normalisers in the reference r_t
// (c = log2(e) / T).  delta_v is evaluated without cancellation error (an
// exact logit difference, then a double-float or fp64 product and sum).
// Where |delta| >= 1/8, 1 - 2^delta is at least 0.083 away from 0 and the
// difference e_t - e_q is already within about 1e-6 of x; below, x is
// e_t (-expm1(delta ln 2)) by a short series.  Every term then carries an
// error of about 1e-6 of itself or less, whatever W.  kappa itself comes from
// the normalisers, which fp32 sums know only to about 1e-7 relative; the draw
// corrects it from the row's own total X = sum_v x_v = S_t - 2^kappa S_d
// (see kappa_zeta).

// |delta| below which a term is formed by the series.
constexpr float kSeries = 0.125f;

// expm1(delta ln 2) for |delta| < kSeries: Taylor series through degree 4
// (truncation below 5e-7 relative).
__device__ __forceinline__ float expm1_2(float d) {
    float s = __builtin_fmaf(d, 9.61812910762847716e-3f, 5.55041086648215800e-2f);
    s = __builtin_fmaf(d, s, 2.40226506959100712e-1f);
    s = __builtin_fmaf(d, s, 6.93147180559945309e-1f);
    return d * s;
}

// delta = (l_d - l_t) log2(e) / T + kappa.  bfloat16 logits differ exactly in
// fp32 (unless their exponents lie more than 15 apart), and the products with
// the double-float scale and offset then carry the cancellation exactly inside
// the fma; float32 logits take the difference and the product in fp64.
template <int DT>
__device__ __forceinline__ float residual_delta(float lt, float ld, const SeqInfo& s);

template <>
__device__ __forceinline__ float residual_delta<SV_BF16>(float lt, float ld, const SeqInfo& s) {
    const float d = ld - lt;
    return __builtin_fmaf(d, s.c_hi, s.k_hi) + __builtin_fmaf(d, s.c_lo, s.k_lo);
}

template <>
__device__ __forceinline__ float residual_delta<SV_F32>(float lt, float ld, const SeqInfo& s) {
    return static_cast<float>(__builtin_fma(static_cast<double>(ld) - static_cast<double>(lt), s.cT, s.kappa));
}

// One element's residual term x (see above) and its e_t and delta.  l_t must
// be finite (masked elements are handled by the callers).
template <int DT>
__device__ __forceinline__ float residual_term(float lt, float ld, const SeqInfo& s, float& et, float& delta) {
    delta = residual_delta<DT>(lt, ld, s);
    const float a = __builtin_fmaf(lt, s.c_lo, __builtin_fmaf(lt, s.c_hi, -s.rt));
    et = __builtin_amdgcn_exp2f(a);
    const float eq = __builtin_amdgcn_exp2f(a + delta);
    const float small = -(et * expm1_2(delta));
    return __builtin_fabsf(delta) < kSeries ? small : et - eq;
}

// A residual whose mass W is known to be at least kFastResidualMass needs
// neither the series nor the sums behind the correction of kappa.  Each term
// is formed as x = e_t (1 - 2^min(delta, 0)), from the same accurate delta as
// residual_term: e_t carries a relative error of about 6e-8 (2 + |a| ln 2)
// (the exponential and its rounded exponent a), which stays relative to x;
// 2^delta an absolute error of about 1.2e-7 and delta's own relative error
// (1e-7) adds at most about 1e-7 more, both times e_t, so the terms of W
// together are off by at most about 3e-7 S_t + 1e-6 W S_t, and the
// normalisers' fp32 error (kappa to about 1e-7, uncorrected here) adds about
// 1e-7 S_t.  The CDF boundaries C / W then move by at most twice that over W
// S_t: about 6e-6 at W = 0.2, inside the 1e-5 band.  The acceptance has two
// lower bounds of W = TV(p, q): q(x) - p(x) at the rejected draft x, and the
// distance between the two rows' tile masses (tile_tv).
constexpr double kFastResidualMass = 0.2;

// M = sum max(0, x) of VE elements, each x = e_t (1 - 2^min(delta, 0)) (see
// above; masked elements weigh 0).
template <int DT, int VE, bool FULL>
__device__ __forceinline__ float residual_mass_fast(const float* vt, const float* vd, const SeqInfo& s) {
    float mm[VE];
#pragma unroll
    for (int j = 0; j < VE; ++j) {
        const float delta = residual_delta<DT>(vt[j], vd[j], s);
        const float a = __builtin_fmaf(vt[j], s.c_lo, __builtin_fmaf(vt[j], s.c_hi, -s.rt));
        const float et = __builtin_amdgcn_exp2f(a);
        const float x = __builtin_fmaf(-et, __builtin_amdgcn_exp2f(__builtin_fminf(delta, 0.f)), et);
        mm[j] = (FULL || vt[j] != -__builtin_inff()) ? x : 0.f;
    }
    return pairwise_sum<VE>(mm);
}

// Residual weights max(0, x) of NE loaded elements (masked elements weigh 0).
template <int DT, int NE, bool FULL>
__device__ __forceinline__ void residual_weights(const float* vt, const float* vd, const SeqInfo& s, float* w) {
#pragma unroll
    for (int j = 0; j < NE; ++j) {
        float et, delta;
        const float x = residual_term<DT>(vt[j], vd[j], s, et, delta);
        w[j] = (FULL || vt[j] != -__builtin_inff()) ? __builtin_fmaxf(x, 0.f) : 0.f;
    }
}

// |delta| below which an element's term may change sign when kappa is
// corrected (see kappa_zeta): a bound on the correction, which fp32
// normalisers and the terms' own errors keep below about 1e-6.
constexpr float kSwitch = 1.9073486328125e-6f;  // 2^-19

// The residual sums of one segment's VE elements held by this lane: M = sum
// max(0, x), E = sum of e_t over the elements with x > 0, X = sum x and SW =
// sum of e_t over the elements with |delta| < kSwitch (masked elements
// contribute nothing).
struct ResidualSums {
    float m, ea, x, sw;
};

template <int DT, int VE, bool FULL>
__device__ __forceinline__ ResidualSums residual_sums(const float* vt, const float* vd, const SeqInfo& s) {
    float mm[VE], ee[VE], xx[VE], ss[VE];
#pragma unroll
    for (int j = 0; j < VE; ++j) {
        float et, delta;
        float t = residual_term<DT>(vt[j], vd[j], s, et, delta);
        if (!FULL && vt[j] == -__builtin_inff()) t = et = 0.f;
        xx[j] = t;
        mm[j] = __builtin_fmaxf(t, 0.f);
        ee[j] = delta < 0.f ? et : 0.f;
        ss[j] = __builtin_fabsf(delta) < kSwitch ? et : 0.f;
    }
    return ResidualSums{pairwise_sum<VE>(mm), pairwise_sum<VE>(ee), pairwise_sum<VE>(xx), pairwise_sum<VE>(ss)};
}

// The same sums without SW: elements within kSwitch of the switch are rare,
// so a streaming pass only tracks the smallest |delta| of the lane in
// `dmin` and forms SW with residual_sw, in a branch, for the tiles of waves
// that have one.  M, E and X are the same as residual_sums'.
template <int DT, int VE, bool FULL>
__device__ __forceinline__ ResidualSums residual_sums_marked(const float* vt, const float* vd, const SeqInfo& s,
                                                             float& dmin) {
    float mm[VE], ee[VE], xx[VE];
#pragma unroll
    for (int j = 0; j < VE; ++j) {
        float et, delta;
        float t = residual_term<DT>(vt[j], vd[j], s, et, delta);
        if (!FULL && vt[j] == -__builtin_inff()) t = et = 0.f;
        xx[j] = t;
        mm[j] = __builtin_fmaxf(t, 0.f);
        ee[j] = delta < 0.f ? et : 0.f;
        dmin = __builtin_fminf(dmin, __builtin_fabsf(delta));
    }
    return ResidualSums{pairwise_sum<VE>(mm), pairwise_sum<VE>(ee), pairwise_sum<VE>(xx), 0.f};
}

// SW of VE elements (residual_sums' value).
template <int DT, int VE, bool FULL>
__device__ __forceinline__ float residual_sw(const float* vt, const float* vd, const SeqInfo& s) {
    float ss[VE];
#pragma unroll
    for (int j = 0; j < VE; ++j) {
        const float delta = residual_delta<DT>(vt[j], vd[j], s);
        const float a = __builtin_fmaf(vt[j], s.c_lo, __builtin_fmaf(vt[j], s.c_hi, -s.rt));
        const float et = __builtin_amdgcn_exp2f(a);
        ss[j] = (FULL || vt[j] != -__builtin_inff()) && __builtin_fabsf(delta) < kSwitch ? et : 0.f;
    }
    return pairwise_sum<VE>(ss);
}

// The correction of kappa from a residual pass at c = 1: X = sum_v x_v =
// S_t (1 - 2^(kappa_used - kappa_true)), so kappa_true = kappa_used + zeta /
// ln 2 with zeta = -ln(1 - X / S_t), accurate to a few 1e-6 of the residual's
// mass W whatever W (each x_v carries an error of about 1e-6 of itself, and
// sum |x_v| = 2 W S_t).  To first order in zeta every term with x > 0 moves
// by -zeta (e_t - x), so a segment's mass becomes M - zeta (E - M); zeta is
// of the order of 1e-7, so second-order terms (1e-14) do not matter.  What
// the first order misses are terms that change sign, those with |delta| <
// |zeta| / ln 2, each by at most 2 |zeta| e_t.  The correction is therefore
// trusted only when |zeta| / ln 2 <= kSwitch and 2 |zeta| SW <= kRedoTol
// times the corrected mass; otherwise the masses are formed again with the
// corrected kappa.
__device__ __forceinline__ double kappa_zeta(double X, double St) {
    const double y = X / St;  // |y| of the order of 1e-7: -ln(1 - y) to within 1e-21
    return y + 0.5 * y * y;
}

constexpr double kRedoTol = 1e-7;

__device__ __forceinline__ bool correction_trusted(double zeta, double sw, double mass) {
    return fabs(zeta) <= static_cast<double>(kSwitch) * 0.69314718055994530942 &&
           2.0 * fabs(zeta) * sw <= kRedoTol * mass;
}

// Sets kappa and its double-float forms.
__device__ __forceinline__ void set_kappa(SeqInfo& s, double kappa) {
    s.kappa = kappa;
    s.k_hi = static_cast<float>(kappa);
    s.k_lo = static_cast<float>(kappa - static_cast<double>(s.k_hi));
}

constexpr double kLn2 = 0.69314718055994530942;

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

// The descriptor's temperature fields from c = log2(e) / T: the double-float
// pair and the double.
__device__ __forceinline__ void temperature_scale_from(double c, SeqInfo& s) {
    s.c_hi = static_cast<float>(c);
    s.c_lo = static_cast<float>(c - static_cast<double>(s.c_hi));
    s.cT = c;
}

__device__ __forceinline__ void temperature_scale(float T, SeqInfo& s) {
    temperature_scale_from(kLog2e / static_cast<double>(T), s);
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
    // the lane's best element by its position in v (a constant per
    // comparison, so no index arithmetic per element), then its row index
    float best = -__builtin_inff();
    int pos = -1;
#pragma unroll
    for (int j = 0; j < U * VE; ++j) {
        if (v[j] > best) {
            best = v[j];
            pos = j;
        }
    }
    const int64_t v0 = tile * (64 * U) + lane;
    const int idx = pos < 0 ? kNoIndex : static_cast<int>((v0 + (pos / VE) * 64) * VE + pos % VE);
    return wave_argmax(ArgMax{best, idx});
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

// Partials handed from one workgroup to another inside a launch.  Each slot
// is two 8-byte words, (f, t0) and (i, t1), written with relaxed
// device-scope atomic stores and read with relaxed device-scope atomic
// loads; (t0, t1) is a tag unique to the call (CallTag).  A reader takes a
// slot once both words carry the call's tag: each word is one atomic
// access, so it then holds this call's value, and no fence is needed (on
// this GPU a device-scope release or acquire writes back or invalidates a
// whole L2).  Words left by an earlier call, by other use of the memory or
// by nothing carry another tag; a tag is 64 bits, so unrelated bytes pass
// for the call's own with probability 2^-64 per slot.
struct TaggedPartial {
    uint64_t w[2];
};
static_assert(sizeof(TaggedPartial) == 16, "a tagged partial is two atomic words");

struct CallTag {
    uint32_t t0, t1;
};

__device__ __forceinline__ void store_partial_tagged(TaggedPartial* p, Partial v, CallTag tag) {
    const uint64_t w0 = (static_cast<uint64_t>(tag.t0) << 32) | __builtin_bit_cast(uint32_t, v.f);
    const uint64_t w1 = (static_cast<uint64_t>(tag.t1) << 32) | static_cast<uint32_t>(v.i);
    __hip_atomic_store(&p->w[0], w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p->w[1], w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whether slot p holds this call's partial; if so, it is in v.
__device__ __forceinline__ bool load_partial_tagged(const TaggedPartial* p, CallTag tag, Partial& v) {
    const uint64_t w0 = __hip_atomic_load(&p->w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t w1 = __hip_atomic_load(&p->w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v.f = __builtin_bit_cast(float, static_cast<uint32_t>(w0));
    v.i = static_cast<int>(static_cast<uint32_t>(w1));
    return static_cast<uint32_t>(w0 >> 32) == tag.t0 && static_cast<uint32_t>(w1 >> 32) == tag.t1;
}

// Sets n tagged partial slots to zero words (tag (0, 0), which no call
// uses), ahead of a launch that hands partials over in them when its stream
// is being captured into a graph, whose replays all carry one tag.
__global__ __launch_bounds__(kBlock) void clear_slots_kernel(TaggedPartial* __restrict__ slots, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (i < n) slots[i] = TaggedPartial{{0, 0}};
}

// Sleep between two reads of published partials (s_sleep units of 64 clocks).
constexpr int kPollSleep = 8;

// group_load's slots (lane l: row l / G, tiles l % G + j G, every tile of
// the row in one load; the lane's row's nT slots at row_slots) filled from
// partials that other workgroups of the launch publish with
// store_partial_tagged: read until all carry the call's tag, at most `polls`
// times with a short sleep between reads.  A partial still missing after
// that is computed by the whole wave with late(rho, tile), which gives the
// publishing wave's own value.  The slots wait in LDS (s_q, kBatch * 64
// partials) meanwhile, which keeps that rare path's registers within the
// kernel's budget.  When the launch's workgroups start in index order none is
// missing by then: the publishing workgroups come first in the grid and wait
// on nothing.  Waves that share one s_q must not both hold partials.
template <class Late>
__device__ __forceinline__ void await_slots(const TaggedPartial* row_slots, bool valid, int nT, int G, CallTag tag,
                                            int polls, Partial* q, Partial* s_q, Late late) {
    const int lane = lane_id();
    const int sl = lane & (G - 1);
    unsigned have = 0;  // bit j: q[j] holds its partial (or the lane has no partial j)
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        q[j] = Partial{0.f, 0};
        if (!valid || sl + j * G >= nT) have |= 1u << j;
    }
    constexpr unsigned kAll = (1u << kBatch) - 1;
    // a wave that holds no partial (every slot invalid) leaves at once, so it
    // never touches s_q, which may be another wave's
    bool any = __builtin_amdgcn_ballot_w64(have != kAll) != 0;
    for (int it = 0; it < polls && any; ++it) {
        if (it > 0) __builtin_amdgcn_s_sleep(kPollSleep);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (!((have >> j) & 1u) && load_partial_tagged(row_slots + sl + j * G, tag, q[j])) have |= 1u << j;
        }
        any = __builtin_amdgcn_ballot_w64(have != kAll) != 0;
    }
    if (!any) return;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) s_q[j * kWave + lane] = q[j];
    __builtin_amdgcn_wave_barrier();
#pragma unroll 1
    for (int j = 0; j < kBatch; ++j) {
        uint64_t m = __builtin_amdgcn_ballot_w64(!((have >> j) & 1u));
        while (m != 0) {
            const int l = __builtin_ctzll(m);
            m &= m - 1;
            const Partial p = late(l / G, static_cast<int64_t>((l & (G - 1)) + j * G));
            if (lane == l) s_q[j * kWave + l] = p;
        }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < kBatch; ++j) q[j] = s_q[j * kWave + lane];
}

// Small calls run in one launch, one workgroup of kSmallBlock threads per
// sequence, with at most kSmallMaxParts row tiles held in LDS.
constexpr int kSmallBlock = 1024;
constexpr int kSmallWaves = kSmallBlock / kWave;
constexpr int kSmallMaxParts = 160;

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

// Half the L1 distance between the tile masses of target row i and draft
// row i, over the tiles of the first kBatch partials of each lane of the
// group (t = l % G + j G), summed over the group: a lower bound of the
// total variation distance TV(p_i, q_i), since merging tokens into tiles can
// only lower it, and so can leaving tiles out.  The target rows' groups are
// the first k, each followed k groups later by its draft row's; the result
// holds in the lanes of target row i's group.  (r, s) is the lane's row's
// combined normaliser, `valid` whether the lane's row is a tested one.
__device__ __forceinline__ float tile_tv(const Partial* q, int nT, int G, bool valid, int r, double s, int k) {
    const int lane = lane_id();
    const int sl = lane & (G - 1);
    const float inv = valid ? __builtin_amdgcn_rcpf(static_cast<float>(s)) : 0.f;  // a bound: 1 ulp suffices
    const int src = min(lane + k * G, kWave - 1);  // the draft row's lane (target lanes only)
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const float m = sl + j * G < nT ? __builtin_ldexpf(q[j].f, q[j].i - r) * inv : 0.f;
        acc += __builtin_fabsf(m - __shfl(m, src, kWave));
    }
    for (int m = G >> 1; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kWave);
    return 0.5f * acc;
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
