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
//              prefix and a descriptor of the final draw;
//   final_part streams only the row(s) the final draw needs (target and draft
//              row a at a rejection, target row k after full acceptance) and
//              writes the residual mass of every 64-vector segment;
//   final_pick one wave per sequence: prefix over the segment masses, picks
//              the segment holding u * W and rescans only that segment to find
//              the token.
// sv_verify_greedy and sv_verify_tree use argmax_rows (the streaming argmax)
// followed by a per-sequence finaliser.
//
// Scheme: "Accelerating Sonar through speculation" (Perplexity, 2025),
// sections "Speculative decoding", "Target-Draft" and "EAGLE"; acceptance
// and residual rule of Leviathan et al., first in that page's references.
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

__device__ __forceinline__ void temperature_scale(float T, float& c_hi, float& c_lo) {
    const double c = kLog2e / static_cast<double>(T);
    c_hi = static_cast<float>(c);
    c_lo = static_cast<float>(c - static_cast<double>(c_hi));
}

// ---------------------------------------------------------------- wave tiles ---

// Softmax partial of one tile: s = sum_v exp2(l_v c - r) with r = ceil(max l c)
// taken over the whole tile, so exp2 never exceeds ~1 and never overflows.
template <int DT, bool VEC, int U, bool FULL>
__device__ __forceinline__ Partial tile_softmax(const void* base, int64_t row_elem, int V, int64_t tile,
                                                float c_hi, float c_lo) {
    constexpr int NE = U * Elem<DT>::per_vec;
    float v[NE];
    load_tile<DT, VEC, U, FULL>(base, row_elem, V, tile, lane_id(), v);
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

// (max, lowest index) of one tile of raw logits.
template <int DT, bool VEC, int U, bool FULL>
__device__ __forceinline__ ArgMax tile_argmax(const void* base, int64_t row_elem, int V, int64_t tile) {
    constexpr int VE = Elem<DT>::per_vec;
    constexpr int NE = U * VE;
    const int lane = lane_id();
    float v[NE];
    load_tile<DT, VEC, U, FULL>(base, row_elem, V, tile, lane, v);
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

// Tile entry points that pick the unmasked path for tiles inside the row.
template <int DT, bool VEC, int U>
__device__ __forceinline__ Partial tile_softmax_any(const void* base, int64_t row_elem, int V, int64_t tile,
                                                    float c_hi, float c_lo) {
    if (tile_is_full<VEC, U>(tile, V, Elem<DT>::per_vec))
        return tile_softmax<DT, VEC, U, VEC>(base, row_elem, V, tile, c_hi, c_lo);
    return tile_softmax<DT, VEC, U, false>(base, row_elem, V, tile, c_hi, c_lo);
}

template <int DT, bool VEC, int U>
__device__ __forceinline__ ArgMax tile_argmax_any(const void* base, int64_t row_elem, int V, int64_t tile) {
    if (tile_is_full<VEC, U>(tile, V, Elem<DT>::per_vec))
        return tile_argmax<DT, VEC, U, VEC>(base, row_elem, V, tile);
    return tile_argmax<DT, VEC, U, false>(base, row_elem, V, tile);
}

// Combine the nT softmax partials of one row: R = max r_t, S = sum s_t 2^(r_t - R).
__device__ inline void combine_softmax(const Partial* p, int nT, int& R, double& S) {
    int r = p[0].i;
    for (int t = 1; t < nT; ++t) r = max(r, p[t].i);
    double s = 0.0;
    for (int t = 0; t < nT; ++t) s += ldexp(static_cast<double>(p[t].f), p[t].i - r);
    R = r;
    S = s;
}

// Combine the nT argmax partials of one row (one lane, sequential).
__device__ inline ArgMax combine_argmax(const Partial* p, int nT) {
    ArgMax a{p[0].f, p[0].i};
    for (int t = 1; t < nT; ++t) a = better(a, ArgMax{p[t].f, p[t].i});
    return a;
}

// The same, with the whole wave striding over the tiles.
__device__ inline ArgMax wave_combine_argmax(const Partial* p, int nT) {
    ArgMax a{-__builtin_inff(), kNoIndex};
    for (int t = lane_id(); t < nT; t += kWave) a = better(a, ArgMax{p[t].f, p[t].i});
    return wave_argmax(a);
}

__device__ __forceinline__ int64_t global_wave() {
    return static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave;
}

// ---------------------------------------------------------------- chain: rowstats ---

// Rows 0 .. B*k-1 are target rows (b, j < k); rows B*k .. 2*B*k-1 are draft
// rows (b, i).  Draft rows of temperature-0 sequences are not needed (the
// one-hot target decides alone) and are skipped.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void chain_rowstats_kernel(const void* __restrict__ target,
                                                                const void* __restrict__ draft,
                                                                const float* __restrict__ temperature,
                                                                int B, int k, int V, int nT,
                                                                Partial* __restrict__ part) {
    const int64_t gw = global_wave();
    const int64_t nbk = static_cast<int64_t>(B) * k;
    if (gw >= 2 * nbk * nT) return;
    const int64_t r = gw / nT;
    const int64_t tile = gw - r * nT;
    const bool is_target = r < nbk;
    const int64_t rr = is_target ? r : r - nbk;
    const int64_t b = rr / k;
    const float T = temperature[b];
    const void* base = is_target ? target : draft;
    const int64_t row_elem = (is_target ? (b * (k + 1) + (rr - b * k)) : rr) * static_cast<int64_t>(V);
    Partial p;
    if (T > 0.f) {
        float c_hi, c_lo;
        temperature_scale(T, c_hi, c_lo);
        p = tile_softmax_any<DT, VEC, U>(base, row_elem, V, tile, c_hi, c_lo);
    } else {
        if (!is_target) return;
        const ArgMax a = tile_argmax_any<DT, VEC, U>(base, row_elem, V, tile);
        p = Partial{a.val, a.idx};
    }
    if (lane_id() == 0) part[r * nT + tile] = p;
}

// ---------------------------------------------------------------- chain: accept ---

template <int DT>
__global__ __launch_bounds__(kWave) void chain_accept_kernel(
    const int32_t* __restrict__ tokens, const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, int B, int k, int V, int nT,
    const Partial* __restrict__ part, SeqInfo* __restrict__ info, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ emitted, float* __restrict__ accept_prob) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const float T = temperature[b];
    const int64_t nbk = static_cast<int64_t>(B) * k;
    bool acc = true;
    double tau = 1.0;
    int x = 0, g = -1, rt = 0, rd = 0;
    double st = 1.0, sd = 1.0;
    if (lane < k) {
        x = tokens[static_cast<int64_t>(b) * k + lane];
        const Partial* pt = part + (static_cast<int64_t>(b) * k + lane) * nT;
        if (static_cast<unsigned>(x) >= static_cast<unsigned>(V)) {
            // a token id outside the vocabulary is never gathered: it is rejected
            acc = false;
            tau = 0.0;
        } else if (T > 0.f) {
            const Partial* pd = part + (nbk + static_cast<int64_t>(b) * k + lane) * nT;
            combine_softmax(pt, nT, rt, st);
            combine_softmax(pd, nT, rd, sd);
            const double c = kLog2e / static_cast<double>(T);
            const double lt = load_elem<DT>(target, (static_cast<int64_t>(b) * (k + 1) + lane) * V + x);
            const double ld = load_elem<DT>(draft, (static_cast<int64_t>(b) * k + lane) * V + x);
            // log2 p - log2 q with log2 p = l c - R - log2 S (same for q)
            const double l2ratio = (lt * c - rt - log2(st)) - (ld * c - rd - log2(sd));
            tau = exp2(fmin(0.0, l2ratio));
            acc = static_cast<double>(uniforms[static_cast<int64_t>(b) * (k + 1) + lane]) < tau;
        } else {
            g = combine_argmax(pt, nT).idx;
            acc = (x == g);
            tau = acc ? 1.0 : 0.0;
        }
    }
    int a = first_lane(lane < k && !acc);
    if (a < 0) a = k;
    if (accept_prob != nullptr && lane < k) accept_prob[static_cast<int64_t>(b) * k + lane] = static_cast<float>(tau);
    int32_t* out = emitted + static_cast<int64_t>(b) * (k + 1);
    for (int j = lane; j <= k; j += kWave) out[j] = j < a ? tokens[static_cast<int64_t>(b) * k + j] : -1;
    if (lane == (a < k ? a : 0)) {
        SeqInfo s{};
        s.a = a;
        temperature_scale(T > 0.f ? T : 1.f, s.c_hi, s.c_lo);
        s.u = uniforms[static_cast<int64_t>(b) * (k + 1) + k];
        if (!(T > 0.f)) {
            if (a < k) {
                out[a] = g;
                s.mode = kFinalDone;
            } else {
                s.mode = kFinalArgmax;
            }
        } else if (a < k) {
            s.mode = kFinalResidual;
            s.rt = static_cast<float>(rt);
            s.inv_st = static_cast<float>(1.0 / st);
            s.rd = static_cast<float>(rd);
            s.inv_sd = static_cast<float>(1.0 / sd);
        } else {
            s.mode = kFinalBonus;
        }
        info[b] = s;
    }
    if (lane == 0) accepted_len[b] = a;
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

// One tile of the final draw's weights: segment masses and the tile's
// reference exponent (0 for the residual, whose weights are absolute).
template <int DT, bool VEC, int U, bool FULL>
__device__ __forceinline__ void final_part_tile(const void* draft, const void* target, int64_t trow, int64_t drow,
                                                int V, int64_t tile, const SeqInfo& s, float* seg, Partial* ti) {
    constexpr int VE = Elem<DT>::per_vec;
    constexpr int NE = U * VE;
    const int lane = lane_id();
    float w[NE];
    float ref = 0.f;
    if (s.mode == kFinalResidual) {
        float vt[NE], vd[NE];
        load_tile<DT, VEC, U, FULL>(target, trow, V, tile, lane, vt);
        load_tile<DT, VEC, U, FULL>(draft, drow, V, tile, lane, vd);
        residual_weights<NE, FULL>(vt, vd, s, w);
    } else {
        float v[NE];
        load_tile<DT, VEC, U, FULL>(target, trow, V, tile, lane, v);
        float mx = v[0];
#pragma unroll
        for (int j = 1; j < NE; ++j) mx = fmaxf(mx, v[j]);
        ref = ceilf(wave_max(mx) * s.c_hi);
        bonus_weights<NE, FULL>(v, s, ref, w);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const float m = wave_sum(pairwise_sum<VE>(w + i * VE));
        if (lane == 0) seg[i] = m;
    }
    if (lane == 0) *ti = Partial{0.f, static_cast<int>(ref)};
}

// Partial pass of the final draw: one wave per (sequence, tile) of the row(s)
// the draw needs.  Writes every segment's mass (segment = the 64 vectors of
// one load instruction) and the tile's reference exponent; at temperature 0
// it writes the tile's argmax instead.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void chain_final_part_kernel(
    const void* __restrict__ draft, const void* __restrict__ target, int B, int k, int V, int nT,
    const SeqInfo* __restrict__ info, float* __restrict__ segmass, Partial* __restrict__ tileinfo) {
    constexpr int VE = Elem<DT>::per_vec;
    const int64_t gw = global_wave();
    if (gw >= static_cast<int64_t>(B) * nT) return;
    const int64_t b = gw / nT;
    const int64_t tile = gw - b * nT;
    const SeqInfo s = info[b];
    if (s.mode == kFinalDone) return;
    const int lane = lane_id();
    const int64_t trow = (b * (k + 1) + s.a) * static_cast<int64_t>(V);
    if (s.mode == kFinalArgmax) {
        const ArgMax a = tile_argmax_any<DT, VEC, U>(target, trow, V, tile);
        if (lane == 0) tileinfo[b * nT + tile] = Partial{a.val, a.idx};
        return;
    }
    const int64_t drow = (b * k + s.a) * static_cast<int64_t>(V);
    float* seg = segmass + (b * nT + tile) * U;
    Partial* ti = tileinfo + b * nT + tile;
    if (tile_is_full<VEC, U>(tile, V, VE))
        final_part_tile<DT, VEC, U, VEC>(draft, target, trow, drow, V, tile, s, seg, ti);
    else
        final_part_tile<DT, VEC, U, false>(draft, target, trow, drow, V, tile, s, seg, ti);
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

// Slow path, one wave: inverse CDF of the target row's own distribution, two
// sequential sweeps over all segments.  Used only when the residual of a
// rejection has no mass at all (the draft and target rows agree to rounding).
template <int DT, bool VEC>
__device__ int pick_from_target_row(const void* target, int64_t trow, int V, int64_t nseg, const SeqInfo& s) {
    constexpr int VE = Elem<DT>::per_vec;
    float w[VE];
    double W = 0.0;
    for (int64_t g = 0; g < nseg; ++g) {
        segment_weights<DT, VEC>(nullptr, target, trow, 0, V, g, s, false, s.rt, w);
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) m += w[e];
        W += static_cast<double>(wave_sum(m));
    }
    const double target_mass = static_cast<double>(s.u) * W;
    double P = 0.0;
    int last = -1;
    for (int64_t g = 0; g < nseg; ++g) {
        segment_weights<DT, VEC>(nullptr, target, trow, 0, V, g, s, false, s.rt, w);
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) m += w[e];
        const double mass = static_cast<double>(wave_sum(m));
        if (mass > 0.0) {
            const int y = pick_in_segment<DT>(w, g, P, 1.0, target_mass);
            if (y >= 0) return y;
            last = last_positive_in_segment<DT>(w, g);
        }
        P += mass;
    }
    return last;
}

// Select pass of the final draw: one wave per sequence.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kWave) void chain_final_pick_kernel(
    const void* __restrict__ draft, const void* __restrict__ target, int B, int k, int V, int nT,
    const SeqInfo* __restrict__ info, const float* __restrict__ segmass, const Partial* __restrict__ tileinfo,
    int32_t* __restrict__ emitted) {
    constexpr int VE = Elem<DT>::per_vec;
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    const SeqInfo s = info[b];
    if (s.mode == kFinalDone) return;
    const Partial* ti = tileinfo + b * nT;
    int y;
    if (s.mode == kFinalArgmax) {
        y = wave_combine_argmax(ti, nT).idx;
    } else {
        const bool residual = s.mode == kFinalResidual;
        const int64_t nseg = static_cast<int64_t>(nT) * U;
        const float* sm = segmass + b * nseg;
        const int64_t trow = (b * (k + 1) + s.a) * static_cast<int64_t>(V);
        const int64_t drow = (b * k + s.a) * static_cast<int64_t>(V);
        // global reference exponent (0 for the residual, whose masses are absolute)
        int R = -0x7fffffff;
        for (int t = lane; t < nT; t += kWave) R = max(R, ti[t].i);
        R = wave_max(R);
        // lane owns a contiguous run of segments; masses in the global scale
        const int64_t per = (nseg + kWave - 1) / kWave;
        const int64_t g0 = min<int64_t>(nseg, lane * per), g1 = min<int64_t>(nseg, g0 + per);
        double tot = 0.0;
        for (int64_t g = g0; g < g1; ++g) tot += ldexp(static_cast<double>(sm[g]), ti[g / U].i - R);
        const double incl = wave_inclusive_scan(tot);
        const double W = __shfl(incl, kWave - 1, kWave);
        double P = __shfl_up(incl, 1, kWave);
        if (lane == 0) P = 0.0;
        if (!(W > 0.0)) {
            y = residual ? pick_from_target_row<DT, VEC>(target, trow, V, nseg, s) : 0;
        } else {
            const double target_mass = static_cast<double>(s.u) * W;
            int64_t found = -1;
            double Pfound = 0.0;
            int64_t last_pos = -1;
            for (int64_t g = g0; g < g1; ++g) {
                const double m = ldexp(static_cast<double>(sm[g]), ti[g / U].i - R);
                if (found < 0 && P + m > target_mass) {
                    found = g;
                    Pfound = P;
                }
                if (m > 0.0) last_pos = g;
                P += m;
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
            const float ref = static_cast<float>(ti[seg / U].i);
            const double scale = ldexp(1.0, ti[seg / U].i - R);
            float w[VE];
            segment_weights<DT, VEC>(draft, target, trow, drow, V, seg, s, residual, ref, w);
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

}  // namespace sv
