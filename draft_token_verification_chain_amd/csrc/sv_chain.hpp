// sv_chain.hpp -- sv_verify_chain: rowstats, acceptance, final draw and pick
// (part of sv_kernels.hpp).
#pragma once

#include "sv_tiles.hpp"

namespace sv {
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

// Partial of tile `tile` of a row, either way the tile ends.
template <int DT, bool VEC, int U>
__device__ __forceinline__ Partial row_tile_partial(const void* base, int64_t row_elem, int V, int64_t tile, float T) {
    return tile_is_full<VEC, U>(tile, V, Elem<DT>::per_vec) ? rowstats_tile<DT, VEC, U, VEC>(base, row_elem, V, tile, T)
                                                            : rowstats_tile<DT, VEC, U, false>(base, row_elem, V, tile, T);
}

// Tile `tile` of target row (b, position rr - b*k) or of draft row rr of a
// chain (partial rows rr and nbk + rr).  The wave of tile 0 also reads the
// row's logit at its draft token into gathered.  With SHARED the partial is
// published to other workgroups of the launch (store_partial_tagged into
// the slots `tagged`, with the call's tag) and gathered is not written: their
// reader takes those logits from the rows.
template <int DT, bool VEC, int U, bool SHARED = false>
__device__ __forceinline__ void rowstats_row_tile(const void* __restrict__ target, const void* __restrict__ draft,
                                                  const float* __restrict__ temperature,
                                                  const int32_t* __restrict__ tokens, int64_t nbk, int k,
                                                  bool is_target, int64_t b, int64_t rr, int64_t tile, int V, int nT,
                                                  Partial* __restrict__ part, float* __restrict__ gathered,
                                                  TaggedPartial* __restrict__ tagged = nullptr, CallTag tag = {}) {
    const int64_t r = is_target ? rr : nbk + rr;
    const void* base = is_target ? target : draft;
    const int64_t row_elem = (is_target ? (b * (k + 1) + (rr - b * k)) : rr) * static_cast<int64_t>(V);
    if (!SHARED && tile == 0) {
        const int x = tokens[rr];  // draft token scored by this row (rr = b * k + position)
        if (lane_id() == 0 && static_cast<unsigned>(x) < static_cast<unsigned>(V))
            gathered[r] = load_elem<DT>(base, row_elem + x);
    }
    const float T = temperature[b];
    const Partial p = row_tile_partial<DT, VEC, U>(base, row_elem, V, tile, T);
    if (lane_id() == 0) {
        if constexpr (SHARED)
            store_partial_tagged(tagged + r * nT + tile, p, tag);
        else
            part[r * nT + tile] = p;
    }
}

// Rows 0 .. B*k-1 are target rows (b, j < k); rows B*k .. 2*B*k-1 are draft
// rows (b, i).  This pass streams the rows of positions j0 .. j0+np-1 of every
// sequence (all of them when j0 = 0 and np = k).  The wave streaming tile 0 of
// a row also reads the row's logit at its draft token into gathered[r], so
// that the acceptance needs no dependent gather.  Draft rows of
// temperature-0 sequences are streamed too, and their partials go unused:
// deciding to skip them would put the temperature's load in front of every
// wave's tile loads.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void chain_rowstats_kernel(const void* __restrict__ target,
                                                                const void* __restrict__ draft,
                                                                const float* __restrict__ temperature,
                                                                const int32_t* __restrict__ tokens,
                                                                int B, int k, int j0, int np, int V, int nT,
                                                                Partial* __restrict__ part,
                                                                float* __restrict__ gathered) {
    const int64_t gw = global_wave();
    const int64_t nbk = static_cast<int64_t>(B) * k;
    const int64_t nbp = static_cast<int64_t>(B) * np;
    if (gw >= 2 * nbp * nT) return;
    const int64_t rp = gw / nT;
    const int64_t tile = gw - rp * nT;
    const bool is_target = rp < nbp;
    const int64_t rq = is_target ? rp : rp - nbp;
    const int64_t b = rq / np;
    const int64_t rr = b * k + j0 + (rq - b * np);
    rowstats_row_tile<DT, VEC, U>(target, draft, temperature, tokens, nbk, k, is_target, b, rr, tile, V, nT, part,
                                  gathered);
}

// ---------------------------------------------------------------- chain: acceptance ---

// Where an acceptance reads the partials that the streaming workgroups of its
// own launch publish (chain_fused_kernel): the rows, for the logits at the
// draft tokens and for any partial still missing after `polls` reads.
struct SharedRows {
    const void* target = nullptr;
    const void* draft = nullptr;
    const TaggedPartial* slots = nullptr;  // the published partials, laid out as `part`
    CallTag tag{};
    int polls = 0;
};

// group_load's slots of sequence b's 2k rows (lane l: row rho = l / G,
// partial row prow) from the partials that the streaming workgroups of the
// launch publish (await_slots); a partial still missing is computed with the
// streaming wave's own arithmetic (row_tile_partial).
template <int DT, bool VEC, int U>
__device__ __forceinline__ void await_partials(int64_t prow, bool valid, int nT, int G, int64_t b, int k, int V,
                                               float T, const SharedRows& sh, Partial* q, Partial* s_q) {
    await_slots(sh.slots + prow * nT, valid, nT, G, sh.tag, sh.polls, q, s_q, [&](int rho, int64_t tile) {
        const bool is_target = rho < k;
        const int64_t row = is_target ? b * (k + 1) + rho : b * k + (rho - k);
        return row_tile_partial<DT, VEC, U>(is_target ? sh.target : sh.draft, row * static_cast<int64_t>(V), V, tile,
                                            T);
    });
}

// Acceptance of sequence b, computed by one wave (the first of its block):
// the row statistics from the streaming partials (G lanes per row, one
// round trip), the 2k logits at the draft tokens, tau_i in the log domain,
// the first rejection by ballot.  Writes the final draw's descriptor into
// *out and, when `publish`, accepted_len, the accepted prefix of emitted
// and -1 after position a (the final token at a is written by the draw's
// pick, or here after a rejection at temperature 0) and accept_prob.
// With npos < k only positions 0 .. npos-1 are tested (no outputs then): the
// return value is the first rejection among them, or npos.  Each tested
// position gets exactly the arithmetic of the full call (the same lanes per
// row and the same order of combination), so the two agree on it.
template <int DT, bool SHARED = false, bool VEC = false, int U = 1>
__device__ __forceinline__ int accept_sequence(const int32_t* __restrict__ tokens,
                                               const float* __restrict__ temperature,
                                               const float* __restrict__ uniforms, int B, int k, int V, int nT,
                                               const Partial* __restrict__ part, const float* __restrict__ gathered,
                                               int64_t b, int npos, bool publish, int32_t* __restrict__ accepted_len,
                                               int32_t* __restrict__ emitted, float* __restrict__ accept_prob,
                                               int* s_r, double* s_s, SeqInfo* out,
                                               const SharedRows& sh = SharedRows{}, Partial* s_q = nullptr) {
    const int lane = lane_id();
    const int64_t nbk = static_cast<int64_t>(B) * k;
    // every load first: none of them depends on another
    const int rows = 2 * k;  // target rows 0..k-1, then draft rows
    int G = kWave;
    while (G > 1 && G * rows > kWave) G >>= 1;
    const int per_pass = kWave / G;
    auto row_of = [&](int rho) -> int64_t { return rho < k ? b * k + rho : nbk + b * k + (rho - k); };
    // rows of the positions tested (all of them in the full call)
    auto tested = [&](int rho) { return rho < rows && (rho < k ? rho : rho - k) < npos; };
    Partial q[kBatch];
    const int rho_first = lane / G;
    if constexpr (!SHARED)
        group_load(part + (tested(rho_first) ? row_of(rho_first) : 0) * nT, nT, G, tested(rho_first), q);
    const float T = temperature[b];
    const float uk = uniforms[b * (k + 1) + k];
    int x = 0;
    float ui = 0.f, lt = 0.f, ld = 0.f;
    if (lane < npos) {
        x = tokens[b * k + lane];
        ui = uniforms[b * (k + 1) + lane];
        if constexpr (SHARED) {
            // the logits at the draft token from the rows themselves
            if (static_cast<unsigned>(x) < static_cast<unsigned>(V)) {
                lt = load_elem<DT>(sh.target, (b * (k + 1) + lane) * static_cast<int64_t>(V) + x);
                ld = load_elem<DT>(sh.draft, (b * k + lane) * static_cast<int64_t>(V) + x);
            }
        } else {
            lt = gathered[b * k + lane];
            ld = gathered[nbk + b * k + lane];
        }
    }
    if constexpr (SHARED)
        await_partials<DT, VEC, U>(row_of(tested(rho_first) ? rho_first : 0), tested(rho_first), nT, G, b, k, V, T,
                                   sh, q, s_q);
    const bool sampled = T > 0.f;
    const bool xok = static_cast<unsigned>(x) < static_cast<unsigned>(V);  // out-of-range ids are rejected
    // the lane's row's normaliser, kept for tile_tv (one pass only)
    int r_own = 0;
    double s_own = 1.0;
    bool v_own = false;
    // row statistics (at temperature 0 only the target rows' argmax matters)
    for (int rho0 = 0; rho0 < rows; rho0 += per_pass) {
        const int rho = rho0 + lane / G;
        const bool valid = tested(rho);
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
            r_own = r;
            s_own = sum;
            v_own = valid;
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
    double lq = 0.0;  // log2 of the draft token's draft probability
    const double c = sampled ? kLog2e / static_cast<double>(T) : kLog2e;
    if (lane < npos) {
        if (!sampled) g = s_r[lane];
        if (!xok) {
            acc = false;
            tau = 0.0;
        } else if (sampled) {
            rt = s_r[lane];
            st = s_s[lane];
            rd = s_r[k + lane];
            sd = s_s[k + lane];
            // log2 p - log2 q with log2 p = l c - R - log2 S (the same for q)
            lq = static_cast<double>(ld) * c - rd - log2_of_sum(sd);
            const double l2ratio = (static_cast<double>(lt) * c - rt - log2_of_sum(st)) - lq;
            // exp2 of a non-positive argument in fp32: relative error about 1e-7
            tau = static_cast<double>(exp2f(static_cast<float>(fmin(0.0, l2ratio))));
            acc = static_cast<double>(ui) < tau;
        } else {
            acc = (x == g);
            tau = acc ? 1.0 : 0.0;
        }
    }
    int a = first_lane(lane < npos && !acc);
    if (a < 0) a = npos;
    if (npos < k) return a;
    // a lower bound of the rejected row's TV(p, q), from the partials still
    // held when one pass covered every row
    float tv_a = 0.f;
    if (sampled && a < k && rows <= per_pass)
        tv_a = __shfl(tile_tv(q, nT, G, v_own, r_own, s_own, k), a * G, kWave);
    int32_t* em = emitted + b * (k + 1);
    if (publish) {
        if (accept_prob != nullptr && lane < k) accept_prob[b * k + lane] = static_cast<float>(tau);
        // em[a] is left to the final token's one writer: below at temperature
        // 0 after a rejection, else the pick, which may run concurrently in
        // another workgroup of the same launch (fused_pick)
        for (int j = lane; j <= k; j += kWave)
            if (j != a) em[j] = j < a ? tokens[b * k + j] : -1;
    }
    if (lane == (a < k ? a : 0)) {
        SeqInfo si{};
        si.a = a;
        temperature_scale_from(c, si);
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
            si.st = static_cast<float>(st);
            // log2(S_t / S_d) in the target row's reference; the draw corrects it
            set_kappa(si, static_cast<double>(rt - rd) + (log2(st) - log2(sd)));
            // lower bounds of the residual's mass: q(x) - p(x) = q(x) (1 - tau),
            // and the rows' tile masses apart
            const double w_lo = fmax(static_cast<double>(exp2f(static_cast<float>(lq))) * (1.0 - tau),
                                     static_cast<double>(tv_a));
            si.fast = w_lo >= kFastResidualMass;
        } else {
            si.mode = kFinalBonus;
        }
        *out = si;
    }
    if (publish && lane == 0) accepted_len[b] = a;
    return a;
}

// Between the two phases of a chain's rowstats: whether each sequence
// accepts all of its drafts 0 .. s-1 (one wave per sequence, kAccWaves per
// workgroup), by accept_sequence over those positions, which is the final
// acceptance's own arithmetic, so the two agree on them.
constexpr int kAccWaves = 4;

template <int DT>
__global__ __launch_bounds__(kAccWaves * kWave) void chain_prefix_kernel(
    const int32_t* __restrict__ tokens, const float* __restrict__ temperature, const float* __restrict__ uniforms,
    int B, int k, int s, int V, int nT, const Partial* __restrict__ part, const float* __restrict__ gathered,
    int32_t* __restrict__ go) {
    __shared__ int s_r[kAccWaves][2 * SV_MAX_DRAFTS];
    __shared__ double s_s[kAccWaves][2 * SV_MAX_DRAFTS];
    const int w = threadIdx.x / kWave;
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kAccWaves + w;
    if (b >= B) return;  // whole waves only; the kernel has no workgroup barrier
    const int a = accept_sequence<DT>(tokens, temperature, uniforms, B, k, V, nT, part, gathered, b, s, false,
                                      nullptr, nullptr, nullptr, s_r[w], s_s[w], nullptr);
    if (lane_id() == 0) go[b] = a == s;
}

// The second phase of a chain's rowstats: the rows of positions s .. k-1 of
// the sequences that chain_prefix found to accept all drafts 0 .. s-1.  One
// workgroup per (sequence, row, group of kWavesPerBlock * tpw tiles), the
// group fastest; the rows are the target rows of positions s .. k-1, then the
// draft rows.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void chain_rowstats_rest_kernel(
    const void* __restrict__ target, const void* __restrict__ draft, const float* __restrict__ temperature,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ go, int B, int k, int s, int V, int nT,
    int groups, int tpw, Partial* __restrict__ part, float* __restrict__ gathered) {
    const int rest = k - s;
    const int64_t per_seq = static_cast<int64_t>(groups) * 2 * rest;
    const int64_t b = blockIdx.x / per_seq;
    if (!go[b]) return;
    const int rem = static_cast<int>(blockIdx.x - b * per_seq);
    const int z = rem / groups;
    const int group = rem - z * groups;
    const bool is_target = z < rest;
    const int64_t rr = b * k + s + (is_target ? z : z - rest);
#pragma unroll 1
    for (int i = 0; i < tpw; ++i) {
        const int64_t tile = (static_cast<int64_t>(group) * tpw + i) * kWavesPerBlock + threadIdx.x / kWave;
        if (tile >= nT) break;
        rowstats_row_tile<DT, VEC, U>(target, draft, temperature, tokens, static_cast<int64_t>(B) * k, k, is_target, b,
                                      rr, tile, V, nT, part, gathered);
    }
}

// One wave per sequence, kAccWaves sequences per workgroup: the acceptance
// of every sequence, its outputs and the descriptor of its final draw.

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
    accept_sequence<DT>(tokens, temperature, uniforms, B, k, V, nT, part, gathered, b, k, true, accepted_len, emitted,
                        accept_prob, s_r[w], s_s[w], info + b);
}

// ---------------------------------------------------------------- chain: final draw ---

// Weights of the final draw for the elements a lane holds.
//   residual: w = max(0, x), x the residual term (p - c q) S_t, see residual_term;
//   bonus:    w = exp2(l c - ref), unnormalised (the draw is scale-free).
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
    if (residual) {
        // both rows' loads out together
        float vd[VE];
        load_tile<DT, VEC, 1, FULL>(target, trow, V, seg, lane_id(), vt);
        load_tile<DT, VEC, 1, FULL>(draft, drow, V, seg, lane_id(), vd);
        residual_weights<DT, VE, FULL>(vt, vd, s, w);
    } else {
        load_tile<DT, VEC, 1, FULL>(target, trow, V, seg, lane_id(), vt);
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
                                           SegMass* __restrict__ seg_out, ArgMax& best) {
    constexpr int VE = Elem<DT>::per_vec;
    constexpr int NE = kFinU * VE;
    const int lane = lane_id();
    static_assert(kFinU == 4, "the four segment sums use one reduce-scatter");
    float a[kFinU];
    int i_own;
    if (mode == kFinalResidual && si.fast) {
        // a residual of large mass (kFastResidualMass): E, X and SW stay 0,
        // so the pick applies no correction
        if constexpr (FULL && VEC) {
            const char* tr = static_cast<const char*>(target) + trow * Elem<DT>::bytes;
            const char* dr = static_cast<const char*>(draft) + drow * Elem<DT>::bytes;
            const int64_t v0 = tile * (64 * kFinU) + lane;
            uint4 rt4[kFinU], rd4[kFinU];
#pragma unroll
            for (int i = 0; i < kFinU; ++i) {
                rt4[i] = *reinterpret_cast<const uint4*>(tr + (v0 + i * 64) * 16);
                rd4[i] = *reinterpret_cast<const uint4*>(dr + (v0 + i * 64) * 16);
            }
#pragma unroll
            for (int i = 0; i < kFinU; ++i) {
                float vt[VE], vd[VE];
                unpack<DT>(rt4[i], vt);
                unpack<DT>(rd4[i], vd);
                a[i] = residual_mass_fast<DT, VE, true>(vt, vd, si);
            }
        } else {
            float w[NE], vd[NE];
            load_tile<DT, VEC, kFinU, FULL>(target, trow, V, tile, lane, w);
            load_tile<DT, VEC, kFinU, FULL>(draft, drow, V, tile, lane, vd);
#pragma unroll
            for (int i = 0; i < kFinU; ++i) a[i] = residual_mass_fast<DT, VE, FULL>(w + i * VE, vd + i * VE, si);
        }
        const float m = wave_sum4(a, i_own);
        const int64_t g = tile * kFinU + i_own;
        if (lane < kFinU && g < nseg) seg_out[g] = residual_seg(m, 0.f, 0.f, 0.f);
        return;
    }
    if (mode == kFinalResidual) {
        // both rows' loads go out together, ahead of any use
        float e[kFinU], x[kFinU];
        float dmin = __builtin_inff();  // masked elements: |delta| = inf or NaN (fmin ignores NaN)
        if constexpr (FULL && VEC) {
            // raw 16-byte vectors, unpacked one segment at a time: fewer live
            // registers, so more waves per SIMD
            const char* tr = static_cast<const char*>(target) + trow * Elem<DT>::bytes;
            const char* dr = static_cast<const char*>(draft) + drow * Elem<DT>::bytes;
            const int64_t v0 = tile * (64 * kFinU) + lane;
            uint4 rt4[kFinU], rd4[kFinU];
#pragma unroll
            for (int i = 0; i < kFinU; ++i) {
                rt4[i] = *reinterpret_cast<const uint4*>(tr + (v0 + i * 64) * 16);
                rd4[i] = *reinterpret_cast<const uint4*>(dr + (v0 + i * 64) * 16);
            }
#pragma unroll
            for (int i = 0; i < kFinU; ++i) {
                float vt[VE], vd[VE];
                unpack<DT>(rt4[i], vt);
                unpack<DT>(rd4[i], vd);
                const ResidualSums r = residual_sums_marked<DT, VE, true>(vt, vd, si, dmin);
                a[i] = r.m;
                e[i] = r.ea;
                x[i] = r.x;
            }
        } else {
            float w[NE], vd[NE];
            load_tile<DT, VEC, kFinU, FULL>(target, trow, V, tile, lane, w);
            load_tile<DT, VEC, kFinU, FULL>(draft, drow, V, tile, lane, vd);
#pragma unroll
            for (int i = 0; i < kFinU; ++i) {
                const ResidualSums r = residual_sums_marked<DT, VE, FULL>(w + i * VE, vd + i * VE, si, dmin);
                a[i] = r.m;
                e[i] = r.ea;
                x[i] = r.x;
            }
        }
        const float m = wave_sum4(a, i_own);
        const float ea = wave_sum4(e, i_own);
        const float xs = wave_sum4(x, i_own);
        // SW only for the rare tiles that have an element near the switch,
        // from the tile loaded again (the first loads are no longer live)
        float ss = 0.f;
        if (__builtin_amdgcn_ballot_w64(dmin < kSwitch) != 0) {
            float sw[kFinU];
            if constexpr (FULL && VEC) {
                // raw vectors again, unpacked one segment at a time (the
                // branch then does not raise the kernel's register count)
                const char* tr = static_cast<const char*>(target) + trow * Elem<DT>::bytes;
                const char* dr = static_cast<const char*>(draft) + drow * Elem<DT>::bytes;
                const int64_t v0 = tile * (64 * kFinU) + lane;
                uint4 rt4[kFinU], rd4[kFinU];
#pragma unroll
                for (int i = 0; i < kFinU; ++i) {
                    rt4[i] = *reinterpret_cast<const uint4*>(tr + (v0 + i * 64) * 16);
                    rd4[i] = *reinterpret_cast<const uint4*>(dr + (v0 + i * 64) * 16);
                }
#pragma unroll
                for (int i = 0; i < kFinU; ++i) {
                    float vt[VE], vd[VE];
                    unpack<DT>(rt4[i], vt);
                    unpack<DT>(rd4[i], vd);
                    sw[i] = residual_sw<DT, VE, true>(vt, vd, si);
                }
            } else {
                float rt[NE], rd[NE];
                load_tile<DT, VEC, kFinU, FULL>(target, trow, V, tile, lane, rt);
                load_tile<DT, VEC, kFinU, FULL>(draft, drow, V, tile, lane, rd);
#pragma unroll
                for (int i = 0; i < kFinU; ++i) sw[i] = residual_sw<DT, VE, FULL>(rt + i * VE, rd + i * VE, si);
            }
            ss = wave_sum4(sw, i_own);
        }
        const int64_t g = tile * kFinU + i_own;
        if (lane < kFinU && g < nseg) seg_out[g] = residual_seg(m, ea, xs, ss);
        return;
    }
    float w[NE];  // the target's logits, then (in place) the weights
    load_tile<DT, VEC, kFinU, FULL>(target, trow, V, tile, lane, w);
    if (mode == kFinalArgmax) {
        best = better(best, argmax_of_tile<DT, kFinU>(w, tile));
        return;
    }
    float mx = w[0];
#pragma unroll
    for (int j = 1; j < NE; ++j) mx = fmaxf(mx, w[j]);
    // a reference over the whole tile (which always holds an element of the row)
    const float ref = ceilf(wave_max(mx) * si.c_hi);
    bonus_weights<NE, FULL>(w, si, ref, w);
#pragma unroll
    for (int i = 0; i < kFinU; ++i) a[i] = pairwise_sum<VE>(w + i * VE);
    const float m = wave_sum4(a, i_own);
    const int64_t g = tile * kFinU + i_own;
    if (lane < kFinU && g < nseg) seg_out[g] = bonus_seg(m, static_cast<int>(ref));
}

// Chunk c of sequence b's final draw, its descriptor known: the workgroup's
// waves stream adjacent tiles of the row(s) the draw needs and write each
// segment's record, or, at temperature 0, the chunk's argmax.
template <int DT, bool VEC>
__device__ __forceinline__ void final_chunk(const void* __restrict__ draft, const void* __restrict__ target, int k,
                                            int V, int64_t b, int c, int nchunk, const SeqInfo& si,
                                            SegMass* __restrict__ segs, Partial* __restrict__ chunkarg,
                                            ArgMax* s_arg) {
    constexpr int VE = Elem<DT>::per_vec;
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    const int64_t trow = (b * (k + 1) + si.a) * static_cast<int64_t>(V);
    const int64_t drow = (b * k + si.a) * static_cast<int64_t>(V);
    const int wave = threadIdx.x / kWave;
    const int64_t tile = static_cast<int64_t>(c) * kFinWaves + wave;  // the workgroup's waves read adjacent tiles
    SegMass* seg_out = segs + b * nseg;
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

template <int DT, bool VEC, int ACC>
__global__ __launch_bounds__(kFinBlock, ACC == kAcceptRead ? 5 : 1) void chain_final_part_kernel(
    const int32_t* __restrict__ tokens, const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, int B, int k, int V, int nT,
    const Partial* __restrict__ part, const float* __restrict__ gathered, int nchunk,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ emitted, float* __restrict__ accept_prob,
    SeqInfo* __restrict__ info, SegMass* __restrict__ segs, Partial* __restrict__ chunkarg) {
    __shared__ ArgMax s_arg[kFinWaves];
    const int64_t b = blockIdx.x / nchunk;
    const int c = static_cast<int>(blockIdx.x - b * nchunk);
    SeqInfo si;
    if constexpr (ACC == kAcceptInline) {
        __shared__ int s_r[2 * SV_MAX_DRAFTS];
        __shared__ double s_s[2 * SV_MAX_DRAFTS];
        __shared__ SeqInfo s_info;
        if (threadIdx.x < kWave)
            accept_sequence<DT>(tokens, temperature, uniforms, B, k, V, nT, part, gathered, b, k, c == 0, accepted_len,
                                emitted, accept_prob, s_r, s_s, &s_info);
        __syncthreads();
        si = uniform_info(s_info);
        if (c == 0 && threadIdx.x == 0) info[b] = si;
        if (si.mode == kFinalDone) return;
    } else if constexpr (ACC == kAcceptNone) {
        // k == 0: draw from target row 0 (its argmax at temperature 0)
        const float T = temperature[b];
        si = SeqInfo{};
        si.mode = T > 0.f ? kFinalBonus : kFinalArgmax;
        temperature_scale(T > 0.f ? T : 1.f, si);
        si.u = uniforms[b];
        if (c == 0 && threadIdx.x == 0) {
            info[b] = si;
            accepted_len[b] = 0;
        }
    } else {
        si = uniform_info(info[b]);
        if (si.mode == kFinalDone) return;
    }
    final_chunk<DT, VEC>(draft, target, k, V, b, c, nchunk, si, segs, chunkarg, s_arg);
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

// The token of a residual or bonus draw from its segment masses `sg` (in
// global or LDS memory), one wave.  Lane l owns a contiguous run of
// segments; a wave prefix over the run totals gives every segment's starting
// mass, the segment holding u * W is found with a ballot, and only that
// segment is read again to find the token.  `first` holds the lane's first
// kSegRun segments, loaded by the caller (ahead of the descriptor).  A
// residual draw first corrects kappa from the row's total X (kappa_zeta) and
// every segment's mass to first order; the segment read again is weighed with
// the corrected kappa, which is also returned.  When that first order cannot
// be trusted (correction_trusted) the token is kRedo: the caller forms the
// masses again with the corrected kappa (exact_residual_masses) and draws
// from them.
constexpr int kSegRun = 8;
constexpr int kRedo = -2;

struct Draw {
    int y;
    double kappa;
};

template <int DT, bool VEC>
__device__ Draw draw_from_segments(const void* draft, const void* target, int64_t trow, int64_t drow, int V,
                                   int64_t nseg, SeqInfo s, const SegMass* sg, const SegMass* first) {
    constexpr int VE = Elem<DT>::per_vec;
    const int lane = lane_id();
    const int64_t per = (nseg + kWave - 1) / kWave;
    const int64_t g0 = min<int64_t>(nseg, lane * per), g1 = min<int64_t>(nseg, g0 + per);
    const bool residual = s.mode == kFinalResidual;
    const int64_t nwin = (per + kSegRun - 1) / kSegRun;
    // segment g of this lane's window w
    const SegMass zero = residual ? residual_seg(0.f, 0.f, 0.f, 0.f) : bonus_seg(0.f, kNoRef);
    auto seg_at = [&](int64_t w, int j) -> SegMass {
        if (w == 0) return first[j];
        // an unconditional load (index clamped), so that a window's loads
        // are in flight together
        const int64_t g = g0 + w * kSegRun + j;
        const SegMass q = sg[min<int64_t>(g, nseg - 1)];
        return g < g1 ? q : zero;
    };
    auto in_run = [&](int64_t w, int j) { return g0 + w * kSegRun + j < g1; };
    // residual: the correction zeta of kappa from the row's total X; bonus:
    // the global reference exponent
    int R = 0;
    double zeta = 0.0, sw = 0.0;
    if (residual) {
        // fp32 sums suffice: zeta needs X to about 1e-6 of sum |x|, and SW is a bound
        float xs = 0.f, ss = 0.f;
        for (int64_t w = 0; w < nwin; ++w)
#pragma unroll
            for (int j = 0; j < kSegRun; ++j) {
                const SegMass q = seg_at(w, j);
                const bool in = in_run(w, j);
                xs += in ? q.x : 0.f;
                ss += in ? q.sw : 0.f;
            }
        zeta = kappa_zeta(static_cast<double>(wave_sum(xs)), static_cast<double>(s.st));
        sw = static_cast<double>(wave_sum(ss));
        set_kappa(s, s.kappa + zeta / kLn2);
    } else {
        R = kNoRef;
        for (int64_t w = 0; w < nwin; ++w)
#pragma unroll
            for (int j = 0; j < kSegRun; ++j) R = max(R, seg_at(w, j).ref);
        R = wave_max(R);
    }
    // masses of this lane's window w in the global scale
    auto window = [&](int64_t w, double* mg) {
#pragma unroll
        for (int j = 0; j < kSegRun; ++j) {
            const SegMass q = seg_at(w, j);
            const double m = static_cast<double>(q.m);
            mg[j] = !in_run(w, j) ? 0.0
                    : residual    ? fmax(0.0, m - zeta * (static_cast<double>(q.ea) - m))
                                  : ldexp(m, q.ref - R);
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
    if (residual && !correction_trusted(zeta, sw, W)) return Draw{kRedo, s.kappa};
    if (!(W > 0.0)) return Draw{residual ? pick_from_target_row<DT, VEC>(target, trow, V, nseg, s) : 0, s.kappa};
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
    const int tref = residual ? 0 : sg[seg].ref;
    const double scale = ldexp(1.0, tref - R);
    float w[VE];
    segment_weights<DT, VEC>(draft, target, trow, drow, V, seg, s, residual, static_cast<float>(tref), w);
    int y = fallback ? -1 : pick_in_segment<DT>(w, seg, Ps, scale, target_mass);
    if (y < 0) y = last_positive_in_segment<DT>(w, seg);
    return Draw{y, s.kappa};
}

// kSegRun segment masses m[c0 ..] (indices clamped into the row's nseg
// segments): unconditional loads, all in flight together.
__device__ __forceinline__ void load_masses(const float* m, int64_t c0, int64_t nseg, float* v) {
#pragma unroll
    for (int j = 0; j < kSegRun; ++j) v[j] = m[min<int64_t>(c0 + j, nseg - 1)];
}

// The sum of segment masses m[a .. e), in index order.
__device__ __forceinline__ double run_sum(const float* m, int64_t a, int64_t e, int64_t nseg) {
    double run = 0.0;
    for (int64_t c0 = a; c0 < e; c0 += kSegRun) {
        float v[kSegRun];
        load_masses(m, c0, nseg, v);
#pragma unroll
        for (int j = 0; j < kSegRun; ++j)
            if (c0 + j < e) run += static_cast<double>(v[j]);
    }
    return run;
}

// Residual masses of every segment of rows trow / drow formed with kappa as
// given in s (every wave of a workgroup of `waves` waves; mass of segment g
// into m[g]).  The caller synchronises the workgroup before reading m.
template <int DT, bool VEC>
__device__ void exact_residual_masses(const void* draft, const void* target, int64_t trow, int64_t drow, int V,
                                      int64_t nseg, const SeqInfo& s, int waves, float* m) {
    constexpr int VE = Elem<DT>::per_vec;
    for (int64_t g = threadIdx.x / kWave; g < nseg; g += waves) {
        float w[VE];
        segment_weights<DT, VEC>(draft, target, trow, drow, V, g, s, true, 0.f, w);
        const float t = wave_sum(pairwise_sum<VE>(w));
        if (lane_id() == 0) m[g] = t;
    }
}

// Inverse CDF of a distribution whose segment masses m are given (one wave;
// returns the token in every lane, or -1 when the masses sum to zero).  The
// segment holding u * W is read again with segment_weights (residual: the
// residual terms with kappa as in s; else exp2(l c - rt)).
template <int DT, bool VEC>
__device__ int pick_from_masses_f(const void* draft, const void* target, int64_t trow, int64_t drow, int V,
                                  int64_t nseg, const SeqInfo& s, bool residual, const float* m, double u) {
    const int lane = lane_id();
    const int64_t per = (nseg + kWave - 1) / kWave;
    const int64_t a = min<int64_t>(nseg, lane * per), e = min<int64_t>(nseg, a + per);
    const double run = run_sum(m, a, e, nseg);
    const double incl = wave_inclusive_scan(run);
    const double W = __shfl(incl, kWave - 1, kWave);
    const double excl = __shfl_up(incl, 1, kWave);  // every lane shuffles
    if (!(W > 0.0)) return -1;
    double P = lane == 0 ? 0.0 : excl;
    const double target_mass = u * W;
    int64_t found = -1, last_pos = -1;
    double Pfound = 0.0;
    for (int64_t c0 = a; c0 < e; c0 += kSegRun) {
        float v[kSegRun];
        load_masses(m, c0, nseg, v);
#pragma unroll
        for (int j = 0; j < kSegRun; ++j) {
            const int64_t g = c0 + j;
            if (g >= e) break;
            const double mg = static_cast<double>(v[j]);
            if (found < 0 && P + mg > target_mass) {
                found = g;
                Pfound = P;
            }
            if (mg > 0.0) last_pos = g;
            P += mg;
        }
    }
    int fl = first_lane(found >= 0);
    int64_t seg;
    double Ps = 0.0;
    bool fallback = false;
    if (fl >= 0) {
        seg = __shfl(found, fl, kWave);
        Ps = __shfl(Pfound, fl, kWave);
    } else {
        const uint64_t mk = __ballot(last_pos >= 0);
        fl = mk ? 63 - __builtin_clzll(mk) : 0;
        seg = mk ? __shfl(last_pos, fl, kWave) : 0;
        fallback = true;
    }
    float w[Elem<DT>::per_vec];
    segment_weights<DT, VEC>(draft, target, trow, drow, V, seg, s, residual, s.rt, w);
    int y = fallback ? -1 : pick_in_segment<DT>(w, seg, Ps, 1.0, target_mass);
    if (y < 0) y = last_positive_in_segment<DT>(w, seg);
    return y;
}

// The lane's first kSegRun segments of draw_from_segments (records past the
// lane's run are never used).  Every load is unconditional, its index clamped
// into the row's segments, so that all of them are in flight together rather
// than each behind a branch and a wait of its own.
__device__ __forceinline__ void first_segments(const SegMass* sg, int64_t nseg, SegMass* first) {
    const int64_t per = (nseg + kWave - 1) / kWave;
    const int64_t g0 = min<int64_t>(nseg, lane_id() * per);
#pragma unroll
    for (int j = 0; j < kSegRun; ++j) first[j] = sg[min<int64_t>(g0 + j, nseg - 1)];
    // keep the scheduler from moving the records' first uses in between the
    // loads, which makes them wait for one another
    __builtin_amdgcn_sched_barrier(0);
}

// A residual draw whose first-order kappa correction is not trusted (see
// draw_from_segments): the workgroup's `waves` waves form the row's masses
// again with the corrected kappa into m, and wave 0 draws from them (the
// target row itself when they sum to zero).  Returns the token in wave 0.
template <int DT, bool VEC>
__device__ int redo_residual_draw(const void* draft, const void* target, int64_t trow, int64_t drow, int V,
                                  int64_t nseg, SeqInfo s, double kappa, int waves, float* m) {
    set_kappa(s, kappa);
    exact_residual_masses<DT, VEC>(draft, target, trow, drow, V, nseg, s, waves, m);
    __syncthreads();
    int y = 0;
    if (threadIdx.x < kWave) {
        y = pick_from_masses_f<DT, VEC>(draft, target, trow, drow, V, nseg, s, true, m, static_cast<double>(s.u));
        if (y < 0) y = pick_from_target_row<DT, VEC>(target, trow, V, nseg, s);
    }
    return y;
}

// Select pass of the final draw: one workgroup per sequence, whose wave 0
// draws the token (the descriptor and the lane's first segments are loaded
// together); the other waves only help when the masses must be formed again
// (redo_residual_draw).
constexpr int kPickBlock = 256;
constexpr int kMaxSegs = SV_MAX_VOCAB / (4 * 64);  // f32 rows have the most segments

template <int DT, bool VEC>
__global__ __launch_bounds__(kPickBlock) void chain_final_pick_kernel(
    const void* __restrict__ draft, const void* __restrict__ target, int k, int V, int nchunk,
    const SeqInfo* __restrict__ info, const SegMass* __restrict__ segs, const Partial* __restrict__ chunkarg,
    int32_t* __restrict__ emitted) {
    constexpr int VE = Elem<DT>::per_vec;
    __shared__ float s_m[kMaxSegs];
    __shared__ double s_kappa;
    __shared__ int s_redo;
    const int64_t b = blockIdx.x;
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    const SegMass* sg = segs + b * nseg;
    // the descriptor and the lane's first segment records are in flight
    // together (a sequence with nothing to draw leaves the records unused);
    // wave 0, which draws, is told apart with a wave-uniform test
    const bool wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x) < kWave;
    const SeqInfo s = info[b];
    SegMass first[kSegRun];
    if (wave0) first_segments(sg, nseg, first);
    if (s.mode == kFinalDone) return;
    const int64_t trow = (b * (k + 1) + s.a) * static_cast<int64_t>(V);
    const int64_t drow = (b * k + s.a) * static_cast<int64_t>(V);
    if (wave0) {
        Draw d{0, s.kappa};
        if (s.mode == kFinalArgmax)
            d.y = wave_combine_argmax(chunkarg + b * nchunk, nchunk).idx;
        else
            d = draw_from_segments<DT, VEC>(draft, target, trow, drow, V, nseg, s, sg, first);
        if (threadIdx.x == 0) {
            s_redo = d.y == kRedo;
            s_kappa = d.kappa;
            if (d.y != kRedo) emitted[b * (k + 1) + s.a] = d.y;
        }
    }
    __syncthreads();
    if (!s_redo) return;
    const int y =
        redo_residual_draw<DT, VEC>(draft, target, trow, drow, V, nseg, s, s_kappa, kPickBlock / kWave, s_m);
    if (threadIdx.x == 0) emitted[b * (k + 1) + s.a] = y;
}

// ---------------------------------------------------------------- chain: rows and draw in one launch ---

// The first pass and the final draw in one launch, for chains whose draw
// recomputes the acceptance in every workgroup and whose 2k rows' partials
// fit one wave's group_load.  Workgroups 0 .. row_blocks-1 stream the rows
// as chain_rowstats_kernel does (without gathered) and publish each tile's
// partial into `slots` with the call's tag (store_partial_tagged); the
// others draw, chunk c of sequence b each, as chain_final_part_kernel with
// the acceptance inline does, reading the sequence's partials as they are
// published (await_partials).  A sequence's draw thus starts as soon as its
// rows are streamed, while the rows of later sequences still stream.
// chain_final_pick_kernel follows.
template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kFinBlock, 5) void chain_fused_kernel(
    const int32_t* __restrict__ tokens, const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, int B, int k, int V, int nT,
    int64_t row_blocks, int nchunk, int polls, TaggedPartial* __restrict__ slots, CallTag tag,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ emitted, float* __restrict__ accept_prob,
    SeqInfo* __restrict__ info, SegMass* __restrict__ segs, Partial* __restrict__ chunkarg) {
    static_assert(kFinBlock == kBlock, "both roles use one workgroup size");
    if (blockIdx.x < row_blocks) {
        const int64_t gw = global_wave();
        const int64_t nbk = static_cast<int64_t>(B) * k;
        if (gw >= 2 * nbk * nT) return;
        const int64_t rp = gw / nT;
        const int64_t tile = gw - rp * nT;
        const bool is_target = rp < nbk;
        const int64_t rr = is_target ? rp : rp - nbk;
        rowstats_row_tile<DT, VEC, U, true>(target, draft, temperature, tokens, nbk, k, is_target, rr / k, rr, tile,
                                            V, nT, nullptr, nullptr, slots, tag);
        return;
    }
    __shared__ ArgMax s_arg[kFinWaves];
    __shared__ int s_r[2 * SV_MAX_DRAFTS];
    __shared__ double s_s[2 * SV_MAX_DRAFTS];
    __shared__ SeqInfo s_info;
    __shared__ Partial s_q[kBatch * kWave];
    const int64_t db = blockIdx.x - row_blocks;
    const int64_t b = db / nchunk;
    const int c = static_cast<int>(db - b * nchunk);
    if (threadIdx.x < kWave)
        accept_sequence<DT, true, VEC, U>(tokens, temperature, uniforms, B, k, V, nT, nullptr, nullptr, b, k, c == 0,
                                          accepted_len, emitted, accept_prob, s_r, s_s, &s_info,
                                          SharedRows{target, draft, slots, tag, polls}, s_q);
    __syncthreads();
    const SeqInfo si = uniform_info(s_info);
    if (c == 0 && threadIdx.x == 0) info[b] = si;
    if (si.mode == kFinalDone) return;
    final_chunk<DT, VEC>(draft, target, k, V, b, c, nchunk, si, segs, chunkarg, s_arg);
}


// ---------------------------------------------------------------- final draw, one workgroup per row ---

// Plain sampling (no drafts): when one row per CU fills the chip, a
// sequence's whole draw is one workgroup's work (rows of at most
// kRowDrawMaxSegs segments).  The descriptor follows from the temperature
// alone; the 16 waves stream the row with final_tile, the segment masses
// going to LDS instead of HBM, and wave 0 draws the token with
// draw_from_segments.  It computes exactly what chain_final_part and
// chain_final_pick compute for k = 0, in one launch.
constexpr int kRowDrawBlock = 1024;
constexpr int kRowDrawWaves = kRowDrawBlock / kWave;
constexpr int kRowDrawMaxSegs = 256;

template <int DT, bool VEC>
__global__ __launch_bounds__(kRowDrawBlock) void chain_row_draw_kernel(const void* __restrict__ target,
                                                                       const float* __restrict__ temperature,
                                                                       const float* __restrict__ uniforms, int V,
                                                                       int32_t* __restrict__ accepted_len,
                                                                       int32_t* __restrict__ emitted) {
    constexpr int VE = Elem<DT>::per_vec;
    __shared__ SegMass s_seg[kRowDrawMaxSegs];
    __shared__ ArgMax s_arg[kRowDrawWaves];
    const int64_t b = blockIdx.x;
    // draw from the sequence's one target row (its argmax at temperature 0)
    const float T = temperature[b];
    SeqInfo si{};
    si.mode = T > 0.f ? kFinalBonus : kFinalArgmax;
    temperature_scale(T > 0.f ? T : 1.f, si);
    si.u = uniforms[b];
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    const int64_t ntile = (nseg + kFinU - 1) / kFinU;
    const int64_t trow = b * static_cast<int64_t>(V);
    const int wave = threadIdx.x / kWave;
    ArgMax best{-__builtin_inff(), kNoIndex};
    for (int64_t tile = wave; tile < ntile; tile += kRowDrawWaves) {
        if (tile_is_full<VEC, kFinU>(tile, V, VE))
            final_tile<DT, VEC, VEC>(nullptr, target, trow, 0, V, tile, nseg, si, si.mode, s_seg, best);
        else
            final_tile<DT, VEC, false>(nullptr, target, trow, 0, V, tile, nseg, si, si.mode, s_seg, best);
    }
    if (lane_id() == 0) s_arg[wave] = best;
    __syncthreads();
    if (wave != 0) return;
    int y;
    if (si.mode == kFinalArgmax) {
        ArgMax r = s_arg[0];
        for (int w = 1; w < kRowDrawWaves; ++w) r = better(r, s_arg[w]);
        y = r.idx;
    } else {
        SegMass first[kSegRun];
        first_segments(s_seg, nseg, first);
        y = draw_from_segments<DT, VEC>(nullptr, target, trow, 0, V, nseg, si, s_seg, first).y;
    }
    if (threadIdx.x == 0) {
        emitted[b] = y;
        accepted_len[b] = 0;
    }
}

// ---------------------------------------------------------------- small chains, one workgroup per sequence ---

// When a sequence's rows are short (at most kSmallMaxSegs segments) and the
// batch is small, launches dominate the three-kernel path, and one workgroup
// per sequence does the whole verification in one launch: its 16 waves
// stream the 2k rows' tiles (rowstats_tile, partials and the draft tokens'
// logits to LDS), wave 0 runs the acceptance from them (accept_sequence on
// the sequence alone, the same code and order of combination as everywhere
// else), the waves then stream the draw's row or rows with final_tile into
// segment records in LDS, and wave 0 draws the token with
// draw_from_segments; when the residual's first-order correction cannot be
// trusted the workgroup forms the masses again (redo_residual_draw).  It
// computes what chain_rowstats, chain_final_part and chain_final_pick
// compute.
constexpr int kSmallMaxSegs = 64;  // rows of at most 32768 bf16 or 16384 f32 logits

template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kSmallBlock) void chain_small_kernel(
    const int32_t* __restrict__ tokens, const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const float* __restrict__ uniforms, int k, int V, int nT,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ emitted, float* __restrict__ accept_prob) {
    constexpr int VE = Elem<DT>::per_vec;
    __shared__ Partial s_part[kSmallMaxParts];
    __shared__ float s_gath[2 * SV_MAX_DRAFTS];
    __shared__ SegMass s_seg[kSmallMaxSegs];
    __shared__ float s_m[kSmallMaxSegs];
    __shared__ ArgMax s_arg[kSmallWaves];
    __shared__ int s_r[2 * SV_MAX_DRAFTS];
    __shared__ double s_s[2 * SV_MAX_DRAFTS];
    __shared__ SeqInfo s_info;
    __shared__ double s_kappa;
    __shared__ int s_redo;
    __shared__ int32_t s_tok[SV_MAX_DRAFTS];
    __shared__ float s_unif[SV_MAX_DRAFTS + 1];
    __shared__ float s_temp;
    const int64_t b = blockIdx.x;
    const int wave = threadIdx.x / kWave;
    SeqInfo si;
    if (k > 0 && threadIdx.x <= SV_MAX_DRAFTS) {
        // the acceptance's scalars, in flight with the row tiles (copied to LDS)
        const int t = threadIdx.x;
        if (t < k) s_tok[t] = tokens[b * k + t];
        if (t <= k) s_unif[t] = uniforms[b * (k + 1) + t];
        if (t == 0) s_temp = temperature[b];
    }
    if (k == 0) {
        // no drafts: a draw from target row 0 (its argmax at temperature 0)
        const float T = temperature[b];
        si = SeqInfo{};
        si.mode = T > 0.f ? kFinalBonus : kFinalArgmax;
        temperature_scale(T > 0.f ? T : 1.f, si);
        si.u = uniforms[b];
        if (threadIdx.x == 0) accepted_len[b] = 0;
    } else {
        // rows 0 .. k-1: target rows, k .. 2k-1: draft rows (the layout
        // accept_sequence reads for a batch of one sequence)
        const float T = temperature[b];
        for (int w = wave; w < 2 * k * nT; w += kSmallWaves) {
            const int rp = w / nT;
            const int tile = w - rp * nT;
            const bool is_target = rp < k;
            const int j = is_target ? rp : rp - k;
            const void* base = is_target ? target : draft;
            const int64_t row_elem = (is_target ? b * (k + 1) + j : b * k + j) * static_cast<int64_t>(V);
            if (tile == 0) {
                const int x = tokens[b * k + j];
                if (lane_id() == 0 && static_cast<unsigned>(x) < static_cast<unsigned>(V))
                    s_gath[rp] = load_elem<DT>(base, row_elem + x);
            }
            const Partial p = tile_is_full<VEC, U>(tile, V, VE) ? rowstats_tile<DT, VEC, U, VEC>(base, row_elem, V, tile, T)
                                                                : rowstats_tile<DT, VEC, U, false>(base, row_elem, V, tile, T);
            if (lane_id() == 0) s_part[w] = p;
        }
        __syncthreads();  // the partials and gathered logits before the acceptance reads them
        if (threadIdx.x < kWave)
            accept_sequence<DT>(s_tok, &s_temp, s_unif, 1, k, V, nT, s_part, s_gath, 0, k, true, accepted_len + b,
                                emitted + b * (k + 1), accept_prob ? accept_prob + b * k : nullptr, s_r, s_s,
                                &s_info);
        __syncthreads();
        si = uniform_info(s_info);
        if (si.mode == kFinalDone) return;
    }
    const int64_t nseg = ((V + VE - 1) / VE + 63) / 64;
    const int64_t ntile = (nseg + kFinU - 1) / kFinU;
    const int64_t trow = (b * (k + 1) + si.a) * static_cast<int64_t>(V);
    const int64_t drow = (b * k + si.a) * static_cast<int64_t>(V);
    ArgMax best{-__builtin_inff(), kNoIndex};
    for (int64_t tile = wave; tile < ntile; tile += kSmallWaves) {
        if (tile_is_full<VEC, kFinU>(tile, V, VE))
            final_tile<DT, VEC, VEC>(draft, target, trow, drow, V, tile, nseg, si, si.mode, s_seg, best);
        else
            final_tile<DT, VEC, false>(draft, target, trow, drow, V, tile, nseg, si, si.mode, s_seg, best);
    }
    if (lane_id() == 0) s_arg[wave] = best;
    __syncthreads();
    int32_t* out = emitted + b * (k + 1) + si.a;
    if (wave == 0) {
        Draw d{0, si.kappa};
        if (si.mode == kFinalArgmax) {
            ArgMax r = s_arg[0];
            for (int w = 1; w < kSmallWaves; ++w) r = better(r, s_arg[w]);
            d.y = r.idx;
        } else {
            SegMass first[kSegRun];
            first_segments(s_seg, nseg, first);
            d = draw_from_segments<DT, VEC>(draft, target, trow, drow, V, nseg, si, s_seg, first);
        }
        if (threadIdx.x == 0) {
            s_redo = d.y == kRedo;
            s_kappa = d.kappa;
            if (d.y != kRedo) *out = d.y;
        }
    }
    __syncthreads();
    if (!s_redo) return;
    const int y = redo_residual_draw<DT, VEC>(draft, target, trow, drow, V, nseg, si, s_kappa, kSmallWaves, s_m);
    if (threadIdx.x == 0) *out = y;
}

}  // namespace sv
