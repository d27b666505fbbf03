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
