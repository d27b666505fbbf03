// sv_commit.hpp -- sv_commit_tokens: the device-side commit (part of sv_kernels.hpp).
#pragma once

#include "sv_common.hpp"

namespace sv {
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
            } else if (a >= width || len < 0 || static_cast<int64_t>(len) + a + 1 > INT32_MAX ||
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
