// LDS staging of chunk rows shared by the chunked forward and backward
// kernels: natural copies (one LDS row per token) and transposed copies (one
// LDS row per head-dim element) of a chunk of a [T][D] tensor, and the
// per-row lookup of a level's weight.
#pragma once
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace loglin {
namespace {

constexpr int kPadT = 4;  // elements of padding on transposed (token-major) LDS rows
constexpr int kPadK = 8;  // elements of padding on natural (head-dim-major) LDS rows

// Blocks are dispatched round-robin over the 8 XCDs of the chip.  Remap the
// hardware block index so that consecutive logical indices (the chunks of one
// head, which share Fenwick nodes) land on the same XCD and its L2.
__device__ __forceinline__ int xcd_local_block(int b, int nblocks) {
    if (nblocks % 8 != 0) return b;
    return (b % 8) * (nblocks / 8) + b / 8;
}

template <typename E>
__device__ __forceinline__ void load_vec16(const E* src, bool ok, E* dst) {
    constexpr int V = 16 / sizeof(E);
    if (ok) {
        const uint4 x = *reinterpret_cast<const uint4*>(src);
        *reinterpret_cast<uint4*>(dst) = x;
    } else {
#pragma unroll
        for (int j = 0; j < V; ++j) dst[j] = E(0);
    }
}

// Stage rows [t0, t0 + C) of a [T][D] tensor into LDS transposed: dst[d][s]
// with row stride C + kPadT; rows past T are zero.
template <typename E, int C>
__device__ __forceinline__ void stage_transposed(const E* __restrict__ src, int D, int nvalid,
                                                 E* dst, const float* scale) {
    constexpr int V = 16 / sizeof(E);
    const int vpr = D / V;
    for (int idx = threadIdx.x; idx < C * vpr; idx += blockDim.x) {
        const int s = idx / vpr;
        const int d0 = (idx - s * vpr) * V;
        E buf[V];
        load_vec16<E>(src + (size_t)s * D + d0, s < nvalid, buf);
        if (scale) {
            const float f = scale[s];
#pragma unroll
            for (int j = 0; j < V; ++j) {
                if constexpr (sizeof(E) == 2) {
                    __bf16 b = (__bf16)(bf16_to_f32(buf[j]) * f);
                    dst[(d0 + j) * (C + kPadT) + s] = __builtin_bit_cast(bf16_t, b);
                } else {
                    dst[(d0 + j) * (C + kPadT) + s] = buf[j] * f;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j) dst[(d0 + j) * (C + kPadT) + s] = buf[j];
        }
    }
}

// Stage rows [t0, t0 + C) of a [T][D] tensor into LDS as is: dst[s][d] with
// row stride D + kPadK; rows past T are zero.
template <typename E, int C>
__device__ __forceinline__ void stage_natural(const E* __restrict__ src, int D, int nvalid,
                                              E* dst) {
    constexpr int V = 16 / sizeof(E);
    const int vpr = D / V;
    for (int idx = threadIdx.x; idx < C * vpr; idx += blockDim.x) {
        const int s = idx / vpr;
        const int d0 = (idx - s * vpr) * V;
        load_vec16<E>(src + (size_t)s * D + d0, s < nvalid, dst + s * (D + kPadK) + d0);
    }
}

template <int LOGC>
__device__ __forceinline__ float pick_level(const float (&lamr)[LOGC + 1], int lev) {
    float r = lamr[0];
#pragma unroll
    for (int l = 1; l <= LOGC; ++l) r = lev == l ? lamr[l] : r;
    return r;
}

}  // namespace
}  // namespace loglin
