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

// Rows [t0, t0 + C) of a [T][D] tensor (D <= DM, a power of two) staged
// into LDS in two halves: chunk_load issues every 16-byte load of the
// thread (at most NV = C DM / (8 NT) for bf16) into registers, without
// branches (rows past T read row t0 and are zeroed by a select), so that all
// of them are in flight at once; chunk_store writes them as a natural copy
// nat[s][d] (row stride D + PADN) and/or a transposed copy tr[d][s] (row
// stride C + kPadT, each token optionally multiplied by scale[s] from LDS);
// either pointer may be null.
// SWZ: the natural copy's column c of row s is stored at c ^ (s & 8) (see
// the backward kernels, whose direct and transpose reads this keeps free of
// bank conflicts).
template <typename E, int C, int DM, int NT, int PADN = kPadK, bool SWZ = false>
struct ChunkRows {
    static constexpr int V = 16 / sizeof(E);
    static constexpr int NV = (C * DM / V + NT - 1) / NT;
    uint4 buf[NV];

    // Vector idx of the thread -> token s and first element d0.  With at
    // least 4 vectors per row, each 64 consecutive vectors (one wave
    // instruction) cover 16 tokens x 4 vectors, so that the 2-byte writes of
    // the transposed copy fall into 32 distinct banks; otherwise row-major.
    __device__ __forceinline__ static void where(int idx, int sh, int& s, int& d0) {
        if (sh >= 2) {
            const int l = idx & 63, w = idx >> 6;
            s = 16 * (w % (C / 16)) + (l & 15);
            d0 = (4 * (w / (C / 16)) + (l >> 4)) * V;
        } else {
            s = idx >> sh;
            d0 = (idx - (s << sh)) * V;
        }
    }

    __device__ __forceinline__ void load(const E* __restrict__ src, int D, int nvalid) {
        const int sh = __builtin_ctz(D / V);
        const int total = C << sh;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = threadIdx.x + u * NT;
            int s, d0;
            where(idx, sh, s, d0);
            const bool ok = idx < total && s < nvalid;
            const int off = ok ? s * D + d0 : 0;
            const uint4 x = *reinterpret_cast<const uint4*>(src + off);
            buf[u] = ok ? x : make_uint4(0u, 0u, 0u, 0u);
        }
    }

    // The transposed copy only, token s scaled by scale_of(s); scale_of is
    // called by every lane for every vector (it may exchange values between
    // lanes), with s clamped to the chunk.
    template <typename F>
    __device__ __forceinline__ void store_tr_scaled(int D, E* tr, F scale_of) const {
        const int sh = __builtin_ctz(D / V);
        const int total = C << sh;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = threadIdx.x + u * NT;
            int s, d0;
            where(idx, sh, s, d0);
            const float f = scale_of(idx < total ? s : 0);
            if (idx < total) {
                E e[V];
                __builtin_memcpy(e, &buf[u], 16);
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    if constexpr (sizeof(E) == 2) {
                        __bf16 b = (__bf16)(bf16_to_f32(e[j]) * f);
                        tr[(d0 + j) * (C + kPadT) + s] = __builtin_bit_cast(bf16_t, b);
                    } else {
                        tr[(d0 + j) * (C + kPadT) + s] = e[j] * f;
                    }
                }
            }
        }
    }

    __device__ __forceinline__ void store(int D, E* nat, E* tr, const float* scale) const {
        const int sh = __builtin_ctz(D / V);
        const int total = C << sh;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = threadIdx.x + u * NT;
            if (idx < total) {
                int s, d0;
                where(idx, sh, s, d0);
                if (nat) *reinterpret_cast<uint4*>(nat + s * (D + PADN) + (SWZ ? d0 ^ (s & 8) : d0)) = buf[u];
                if (tr) {
                    E e[V];
                    __builtin_memcpy(e, &buf[u], 16);
                    const float f = scale ? scale[s] : 1.f;
#pragma unroll
                    for (int j = 0; j < V; ++j) {
                        if (scale) {
                            if constexpr (sizeof(E) == 2) {
                                __bf16 b = (__bf16)(bf16_to_f32(e[j]) * f);
                                tr[(d0 + j) * (C + kPadT) + s] = __builtin_bit_cast(bf16_t, b);
                            } else {
                                tr[(d0 + j) * (C + kPadT) + s] = e[j] * f;
                            }
                        } else {
                            tr[(d0 + j) * (C + kPadT) + s] = e[j];
                        }
                    }
                }
            }
        }
    }
};

template <int LOGC>
__device__ __forceinline__ float pick_level(const float (&lamr)[LOGC + 1], int lev) {
    float r = lamr[0];
#pragma unroll
    for (int l = 1; l <= LOGC; ++l) r = lev == l ? lamr[l] : r;
    return r;
}

}  // namespace
}  // namespace loglin
