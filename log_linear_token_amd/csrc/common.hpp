// Device helpers shared by the gfx950 kernels of the log-linear token mixer:
// element types, MFMA wrappers with their lane layouts, and Fenwick indexing.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loglin {

typedef unsigned short bf16_t;  // bf16 storage (raw bits)
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWave = 64;

// Broadcast lane 0's value to the whole wave as a wave-uniform (scalar) value.
// The builtin works on 32-bit integers, so the float travels as its bits.
__device__ __forceinline__ float wave_uniform(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }

// ---------------------------------------------------------------------------
// Fenwick indexing ("Log-linear attention, and what a logarithm buys", sec. 2)
//
// Query t sees the sentinel bucket {t} at level 0; the earlier tokens are cut
// greedily into power-of-two buckets, oldest (largest) first.  Key s < t lies
// in the bucket whose level is one more than the index of the highest bit in
// which s and t differ.
__device__ __forceinline__ int fenwick_level(uint32_t t, uint32_t s) {
    return t == s ? 0 : 32 - __builtin_clz(t ^ s);
}
// trailing zero bits of t >= 1 (the page's lssb)
__device__ __forceinline__ int lssb(uint64_t t) { return __builtin_ctzll(t); }

// ---------------------------------------------------------------------------
// MFMA 16 x 16 tiles, fp32 accumulators.  For an M x K by K x N product with
// M = N = 16 and kpl operand values per lane (K = 4 * kpl):
//   A[m][k]: lane l holds A[l % 16][(l / 16) * kpl + i], i < kpl
//   B[k][n]: lane l holds B[(l / 16) * kpl + i][l % 16], i < kpl
//   C[m][n]: lane l holds C[(l / 16) * 4 + i][l % 16],   i < 4
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {  // K = 32
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(bf16x4 a, bf16x4 b, f32x4 c) {  // K = 16
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {  // K = 4, fp32
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operand fragments for a contraction over a contiguous dimension of length
// KS per step: kpl consecutive elements per lane.
template <typename E, int KS>
struct Frag;
template <>
struct Frag<bf16_t, 32> {
    typedef bf16x8 type;
    static constexpr int kpl = 8;
    __device__ static type load(const bf16_t* p) {  // 16-byte aligned
        return *reinterpret_cast<const bf16x8*>(p);
    }
    __device__ static type from_f32(const float* p) {  // 32-byte aligned, rounds to bf16
        const float4 x = reinterpret_cast<const float4*>(p)[0];
        const float4 y = reinterpret_cast<const float4*>(p)[1];
        type r;
        r[0] = (__bf16)x.x; r[1] = (__bf16)x.y; r[2] = (__bf16)x.z; r[3] = (__bf16)x.w;
        r[4] = (__bf16)y.x; r[5] = (__bf16)y.y; r[6] = (__bf16)y.z; r[7] = (__bf16)y.w;
        return r;
    }
};
template <>
struct Frag<bf16_t, 16> {
    typedef bf16x4 type;
    static constexpr int kpl = 4;
    __device__ static type load(const bf16_t* p) {  // 8-byte aligned
        return *reinterpret_cast<const bf16x4*>(p);
    }
    __device__ static type from_f32(const float* p) {  // 16-byte aligned
        const float4 x = *reinterpret_cast<const float4*>(p);
        type r;
        r[0] = (__bf16)x.x; r[1] = (__bf16)x.y; r[2] = (__bf16)x.z; r[3] = (__bf16)x.w;
        return r;
    }
};
template <>
struct Frag<float, 4> {
    typedef float type;
    static constexpr int kpl = 1;
    __device__ static type load(const float* p) { return *p; }
    __device__ static type from_f32(const float* p) { return *p; }
};

// Contraction step over the head dimension for each element type.
template <typename E, int DK>
struct HeadStep {
    static constexpr int KS = 32;
};
template <>
struct HeadStep<bf16_t, 16> {
    static constexpr int KS = 16;
};
template <int DK>
struct HeadStep<float, DK> {
    static constexpr int KS = 4;
};

__device__ __forceinline__ bf16x4 pack4(float a, float b, float c, float d) {
    bf16x4 r;
    r[0] = (__bf16)a; r[1] = (__bf16)b; r[2] = (__bf16)c; r[3] = (__bf16)d;
    return r;
}

// Inclusive prefix sum of n <= 128 floats held in LDS (src -> dst), done by
// one wave in a fixed order so that every kernel that calls it gets bitwise
// the same values.  Must be called by all lanes of exactly one wave.
__device__ __forceinline__ void wave_cumsum(const float* src, float* dst, int n) {
    const int lane = threadIdx.x & (kWave - 1);
    // each lane owns two consecutive elements
    float x0 = 2 * lane < n ? src[2 * lane] : 0.f;
    float x1 = 2 * lane + 1 < n ? src[2 * lane + 1] : 0.f;
    float s = x0 + x1;
    float incl = s;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        float y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
    }
    const float excl = incl - s;
    if (2 * lane < n) dst[2 * lane] = excl + x0;
    if (2 * lane + 1 < n) dst[2 * lane + 1] = excl + x0 + x1;
}

}  // namespace loglin
