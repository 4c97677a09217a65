// Tile machinery shared by the fused forward and the prefill states (gfx950):
// the 64-token tile geometry, the swizzled LDS layouts and their reads, the
// LDS-DMA copies of tiles, the tile decay and the tile state on the matrix
// cores.  Everything here is internal to the translation unit that includes it.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace loglin {
namespace {


typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;


constexpr int TC = 64;        // tokens per tile
constexpr int NRB = TC / 16;  // 16-row blocks per tile
constexpr int LOGTC = 6;
constexpr int PPAD = 8;       // bf16 padding per row of the P tile
constexpr int PROW = TC + PPAD;

// ---------------------------------------------------------------------------
// Swizzled LDS tiles: 64 rows of CPR 16-byte chunks; chunk c of row r is
// stored at position c ^ swz(r).  The swizzles keep 16-byte reads of 16
// consecutive rows, the paired 8-byte reads of the level products and the
// transpose reads free of bank conflicts for CPR = 8 and 16.

template <int CPR>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CPR == 16) {
        return (((r & 7) ^ ((r >> 1) & 4)) << 1) | ((r >> 3) & 1);
    } else if constexpr (CPR == 8) {
        const int u = (r >> 1) & 7;
        return (u & 4) | ((u & 1) << 1) | ((u >> 1) & 1);
    } else if constexpr (CPR == 4) {
        return (((r >> 1) & 7) ^ ((r >> 3) & 1)) & 3;
    } else {
        return (r >> 3) & 1;
    }
}

// element offset of (row, col) in a swizzled tile with D columns
template <int D>
__device__ __forceinline__ int toff(int r, int col) {
    constexpr int CPR = D / 8;
    return (r * CPR + ((col >> 3) ^ swz<CPR>(r))) * 8 + (col & 7);
}

template <int D>
__device__ __forceinline__ bf16x8 ld8(const bf16_t* t, int r, int col) {  // col % 8 == 0
    return *reinterpret_cast<const bf16x8*>(t + toff<D>(r, col));
}
template <int D>
__device__ __forceinline__ bf16x4 ld4(const bf16_t* t, int r, int col) {  // col % 4 == 0
    return *reinterpret_cast<const bf16x4*>(t + toff<D>(r, col));
}

// Transpose read of a 16-wide column block: lane l of 16-lane group g gets
// X[k0 + 8g + i][n0 + l % 16] for i < 8 (X row-major [token][column]).
// Within a group, lane j supplies the row k + j/4 and columns n + 4 (j % 4);
// the hardware returns column n + j of rows k..k+3.
template <int D>
__device__ __forceinline__ bf16x8 ld_tr8(const bf16_t* t, int k0, int n0) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j = lane & 15;
    const int r = k0 + 8 * g + (j >> 2);
    const int c = n0 + 4 * (j & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(t + toff<D>(r, c)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(t + toff<D>(r + 4, c)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (lds is
// uniform over the wave).  Written as inline assembly so that the compiler
// does not track these loads: it would otherwise wait for them before the
// first read of any LDS buffer.  Completion is awaited explicitly with
// s_waitcnt vmcnt(0) before the barrier that publishes a tile.
// Transpose read with free column quads: lane l of group g gets
// X[k0 + 8g + i][cbase + 8 (m / 4) + m % 4] for i < 8, m = l % 16, i.e. the
// MFMA row m of the result covers columns cbase + 8q .. cbase + 8q + 3 for
// q = m / 4.  Two such reads with cbase and cbase + 4 give C-layout rows
// 4g..4g+3 that together hold 8 consecutive columns per lane group.
template <int D>
__device__ __forceinline__ bf16x8 ld_tr8_q(const bf16_t* t, int k0, int cbase) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j = lane & 15;
    const int r = k0 + 8 * g + (j >> 2);
    const int c = cbase + 8 * (j & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(t + toff<D>(r, c)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(t + toff<D>(r + 4, c)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void dma16(const void* g, void* lds) {
    // the low 32 bits of a generic pointer into LDS are the LDS address
    const uint32_t l = (uint32_t)(uintptr_t)lds;
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(__builtin_amdgcn_readfirstlane(l)), "v"(g)
        : "memory", "m0");
}
// 4 bytes per lane into LDS at lds + 4 * lane (any 4-byte alignment)
__device__ __forceinline__ void dma4(const void* g, void* lds) {
    const uint32_t l = (uint32_t)(uintptr_t)lds;
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off"
        :
        : "s"(__builtin_amdgcn_readfirstlane(l)), "v"(g)
        : "memory", "m0");
}

// The same copy from a uniform base address plus a per-lane 32-bit byte offset
// (the scalar-base form of the instruction: no 64-bit address arithmetic per
// lane).  NT marks the data as read for the last time (non-temporal).
template <bool NT = false>
__device__ __forceinline__ void dma16o(const void* base, uint32_t off, void* lds) {
    const uint32_t l = (uint32_t)(uintptr_t)lds;
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t bu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    if constexpr (NT) {
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %2 nt"
            :
            : "s"(__builtin_amdgcn_readfirstlane(l)), "v"(off), "s"(bu)
            : "memory", "m0");
    } else {
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %2"
            :
            : "s"(__builtin_amdgcn_readfirstlane(l)), "v"(off), "s"(bu)
            : "memory", "m0");
    }
}

// Copy plan of a whole 64-row tile with D bf16 columns: the tile is NI
// wave-instructions of 1 KB (RPI rows each); a wave issues those with index
// w + NWI k.  The swizzle repeats every 16 rows, so when the stride NWI
// covers whole repeats the lane offsets of a wave's instructions differ by a
// uniform amount, added to the scalar base, and one offset register serves
// them all; otherwise every instruction keeps its own offset.
template <int D, int NWI>
struct TileCopy {
    static constexpr int CPR = D / 8;                   // 16-byte chunks per row
    static constexpr int NI = TC * CPR / 64;            // wave-instructions per tile
    static constexpr int RPI = TC / NI;                 // rows per instruction
    static constexpr int UP = CPR / 4 > 1 ? CPR / 4 : 1;  // instructions per swizzle repeat
    static constexpr bool ONE = NWI % UP == 0;
    static constexpr int PER = (NI + NWI - 1) / NWI;
    static constexpr int NOFF = ONE ? 1 : PER;
    uint32_t off[NOFF];                                 // byte offsets from the tile's first row
    uint32_t step;                                      // bytes between a wave's instructions (ONE)

    // pitch: row length of the matrix in elements; col0: first column copied
    __device__ __forceinline__ void init(int pitch, int col0, int w) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int k = 0; k < NOFF; ++k) {
            const int pch = (w + NWI * k) * 64 + lane;
            const int r = pch / CPR, pc = pch % CPR;
            off[k] = (uint32_t)(r * pitch + col0 + (pc ^ swz<CPR>(r)) * 8) * 2u;
        }
        step = (uint32_t)(NWI * RPI * pitch) * 2u;
    }
    template <bool NT = false>
    __device__ __forceinline__ void issue(const bf16_t* tile, bf16_t* lds, int w) const {
        const char* base = reinterpret_cast<const char*>(tile);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int u = w + NWI * k;
            if (NI % NWI == 0 || u < NI) {
                if constexpr (ONE) dma16o<NT>(base + (size_t)k * step, off[0], lds + u * 512);
                else dma16o<NT>(base, off[k], lds + u * 512);
            }
        }
    }
};

// Copies rows [0, 64) of a bf16 [rows][pitch] matrix, columns [col0, col0 + D),
// into a swizzled LDS tile.  Rows at or past nvalid repeat row nvalid - 1
// (finite values; they only meet masked or discarded entries).  Each wave
// instruction fills 1 KB of consecutive LDS chunks; a lane picks the source
// chunk that belongs at its position.
template <int D, int NW>
__device__ __forceinline__ void dma_tile(const bf16_t* __restrict__ src, size_t pitch, int col0,
                                         int nvalid, bf16_t* lds, int wave) {
    constexpr int CPR = D / 8;
    constexpr int NI = TC * CPR / 64;
    const int lane = threadIdx.x & 63;
    for (int u = wave; u < NI; u += NW) {
        const int pch = u * 64 + lane;
        const int r = pch / CPR, pc = pch % CPR;
        const int lc = pc ^ swz<CPR>(r);
        const int rs = min(r, nvalid - 1);
        dma16(src + (size_t)rs * pitch + col0 + lc * 8, lds + u * 512);
    }
}

__device__ __forceinline__ bf16x8 cvt8(const f32x4& a, const f32x4& b) {
    bf16x8 r;
    r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
    r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
    return r;
}
__device__ __forceinline__ bf16x4 cvt4(const f32x4& a) {
    bf16x4 r;
    r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
    return r;
}

// Sum over the four 16-lane rows of a wave, in every lane (lane l gets the
// sum of lanes l % 16, + 16, + 32, + 48): the row-swap instructions of
// gfx950 pair rows (0,1), (2,3), then halves, with no LDS traffic.
__device__ __forceinline__ float sum_rows4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Four values per lane (x[r] for 16-row block r of a tile, this lane's part
// of token m = lane % 16) summed over the four 16-lane rows at once: row g
// of the result holds the total of x[g] for token m.  Two row-pair swaps
// fold (x0, x1) and (x2, x3) over rows (0,1) and (2,3); one half swap folds
// the pairs over the halves.
__device__ __forceinline__ float sum_rows4_x4(float x0, float x1, float x2, float x3) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x2), __float_as_uint(x3), false, false);
    const float v = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // rows: x0(01) x1(01) x0(23) x1(23)
    const float u = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // rows: x2(01) x3(01) x2(23) x3(23)
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(u), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ int xcd_block(int b, int nblocks) {
    if (nblocks % 8 != 0) return b;
    return (b % 8) * (nblocks / 8) + b / 8;
}

// Head-dimension contraction: steps of 32 with the K=32 MFMA (16 for d_k = 16).
template <int DK>
struct HD {
    static constexpr int KS = DK >= 32 ? 32 : 16;
    static constexpr int NKS = DK / KS;
    static constexpr int NDT = DK / 16;
    typedef typename std::conditional<(DK >= 32), bf16x8, bf16x4>::type frag;
};

// Tile-local decay of one wave: lane s gets A_s (inclusive cumsum of a over
// the tile); the wave's private LDS rows receive A and e_s = exp(A_end - A_s).
// Returns the tile total A_end, uniform over the wave.
// DPP controls (GFX9): row_shr:n shifts within rows of 16 lanes; row_bcast
// 15 / 31 broadcast lane 15 of each row (31 of each half) to the next rows.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_or_zero(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWMASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele within rows
// of 16 lanes, then the row totals carried across rows).
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_or_zero<0x111, 0xf>(x);  // row_shr:1
    x += dpp_or_zero<0x112, 0xf>(x);  // row_shr:2
    x += dpp_or_zero<0x114, 0xf>(x);  // row_shr:4
    x += dpp_or_zero<0x118, 0xf>(x);  // row_shr:8
    x += dpp_or_zero<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_or_zero<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

__device__ __forceinline__ float tile_decay(const float* a_tile, float* Aw, float* Ew) {
    const int lane = threadIdx.x & 63;
    const float x = wave_inclusive_sum(a_tile[lane]);
    const float end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
    Aw[lane] = x;
    Ew[lane] = __expf(end - x);
    return end;
}

// U = K^T diag(e) V over the staged tile, for this wave's 16 columns and the
// NT / 2 contraction steps of 32 head-dim rows starting at step ks0 (d_k >= 32):
// u[2 j] holds rows 32 (ks0 + j) + 8g + i and u[2 j + 1] rows 32 (ks0 + j) +
// 8g + 4 + i (C layout, lane group g), so that the pair is the A operand of
// a level product over those 32 rows with natural 8-wide lane groups.
// For d_k = 16 (NT = 1): u[0] holds rows 4g + i.  vf[sp] are the V fragments
// (lane: V[32 sp + 8g + i][column]) shared with the P V product.
// Operand reads are issued ahead of the products: for both 32-token halves
// at once when BOTH (more registers, more overlap), else one half at a time.
template <int DK, int NT, bool BOTH>
__device__ __forceinline__ void tile_state(f32x4 (&u)[NT], int ks0, const bf16_t* Ks,
                                           const bf16x8 (&vf)[2], const float* Ew) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    constexpr int NR = DK >= 32 ? NT : 1;  // K fragments per 32-token half
    constexpr int NB = BOTH ? 2 : 1;       // halves whose reads are in flight together
    float4 e[NB][2];
    bf16x8 kq[NB][NR];
    auto load = [&](int sp, int slot) __attribute__((always_inline)) {
        e[slot][0] = *reinterpret_cast<const float4*>(Ew + 32 * sp + 8 * g);
        e[slot][1] = *reinterpret_cast<const float4*>(Ew + 32 * sp + 8 * g + 4);
        if constexpr (DK >= 32) {
#pragma unroll
            for (int j = 0; j < NT / 2; ++j) {
                kq[slot][2 * j] = ld_tr8_q<DK>(Ks, 32 * sp, 32 * (ks0 + j));
                kq[slot][2 * j + 1] = ld_tr8_q<DK>(Ks, 32 * sp, 32 * (ks0 + j) + 4);
            }
        } else {
            kq[slot][0] = ld_tr8<DK>(Ks, 32 * sp, 0);
        }
    };
    auto product = [&](int sp, int slot) __attribute__((always_inline)) {
        const float ev[8] = {e[slot][0].x, e[slot][0].y, e[slot][0].z, e[slot][0].w,
                             e[slot][1].x, e[slot][1].y, e[slot][1].z, e[slot][1].w};
        bf16x8 b;
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = (__bf16)((float)vf[sp][i] * ev[i]);
#pragma unroll
        for (int j = 0; j < NR; ++j) u[j] = mma(kq[slot][j], b, u[j]);
    };
    if constexpr (BOTH) {
        load(0, 0);
        load(1, 1);
        __builtin_amdgcn_sched_barrier(0);
        product(0, 0);
        product(1, 1);
    } else {
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            load(sp, 0);
            __builtin_amdgcn_sched_barrier(0);
            product(sp, 0);
        }
    }
}

// Fragment of the bf16 copy of a Fenwick node written by the scan:
// [node][column block of 16][contraction step][lane][8 or 4 bf16].
template <int DK>
__device__ __forceinline__ size_t frag_index(size_t node_global, int ncb, int cblk, int ks) {
    constexpr int NKS = HD<DK>::NKS;
    constexpr int PER = DK >= 32 ? 8 : 4;
    return (((node_global * ncb + cblk) * NKS + ks) * 64 + (threadIdx.x & 63)) * PER;
}

}  // namespace
}  // namespace loglin
