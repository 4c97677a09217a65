// Fused chunked forward of the log-linear token mixer for bf16 inputs (gfx950).
//
// The chunked form of "Log-linear attention, and what a logarithm buys"
// (section 3) evaluated with the Fenwick states held in registers: one block
// walks the 64-token tiles of a segment in order, and for every tile
//   - the intra-tile block: S^T = K Q^T on MFMA, masked in registers with
//     lambda_t^(level(t,s)) e^(A_t - A_s), stored to LDS as bf16 P, then
//     O^T = V^T P^T on MFMA;
//   - the coarse levels: for each set bit of the tile index a state G holding
//     the decayed sum of k v^T over the matching block of earlier tiles,
//     read with one MFMA per row block and weighted per row by
//     lambda_t^(level) e^(A_t - A_end(block));
//   - the tile's own state U = K^T diag(e^(A_end - A_s)) V (MFMA), which the
//     Fenwick update of section 2, run over tiles, folds together with the
//     states of the levels below lssb(tile+1) into the next level.
// Levels inside the segment (up to kMaxLocal) live in registers as fp32 MFMA
// accumulators and never touch memory.  The levels above the segment are the
// same for all of its tiles; they come from two small launches before the main
// one: seg_state (the decayed state of every segment but the last) and the
// Fenwick scan over segments (fenwick_scan in fwd_chunked.hip), and sit in LDS
// as bf16 MFMA operands.
//
// One wave owns 16 columns of d_v and computes them for all 64 rows of a tile;
// the waves of a block share the tile's Q, K, V^T, P and lambda through LDS.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace loglin {

static_assert(sizeof(bf16_t_storage) == sizeof(bf16_t), "bf16 storage");

namespace {

constexpr int TC = 64;          // tokens per tile
constexpr int NRB = TC / 16;    // 16-row blocks per tile
constexpr int LOGTC = 6;
constexpr int PAD = 8;          // bf16 elements of padding per LDS row (16 bytes)
constexpr int kTopMax = 16;     // coarse slots tracked (LDS use is checked on the host)

struct Lds {
    int q, k, kt, vt, p, lam, araw, aloc, ev, top, total;
};

__host__ __device__ inline int round16(int x) { return (x + 15) & ~15; }

// Byte offsets of the fused kernel's LDS regions (the host sizes the launch
// with the same function).
__host__ __device__ inline Lds fused_lds(int dk, int dvw, int lu, int ntop) {
    Lds o;
    int off = 0;
    o.q = off;    off += round16(TC * (dk + PAD) * 2);
    o.k = off;    off += round16(TC * (dk + PAD) * 2);
    o.kt = off;   off += round16(dk * (TC + PAD) * 2);
    o.vt = off;   off += round16(dvw * (TC + PAD) * 2);
    o.p = off;    off += round16(TC * (TC + PAD) * 2);
    o.lam = off;  off += round16(TC * lu * 4);
    o.araw = off; off += round16(TC * 4);
    o.aloc = off; off += round16(TC * 4);
    o.ev = off;   off += round16(TC * 4);
    o.top = off;  off += round16(ntop * dk * dvw * 2);
    o.total = off;
    return o;
}

// LDS of the segment-state kernel: K^T, V^T, a, A, e.
__host__ __device__ inline int segstate_lds(int dk, int dvw) {
    return round16(dk * (TC + PAD) * 2) + round16(dvw * (TC + PAD) * 2) + 3 * round16(TC * 4);
}

__device__ __forceinline__ int xcd_block(int b, int nblocks) {
    if (nblocks % 8 != 0) return b;
    return (b % 8) * (nblocks / 8) + b / 8;
}

__device__ __forceinline__ uint32_t pack2(bf16_t lo, bf16_t hi) {
    return (uint32_t)lo | ((uint32_t)hi << 16);
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

// Head-dimension contraction step: 32 with the K=32 MFMA, 16 for d_k = 16.
template <int DK>
struct HD {
    static constexpr int KS = DK >= 32 ? 32 : 16;
    static constexpr int NKS = DK / KS;
    typedef typename std::conditional<(DK >= 32), bf16x8, bf16x4>::type frag;
    static constexpr int KPL = DK >= 32 ? 8 : 4;
};

// ---------------------------------------------------------------------------
// Tile staging: global -> registers (prefetch) -> LDS.

template <int DK, int NW>
struct TileRegs {
    static constexpr int NT = NW * 64;
    static constexpr int DVW = NW * 16;
    static constexpr int QV = TC * DK / 8;                 // 16-byte vectors of Q
    static constexpr int KP = (TC / 2) * (DK / 8);         // token pairs x 8 head dims of K
    static constexpr int VP = (TC / 2) * (DVW / 8);        // token pairs x 8 columns of V
    static constexpr int NQ = (QV + NT - 1) / NT;
    static constexpr int NK = (KP + NT - 1) / NT;
    static constexpr int NV = (VP + NT - 1) / NT;
    static constexpr int LUMAX = 24;                        // levels staged per token (max)
    static constexpr int NL = (TC * LUMAX + NT - 1) / NT;
    uint4 q[NQ];
    uint4 k[NK][2];
    uint4 v[NV][2];
    float a;
    float lam[NL];
};

// Loads tile `i` (tokens i*TC ...) of sequence row0 into registers; rows past
// T are zero.  withQ=false skips Q and lambda (segment-state kernel).
template <int DK, int NW, bool withQ>
__device__ __forceinline__ void load_tile(TileRegs<DK, NW>& R, const bf16_t* __restrict__ q,
                                          const bf16_t* __restrict__ k,
                                          const bf16_t* __restrict__ v, const float* __restrict__ a,
                                          const float* __restrict__ lam, size_t row0, int t0, int T,
                                          int dv, int cb, int L, int lu) {
    typedef TileRegs<DK, NW> TR;
    const int tid = threadIdx.x;
    const int nvalid = min(TC, T - t0);
    const uint4 z = make_uint4(0, 0, 0, 0);
    const size_t r0 = row0 + t0;
    if constexpr (withQ) {
#pragma unroll
        for (int u = 0; u < TR::NQ; ++u) {
            const int x = tid + u * TR::NT;
            if (x < TR::QV) {
                const int s = x / (DK / 8), d0 = (x % (DK / 8)) * 8;
                R.q[u] = s < nvalid ? *reinterpret_cast<const uint4*>(q + (r0 + s) * DK + d0) : z;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < TR::NK; ++u) {
        const int x = tid + u * TR::NT;
        if (x < TR::KP) {
            const int ps = x % (TC / 2), d0 = (x / (TC / 2)) * 8;
            const int s = 2 * ps;
            R.k[u][0] = s < nvalid ? *reinterpret_cast<const uint4*>(k + (r0 + s) * DK + d0) : z;
            R.k[u][1] =
                s + 1 < nvalid ? *reinterpret_cast<const uint4*>(k + (r0 + s + 1) * DK + d0) : z;
        }
    }
#pragma unroll
    for (int u = 0; u < TR::NV; ++u) {
        const int x = tid + u * TR::NT;
        if (x < TR::VP) {
            const int ps = x % (TC / 2), c = cb + (x / (TC / 2)) * 8;
            const int s = 2 * ps;
            R.v[u][0] = s < nvalid ? *reinterpret_cast<const uint4*>(v + (r0 + s) * dv + c) : z;
            R.v[u][1] =
                s + 1 < nvalid ? *reinterpret_cast<const uint4*>(v + (r0 + s + 1) * dv + c) : z;
        }
    }
    if (tid < TC) R.a = tid < nvalid ? a[r0 + tid] : 0.f;
    if constexpr (withQ) {
#pragma unroll
        for (int u = 0; u < TR::NL; ++u) {
            const int x = tid + u * TR::NT;
            if (x < TC * lu) {
                const int s = x / lu, l = x - s * lu;
                R.lam[u] = s < nvalid ? lam[(r0 + s) * L + l] : 0.f;
            }
        }
    }
}

// Writes a loaded tile to LDS: Q and K as [token][d_k], K^T [d_k][token],
// V^T [column][token], lambda [token][level], raw a.
template <int DK, int NW, bool withQ>
__device__ __forceinline__ void store_tile(const TileRegs<DK, NW>& R, bf16_t* Qs, bf16_t* Ks,
                                           bf16_t* KTs, bf16_t* VTs, float* lam_s, float* araw,
                                           int lu) {
    typedef TileRegs<DK, NW> TR;
    constexpr int QROW = DK + PAD, TROW = TC + PAD;
    const int tid = threadIdx.x;
    if constexpr (withQ) {
#pragma unroll
        for (int u = 0; u < TR::NQ; ++u) {
            const int x = tid + u * TR::NT;
            if (x < TR::QV) {
                const int s = x / (DK / 8), d0 = (x % (DK / 8)) * 8;
                *reinterpret_cast<uint4*>(Qs + s * QROW + d0) = R.q[u];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < TR::NK; ++u) {
        const int x = tid + u * TR::NT;
        if (x < TR::KP) {
            const int ps = x % (TC / 2), d0 = (x / (TC / 2)) * 8;
            const int s = 2 * ps;
            if constexpr (withQ) {
                *reinterpret_cast<uint4*>(Ks + s * QROW + d0) = R.k[u][0];
                *reinterpret_cast<uint4*>(Ks + (s + 1) * QROW + d0) = R.k[u][1];
            }
            const bf16_t* e0 = reinterpret_cast<const bf16_t*>(&R.k[u][0]);
            const bf16_t* e1 = reinterpret_cast<const bf16_t*>(&R.k[u][1]);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint32_t*>(KTs + (d0 + j) * TROW + s) = pack2(e0[j], e1[j]);
        }
    }
#pragma unroll
    for (int u = 0; u < TR::NV; ++u) {
        const int x = tid + u * TR::NT;
        if (x < TR::VP) {
            const int ps = x % (TC / 2), c0 = (x / (TC / 2)) * 8;
            const int s = 2 * ps;
            const bf16_t* e0 = reinterpret_cast<const bf16_t*>(&R.v[u][0]);
            const bf16_t* e1 = reinterpret_cast<const bf16_t*>(&R.v[u][1]);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint32_t*>(VTs + (c0 + j) * TROW + s) = pack2(e0[j], e1[j]);
        }
    }
    if (tid < TC) araw[tid] = R.a;
    if constexpr (withQ) {
#pragma unroll
        for (int u = 0; u < TR::NL; ++u) {
            const int x = tid + u * TR::NT;
            if (x < TC * lu) lam_s[x] = R.lam[u];
        }
    }
}

// Wave 0: local inclusive cumsum of a and e_s = exp(A_end - A_s).
__device__ __forceinline__ void tile_decay(const float* araw, float* aloc, float* ev) {
    wave_cumsum(araw, aloc, TC);
    __builtin_amdgcn_wave_barrier();
    const int lane = threadIdx.x & 63;
    const float end = __shfl(aloc[TC - 1], 0);  // all lanes read the same slot
    ev[lane] = __expf(end - aloc[lane]);
}

// U (d_k x 16 columns of this wave) of the staged tile: U = K^T diag(e) V.
// Accumulates into u (C-layout: lane holds U[16 kt + 4 g + i][c0 + m16]).
template <int DK>
__device__ __forceinline__ void tile_state(f32x4 (&u)[DK / 16], const bf16_t* KTs,
                                           const bf16_t* VTs, const float* ev, int wave) {
    constexpr int TROW = TC + PAD;
    const int lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ss = 0; ss < TC / 32; ++ss) {
        const int s0 = 32 * ss + 8 * g;
        const bf16x8 vr = *reinterpret_cast<const bf16x8*>(VTs + (wave * 16 + m16) * TROW + s0);
        const float4 e0 = *reinterpret_cast<const float4*>(ev + s0);
        const float4 e1 = *reinterpret_cast<const float4*>(ev + s0 + 4);
        bf16x8 b;
        b[0] = (__bf16)((float)vr[0] * e0.x); b[1] = (__bf16)((float)vr[1] * e0.y);
        b[2] = (__bf16)((float)vr[2] * e0.z); b[3] = (__bf16)((float)vr[3] * e0.w);
        b[4] = (__bf16)((float)vr[4] * e1.x); b[5] = (__bf16)((float)vr[5] * e1.y);
        b[6] = (__bf16)((float)vr[6] * e1.z); b[7] = (__bf16)((float)vr[7] * e1.w);
#pragma unroll
        for (int kt = 0; kt < DK / 16; ++kt) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(KTs + (16 * kt + m16) * TROW + s0);
            u[kt] = mma(ka, b, u[kt]);
        }
    }
}

template <int N>
__device__ __forceinline__ float pick(const float (&x)[N], int idx) {
    float r = x[0];
#pragma unroll
    for (int l = 1; l < N; ++l) r = idx == l ? x[l] : r;
    return r;
}

// Scores of row block RB against key blocks 0..RB, masked, to LDS as bf16.
template <int DK, int RB>
__device__ __forceinline__ void tile_scores(const bf16_t* Qs, const bf16_t* Ks, bf16_t* Ps,
                                            const float* aloc, const float* lam_s, int lu) {
    constexpr int QROW = DK + PAD, TROW = TC + PAD;
    typedef HD<DK> H;
    const int lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
    const int r = 16 * RB + m16;
    typename H::frag qb[H::NKS];
#pragma unroll
    for (int ks = 0; ks < H::NKS; ++ks)
        qb[ks] = *reinterpret_cast<const typename H::frag*>(Qs + r * QROW + ks * H::KS +
                                                             g * H::KPL);
    f32x4 acc[RB + 1];
#pragma unroll
    for (int sb = 0; sb <= RB; ++sb) acc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < H::NKS; ++ks) {
#pragma unroll
        for (int sb = 0; sb <= RB; ++sb) {
            const typename H::frag ka = *reinterpret_cast<const typename H::frag*>(
                Ks + (16 * sb + m16) * QROW + ks * H::KS + g * H::KPL);
            acc[sb] = mma(ka, qb[ks], acc[sb]);
        }
    }
    float lamr[LOGTC + 1];
#pragma unroll
    for (int l = 0; l <= LOGTC; ++l) lamr[l] = l < lu ? lam_s[r * lu + l] : 0.f;
    const float Ar = aloc[r];
#pragma unroll
    for (int sb = 0; sb <= RB; ++sb) {
        float w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 16 * sb + 4 * g + i;
            w[i] = s <= r ? acc[sb][i] * pick(lamr, fenwick_level(r, s)) * __expf(Ar - aloc[s])
                          : 0.f;
        }
        *reinterpret_cast<bf16x4*>(Ps + r * TROW + 16 * sb + 4 * g) = pack4(w[0], w[1], w[2], w[3]);
    }
    if constexpr ((RB & 1) == 0 && RB + 1 < NRB) {
        // the K=32 product below pairs key blocks; the block past the diagonal is zero
        *reinterpret_cast<bf16x4*>(Ps + r * TROW + 16 * (RB + 1) + 4 * g) = bf16x4{};
    }
}

template <int DK, int NW>
__device__ __forceinline__ void scores_for_wave(int wave, const bf16_t* Qs, const bf16_t* Ks,
                                                bf16_t* Ps, const float* aloc,
                                                const float* lam_s, int lu) {
#pragma unroll
    for (int rb0 = 0; rb0 < NRB; rb0 += NW) {
        const int rb = rb0 + wave;
        switch (rb) {
            case 0: tile_scores<DK, 0>(Qs, Ks, Ps, aloc, lam_s, lu); break;
            case 1: tile_scores<DK, 1>(Qs, Ks, Ps, aloc, lam_s, lu); break;
            case 2: tile_scores<DK, 2>(Qs, Ks, Ps, aloc, lam_s, lu); break;
            case 3: tile_scores<DK, 3>(Qs, Ks, Ps, aloc, lam_s, lu); break;
            default: break;
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Segment states: for each (bh, segment except the last, column block) the
// decayed sum of k v^T over the segment, fp32 [d_v][d_k] at the segment's end.

template <int DK, int NW>
__global__ __launch_bounds__(NW * 64) void k_seg_state(FusedParams p) {
    typedef TileRegs<DK, NW> TR;
    constexpr int DVW = NW * 16;
    constexpr int NDT = DK / 16;
    extern __shared__ __align__(16) char smem[];
    bf16_t* KTs = reinterpret_cast<bf16_t*>(smem);
    bf16_t* VTs = reinterpret_cast<bf16_t*>(smem + round16(DK * (TC + PAD) * 2));
    float* araw = reinterpret_cast<float*>(smem + round16(DK * (TC + PAD) * 2) +
                                           round16(DVW * (TC + PAD) * 2));
    float* aloc = araw + round16(TC * 4) / 4;
    float* ev = aloc + round16(TC * 4) / 4;

    const int nsegs = p.nseg - 1;
    int blk = xcd_block(blockIdx.x, gridDim.x);
    const int dvb = blk % p.ndvb;
    blk /= p.ndvb;
    const int seg = blk % nsegs;
    const int bh = blk / nsegs;
    const int cb = dvb * DVW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
    const size_t row0 = (size_t)bh * p.T;
    const int tile0 = seg << p.m, ntl = 1 << p.m;

    f32x4 u[NDT];
#pragma unroll
    for (int kt = 0; kt < NDT; ++kt) u[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float total = 0.f;
    TR R;
    load_tile<DK, NW, false>(R, nullptr, p.k, p.v, p.a, nullptr, row0, tile0 * TC, p.T, p.dv, cb,
                             p.L, p.LU);
    for (int il = 0; il < ntl; ++il) {
        __syncthreads();
        store_tile<DK, NW, false>(R, nullptr, nullptr, KTs, VTs, nullptr, araw, p.LU);
        __syncthreads();
        if (il + 1 < ntl)
            load_tile<DK, NW, false>(R, nullptr, p.k, p.v, p.a, nullptr, row0,
                                     (tile0 + il + 1) * TC, p.T, p.dv, cb, p.L, p.LU);
        if (wave == 0) tile_decay(araw, aloc, ev);
        __syncthreads();
        const float tot = wave_uniform(aloc[TC - 1]);
        const float f = __expf(tot);
#pragma unroll
        for (int kt = 0; kt < NDT; ++kt) {
            u[kt][0] *= f; u[kt][1] *= f; u[kt][2] *= f; u[kt][3] *= f;
        }
        tile_state<DK>(u, KTs, VTs, ev, wave);
        total += tot;
    }
    float* dst = p.useg + ((size_t)bh * p.nseg + seg) * p.dv * DK;
    const int c = cb + wave * 16 + m16;
#pragma unroll
    for (int kt = 0; kt < NDT; ++kt)
        *reinterpret_cast<float4*>(dst + (size_t)c * DK + 16 * kt + 4 * g) =
            make_float4(u[kt][0], u[kt][1], u[kt][2], u[kt][3]);
    if (threadIdx.x == 0 && dvb == 0) p.stot[(size_t)bh * p.nseg + seg] = total;
}

// ---------------------------------------------------------------------------
// Main fused kernel: one block per (bh, segment, column block).

template <int DK, int NW>
__global__ __launch_bounds__(NW * 64) void k_fused_fwd(FusedParams p) {
    typedef TileRegs<DK, NW> TR;
    typedef HD<DK> H;
    constexpr int DVW = NW * 16;
    constexpr int NDT = DK / 16;
    constexpr int QROW = DK + PAD, TROW = TC + PAD;
    extern __shared__ __align__(16) char smem[];
    const Lds lo = fused_lds(DK, DVW, p.LU, p.ntop);
    bf16_t* Qs = reinterpret_cast<bf16_t*>(smem + lo.q);
    bf16_t* Ks = reinterpret_cast<bf16_t*>(smem + lo.k);
    bf16_t* KTs = reinterpret_cast<bf16_t*>(smem + lo.kt);
    bf16_t* VTs = reinterpret_cast<bf16_t*>(smem + lo.vt);
    bf16_t* Ps = reinterpret_cast<bf16_t*>(smem + lo.p);
    float* lam_s = reinterpret_cast<float*>(smem + lo.lam);
    float* araw = reinterpret_cast<float*>(smem + lo.araw);
    float* aloc = reinterpret_cast<float*>(smem + lo.aloc);
    float* ev = reinterpret_cast<float*>(smem + lo.ev);
    typename H::frag* top = reinterpret_cast<typename H::frag*>(smem + lo.top);

    int blk = xcd_block(blockIdx.x, gridDim.x);
    const int dvb = blk % p.ndvb;
    blk /= p.ndvb;
    const int seg = blk % p.nseg;
    const int bh = blk / p.nseg;
    const int cb = dvb * DVW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
    const int c0 = cb + wave * 16;  // first column of this wave
    const size_t row0 = (size_t)bh * p.T;
    const int tile0 = seg << p.m;
    const int ntl = min(1 << p.m, p.ntiles - tile0);
    const int lu = p.LU;

    // coarse levels of this segment: Fenwick nodes over segments, bf16 in LDS
    float logd_top[kTopMax];
#pragma unroll
    for (int q = 0; q < kTopMax; ++q) {
        logd_top[q] = 0.f;
        if (q < p.ntop && ((seg >> q) & 1)) {
            const int node = ((seg >> q) << q) - 1;
            const double* cum = p.scum + (size_t)bh * p.nseg;
            logd_top[q] = (float)(cum[seg - 1] - cum[node]);
            const float* G = p.useg + ((size_t)bh * p.nseg + node) * p.dv * DK +
                             (size_t)(c0 + m16) * DK;
#pragma unroll
            for (int ks = 0; ks < H::NKS; ++ks) {
                typename H::frag f;
                if constexpr (DK >= 32) {
                    const float4 x = *reinterpret_cast<const float4*>(G + 32 * ks + 4 * g);
                    const float4 y = *reinterpret_cast<const float4*>(G + 32 * ks + 16 + 4 * g);
                    f = cvt8(f32x4{x.x, x.y, x.z, x.w}, f32x4{y.x, y.y, y.z, y.w});
                } else {
                    const float4 x = *reinterpret_cast<const float4*>(G + 4 * g);
                    f = cvt4(f32x4{x.x, x.y, x.z, x.w});
                }
                top[((q * NW + wave) * H::NKS + ks) * 64 + lane] = f;
            }
        }
    }

    // levels inside the segment: fp32 states in registers
    f32x4 G[kMaxLocal][NDT];
    float logd_loc[kMaxLocal];
#pragma unroll
    for (int s = 0; s < kMaxLocal; ++s) logd_loc[s] = 0.f;

    TR R;
    load_tile<DK, NW, true>(R, p.q, p.k, p.v, p.a, p.lam, row0, tile0 * TC, p.T, p.dv, cb, p.L,
                            lu);
    for (int il = 0; il < ntl; ++il) {
        const int i = tile0 + il;
        const int nvalid = min(TC, p.T - i * TC);
        __syncthreads();
        store_tile<DK, NW, true>(R, Qs, Ks, KTs, VTs, lam_s, araw, lu);
        __syncthreads();
        if (il + 1 < ntl)
            load_tile<DK, NW, true>(R, p.q, p.k, p.v, p.a, p.lam, row0, (i + 1) * TC, p.T, p.dv,
                                    cb, p.L, lu);
        if (wave == 0) tile_decay(araw, aloc, ev);
        __syncthreads();
        scores_for_wave<DK, NW>(wave, Qs, Ks, Ps, aloc, lam_s, lu);
        __syncthreads();
        const float tot = wave_uniform(aloc[TC - 1]);  // wave-uniform

        // ---- outputs of this wave's 16 columns, all rows of the tile
        f32x4 o[NRB];
        typename H::frag qp[NRB][H::NKS];
        float Ar[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            o[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r = 16 * rb + m16;
            Ar[rb] = aloc[r];
#pragma unroll
            for (int ks = 0; ks < H::NKS; ++ks) {
                if constexpr (DK >= 32) {
                    // head-dim order of the register states: 4g..4g+3, 16+4g..16+4g+3
                    const bf16x4 x = *reinterpret_cast<const bf16x4*>(Qs + r * QROW + 32 * ks + 4 * g);
                    const bf16x4 y =
                        *reinterpret_cast<const bf16x4*>(Qs + r * QROW + 32 * ks + 16 + 4 * g);
                    qp[rb][ks] = bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
                } else {
                    qp[rb][ks] = *reinterpret_cast<const bf16x4*>(Qs + r * QROW + 4 * g);
                }
            }
        }
        // intra-tile block: O^T = V^T P^T over pairs of 16-token key blocks
#pragma unroll
        for (int sp = 0; sp < NRB / 2; ++sp) {
            const bf16x8 va =
                *reinterpret_cast<const bf16x8*>(VTs + (wave * 16 + m16) * TROW + 32 * sp + 8 * g);
#pragma unroll
            for (int rb = 2 * sp; rb < NRB; ++rb) {
                const int r = 16 * rb + m16;
                const bf16x8 pb = *reinterpret_cast<const bf16x8*>(Ps + r * TROW + 32 * sp + 8 * g);
                o[rb] = mma(va, pb, o[rb]);
            }
        }
        // levels inside the segment
#pragma unroll
        for (int s = 0; s < kMaxLocal; ++s) {
            if (s < p.m && ((il >> s) & 1)) {
                typename H::frag ga[H::NKS];
#pragma unroll
                for (int ks = 0; ks < H::NKS; ++ks) {
                    if constexpr (DK >= 32) ga[ks] = cvt8(G[s][2 * ks], G[s][2 * ks + 1]);
                    else ga[ks] = cvt4(G[s][ks]);
                }
                f32x4 y[NRB];
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) y[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < H::NKS; ++ks)
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) y[rb] = mma(ga[ks], qp[rb][ks], y[rb]);
                const int lev = LOGTC + s + 1;
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    const float w = lam_s[(16 * rb + m16) * lu + lev] * __expf(Ar[rb] + logd_loc[s]);
                    o[rb][0] += w * y[rb][0];
                    o[rb][1] += w * y[rb][1];
                    o[rb][2] += w * y[rb][2];
                    o[rb][3] += w * y[rb][3];
                }
            }
        }
        // levels above the segment
#pragma unroll
        for (int q = 0; q < kTopMax; ++q) {
            if (q < p.ntop && ((seg >> q) & 1)) {
                f32x4 y[NRB];
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) y[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < H::NKS; ++ks) {
                    const typename H::frag ga = top[((q * NW + wave) * H::NKS + ks) * 64 + lane];
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) y[rb] = mma(ga, qp[rb][ks], y[rb]);
                }
                const int lev = LOGTC + p.m + q + 1;
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    const float w = lam_s[(16 * rb + m16) * lu + lev] * __expf(Ar[rb] + logd_top[q]);
                    o[rb][0] += w * y[rb][0];
                    o[rb][1] += w * y[rb][1];
                    o[rb][2] += w * y[rb][2];
                    o[rb][3] += w * y[rb][3];
                }
            }
        }
        float* orow = p.out + (row0 + (size_t)i * TC) * p.dv + c0 + 4 * g;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const int r = 16 * rb + m16;
            if (r < nvalid)
                *reinterpret_cast<float4*>(orow + (size_t)r * p.dv) =
                    make_float4(o[rb][0], o[rb][1], o[rb][2], o[rb][3]);
        }

        // ---- Fenwick update over tiles: fold the tile's state and the slots
        // below lssb(il+1) into slot lssb(il+1)
        if (il + 1 < ntl) {
            f32x4 u[NDT];
#pragma unroll
            for (int kt = 0; kt < NDT; ++kt) u[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            tile_state<DK>(u, KTs, VTs, ev, wave);
            const int j = lssb((uint64_t)il + 1);
#pragma unroll
            for (int s = 0; s < kMaxLocal; ++s) {
                if (s < j) {
                    const float w = __expf(logd_loc[s] + tot);
#pragma unroll
                    for (int kt = 0; kt < NDT; ++kt) {
                        u[kt][0] += w * G[s][kt][0];
                        u[kt][1] += w * G[s][kt][1];
                        u[kt][2] += w * G[s][kt][2];
                        u[kt][3] += w * G[s][kt][3];
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < kMaxLocal; ++s) {
                if (s == j) {
#pragma unroll
                    for (int kt = 0; kt < NDT; ++kt) G[s][kt] = u[kt];
                    logd_loc[s] = 0.f;
                } else {
                    logd_loc[s] += tot;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < kTopMax; ++q) logd_top[q] += tot;
    }
}

// ---------------------------------------------------------------------------
// host side

FusedPlan plan_fused(int BH, int T, int dk, int dv, int lu, int force_m) {
    FusedPlan pl{};
    if (lu > TileRegs<16, 4>::LUMAX) return pl;  // too many levels to stage per token
    const int nw = dv >= 64 ? 4 : dv / 16;
    pl.dvw = nw * 16;
    pl.ndvb = dv / pl.dvw;
    pl.ntiles = (T + TC - 1) / TC;
    const long per_seg_blocks = (long)BH * pl.ndvb;
    const int lds_cap = 160 * 1024;
    // Largest segment (fewest extra reads of K and V by the segment-state
    // pass) that still gives every CU a block; if no size does, the smallest
    // segment whose coarse levels still fit in LDS.
    int best = -1, smallest_fit = -1;
    for (int m = kMaxLocal; m >= 0; --m) {
        const int nseg = (pl.ntiles + (1 << m) - 1) >> m;
        int ntop = 0;
        while ((1 << ntop) < nseg) ++ntop;  // bit_length(nseg - 1)
        if (ntop > kTopMax || fused_lds(dk, pl.dvw, lu, ntop).total > lds_cap) break;
        smallest_fit = m;
        if (per_seg_blocks * nseg >= 256) {
            best = m;
            break;
        }
    }
    if (best < 0) best = smallest_fit;
    if (force_m >= 0) {  // a requested segment size, if its coarse levels fit
        const int nseg = (pl.ntiles + (1 << force_m) - 1) >> force_m;
        int ntop = 0;
        while ((1 << ntop) < nseg) ++ntop;
        best = (force_m <= kMaxLocal && ntop <= kTopMax &&
                fused_lds(dk, pl.dvw, lu, ntop).total <= lds_cap) ? force_m : -1;
    }
    if (best < 0) return pl;
    pl.m = best;
    pl.nseg = (pl.ntiles + (1 << best) - 1) >> best;
    pl.ntop = 0;
    while ((1 << pl.ntop) < pl.nseg) ++pl.ntop;
    pl.lds_main = fused_lds(dk, pl.dvw, lu, pl.ntop).total;
    pl.lds_seg = segstate_lds(dk, pl.dvw);
    pl.ok = 1;
    return pl;
}

namespace {

template <int DK, int NW>
hipError_t launch_fused_t(const FusedParams& p, const FwdParams& scan, unsigned stages,
                          hipStream_t stream, int lds_main, int lds_seg) {
    hipError_t err;
    if (p.nseg > 1 && (stages & kStageChunkState)) {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_seg_state<DK, NW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, lds_seg);
        if (err != hipSuccess) return err;
        const unsigned nblk = (unsigned)p.BH * (p.nseg - 1) * p.ndvb;
        hipLaunchKernelGGL((k_seg_state<DK, NW>), dim3(nblk), dim3(NW * 64), lds_seg, stream, p);
    }
    if (p.nseg > 1 && (stages & kStageScan)) {
        err = launch_fenwick_scan(scan, stream);
        if (err != hipSuccess) return err;
    }
    if (stages & kStageOutput) {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fused_fwd<DK, NW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, lds_main);
        if (err != hipSuccess) return err;
        const unsigned nblk = (unsigned)p.BH * p.nseg * p.ndvb;
        hipLaunchKernelGGL((k_fused_fwd<DK, NW>), dim3(nblk), dim3(NW * 64), lds_main, stream, p);
    }
    return hipGetLastError();
}

template <int DK>
hipError_t launch_fused_dk(const FusedParams& p, const FwdParams& scan, unsigned stages,
                           hipStream_t s, int lm, int ls) {
    switch (p.dvw) {
        case 16: return launch_fused_t<DK, 1>(p, scan, stages, s, lm, ls);
        case 32: return launch_fused_t<DK, 2>(p, scan, stages, s, lm, ls);
        case 64: return launch_fused_t<DK, 4>(p, scan, stages, s, lm, ls);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fused_fwd(const FusedParams& p, const FwdParams& scan, unsigned stages,
                            int lds_main, int lds_seg, hipStream_t stream) {
    switch (p.dk) {
        case 16: return launch_fused_dk<16>(p, scan, stages, stream, lds_main, lds_seg);
        case 32: return launch_fused_dk<32>(p, scan, stages, stream, lds_main, lds_seg);
        case 64: return launch_fused_dk<64>(p, scan, stages, stream, lds_main, lds_seg);
        case 128: return launch_fused_dk<128>(p, scan, stages, stream, lds_main, lds_seg);
    }
    return hipErrorInvalidValue;
}

}  // namespace loglin
