// Chunked forward of the log-linear token mixer on gfx950.
//
// "Log-linear attention, and what a logarithm buys", section 3: with chunk
// size C the Fenwick mask splits into a block diagonal of causal C x C blocks
// (every level up to log2 C lives inside a chunk) plus one term per coarser
// level.  For a query in chunk i and a key in an earlier chunk j the level is
// log2(C) + floor(log2(i XOR j)) + 1, so the keys of coarse level
// log2(C) + p + 1 are exactly the 2^p chunks of the block that ends at chunk
// ((i >> p) << p) - 1, present when bit p of i is set.  Writing G(e) for the
// decayed sum of k v^T over such a block, taken at the end of its last chunk
// e, the output of token t in chunk i is
//
//   o_t = sum_{s in chunk i, s <= t} lambda_t^(level) e^(A_t - A_s) (q_t.k_s) v_s
//       + sum_{p : bit p of i} lambda_t^(log2 C + p + 1) e^(A_t - A_end(e_p)) q_t^T G(e_p).
//
// Three kernels:
//   chunk_state   U_i = sum_{s in chunk i} e^(A_end(i) - A_s) v_s k_s^T   (MFMA)
//   fenwick_scan  G(i) for every chunk i: the Fenwick recurrence of section 2
//                 run over chunks -- U_i plus the decayed live nodes of levels
//                 below lssb(i+1), i.e. the block of 2^lssb(i+1) chunks ending
//                 at i -- computed in place over U (HBM-streaming).
//   chunk_output  the intra-chunk block (S^T = K Q^T on MFMA, masked in
//                 registers, then P V on MFMA) plus Q G(e_p) for each set bit
//                 of i (MFMA), weighted per row, one write of the output.
//
// Workspace layout (per (batch*head) bh, chunk i):
//   ust [BH][N][dv][dk] fp32   U_i transposed, then G(i) transposed
//   tot [BH][N]         fp32   sum of a over the chunk
//   cum [BH][N]         fp64   A at the end of each chunk (prefix of tot)
#include <type_traits>

#include "chunk_stage.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace loglin {

namespace {

// --------------------------------------------------------------------------
// chunk_state: U_i^T = sum_s e^(A_end - A_s) v_s k_s^T  -> ust[bh][i] ([dv][dk])

template <typename E, int C>
__global__ __launch_bounds__(256) void k_chunk_state(FwdParams p) {
    extern __shared__ __align__(16) char smem[];
    const int blk = xcd_local_block(blockIdx.x, gridDim.x);
    const int bh = blk / p.N;
    const int i = blk - bh * p.N;
    const int t0 = i * C;
    const int nvalid = min(C, p.T - t0);
    E* KT = reinterpret_cast<E*>(smem);
    E* VT = KT + p.dk * (C + kPadT);
    const size_t row0 = (size_t)bh * p.T + t0;
    const int lane0 = threadIdx.x & (kWave - 1);

    // Every load first, without branches (rows past T read the chunk's first
    // row and are zeroed): a of tokens 2l and 2l + 1 in lane l of every wave,
    // and the chunk's k and v rows.
    const float a0 = p.a[row0 + min(2 * lane0, nvalid - 1)];
    const float a1 = p.a[row0 + min(2 * lane0 + 1, nvalid - 1)];
    ChunkRows<E, C, 128, 256> kr, vr;
    kr.load(static_cast<const E*>(p.k) + row0 * p.dk, p.dk, nvalid);
    vr.load(static_cast<const E*>(p.v) + row0 * p.dv, p.dv, nvalid);
    // chunk-local inclusive sum of a in registers (each wave the whole
    // chunk); the chunk total is lane 63's sum
    const bool ok0 = 2 * lane0 < nvalid, ok1 = 2 * lane0 + 1 < nvalid;
    const float x0 = ok0 ? a0 : 0.f, x1 = ok1 ? a1 : 0.f;
    float incl = x0 + x1;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float y = __shfl_up(incl, off, kWave);
        if (lane0 >= off) incl += y;
    }
    const float Aend = __shfl(incl, kWave - 1, kWave);
    const float e0 = ok0 ? __expf(Aend - (incl - x1)) : 0.f;
    const float e1 = ok1 ? __expf(Aend - incl) : 0.f;
    kr.store(p.dk, nullptr, KT, nullptr);
    vr.store_tr_scaled(p.dv, VT, [&](int s) __attribute__((always_inline)) {
        const float y0 = __shfl(e0, s >> 1, kWave), y1 = __shfl(e1, s >> 1, kWave);
        return (s & 1) ? y1 : y0;
    });
    if (threadIdx.x == 0) p.tot[(size_t)bh * p.N + i] = Aend;
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int m = lane & 15, g = lane >> 4;
    const int ntk = p.dk / 16;
    const int ntiles = (p.dv / 16) * ntk;
    float* dstU = p.ust + ((size_t)bh * p.N + i) * p.dv * p.dk;
    for (int tile = wave; tile < ntiles; tile += nw) {
        const int cv0 = (tile / ntk) * 16, ck0 = (tile % ntk) * 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const E* va = VT + (cv0 + m) * (C + kPadT) + 4 * g;
        const E* kb = KT + (ck0 + m) * (C + kPadT) + 4 * g;
#pragma unroll
        for (int S = 0; S < C / 16; ++S) {
            if constexpr (sizeof(E) == 2) {
                acc = mma(Frag<bf16_t, 16>::load(va + 16 * S), Frag<bf16_t, 16>::load(kb + 16 * S),
                          acc);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) acc = mma(va[16 * S + j], kb[16 * S + j], acc);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) dstU[(size_t)(cv0 + 4 * g + r) * p.dk + ck0 + m] = acc[r];
    }
}

// --------------------------------------------------------------------------
// fenwick_scan: one thread per (bh, 4 state elements), walking the chunks.

constexpr int kScanLevels = 16;  // supports up to 2^16 chunks per sequence
constexpr int kScanDepth = 8;    // loads kept in flight per thread

// The state entering the scan for chunk (segment) i: U_i itself, or, when the
// states were computed in NSUB sub-ranges, the sub-range states decayed to the
// end of the segment and summed in order.
template <int NSUB>
struct ScanLoad {
    float4 part[NSUB];
    float tp[NSUB];  // decay totals of the segment (NSUB == 1) or of its sub-ranges,
                     // loaded with the states rather than when they are combined
    __device__ void issue(const FwdParams& p, int bh, int e4, int per4, int i) {
        if constexpr (NSUB == 1) {
            part[0] = reinterpret_cast<const float4*>(p.ust)[((size_t)bh * p.N + i) * per4 + e4];
            tp[0] = p.tot[(size_t)bh * p.N + i];
        } else {
            const float4* src = reinterpret_cast<const float4*>(p.upart) +
                                (((size_t)bh * p.N + i) * NSUB) * per4 + e4;
            const float* t = p.tpart + ((size_t)bh * p.N + i) * NSUB;
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                part[s] = src[(size_t)s * per4];
                tp[s] = t[s];
            }
        }
    }
    // returns the combined state; *total receives the segment's decay total
    __device__ float4 combine(const FwdParams& p, int bh, int i, float* total) const {
        if constexpr (NSUB == 1) {
            *total = tp[0];
            return part[0];
        } else {
            float4 acc = part[NSUB - 1];
            float after = tp[NSUB - 1];  // decay of the sub-ranges after s
#pragma unroll
            for (int s = NSUB - 2; s >= 0; --s) {
                const float w = __expf(after);
                acc.x += w * part[s].x;
                acc.y += w * part[s].y;
                acc.z += w * part[s].z;
                acc.w += w * part[s].w;
                after += tp[s];
            }
            *total = after;
            return acc;
        }
    }
};

// Decay total of chunk (segment) i, summed as ScanLoad::combine sums it.
template <int NSUB>
__device__ __forceinline__ float chunk_total(const FwdParams& p, int bh, int i) {
    if constexpr (NSUB == 1) {
        return p.tot[(size_t)bh * p.N + i];
    } else {
        const float* t = p.tpart + ((size_t)bh * p.N + i) * NSUB;
        float after = t[NSUB - 1];
#pragma unroll
        for (int s = NSUB - 2; s >= 0; --s) after += t[s];
        return after;
    }
}

// Where node i's four elements e4 go: the fp32 node over ust, the bf16 copies
// (row order, or the fused kernel's fragment order; see k_fenwick_scan).
__device__ __forceinline__ size_t node_frag_offset(const FwdParams& p, int e4) {
    const int e = 4 * e4;
    const int col = e / p.dk, d0 = e % p.dk;
    const int cblk = col >> 4, m = col & 15;
    if (p.dk >= 32) {
        const int j = d0 >> 5, w32 = d0 & 31, g = w32 >> 3, half = (w32 >> 2) & 1;
        return (((size_t)cblk * (p.dk / 32) + j) * 64 + 16 * g + m) * 8 + 4 * half;
    }
    return ((size_t)cblk * 64 + 16 * (d0 >> 2) + m) * 4;
}
__device__ __forceinline__ void store_node(const FwdParams& p, int bh, int e4, int per4, int i,
                                           const float4& acc) {
    if (!p.nodes16_only)
        reinterpret_cast<float4*>(p.ust)[((size_t)bh * p.N + i) * per4 + e4] = acc;
    bf16x4 h;
    h[0] = (__bf16)acc.x; h[1] = (__bf16)acc.y; h[2] = (__bf16)acc.z; h[3] = (__bf16)acc.w;
    if (p.gnode16)
        *reinterpret_cast<bf16x4*>(p.gnode16 + ((size_t)bh * p.N + i) * per4 * 4 + 4 * e4) = h;
    if (p.gfrag) {
        const size_t fstride = (size_t)p.dv * p.dk;
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16_t*>(p.gfrag) + ((size_t)bh * p.N + i) * fstride +
                                   node_frag_offset(p, e4)) = h;
    }
}

// The nodes over chunks formed independently, one thread per (bh, node,
// 4 state elements): node i is the decayed sum, to the end of chunk i, of
// the states of the 2^lssb(i + 1) chunks ending at i, here by Horner's rule
// over them (the scan below reaches the same sums through its running
// levels).  It reads each state once per node that covers it instead of
// once, so it serves where the scan's walk, one thread per (bh, 4 elements),
// would leave most of the GPU idle; and only where no node overwrites a
// state another thread reads: sub-range states (NSUB > 1), or no fp32 copy
// of the nodes (nodes16_only).
template <int NSUB>
__global__ __launch_bounds__(256) void k_fenwick_nodes(FwdParams p) {
    const int per4 = p.dv * p.dk / 4;
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long per_bh = (long)p.nscan * per4;
    const int bh = (int)(gid / per_bh);
    if (bh >= p.BH) return;
    const long rem = gid - (long)bh * per_bh;
    const int i = (int)(rem / per4);
    const int e4 = (int)(rem - (long)i * per4);
    const int r0 = i + 1 - (1 << lssb((uint64_t)i + 1));
    const int width = i + 1 - r0;
    // the node's states, kDepth loads in flight (issued before the totals)
    constexpr int kDepth = 4;
    ScanLoad<NSUB> ring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
        if (d < width) ring[d].issue(p, bh, e4, per4, r0 + d);
    // decay total up to the end of each chunk, in fp64 as the scan forms it
    // (the totals before the node loaded eight at a time, summed in order)
    double c = 0.0;
    int r = 0;
    for (; r + 8 <= r0; r += 8) {
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = chunk_total<NSUB>(p, bh, r + u);
#pragma unroll
        for (int u = 0; u < 8; ++u) c += (double)t[u];
    }
    for (; r < r0; ++r) c += (double)chunk_total<NSUB>(p, bh, r);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < width; k0 += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int k = k0 + d;
            if (k < width) {
                float total;
                const float4 st = ring[d].combine(p, bh, r0 + k, &total);
                if (k + kDepth < width) ring[d].issue(p, bh, e4, per4, r0 + k + kDepth);
                const float w = k == 0 ? 0.f : __expf(total);  // chunk r0 + k's decay onto the sum
                acc.x = w * acc.x + st.x;
                acc.y = w * acc.y + st.y;
                acc.z = w * acc.z + st.z;
                acc.w = w * acc.w + st.w;
                c += (double)total;
            }
        }
    }
    store_node(p, bh, e4, per4, i, acc);
    if (e4 == 0) p.cum[(size_t)bh * p.N + i] = c;
}

template <int NSUB>
__global__ __launch_bounds__(256) void k_fenwick_scan(FwdParams p) {
    constexpr int DEPTH = NSUB >= 8 ? 1 : kScanDepth / NSUB;  // segments kept in flight
    const int per4 = p.dv * p.dk / 4;
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int bh = (int)(gid / per4);
    const int e4 = (int)(gid - (long)bh * per4);
    if (bh >= p.BH) return;
    const int n = p.nscan;  // nodes produced: 0 .. n-1
    float4* base = reinterpret_cast<float4*>(p.ust) + (size_t)bh * p.N * per4 + e4;
    double* cum = p.cum + (size_t)bh * p.N;

    // bf16 copy of each node in the operand order of the fused kernel's level
    // products: [node][column block of 16][32-wide step][lane][8], lane 16g + m
    // holding rows 8g..8g+7 of the step for column m; for d_k = 16 one step of
    // 4 rows (4g..4g+3) per lane.
    bf16_t* frag = nullptr;
    size_t fstride = 0;
    if (p.gfrag) {
        fstride = (size_t)p.dv * p.dk;
        frag = reinterpret_cast<bf16_t*>(p.gfrag) + (size_t)bh * p.N * fstride + node_frag_offset(p, e4);
    }
    float4 live[kScanLevels];
    double lcum[kScanLevels];
#pragma unroll
    for (int q = 0; q < kScanLevels; ++q) {
        live[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        lcum[q] = 0.0;
    }
    ScanLoad<NSUB> ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (d < n) ring[d].issue(p, bh, e4, per4, d);
    double c = 0.0;
    for (int i0 = 0; i0 < n; i0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int i = i0 + d;
            if (i < n) {
                float total;
                float4 acc = ring[d].combine(p, bh, i, &total);
                if (i + DEPTH < n) ring[d].issue(p, bh, e4, per4, i + DEPTH);
                c += (double)total;
                const int j = lssb((uint64_t)i + 1);
#pragma unroll
                for (int q = 0; q < kScanLevels; ++q) {
                    if (q < j) {
                        const float w = __expf((float)(c - lcum[q]));
                        acc.x += w * live[q].x;
                        acc.y += w * live[q].y;
                        acc.z += w * live[q].z;
                        acc.w += w * live[q].w;
                    }
                }
#pragma unroll
                for (int q = 0; q < kScanLevels; ++q) {
                    if (q == j) {
                        live[q] = acc;
                        lcum[q] = c;
                    }
                }
                if (!p.nodes16_only) base[(size_t)i * per4] = acc;
                if (p.gnode16) {
                    bf16x4 h;
                    h[0] = (__bf16)acc.x; h[1] = (__bf16)acc.y; h[2] = (__bf16)acc.z;
                    h[3] = (__bf16)acc.w;
                    *reinterpret_cast<bf16x4*>(p.gnode16 + ((size_t)bh * p.N + i) * per4 * 4 + 4 * e4) = h;
                }
                if (frag) {
                    bf16x4 h;
                    h[0] = (__bf16)acc.x; h[1] = (__bf16)acc.y; h[2] = (__bf16)acc.z;
                    h[3] = (__bf16)acc.w;
                    *reinterpret_cast<bf16x4*>(frag + (size_t)i * fstride) = h;
                }
                if (e4 == 0) cum[i] = c;
            }
        }
    }
}

// --------------------------------------------------------------------------
// chunk_output: intra-chunk block plus the coarse levels, one block per chunk,
// one wave per 16 query rows.

template <typename E, int C, int DK>
__global__ __launch_bounds__(C / 16 * 64) void k_chunk_output(FwdParams p) {
    constexpr int NW = C / 16;
    constexpr int LOGC = (C == 16) ? 4 : (C == 32) ? 5 : (C == 64) ? 6 : 7;
    constexpr int KS = HeadStep<E, DK>::KS;
    constexpr int NKS = DK / KS;
    typedef Frag<E, KS> FR;
    typedef typename FR::type frag_t;
    constexpr int KPL = FR::kpl;

    extern __shared__ __align__(16) char smem[];
    const int blk = xcd_local_block(blockIdx.x, gridDim.x);
    const int bh = blk / p.N;
    const int i = blk - bh * p.N;
    const int t0 = i * C;
    const int nvalid = min(C, p.T - t0);
    const int dv = p.dv;
    float* a_raw = reinterpret_cast<float*>(smem);
    float* A = a_raw + C;
    E* Kn = reinterpret_cast<E*>(A + C);
    E* VT = Kn + C * (DK + kPadK);
    const size_t row0 = (size_t)bh * p.T + t0;

    for (int s = threadIdx.x; s < C; s += blockDim.x) a_raw[s] = s < nvalid ? p.a[row0 + s] : 0.f;
    stage_natural<E, C>(static_cast<const E*>(p.k) + row0 * DK, DK, nvalid, Kn);
    stage_transposed<E, C>(static_cast<const E*>(p.v) + row0 * dv, dv, nvalid, VT, nullptr);
    __syncthreads();
    if (threadIdx.x < kWave) wave_cumsum(a_raw, A, C);
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int R = threadIdx.x / kWave;  // row block of this wave
    const int m = lane & 15, g = lane >> 4;
    const int r = 16 * R + m;           // query row within the chunk
    const bool rvalid = r < nvalid;
    const size_t trow = row0 + r;

    // Q row r as the B operand of S^T = K Q^T (contraction over the head dim)
    frag_t qf[NKS];
    const E* qrow = static_cast<const E*>(p.q) + trow * DK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (rvalid) {
            qf[ks] = FR::load(qrow + ks * KS + g * KPL);
        } else {
            qf[ks] = frag_t{};
        }
    }
    // lambda of row r at the levels inside a chunk
    float lamr[LOGC + 1];
    const float* lrow = p.lam + trow * p.L;
#pragma unroll
    for (int l = 0; l <= LOGC; ++l) lamr[l] = (rvalid && l < p.L) ? lrow[l] : 0.f;
    const float Ar = A[r];

    // P^T tiles: the masked scores, kept as B operands of O^T = V^T P^T
    typedef typename std::conditional<sizeof(E) == 2, bf16x4, f32x4>::type pfrag_t;
    pfrag_t P[NW];
#pragma unroll
    for (int S = 0; S < NW; ++S) {
        if (S <= R) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const E* krow = Kn + (16 * S + m) * (DK + kPadK) + g * KPL;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) acc = mma(FR::load(krow + ks * KS), qf[ks], acc);
            float w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int s = 16 * S + 4 * g + q;
                const float lam = pick_level<LOGC>(lamr, fenwick_level(r, s));
                w[q] = s <= r ? acc[q] * lam * __expf(Ar - A[s]) : 0.f;
            }
            if constexpr (sizeof(E) == 2) {
                P[S] = pack4(w[0], w[1], w[2], w[3]);
            } else {
                P[S] = f32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }

    const double* cum = p.cum + (size_t)bh * p.N;
    float* orow = p.out + trow * dv;
    for (int cv0 = 0; cv0 < dv; cv0 += 16) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const E* vrow = VT + (cv0 + m) * (C + kPadT) + 4 * g;
#pragma unroll
        for (int S = 0; S < NW; ++S) {
            if (S <= R) {
                if constexpr (sizeof(E) == 2) {
                    acc = mma(Frag<bf16_t, 16>::load(vrow + 16 * S), P[S], acc);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc = mma(vrow[16 * S + j], P[S][j], acc);
                }
            }
        }
        // coarse levels: one Fenwick node per set bit of the chunk index
        for (int pb = 0; (i >> pb) != 0; ++pb) {
            if (!((i >> pb) & 1)) continue;
            const int node = ((i >> pb) << pb) - 1;
            const float dl = (float)(cum[i - 1] - cum[node]);
            const int lev = LOGC + pb + 1;
            const float w = rvalid ? lrow[lev] * __expf(Ar + dl) : 0.f;
            const float* G = p.ust + ((size_t)bh * p.N + node) * dv * DK + (size_t)(cv0 + m) * DK +
                             g * KPL;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) y = mma(FR::from_f32(G + ks * KS), qf[ks], y);
            acc[0] += w * y[0];
            acc[1] += w * y[1];
            acc[2] += w * y[2];
            acc[3] += w * y[3];
        }
        if (rvalid)
            *reinterpret_cast<float4*>(orow + cv0 + 4 * g) = make_float4(acc[0], acc[1], acc[2],
                                                                          acc[3]);
    }
}

template <typename E, int C>
size_t state_smem(int dk, int dv) {
    return (size_t)(dk + dv) * (C + kPadT) * sizeof(E);
}
template <typename E, int C, int DK>
size_t output_smem(int dv) {
    return 2 * C * sizeof(float) + (size_t)C * (DK + kPadK) * sizeof(E) +
           (size_t)dv * (C + kPadT) * sizeof(E);
}

template <typename E, int C, int DK>
hipError_t launch_typed(const FwdParams& p, unsigned stages, hipStream_t stream) {
    const int nblk = p.BH * p.N;
    if (p.N > 1 && (stages & kStageChunkState)) {
        const size_t sm1 = state_smem<E, C>(p.dk, p.dv);
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_chunk_state<E, C>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm1);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((k_chunk_state<E, C>), dim3(nblk), dim3(256), sm1, stream, p);
    }
    if (p.N > 1 && (stages & kStageScan)) {
        hipError_t err = launch_fenwick_scan(p, stream);
        if (err != hipSuccess) return err;
    }
    if (!(stages & kStageOutput)) return hipGetLastError();
    const size_t sm3 = output_smem<E, C, DK>(p.dv);
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_chunk_output<E, C, DK>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm3);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_chunk_output<E, C, DK>), dim3(nblk), dim3(C / 16 * 64), sm3, stream, p);
    return hipGetLastError();
}

template <typename E, int C>
hipError_t launch_c(const FwdParams& p, unsigned st, hipStream_t s) {
    switch (p.dk) {
        case 16: return launch_typed<E, C, 16>(p, st, s);
        case 32: return launch_typed<E, C, 32>(p, st, s);
        case 64: return launch_typed<E, C, 64>(p, st, s);
        case 128: return launch_typed<E, C, 128>(p, st, s);
    }
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_e(const FwdParams& p, unsigned st, hipStream_t s) {
    switch (p.C) {
        case 16: return launch_c<E, 16>(p, st, s);
        case 32: return launch_c<E, 32>(p, st, s);
        case 64: return launch_c<E, 64>(p, st, s);
        case 128: return launch_c<E, 128>(p, st, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fenwick_scan(const FwdParams& p, hipStream_t stream) {
    if (p.nscan <= 0) return hipSuccess;
    const long threads = (long)p.BH * (p.dv * p.dk / 4);
    const dim3 grid((unsigned)((threads + 255) / 256));
    const int nsub = p.upart ? p.nsub : 1;
    if ((nsub > 1 || p.nodes16_only) && p.nscan >= 4 && grid.x < 256) {
        // the walk would run on fewer blocks than the GPU has compute units:
        // every node by a thread of its own
        const dim3 g2((unsigned)((threads * p.nscan + 255) / 256));
        switch (nsub) {
            case 1: hipLaunchKernelGGL(k_fenwick_nodes<1>, g2, dim3(256), 0, stream, p); break;
            case 2: hipLaunchKernelGGL(k_fenwick_nodes<2>, g2, dim3(256), 0, stream, p); break;
            case 4: hipLaunchKernelGGL(k_fenwick_nodes<4>, g2, dim3(256), 0, stream, p); break;
            case 8: hipLaunchKernelGGL(k_fenwick_nodes<8>, g2, dim3(256), 0, stream, p); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (p.upart ? p.nsub : 1) {
        case 1: hipLaunchKernelGGL(k_fenwick_scan<1>, grid, dim3(256), 0, stream, p); break;
        case 2: hipLaunchKernelGGL(k_fenwick_scan<2>, grid, dim3(256), 0, stream, p); break;
        case 4: hipLaunchKernelGGL(k_fenwick_scan<4>, grid, dim3(256), 0, stream, p); break;
        case 8: hipLaunchKernelGGL(k_fenwick_scan<8>, grid, dim3(256), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fwd_chunked(const FwdParams& p, bool bf16, unsigned stages, hipStream_t stream) {
    return bf16 ? launch_e<bf16_t>(p, stages, stream) : launch_e<float>(p, stages, stream);
}

}  // namespace loglin
