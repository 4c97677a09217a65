// Chunked forward of the log-linear Gated DeltaNet on gfx950.
//
// "Log-linear attention, and what a logarithm buys": Gated DeltaNet changes
// the query-key interaction, not the mask (section 1), and the log-linear
// lift composes its temporal mask with the Fenwick level mask (section 3).
// With the gated delta rule of the Gated DeltaNet paper (the page's source 3)
// every bucket state takes the transition G_t = alpha_t (I - beta_t k_t k_t^T)
// and the new token writes beta_t k_t v_t^T, so the weight of key s in o_t is
//     lambda_t^(level(t,s)) beta_s q_t^T Phi(t,s) k_s,   Phi(t,s) = G_t ... G_{s+1}.
//
// Chunks of 64 tokens.  Inside chunk i (tokens t0..t0+63, b_t the sum of a
// from t0 to t, g = b at the chunk's end) the transitions between chunk
// tokens have the compact (UT) form: with
//     N = (I + diag(beta) (K K^T (.) Gamma (.) strict lower))^-1,  Gamma[r,s] = e^(b_r - b_s),
//     Tb = N diag(beta)  (lower triangular),
// the chunk's own block is P = ((Q K^T (.) Gamma (.) L) Tb) (.) Lambda, and
// the chunk acts on a state X taken at t0 - 1 as
//     read by token t:   q'_t^T X,  q'_t = e^(b_t) q_t - ((Q K^T (.) Gamma (.) L) W)_t
//     carried to its end: F X,       F = e^g I - Khat^T W
// with W = Tb diag(e^b) K and Khat_s = e^(g - b_s) k_s; its own tokens add
// U = Khat^T (Tb V) to a state at its end.
//
// Two kernels:
//   k_gdn_chunk   one block per (bh, chunk), every chunk in parallel: P and the
//                 chunk's own output (written to out), and q', F and U to the
//                 workspace (fp32 matrix cores, the inverse by 16 x 16 blocks).
//   k_gdn_levels  one block per (bh, 16 output columns) walks the chunks in
//                 order holding the Fenwick level states over chunks (section
//                 2's recurrence with chunks as tokens and F as the
//                 transition); for a chunk with bit p set it reads level p+1
//                 through q' with lambda of level log2(64) + p + 1 and adds it
//                 to the output.
//
// Workspace (per bh, chunk i):
//   F  [BH][N][DK*DK]  fp32, in the A-operand order of the 16x16x4 MFMA
//   Qp [BH][N][64*DK]  fp32, q' in the same order
//   U  [BH][N][DK][DV] fp32
#include "chunk_stage.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace loglin {

namespace {

constexpr int GC = kGdnChunk;  // tokens per chunk
constexpr int kChunkThreads = 512;
constexpr int kLevelThreads = 256;
constexpr int kLevelCols = 16;   // output columns per level-walk block
constexpr int kXPitch = kLevelCols + 4;

// fp32 MFMA over k in [kb, ke) (multiple of 4): acc += A(m, k) B(k, n) for one
// 16 x 16 tile; fa(m, k) and fb(k, n) give the operands with m, n < 16.
template <class FA, class FB>
__device__ __forceinline__ f32x4 mm_f32(FA fa, FB fb, int kb, int ke, f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    for (int k = kb; k < ke; k += 4) acc = mma(fa(r, k + q), fb(k + q, r), acc);
    return acc;
}

// lower-triangular 16 x 16 tile j of a 64 x 64 matrix (j < 10) -> (row, col) tile
__device__ __forceinline__ void tri_tile(int j, int& ti, int& tj) {
    ti = j < 1 ? 0 : j < 3 ? 1 : j < 6 ? 2 : 3;
    tj = j - ti * (ti + 1) / 2;
}

// index in A-operand order: value (row m, col k) of a [rows][D] matrix as the
// 16x16x4 MFMA reads it -- tile of 16 rows, groups of 4 k-steps, lane, step
__device__ __forceinline__ size_t frag_index(int m, int k, int D) {
    const int rt = m >> 4, ks = k >> 2;
    const int lane = (m & 15) + 16 * (k & 3);
    return (((size_t)rt * (D / 16) + (ks >> 2)) * 64 + lane) * 4 + (ks & 3);
}

template <typename E>
__device__ __forceinline__ float ld(const E* p) {
    return to_f32(*p);
}

template <typename E, int DK, int DV>
struct ChunkSmem {
    static constexpr int PK = DK + 4, PV = DV + 4, PC = GC + 4;
    static constexpr size_t q_off = 0;
    static constexpr size_t k_off = q_off + sizeof(E) * GC * PK;
    static constexpr size_t v_off = k_off + sizeof(E) * GC * PK;
    static constexpr size_t y_off = (v_off + sizeof(E) * GC * PV + 15) / 16 * 16;
    static constexpr size_t t_off = y_off + 4 * GC * PC;
    static constexpr size_t w_off = t_off + 4 * GC * PC;
    static constexpr size_t b_off = w_off + 4 * GC * PK;
    static constexpr size_t beta_off = b_off + 4 * GC;
    static constexpr size_t a_off = beta_off + 4 * GC;
    static constexpr size_t lam_off = a_off + 4 * GC;     // [64][8] levels 0..6
    static constexpr size_t g_off = lam_off + 4 * GC * 8; // [3][16][20] inverse temps
    static constexpr size_t total = g_off + 4 * 3 * 16 * 20;
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kChunkThreads) void k_gdn_chunk(GdnParams p) {
    using S = ChunkSmem<E, DK, DV>;
    constexpr int PK = S::PK, PV = S::PV, PC = S::PC;
    extern __shared__ __align__(16) char smem[];
    E* sQ = reinterpret_cast<E*>(smem + S::q_off);
    E* sK = reinterpret_cast<E*>(smem + S::k_off);
    E* sV = reinterpret_cast<E*>(smem + S::v_off);
    float* sY = reinterpret_cast<float*>(smem + S::y_off);
    float* sT = reinterpret_cast<float*>(smem + S::t_off);
    float* sW = reinterpret_cast<float*>(smem + S::w_off);
    float* sb = reinterpret_cast<float*>(smem + S::b_off);
    float* sbeta = reinterpret_cast<float*>(smem + S::beta_off);
    float* sa = reinterpret_cast<float*>(smem + S::a_off);
    float* slam = reinterpret_cast<float*>(smem + S::lam_off);
    float* sG = reinterpret_cast<float*>(smem + S::g_off);

    const int blk = xcd_local_block(blockIdx.x, gridDim.x);
    const int bh = blk / p.N;
    const int ci = blk - bh * p.N;
    const int t0 = ci * GC;
    const int nvalid = min(GC, p.T - t0);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const size_t row0 = (size_t)bh * p.T + t0;

    // ---- stage the chunk: q, k, v rows (zero past T), a, beta, lambda 0..6
    {
        const E* q = static_cast<const E*>(p.q) + row0 * DK;
        const E* k = static_cast<const E*>(p.k) + row0 * DK;
        const E* v = static_cast<const E*>(p.v) + row0 * DV;
        for (int e = tid; e < GC * DK; e += kChunkThreads) {
            const int r = e / DK, c = e - r * DK;
            const bool ok = r < nvalid;
            sQ[r * PK + c] = ok ? q[(size_t)r * DK + c] : E(0);
            sK[r * PK + c] = ok ? k[(size_t)r * DK + c] : E(0);
        }
        for (int e = tid; e < GC * DV; e += kChunkThreads) {
            const int r = e / DV, c = e - r * DV;
            sV[r * PV + c] = r < nvalid ? v[(size_t)r * DV + c] : E(0);
        }
        if (tid < GC) {
            const bool ok = tid < nvalid;
            sa[tid] = ok ? p.a[row0 + tid] : 0.f;
            sbeta[tid] = ok ? p.beta[row0 + tid] : 0.f;
        }
        const int nl = min(p.L, 7);
        for (int e = tid; e < GC * 8; e += kChunkThreads) {
            const int r = e >> 3, l = e & 7;
            slam[e] = (r < nvalid && l < nl) ? p.lam[(row0 + r) * p.L + l] : 0.f;
        }
        // upper tiles of Y and of the system stay zero
        for (int e = tid; e < GC * GC; e += kChunkThreads) {
            const int r = e / GC, c = e - r * GC;
            if ((c >> 4) > (r >> 4)) {
                sY[r * PC + c] = 0.f;
                sT[r * PC + c] = 0.f;
            }
        }
    }
    __syncthreads();
    if (wave == 0) wave_cumsum(sa, sb, GC);
    __syncthreads();

    // ---- Q K^T and K K^T on the lower tiles, masked and decayed
    for (int j = wave; j < 20; j += kChunkThreads / 64) {
        const bool isq = j < 10;
        int ti, tj;
        tri_tile(isq ? j : j - 10, ti, tj);
        const E* A = isq ? sQ : sK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mm_f32([&](int m, int k) { return ld(A + (16 * ti + m) * PK + k); },
                     [&](int k, int n) { return ld(sK + (16 * tj + n) * PK + k); }, 0, DK, acc);
        const int n = 16 * tj + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * ti + (lane >> 4) * 4 + i;
            const float dec = m >= n ? __expf(sb[m] - sb[n]) : 0.f;
            if (isq)
                sY[m * PC + n] = m >= n ? acc[i] * dec : 0.f;
            else
                sT[m * PC + n] = m > n ? sbeta[m] * acc[i] * dec : 0.f;
        }
    }
    __syncthreads();

    // ---- N = (I + A)^-1 by 16 x 16 blocks: the diagonal blocks by forward
    // substitution (lane c holds column c), then the blocks below them row by
    // row: N_ij = -N_ii sum_{k=j..i-1} A_ik N_kj.
    if (wave < 4 && lane < 16) {
        const int o = 16 * wave, c = lane;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = r == c ? 1.f : 0.f;
#pragma unroll
            for (int u = 0; u < r; ++u) s -= sT[(o + r) * PC + o + u] * x[u];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(o + r) * PC + o + c] = x[r];
    }
    __syncthreads();
    for (int bi = 1; bi < 4; ++bi) {
        // G_ij = sum_{k=j..i-1} A_ik N_kj into temp j (waves 0..i-1)
        if (wave < bi) {
            const int bj = wave;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int bk = bj; bk < bi; ++bk)
                acc = mm_f32([&](int m, int k) { return sT[(16 * bi + m) * PC + 16 * bk + k]; },
                             [&](int k, int n) { return sT[(16 * bk + k) * PC + 16 * bj + n]; }, 0,
                             16, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) sG[(bj * 16 + (lane >> 4) * 4 + i) * 20 + (lane & 15)] = acc[i];
        }
        __syncthreads();
        if (wave < bi) {
            const int bj = wave;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mm_f32([&](int m, int k) { return sT[(16 * bi + m) * PC + 16 * bi + k]; },
                         [&](int k, int n) { return sG[(bj * 16 + k) * 20 + n]; }, 0, 16, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sT[(16 * bi + (lane >> 4) * 4 + i) * PC + 16 * bj + (lane & 15)] = -acc[i];
        }
        __syncthreads();
    }
    // Tb = N diag(beta)
    for (int e = tid; e < GC * GC; e += kChunkThreads) {
        const int r = e / GC, c = e - r * GC;
        if (c <= r) sT[r * PC + c] *= sbeta[c];
    }
    __syncthreads();

    // ---- W = Tb diag(e^b) K -> sW;  U0 = Tb V and P = (Y Tb) (.) Lambda -> registers
    constexpr int NW = 4 * (DK / 16);
    for (int j = wave; j < NW; j += kChunkThreads / 64) {
        const int ti = j / (DK / 16), tn = j % (DK / 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mm_f32([&](int m, int k) { return sT[(16 * ti + m) * PC + k]; },
                     [&](int k, int n) { return ld(sK + k * PK + 16 * tn + n) * __expf(sb[k]); },
                     0, 16 * (ti + 1), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sW[(16 * ti + (lane >> 4) * 4 + i) * PK + 16 * tn + (lane & 15)] = acc[i];
    }
    constexpr int NU = 4 * (DV / 16);
    constexpr int NUW = (NU + 7) / 8;  // U0 tiles per wave
    f32x4 u0[NUW];
#pragma unroll
    for (int x = 0; x < NUW; ++x) {
        u0[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int j = wave + 8 * x;
        if (j < NU) {
            const int ti = j / (DV / 16), tn = j % (DV / 16);
            u0[x] = mm_f32([&](int m, int k) { return sT[(16 * ti + m) * PC + k]; },
                           [&](int k, int n) { return ld(sV + k * PV + 16 * tn + n); }, 0,
                           16 * (ti + 1), u0[x]);
        }
    }
    f32x4 pt[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        pt[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int j = wave + 8 * x;
        if (j < 10) {
            int ti, tj;
            tri_tile(j, ti, tj);
            pt[x] = mm_f32([&](int m, int k) { return sY[(16 * ti + m) * PC + k]; },
                           [&](int k, int n) { return sT[k * PC + 16 * tj + n]; }, 16 * tj,
                           16 * (ti + 1), pt[x]);
            const int n = 16 * tj + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * ti + (lane >> 4) * 4 + i;
                const int lev = fenwick_level((uint32_t)m, (uint32_t)n);
                pt[x][i] = m >= n ? pt[x][i] * slam[m * 8 + lev] : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- q' = e^b Q - Y W -> workspace (A-operand order); chunk 0 reads no level
    float* Qp = p.N > 1 ? p.qp + ((size_t)bh * p.N + ci) * GC * DK : nullptr;
    for (int j = wave; j < (ci > 0 ? NW : 0); j += kChunkThreads / 64) {
        const int ti = j / (DK / 16), tn = j % (DK / 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mm_f32([&](int m, int k) { return sY[(16 * ti + m) * PC + k]; },
                     [&](int k, int n) { return sW[k * PK + 16 * tn + n]; }, 0, 16 * (ti + 1), acc);
        const int n = 16 * tn + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * ti + (lane >> 4) * 4 + i;
            Qp[frag_index(m, n, DK)] = __expf(sb[m]) * ld(sQ + m * PK + n) - acc[i];
        }
    }
    __syncthreads();
    // P over Y, U0 over the system (both dead now)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int j = wave + 8 * x;
        if (j < 10) {
            int ti, tj;
            tri_tile(j, ti, tj);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sY[(16 * ti + (lane >> 4) * 4 + i) * PC + 16 * tj + (lane & 15)] = pt[x][i];
        }
    }
#pragma unroll
    for (int x = 0; x < NUW; ++x) {
        const int j = wave + 8 * x;
        if (j < NU) {
            const int ti = j / (DV / 16), tn = j % (DV / 16);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sT[(16 * ti + (lane >> 4) * 4 + i) * PC + 16 * tn + (lane & 15)] = u0[x][i];
        }
    }
    __syncthreads();

    // ---- the chunk's own output P V; F = e^g I - Khat^T W; U = Khat^T U0
    const float g = sb[GC - 1];
    for (int j = wave; j < NU; j += kChunkThreads / 64) {
        const int ti = j / (DV / 16), tn = j % (DV / 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mm_f32([&](int m, int k) { return sY[(16 * ti + m) * PC + k]; },
                     [&](int k, int n) { return ld(sV + k * PV + 16 * tn + n); }, 0, 16 * (ti + 1),
                     acc);
        const int n = 16 * tn + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * ti + (lane >> 4) * 4 + i;
            if (m < nvalid) p.out[(row0 + m) * DV + n] = acc[i];
        }
    }
    if (ci + 1 < p.N) {  // the last chunk's transition and state are never read
        float* F = p.fmat + ((size_t)bh * p.N + ci) * DK * DK;
        constexpr int NF = (DK / 16) * (DK / 16);
        for (int j = wave; j < NF; j += kChunkThreads / 64) {
            const int ti = j / (DK / 16), tn = j % (DK / 16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mm_f32([&](int m, int k) { return ld(sK + k * PK + 16 * ti + m) * __expf(g - sb[k]); },
                         [&](int k, int n) { return sW[k * PK + 16 * tn + n]; }, 0, GC, acc);
            const int n = 16 * tn + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * ti + (lane >> 4) * 4 + i;
                F[frag_index(m, n, DK)] = (m == n ? __expf(g) : 0.f) - acc[i];
            }
        }
        float* U = p.ust + ((size_t)bh * p.N + ci) * DK * DV;
        constexpr int NS = (DK / 16) * (DV / 16);
        for (int j = wave; j < NS; j += kChunkThreads / 64) {
            const int ti = j / (DV / 16), tn = j % (DV / 16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mm_f32([&](int m, int k) { return ld(sK + k * PK + 16 * ti + m) * __expf(g - sb[k]); },
                         [&](int k, int n) { return sT[k * PC + 16 * tn + n]; }, 0, GC, acc);
            const int n = 16 * tn + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * ti + (lane >> 4) * 4 + i;
                U[(size_t)m * DV + n] = acc[i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// level walk over chunks

template <int DK>
__global__ __launch_bounds__(kLevelThreads) void k_gdn_levels(GdnParams p) {
    extern __shared__ __align__(16) float sx[];       // [nlev][DK][kXPitch] level states
    float* slam = sx + (size_t)p.nlev * DK * kXPitch;  // [64][nlev] lambda of coarse levels
    constexpr int RT = DK / 64;  // row tiles of the state per wave (4 waves)
    const int ncb = p.dv / kLevelCols;
    const int blk = xcd_local_block(blockIdx.x, gridDim.x);
    const int bh = blk / ncb, cb = blk - bh * ncb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int col0 = cb * kLevelCols;
    const int N = p.N;
    constexpr int c = 6;  // log2 of the chunk size: chunk level p+1 is mask level c+p+1

    for (int e = tid; e < p.nlev * DK * kXPitch; e += kLevelThreads) sx[e] = 0.f;

    for (int ci = 0; ci < N; ++ci) {
        const int t0 = ci * GC;
        const int nvalid = min(GC, p.T - t0);
        const size_t row0 = (size_t)bh * p.T + t0;
        __syncthreads();  // the previous chunk's state writes and lambda reads are done
        for (int e = tid; e < GC * p.nlev; e += kLevelThreads) {
            const int r = e / p.nlev, l = e - r * p.nlev;
            const int lev = c + 1 + l;
            slam[e] = (r < nvalid && lev < p.L) ? p.lam[(row0 + r) * p.L + lev] : 0.f;
        }
        __syncthreads();

        // read-out of the live levels (bits of ci) for tokens 16*wave .. +15
        if (ci > 0) {
            const float4* qp = reinterpret_cast<const float4*>(p.qp + ((size_t)bh * N + ci) * GC * DK);
            float4 qf[DK / 16];
#pragma unroll
            for (int g = 0; g < DK / 16; ++g) qf[g] = qp[((size_t)wave * (DK / 16) + g) * 64 + lane];
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            for (unsigned bits = (unsigned)ci; bits; bits &= bits - 1) {
                const int l = __builtin_ctz(bits);  // chunk level l+1
                const float* X = sx + (size_t)l * DK * kXPitch;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < DK / 16; ++g) {
                    acc = mma(qf[g].x, X[(16 * g + 0 + q4) * kXPitch + r16], acc);
                    acc = mma(qf[g].y, X[(16 * g + 4 + q4) * kXPitch + r16], acc);
                    acc = mma(qf[g].z, X[(16 * g + 8 + q4) * kXPitch + r16], acc);
                    acc = mma(qf[g].w, X[(16 * g + 12 + q4) * kXPitch + r16], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] += slam[(16 * wave + q4 * 4 + i) * p.nlev + l] * acc[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * wave + q4 * 4 + i;
                if (m < nvalid) {
                    float* dst = p.out + (row0 + m) * p.dv + col0 + r16;
                    *dst += o[i];
                }
            }
        }
        if (ci + 1 >= N) break;

        // merge levels 1..j (bits 0..j-1 of ci) into level j+1, then carry every
        // live level through F: X_{j+1} = F (X_1 + ... + X_j) + U, X_l = F X_l above
        const int jm = __builtin_ctz((unsigned)(ci + 1));
        float* Xm = sx + (size_t)jm * DK * kXPitch;
        for (int e = tid; e < DK * kLevelCols; e += kLevelThreads) {
            const int r = e / kLevelCols, cc = e - r * kLevelCols;
            float s = 0.f;
            for (int l = 0; l < jm; ++l) s += sx[((size_t)l * DK + r) * kXPitch + cc];
            Xm[r * kXPitch + cc] = s;
        }
        const float4* fp = reinterpret_cast<const float4*>(p.fmat + ((size_t)bh * N + ci) * DK * DK);
        float4 ff[RT][DK / 16];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int g = 0; g < DK / 16; ++g)
                ff[t][g] = fp[((size_t)(wave * RT + t) * (DK / 16) + g) * 64 + lane];
        const float* U = p.ust + ((size_t)bh * N + ci) * DK * p.dv;
        __syncthreads();
        for (unsigned bits = ((unsigned)ci >> jm) | 1u; bits; bits &= bits - 1) {
            const int l = jm + __builtin_ctz(bits);  // slot of chunk level l+1
            float* X = sx + (size_t)l * DK * kXPitch;
            f32x4 nx[RT];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                nx[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < DK / 16; ++g) {
                    nx[t] = mma(ff[t][g].x, X[(16 * g + 0 + q4) * kXPitch + r16], nx[t]);
                    nx[t] = mma(ff[t][g].y, X[(16 * g + 4 + q4) * kXPitch + r16], nx[t]);
                    nx[t] = mma(ff[t][g].z, X[(16 * g + 8 + q4) * kXPitch + r16], nx[t]);
                    nx[t] = mma(ff[t][g].w, X[(16 * g + 12 + q4) * kXPitch + r16], nx[t]);
                }
                if (l == jm) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 16 * (wave * RT + t) + q4 * 4 + i;
                        nx[t][i] += U[(size_t)m * p.dv + col0 + r16];
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    X[(16 * (wave * RT + t) + q4 * 4 + i) * kXPitch + r16] = nx[t][i];
            __syncthreads();
        }
    }
}

template <typename K>
hipError_t set_smem(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename E, int DK, int DV>
hipError_t launch_chunk(const GdnParams& p, hipStream_t stream) {
    constexpr size_t sm = ChunkSmem<E, DK, DV>::total;
    static_assert(sm <= kGdnLdsMax, "chunk kernel LDS");
    hipError_t e = set_smem(&k_gdn_chunk<E, DK, DV>, sm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gdn_chunk<E, DK, DV>), dim3((unsigned)(p.BH * p.N)), dim3(kChunkThreads),
                       sm, stream, p);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_levels(const GdnParams& p, hipStream_t stream) {
    const size_t sm = gdn_levels_smem(DK, p.nlev);
    hipError_t e = set_smem(&k_gdn_levels<DK>, sm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gdn_levels<DK>), dim3((unsigned)(p.BH * (p.dv / kLevelCols))),
                       dim3(kLevelThreads), sm, stream, p);
    return hipGetLastError();
}

template <typename E, int DK>
hipError_t launch_chunk_dv(const GdnParams& p, hipStream_t stream) {
    switch (p.dv) {
        case 16: return launch_chunk<E, DK, 16>(p, stream);
        case 32: return launch_chunk<E, DK, 32>(p, stream);
        case 64: return launch_chunk<E, DK, 64>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t gdn_levels_smem(int dk, int nlev) {
    return sizeof(float) * ((size_t)nlev * dk * kXPitch + (size_t)GC * nlev);
}

hipError_t launch_gdn_fwd(const GdnParams& p, bool bf16, unsigned stages, hipStream_t stream) {
    hipError_t e = hipSuccess;
    if (stages & 1u) {
        if (bf16)
            e = p.dk == 128 ? launch_chunk_dv<bf16_t, 128>(p, stream)
                            : launch_chunk_dv<bf16_t, 64>(p, stream);
        else
            e = p.dk == 128 ? launch_chunk_dv<float, 128>(p, stream)
                            : launch_chunk_dv<float, 64>(p, stream);
        if (e != hipSuccess) return e;
    }
    if ((stages & 2u) && p.N > 1)
        e = p.dk == 128 ? launch_levels<128>(p, stream) : launch_levels<64>(p, stream);
    return e;
}

}  // namespace loglin
