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

// N = (I + A)^-1 in place for the strictly lower 64 x 64 matrix A held in T
// (fp32, row pitch pc; the tiles above the diagonal are zero), by 16 x 16
// blocks: the diagonal blocks by forward substitution (lane c of waves 0..3
// holds column c of block w), then the blocks below them row by row,
// N_ij = -N_ii sum_{k=j..i-1} A_ik N_kj on the fp32 matrix cores (temporaries
// in G, [3][16][20]).  Called by all threads of a block of >= 4 waves.
__device__ __forceinline__ void invert_unit_lower(float* T, int pc, float* G) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (wave < 4 && lane < 16) {
        const int o = 16 * wave, c = lane;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = r == c ? 1.f : 0.f;
#pragma unroll
            for (int u = 0; u < r; ++u) s -= T[(o + r) * pc + o + u] * x[u];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) T[(o + r) * pc + o + c] = x[r];
    }
    __syncthreads();
    for (int bi = 1; bi < 4; ++bi) {
        // G_ij = sum_{k=j..i-1} A_ik N_kj into temp j (waves 0..i-1)
        if (wave < bi) {
            const int bj = wave;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int bk = bj; bk < bi; ++bk)
                acc = mm_f32([&](int m, int k) { return T[(16 * bi + m) * pc + 16 * bk + k]; },
                             [&](int k, int n) { return T[(16 * bk + k) * pc + 16 * bj + n]; }, 0,
                             16, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) G[(bj * 16 + (lane >> 4) * 4 + i) * 20 + (lane & 15)] = acc[i];
        }
        __syncthreads();
        if (wave < bi) {
            const int bj = wave;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mm_f32([&](int m, int k) { return T[(16 * bi + m) * pc + 16 * bi + k]; },
                         [&](int k, int n) { return G[(bj * 16 + k) * 20 + n]; }, 0, 16, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                T[(16 * bi + (lane >> 4) * 4 + i) * pc + 16 * bj + (lane & 15)] = -acc[i];
        }
        __syncthreads();
    }
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

    invert_unit_lower(sT, PC, sG);
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

// ---------------------------------------------------------------------------
// bf16 inputs: the same two stages on the 16 x 16 x 32 bf16 matrix cores.
//
// Products whose results carry from chunk to chunk (W, F and the level states
// of the walk) take each fp32 operand in two bf16 pieces, x = hi + lo with
// hi = bf16(x) and lo = bf16(x - hi), and form A B as Ah Bh + Ah Bl + Al Bh
// (about 16 significant bits; bf16 inputs are exact and need no lo piece).
// The chunk's own block, its state U and the read-out queries take one bf16
// piece (their rounding does not compound); the inverse stays in fp32.
// Operands of the 16x16x32 MFMA are read 16 bytes per lane: A as rows m with
// k contiguous, B as rows n with k contiguous (B transposed); every array has
// a row pitch of its length plus 8 elements.
//
// Workspace (per bh, chunk), in the byte sizes of the fp32 stages:
//   F   hi then lo, [DK*DK] bf16 each, in the A-operand order of the walk
//   Qp  [64*DK] bf16, q' in the same order
//   U   fp32 in the walk's accumulator order: [DV/16][DK/16][64 lanes][4]

constexpr int P64 = GC + 8;         // pitch of rows of 64 elements
constexpr int kMaxWalkLevels = kGdnMaxWalkLevelsBf;  // chunk levels the bf16 walk holds

__device__ __forceinline__ f32x4 mm_bf(const bf16_t* A, int lda, const bf16_t* Bt, int ldb, int kb,
                                       int ke, f32x4 acc) {
    const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    for (int k = kb; k < ke; k += 32) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + k + 8 * q);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * ldb + k + 8 * q);
        acc = mma(a, b, acc);
    }
    return acc;
}

__device__ __forceinline__ bf16_t bf_of(float x) { return __builtin_bit_cast(bf16_t, (__bf16)x); }
__device__ __forceinline__ void split_bf(float x, bf16_t& hi, bf16_t& lo) {
    const __bf16 h = (__bf16)x;
    hi = __builtin_bit_cast(bf16_t, h);
    lo = bf_of(x - (float)h);
}
// four bf16 in one 8-byte store
__device__ __forceinline__ void st4(bf16_t* dst, bf16_t a, bf16_t b, bf16_t c, bf16_t d) {
    const uint2 v = make_uint2((uint32_t)a | ((uint32_t)b << 16), (uint32_t)c | ((uint32_t)d << 16));
    *reinterpret_cast<uint2*>(dst) = v;
}
// index of (row m, col k) of a [rows][D] matrix in the A-operand order of the
// 16x16x32 MFMA: tile of 16 rows, 32-wide k-step, lane, element
__device__ __forceinline__ size_t frag16(int m, int k, int D) {
    const int lane = (m & 15) + 16 * ((k & 31) >> 3);
    return ((((size_t)(m >> 4) * (D / 32) + (k >> 5)) * 64 + lane) << 3) + (k & 7);
}
// contraction end of a lower-triangular row tile ti, rounded up to the k-step
__device__ __forceinline__ int tri_end(int ti) { return min(GC, (16 * (ti + 1) + 31) & ~31); }

template <int DK, int DV>
struct ChunkBfSmem {
    static constexpr int PK = DK + 8, PC = GC + 4;
    static constexpr size_t q_off = 0;                                  // Q  [64][PK]
    static constexpr size_t k_off = q_off + 2 * GC * PK;                 // K  [64][PK]
    static constexpr size_t kt_off = k_off + 2 * GC * PK;                // K^T [DK][P64]
    static constexpr size_t vt_off = kt_off + 2 * DK * P64;              // V^T [DV][P64]
    static constexpr size_t yh_off = vt_off + 2 * DV * P64;              // Y (then P) [64][P64]
    static constexpr size_t b_off = yh_off + 2 * GC * P64;               // b, beta, a [64] each
    static constexpr size_t lam_off = b_off + 4 * 3 * GC;                // [64][8]
    static constexpr size_t g_off = lam_off + 4 * GC * 8;                // inverse temps [3][16][20]
    static constexpr size_t u_off = g_off + 4 * 3 * 16 * 20;             // union region
    // phase 1: the system (fp32) and Tb, Tb diag(e^b) in two pieces, Tb^T
    static constexpr size_t t_size = 4 * GC * PC;
    static constexpr size_t tb_size = 2 * GC * P64;
    static constexpr size_t phase1 = t_size + 5 * tb_size;
    // phase 2: W^T, (diag(e^(g-b)) W)^T in two pieces, (diag(e^(g-b)) U0)^T in two
    static constexpr size_t wt_size = 2 * DK * P64;
    static constexpr size_t ut_size = 2 * DV * P64;
    static constexpr size_t phase2 = 3 * wt_size + 2 * ut_size;
    static constexpr size_t total = u_off + (phase1 > phase2 ? phase1 : phase2);
};

template <int DK, int DV>
__global__ __launch_bounds__(kChunkThreads) void k_gdn_chunk_bf(GdnParams p) {
    using S = ChunkBfSmem<DK, DV>;
    constexpr int PK = S::PK, PC = S::PC;
    constexpr int NWV = kChunkThreads / 64;
    extern __shared__ __align__(16) char smem[];
    bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + S::q_off);
    bf16_t* sK = reinterpret_cast<bf16_t*>(smem + S::k_off);
    bf16_t* sKt = reinterpret_cast<bf16_t*>(smem + S::kt_off);
    bf16_t* sVt = reinterpret_cast<bf16_t*>(smem + S::vt_off);
    bf16_t* sYh = reinterpret_cast<bf16_t*>(smem + S::yh_off);
    float* sb = reinterpret_cast<float*>(smem + S::b_off);
    float* sbeta = sb + GC;
    float* sa = sbeta + GC;
    float* slam = reinterpret_cast<float*>(smem + S::lam_off);
    float* sG = reinterpret_cast<float*>(smem + S::g_off);
    char* un = smem + S::u_off;
    float* sT = reinterpret_cast<float*>(un);
    bf16_t* Tbh = reinterpret_cast<bf16_t*>(un + S::t_size);
    bf16_t* Tbl = Tbh + GC * P64;
    bf16_t* Tph = Tbl + GC * P64;
    bf16_t* Tpl = Tph + GC * P64;
    bf16_t* TbT = Tpl + GC * P64;
    bf16_t* WTh = reinterpret_cast<bf16_t*>(un);
    bf16_t* WpTh = WTh + DK * P64;
    bf16_t* WpTl = WpTh + DK * P64;
    bf16_t* U0h = WpTl + DK * P64;
    bf16_t* U0l = U0h + DV * P64;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, r16 = lane & 15, q4 = lane >> 4;
    const int total = p.BH * p.N;

    // A block works through chunks blockIdx.x, + gridDim.x, ...; the next
    // chunk's inputs are loaded into registers while the current one is worked.
    constexpr int NQK = GC * DK / 8 / kChunkThreads;                      // 16-byte pieces of q (k)
    constexpr int NVV = (GC * DV / 8 + kChunkThreads - 1) / kChunkThreads;  // of v
    static_assert(GC * 8 == kChunkThreads, "one lambda entry per thread");
    struct In {
        uint4 q[NQK], k[NQK], v[NVV];
        float a, beta, lam;
        int nv;  // valid tokens of the chunk (rows past it are zeroed when staged)
    };
    auto fetch = [&](int cb, In& R) __attribute__((always_inline)) {
        const int fbh = cb / p.N, fci = cb - fbh * p.N;
        const int nv = min(GC, p.T - fci * GC);
        const size_t r0 = (size_t)fbh * p.T + (size_t)fci * GC;
        const bf16_t* q = static_cast<const bf16_t*>(p.q) + r0 * DK;
        const bf16_t* k = static_cast<const bf16_t*>(p.k) + r0 * DK;
        const bf16_t* v = static_cast<const bf16_t*>(p.v) + r0 * DV;
        // lane l of a wave takes token row l: the transposed copies below then
        // write 64 consecutive tokens per store.  Every load is issued, rows
        // past T reading the chunk's last valid row (zeroed when staged): a
        // load under a branch leaves the compiler unsure how many memory
        // operations follow it, and it then waits for all of them (the
        // previous chunk's stores) before this chunk's data are used.  The
        // loaded registers are not touched here, so the loads stay in flight.
        R.nv = nv;
#pragma unroll
        for (int u = 0; u < NQK; ++u) {
            const int e = tid + u * kChunkThreads;
            const int r = min(e % GC, nv - 1), c8 = (e / GC) * 8;
            R.q[u] = *reinterpret_cast<const uint4*>(q + (size_t)r * DK + c8);
            R.k[u] = *reinterpret_cast<const uint4*>(k + (size_t)r * DK + c8);
        }
#pragma unroll
        for (int u = 0; u < NVV; ++u) {
            const int e = min(tid + u * kChunkThreads, GC * DV / 8 - 1);
            const int r = min(e % GC, nv - 1), c8 = (e / GC) * 8;
            R.v[u] = *reinterpret_cast<const uint4*>(v + (size_t)r * DV + c8);
        }
        const int tc = min(tid, nv - 1);
        R.a = p.a[r0 + tc];
        R.beta = p.beta[r0 + tc];
        const int r = min(tid >> 3, nv - 1), l = min(tid & 7, min(p.L, 7) - 1);
        R.lam = p.lam[(r0 + r) * p.L + l];
    };
    // q, k rows and k^T; v^T; a, beta, lambda 0..6 to LDS; the tiles above the
    // diagonal of Y and of the system zeroed
    auto stage = [&](const In& R) __attribute__((always_inline)) {
        const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < NQK; ++u) {
            const int e = tid + u * kChunkThreads;
            const int r = e % GC, c8 = (e / GC) * 8;
            const uint4 xq = r < R.nv ? R.q[u] : z, xk = r < R.nv ? R.k[u] : z;
            *reinterpret_cast<uint4*>(sQ + r * PK + c8) = xq;
            *reinterpret_cast<uint4*>(sK + r * PK + c8) = xk;
            const bf16_t* kk = reinterpret_cast<const bf16_t*>(&xk);
#pragma unroll
            for (int i = 0; i < 8; ++i) sKt[(c8 + i) * P64 + r] = kk[i];
        }
#pragma unroll
        for (int u = 0; u < NVV; ++u) {
            const int e = tid + u * kChunkThreads;
            if (e < GC * DV / 8) {
                const int r = e % GC, c8 = (e / GC) * 8;
                const uint4 xv = r < R.nv ? R.v[u] : z;
                const bf16_t* vv = reinterpret_cast<const bf16_t*>(&xv);
#pragma unroll
                for (int i = 0; i < 8; ++i) sVt[(c8 + i) * P64 + r] = vv[i];
            }
        }
        if (tid < GC) {
            sa[tid] = tid < R.nv ? R.a : 0.f;
            sbeta[tid] = tid < R.nv ? R.beta : 0.f;
        }
        slam[tid] = ((tid >> 3) < R.nv && (tid & 7) < min(p.L, 7)) ? R.lam : 0.f;
        for (int e = tid; e < GC * GC; e += kChunkThreads) {
            const int r = e / GC, c = e - r * GC;
            if ((c >> 4) > (r >> 4)) {
                sYh[r * P64 + c] = 0;
                sT[r * PC + c] = 0.f;
            }
        }
    };

    In nxt;
    if ((int)blockIdx.x < total) fetch(blockIdx.x, nxt);
    for (int blk = blockIdx.x; blk < total; blk += gridDim.x) {
    const int bh = blk / p.N;
    const int ci = blk - bh * p.N;
    const int t0 = ci * GC;
    const int nvalid = min(GC, p.T - t0);
    const size_t row0 = (size_t)bh * p.T + t0;
    __syncthreads();  // every wave is done with the previous chunk's LDS
    stage(nxt);
    if (blk + (int)gridDim.x < total) fetch(blk + gridDim.x, nxt);
    __syncthreads();
    if (wave == 0) wave_cumsum(sa, sb, GC);
    __syncthreads();

    // ---- Q K^T -> Y (one bf16 piece); K K^T -> the system (fp32)
    for (int j = wave; j < 20; j += NWV) {
        const bool isq = j < 10;
        int ti, tj;
        tri_tile(isq ? j : j - 10, ti, tj);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mm_bf((isq ? sQ : sK) + 16 * ti * PK, PK, sK + 16 * tj * PK, PK, 0, DK, acc);
        const int n = 16 * tj + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * ti + q4 * 4 + i;
            const float dec = m >= n ? __expf(sb[m] - sb[n]) : 0.f;
            if (isq)
                sYh[m * P64 + n] = bf_of(m >= n ? acc[i] * dec : 0.f);
            else
                sT[m * PC + n] = m > n ? sbeta[m] * acc[i] * dec : 0.f;
        }
    }
    __syncthreads();
    invert_unit_lower(sT, PC, sG);
    // Tb = N diag(beta) and Tb diag(e^b), each in two pieces; Tb^T (one piece)
    for (int e = tid; e < GC * GC; e += kChunkThreads) {
        const int r = e / GC, c = e - r * GC;
        const float tb = sT[r * PC + c] * sbeta[c];
        bf16_t h, l;
        split_bf(tb, h, l);
        Tbh[r * P64 + c] = h;
        Tbl[r * P64 + c] = l;
        TbT[c * P64 + r] = h;
        split_bf(tb * __expf(sb[c]), h, l);
        Tph[r * P64 + c] = h;
        Tpl[r * P64 + c] = l;
    }
    __syncthreads();

    // ---- W = Tb diag(e^b) K, U0 = Tb V, P = (Y Tb) (.) Lambda -> registers
    constexpr int NW = 4 * (DK / 16);
    constexpr int NWW = NW / NWV;  // W tiles per wave
    f32x4 w[NWW];
#pragma unroll
    for (int x = 0; x < NWW; ++x) {
        const int j = wave + NWV * x;
        const int ti = j / (DK / 16), tn = j % (DK / 16);
        const int ke = tri_end(ti);
        w[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        w[x] = mm_bf(Tph + 16 * ti * P64, P64, sKt + 16 * tn * P64, P64, 0, ke, w[x]);
        w[x] = mm_bf(Tpl + 16 * ti * P64, P64, sKt + 16 * tn * P64, P64, 0, ke, w[x]);
    }
    constexpr int NU = 4 * (DV / 16);
    constexpr int NUW = (NU + NWV - 1) / NWV;
    f32x4 u0[NUW];
#pragma unroll
    for (int x = 0; x < NUW; ++x) {
        u0[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int j = wave + NWV * x;
        if (j < NU) {
            const int ti = j / (DV / 16), tn = j % (DV / 16);
            const int ke = tri_end(ti);
            u0[x] = mm_bf(Tbh + 16 * ti * P64, P64, sVt + 16 * tn * P64, P64, 0, ke, u0[x]);
            u0[x] = mm_bf(Tbl + 16 * ti * P64, P64, sVt + 16 * tn * P64, P64, 0, ke, u0[x]);
        }
    }
    f32x4 pt[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        pt[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int j = wave + NWV * x;
        if (j < 10) {
            int ti, tj;
            tri_tile(j, ti, tj);
            pt[x] = mm_bf(sYh + 16 * ti * P64, P64, TbT + 16 * tj * P64, P64, (16 * tj) & ~31,
                          tri_end(ti), pt[x]);
            const int n = 16 * tj + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * ti + q4 * 4 + i;
                pt[x][i] = m >= n ? pt[x][i] * slam[m * 8 + fenwick_level((uint32_t)m, (uint32_t)n)] : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- W^T, (e^(g-b) W)^T in two pieces, (e^(g-b) U0)^T in two pieces
    const float g = sb[GC - 1];
#pragma unroll
    for (int x = 0; x < NWW; ++x) {
        const int j = wave + NWV * x;
        const int ti = j / (DK / 16), tn = j % (DK / 16);
        const int s0 = 16 * ti + q4 * 4, d = 16 * tn + r16;
        bf16_t hh[4], ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hh[i] = bf_of(w[x][i]);
            split_bf(w[x][i] * __expf(g - sb[s0 + i]), ph[i], pl[i]);
        }
        st4(WTh + d * P64 + s0, hh[0], hh[1], hh[2], hh[3]);
        st4(WpTh + d * P64 + s0, ph[0], ph[1], ph[2], ph[3]);
        st4(WpTl + d * P64 + s0, pl[0], pl[1], pl[2], pl[3]);
    }
#pragma unroll
    for (int x = 0; x < NUW; ++x) {
        const int j = wave + NWV * x;
        if (j < NU) {
            const int ti = j / (DV / 16), tn = j % (DV / 16);
            const int s0 = 16 * ti + q4 * 4, c = 16 * tn + r16;
            bf16_t ph[4], pl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) split_bf(u0[x][i] * __expf(g - sb[s0 + i]), ph[i], pl[i]);
            st4(U0h + c * P64 + s0, ph[0], ph[1], ph[2], ph[3]);
            st4(U0l + c * P64 + s0, pl[0], pl[1], pl[2], pl[3]);
        }
    }
    __syncthreads();

    // ---- q' = e^b Q - Y W (read by the walk from chunk 1 on), F and U (for
    // every chunk but the last)
    // Each of q', F and the chunk output is formed transposed (operands
    // swapped), so that a lane's four results are consecutive in the layout
    // the walk reads and go out as one store.
    // q', F and U are formed and stored for every chunk, also where the walk
    // does not read them (q' of chunk 0, F and U of a sequence's last chunk:
    // their workspace slots exist), so that every chunk issues the same
    // stores and the wait for the next chunk's loads counts them exactly
    {
        bf16_t* Qp = reinterpret_cast<bf16_t*>(p.qp) + ((size_t)bh * p.N + ci) * GC * DK;
#pragma unroll
        for (int x = 0; x < NWW; ++x) {
            const int j = wave + NWV * x;
            const int td = j / 4, tt = j % 4;  // q'^T tile: rows d (16 td..), columns t (16 tt..)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            // Y is lower triangular: token tile tt contracts over s < 16 (tt + 1)
            acc = mm_bf(WTh + 16 * td * P64, P64, sYh + 16 * tt * P64, P64, 0, tri_end(tt), acc);
            const int t = 16 * tt + r16, d0 = 16 * td + q4 * 4;
            const float eb = __expf(sb[t]);
            bf16_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = bf_of(eb * bf16_to_f32(sQ[t * PK + d0 + i]) - acc[i]);
            st4(Qp + frag16(t, d0, DK), h[0], h[1], h[2], h[3]);
        }
    }
    {
        bf16_t* Fh = reinterpret_cast<bf16_t*>(p.fmat) + ((size_t)bh * p.N + ci) * 2 * DK * DK;
        bf16_t* Fl = Fh + DK * DK;
        const float eg = __expf(g);
        constexpr int NF = (DK / 16) * (DK / 16);
        static_assert(NF % NWV == 0, "F tiles per wave");
#pragma unroll 1
        for (int x = 0; x < NF / NWV; ++x) {
            const int j = wave + NWV * x;
            const int tc = j / (DK / 16), tr = j % (DK / 16);  // F^T tile: rows d' (16 tc..), cols d
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mm_bf(WpTh + 16 * tc * P64, P64, sKt + 16 * tr * P64, P64, 0, GC, acc);
            acc = mm_bf(WpTl + 16 * tc * P64, P64, sKt + 16 * tr * P64, P64, 0, GC, acc);
            const int d = 16 * tr + r16, e0 = 16 * tc + q4 * 4;  // F row d, columns e0..e0+3
            bf16_t h[4], l[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) split_bf((d == e0 + i ? eg : 0.f) - acc[i], h[i], l[i]);
            const size_t fi = frag16(d, e0, DK);
            st4(Fh + fi, h[0], h[1], h[2], h[3]);
            st4(Fl + fi, l[0], l[1], l[2], l[3]);
        }
        f32x4* U = reinterpret_cast<f32x4*>(p.ust + ((size_t)bh * p.N + ci) * DK * DV);
        constexpr int NS = (DK / 16) * (DV / 16);
#pragma unroll 1
        for (int x = 0; x < (NS + NWV - 1) / NWV; ++x) {
            const int j = wave + NWV * x;
            if (NS % NWV != 0 && j >= NS) break;
            const int ti = j % (DK / 16), tn = j / (DK / 16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mm_bf(sKt + 16 * ti * P64, P64, U0h + 16 * tn * P64, P64, 0, GC, acc);
            acc = mm_bf(sKt + 16 * ti * P64, P64, U0l + 16 * tn * P64, P64, 0, GC, acc);
            U[((size_t)tn * (DK / 16) + ti) * 64 + lane] = acc;
        }
    }
    __syncthreads();
    // ---- P over Y, then the chunk's own output P V
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int j = wave + NWV * x;
        if (j < 10) {
            int ti, tj;
            tri_tile(j, ti, tj);
#pragma unroll
            for (int i = 0; i < 4; ++i) sYh[(16 * ti + q4 * 4 + i) * P64 + 16 * tj + r16] = bf_of(pt[x][i]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < (NU + NWV - 1) / NWV; ++x) {
        const int j = wave + NWV * x;
        if (NU % NWV != 0 && j >= NU) break;
        const int tt = j / (DV / 16), tc = j % (DV / 16);  // O^T tile: rows c, columns t
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mm_bf(sVt + 16 * tc * P64, P64, sYh + 16 * tt * P64, P64, 0, tri_end(tt), acc);
        const int t = 16 * tt + r16;
        if (t < nvalid)
            *reinterpret_cast<f32x4*>(p.out + (row0 + t) * DV + 16 * tc + q4 * 4) = acc;
    }
    }  // chunks of this block
}

// Level walk for bf16 inputs: one block of 8 waves per (bh, 16 output
// columns).  Each level state is kept transposed (16 columns x DK) in two
// bf16 pieces; wave w < DK/16 carries rows 16w..16w+15 of every state through
// F (three products per step), waves 0..3 read tokens 16w..16w+15 out.  The
// next chunk's F, q', U and chunk output are loaded while this one is worked.
template <int DK>
__global__ __launch_bounds__(kChunkThreads) void k_gdn_levels_bf(GdnParams p) {
    constexpr int XP = DK + 8;
    constexpr int NKS = DK / 32;
    constexpr int SLOT = 2 * kLevelCols * XP;  // bf16 elements of one level (hi, lo)
    extern __shared__ __align__(16) char smem[];
    bf16_t* sx = reinterpret_cast<bf16_t*>(smem);
    float* slam0 = reinterpret_cast<float*>(smem + sizeof(bf16_t) * (size_t)p.nlev * SLOT);
    const int nlev = p.nlev;
    const int ncb = p.dv / kLevelCols;
    const int blk = xcd_local_block(blockIdx.x, gridDim.x);
    const int bh = blk / ncb, cb = blk - bh * ncb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int col0 = cb * kLevelCols;
    const int N = p.N;
    constexpr int c6 = 6;  // chunk level p+1 is mask level 6+p+1
    const bool trans = wave < DK / 16, reads = wave < 4;

    // lambda of the coarse levels of a chunk: at most 64 * 14 values, two per
    // thread, loaded with the chunk's other registers and stored to LDS later.
    // Every load of a chunk is issued without a branch or a select on its
    // value (indices clamped to valid memory): a select that consumed a load
    // would make the compiler wait for it where it is issued, and a load
    // under a branch leaves it unsure how many memory operations follow.
    // Entries outside the chunk or the lambda row are zeroed when stored.
    constexpr int NLR = (GC * kMaxWalkLevels + kChunkThreads - 1) / kChunkThreads;
    auto load_lam = [&](int ci, float (&lr)[NLR]) __attribute__((always_inline)) {
        const size_t r0 = (size_t)bh * p.T + (size_t)ci * GC;
        const int nv = min(GC, p.T - ci * GC);
#pragma unroll
        for (int u = 0; u < NLR; ++u) {
            const int e = min(tid + u * kChunkThreads, GC * nlev - 1);
            const int r = min(e / nlev, nv - 1), l = e - (e / nlev) * nlev;
            const int lev = min(c6 + 1 + l, p.L - 1);
            lr[u] = p.lam[(r0 + r) * p.L + lev];
        }
    };
    auto store_lam = [&](const float (&lr)[NLR], int nv, float* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NLR; ++u) {
            const int e = tid + u * kChunkThreads;
            if (e < GC * nlev) {
                const int r = e / nlev, lev = c6 + 1 + (e - r * nlev);
                dst[e] = (r < nv && lev < p.L) ? lr[u] : 0.f;
            }
        }
    };
    // registers of one chunk: F rows of this wave (two pieces), q' rows, U,
    // chunk output, coarse lambda
    struct Regs {
        bf16x8 fh[NKS], fl[NKS], qf[NKS];
        f32x4 u, o;
        float lam[NLR];
        int nv;  // valid tokens of the chunk
    };
    // the chunk kernel leaves q', F and U for every chunk, so the loads do not
    // depend on the chunk index; each wave loads what its role uses
    auto load = [&](int ci, Regs& R) __attribute__((always_inline)) {
        const size_t slot = (size_t)bh * N + ci;
        if (trans) {
            const bf16x8* fh = reinterpret_cast<const bf16x8*>(p.fmat) + slot * 2 * DK * DK / 8;
            const bf16x8* fl = fh + DK * DK / 8;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                R.fh[ks] = fh[((size_t)wave * NKS + ks) * 64 + lane];
                R.fl[ks] = fl[((size_t)wave * NKS + ks) * 64 + lane];
            }
            R.u = reinterpret_cast<const f32x4*>(p.ust + slot * DK * p.dv)[((size_t)cb * (DK / 16) + wave) * 64 + lane];
        }
        load_lam(ci, R.lam);
        R.nv = min(GC, p.T - ci * GC);
        if (reads) {
            const bf16x8* qp = reinterpret_cast<const bf16x8*>(p.qp) + slot * GC * DK / 8;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) R.qf[ks] = qp[((size_t)wave * NKS + ks) * 64 + lane];
            const size_t r0 = (size_t)bh * p.T + (size_t)ci * GC;
            // rows past the chunk read its last row; the read-out stores rows < nv only
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = min(16 * wave + q4 * 4 + i, R.nv - 1);
                R.o[i] = p.out[(r0 + m) * p.dv + col0 + r16];
            }
        }
    };

    for (int e = tid; e < nlev * SLOT; e += kChunkThreads) sx[e] = 0;
    Regs cur, nxt;
    load(0, nxt);
    store_lam(nxt.lam, nxt.nv, slam0);
    __syncthreads();

    for (int ci = 0; ci < N; ++ci) {
        cur = nxt;
        if (ci + 1 < N) load(ci + 1, nxt);
        float* slam = slam0 + (ci & 1) * GC * nlev;
        const int nvalid = min(GC, p.T - ci * GC);
        const size_t row0 = (size_t)bh * p.T + (size_t)ci * GC;

        // read-out of the live levels (bits of ci)
        if (reads && ci > 0) {
            f32x4 o = cur.o;
            for (unsigned bits = (unsigned)ci; bits; bits &= bits - 1) {
                const int l = __builtin_ctz(bits);
                const bf16_t* Xh = sx + (size_t)l * SLOT + r16 * XP + 8 * q4;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = mma(cur.qf[ks], *reinterpret_cast<const bf16x8*>(Xh + 32 * ks), acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] += slam[(16 * wave + q4 * 4 + i) * nlev + l] * acc[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * wave + q4 * 4 + i;
                if (m < nvalid) p.out[(row0 + m) * p.dv + col0 + r16] = o[i];
            }
        }
        if (ci + 1 >= N) break;

        // merge levels 1..j (slots 0..j-1) into slot j, in fp32 from the pieces
        const int jm = __builtin_ctz((unsigned)(ci + 1));
        for (int e = tid; e < kLevelCols * DK / 4; e += kChunkThreads) {
            const int c = e / (DK / 4), d4 = (e - c * (DK / 4)) * 4;
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
            for (int l = 0; l < jm; ++l) {
                const bf16_t* h = sx + (size_t)l * SLOT + c * XP + d4;
                const bf16_t* lo = h + kLevelCols * XP;
#pragma unroll
                for (int i = 0; i < 4; ++i) s4[i] += bf16_to_f32(h[i]) + bf16_to_f32(lo[i]);
            }
            bf16_t hh[4], ll[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) split_bf(s4[i], hh[i], ll[i]);
            bf16_t* dh = sx + (size_t)jm * SLOT + c * XP + d4;
            st4(dh, hh[0], hh[1], hh[2], hh[3]);
            st4(dh + kLevelCols * XP, ll[0], ll[1], ll[2], ll[3]);
        }
        __syncthreads();

        // carry: slot jm (the merged level, plus U) and the live slots above
        const unsigned tbits = ((unsigned)ci >> jm) | 1u;
        f32x4 nx[kMaxWalkLevels];
        if (trans) {
#pragma unroll
            for (int x = 0; x < kMaxWalkLevels; ++x) {
                nx[x] = f32x4{0.f, 0.f, 0.f, 0.f};
                if ((tbits >> x) & 1u) {
                    const bf16_t* Xh = sx + (size_t)(jm + x) * SLOT + r16 * XP + 8 * q4;
                    const bf16_t* Xl = Xh + kLevelCols * XP;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const bf16x8 bh8 = *reinterpret_cast<const bf16x8*>(Xh + 32 * ks);
                        const bf16x8 bl8 = *reinterpret_cast<const bf16x8*>(Xl + 32 * ks);
                        nx[x] = mma(cur.fh[ks], bh8, nx[x]);
                        nx[x] = mma(cur.fh[ks], bl8, nx[x]);
                        nx[x] = mma(cur.fl[ks], bh8, nx[x]);
                    }
                    if (x == 0) {
                        nx[x][0] += cur.u[0];
                        nx[x][1] += cur.u[1];
                        nx[x][2] += cur.u[2];
                        nx[x][3] += cur.u[3];
                    }
                }
            }
        }
        __syncthreads();
        if (trans) {
#pragma unroll
            for (int x = 0; x < kMaxWalkLevels; ++x) {
                if ((tbits >> x) & 1u) {
                    bf16_t hh[4], ll[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) split_bf(nx[x][i], hh[i], ll[i]);
                    bf16_t* dh = sx + (size_t)(jm + x) * SLOT + r16 * XP + 16 * wave + 4 * q4;
                    st4(dh, hh[0], hh[1], hh[2], hh[3]);
                    st4(dh + kLevelCols * XP, ll[0], ll[1], ll[2], ll[3]);
                }
            }
        }
        store_lam(nxt.lam, nxt.nv, slam0 + ((ci + 1) & 1) * GC * nlev);
        __syncthreads();
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

template <int DK, int DV>
hipError_t launch_chunk_bf(const GdnParams& p, hipStream_t stream) {
    constexpr size_t sm = ChunkBfSmem<DK, DV>::total;
    static_assert(sm <= kGdnLdsMax, "chunk kernel LDS");
    hipError_t e = set_smem(&k_gdn_chunk_bf<DK, DV>, sm);
    if (e != hipSuccess) return e;
    // one resident block per compute unit (the LDS of one block), each working
    // through its share of the chunks
    int dev = 0, ncu = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const long total = (long)p.BH * p.N;
    const unsigned grid = (unsigned)(total < ncu ? total : ncu);
    hipLaunchKernelGGL((k_gdn_chunk_bf<DK, DV>), dim3(grid), dim3(kChunkThreads), sm, stream, p);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_levels_bf(const GdnParams& p, hipStream_t stream) {
    const size_t sm = gdn_levels_smem_bf(DK, p.nlev);
    hipError_t e = set_smem(&k_gdn_levels_bf<DK>, sm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gdn_levels_bf<DK>), dim3((unsigned)(p.BH * (p.dv / kLevelCols))),
                       dim3(kChunkThreads), sm, stream, p);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_chunk_bf_dv(const GdnParams& p, hipStream_t stream) {
    switch (p.dv) {
        case 16: return launch_chunk_bf<DK, 16>(p, stream);
        case 32: return launch_chunk_bf<DK, 32>(p, stream);
        case 64: return launch_chunk_bf<DK, 64>(p, stream);
    }
    return hipErrorInvalidValue;
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

size_t gdn_levels_smem_bf(int dk, int nlev) {
    return sizeof(bf16_t) * (size_t)nlev * 2 * kLevelCols * (dk + 8) + sizeof(float) * 2 * GC * nlev;
}

hipError_t launch_gdn_fwd(const GdnParams& p, bool bf16, unsigned stages, hipStream_t stream) {
    hipError_t e = hipSuccess;
    if (stages & 1u) {
        if (bf16)
            e = p.dk == 128 ? launch_chunk_bf_dv<128>(p, stream) : launch_chunk_bf_dv<64>(p, stream);
        else
            e = p.dk == 128 ? launch_chunk_dv<float, 128>(p, stream)
                            : launch_chunk_dv<float, 64>(p, stream);
        if (e != hipSuccess) return e;
    }
    if ((stages & 2u) && p.N > 1) {
        if (bf16)
            e = p.dk == 128 ? launch_levels_bf<128>(p, stream) : launch_levels_bf<64>(p, stream);
        else
            e = p.dk == 128 ? launch_levels<128>(p, stream) : launch_levels<64>(p, stream);
    }
    return e;
}

}  // namespace loglin
