// Backward pass of the chunked log-linear token mixer on gfx950.
//
// "Log-linear attention, and what a logarithm buys", section 3 trains the
// mixer with chunked matrix products forward and backward, and section 6
// notes that the gradients of the lambda terms are derived by hand.  For the
// loss sum(O (.) dO) with O = (Q K^T (.) M) V and
// M[t, s] = lambda_t^(level(t, s)) e^(A_t - A_s):
//
//   dQ = (dP (.) M) K                     dP = dO V^T
//   dK = (dP (.) M)^T Q,  dV = (Q K^T (.) M)^T dO
//   dlambda_t^(l) = sum over the keys s of level l of dP[t, s] (q_t . k_s) e^(A_t - A_s)
//   da_j = sum_{t >= j} (q_t . dq_t - k_t . dk_t)
//
// (the last line: A_t enters row t of M with a plus sign and column t with a
// minus, and a_j is part of every A_t with t >= j).  The chunk split is the
// forward's: inside a chunk the C x C block is materialised; the coarse
// levels go through states.
//
//   dq / dlambda  for query chunk i, one Fenwick node per set bit p of i,
//                 built by the forward's chunk-state and scan kernels over k
//                 and v swapped (G'(e) = sum e^(A_end(e) - A_s) k_s v_s^T):
//                   dq_t += lambda_t^(l) e^(A_t - A_end(e)) G'(e) dO_t
//                   dlambda_t^(l) = e^(A_t - A_end(e)) q_t^T G'(e) dO_t
//   rstate        the keys of chunk i reach the queries of the block of 2^p
//                 chunks starting at j = ((i >> p) | 1) << p at level
//                 log2 C + p + 1, for each clear bit p of i.  Every chunk
//                 j >= 1 starts exactly one such block (p = lssb(j)), whose
//                 state is
//                   R(j) = sum_{t in block} lambda_t^(log2 C + p + 1) e^(A_t - A_(jC-1)) q_t dO_t^T
//   dk / dv       dk_s += e^(A_(jC-1) - A_s) R(j) v_s,  dv_s += e^(A_(jC-1) - A_s) R(j)^T k_s
//                 plus the chunk's own block
//   da            the suffix sums of q_t . dq_t - k_t . dk_t
//
// Workspace (per (batch*head) bh): the forward's chunk-state and node
// buffers; R at the index j of its block's first chunk ([N][dk][dv]); the two
// dot products per token.  fp32 inputs keep G' and R in fp32 and R^T
// ([N][dv][dk]) beside R.  bf16 inputs keep G' ([N][dk][dv], in the R^T
// region) and R in bf16 only: the operand form the dq and dk/dv kernels stage
// (R^T is then read from R through LDS transpose reads).
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "chunk_stage.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace loglin {

namespace {

// Contraction steps of the backward's matrix-core products: bf16 K = 16
// (4 values a lane, the operand layout of the P hand-off), fp32 K = 4.
template <typename E>
struct BStep {
    static constexpr int KS = 16;
};
template <>
struct BStep<float> {
    static constexpr int KS = 4;
};

// Coarse levels a chunk can have: bit_length(N - 1) for N < 2^31 chunks.
constexpr int kMaxLev = 32;

// Layout of the bf16 natural copies and staged states in LDS: rows padded by
// 16 elements (64 or 128 + 16: consecutive rows start 8 banks apart), and
// within each 16 rows, rows 8..15 store column c at c ^ 8.  Then the 8-byte
// operand reads of 16 rows x 2 lane groups and the transpose reads of
// 8 rows x 4 column quads each cover 64 distinct banks.
constexpr int kPadB = 16;
__device__ __forceinline__ int swz8(int row, int col) { return col ^ (row & 8); }

template <int C>
struct LogC {
    static constexpr int v = C == 16 ? 4 : C == 32 ? 5 : C == 64 ? 6 : 7;
};

// A operand rows x0 .. x0 + 15 of a staged chunk, contraction step ks over
// the head dim: bf16 reads the natural copy (D + kPadB per row), fp32 the
// transposed one (one element a lane).
template <typename E, int C>
__device__ __forceinline__ typename Frag<E, BStep<E>::KS>::type rows_op(const E* nat, const E* tr,
                                                                        int D, int x0, int ks,
                                                                        int m, int g) {
    if constexpr (sizeof(E) == 2) {
        return Frag<E, 16>::load(nat + (x0 + m) * (D + kPadB) + swz8(m, ks * 16 + 4 * g));  // x0 % 16 == 0
    } else {
        return tr[(ks * 4 + g) * (C + kPadT) + x0 + m];
    }
}

// B operand of the lane's own token row (row n = lane % 16), step ks; zero
// unless ok.  `row` must be readable either way: the load is unconditional,
// so that a run of these loads has no branch between them.
template <typename E>
__device__ __forceinline__ typename Frag<E, BStep<E>::KS>::type own_op(const E* row, bool ok, int ks,
                                                                       int g) {
    typedef typename Frag<E, BStep<E>::KS>::type frag_t;
    frag_t x;
    if constexpr (sizeof(E) == 2) {
        x = Frag<E, 16>::load(row + ks * 16 + 4 * g);
    } else {
        x = row[ks * 4 + g];
    }
    return ok ? x : frag_t{};
}

// the C-layout tile (4 values of column m) as the B operand of the next product
template <typename E>
struct Hand {
    typedef typename std::conditional<sizeof(E) == 2, bf16x4, f32x4>::type type;
    __device__ static type pack(float a, float b, float c, float d) {
        if constexpr (sizeof(E) == 2) {
            return pack4(a, b, c, d);
        } else {
            return f32x4{a, b, c, d};
        }
    }
};

// acc += X^T-rows (x0 + m, the transposed copy) times a handed-off tile of
// 16 tokens starting at 16 S
template <typename E, int C>
__device__ __forceinline__ f32x4 mma_hand(const E* tr, int x0, int S, typename Hand<E>::type h,
                                          f32x4 acc, int m, int g) {
    const E* row = tr + (x0 + m) * (C + kPadT) + 16 * S + 4 * g;
    if constexpr (sizeof(E) == 2) {
        return mma(Frag<bf16_t, 16>::load(row), h, acc);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mma(row[j], h[j], acc);
        return acc;
    }
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// A operand of rows c0 .. c0 + 15 of X^T, contraction rows k0 .. k0 + 15 of X,
// for a row-major bf16 LDS matrix X (row stride pitch elements, 8-byte aligned
// rows): lane (m, g) gets X[k0 + 4g + i][c0 + m], i < 4.  One LDS transpose
// read: in each group of 16 lanes, lane j names row k0 + 4g + j / 4 and
// columns c0 + 4 (j % 4) .. + 3, and receives column c0 + j of the four rows.
__device__ __forceinline__ bf16x4 tr_op(const bf16_t* X, int pitch, int k0, int c0, int m, int g) {
    const int r = k0 + 4 * g + (m >> 2);  // k0 % 16 == 0: the swizzle of X applies
    const bf16_t* a = X + r * pitch + swz8(r, c0 + 4 * (m & 3));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)a);
}

// acc += (the chunk's [C][D] matrix X)^T rows x0 .. x0 + 15 times a handed-off
// tile of 16 tokens starting at 16 S: bf16 reads the natural copy
// ([C][D + kPadB]) through transpose reads, fp32 the transposed copy.
template <typename E, int C>
__device__ __forceinline__ f32x4 hand_mma(const E* X, int D, int x0, int S, typename Hand<E>::type h,
                                          f32x4 acc, int m, int g) {
    if constexpr (sizeof(E) == 2) {
        return mma(tr_op(X, D + kPadB, 16 * S, x0, m, g), h, acc);
    } else {
        return mma_hand<E, C>(X, x0, S, h, acc, m, g);
    }
}

__device__ __forceinline__ float sum_groups(float x) {  // over the 4 lanes of one column
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

// One carried state ([rows][cols] bf16 in global memory, rows * cols =
// 8 NS NT) on its way to LDS: load() issues the thread's NS 16-byte loads
// into registers, where they stay in flight while the previous state is
// being used; store() writes them in the swizzled layout (row stride
// cols + kPadB).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

template <int NS, int NT>
struct StateRegs16 {
    u32x4 buf[NS];  // a clang vector type, so that the array stays in registers
    __device__ __forceinline__ void load(const bf16_t* __restrict__ g) {
#pragma unroll
        for (int u = 0; u < NS; ++u) buf[u] = reinterpret_cast<const u32x4*>(g)[threadIdx.x + u * NT];
    }
    __device__ __forceinline__ void store(int cols, bf16_t* dst) const {
        const int sh = __builtin_ctz(cols / 8);
        const int mask = (1 << sh) - 1;
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int idx = threadIdx.x + u * NT;
            const int r = idx >> sh, c = (idx & mask) << 3;
            *reinterpret_cast<u32x4*>(dst + r * (cols + kPadB) + swz8(r, c)) = buf[u];
        }
    }
};

// Rows [r0, r0 + nr) of a row-major bf16 matrix with `cols` columns (a power
// of two >= 8) into LDS, row stride cols + kPadB; NT threads, each round's
// loads (8 per thread) in flight before its LDS writes.
template <int NT>
__device__ __forceinline__ void stage_rows16(const bf16_t* __restrict__ g, int cols, int r0, int nr,
                                             bf16_t* dst) {
    constexpr int RD = 8;
    const int sh = __builtin_ctz(cols / 8);
    const int mask = (1 << sh) - 1;
    const int total = nr << sh;  // 16-byte vectors
    const uint4* src = reinterpret_cast<const uint4*>(g + (size_t)r0 * cols);
    for (int base = 0; base < total; base += RD * NT) {
        uint4 buf[RD];
#pragma unroll
        for (int u = 0; u < RD; ++u) {  // no branch: out-of-range lanes read vector 0
            const int idx = base + threadIdx.x + u * NT;
            buf[u] = src[idx < total ? idx : 0];
        }
#pragma unroll
        for (int u = 0; u < RD; ++u) {
            const int idx = base + threadIdx.x + u * NT;
            if (idx < total)
                *reinterpret_cast<uint4*>(dst + (idx >> sh) * (cols + kPadB) +
                                          swz8(idx >> sh, (idx & mask) << 3)) = buf[u];
        }
    }
}


// --------------------------------------------------------------------------
// dq and dlambda: one block per chunk, one wave per 16 query rows

template <typename E, int C, int DM, int FDK, int FDV>
__global__ __launch_bounds__(C / 16 * 64, C == 128 ? 2 : 3) void k_bwd_dq(BwdParams p) {
    constexpr int NW = C / 16;
    constexpr int NT = NW * kWave;
    constexpr int LOGC = LogC<C>::v;
    constexpr int KS = BStep<E>::KS;
    constexpr int MAXK = DM / KS;
    constexpr int NB = DM / 16;
    constexpr int NLC = C * kMaxLev / NT;  // coarse lambda values staged per thread
    typedef Frag<E, KS> FR;
    typedef typename FR::type frag_t;
    constexpr int KPL = FR::kpl;
    constexpr bool NAT = sizeof(E) == 2;

    extern __shared__ __align__(16) char smem[];
    const int blk = xcd_local_block(blockIdx.x, gridDim.x);
    const int bh = blk / p.N;
    const int i = blk - bh * p.N;
    const int t0 = i * C;
    const int nvalid = min(C, p.T - t0);
    const int dk = FDK ? FDK : p.dk, dv = FDV ? FDV : p.dv;  // FDK, FDV: head dims fixed at compile time
    const int L = p.L, nlev = p.nlev;
    const int nkk = dk / KS, nkv = dv / KS;
    float* a_raw = reinterpret_cast<float*>(smem);
    float* A = a_raw + C;
    float* dlog = A + C;                       // [kMaxLev] A(end of chunk i-1) - A(node) per set bit
    float* lamco = dlog + kMaxLev;             // [C][nlev] lambda of the coarse levels
    // the chunk's K and V: bf16 natural ([C][d + kPadB]), fp32 transposed
    // ([d][C + kPadT]); then (bf16) one carried state, p.st_elems elements
    E* Kc = reinterpret_cast<E*>(lamco + C * nlev);
    E* Vc = Kc + (NAT ? C * (dk + kPadB) : dk * (C + kPadT));
    E* Gs = Vc + (NAT ? C * (dv + kPadB) : dv * (C + kPadT));
    const size_t row0 = (size_t)bh * p.T + t0;

    const int lane = threadIdx.x & (kWave - 1);
    const int R = threadIdx.x / kWave;
    const int m = lane & 15, g = lane >> 4;
    const int r = 16 * R + m;
    const bool rvalid = r < nvalid;
    const size_t trow = row0 + r;
    const size_t lrow0 = row0 + (rvalid ? r : 0);  // the row the loads read (row t0 past T)

    // Every global load of the prologue is issued before the first LDS
    // write, without branches, so that they are all in flight together:
    // the lane's own dO and q fragments and lambda, the chunk's a, K and V,
    // and the scalars of the coarse levels.
    const E* qrow = static_cast<const E*>(p.q) + lrow0 * dk;
    const E* orow = static_cast<const E*>(p.dout) + lrow0 * dv;
    frag_t df[MAXK], qf[MAXK];
#pragma unroll
    for (int ks = 0; ks < MAXK; ++ks) {
        df[ks] = ks < nkv ? own_op<E>(orow, rvalid, ks, g) : frag_t{};
        qf[ks] = ks < nkk ? own_op<E>(qrow, rvalid, ks, g) : frag_t{};
    }
    const float* lrow = p.lam + lrow0 * L;
    float lamr[LOGC + 1];
#pragma unroll
    for (int l = 0; l <= LOGC; ++l) {
        const float x = lrow[min(l, L - 1)];
        lamr[l] = (rvalid && l < L) ? x : 0.f;
    }
    const float av = p.a[row0 + min((int)threadIdx.x, nvalid - 1)];
    float lco[NLC];
#pragma unroll
    for (int u = 0; u < NLC; ++u) {
        const int idx = threadIdx.x + u * NT;
        const int rr = nlev > 0 ? idx / nlev : 0, pb = idx - rr * nlev;
        const size_t row = row0 + min(rr, nvalid - 1);
        lco[u] = p.lam[row * L + min(LOGC + 1 + pb, L - 1)];
    }
    float dl0 = 0.f;
    if (threadIdx.x < nlev) {  // at most one load per thread
        const int pb = threadIdx.x;
        const bool set = (i >> pb) & 1;
        const int node = set ? ((i >> pb) << pb) - 1 : 0;
        const double* cum = p.cum + (size_t)bh * p.N;
        const double ce = cum[set ? i - 1 : 0];  // set implies i >= 1
        dl0 = set ? (float)(ce - cum[node]) : 0.f;
    }
    const E* kg = static_cast<const E*>(p.k) + row0 * dk;
    const E* vg = static_cast<const E*>(p.v) + row0 * dv;
    ChunkRows<E, C, DM, NT, kPadB, true> kr, vr;
    kr.load(kg, dk, nvalid);
    vr.load(vg, dv, nvalid);
    // the first coarse node (lowest set bit of i) as well: its loads stay in
    // flight through the staging and the chunk's own block
    constexpr bool PF = NAT && FDK > 0 && FDV > 0;
    constexpr int NS = PF ? FDK * FDV / (8 * NT) : 1;
    auto node_idx = [&](int pb) __attribute__((always_inline)) {
        return ((size_t)bh * p.N + ((i >> pb) << pb) - 1) * dk * dv;
    };
    StateRegs16<NS, NT> st;
    if constexpr (PF) {
        if (i) st.load(p.gnode16 + node_idx(__builtin_ctz((unsigned)i)));
    }

    if (threadIdx.x < C) a_raw[threadIdx.x] = (int)threadIdx.x < nvalid ? av : 0.f;
    if (threadIdx.x < nlev) dlog[threadIdx.x] = dl0;
#pragma unroll
    for (int u = 0; u < NLC; ++u) {
        const int idx = threadIdx.x + u * NT;
        if (idx < C * nlev) lamco[idx] = lco[u];
    }
    kr.store(dk, NAT ? Kc : nullptr, NAT ? nullptr : Kc, nullptr);
    vr.store(dv, NAT ? Vc : nullptr, NAT ? nullptr : Vc, nullptr);
    __syncthreads();
    if (threadIdx.x < kWave) wave_cumsum(a_raw, A, C);
    __syncthreads();
    const float Ar = A[r];

    // q in the C layout of the dq tiles (column 16 cb + 4 g + j of row r):
    // for bf16 exactly the elements of the lane's own q fragments
    float qv[NB][4];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (NAT) {
                qv[cb][j] = 16 * cb < dk ? (float)qf[cb][j] : 0.f;
            } else {
                const float x = qrow[16 * cb < dk ? 16 * cb + 4 * g + j : 0];
                qv[cb][j] = (rvalid && 16 * cb < dk) ? x : 0.f;
            }
        }
    }

    // The chunk's own block, one tile of 16 keys S <= R at a time: dS = dO V^T
    // and Q K^T, weighted into Z = dS (.) M and handed straight to the dq
    // product K^T Z^T.  A runtime loop, so that the accumulators are updated
    // in place rather than merged across branches.
    float dl[LOGC + 1];
#pragma unroll
    for (int l = 0; l <= LOGC; ++l) dl[l] = 0.f;
    f32x4 acc[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int S = 0; S <= R; ++S) {
        f32x4 ds = {0.f, 0.f, 0.f, 0.f}, sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < MAXK; ++ks)
            if (ks < nkv) ds = mma(rows_op<E, C>(Vc, Vc, dv, 16 * S, ks, m, g), df[ks], ds);
#pragma unroll
        for (int ks = 0; ks < MAXK; ++ks)
            if (ks < nkk) sc = mma(rows_op<E, C>(Kc, Kc, dk, 16 * S, ks, m, g), qf[ks], sc);
        float w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int s = 16 * S + 4 * g + q;
            const int lev = fenwick_level(r, s);
            const float dec = s <= r ? __expf(Ar - A[s]) : 0.f;
            w[q] = ds[q] * pick_level<LOGC>(lamr, lev) * dec;
            const float gq = ds[q] * sc[q] * dec;
#pragma unroll
            for (int l = 0; l <= LOGC; ++l) dl[l] += lev == l ? gq : 0.f;
        }
        const typename Hand<E>::type Zs = Hand<E>::pack(w[0], w[1], w[2], w[3]);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
            if (16 * cb < dk) acc[cb] = hand_mma<E, C>(Kc, dk, 16 * cb, S, Zs, acc[cb], m, g);
    }

    // one term per coarse level: the set bits of i, lowest first.  With the
    // head dims fixed at compile time (PF) the whole node is staged at once
    // and the next node's loads are issued before the current one is used;
    // otherwise the node is staged in rounds of srows of its dk rows.
    float* glrow = p.glam + trow * L;
    unsigned bits = (unsigned)i;
    while (bits) {
        const int pb = __builtin_ctz(bits);
        bits &= bits - 1;
        const int lev = LOGC + pb + 1;
        const float e = rvalid ? __expf(Ar + dlog[pb]) : 0.f;
        const float lw = e * lamco[r * nlev + pb];
        float dot = 0.f;
        if constexpr (PF) {
            const int pitch = dv + kPadB;
            __syncthreads();  // the previous node's reads are done
            st.store(dv, Gs);
            __syncthreads();
            if (bits) st.load(p.gnode16 + node_idx(__builtin_ctz(bits)));
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if (16 * cb < dk) {
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
                    const E* grow = Gs + (16 * cb + m) * pitch;
#pragma unroll
                    for (int ks = 0; ks < MAXK; ++ks)
                        if (ks < nkv) y = mma(Frag<bf16_t, 16>::load(grow + swz8(m, ks * 16 + 4 * g)), df[ks], y);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[cb][j] += lw * y[j];
                        dot += qv[cb][j] * y[j];
                    }
                }
            }
        } else if constexpr (NAT) {
            const int pitch = dv + kPadB;
            const int srows = min(dk, (p.st_elems / pitch) & ~15);
            for (int r0 = 0; r0 < dk; r0 += srows) {
                __syncthreads();  // the previous round's reads are done
                stage_rows16<NT>(p.gnode16 + node_idx(pb), dv, r0, min(srows, dk - r0), Gs);
                __syncthreads();
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) {
                    if (16 * cb < dk && 16 * cb >= r0 && 16 * cb < r0 + srows) {
                        f32x4 y = {0.f, 0.f, 0.f, 0.f};
                        const E* grow = Gs + (16 * cb - r0 + m) * pitch;  // r0 % 16 == 0
#pragma unroll
                        for (int ks = 0; ks < MAXK; ++ks)
                            if (ks < nkv)
                                y = mma(Frag<bf16_t, 16>::load(grow + swz8(m, ks * 16 + 4 * g)), df[ks], y);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            acc[cb][j] += lw * y[j];
                            dot += qv[cb][j] * y[j];
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if (16 * cb < dk) {
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
                    const float* grow = p.gnode + node_idx(pb) + (size_t)(16 * cb + m) * dv + g * KPL;
#pragma unroll
                    for (int ks = 0; ks < MAXK; ++ks)
                        if (ks < nkv) y = mma(FR::from_f32(grow + ks * KS), df[ks], y);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[cb][j] += lw * y[j];
                        dot += qv[cb][j] * y[j];
                    }
                }
            }
        }
        dot = sum_groups(dot) * e;
        if (rvalid && g == 0) glrow[lev] = dot;
    }

    float da1 = 0.f;
    float* dqrow = p.gq + trow * dk;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        if (16 * cb < dk) {
#pragma unroll
            for (int j = 0; j < 4; ++j) da1 += acc[cb][j] * qv[cb][j];
            if (rvalid)
                *reinterpret_cast<float4*>(dqrow + 16 * cb + 4 * g) =
                    make_float4(acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]);
        }
    }
    da1 = sum_groups(da1);
#pragma unroll
    for (int l = 0; l <= LOGC; ++l) dl[l] = sum_groups(dl[l]);
    if (rvalid && g == 0) {
        p.dA1[trow] = da1;
#pragma unroll
        for (int l = 0; l <= LOGC; ++l)
            if (l < L) glrow[l] = dl[l];
        for (int l = LOGC + 1; l < L; ++l) {
            const int pb = l - LOGC - 1;
            if (pb >= 31 || !((i >> pb) & 1)) glrow[l] = 0.f;  // a level this row does not reach
        }
    }
}

// --------------------------------------------------------------------------
// R(j): the lambda-weighted state of the block of chunks that starts at
// chunk j, for the keys of its left sibling.  Blocks are taken largest first.
// The loads of chunk c + 1 are issued before the products of chunk c.

template <typename E, int C, int DM, int FDK, int FDV>
__global__ __launch_bounds__(256, 2) void k_bwd_rstate(BwdParams p) {
    constexpr int LOGC = LogC<C>::v;
    // head dims fixed at compile time (FDK, FDV > 0) size the registers to
    // them, which leaves room for two chunks in flight (DEPTH 2)
    constexpr int QD = FDK ? FDK : DM, OD = FDV ? FDV : DM;
    constexpr int MAXT = ((QD / 16) * (OD / 16) + 3) / 4;  // tiles of 16 x 16 per wave, 4 waves
    constexpr int NVIN = (C * QD + C * OD) * (int)sizeof(E) / 16 / 256;  // 16-byte loads per thread and chunk
    constexpr int DEPTH = (FDK && FDV && NVIN <= 8) ? 2 : 1;
    extern __shared__ __align__(16) char smem[];
    int x = blockIdx.x, lev = -1, j = 0, bh = 0;
    for (int pp = p.nlev - 1; pp >= 0; --pp) {
        const int first = 1 << pp;
        if (first >= p.N) continue;
        const int cnt = (p.N - 1 - first) / (2 << pp) + 1;
        if (x < cnt * p.BH) {
            bh = x % p.BH;
            j = (x / p.BH) * (2 << pp) + first;
            lev = pp;
            break;
        }
        x -= cnt * p.BH;
    }
    if (lev < 0) return;
    const int jend = min(j + (1 << lev), p.N);
    const int lidx = LOGC + lev + 1;
    const int dk = FDK ? FDK : p.dk, dv = FDV ? FDV : p.dv;
    const int tid = threadIdx.x;
    // two copies of the chunk's scaled Q^T and dO^T where the LDS allows
    // (p.rs_nbuf == 2): chunk c is written into copy c & 1 while the products
    // of chunk c - 1 may still read the other, so that one barrier per chunk
    // suffices; with one copy a second barrier guards the overwrite
    const int csz = (dk + dv) * (C + kPadT);
    E* buf0 = reinterpret_cast<E*>(smem);
    const double* cum = p.cum + (size_t)bh * p.N;
    const double cj = cum[j - 1];

    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int nw = blockDim.x / kWave;
    const int m = lane & 15, g = lane >> 4;
    const int ncv = dv / 16;
    const int ntiles = (dk / 16) * ncv;
    f32x4 acc[MAXT];
#pragma unroll
    for (int u = 0; u < MAXT; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A chunk's loads, all branch-free: every wave reads a and lambda of the
    // whole chunk (lane l: tokens 2l and 2l + 1; rows past T read the chunk's
    // first row), A at the end of the previous chunk, and the chunk's q and
    // dO rows.  Two chunks are in flight ahead of the one being used.
    struct Loaded {
        ChunkRows<E, C, QD, 256> qr;
        ChunkRows<E, C, OD, 256> orr;
        float a0, a1, l0, l1, base;
    };
    Loaded ld0, ld1;
    auto load = [&](Loaded& L, int c) __attribute__((always_inline)) {
        const int nvalid = min(C, p.T - c * C);
        const size_t row0 = (size_t)bh * p.T + (size_t)c * C;
        const size_t r0 = row0 + min(2 * lane, nvalid - 1), r1 = row0 + min(2 * lane + 1, nvalid - 1);
        L.a0 = p.a[r0];
        L.a1 = p.a[r1];
        L.l0 = p.lam[r0 * p.L + lidx];
        L.l1 = p.lam[r1 * p.L + lidx];
        L.base = (float)(cum[c - 1] - cj);
        L.qr.load(static_cast<const E*>(p.q) + row0 * dk, dk, nvalid);
        L.orr.load(static_cast<const E*>(p.dout) + row0 * dv, dv, nvalid);
    };
    auto step = [&](Loaded& L, int c) __attribute__((always_inline)) {
        const int nvalid = min(C, p.T - c * C);
        if (p.rs_nbuf == 1 && c > j) __syncthreads();  // the products of chunk c - 1 are done
        E* QT = buf0 + (p.rs_nbuf == 2 ? (c & 1) * csz : 0);  // [dk][C + kPadT], scaled rows
        E* OT = QT + dk * (C + kPadT);  // [dv][C + kPadT]
        // chunk-local inclusive sum of a in registers (each wave the whole
        // chunk), then e_t = lambda_t exp(A_t - A(end of block j - 1))
        const bool ok0 = 2 * lane < nvalid, ok1 = 2 * lane + 1 < nvalid;
        const float x0 = ok0 ? L.a0 : 0.f, x1 = ok1 ? L.a1 : 0.f;
        float incl = x0 + x1;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        const float e0 = ok0 ? L.l0 * __expf(L.base + incl - x1) : 0.f;
        const float e1 = ok1 ? L.l1 * __expf(L.base + incl) : 0.f;
        L.qr.store_tr_scaled(dk, QT, [&](int s) __attribute__((always_inline)) {
            const float y0 = __shfl(e0, s >> 1, kWave), y1 = __shfl(e1, s >> 1, kWave);
            return (s & 1) ? y1 : y0;
        });
        L.orr.store(dv, nullptr, OT, nullptr);
        __syncthreads();  // chunk c staged; every wave is past the products of chunk c - 1
        if (c + DEPTH < jend) load(L, c + DEPTH);
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {
            const int tile = wave + u * nw;
            if (tile < ntiles) {
                const int d0 = (tile / ncv) * 16, c0 = (tile % ncv) * 16;
                const E* qa = QT + (d0 + m) * (C + kPadT) + 4 * g;
                const E* ob = OT + (c0 + m) * (C + kPadT) + 4 * g;
#pragma unroll
                for (int S = 0; S < C / 16; ++S) {
                    if constexpr (sizeof(E) == 2) {
                        acc[u] = mma(Frag<bf16_t, 16>::load(qa + 16 * S), Frag<bf16_t, 16>::load(ob + 16 * S),
                                     acc[u]);
                    } else {
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) acc[u] = mma(qa[16 * S + jj], ob[16 * S + jj], acc[u]);
                    }
                }
            }
        }
    };
    load(ld0, j);
    if constexpr (DEPTH == 2) {
        if (j + 1 < jend) load(ld1, j + 1);
        for (int c = j; c < jend; c += 2) {
            step(ld0, c);
            if (c + 1 < jend) step(ld1, c + 1);
        }
    } else {
        for (int c = j; c < jend; ++c) step(ld0, c);
    }
    if constexpr (sizeof(E) == 2) {
        // bf16 inputs: R alone, in bf16 ([dk][dv]), the one operand form the
        // dk / dv kernel stages (it reads R^T through transpose reads)
        bf16_t* Rd = p.rst16 + ((size_t)bh * p.N + j) * dk * dv;
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {
            const int tile = wave + u * nw;
            if (tile < ntiles) {
                const int d0 = (tile / ncv) * 16, c0 = (tile % ncv) * 16;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    Rd[(size_t)(d0 + 4 * g + q) * dv + c0 + m] = __builtin_bit_cast(bf16_t, (__bf16)acc[u][q]);
            }
        }
    } else {
        float* Rd = p.rst + ((size_t)bh * p.N + j) * dk * dv;
        float* RTd = p.rstT + ((size_t)bh * p.N + j) * dv * dk;
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {
            const int tile = wave + u * nw;
            if (tile < ntiles) {
                const int d0 = (tile / ncv) * 16, c0 = (tile % ncv) * 16;
#pragma unroll
                for (int q = 0; q < 4; ++q) Rd[(size_t)(d0 + 4 * g + q) * dv + c0 + m] = acc[u][q];
                *reinterpret_cast<float4*>(RTd + (size_t)(c0 + m) * dk + d0 + 4 * g) =
                    make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
            }
        }
    }
}

// --------------------------------------------------------------------------
// dk and dv: one block per chunk, one wave per 16 key rows

template <typename E, int C, int DM, int FDK, int FDV>
__global__ __launch_bounds__(C / 16 * 64, C == 128 ? 2 : 3) void k_bwd_dkv(BwdParams p) {
    constexpr int NW = C / 16;
    constexpr int LOGC = LogC<C>::v;
    constexpr int KS = BStep<E>::KS;
    constexpr int MAXK = DM / KS;
    constexpr int NB = DM / 16;
    typedef Frag<E, KS> FR;
    typedef typename FR::type frag_t;
    constexpr int KPL = FR::kpl;
    constexpr bool NAT = sizeof(E) == 2;

    extern __shared__ __align__(16) char smem[];
    const int blk = xcd_local_block(blockIdx.x, gridDim.x);
    const int bh = blk / p.N;
    const int i = blk - bh * p.N;
    const int t0 = i * C;
    const int nvalid = min(C, p.T - t0);
    const int dk = FDK ? FDK : p.dk, dv = FDV ? FDV : p.dv;  // FDK, FDV: head dims fixed at compile time
    const int L = p.L, nlev = p.nlev;
    const int nkk = dk / KS, nkv = dv / KS;
    constexpr int NT = NW * kWave;
    constexpr int NLM = (C * (LOGC + 1) + NT - 1) / NT;  // intra-chunk lambda values per thread
    float* a_raw = reinterpret_cast<float*>(smem);
    float* A = a_raw + C;
    float* wlog = A + C;                          // [kMaxLev] A(end of block j - 1) - A(end of chunk i - 1)
    float* lamc = wlog + kMaxLev;                 // [C][LOGC + 1]
    // the chunk's Q and dO: bf16 natural ([C][d + kPadB]), fp32 transposed
    // ([d][C + kPadT]); then (bf16) one carried state, p.st_elems elements
    E* Qc = reinterpret_cast<E*>(lamc + C * (LOGC + 1));
    E* Oc = Qc + (NAT ? C * (dk + kPadB) : dk * (C + kPadT));
    E* Ss = Oc + (NAT ? C * (dv + kPadB) : dv * (C + kPadT));
    const size_t row0 = (size_t)bh * p.T + t0;

    const int lane = threadIdx.x & (kWave - 1);
    const int R = threadIdx.x / kWave;
    const int m = lane & 15, g = lane >> 4;
    const int s = 16 * R + m;  // key row within the chunk
    const bool svalid = s < nvalid;
    const size_t srow = row0 + s;
    const size_t lrow0 = row0 + (svalid ? s : 0);  // the row the loads read (row t0 past T)

    // Every global load of the prologue is issued before the first LDS
    // write, without branches: the lane's own k and v fragments, the chunk's
    // a, lambda (intra-chunk levels), Q and dO, and the decays of the coarse
    // levels.
    const E* krow = static_cast<const E*>(p.k) + lrow0 * dk;
    const E* vrow = static_cast<const E*>(p.v) + lrow0 * dv;
    frag_t vf[MAXK], kf[MAXK];
#pragma unroll
    for (int ks = 0; ks < MAXK; ++ks) {
        vf[ks] = ks < nkv ? own_op<E>(vrow, svalid, ks, g) : frag_t{};
        kf[ks] = ks < nkk ? own_op<E>(krow, svalid, ks, g) : frag_t{};
    }
    const float av = p.a[row0 + min((int)threadIdx.x, nvalid - 1)];
    float lm[NLM];
#pragma unroll
    for (int u = 0; u < NLM; ++u) {
        const int x = threadIdx.x + u * NT;
        const int t = x / (LOGC + 1), l = x - t * (LOGC + 1);
        const float y = p.lam[(row0 + min(t, nvalid - 1)) * L + min(l, L - 1)];
        lm[u] = (t < nvalid && l < L) ? y : 0.f;
    }
    float wl = 0.f;
    if (threadIdx.x < nlev) {  // at most two loads per thread
        const int pb = threadIdx.x;
        const int j = ((i >> pb) | 1) << pb;
        const bool use = !((i >> pb) & 1) && j < p.N;
        const double* cum = p.cum + (size_t)bh * p.N;
        const double cj = cum[use ? j - 1 : 0];
        const double ci = cum[i > 0 ? i - 1 : 0];
        wl = use ? (float)(cj - (i > 0 ? ci : 0.0)) : 0.f;
    }
    const E* qg = static_cast<const E*>(p.q) + row0 * dk;
    const E* og = static_cast<const E*>(p.dout) + row0 * dv;
    ChunkRows<E, C, DM, NT, kPadB, true> qr, orr;
    qr.load(qg, dk, nvalid);
    orr.load(og, dv, nvalid);
    // the coarse levels this chunk feeds (clear bits pb of i whose block
    // j = ((i >> pb) | 1) << pb exists), and the first one's state, whose
    // loads stay in flight through the staging and the chunk's own block
    unsigned todo = 0;
    for (int pb = 0; pb < nlev; ++pb)
        if (!((i >> pb) & 1) && ((((i >> pb) | 1) << pb) < p.N)) todo |= 1u << pb;
    auto block_of = [&](int pb) __attribute__((always_inline)) {
        return (size_t)bh * p.N + (((i >> pb) | 1) << pb);
    };
    constexpr int NSR = (NAT && FDK > 0 && FDV > 0) ? FDK * FDV / (8 * NT) : 1;
    StateRegs16<NSR, NT> str;
    if constexpr (NAT && FDK > 0 && FDV > 0) {
        if (todo) str.load(p.rst16 + block_of(__builtin_ctz(todo)) * dk * dv);
    }

    if (threadIdx.x < C) a_raw[threadIdx.x] = (int)threadIdx.x < nvalid ? av : 0.f;
    if (threadIdx.x < nlev) wlog[threadIdx.x] = wl;
#pragma unroll
    for (int u = 0; u < NLM; ++u) {
        const int x = threadIdx.x + u * NT;
        if (x < C * (LOGC + 1)) lamc[x] = lm[u];
    }
    qr.store(dk, NAT ? Qc : nullptr, NAT ? nullptr : Qc, nullptr);
    orr.store(dv, NAT ? Oc : nullptr, NAT ? nullptr : Oc, nullptr);
    __syncthreads();
    if (threadIdx.x < kWave) wave_cumsum(a_raw, A, C);
    __syncthreads();
    const float As = A[s];

    // The chunk's own block, transposed: dk^T[d][s] = sum_t Q^T[d][t] Z[t][s]
    // with Z = dP (.) M (dP from dO and v_s), dv^T[c][s] = sum_t dO^T[c][t] P[t][s]
    // with P = (Q K^T) (.) M (from q and k_s).  One tile of 16 rows t, S >= R,
    // at a time, handed straight to the gradient product (a runtime loop:
    // accumulators updated in place).
    auto tiles = [&](auto kpass, f32x4 (&acc)[NB]) __attribute__((always_inline)) {
        constexpr bool GK = decltype(kpass)::value;
        const int dout_dim = GK ? dk : dv;       // columns of the gradient
        const int nkc = GK ? nkv : nkk;          // contraction steps of the tile products
        const E* tn = GK ? Oc : Qc;              // rows t of the tile products
        const E* ht = GK ? Qc : Oc;              // the hand-off product's matrix
        const int hd = GK ? dk : dv;
        const frag_t* own = GK ? vf : kf;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int S = R; S < NW; ++S) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < MAXK; ++ks)
                if (ks < nkc) x = mma(rows_op<E, C>(tn, tn, GK ? dv : dk, 16 * S, ks, m, g), own[ks], x);
            float z[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = 16 * S + 4 * g + q;
                const float dec = t >= s ? __expf(A[t] - As) : 0.f;
                z[q] = x[q] * lamc[t * (LOGC + 1) + fenwick_level(t, s)] * dec;
            }
            const typename Hand<E>::type Hs = Hand<E>::pack(z[0], z[1], z[2], z[3]);
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
                if (16 * cb < dout_dim) acc[cb] = hand_mma<E, C>(ht, hd, 16 * cb, S, Hs, acc[cb], m, g);
        }
    };
    f32x4 acck[NB], accv[NB];
    tiles(std::integral_constant<bool, true>{}, acck);
    tiles(std::integral_constant<bool, false>{}, accv);

    // Later blocks that see this chunk at a coarse level: the clear bits pb
    // of i whose block j = ((i >> pb) | 1) << pb exists, lowest first; each
    // adds w_s R(j) v_s to dk_s and w_s R(j)^T k_s to dv_s.
    if constexpr (NAT) {
        // R(j) is bf16 [dk][dv]: staged once per level for both products; the
        // dk rows read it as is (contraction over dv), the dv rows through
        // transpose reads (contraction over dk).  With the head dims fixed at
        // compile time (PF) it is staged whole and the next state's loads are
        // issued before the current one is used; otherwise in rounds of
        // srows of its dk rows.
        constexpr bool PF = FDK > 0 && FDV > 0;
        const int pitch = dv + kPadB;
        auto use = [&](float w, int r0, int nr) __attribute__((always_inline)) {
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if (16 * cb < dk && 16 * cb >= r0 && 16 * cb < r0 + nr) {
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
                    const E* rr = Ss + (16 * cb - r0 + m) * pitch;  // r0 % 16 == 0
#pragma unroll
                    for (int ks = 0; ks < MAXK; ++ks)
                        if (ks < nkv) y = mma(Frag<bf16_t, 16>::load(rr + swz8(m, ks * 16 + 4 * g)), vf[ks], y);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acck[cb][q] += w * y[q];
                }
            }
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if (16 * cb < dv) {
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < MAXK; ++ks)
                        if (ks < nkk && 16 * ks >= r0 && 16 * ks < r0 + nr)
                            y = mma(tr_op(Ss, pitch, 16 * ks - r0, 16 * cb, m, g), kf[ks], y);
#pragma unroll
                    for (int q = 0; q < 4; ++q) accv[cb][q] += w * y[q];
                }
            }
        };
        if constexpr (PF) {
            StateRegs16<NSR, NT>& st = str;
            while (todo) {
                const int pb = __builtin_ctz(todo);
                todo &= todo - 1;
                const float w = svalid ? __expf(wlog[pb] - As) : 0.f;
                __syncthreads();  // the previous state's reads are done
                st.store(dv, Ss);
                __syncthreads();
                if (todo) st.load(p.rst16 + block_of(__builtin_ctz(todo)) * dk * dv);
                use(w, 0, dk);
            }
        } else {
            const int srows = min(dk, (p.st_elems / pitch) & ~15);
            while (todo) {
                const int pb = __builtin_ctz(todo);
                todo &= todo - 1;
                const float w = svalid ? __expf(wlog[pb] - As) : 0.f;
                const bf16_t* Rg = p.rst16 + block_of(pb) * dk * dv;
                for (int r0 = 0; r0 < dk; r0 += srows) {
                    const int nr = min(srows, dk - r0);
                    __syncthreads();  // the previous round's reads are done
                    stage_rows16<NT>(Rg, dv, r0, nr, Ss);
                    __syncthreads();
                    use(w, r0, nr);
                }
            }
        }
    } else {
        // fp32 inputs: R and R^T read from global memory
        while (todo) {
            const int pb = __builtin_ctz(todo);
            todo &= todo - 1;
            const float w = svalid ? __expf(wlog[pb] - As) : 0.f;
            const float* Rk = p.rst + block_of(pb) * dk * dv;
            const float* Rv = p.rstT + block_of(pb) * dv * dk;
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if (16 * cb < dk) {
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
                    const float* rr = Rk + (size_t)(16 * cb + m) * dv + g * KPL;
#pragma unroll
                    for (int ks = 0; ks < MAXK; ++ks)
                        if (ks < nkv) y = mma(FR::from_f32(rr + ks * KS), vf[ks], y);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acck[cb][q] += w * y[q];
                }
                if (16 * cb < dv) {
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
                    const float* rr = Rv + (size_t)(16 * cb + m) * dk + g * KPL;
#pragma unroll
                    for (int ks = 0; ks < MAXK; ++ks)
                        if (ks < nkk) y = mma(FR::from_f32(rr + ks * KS), kf[ks], y);
#pragma unroll
                    for (int q = 0; q < 4; ++q) accv[cb][q] += w * y[q];
                }
            }
        }
    }

    // outputs, and k_s . dk_s for the decay gradient (k in the C layout of
    // the dk tiles: for bf16 exactly the elements of the lane's own k fragments)
    float da2 = 0.f;
    float* gkrow = p.gk + srow * dk;
    float* gvrow = p.gv + srow * dv;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        if (16 * cb < dk) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float kq;
                if constexpr (NAT) {
                    kq = (float)kf[cb][q];
                } else {
                    const float x = krow[16 * cb + 4 * g + q];
                    kq = svalid ? x : 0.f;
                }
                da2 += acck[cb][q] * kq;
            }
            if (svalid)
                *reinterpret_cast<float4*>(gkrow + 16 * cb + 4 * g) =
                    make_float4(acck[cb][0], acck[cb][1], acck[cb][2], acck[cb][3]);
        }
        if (16 * cb < dv && svalid)
            *reinterpret_cast<float4*>(gvrow + 16 * cb + 4 * g) =
                make_float4(accv[cb][0], accv[cb][1], accv[cb][2], accv[cb][3]);
    }
    da2 = sum_groups(da2);
    if (svalid && g == 0) p.dA2[srow] = da2;
}

// --------------------------------------------------------------------------
// da_j = sum_{t >= j} (dA1_t - dA2_t): one block per (batch, head), walking
// the sequence from its end in tiles of 2048 tokens (8 consecutive tokens a
// thread, so that loads and stores are contiguous over the block); fp64
// sums, the sum of the later tiles carried from tile to tile.

__global__ __launch_bounds__(256) void k_bwd_da(BwdParams p) {
    constexpr int PT = 8, NT = 256, TILE = PT * NT;
    __shared__ double part[NT];
    const int tid = threadIdx.x;
    const size_t base = (size_t)blockIdx.x * p.T;
    double carry = 0.0;  // the tokens after the current tile
    for (int t1 = p.T; t1 > 0; t1 -= TILE) {
        const int t0 = max(0, t1 - TILE);
        double x[PT];
        double sum = 0.0;
#pragma unroll
        for (int j = 0; j < PT; ++j) {  // no branch: past t1 reads token t0 and is zeroed
            const int t = t0 + tid * PT + j;
            const int tc = t < t1 ? t : t0;
            const double y = (double)p.dA1[base + tc] - (double)p.dA2[base + tc];
            x[j] = t < t1 ? y : 0.0;
            sum += x[j];
        }
        part[tid] = sum;
        __syncthreads();
        // inclusive suffix scan over the threads (Hillis-Steele)
        for (int off = 1; off < NT; off <<= 1) {
            const double y = tid + off < NT ? part[tid + off] : 0.0;
            __syncthreads();
            part[tid] += y;
            __syncthreads();
        }
        double run = carry + part[tid] - sum;  // the threads after this one, and the later tiles
#pragma unroll
        for (int j = PT - 1; j >= 0; --j) {
            const int t = t0 + tid * PT + j;
            run += x[j];
            if (t < t1) p.ga[base + t] = (float)run;
        }
        carry += part[0];
        __syncthreads();  // part[] is rewritten by the next tile
    }
}

// The same suffix sums over more blocks (the one-block-per-head kernel above
// walks the sequence serially): pieces of 1024 tokens per (batch, head).
// First each piece's total, then each piece's suffix sums plus the totals of
// the later pieces; fp64 throughout.
constexpr int kDaPiece = 1024;

__global__ __launch_bounds__(256) void k_bwd_da_part(BwdParams p, double* __restrict__ parts, int np) {
    constexpr int NT = 256, PT = kDaPiece / NT;
    __shared__ double red[NT / 64];
    const int bh = blockIdx.x / np, pc = blockIdx.x - bh * np;
    const size_t base = (size_t)bh * p.T;
    const int t0 = pc * kDaPiece + threadIdx.x * PT;
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int t = t0 + j;
        if (t < p.T) sum += (double)p.dA1[base + t] - (double)p.dA2[base + t];
    }
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) parts[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void k_bwd_da_scan(BwdParams p, const double* __restrict__ parts, int np) {
    constexpr int NT = 256, PT = kDaPiece / NT;
    __shared__ double part[NT];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / np, pc = blockIdx.x - bh * np;
    const size_t base = (size_t)bh * p.T;
    const int t0 = pc * kDaPiece + tid * PT;
    // the later pieces of this (batch, head)
    double carry = 0.0;
    for (int u = pc + 1; u < np; ++u) carry += parts[(size_t)bh * np + u];
    double x[PT];
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int t = t0 + j;
        x[j] = t < p.T ? (double)p.dA1[base + t] - (double)p.dA2[base + t] : 0.0;
        sum += x[j];
    }
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {  // inclusive suffix scan over the threads
        const double y = tid + off < NT ? part[tid + off] : 0.0;
        __syncthreads();
        part[tid] += y;
        __syncthreads();
    }
    double run = carry + part[tid] - sum;  // the later threads and pieces
#pragma unroll
    for (int j = PT - 1; j >= 0; --j) {
        const int t = t0 + j;
        run += x[j];
        if (t < p.T) p.ga[base + t] = (float)run;
    }
}

// A at the end of every chunk for the R(j) and dk / dv stages: one block per
// (batch, head), walking the sequence in tiles of 8192 tokens.  Each thread
// sums two strips of 16 consecutive tokens (fp32, in token order; 16-byte
// loads where the strip is whole and aligned), a chunk's total is the sum of
// its strips in order (C is a multiple of 16; at most 256 chunks a tile), and the chunk totals are
// summed in fp64, the earlier tiles' sum carried.
__global__ __launch_bounds__(256) void k_bwd_chunk_cum(BwdParams p) {
    constexpr int NT = 256, S = 16, NS = 2 * NT;  // strips per tile
    __shared__ float strip[NS];
    __shared__ double part[NT];
    const int tid = threadIdx.x;
    const size_t base = (size_t)blockIdx.x * p.T;
    const int spc = p.C / S;        // strips per chunk
    const int cpt = min(NS / spc, NT);  // chunks per tile
    const bool vec = (p.T % 4) == 0 && (reinterpret_cast<uintptr_t>(p.a) % 16) == 0;
    double carry = 0.0;
    for (int c0 = 0; c0 < p.N; c0 += cpt) {
        const int tt0 = c0 * p.C;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int sidx = u * NT + tid;
            if (sidx >= cpt * spc) break;
            const int t = tt0 + sidx * S;
            float tot = 0.f;
            if (vec && t + S <= p.T) {
                const float4* src = reinterpret_cast<const float4*>(p.a + base + t);
#pragma unroll
                for (int k = 0; k < S / 4; ++k) {
                    const float4 y = src[k];
                    tot += y.x;
                    tot += y.y;
                    tot += y.z;
                    tot += y.w;
                }
            } else {
                for (int k = 0; k < S; ++k)
                    if (t + k < p.T) tot += p.a[base + t + k];
            }
            strip[sidx] = tot;
        }
        __syncthreads();
        const int c = c0 + tid;
        float ct = 0.f;
        if (tid < cpt && c < p.N)
            for (int k = 0; k < spc; ++k) ct += strip[tid * spc + k];
        part[tid] = ct;
        __syncthreads();
        for (int off = 1; off < NT; off <<= 1) {  // inclusive prefix (Hillis-Steele)
            const double y = tid >= off ? part[tid - off] : 0.0;
            __syncthreads();
            part[tid] += y;
            __syncthreads();
        }
        // p.cum is read-only for the other stages; this kernel fills it
        if (tid < cpt && c < p.N) const_cast<double*>(p.cum)[(size_t)blockIdx.x * p.N + c] = carry + part[tid];
        carry += part[cpt - 1];
        __syncthreads();  // strip[] and part[] are rewritten by the next tile
    }
}

// dlambda and q . dq summed over the column blocks of the fused dq pass.
// One block per 64 tokens of one (batch, head): the level-major parts are
// read a level at a time (64 consecutive tokens), transposed through LDS and
// written as whole [token][L] rows.
__global__ __launch_bounds__(256) void k_bwd_dlam_sum(BwdParams p, const float* __restrict__ dlp,
                                                       const float* __restrict__ dqd, int ndvb,
                                                       int lu) {
    __shared__ float tile[64][65];
    const int ntb = (p.T + 63) / 64;
    const int bh = blockIdx.x / ntb;
    const int t0 = (blockIdx.x % ntb) * 64;
    const int nt = min(64, p.T - t0);
    const size_t rows = (size_t)p.BH * p.T;
    for (int e = threadIdx.x; e < 64 * lu; e += 256) {
        const int l = e >> 6, t = e & 63;
        float s = 0.f;
        if (t < nt)
            for (int b = 0; b < ndvb; ++b)
                s += dlp[(((size_t)b * p.BH + bh) * lu + l) * p.T + t0 + t];
        tile[t][l] = s;
    }
    __syncthreads();
    float* g = p.glam + ((size_t)bh * p.T + t0) * p.L;
    for (int e = threadIdx.x; e < nt * p.L; e += 256) {
        const int t = e / p.L, l = e - t * p.L;
        g[e] = l < lu ? tile[t][l] : 0.f;
    }
    if (threadIdx.x < nt) {
        const size_t row = (size_t)bh * p.T + t0 + threadIdx.x;
        float d = 0.f;
        for (int b = 0; b < ndvb; ++b) d += dqd[(size_t)b * rows + row];
        p.dA1[row] = d;
    }
}

// LDS of the chunk's two staged matrices (head dims dk and dv)
template <typename E, int C>
size_t chunk_pair_elems(int dk, int dv) {
    return sizeof(E) == 2 ? (size_t)C * (dk + kPadB) + (size_t)C * (dv + kPadB)
                          : (size_t)(dk + dv) * (C + kPadT);
}
template <typename E, int C>
size_t dq_smem(int dk, int dv, int nlev) {
    return (2 * C + kMaxLev + (size_t)C * nlev) * sizeof(float) + chunk_pair_elems<E, C>(dk, dv) * sizeof(E);
}
template <typename E, int C>
size_t dkv_smem(int dk, int dv) {
    return (2 * C + kMaxLev + (size_t)C * (LogC<C>::v + 1)) * sizeof(float) +
           chunk_pair_elems<E, C>(dk, dv) * sizeof(E);
}
template <typename E, int C>
size_t rstate_smem(int dk, int dv, int nbuf) {
    return nbuf * (size_t)(dk + dv) * (C + kPadT) * sizeof(E);
}

constexpr size_t kLdsMax = 160 * 1024;  // bytes of LDS one block may use on gfx950

// bf16 elements of the state-staging buffer behind `base` bytes of other LDS:
// the whole state when it fits, else as many 16-row rounds as fit.  0 for
// fp32 inputs (the fp32 path reads states from global memory) and -1 when
// not even one round of 16 rows fits.
template <typename E>
long state_elems(size_t base, int dk, int dv) {
    if (sizeof(E) != 2) return 0;
    const long need = (long)dk * (dv + kPadB);  // every staged state is [dk][dv]
    const long avail = base < kLdsMax ? (long)((kLdsMax - base) / 2) : 0;
    const long minimum = 16L * (dv + kPadB);
    const long got = std::min(need, avail);
    return got >= minimum ? got : -1;
}

template <typename K>
hipError_t set_smem(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// FDK, FDV: the head dims when fixed at compile time (0: read from p)
template <typename E, int C, int DM, int FDK = 0, int FDV = 0>
hipError_t launch_bwd_typed(const BwdParams& p, hipStream_t stream) {
    const int nblk = p.BH * p.N;
    BwdParams p1 = p, p3 = p;
    size_t s1 = dq_smem<E, C>(p.dk, p.dv, p.nlev);
    const long e1 = state_elems<E>(s1, p.dk, p.dv);
    size_t s3 = dkv_smem<E, C>(p.dk, p.dv);
    const long e3 = state_elems<E>(s3, p.dk, p.dv);
    if (e1 < 0 || e3 < 0) return hipErrorInvalidValue;
    p1.st_elems = (int)e1;
    p3.st_elems = (int)e3;
    s1 += (size_t)e1 * sizeof(E);
    s3 += (size_t)e3 * sizeof(E);
    // the compile-time head-dim kernels stage every carried state whole:
    // where it does not fit the LDS, the generic kernel runs instead
    const long whole = (long)p.dk * (p.dv + kPadB);
    const bool f1 = FDK > 0 && e1 >= whole, f3 = FDK > 0 && e3 >= whole;
    hipError_t err = hipSuccess;
    if (p.dq_done) {
        // dq, dlambda and dA1 come from the fused dq pass
    } else if (f1) {
        err = set_smem(&k_bwd_dq<E, C, DM, FDK, FDV>, s1);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((k_bwd_dq<E, C, DM, FDK, FDV>), dim3(nblk), dim3(C / 16 * 64), s1, stream, p1);
    } else {
        err = set_smem(&k_bwd_dq<E, C, DM, 0, 0>, s1);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((k_bwd_dq<E, C, DM, 0, 0>), dim3(nblk), dim3(C / 16 * 64), s1, stream, p1);
    }
    // R(j): one walk over the query chunks where it applies (LOGLIN_BWD_RSTATE=blocks
    // keeps the block-per-R(j) kernel below), else one block per R(j)
    // dk and dv: one reverse walk per segment where it applies (it builds the
    // R(j) inside a segment itself; LOGLIN_BWD_DKV=chunks keeps the
    // block-per-chunk kernel below)
    bool walked = false, kvwalk = false;
    if constexpr (sizeof(E) == 2 && C == 64) {
        const char* mode = getenv("LOGLIN_BWD_RSTATE");
        const char* kvmode = getenv("LOGLIN_BWD_DKV");
        if (p.N > 1 && !(mode && strcmp(mode, "blocks") == 0) && bwd_rwalk_applies(p)) {
            kvwalk = !(kvmode && strcmp(kvmode, "chunks") == 0) && bwd_kvwalk_applies(p);
            err = launch_bwd_rwalk(p, kvwalk, stream);
            if (err != hipSuccess) return err;
            walked = true;
        }
    }
    if (p.N > 1 && !walked) {
        BwdParams p2 = p;
        p2.rs_nbuf = rstate_smem<E, C>(p.dk, p.dv, 2) <= kLdsMax ? 2 : 1;
        const size_t s2 = rstate_smem<E, C>(p.dk, p.dv, p2.rs_nbuf);
        err = set_smem(&k_bwd_rstate<E, C, DM, FDK, FDV>, s2);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((k_bwd_rstate<E, C, DM, FDK, FDV>), dim3(p.BH * (p.N - 1)), dim3(256), s2, stream,
                           p2);
    }
    if (kvwalk) {
        err = launch_bwd_kvwalk(p, stream);
        if (err != hipSuccess) return err;
    } else if (f3) {
        err = set_smem(&k_bwd_dkv<E, C, DM, FDK, FDV>, s3);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((k_bwd_dkv<E, C, DM, FDK, FDV>), dim3(nblk), dim3(C / 16 * 64), s3, stream, p3);
    } else {
        err = set_smem(&k_bwd_dkv<E, C, DM, 0, 0>, s3);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((k_bwd_dkv<E, C, DM, 0, 0>), dim3(nblk), dim3(C / 16 * 64), s3, stream, p3);
    }
    if (p.cum && (long)((p.T + kDaPiece - 1) / kDaPiece) <= (long)p.N) {
        // the piece totals go to the chunk-decay region ([BH][N] doubles), which
        // nothing reads after the dk / dv stage
        const int np = (p.T + kDaPiece - 1) / kDaPiece;
        double* parts = const_cast<double*>(p.cum);
        hipLaunchKernelGGL(k_bwd_da_part, dim3(p.BH * np), dim3(256), 0, stream, p, parts, np);
        hipLaunchKernelGGL(k_bwd_da_scan, dim3(p.BH * np), dim3(256), 0, stream, p,
                           static_cast<const double*>(parts), np);
    } else {
        hipLaunchKernelGGL(k_bwd_da, dim3(p.BH), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

template <typename E, int C>
hipError_t launch_bwd_c(const BwdParams& p, hipStream_t s) {
    // bf16 head-dim pairs of the measured workloads get kernels with the
    // dims fixed at compile time (every head-dim branch folded away)
    if constexpr (sizeof(E) == 2 && C == 64) {
        if (p.dk == 128 && p.dv == 64) return launch_bwd_typed<E, C, 128, 128, 64>(p, s);
        if (p.dk == 64 && p.dv == 64) return launch_bwd_typed<E, C, 64, 64, 64>(p, s);
    }
    if constexpr (sizeof(E) == 2 && C == 128) {
        if (p.dk == 128 && p.dv == 128) return launch_bwd_typed<E, C, 128, 128, 128>(p, s);
    }
    switch (p.dk > p.dv ? p.dk : p.dv) {
        case 16: return launch_bwd_typed<E, C, 16>(p, s);
        case 32: return launch_bwd_typed<E, C, 32>(p, s);
        case 64: return launch_bwd_typed<E, C, 64>(p, s);
        case 128: return launch_bwd_typed<E, C, 128>(p, s);
    }
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_bwd_e(const BwdParams& p, hipStream_t s) {
    switch (p.C) {
        case 16: return launch_bwd_c<E, 16>(p, s);
        case 32: return launch_bwd_c<E, 32>(p, s);
        case 64: return launch_bwd_c<E, 64>(p, s);
        case 128: return launch_bwd_c<E, 128>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_chunk_cum(const BwdParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(k_bwd_chunk_cum, dim3(p.BH), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_bwd_dlam_sum(const BwdParams& p, const float* dlp, const float* dqd, int ndvb,
                               int lu, hipStream_t stream) {
    const unsigned blocks = (unsigned)p.BH * ((p.T + 63) / 64);
    hipLaunchKernelGGL(k_bwd_dlam_sum, dim3(blocks), dim3(256), 0, stream, p, dlp, dqd, ndvb, lu);
    return hipGetLastError();
}

hipError_t launch_bwd_chunked(const BwdParams& p, bool bf16, hipStream_t stream) {
    return bf16 ? launch_bwd_e<bf16_t>(p, stream) : launch_bwd_e<float>(p, stream);
}

}  // namespace loglin
