// Block states R(j) of the backward's dk / dv stage, built in one pass over
// the query chunks (bf16 inputs, 64-token chunks, d_v = 64; gfx950).
//
// "Log-linear attention, and what a logarithm buys", sections 2-3: the keys
// of chunk i reach the queries of the block of 2^p chunks starting at
// j = ((i >> p) | 1) << p at level log2 C + p + 1.  The dk / dv kernel reads,
// for every such block,
//     R(j) = sum over t in the block of lambda_t^(log2 C + p + 1) e^(A_t - A(end of chunk j - 1)) q_t dO_t^T
// ([d_k][d_v], bf16).  Query chunk i belongs to the block of level p that
// starts at (i >> p) << p exactly when bit p of i is set, so a walk over the
// chunks in order can build every block from the chunks it visits: one
// fp32 accumulator per level, the chunk's products added to the levels whose
// bit is set, the state written when the block's last chunk is done.  Every
// query chunk is read once (a block per level would read it once per set bit).
//
// One block per (batch*head, segment of 2^m chunks).  Levels below m close
// inside the segment.  A block of a level p >= m spans several segments: each
// segment leaves its part (fp32, same reference point e^(-A(end of chunk j - 1)))
// and a second kernel sums the parts of each such block.
//
// Data movement: q, dO, lambda and a of the next chunk are copied global ->
// LDS by the LDS-DMA path two chunks ahead of the one in use (three
// buffers: one block per compute unit needs that depth to cover the latency).  Eight
// waves; wave w owns the 16 columns 16 (w % 4) of d_v and half of d_k, i.e.
// d_k / 32 output blocks of 16 x 16 per level, accumulated on the
// 16x16x32 bf16 matrix cores with the chunk's 64 tokens as the contraction.
// The per-token weight (lambda of the level times the decay) scales the dO
// operand in registers (rounded to bf16 once, as the staged operand of the
// other R(j) path is).

#include "tile_ops.hpp"

namespace loglin {

namespace {

constexpr int kRwWaves = 8;
constexpr int kRwSlots = 8;   // levels p < 8, i.e. at most 256 chunks
constexpr int kRwMaxL = 32;   // lambda row length staged per token
constexpr int kRwLogC = 6;    // 64-token chunks
constexpr int kRwMaxM = 5;    // at most 32 chunks per segment

// s_waitcnt with only the vector-memory counter bounded: at most N vector
// memory operations of this wave still outstanding (expcnt, lgkmcnt at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ bf16x8 scale8(const bf16x8& x, const float4& w0, const float4& w1) {
    bf16x8 r;
    r[0] = (__bf16)((float)x[0] * w0.x);
    r[1] = (__bf16)((float)x[1] * w0.y);
    r[2] = (__bf16)((float)x[2] * w0.z);
    r[3] = (__bf16)((float)x[3] * w0.w);
    r[4] = (__bf16)((float)x[4] * w1.x);
    r[5] = (__bf16)((float)x[5] * w1.y);
    r[6] = (__bf16)((float)x[6] * w1.z);
    r[7] = (__bf16)((float)x[7] * w1.w);
    return r;
}

struct RwalkArgs {
    int m;          // chunks per segment = 2^m
    int nseg;       // segments per (batch*head)
    int ntop;       // levels p >= m that exist (nlev - m, or 0)
    int lam_dma;    // lambda rows of a whole chunk are 16-byte aligned
    int a_dma;      // a of a whole chunk is 16-byte aligned
    float* part;    // [BH][nseg][ntop][dk][dv] parts of the blocks of levels >= m
                    // (nseg ntop <= N: within an fp32 [BH][N][dk][dv] region)
};

// NSLOT: levels p < NSLOT (at most 2^NSLOT chunks)
template <int DK, int DV, int NSLOT>
__global__ __launch_bounds__(kRwWaves * 64, 1) void k_bwd_rwalk(BwdParams p, RwalkArgs w) {
    static_assert(DV == 64 && (DK == 64 || DK == 128), "head dims of this kernel");
    static_assert(NSLOT <= kRwSlots, "one wave per level for the weights");
    constexpr int NRBW = DK / 32;  // 16-row blocks of d_k per wave
    // three chunk buffers: chunks il + 1 and il + 2 are in flight while il is used
    __shared__ __align__(16) bf16_t sQ0[TC * DK];
    __shared__ __align__(16) bf16_t sQ1[TC * DK];
    __shared__ __align__(16) bf16_t sQ2[TC * DK];
    __shared__ __align__(16) bf16_t sO0[TC * DV];
    __shared__ __align__(16) bf16_t sO1[TC * DV];
    __shared__ __align__(16) bf16_t sO2[TC * DV];
    __shared__ __align__(16) float sL0[TC * kRwMaxL];
    __shared__ __align__(16) float sL1[TC * kRwMaxL];
    __shared__ __align__(16) float sL2[TC * kRwMaxL];
    __shared__ __align__(16) float sa0[TC];
    __shared__ __align__(16) float sa1[TC];
    __shared__ __align__(16) float sa2[TC];
    __shared__ __align__(16) float sW[kRwSlots][TC];  // per-token weights of each level
    // A at the end of chunks i0 - 1 .. i0 + 2^m - 1 (sCum[k]: chunk i0 - 1 + k),
    // and at the end of chunk j - 1 for the blocks of levels >= m
    __shared__ double sCum[(1 << kRwMaxM) + 1];
    __shared__ double sTop[kRwSlots];

    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int seg = blk % w.nseg;
    const int bh = blk / w.nseg;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
    const int c0 = 16 * (wave & 3);           // this wave's d_v columns
    const int d0 = (wave >> 2) * (DK / 2);    // and d_k rows
    const int N = p.N, L = p.L, T = p.T, nlev = p.nlev;
    const int i0 = seg << w.m;
    const int ntl = min(1 << w.m, N - i0);
    const size_t row0 = (size_t)bh * T;
    const double* cum = p.cum + (size_t)bh * N;
    const bf16_t* q = reinterpret_cast<const bf16_t*>(p.q);
    const bf16_t* dout = reinterpret_cast<const bf16_t*>(p.dout);
    bf16_t* rst = reinterpret_cast<bf16_t*>(p.rst16);

    typedef TileCopy<DK, kRwWaves> CQ;
    typedef TileCopy<DV, kRwWaves> CO;
    // copy instructions every wave issues per chunk at least (q and dO; the
    // lambda and a copies come on top for some waves)
    constexpr int KMIN = CQ::NI / kRwWaves + CO::NI / kRwWaves;
    static_assert(CQ::NI % kRwWaves == 0 && CO::NI % kRwWaves == 0, "even copy split");
    CQ cq;
    CO co;
    cq.init(DK, 0, wave);
    co.init(DV, 0, wave);
    // chunk il of the segment into LDS; rows past T: q and dO repeat the last
    // row (their weight is zero), lambda and a are zero
    auto issue = [&](int il, bf16_t* Qd, bf16_t* Od, float* Ld, float* ad) __attribute__((always_inline)) {
        const int t0 = (i0 + il) * TC;
        const int nvalid = min(TC, T - t0);
        const size_t r = row0 + t0;
        const bool whole = nvalid == TC;
        if (whole) {
            cq.issue(q + r * DK, Qd, wave);
            co.issue(dout + r * DV, Od, wave);
        } else {
            dma_tile<DK, kRwWaves>(q + r * DK, DK, 0, nvalid, Qd, wave);
            dma_tile<DV, kRwWaves>(dout + r * DV, DV, 0, nvalid, Od, wave);
        }
        if (whole && w.lam_dma) {
            const int nch = 16 * L;  // 64 rows x L floats in 16-byte pieces
            for (int u = wave; u * 64 < nch; u += kRwWaves)
                if (u * 64 + lane < nch) dma16o(p.lam + r * L, 16u * (u * 64 + lane), Ld + u * 256);
        } else {
            const int nel = nvalid * L;
            for (int u = wave; u * 64 < TC * L; u += kRwWaves) {
                const int x = u * 64 + lane;
                if (x < nel) dma4(p.lam + r * L + x, Ld + u * 64);
                else if (x < TC * L) Ld[x] = 0.f;
            }
        }
        if (wave == kRwWaves - 1) {
            if (whole && w.a_dma) {
                if (lane < TC / 4) dma16o(p.a + r, 16u * lane, ad);
            } else if (lane < nvalid) {
                dma4(p.a + r + lane, ad);
            } else {
                ad[lane] = 0.f;
            }
        }
    };

    // the decay offsets come from LDS: a vector load of cum inside the loop
    // would make the compiler wait for every copy in flight
    for (int k = threadIdx.x; k <= ntl; k += kRwWaves * 64)
        sCum[k] = i0 + k >= 1 ? cum[i0 - 1 + k] : 0.0;
    if (threadIdx.x < NSLOT) {
        const int pl = threadIdx.x;
        const int j = (i0 >> pl) << pl;
        sTop[pl] = (pl >= w.m && pl < nlev && ((i0 >> pl) & 1)) ? cum[j - 1] : 0.0;
    }
    __syncthreads();

    f32x4 acc[NSLOT][NRBW];
#pragma unroll
    for (int s = 0; s < NSLOT; ++s)
#pragma unroll
        for (int rb = 0; rb < NRBW; ++rb) acc[s][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Blocks of levels below m that end with chunk i: R(j) out in bf16, the
    // accumulator cleared (level p is idle for the next chunk, whose bit p is
    // clear).  Called one chunk late, before that chunk's copies are issued,
    // so that these stores are older than the copies the next wait is for.
    // Lane (m16, g) holds R[d0 + 16 rb + m16][c0 + 4g .. c0 + 4g + 3].
    auto flush = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int pl = 0; pl < NSLOT; ++pl) {
            if (pl < w.m && pl < nlev && ((i >> pl) & 1)) {
                const int j = (i >> pl) << pl;
                if (i + 1 == min(j + (1 << pl), N)) {
                    bf16_t* dst = rst + ((size_t)bh * N + j) * DK * DV;
#pragma unroll
                    for (int rb = 0; rb < NRBW; ++rb) {
                        *reinterpret_cast<bf16x4*>(dst + (size_t)(d0 + 16 * rb + m16) * DV + c0 + 4 * g) =
                            pack4(acc[pl][rb][0], acc[pl][rb][1], acc[pl][rb][2], acc[pl][rb][3]);
                        acc[pl][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
        }
    };

    // chunk il is in buffer c; il + 1 was issued before; il + 2 goes to
    // buffer n2 (that of chunk il - 1, which every wave has finished)
    auto body = [&](int il, const bf16_t* Qc, const bf16_t* Oc, const float* Lc, const float* ac,
                    bf16_t* Qn2, bf16_t* On2, float* Ln2, float* an2) __attribute__((always_inline)) {
        // this wave's copies of chunk il have landed (at least KMIN copies of
        // il + 1, issued after them, may still be in flight); after the
        // barrier every wave's have, and every wave is done with chunk il - 1
        if (il + 1 < ntl) wait_vm<KMIN>();
        else wait_vm<0>();
        __syncthreads();
        const int i = i0 + il;
        if (il > 0) flush(i - 1);
        if (il + 2 < ntl) issue(il + 2, Qn2, On2, Ln2, an2);
        const int nvalid = min(TC, T - i * TC);
        {
            // wave pl: the weights of level pl for the chunk's 64 tokens,
            // lambda_t^(log2 C + pl + 1) e^(A_t - A(end of chunk j - 1))
            const int pl = wave;
            const float x = wave_inclusive_sum(ac[lane]);  // A_t - A(end of chunk i - 1)
            if (pl < NSLOT && pl < nlev && ((i >> pl) & 1)) {
                const int j = (i >> pl) << pl;
                const double cj = pl < w.m ? sCum[j - i0] : sTop[pl];
                const float base = (float)(sCum[i - i0] - cj);
                const float lam = Lc[lane * L + kRwLogC + pl + 1];
                sW[pl][lane] = lane < nvalid ? lam * __expf(x + base) : 0.f;
            }
        }
        __syncthreads();  // the weights
        // per 32-token half: the operands shared by every level, dO^T (this
        // wave's columns) and q^T (its d_k rows), then each level's products
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 ao = ld_tr8<DV>(Oc, 32 * ks, c0);
            bf16x8 bq[NRBW];
#pragma unroll
            for (int rb = 0; rb < NRBW; ++rb) bq[rb] = ld_tr8<DK>(Qc, 32 * ks, d0 + 16 * rb);
#pragma unroll
            for (int pl = 0; pl < NSLOT; ++pl) {
                if (pl < nlev && ((i >> pl) & 1)) {
                    const float4 w0 = *reinterpret_cast<const float4*>(&sW[pl][32 * ks + 8 * g]);
                    const float4 w1 = *reinterpret_cast<const float4*>(&sW[pl][32 * ks + 8 * g + 4]);
                    const bf16x8 sc = scale8(ao, w0, w1);
#pragma unroll
                    for (int rb = 0; rb < NRBW; ++rb) acc[pl][rb] = mma(sc, bq[rb], acc[pl][rb]);
                }
            }
        }
    };

    issue(0, sQ0, sO0, sL0, sa0);
    if (ntl > 1) issue(1, sQ1, sO1, sL1, sa1);
    for (int il = 0; il < ntl; il += 3) {
        body(il, sQ0, sO0, sL0, sa0, sQ2, sO2, sL2, sa2);
        if (il + 1 < ntl) body(il + 1, sQ1, sO1, sL1, sa1, sQ0, sO0, sL0, sa0);
        if (il + 2 < ntl) body(il + 2, sQ2, sO2, sL2, sa2, sQ1, sO1, sL1, sa1);
    }
    flush(i0 + ntl - 1);
    // this segment's parts of the blocks of levels >= m that it belongs to
#pragma unroll
    for (int pl = 0; pl < NSLOT; ++pl) {
        if (pl >= w.m && pl < nlev && ((i0 >> pl) & 1)) {
            float* dst = w.part + (((size_t)bh * w.nseg + seg) * w.ntop + (pl - w.m)) * DK * DV;
#pragma unroll
            for (int rb = 0; rb < NRBW; ++rb)
                *reinterpret_cast<f32x4*>(dst + (size_t)(d0 + 16 * rb + m16) * DV + c0 + 4 * g) = acc[pl][rb];
        }
    }
}

// R(j) of the blocks of levels p >= m: the sum of the parts of the segments
// the block covers (all taken relative to the block's start), in bf16.
// One block of 256 threads per (batch*head, such j).
template <int DK, int DV>
__global__ __launch_bounds__(256) void k_bwd_rcombine(BwdParams p, RwalkArgs w) {
    int x = blockIdx.x, lev = -1, j = 0, bh = 0;
    for (int pp = w.m; pp < p.nlev; ++pp) {
        const int first = 1 << pp;
        const int cnt = first < p.N ? (p.N - 1 - first) / (2 << pp) + 1 : 0;
        if (x < cnt * p.BH) {
            bh = x % p.BH;
            j = (x / p.BH) * (2 << pp) + first;
            lev = pp;
            break;
        }
        x -= cnt * p.BH;
    }
    if (lev < 0) return;
    const int s0 = j >> w.m;
    const int s1 = min(s0 + (1 << (lev - w.m)), w.nseg);
    constexpr int NE = DK * DV / 4;  // float4 elements of a state
    const float4* src = reinterpret_cast<const float4*>(w.part);
    bf16_t* dst = reinterpret_cast<bf16_t*>(p.rst16) + ((size_t)bh * p.N + j) * DK * DV;
    for (int e = threadIdx.x; e < NE; e += 256) {
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sg = s0; sg < s1; ++sg) {
            const float4 y = src[(((size_t)bh * w.nseg + sg) * w.ntop + (lev - w.m)) * NE + e];
            s.x += y.x;
            s.y += y.y;
            s.z += y.z;
            s.w += y.w;
        }
        *reinterpret_cast<bf16x4*>(dst + 4 * (size_t)e) = pack4(s.x, s.y, s.z, s.w);
    }
}

template <int DK>
hipError_t launch_rwalk_dk(const BwdParams& p, const RwalkArgs& w, hipStream_t stream) {
    if (p.nlev <= 7)
        hipLaunchKernelGGL((k_bwd_rwalk<DK, 64, 7>), dim3(p.BH * w.nseg), dim3(kRwWaves * 64), 0, stream, p, w);
    else
        hipLaunchKernelGGL((k_bwd_rwalk<DK, 64, 8>), dim3(p.BH * w.nseg), dim3(kRwWaves * 64), 0, stream, p, w);
    if (w.ntop > 0) {
        long nj = 0;
        for (int pp = w.m; pp < p.nlev; ++pp) {
            const int first = 1 << pp;
            if (first < p.N) nj += (p.N - 1 - first) / (2 << pp) + 1;
        }
        if (nj > 0)
            hipLaunchKernelGGL((k_bwd_rcombine<DK, 64>), dim3((unsigned)(nj * p.BH)), dim3(256), 0, stream, p, w);
    }
    return hipGetLastError();
}

}  // namespace

namespace {
bool rwalk_plan(const BwdParams& p, RwalkArgs& w) {
    if (p.C != 64 || p.dv != 64 || (p.dk != 64 && p.dk != 128)) return false;
    if (p.N < 2 || p.nlev > kRwSlots || p.L > kRwMaxL || p.L < kRwLogC + p.nlev + 1) return false;
    // segments of 32 chunks; shorter ones where that leaves under 256 blocks
    // and the parts still fit their region (nseg ntop <= N)
    auto nseg_of = [&](int m) { return (p.N + (1 << m) - 1) >> m; };
    auto ntop_of = [&](int m) { return p.nlev > m ? p.nlev - m : 0; };
    w.m = kRwMaxM;
    while (w.m > 2 && (long)p.BH * nseg_of(w.m) < 256 &&
           (long)nseg_of(w.m - 1) * ntop_of(w.m - 1) <= p.N)
        --w.m;
    w.nseg = nseg_of(w.m);
    w.ntop = ntop_of(w.m);
    if ((long)w.nseg * w.ntop > p.N) return false;
    // the parts go to the fp32-sized region that held the bf16 nodes of the
    // dq kernel (launched before this one; nothing after it reads them)
    w.part = p.rstT;
    w.lam_dma = ((long)p.T * p.L) % 4 == 0 && reinterpret_cast<uintptr_t>(p.lam) % 16 == 0;
    w.a_dma = p.T % 4 == 0 && reinterpret_cast<uintptr_t>(p.a) % 16 == 0;
    return true;
}
}  // namespace

bool bwd_rwalk_applies(const BwdParams& p) {
    RwalkArgs w{};
    return rwalk_plan(p, w);
}

hipError_t launch_bwd_rwalk(const BwdParams& p, hipStream_t stream) {
    RwalkArgs w{};
    if (!rwalk_plan(p, w)) return hipErrorInvalidValue;
    return p.dk == 128 ? launch_rwalk_dk<128>(p, w, stream) : launch_rwalk_dk<64>(p, w, stream);
}

}  // namespace loglin
