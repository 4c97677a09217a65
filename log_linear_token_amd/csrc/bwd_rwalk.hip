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
constexpr int kRwCoarse = 2;  // slots of the walk that builds only the levels spanning segments

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
    int pmin;       // levels p < pmin are not built (0, or m when the dk / dv
                    // walk builds the levels inside a segment itself)
    int pm, pnseg, pntop;  // the dk / dv walk: segment log2, count and levels of the
                           // parts the R(j) walk left (its m, nseg, ntop)
    int lam_dma;    // lambda rows of a whole chunk are 16-byte aligned
    int a_dma;      // a of a whole chunk is 16-byte aligned
    float* part;    // [BH][nseg][ntop][dk][dv] parts of the blocks of levels >= m
                    // (nseg ntop <= N: within an fp32 [BH][N][dk][dv] region)
};

// NSLOT: levels p < NSLOT (at most 2^NSLOT chunks); NB chunk buffers: three
// (chunks il + 1 and il + 2 in flight while il is used, one block per compute
// unit) or two (il + 1 in flight; 65 KB, so that two blocks share a compute
// unit: the walk that builds only the blocks spanning segments runs twice
// as many shorter segments)
// COARSE: only the levels p >= pmin, all of which span segments (pmin > m):
// slot s accumulates level pmin + s, whose set bits are those of the
// segment's first chunk for all its chunks; with NSLOT = 2 slots the
// accumulators fit two blocks per compute unit (four waves per SIMD, the
// second launch bound).
template <int DK, int DV, int NSLOT, int NB, bool COARSE>
__global__ __launch_bounds__(kRwWaves * 64, COARSE ? 4 : 1) void k_bwd_rwalk(BwdParams p, RwalkArgs w) {
    static_assert(DV == 64 && (DK == 64 || DK == 128), "head dims of this kernel");
    static_assert(NSLOT <= kRwSlots, "one wave per level for the weights");
    static_assert(NB == 2 || NB == 3, "chunk buffers");
    auto lvl = [&](int s) __attribute__((always_inline)) { return COARSE ? w.pmin + s : s; };
    constexpr int NRBW = DK / 32;  // 16-row blocks of d_k per wave
    __shared__ __align__(16) bf16_t sQ[NB][TC * DK];
    __shared__ __align__(16) bf16_t sO[NB][TC * DV];
    __shared__ __align__(16) float sL[NB][TC * kRwMaxL];
    __shared__ __align__(16) float sa[NB][TC];
    __shared__ __align__(16) float sW[kRwSlots][TC];  // per-token weights of each level
    // A at the end of chunks i0 - 1 .. i0 + 2^m - 1 (sCum[k]: chunk i0 - 1 + k),
    // and at the end of chunk j - 1 for the blocks of levels >= m
    __shared__ double sCum[(1 << kRwMaxM) + 1];
    __shared__ double sTop[kRwSlots];

    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int seg = blk % w.nseg;
    const int bh = blk / w.nseg;
    // levels pmin <= p < nlev only: a segment none of whose chunks has such a
    // bit set (for p >= m: the segment index has none) has nothing to build
    {
        const int i0s = seg << w.m;
        const int top = (1 << p.nlev) - 1;
        const int low = w.pmin < w.m ? ((1 << w.m) - 1) & ~((1 << w.pmin) - 1) : 0;
        if (((i0s & top) >> w.pmin) == 0 && low == 0) return;
    }
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
    if (threadIdx.x < kRwSlots) {
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
        if constexpr (COARSE) return;
#pragma unroll
        for (int pl = 0; pl < NSLOT; ++pl) {
            if (pl >= w.pmin && pl < w.m && pl < nlev && ((i >> pl) & 1)) {
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
        if constexpr (NB == 3) {
            if (il + 1 < ntl) wait_vm<KMIN>();
            else wait_vm<0>();
        } else {
            wait_vm<0>();
        }
        __syncthreads();
        const int i = i0 + il;
        if (il > 0) flush(i - 1);
        // the next copies go to the buffer every wave has finished with: that
        // of chunk il - 1 (three buffers: chunk il + 2; two: chunk il + 1)
        if (il + NB - 1 < ntl) issue(il + NB - 1, Qn2, On2, Ln2, an2);
        const int nvalid = min(TC, T - i * TC);
        {
            // wave pl: the weights of level pl for the chunk's 64 tokens,
            // lambda_t^(log2 C + pl + 1) e^(A_t - A(end of chunk j - 1))
            const int pl = wave, lv = lvl(pl);
            const float x = wave_inclusive_sum(ac[lane]);  // A_t - A(end of chunk i - 1)
            if (pl < NSLOT && lv >= w.pmin && lv < nlev && ((i >> lv) & 1)) {
                const int j = (i >> lv) << lv;
                const double cj = lv < w.m ? sCum[j - i0] : sTop[lv];
                const float base = (float)(sCum[i - i0] - cj);
                const float lam = Lc[lane * L + kRwLogC + lv + 1];
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
                const int lv = lvl(pl);
                if (lv >= w.pmin && lv < nlev && ((i >> lv) & 1)) {
                    const float4 w0 = *reinterpret_cast<const float4*>(&sW[pl][32 * ks + 8 * g]);
                    const float4 w1 = *reinterpret_cast<const float4*>(&sW[pl][32 * ks + 8 * g + 4]);
                    const bf16x8 sc = scale8(ao, w0, w1);
#pragma unroll
                    for (int rb = 0; rb < NRBW; ++rb) acc[pl][rb] = mma(sc, bq[rb], acc[pl][rb]);
                }
            }
        }
    };

    if constexpr (NB == 3) {
        issue(0, sQ[0], sO[0], sL[0], sa[0]);
        if (ntl > 1) issue(1, sQ[1], sO[1], sL[1], sa[1]);
        for (int il = 0; il < ntl; il += 3) {
            body(il, sQ[0], sO[0], sL[0], sa[0], sQ[NB - 1], sO[NB - 1], sL[NB - 1], sa[NB - 1]);
            if (il + 1 < ntl) body(il + 1, sQ[1], sO[1], sL[1], sa[1], sQ[0], sO[0], sL[0], sa[0]);
            if (il + 2 < ntl)
                body(il + 2, sQ[NB - 1], sO[NB - 1], sL[NB - 1], sa[NB - 1], sQ[1], sO[1], sL[1], sa[1]);
        }
    } else {
        issue(0, sQ[0], sO[0], sL[0], sa[0]);
        for (int il = 0; il < ntl; il += 2) {
            body(il, sQ[0], sO[0], sL[0], sa[0], sQ[1], sO[1], sL[1], sa[1]);
            if (il + 1 < ntl) body(il + 1, sQ[1], sO[1], sL[1], sa[1], sQ[0], sO[0], sL[0], sa[0]);
        }
    }
    flush(i0 + ntl - 1);
    // this segment's parts of the blocks of levels >= m that it belongs to
#pragma unroll
    for (int pl = 0; pl < NSLOT; ++pl) {
        const int lv = lvl(pl);
        if (lv >= w.m && lv >= w.pmin && lv < nlev && ((i0 >> lv) & 1)) {
            float* dst = w.part + (((size_t)bh * w.nseg + seg) * w.ntop + (lv - w.m)) * DK * DV;
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

// ---------------------------------------------------------------------------
// dk, dv and k_s . dk_s in one reverse walk per (batch*head, segment of 2^m
// chunks) (bf16, 64-token chunks, d_k = 128, d_v = 64).
//
// Outside its own chunk i, key s meets the queries of the block of 2^p chunks
// starting at j_p = ((i >> p) | 1) << p for each clear bit p of i, with the
// block state R(j_p) of the R(j) walk above.  The key's side of the mask is a
// decay alone, e^(-A_s), so the blocks combine before the products:
//     dk_s += e^(A(end of i) - A_s) R~ v_s,   dv_s += e^(A(end of i) - A_s) R~^T k_s,
//     R~(i) = sum over the clear bits p of e^(A(end of j_p - 1) - A(end of i)) R(j_p),
// one pair of products per chunk whatever the number of blocks.  Walking the
// segment's chunks from its last to its first, a block of level p < m inside
// the segment is complete exactly when the walk reaches the 2^p chunks that
// read it (they come right before it), so these blocks accumulate in fp32
// registers as the walk passes their chunks: chunk i adds its queries to the
// level-p block for each set bit p of i, the accumulator cleared when the walk
// enters the next block of that level.  The blocks of levels p >= m lie in
// later segments; their R(j) come from the R(j) walk, combined once at the
// start with the weights e^(A(end of j - 1) - A(end of the segment)).
// The chunk's own causal block adds (dP (.) M)^T Q to dk and ((Q K^T) (.) M)^T dO
// to dv, with dP = dO v^T and M = lambda_t^(level) e^(A_t - A_s).
//
// Eight waves.  Wave w owns d_k columns 16 w .. 16 w + 15 of every block state
// and of dk (all 64 keys), and dv columns 16 (w % 4) for the keys 32 (w / 4)
// .. + 31.  The accumulated states are transposed (rows d_v, the dO operand
// read with free column quads) so that each lane's fp32 entries are the
// natural 8-wide d_v groups of the R~ operand of the dk product; the dv product
// reads R~ back from LDS by transpose reads.  Chunks arrive by LDS-DMA one
// ahead of use (two buffers); the results of a chunk are stored after the
// next chunk's barrier, before that chunk's successor is requested.

constexpr int kKvWaves = 8;
constexpr int kKvMaxL = 24;   // lambda row length staged per token

template <int DK, int DV>
__global__ __launch_bounds__(kKvWaves * 64, 1) void k_bwd_kvwalk(BwdParams p, RwalkArgs w) {
    static_assert(DK == 16 * kKvWaves && DV == 64, "head dims of this kernel");
    constexpr int MM = kRwMaxM;  // levels kept in registers: p < m <= MM
    static_assert(MM + 3 <= kKvWaves, "one wave per level weight");
    __shared__ __align__(16) bf16_t sQ[2][TC * DK];
    __shared__ __align__(16) bf16_t sK[2][TC * DK];
    __shared__ __align__(16) bf16_t sV[2][TC * DV];
    __shared__ __align__(16) bf16_t sO[2][TC * DV];
    __shared__ __align__(16) float sL[2][TC * kKvMaxL];
    __shared__ __align__(16) float sa[2][TC];
    __shared__ __align__(16) bf16_t sZ[TC * TC];   // (dP (.) M)^T: [key][query]
    __shared__ __align__(16) bf16_t sP[TC * TC];   // ((Q K^T) (.) M)^T
    __shared__ __align__(16) bf16_t sR[DK * DV];   // R~ of the chunk: [d_k][d_v]
    __shared__ __align__(16) float sW[MM][TC];     // query weights of the levels the chunk feeds
    __shared__ __align__(16) float sE[TC];         // e^(A(end of chunk) - A_s)
    __shared__ __align__(16) float sAw[kKvWaves][TC];  // per wave: A_t - A(end of the chunk before)
    __shared__ __align__(16) float sDa[2][kKvWaves][TC];  // per wave: its part of k_s . dk_s
    // per chunk of the segment: the weights of the blocks that make R~ (level
    // p, and the blocks after the segment at MM; zero where not used), and
    // the offsets A(end of chunk - 1) - A(end of block start - 1) of the query
    // weights of the blocks the chunk feeds
    __shared__ float sCw[1 << kRwMaxM][MM + 1];
    __shared__ float sBw[1 << kRwMaxM][MM];

    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int seg = blk % w.nseg;
    const int bh = blk / w.nseg;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
    const int N = p.N, L = p.L, T = p.T, nlev = p.nlev;
    const int i0 = seg << w.m;
    const int ntl = min(1 << w.m, N - i0);
    const int mm = min(w.m, nlev);
    const size_t row0 = (size_t)bh * T;
    const double* cum = p.cum + (size_t)bh * N;
    const bf16_t* q = reinterpret_cast<const bf16_t*>(p.q);
    const bf16_t* k = reinterpret_cast<const bf16_t*>(p.k);
    const bf16_t* v = reinterpret_cast<const bf16_t*>(p.v);
    const bf16_t* dout = reinterpret_cast<const bf16_t*>(p.dout);

    typedef TileCopy<DK, kKvWaves> CK;
    typedef TileCopy<DV, kKvWaves> CV;
    CK ck;
    CV cv;
    ck.init(DK, 0, wave);
    cv.init(DV, 0, wave);
    // chunk il of the segment into buffer b, in four parts (q; k; v and dO;
    // lambda and a) that the body issues between its computations, so that
    // the copies of the eight waves do not queue up at once; rows past T: q,
    // k, v and dO repeat the last row (their weights are zero or their
    // outputs unused), lambda and a are zero
    auto issue = [&](int il, int b, int part) __attribute__((always_inline)) {
        const int t0 = (i0 + il) * TC;
        const int nvalid = min(TC, T - t0);
        const size_t r = row0 + t0;
        if (part == 0) {
            if (nvalid == TC) ck.issue(q + r * DK, sQ[b], wave);
            else dma_tile<DK, kKvWaves>(q + r * DK, DK, 0, nvalid, sQ[b], wave);
        } else if (part == 1) {
            if (nvalid == TC) ck.issue(k + r * DK, sK[b], wave);
            else dma_tile<DK, kKvWaves>(k + r * DK, DK, 0, nvalid, sK[b], wave);
        } else if (part == 2) {
            if (nvalid == TC) {
                cv.issue(v + r * DV, sV[b], wave);
                cv.issue(dout + r * DV, sO[b], wave);
            } else {
                dma_tile<DV, kKvWaves>(v + r * DV, DV, 0, nvalid, sV[b], wave);
                dma_tile<DV, kKvWaves>(dout + r * DV, DV, 0, nvalid, sO[b], wave);
            }
        } else {
            float* Ld = sL[b];
            if (nvalid == TC && w.lam_dma) {
                const int nch = 16 * L;  // 64 rows x L floats in 16-byte pieces
                for (int u = wave; u * 64 < nch; u += kKvWaves)
                    if (u * 64 + lane < nch) dma16o(p.lam + r * L, 16u * (u * 64 + lane), Ld + u * 256);
            } else {
                const int nel = nvalid * L;
                for (int u = wave; u * 64 < TC * L; u += kKvWaves) {
                    const int x = u * 64 + lane;
                    if (x < nel) dma4(p.lam + r * L + x, Ld + u * 64);
                    else if (x < TC * L) Ld[x] = 0.f;
                }
            }
            if (wave == kKvWaves - 1) {
                if (nvalid == TC && w.a_dma) {
                    if (lane < TC / 4) dma16o(p.a + r, 16u * lane, sa[b]);
                } else if (lane < nvalid) {
                    dma4(p.a + r + lane, sa[b]);
                } else {
                    sa[b][lane] = 0.f;
                }
            }
        }
    };

    // the walk's first chunk (the segment's last) is requested before the
    // prologue's own loads, so that their latencies overlap
#pragma unroll
    for (int part = 0; part < 4; ++part) issue(ntl - 1, (ntl - 1) & 1, part);

    // the blocks of levels >= m after the segment, combined at its end: this
    // lane's share, d_k row 16 w + n16, d_v 32 ks + 8 g + (0..7).  Each such
    // block is the sum of the fp32 parts the R(j) walk left for the segments
    // it covers (all relative to the block's start).  Only a full segment that
    // is not the last has such blocks (A at the end of the sequence's last
    // chunk is never read).
    f32x4 nc[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) nc[ks][0] = nc[ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool coarse = false;
    for (int pl = w.m; pl < nlev; ++pl) {
        const int j = ((i0 >> pl) | 1) << pl;
        if (((i0 >> pl) & 1) || j >= N) continue;
        coarse = true;
        const float wt = __expf((float)(cum[j - 1] - cum[i0 + ntl - 1]));
        const int s0 = j >> w.pm, s1 = min(s0 + (1 << (pl - w.pm)), w.pnseg);
        // four parts' loads in flight at once (past the last part: the last
        // one again, weighted zero)
        for (int sb = s0; sb < s1; sb += 4) {
            f32x4 x[4][2][2];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int sg = min(sb + u, s1 - 1);
                const float* R = w.part + (((size_t)bh * w.pnseg + sg) * w.pntop + (pl - w.pm)) * DK * DV +
                                 (size_t)(16 * wave + n16) * DV + 8 * g;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    x[u][ks][0] = *reinterpret_cast<const f32x4*>(R + 32 * ks);
                    x[u][ks][1] = *reinterpret_cast<const f32x4*>(R + 32 * ks + 4);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float wu = sb + u < s1 ? wt : 0.f;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        nc[ks][0][e] += wu * x[u][ks][0][e];
                        nc[ks][1][e] += wu * x[u][ks][1][e];
                    }
            }
        }
    }

    for (int x = threadIdx.x; x < ntl * (MM + 1); x += kKvWaves * 64) {
        const int il = x / (MM + 1), pl = x - il * (MM + 1);
        float c = 0.f;
        if (pl == MM) {
            if (coarse) c = __expf((float)(cum[i0 + ntl - 1] - cum[i0 + il]));
        } else {
            const int jr = ((il >> pl) | 1) << pl;
            if (pl < mm && !((il >> pl) & 1) && jr < ntl)
                c = __expf((float)(cum[i0 + jr - 1] - cum[i0 + il]));
        }
        sCw[il][pl] = c;
    }
    for (int x = threadIdx.x; x < ntl * MM; x += kKvWaves * 64) {
        const int il = x / MM, pl = x - il * MM;
        const int jb = (il >> pl) << pl;
        const double ce = i0 + il >= 1 ? cum[i0 + il - 1] : 0.0;
        const double cb = i0 + jb >= 1 ? cum[i0 + jb - 1] : 0.0;
        sBw[il][pl] = (float)(ce - cb);
    }

    f32x4 acc[MM][2][2];
#pragma unroll
    for (int pl = 0; pl < MM; ++pl)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc[pl][ks][0] = acc[pl][ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // results of the chunk last computed, stored after the next barrier
    f32x4 dk4[4], dv2[2];
    const int vb = wave & 3;          // this wave's d_v block
    const int kb0 = 2 * (wave >> 2);  // and its first key block for dv

    // results of chunk il: dk rows of key block kb (this wave's 16 columns),
    // dv rows of its key block kb0 + jb, and k . dk (the last wave)
    auto store_dk = [&](int il, int kb, int zv) __attribute__((always_inline)) {
        const int n16 = (lane & 15) + zv, g = (lane >> 4) + zv;
        const int t0 = (i0 + il) * TC;
        const int s = 16 * kb + n16;
        float* gk = p.gk + (row0 + t0) * DK;  // uniform row base plus a 32-bit lane offset
        if (s < T - t0) *reinterpret_cast<f32x4*>(gk + (uint32_t)(s * DK + 16 * wave + 4 * g)) = dk4[kb];
    };
    auto store_dv = [&](int il, int jb, int zv) __attribute__((always_inline)) {
        const int n16 = (lane & 15) + zv, g = (lane >> 4) + zv;
        const int t0 = (i0 + il) * TC;
        const int s = 16 * (kb0 + jb) + n16;
        float* gv = p.gv + (row0 + t0) * DV;
        if (s < T - t0) *reinterpret_cast<f32x4*>(gv + (uint32_t)(s * DV + 16 * vb + 4 * g)) = dv2[jb];
    };
    auto store_da = [&](int il) __attribute__((always_inline)) {
        if (wave == kKvWaves - 1) {
            const int t0 = (i0 + il) * TC;
            float d = 0.f;
#pragma unroll
            for (int u = 0; u < kKvWaves; ++u) d += sDa[il & 1][u][lane];
            if (lane < T - t0) p.dA2[row0 + t0 + lane] = d;
        }
    };

    for (int il = ntl - 1; il >= 0; --il) {
        const int cur = il & 1;
        wait_vm<0>();
        __syncthreads();  // chunk il has landed; every wave is done with chunk il + 1
        // the lane indices through an opaque zero: the per-lane address
        // arithmetic of the body is then redone in place each chunk instead
        // of being hoisted out of the loop, where it would be held (or
        // spilled) beside the level accumulators
        int zv;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zv));
        const int n16 = (lane & 15) + zv, g = (lane >> 4) + zv;
        if (il > 0) issue(il - 1, cur ^ 1, 0);
        const bf16_t* Qs = sQ[cur];
        const bf16_t* Ks = sK[cur];
        const bf16_t* Vs = sV[cur];
        const bf16_t* Os = sO[cur];
        const float* Ls = sL[cur];
        const int nvalid = min(TC, T - (i0 + il) * TC);

        // this wave's copy of the chunk's decay: x_t = A_t - A(end of chunk il - 1)
        const float x = wave_inclusive_sum(sa[cur][lane]);
        const float xend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
        sAw[wave][lane] = x;
        // shared weights: e^(A(end) - A_s) (wave 2) and, wave 3 + p, the weights
        // of the queries of this chunk in the level-p block it belongs to
        if (wave == 2) {
            sE[lane] = __expf(xend - x);
        } else if (wave >= 3) {
            const int pl = wave - 3;
            if (pl < mm && ((il >> pl) & 1)) {
                const float base = sBw[il][pl];
                const float lam = Ls[lane * L + kRwLogC + pl + 1];
                sW[pl][lane] = lane < nvalid ? lam * __expf(x + base) : 0.f;
            }
        }

        // the causal block: 16 x 16 blocks (query block rb >= key block sb),
        // one or two per wave; lane (n16, g) holds query 16 rb + 4g + i, key 16 sb + n16
        auto score = [&](int tau) __attribute__((always_inline)) {
            const int rb = tau < 1 ? 0 : tau < 3 ? 1 : tau < 6 ? 2 : 3;
            const int sb = tau - rb * (rb + 1) / 2;
            bf16x8 of[2], vf[2], qf[4], kf[4];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                of[ks] = ld8<DV>(Os, 16 * rb + n16, 32 * ks + 8 * g);
                vf[ks] = ld8<DV>(Vs, 16 * sb + n16, 32 * ks + 8 * g);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                qf[ks] = ld8<DK>(Qs, 16 * rb + n16, 32 * ks + 8 * g);
                kf[ks] = ld8<DK>(Ks, 16 * sb + n16, 32 * ks + 8 * g);
            }
            const int s = 16 * sb + n16;
            const float As = sAw[wave][s];
            const float4 At = *reinterpret_cast<const float4*>(&sAw[wave][16 * rb + 4 * g]);
            __builtin_amdgcn_sched_barrier(0);
            f32x4 dp = {0.f, 0.f, 0.f, 0.f}, sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) dp = mma(of[ks], vf[ks], dp);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) sc = mma(qf[ks], kf[ks], sc);
            const float Atv[4] = {At.x, At.y, At.z, At.w};
            float z[4], pp[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * rb + 4 * g + i;
                const int lvl = sb < rb ? 5 + (31 - __builtin_clz(rb ^ sb)) : fenwick_level(t, s);
                const float wt = Ls[t * L + lvl] * __expf(Atv[i] - As);
                const bool keep = sb < rb || t >= s;
                z[i] = keep ? dp[i] * wt : 0.f;
                pp[i] = keep ? sc[i] * wt : 0.f;
            }
            *reinterpret_cast<bf16x4*>(sZ + toff<TC>(s, 16 * rb + 4 * g)) = pack4(z[0], z[1], z[2], z[3]);
            *reinterpret_cast<bf16x4*>(sP + toff<TC>(s, 16 * rb + 4 * g)) = pack4(pp[0], pp[1], pp[2], pp[3]);
            if (sb == rb && (rb & 1) == 0) {
                // the block past the diagonal (keys of block rb + 1, queries of
                // block rb), which the 32-query products pair with this one
                *reinterpret_cast<bf16x4*>(sZ + toff<TC>(s + 16, 16 * rb + 4 * g)) = bf16x4{};
                *reinterpret_cast<bf16x4*>(sP + toff<TC>(s + 16, 16 * rb + 4 * g)) = bf16x4{};
            }
        };
        if (il > 0) issue(il - 1, cur ^ 1, 1);
        score(wave);
        if (wave < 2) score(wave + 8);
        if (il > 0) issue(il - 1, cur ^ 1, 2);

        // R~ share of this wave (d_k row 16 w + n16, d_v 32 ks + 8 g + 0..7):
        // operand of the dk product in registers, and to LDS for the dv product
        bf16x8 rf[2];
        {
            const float wc = sCw[il][MM];
            f32x4 r[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h) r[ks][h] = wc * nc[ks][h];
#pragma unroll
            for (int pl = 0; pl < MM; ++pl) {
                const int jr = ((il >> pl) | 1) << pl;
                if (pl < mm && !((il >> pl) & 1) && jr < ntl) {
                    const float c = sCw[il][pl];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int h = 0; h < 2; ++h) r[ks][h] += c * acc[pl][ks][h];
                }
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                rf[ks] = cvt8(r[ks][0], r[ks][1]);
                *reinterpret_cast<bf16x8*>(sR + toff<DV>(16 * wave + n16, 32 * ks + 8 * g)) = rf[ks];
            }
        }
        if (il > 0) issue(il - 1, cur ^ 1, 3);
        __syncthreads();  // the chunk's weights, (dP (.) M)^T, ((Q K^T) (.) M)^T and R~
        // the previous chunk's results go out block by block between this
        // chunk's products (each right before its registers are reused)
        const bool prev = il + 1 < ntl;
        if (prev) store_da(il + 1);

        // dk^T (rows d_k 16 w + 4g + i, column key 16 kb + n16): the causal
        // block, then e^(A(end) - A_s) R~ v_s
        bf16x8 qT[2];
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) qT[sp] = ld_tr8<DK>(Qs, 32 * sp + zv, 16 * wave);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (prev) store_dk(il + 1, kb, zv);
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sp = 0; sp < 2; ++sp)
                if (kb < 2 || sp == 1) a = mma(qT[sp], ld8<TC>(sZ, 16 * kb + n16, 32 * sp + 8 * g), a);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) t = mma(rf[ks], ld8<DV>(Vs, 16 * kb + n16, 32 * ks + 8 * g), t);
            const float e = sE[16 * kb + n16];
#pragma unroll
            for (int i = 0; i < 4; ++i) dk4[kb][i] = a[i] + e * t[i];
            // one key block's operands in registers at a time
            __builtin_amdgcn_sched_barrier(0);
        }
        // dv^T (rows d_v 16 vb + 4g + i, column key 16 kb + n16) for two key blocks
        {
            bf16x8 oT[2], rT[4];
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) oT[sp] = ld_tr8<DV>(Os, 32 * sp + zv, 16 * vb);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) rT[ks] = ld_tr8<DV>(sR, 32 * ks + zv, 16 * vb);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                if (prev) store_dv(il + 1, jb, zv);
                const int kb = kb0 + jb;
                f32x4 a = {0.f, 0.f, 0.f, 0.f}, t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sp = 0; sp < 2; ++sp)
                    if (kb < 2 || sp == 1) a = mma(oT[sp], ld8<TC>(sP, 16 * kb + n16, 32 * sp + 8 * g), a);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) t = mma(rT[ks], ld8<DK>(Ks, 16 * kb + n16, 32 * ks + 8 * g), t);
                const float e = sE[16 * kb + n16];
#pragma unroll
                for (int i = 0; i < 4; ++i) dv2[jb][i] = a[i] + e * t[i];
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // this wave's part of k_s . dk_s (its 16 d_k columns), summed over the
        // lane rows: lane 16 g + n16 gets key 16 g + n16
        {
            float xk[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x4 kk = ld4<DK>(Ks, 16 * kb + n16, 16 * wave + 4 * g);
                xk[kb] = (float)kk[0] * dk4[kb][0] + (float)kk[1] * dk4[kb][1] +
                         (float)kk[2] * dk4[kb][2] + (float)kk[3] * dk4[kb][3];
            }
            sDa[il & 1][wave][lane] = sum_rows4_x4(xk[0], xk[1], xk[2], xk[3]);
        }

        // the chunk's queries into the blocks it belongs to (set bits p < m):
        // R^T[d_v][d_k] += dO^T diag(weights) Q, d_v rows in column quads
#pragma unroll
        for (int pl = 0; pl < MM; ++pl) {
            if (pl < mm && ((il >> pl) & 1) && (((il + 1) & ((2 << pl) - 1)) == 0)) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) acc[pl][ks][0] = acc[pl][ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            bf16x8 oq[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h) oq[ks][h] = ld_tr8_q<DV>(Os, 32 * sp + zv, 32 * ks + 4 * h);
#pragma unroll
            for (int pl = 0; pl < MM; ++pl) {
                if (pl < mm && ((il >> pl) & 1)) {
                    const float4 w0 = *reinterpret_cast<const float4*>(&sW[pl][32 * sp + 8 * g]);
                    const float4 w1 = *reinterpret_cast<const float4*>(&sW[pl][32 * sp + 8 * g + 4]);
                    const bf16x8 bs = scale8(qT[sp], w0, w1);
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int h = 0; h < 2; ++h) acc[pl][ks][h] = mma(oq[ks][h], bs, acc[pl][ks][h]);
                }
            }
        }
    }
    __syncthreads();  // the last chunk's k . dk parts
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) store_dk(0, kb, 0);
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) store_dv(0, jb, 0);
    store_da(0);
}

bool kvwalk_applies(const BwdParams& p, const RwalkArgs& w) {
    return p.dk == 16 * kKvWaves && p.dv == 64 && p.L <= kKvMaxL && w.m <= kRwMaxM;
}

template <int DK>
hipError_t launch_rwalk_dk(const BwdParams& p, const RwalkArgs& w, hipStream_t stream) {
    if (w.pmin > w.m)  // the spanning levels alone, segments shorter than the dk / dv walk's
        hipLaunchKernelGGL((k_bwd_rwalk<DK, 64, kRwCoarse, 2, true>), dim3(p.BH * w.nseg), dim3(kRwWaves * 64),
                           0, stream, p, w);
    else if (p.nlev <= 7)
        hipLaunchKernelGGL((k_bwd_rwalk<DK, 64, 7, 3, false>), dim3(p.BH * w.nseg), dim3(kRwWaves * 64), 0,
                           stream, p, w);
    else
        hipLaunchKernelGGL((k_bwd_rwalk<DK, 64, 8, 3, false>), dim3(p.BH * w.nseg), dim3(kRwWaves * 64), 0,
                           stream, p, w);
    // (with pmin = m the dk / dv walk sums the parts of the blocks itself)
    if (w.ntop > 0 && w.pmin < w.m) {
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

// The R(j) walk that leaves only the parts of the blocks of levels >= m of
// the dk / dv walk (w: that walk's plan): segments of 2^(m-1) chunks where
// those levels fit the coarse kernel's slots and the parts their region (two
// blocks per compute unit, twice the blocks), else the dk / dv walk's own.
RwalkArgs coarse_plan(const BwdParams& p, const RwalkArgs& w) {
    RwalkArgs r = w;
    r.pmin = w.m;
    const int mr = w.m - 1;
    if (mr >= 2 && p.nlev - w.m <= kRwCoarse) {
        const int nseg = (p.N + (1 << mr) - 1) >> mr;
        const int ntop = p.nlev - mr;
        if ((long)nseg * ntop <= p.N) {
            r.m = mr;
            r.nseg = nseg;
            r.ntop = ntop;
        }
    }
    return r;
}

bool bwd_rwalk_applies(const BwdParams& p) {
    RwalkArgs w{};
    return rwalk_plan(p, w);
}

bool bwd_kvwalk_applies(const BwdParams& p) {
    RwalkArgs w{};
    return rwalk_plan(p, w) && kvwalk_applies(p, w);
}

hipError_t launch_bwd_rwalk(const BwdParams& p, bool coarse_only, hipStream_t stream) {
    RwalkArgs w{};
    if (!rwalk_plan(p, w)) return hipErrorInvalidValue;
    w.pmin = 0;
    if (coarse_only) w = coarse_plan(p, w);
    return p.dk == 128 ? launch_rwalk_dk<128>(p, w, stream) : launch_rwalk_dk<64>(p, w, stream);
}

hipError_t launch_bwd_kvwalk(const BwdParams& p, hipStream_t stream) {
    RwalkArgs w{};
    if (!rwalk_plan(p, w) || !kvwalk_applies(p, w)) return hipErrorInvalidValue;
    const RwalkArgs r = coarse_plan(p, w);
    w.pm = r.m;
    w.pnseg = r.nseg;
    w.pntop = r.ntop;
    hipLaunchKernelGGL((k_bwd_kvwalk<128, 64>), dim3(p.BH * w.nseg), dim3(kKvWaves * 64), 0, stream, p, w);
    return hipGetLastError();
}

}  // namespace loglin
