// Fused chunked forward of the log-linear token mixer for bf16 inputs (gfx950).
//
// The chunked form of "Log-linear attention, and what a logarithm buys"
// (section 3) evaluated with the Fenwick states held in registers.  The
// sequence is cut into 64-token tiles and the tiles into segments of 2^m
// tiles; one block walks the tiles of one segment in order and, per tile,
//   - the intra-tile block: S^T = K Q^T on MFMA, weighted in registers by
//     lambda_t^(level(t,s)) e^(A_t - A_s) for s <= t, stored to LDS as bf16 P,
//     then O^T = V^T P^T on MFMA;
//   - the levels above the tile: for each set bit of the tile index a state G
//     holding the decayed sum of k v^T over the matching block of earlier
//     tiles, read as G^T Q^T on MFMA and weighted per row by
//     lambda_t^(level) e^(A_t - A_end(block));
//   - the tile's own state U = K^T diag(e^(A_end - A_s)) V (MFMA), folded by
//     the Fenwick update of section 2, run over tiles, together with the
//     levels below lssb(tile + 1) into the next level.
// Levels inside the segment live in registers as bf16 MFMA operands; the
// Fenwick merge that builds a level sums in fp32 (tile state, decayed lower
// levels) and rounds the result once.
// The levels above the segment are the same for all of its tiles; a
// segment-state kernel (k_seg_state) and the Fenwick scan over segments
// (fenwick_scan in fwd_chunked.hip) provide them as bf16 MFMA operand
// fragments, which the main kernel loads into registers once per block.
//
// Data movement: Q, K, V (and lambda, a where aligned) of the next tile are
// copied global -> LDS by the LDS-DMA path (global_load_lds_dwordx4) while the
// current tile is computed (two buffers, kept in distinct __shared__ arrays so
// that the compiler's alias analysis does not serialise the copies).  Tiles
// are stored row-major with an XOR swizzle of their 16-byte chunks; operands
// that contract over tokens (V^T for P V, K^T and V for the tile state) are
// read with the LDS transpose read (ds_read_b64_tr_b16), so no transposed
// copy is ever written.
//
// Two waves own 16 columns of d_v (for d_k >= 64; one wave otherwise): each
// holds half of the head dimension of every level state, contracts over it,
// and the halves of the level products are summed through LDS.

#include "tile_ops.hpp"

namespace loglin {

static_assert(sizeof(bf16_t_storage) == sizeof(bf16_t), "bf16 storage");

namespace {

// One 16 x 16 block of masked, weighted scores (rows 16 rb.., keys 16 sb..) to
// the P tile as bf16.  The diagonal block of an even row block also writes the
// block past the diagonal, which the K=32 P V product pairs with it, as zeros.
template <int DK>
__device__ __forceinline__ void score_block(int rb, int sb, const bf16_t* Qs, const bf16_t* Ks,
                                            bf16_t* Ps, const float* Aw, const float* lam_s,
                                            int L) {
    typedef HD<DK> H;
    const int lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
    const int t = 16 * rb + m16;
    // every LDS read of the block is issued before the first product, so
    // their latencies overlap instead of adding up
    typename H::frag kf[H::NKS], qf[H::NKS];
#pragma unroll
    for (int ks = 0; ks < H::NKS; ++ks) {
        if constexpr (DK >= 32) {
            kf[ks] = ld8<DK>(Ks, 16 * sb + m16, ks * 32 + 8 * g);
            qf[ks] = ld8<DK>(Qs, t, ks * 32 + 8 * g);
        } else {
            kf[ks] = ld4<DK>(Ks, 16 * sb + m16, 4 * g);
            qf[ks] = ld4<DK>(Qs, t, 4 * g);
        }
    }
    const float* lam_t = lam_s + t * L;  // levels inside a tile are < L (see the host checks)
    const float At = Aw[t];
    const float4 As = *reinterpret_cast<const float4*>(Aw + 16 * sb + 4 * g);
    float lam[4];
    if (sb < rb) {
        // every key of an earlier 16-block differs from t first in bit
        // 4 + floor(log2(rb ^ sb)): one level for the whole block
        lam[0] = lam[1] = lam[2] = lam[3] = lam_t[5 + (31 - __builtin_clz(rb ^ sb))];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[i] = lam_t[fenwick_level(t, 16 * sb + 4 * g + i)];
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < H::NKS; ++ks) acc = mma(kf[ks], qf[ks], acc);
    const float Asv[4] = {As.x, As.y, As.z, As.w};
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // diagonal block: causal mask by selection (the masked entries'
        // values are discarded whatever they are)
        const float x = acc[i] * lam[i] * __expf(At - Asv[i]);
        w[i] = (sb < rb || 16 * sb + 4 * g + i <= t) ? x : 0.f;
    }
    *reinterpret_cast<bf16x4*>(Ps + t * PROW + 16 * sb + 4 * g) = pack4(w[0], w[1], w[2], w[3]);
    if (sb == rb && (rb & 1) == 0)
        *reinterpret_cast<bf16x4*>(Ps + t * PROW + 16 * (rb + 1) + 4 * g) = bf16x4{};
}

// The dq pass of the backward runs this kernel with the operands swapped
// (queries dO, keys v, values k: dq = ((dO v^T) (.) M) k) and needs, besides
// the weighted block, the gradient of lambda: for the levels inside the tile
//   dlambda_t^(l) = sum over the keys s of level l of dP[t, s] S[t, s] e^(A_t - A_s)
// with dP = dO v^T (the block's unweighted scores) and S = q k^T.  S is taken
// over this column block's 64 columns of q and k only (k is the staged value
// tile, q the extra tile Qo); the column blocks' partial sums add up.  Row
// sums per level go to LDS: sDi[tau][row] for the blocks below the diagonal
// (one level each), sDd[rb][level][row] for the diagonal blocks (levels 0..4).
template <int DK, int DVW>
__device__ __forceinline__ void score_block_bwd(int rb, int sb, const bf16_t* Qs, const bf16_t* Ks,
                                                const bf16_t* Qo, const bf16_t* Vs, bf16_t* Ps,
                                                const float* Aw, const float* lam_s, int L,
                                                float* sDi, float* sDd) {
    typedef HD<DK> H;
    const int lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
    const int t = 16 * rb + m16;
    typename H::frag kf[H::NKS], qf[H::NKS];
#pragma unroll
    for (int ks = 0; ks < H::NKS; ++ks) {
        kf[ks] = ld8<DK>(Ks, 16 * sb + m16, ks * 32 + 8 * g);
        qf[ks] = ld8<DK>(Qs, t, ks * 32 + 8 * g);
    }
    bf16x8 kf2[DVW / 32], qf2[DVW / 32];
#pragma unroll
    for (int ks = 0; ks < DVW / 32; ++ks) {
        kf2[ks] = ld8<DVW>(Vs, 16 * sb + m16, ks * 32 + 8 * g);
        qf2[ks] = ld8<DVW>(Qo, t, ks * 32 + 8 * g);
    }
    const float* lam_t = lam_s + t * L;
    const float At = Aw[t];
    const float4 As = *reinterpret_cast<const float4*>(Aw + 16 * sb + 4 * g);
    int lev[4];
    if (sb < rb) {
        lev[0] = lev[1] = lev[2] = lev[3] = 5 + (31 - __builtin_clz(rb ^ sb));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) lev[i] = fenwick_level(t, 16 * sb + 4 * g + i);
    }
    float lam[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lam[i] = lam_t[lev[i]];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < H::NKS; ++ks) acc = mma(kf[ks], qf[ks], acc);
#pragma unroll
    for (int ks = 0; ks < DVW / 32; ++ks) acc2 = mma(kf2[ks], qf2[ks], acc2);
    const float Asv[4] = {As.x, As.y, As.z, As.w};
    float w[4], xd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool keep = sb < rb || 16 * sb + 4 * g + i <= t;
        const float e = __expf(At - Asv[i]);
        w[i] = keep ? acc[i] * lam[i] * e : 0.f;
        xd[i] = keep ? acc[i] * acc2[i] * e : 0.f;
    }
    *reinterpret_cast<bf16x4*>(Ps + t * PROW + 16 * sb + 4 * g) = pack4(w[0], w[1], w[2], w[3]);
    if (sb == rb && (rb & 1) == 0)
        *reinterpret_cast<bf16x4*>(Ps + t * PROW + 16 * (rb + 1) + 4 * g) = bf16x4{};
    if (sb < rb) {
        const float v = sum_rows4(xd[0] + xd[1] + xd[2] + xd[3]);
        if (g == 0) sDi[(rb * (rb + 1) / 2 + sb) * 16 + m16] = v;
    } else {
        // levels 0..4 of the diagonal block: 0..3 in one four-way row
        // reduction (lane (m16, g) ends with level g of token m16), 4 alone
        float x[5];
#pragma unroll
        for (int l = 0; l < 5; ++l) {
            x[l] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[l] += lev[i] == l ? xd[i] : 0.f;
        }
        sDd[(rb * 5 + g) * 16 + m16] = sum_rows4_x4(x[0], x[1], x[2], x[3]);
        const float v4 = sum_rows4(x[4]);
        if (g == 0) sDd[(rb * 5 + 4) * 16 + m16] = v4;
    }
}

// The ten causal 16 x 16 score blocks of a tile.  With eight waves, waves
// 0 and 1 take three blocks, waves 2 and 3 two and waves 4-7 none (those make
// the tile copies and the output stores); otherwise, and in the dq pass (whose
// blocks carry a second product and the dlambda sums), they are dealt
// round-robin.
template <int DK, int NWT, bool BWD = false, int DVW = 64>
__device__ __forceinline__ void scores_for_wave(int wave, const bf16_t* Qs, const bf16_t* Ks,
                                                bf16_t* Ps, const float* Aw, const float* lam_s,
                                                int L, const bf16_t* Qo = nullptr,
                                                const bf16_t* Vs = nullptr, float* sDi = nullptr,
                                                float* sDd = nullptr) {
    auto block = [&](int tau) __attribute__((always_inline)) {
        const int rb = tau < 1 ? 0 : tau < 3 ? 1 : tau < 6 ? 2 : 3;
        if constexpr (BWD)
            score_block_bwd<DK, DVW>(rb, tau - rb * (rb + 1) / 2, Qs, Ks, Qo, Vs, Ps, Aw, lam_s, L, sDi, sDd);
        else
            score_block<DK>(rb, tau - rb * (rb + 1) / 2, Qs, Ks, Ps, Aw, lam_s, L);
    };
    if constexpr (NWT == 8 && !BWD) {
        // one loop (a single call site): waves 0-3 take tau = w, w + 4 and
        // waves 0 and 1 also w + 8
        const int t1 = wave < 2 ? wave + 12 : wave < 4 ? wave + 8 : 0;
        for (int tau = wave; tau < t1; tau += 4) block(tau);
    } else if constexpr (NWT == 8 && BWD && DVW == 64) {
        // the diagonal blocks (tau 0, 2, 5, 9: five levels of dlambda sums)
        // cost about twice the others: one each for waves 2-5, which also
        // issue copies; waves 0 and 1 (no copies) take two of the others
        // (1, 3 and 4, 6), waves 6 and 7 one (7, 8)
        constexpr unsigned kFirst = 0x87952041u;   // 4 bits per wave
        constexpr unsigned kSecond = 0x63u;
        const int n = wave < 2 ? 2 : 1;
#pragma unroll 1  // one call site of the block (unrolled, the two copies spill)
        for (int x = 0; x < n; ++x) block((int)(((x ? kSecond : kFirst) >> (4 * wave)) & 15u));
    } else {
        for (int tau = wave; tau < NRB * (NRB + 1) / 2; tau += NWT) block(tau);
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Segment states: for each (bh, segment except the last, column block) the
// decayed sum of k v^T over the segment, fp32 [d_v][d_k] at the segment's end
// (TR: stored as [d_k][d_v], the state of the problem with k and v swapped).

template <int DK, int NW, bool TR = false>
__global__ __launch_bounds__(NW * 64) void k_seg_state(FusedParams p) {
    constexpr int DVW = NW * 16;
    constexpr int NDT = DK / 16;
    __shared__ __align__(16) bf16_t sK0[TC * DK];
    __shared__ __align__(16) bf16_t sK1[TC * DK];
    __shared__ __align__(16) bf16_t sV0[TC * DVW];
    __shared__ __align__(16) bf16_t sV1[TC * DVW];
    __shared__ __align__(16) float sa0[TC];
    __shared__ __align__(16) float sa1[TC];
    // tile decay, one copy per tile buffer, computed by wave 0 (which copies
    // a) as soon as its copy has landed
    __shared__ __align__(16) float sAw0[TC];
    __shared__ __align__(16) float sAw1[TC];
    __shared__ __align__(16) float sEw0[TC];
    __shared__ __align__(16) float sEw1[TC];

    const int nsegs = p.nseg - 1;
    const int nsub = 1 << (p.m - p.msub);
    int blk = xcd_block(blockIdx.x, gridDim.x);
    const int dvb = blk % p.ndvb;
    blk /= p.ndvb;
    const int sub = blk % nsub;
    blk /= nsub;
    const int seg = blk % nsegs;
    const int bh = blk / nsegs;
    const int cb = dvb * DVW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
    const size_t row0 = (size_t)bh * p.T;
    // every tile of a non-last segment is whole
    const int tile0 = (seg << p.m) + (sub << p.msub), ntl = 1 << p.msub;

    TileCopy<DK, NW> ck;
    TileCopy<DVW, NW> cv;
    ck.init(DK, 0, wave);
    cv.init(p.dv, cb, wave);
    auto issue = [&](int il, bf16_t* Kd, bf16_t* Vd, float* ad) __attribute__((always_inline)) {
        const size_t r = row0 + (size_t)(tile0 + il) * TC;
        ck.issue(p.k + r * DK, Kd, wave);
        cv.issue(p.v + r * p.dv, Vd, wave);
        if (p.a_dma) {
            if (wave == 0 && lane < TC / 4) dma16o(p.a + r, 16u * lane, ad);
        } else if (wave == 0) {
            dma4(p.a + r + lane, ad);
        }
    };

    f32x4 u[NDT];
#pragma unroll
    for (int kt = 0; kt < NDT; ++kt) u[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float total = 0.f;

    auto body = [&](int il, const bf16_t* Kc, const bf16_t* Vc, const float* Awc, const float* Ewc,
                    bf16_t* Kn, bf16_t* Vn, float* an, float* Awn, float* Ewn)
        __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (il + 1 < ntl) issue(il + 1, Kn, Vn, an);
        const float tot = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(Awc[TC - 1])));
        const float f = __expf(tot);
#pragma unroll
        for (int kt = 0; kt < NDT; ++kt) {
            u[kt][0] *= f; u[kt][1] *= f; u[kt][2] *= f; u[kt][3] *= f;
        }
        bf16x8 vf[2];
        vf[0] = ld_tr8<DVW>(Vc, 0, 16 * wave);
        vf[1] = ld_tr8<DVW>(Vc, 32, 16 * wave);
        tile_state<DK, NDT, false>(u, 0, Kc, vf, Ewc);
        total += tot;
        if (wave == 0 && il + 1 < ntl) {
            __builtin_amdgcn_s_waitcnt(0);
            tile_decay(an, Awn, Ewn);
        }
    };

    issue(0, sK0, sV0, sa0);
    if (wave == 0) {
        __builtin_amdgcn_s_waitcnt(0);
        tile_decay(sa0, sAw0, sEw0);
    }
    for (int il = 0; il < ntl; il += 2) {
        body(il, sK0, sV0, sAw0, sEw0, sK1, sV1, sa1, sAw1, sEw1);
        if (il + 1 < ntl) body(il + 1, sK1, sV1, sAw1, sEw1, sK0, sV0, sa0, sAw0, sEw0);
    }
    // the whole segment's state, or one of its sub-range states (the scan
    // decays and sums those in order)
    const size_t slot = ((size_t)bh * p.nseg + seg) * nsub + sub;
    float* dst = (nsub == 1 ? p.useg : p.upart) + slot * p.dv * DK;
    const int c = cb + wave * 16 + m16;
#pragma unroll
    for (int kt = 0; kt < NDT; ++kt) {
        // row of u[kt] (see tile_state): 32 (kt / 2) + 8g + 4 (kt % 2), or 4g for d_k = 16
        const int row = DK >= 32 ? 32 * (kt / 2) + 8 * g + 4 * (kt % 2) : 4 * g;
        if constexpr (TR) {
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(size_t)(row + r) * p.dv + c] = u[kt][r];
        } else {
            *reinterpret_cast<float4*>(dst + (size_t)c * DK + row) =
                make_float4(u[kt][0], u[kt][1], u[kt][2], u[kt][3]);
        }
    }
    if (threadIdx.x == 0 && dvb == 0) (nsub == 1 ? p.stot : p.tpart)[slot] = total;
}

// ---------------------------------------------------------------------------
// Main fused kernel: one block per (bh, segment, column block).
//   NW      waves per 16-column slab set (the block covers 16 NW columns)
//   NH      waves per column slab; each holds 1/NH of the head dimension of
//           every state and contracts only over that part, the partial level
//           products of the NH waves of a slab being summed through LDS
//   MLOC    register-resident levels inside a segment (segments of <= 2^MLOC tiles)
//   TOPMAX  levels above the segment held as bf16 fragments

//   BWD     the dq pass of the backward (operands swapped, see score_block_bwd):
//           also stages this column block's columns of q (p.qo) and writes
//           the block's partial dlambda rows to p.dlp

template <int DK, int NW, int NH, int MLOC, int TOPMAX, bool BWD>
__global__ __launch_bounds__(NW * NH * 64, 1) void k_fused_fwd(FusedParams p) {
    typedef HD<DK> H;
    constexpr int NWT = NW * NH;            // waves per block
    // the backward's dq pass as one block of 128 columns (one wave per slab)
    constexpr bool WIDE = BWD && NH == 1 && NWT == 8;
    constexpr int DVW = NW * 16;
    constexpr int NKSH = H::NKS / NH;       // contraction steps of this wave's head-dim part
    constexpr int NDTH = H::NDT / NH;       // 16-row state blocks of this wave's part

    static_assert(NKSH >= 1 && NDTH >= 1, "head dimension too small for the split");
    __shared__ __align__(16) bf16_t sQ0[TC * DK];
    __shared__ __align__(16) bf16_t sQ1[TC * DK];
    __shared__ __align__(16) bf16_t sK0[TC * DK];
    __shared__ __align__(16) bf16_t sK1[TC * DK];
    __shared__ __align__(16) bf16_t sV0[TC * DVW];
    __shared__ __align__(16) bf16_t sV1[TC * DVW];
    __shared__ __align__(16) float sL0[TC * kFusedMaxL];
    __shared__ __align__(16) float sL1[TC * kFusedMaxL];
    __shared__ __align__(16) float sa0[TC];
    __shared__ __align__(16) float sa1[TC];
    __shared__ __align__(16) bf16_t sP[TC * PROW];
    // tile decay (A_s and e^(A_end - A_s)), one copy per tile buffer, computed
    // by the wave that copies a, as soon as its copy has landed
    __shared__ __align__(16) float sAw0[TC];
    __shared__ __align__(16) float sAw1[TC];
    __shared__ __align__(16) float sEw0[TC];
    __shared__ __align__(16) float sEw1[TC];
    __shared__ __align__(16) f32x4 sX[(NH > 1 ? NH * NW * NRB : 1) * 64];  // partial outputs
    // dq pass: q's columns of this block, and the per-row dlambda partial sums
    // (levels inside the tile from the score blocks; per wave and level slot
    // for the levels above it: slot s < MLOC local level s, MLOC + q top level q)
    constexpr int NLS = MLOC + TOPMAX;
    static_assert(NRB == 4, "the four-row-block lane reductions");
    __shared__ __align__(16) bf16_t sQo0[BWD ? TC * DVW : 8];
    __shared__ __align__(16) bf16_t sQo1[BWD ? TC * DVW : 8];
    __shared__ __align__(16) float sDl[BWD ? NLS * NWT * TC : 4];
    __shared__ __align__(16) float sDi[BWD ? 10 * 16 : 4];
    __shared__ __align__(16) float sDd[BWD ? NRB * 5 * 16 : 4];
    // per wave q_t . (its part of dq_t), by tile parity: summed over the
    // waves after the next tile's first barrier (q . dq from the dq this
    // pass writes, the rounding the dk / dv stage sees as well)
    __shared__ __align__(16) float sDq[BWD ? 2 * NWT * TC : 4];
    // one-block dq pass writing dlambda rows: the tile's [token][L] block, by
    // tile parity, stored after the next tile's first barrier
    __shared__ __align__(16) float sGl[WIDE ? 2 * TC * kFusedMaxL : 4];
    // sX slots hold the 64 lanes of a C-layout fragment; lane l of slab cs is
    // stored at l ^ ((l / 16 + 4 (cs & 1)) & 7), so that the whole-row reads
    // of the finishers (eight lanes over two slabs and four lane groups per
    // LDS cycle) fall in distinct banks
    auto xswz = [](int l, int slab) __attribute__((always_inline)) {
        return l ^ (((l >> 4) + 4 * (slab & 1)) & 7);
    };

    int blk = xcd_block(blockIdx.x, gridDim.x);
    const int dvb = blk % p.ndvb;
    blk /= p.ndvb;
    const int seg = blk % p.nseg;
    const int bh = blk / p.nseg;
    const int cb = dvb * DVW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cs = wave % NW, hh = wave / NW;  // column slab, head-dim part
    const int lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
    const int c0 = cb + cs * 16;  // first column of this wave
    const int ks0 = hh * NKSH;
    const size_t row0 = (size_t)bh * p.T;
    const int tile0 = seg << p.m;
    const int ntl = min(1 << p.m, p.ntiles - tile0);
    const int L = p.L;         // lambda row length in global memory
    const int LP = p.lpitch;   // lambda row length in LDS

    // levels above the segment: Fenwick nodes over segments, bf16 fragments
    typename H::frag top[TOPMAX][NKSH];
    float logd_top[TOPMAX];
#pragma unroll
    for (int q = 0; q < TOPMAX; ++q) {
        logd_top[q] = 0.f;
        if (q < p.ntop && ((seg >> q) & 1)) {
            const int node = ((seg >> q) << q) - 1;
            const double* cum = p.scum + (size_t)bh * p.nseg;
            logd_top[q] = (float)(cum[seg - 1] - cum[node]);
            const size_t ng = (size_t)bh * p.nseg + node;
#pragma unroll
            for (int ks = 0; ks < NKSH; ++ks)
                top[q][ks] = *reinterpret_cast<const typename H::frag*>(
                    p.gfrag + frag_index<DK>(ng, p.dv / 16, c0 / 16, ks0 + ks));
        } else {
#pragma unroll
            for (int ks = 0; ks < NKSH; ++ks) top[q][ks] = typename H::frag{};
        }
    }

    // Issuing waves make the copies of the next tile and, with the d_k split,
    // sum and store the previous tile's output, both after their scores.
    // With eight waves, waves 4-7 (no score blocks) store the output and copy
    // Q and K, and waves 2 and 3 (two score blocks) copy V, lambda and a;
    // otherwise every wave does its share of everything.
    // The dq pass as one block of 128 columns (one wave per 16-column slab,
    // NH = 1): its V and q tiles are 16 KB each, so waves 0-3 copy those,
    // lambda and a, and waves 4-7 Q and K; every wave stores its own rows.
    constexpr int NIW = NWT == 8 ? 4 : NWT;      // Q/K copies and stores
    const bool issuer = wave >= NWT - NIW;
    const int iw = issuer ? wave - (NWT - NIW) : 0;
    constexpr int NIW1 = WIDE ? 4 : NWT == 8 ? 2 : NIW;  // V, lambda and a copies
    constexpr int P1W0 = WIDE ? 0 : NWT == 8 ? 2 : NWT - NIW;
    const bool issuer1 = wave >= P1W0 && wave < P1W0 + NIW1;
    const int i1 = issuer1 ? wave - P1W0 : 0;
    const bool dwave = wave == P1W0;  // copies a; computes each tile's decay
    TileCopy<DK, NIW> cqk;  // Q and K tiles share the layout
    TileCopy<DVW, NIW1> cv;
    TileCopy<DVW, NIW1> cqo;  // dq pass: q's columns, laid out as the value tile
    cqk.init(DK, 0, iw);
    cv.init(p.dv, cb, i1);
    if constexpr (BWD) cqo.init(p.dv, cb, i1);

    // Every tile input goes global -> LDS through the DMA path: 16-byte
    // copies where rows are whole and aligned, 4-byte copies of lambda and a
    // otherwise (entries past the sequence are stored as zeros).
    // part 0: Q and K (issuing waves iw); part 1: V, lambda and a (issuing
    // waves i1)
    auto issue = [&](int il, int part, bf16_t* Qd, bf16_t* Kd, bf16_t* Vd, float* Ld, float* ad,
                     bf16_t* Qod) __attribute__((always_inline)) {
        const int t0 = (tile0 + il) * TC;
        const int nvalid = min(TC, p.T - t0);
        const size_t r = row0 + t0;
        const bool whole = nvalid == TC;
        if (part == 0) {
            if (whole) {
                // the forward's last read of q, k, v, lambda and a
                cqk.template issue<true>(p.q + r * DK, Qd, iw);
                cqk.template issue<true>(p.k + r * DK, Kd, iw);
            } else {
                dma_tile<DK, NIW>(p.q + r * DK, DK, 0, nvalid, Qd, iw);
                dma_tile<DK, NIW>(p.k + r * DK, DK, 0, nvalid, Kd, iw);
            }
            return;
        }
        if (whole) cv.template issue<true>(p.v + r * p.dv, Vd, i1);
        else dma_tile<DVW, NIW1>(p.v + r * p.dv, p.dv, cb, nvalid, Vd, i1);
        if constexpr (BWD) {
            if (whole) cqo.template issue<true>(p.qo + r * p.dv, Qod, i1);
            else dma_tile<DVW, NIW1>(p.qo + r * p.dv, p.dv, cb, nvalid, Qod, i1);
        }
        // lambda from the last issuing wave down (those hold fewer Q/K/V jobs)
        const int lw = NIW1 - 1 - i1;
        if (whole && p.lam_dma) {
            const int nch = 16 * L;  // 64 rows x L floats
            for (int u = lw; u * 64 < nch; u += NIW1)
                if (u * 64 + lane < nch) dma16o<true>(p.lam + r * L, 16u * (u * 64 + lane), Ld + u * 256);
        } else {
            const int nel = nvalid * LP;
            for (int u = lw; u * 64 < TC * LP; u += NIW1) {
                const int x = u * 64 + lane;
                if (x < nel) {
                    const int row = x / LP, l = x - row * LP;
                    dma4(p.lam + (r + row) * L + l, Ld + u * 64);
                } else if (x < TC * LP) {
                    Ld[x] = 0.f;
                }
            }
        }
        if (i1 == 0) {
            if (whole && p.a_dma) {
                if (lane < TC / 4) dma16o<true>(p.a + r, 16u * lane, ad);
            } else if (lane < nvalid) {
                dma4(p.a + r + lane, ad);
            } else {
                ad[lane] = 0.f;
            }
        }
    };

    bf16x4 G[MLOC][NDTH];
    float logd_loc[MLOC];
#pragma unroll
    for (int s = 0; s < MLOC; ++s) {
        logd_loc[s] = 0.f;
#pragma unroll
        for (int kt = 0; kt < NDTH; ++kt) G[s][kt] = bf16x4{};
    }

    // Output of the previous tile (d_k split only): after the P V product
    // each wave leaves its partial rows (its half of the level products, and
    // the intra-tile part for the row blocks it owns) in sX; after the next
    // tile's first barrier the issuing waves of the last head-dim part sum
    // the NH partials of their column slab and store the rows, so the
    // exchange costs no barrier of its own.
    int prev_tile = -1, prev_valid = 0;
    // The finisher of slab cs takes the row blocks rb = cs (mod NW) across
    // all DVW columns, so that each store covers whole rows (DVW * 4 bytes
    // of a row per LPR lanes) instead of 64-byte pieces of 16 rows.
    auto finish_prev = [&]() __attribute__((always_inline)) {
        constexpr int LPR = NW * 4;     // lanes per row (16 bytes each)
        constexpr int RPI = 64 / LPR;   // rows per store
        const int c = (lane % LPR) * 4;  // column within the block
        const int m0 = lane / LPR;       // row within the store
        for (int rb = cs; rb < NRB; rb += NW) {
            const f32x4* xs = sX + ((c / 16) * NRB + rb) * 64;
            float* op = p.out + (row0 + (size_t)prev_tile * TC + 16 * rb + m0) * p.dv + cb + c;
#pragma unroll
            for (int k = 0; k < 16 / RPI; ++k) {
                // the C-layout lane holding (row m0 + RPI k, column c) of slab c / 16
                const int at = xswz(((c % 16) / 4) * 16 + m0 + k * RPI, c / 16);
                f32x4 x = xs[at];
#pragma unroll
                for (int h = 1; h < NH; ++h) {
                    const f32x4 y = xs[at + h * NW * NRB * 64];
                    x[0] += y[0]; x[1] += y[1]; x[2] += y[2]; x[3] += y[3];
                }
                if (16 * rb + k * RPI + m0 < prev_valid)  // written once: non-temporal
                    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(op + (size_t)(k * RPI) * p.dv));
            }
        }
    };
    const bool finisher = NH > 1 && hh == NH - 1;
    // dq pass: q . dq of tile il of the segment (its rows < T), this column
    // block's part, summed over the waves' parts
    auto finish_qdq = [&](int il) __attribute__((always_inline)) {
        if constexpr (BWD) {
            const int t = threadIdx.x;
            const int t0 = (tile0 + il) * TC;
            if (t < TC && t0 + t < p.T) {
                float x = 0.f;
#pragma unroll
                for (int u = 0; u < NWT; ++u) x += sDq[((il & 1) * NWT + u) * TC + t];
                p.dqd[((size_t)dvb * p.BH + bh) * p.T + t0 + t] = x;
            }
        }
    };
    // one-block dq pass: the dlambda rows of tile il of the segment, nvalid x
    // L consecutive floats
    auto store_rows = [&](int il) __attribute__((always_inline)) {
        if constexpr (WIDE) {
            if (p.dlam_rows) {
                const int t0 = (tile0 + il) * TC;
                const int n = min(TC, p.T - t0) * p.L;
                float* dst = p.dlam_rows + ((size_t)bh * p.T + t0) * p.L;
                const float* src = sGl + (il & 1) * TC * kFusedMaxL;
                // 16-byte stores where the rows start on 16 bytes: the
                // output on 16 bytes and T L % 4 == 0 (t0 is a multiple of 64)
                const bool al16 = (reinterpret_cast<uintptr_t>(p.dlam_rows) & 15) == 0 &&
                                  ((long)p.T * p.L) % 4 == 0;
                const int n4 = al16 ? n >> 2 : 0;
                for (int x = threadIdx.x; x < n4; x += NWT * 64)
                    reinterpret_cast<f32x4*>(dst)[x] = reinterpret_cast<const f32x4*>(src)[x];
                for (int x = 4 * n4 + threadIdx.x; x < n; x += NWT * 64) dst[x] = src[x];
            }
        }
    };

    const int lane_k = lane, m16_k = m16, g_k = g;  // the body's lane indices (see there)
    // dq pass: A at the end of each tile of the segment (fp64), from A before it
    double run_cum = 0.0;
    if constexpr (BWD) {
        if (p.ccum && seg > 0) run_cum = p.scum[(size_t)bh * p.nseg + seg - 1];
    }
    auto body = [&](int il, const bf16_t* Qc, const bf16_t* Kc, const bf16_t* Vc,
                    const float* Lc, const float* Awc, const float* Ewc, const bf16_t* Qoc,
                    bf16_t* Qn, bf16_t* Kn, bf16_t* Vn, float* Ln, float* an, float* Awn,
                    float* Ewn, bf16_t* Qon) __attribute__((always_inline)) {
        // tile il is in LDS and every wave is done with tile il - 1
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // one-block dq pass: the lane indices through an opaque zero, so that
        // the body's per-lane address arithmetic is redone in place each tile
        // instead of being hoisted out of the loop and spilled (a spill
        // reload there makes the copying waves wait for their own copies)
        int zv = 0;
        if constexpr (WIDE) asm volatile("v_mov_b32 %0, 0" : "=v"(zv));
        const int lane = WIDE ? (int)(threadIdx.x & 63) + zv : lane_k;
        const int m16 = WIDE ? lane & 15 : m16_k, g = WIDE ? lane >> 4 : g_k;
        if constexpr (BWD) {
            if (il > 0) finish_qdq(il - 1);
            if (il > 0) store_rows(il - 1);
        }
        if constexpr (NH > 1) {
            if (finisher && !issuer && prev_tile >= 0) finish_prev();
        }
        const int i = tile0 + il;
        const int nvalid = min(TC, p.T - i * TC);
        const float tot = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(Awc[TC - 1])));
        if constexpr (BWD) {
            if (p.ccum) {
                run_cum += (double)tot;
                if (threadIdx.x == 0 && dvb == 0) p.ccum[(size_t)bh * p.ntiles + i] = run_cum;
            }
        }
        // dq pass: the issuing waves of Q and K store and copy before their
        // scores, so that their queue stalls overlap the other waves' scores
        // and not the waves 2 and 3 copying V, q, lambda and a after theirs
        if (BWD && issuer) {
            if constexpr (NH > 1) {
                if (finisher && prev_tile >= 0) finish_prev();
            }
            if (il + 1 < ntl) issue(il + 1, 0, Qn, Kn, Vn, Ln, an, Qon);
        }
        if constexpr (BWD)
            scores_for_wave<DK, NWT, true, DVW>(wave, Qc, Kc, sP, Awc, Lc, LP, Qoc, Vc, sDi, sDd);
        else
            scores_for_wave<DK, NWT>(wave, Qc, Kc, sP, Awc, Lc, LP);
        if (!BWD && issuer) {
            if constexpr (NH > 1) {
                if (finisher && prev_tile >= 0) finish_prev();
            }
            if (il + 1 < ntl) issue(il + 1, 0, Qn, Kn, Vn, Ln, an, Qon);
        }
        if (issuer1 && il + 1 < ntl) issue(il + 1, 1, Qn, Kn, Vn, Ln, an, Qon);

        // ---- level products (this wave's head-dim part, all rows), before the
        // barrier that publishes P: they do not need it.  The weight of level
        // l for row t is lambda_t^(l) e^(A_t) e^(logd_l); the per-level part
        // is applied here, e^(A_t) once per row block at the end.
        f32x4 lv[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) lv[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Q fragments of the level products (this wave's head-dim part, all
        // row blocks): 8 consecutive head-dim rows per lane group, the order in
        // which tile_state lays out the register states.  Read once per tile.
        // (the one-block dq pass reads them from LDS at each use instead: its
        // register levels cover all of d_k, and kept here they would spill)
        typename H::frag qf[WIDE ? 1 : NRB][NKSH];
        auto qfrag = [&](int rb, int ks) __attribute__((always_inline)) {
            typename H::frag x;
            if constexpr (DK >= 32) x = ld8<DK>(Qc, 16 * rb + m16, 32 * (ks0 + ks) + 8 * g);
            else x = ld4<DK>(Qc, 16 * rb + m16, 4 * g);
            return x;
        };
        if constexpr (!WIDE) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int ks = 0; ks < NKSH; ++ks) qf[rb][ks] = qfrag(rb, ks);
        }
        // dq pass: q at (row 16 rb + m16, columns c0 + 4g .. + 3), the columns
        // of this lane's level-product outputs
        float qv[BWD && !WIDE ? NRB : 1][4];
        auto qval = [&](int rb, float (&x)[4]) __attribute__((always_inline)) {
            const bf16x4 y = ld4<DVW>(Qoc, 16 * rb + m16, 16 * cs + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (float)y[r];
        };
        if constexpr (BWD && !WIDE) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) qval(rb, qv[rb]);
        }
        auto add_level = [&](const typename H::frag (&ga)[NKSH], int lev, float logd, int slot)
            __attribute__((always_inline)) {
            const float d = __expf(logd);
            float w[NRB];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) w[rb] = Lc[(16 * rb + m16) * LP + lev];
            f32x4 y[NRB];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                y[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKSH; ++ks) {
                    if constexpr (WIDE) y[rb] = mma(ga[ks], qfrag(rb, ks), y[rb]);
                    else y[rb] = mma(ga[ks], qf[rb][ks], y[rb]);
                }
            }
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const float wr = w[rb] * d;
                lv[rb][0] += wr * y[rb][0];
                lv[rb][1] += wr * y[rb][1];
                lv[rb][2] += wr * y[rb][2];
                lv[rb][3] += wr * y[rb][3];
            }
            if constexpr (BWD) {
                // this wave's part of q_t . (level product) e^(logd); e^(A_t)
                // is applied when the parts are summed.  Lane (m16, g) ends
                // with row block g's total for token 16 g + m16.
                float x[NRB];
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    float qq[4];
                    if constexpr (WIDE) qval(rb, qq);
                    else for (int r = 0; r < 4; ++r) qq[r] = qv[rb][r];
                    x[rb] = qq[0] * y[rb][0] + qq[1] * y[rb][1] + qq[2] * y[rb][2] + qq[3] * y[rb][3];
                }
                sDl[(slot * NWT + wave) * TC + lane] = d * sum_rows4_x4(x[0], x[1], x[2], x[3]);
            }
        };
        // levels inside the segment
#pragma unroll
        for (int s = 0; s < MLOC; ++s) {
            if (s < p.m && ((il >> s) & 1)) {
                typename H::frag ga[NKSH];
#pragma unroll
                for (int ks = 0; ks < NKSH; ++ks) {
                    if constexpr (DK >= 32) ga[ks] = __builtin_shufflevector(G[s][2 * ks], G[s][2 * ks + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                    else ga[ks] = G[s][ks];
                }
                add_level(ga, LOGTC + s + 1, logd_loc[s], s);
            }
        }
        // levels above the segment
#pragma unroll
        for (int q = 0; q < TOPMAX; ++q)
            if (q < p.ntop && ((seg >> q) & 1)) add_level(top[q], LOGTC + p.m + q + 1, logd_top[q], MLOC + q);
        __syncthreads();
        if constexpr (BWD) {
            // the tile's dlambda for this column block, level-major ([LU][T]
            // rows of dlp): wave w takes the levels w, w + NWT, ..., lane t the
            // token; levels 0..4 from the diagonal score blocks, 5 and 6 from
            // the blocks below it, the levels above the tile from the level
            // products (summed over the waves' parts, times e^(A_t))
            const int t = lane, rb = t >> 4, mm = t & 15;
            float* dst = p.dlp + ((size_t)dvb * p.BH + bh) * (size_t)p.LU * p.T + (size_t)i * TC + t;
            // (written as rows: the levels past LU stay zero from the start)
            for (int l = wave; l < p.LU; l += NWT) {
                float val = 0.f;
                if (l <= 4) {
                    val = sDd[(rb * 5 + l) * 16 + mm];
                } else if (l == 5) {
                    if (rb & 1) val = sDi[(rb * (rb + 1) / 2 + rb - 1) * 16 + mm];
                } else if (l == 6) {
                    if (rb >= 2) val = sDi[(rb * (rb + 1) / 2) * 16 + mm] + sDi[(rb * (rb + 1) / 2 + 1) * 16 + mm];
                } else {
                    const int sl = l - LOGTC - 1;
                    int slot = -1;
                    if (sl < p.m) {
                        if (sl < MLOC && ((il >> sl) & 1)) slot = sl;
                    } else if (sl - p.m < p.ntop && sl - p.m < TOPMAX && ((seg >> (sl - p.m)) & 1)) {
                        slot = MLOC + sl - p.m;
                    }
                    if (slot >= 0) {
                        float x = 0.f;
#pragma unroll
                        for (int u = 0; u < NWT; ++u) x += sDl[(slot * NWT + u) * TC + t];
                        val = x * __expf(Awc[t]);
                    }
                }
                if constexpr (WIDE) {
                    if (p.dlam_rows) sGl[(il & 1) * TC * kFusedMaxL + t * p.L + l] = val;
                    else if (t < nvalid) dst[(size_t)l * p.T] = val;
                } else {
                    if (t < nvalid) dst[(size_t)l * p.T] = val;
                }
            }
        }

        // ---- intra-tile P V for the row blocks this wave writes
        bf16x8 vf[2];
        vf[0] = ld_tr8<DVW>(Vc, 0, 16 * cs);
        vf[1] = ld_tr8<DVW>(Vc, 32, 16 * cs);
        float eA[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) eA[rb] = Awc[16 * rb + m16];
        f32x4 o[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const float e = __expf(eA[rb]);
            o[rb] = f32x4{e * lv[rb][0], e * lv[rb][1], e * lv[rb][2], e * lv[rb][3]};
        }
        // the intra-tile part: all row blocks in the first head-dim half (the
        // second half, slower to issue after the barrier, adds none); row
        // block rb pairs with the first rb / 2 + 1 32-key halves of P
        if (hh == 0) {
            bf16x8 pf[NRB][2];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int sp = 0; sp <= rb / 2; ++sp)
                    pf[rb][sp] = *reinterpret_cast<const bf16x8*>(sP + (16 * rb + m16) * PROW + 32 * sp + 8 * g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int sp = 0; sp <= rb / 2; ++sp) o[rb] = mma(vf[sp], pf[rb][sp], o[rb]);
        }

        if constexpr (BWD) {
            float x[NRB];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                float qq[4];
                if constexpr (WIDE) qval(rb, qq);
                else for (int r = 0; r < 4; ++r) qq[r] = qv[rb][r];
                x[rb] = qq[0] * o[rb][0] + qq[1] * o[rb][1] + qq[2] * o[rb][2] + qq[3] * o[rb][3];
            }
            sDq[((il & 1) * NWT + wave) * TC + lane] = sum_rows4_x4(x[0], x[1], x[2], x[3]);
        }
        if constexpr (NH > 1) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) sX[((hh * NW + cs) * NRB + rb) * 64 + xswz(lane, cs)] = o[rb];
            prev_tile = i;
            prev_valid = nvalid;
        } else {
            float* orow = p.out + (row0 + (size_t)i * TC) * p.dv + c0 + 4 * g;
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const int r = 16 * rb + m16;
                if (r < nvalid)  // written once: non-temporal
                    __builtin_nontemporal_store(o[rb], reinterpret_cast<f32x4*>(orow + (size_t)r * p.dv));
            }
        }

        // ---- Fenwick update over tiles: fold the tile's state and the slots
        // below lssb(il + 1) into slot lssb(il + 1)
        if (il + 1 < ntl) {
            f32x4 u[NDTH];
#pragma unroll
            for (int kt = 0; kt < NDTH; ++kt) u[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            tile_state<DK, NDTH, true>(u, ks0, Kc, vf, Ewc);
            const int j = lssb((uint64_t)il + 1);
#pragma unroll
            for (int s = 0; s < MLOC; ++s) {
                if (s < j) {
                    const float w = __expf(logd_loc[s] + tot);
#pragma unroll
                    for (int kt = 0; kt < NDTH; ++kt) {
                        u[kt][0] += w * (float)G[s][kt][0];
                        u[kt][1] += w * (float)G[s][kt][1];
                        u[kt][2] += w * (float)G[s][kt][2];
                        u[kt][3] += w * (float)G[s][kt][3];
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < MLOC; ++s) {
                if (s == j) {
#pragma unroll
                    for (int kt = 0; kt < NDTH; ++kt) G[s][kt] = cvt4(u[kt]);
                    logd_loc[s] = 0.f;
                } else {
                    logd_loc[s] += tot;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < TOPMAX; ++q) logd_top[q] += tot;
        // the next tile's decay, from its a (this wave's own copy)
        if (dwave && il + 1 < ntl) {
            __builtin_amdgcn_s_waitcnt(0);
            tile_decay(an, Awn, Ewn);
        }
    };

    if constexpr (WIDE) {
        // dlambda rows: levels LU..L-1 of every staged row are zero
        if (p.dlam_rows)
            for (int x = threadIdx.x; x < 2 * TC * kFusedMaxL; x += NWT * 64) sGl[x] = 0.f;
    }
    if (issuer) issue(0, 0, sQ0, sK0, sV0, sL0, sa0, sQo0);
    if (issuer1) issue(0, 1, sQ0, sK0, sV0, sL0, sa0, sQo0);
    if (dwave) {
        __builtin_amdgcn_s_waitcnt(0);
        tile_decay(sa0, sAw0, sEw0);
    }
    for (int il = 0; il < ntl; il += 2) {
        body(il, sQ0, sK0, sV0, sL0, sAw0, sEw0, sQo0, sQ1, sK1, sV1, sL1, sa1, sAw1, sEw1, sQo1);
        if (il + 1 < ntl)
            body(il + 1, sQ1, sK1, sV1, sL1, sAw1, sEw1, sQo1, sQ0, sK0, sV0, sL0, sa0, sAw0, sEw0, sQo0);
    }
    if constexpr (NH > 1 || BWD) {
        __syncthreads();
        if constexpr (NH > 1) {
            if (finisher) finish_prev();
        }
        if constexpr (BWD) {
            finish_qdq(ntl - 1);
            store_rows(ntl - 1);
        }
    }
}

// ---------------------------------------------------------------------------
// host side

namespace {

// Register budgets of the main kernel: (levels inside a segment, levels above it).
struct Combo {
    int mloc, topmax;
};
constexpr Combo kCombos[] = {{2, 4}, {3, 4}, {5, 2}, {5, 5}, {3, 7}};
constexpr int kNumCombos = sizeof(kCombos) / sizeof(kCombos[0]);

int bit_len(long x) {
    int n = 0;
    while (x > 0) {
        ++n;
        x >>= 1;
    }
    return n;
}

}  // namespace

FusedPlan plan_fused(int BH, int T, int dk, int dv, int lu, int force_m, int force_split, int max_dvw) {
    FusedPlan pl{};
    if (lu > kFusedMaxL) return pl;  // lambda levels staged per token
    const int dvw = dv >= max_dvw ? max_dvw : dv >= 64 ? 64 : dv;
    pl.dvw = dvw;
    pl.ndvb = dv / dvw;
    pl.ntiles = (T + TC - 1) / TC;
    const long pairs = (long)BH * pl.ndvb;
    const long slots = 256;  // one resident block per CU (register budget)
    // Cost: the serial tiles a CU walks, rounds of resident blocks x tiles per
    // block.
    int best = -1, best_combo = -1;
    long best_cost = 0;
    for (int m = 0; m <= 5; ++m) {
        if (force_m >= 0 && m != force_m) continue;
        const long nseg = (pl.ntiles + (1L << m) - 1) >> m;
        const int ntop = bit_len(nseg - 1);
        int combo = -1;
        for (int c = 0; c < kNumCombos; ++c)
            if (m <= kCombos[c].mloc && ntop <= kCombos[c].topmax) {
                combo = c;
                break;
            }
        if (combo < 0) continue;
        const long blocks = pairs * nseg;
        const long rounds = (blocks + slots - 1) / slots;
        const long cost = rounds * (1L << m);
        // equal cost: the longer segment (fewer segment states and nodes)
        if (best < 0 || cost <= best_cost) {
            best = m;
            best_cost = cost;
            best_combo = combo;
        }
    }
    if (best < 0) return pl;
    pl.m = best;
    pl.nseg = (int)((pl.ntiles + (1L << best) - 1) >> best);
    pl.ntop = bit_len(pl.nseg - 1);
    pl.combo = best_combo;
    // segment states in up to 8 sub-ranges: the fewest that give every CU a
    // block (more sub-ranges add partial states to write and combine)
    pl.msub = best;
    while (pl.msub > 0 && best - pl.msub < 3 &&
           pairs * (pl.nseg - 1) * (1L << (best - pl.msub)) < 256)
        --pl.msub;
    if (force_split >= 0) pl.msub = best > force_split ? best - force_split : 0;
    pl.ok = 1;
    return pl;
}

namespace {

template <int DK, int NW, int MLOC, int TOPMAX>
hipError_t launch_main(const FusedParams& p, hipStream_t stream) {
    const unsigned nblk = (unsigned)p.BH * p.nseg * p.ndvb;
    if constexpr (NW == 8) {
        // 128 columns in one block: only the backward's dq pass (d_k' = 64,
        // one wave per 16-column slab holding all of d_k') with five register
        // levels and two above the segment (the 8K plan; other plans use
        // two 64-column blocks)
        if constexpr (DK == 64 && MLOC == 5 && TOPMAX == 2) {
            if (p.qo) {
                hipLaunchKernelGGL((k_fused_fwd<DK, 8, 1, MLOC, TOPMAX, true>), dim3(nblk), dim3(8 * 64), 0,
                                   stream, p);
                return hipGetLastError();
            }
        }
        return hipErrorInvalidValue;
    } else {
        constexpr int NH = DK >= 64 ? 2 : 1;  // two waves share a column slab, each half of d_k
        if (p.qo) {
            // the backward's dq pass: d_v = 64 (the contraction here) only
            if constexpr (DK == 64 && NW == 4) {
                hipLaunchKernelGGL((k_fused_fwd<DK, NW, NH, MLOC, TOPMAX, true>), dim3(nblk),
                                   dim3(NW * NH * 64), 0, stream, p);
                return hipGetLastError();
            }
            return hipErrorInvalidValue;
        }
        hipLaunchKernelGGL((k_fused_fwd<DK, NW, NH, MLOC, TOPMAX, false>), dim3(nblk), dim3(NW * NH * 64), 0,
                           stream, p);
        return hipGetLastError();
    }
}

template <int DK, int NW>
hipError_t launch_fused_t(const FusedParams& p, const FwdParams& scan, unsigned stages,
                          hipStream_t stream) {
    hipError_t err;
    if (p.nseg > 1 && (stages & kStageChunkState)) {
        const unsigned nblk = (unsigned)p.BH * (p.nseg - 1) * (1u << (p.m - p.msub)) * p.ndvb;
        if constexpr (DK == 64 && NW == 8) {
            // the one-block dq pass (keys v, d_k' = 64; values k, 128 columns):
            // its states sum v k^T, the transpose of the forward's k v^T over
            // the same segments, so the forward's kernel (keys k, values v in
            // one 64-column block) builds them and stores them transposed;
            // the scan over them is elementwise
            FusedParams sp = p;
            sp.k = p.v;
            sp.v = p.k;
            sp.dv = 64;
            sp.ndvb = 1;
            hipLaunchKernelGGL((k_seg_state<128, 4, true>), dim3(nblk), dim3(4 * 64), 0, stream, sp);
        } else {
            hipLaunchKernelGGL((k_seg_state<DK, NW>), dim3(nblk), dim3(NW * 64), 0, stream, p);
        }
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (p.nseg > 1 && (stages & kStageScan)) {
        err = launch_fenwick_scan(scan, stream);
        if (err != hipSuccess) return err;
    }
    if (stages & kStageOutput) {
        switch (p.combo) {
            case 0: return launch_main<DK, NW, kCombos[0].mloc, kCombos[0].topmax>(p, stream);
            case 1: return launch_main<DK, NW, kCombos[1].mloc, kCombos[1].topmax>(p, stream);
            case 2: return launch_main<DK, NW, kCombos[2].mloc, kCombos[2].topmax>(p, stream);
            case 3: return launch_main<DK, NW, kCombos[3].mloc, kCombos[3].topmax>(p, stream);
            case 4: return launch_main<DK, NW, kCombos[4].mloc, kCombos[4].topmax>(p, stream);
        }
        return hipErrorInvalidValue;
    }
    return hipSuccess;
}

template <int DK>
hipError_t launch_fused_dk(const FusedParams& p, const FwdParams& scan, unsigned stages,
                           hipStream_t s) {
    switch (p.dvw) {
        case 16: return launch_fused_t<DK, 1>(p, scan, stages, s);
        case 32: return launch_fused_t<DK, 2>(p, scan, stages, s);
        case 64: return launch_fused_t<DK, 4>(p, scan, stages, s);
        case 128:
            if constexpr (DK == 64) return launch_fused_t<DK, 8>(p, scan, stages, s);
            break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fused_fwd(const FusedParams& p, const FwdParams& scan, unsigned stages,
                            hipStream_t stream) {
    switch (p.dk) {
        case 16: return launch_fused_dk<16>(p, scan, stages, stream);
        case 32: return launch_fused_dk<32>(p, scan, stages, stream);
        case 64: return launch_fused_dk<64>(p, scan, stages, stream);
        case 128: return launch_fused_dk<128>(p, scan, stages, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace loglin
