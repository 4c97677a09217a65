// Fenwick level states after a prefill, for continuing with decode steps.
//
// "Log-linear attention, and what a logarithm buys", section 2: after the T
// tokens 0..T-1 the state a decode step at position T reads is, for level 0,
// the last token's k v^T, and for each set bit p of T - 1 the bucket of 2^p
// tokens that the greedy (oldest, largest first) decomposition of the prefix
// gives that bit, at level p + 1.  With the scalar gate (sections 1 and 3)
// every token is decayed to position T - 1:
//     S^(l) = sum over s in bucket l of exp(A_{T-1} - A_s) k_s v_s^T.
// Token s of the prefix lies in the bucket of level floor(log2((T-1) xor s)) + 1.
//
// The prefix is cut into jobs: whole 512-token pieces of the buckets of 512
// tokens or more (every such bucket is a whole number of aligned pieces), one
// job per smaller bucket, and one for level 0.  Each job's decayed sum is
// computed for bf16 inputs on the matrix cores (k_prefill_job, with the
// forward's tile machinery), for fp32 inputs with fp32 vector FMAs
// (k_prefill_part).  A level of one job is written
// to the state layout the decode state loads ([B, H, Lmax, dk, dv]) by its job;
// k_prefill_sum adds the pieces of the longer buckets and zeroes the slots
// that are not live.
#include "tile_ops.hpp"

namespace loglin {

namespace {

constexpr int kThr = 256;
constexpr int kTile = 64;

// Prefill states (bf16 inputs): one block per (bh, job, column block) sums
// exp(A_{s1-1} - A_s) k_s v_s^T over the job's tokens [s0, s1) tile by tile
// (the forward's tile state, with the tokens outside the job masked), decays
// the sum to position T - 1 and writes it, [d_k][d_v], to the state of its
// level (a level of one job) or to the job's slot of the workspace.  The jobs
// are described with PrefillJob (kernels.hpp).

// Tile decay restricted to the tokens [lo, hi) of the tile: the others get
// a = 0 (no decay) and e = 0 (no contribution).
__device__ __forceinline__ float tile_decay_masked(const float* a_tile, int lo, int hi, float* Aw,
                                                   float* Ew) {
    const int lane = threadIdx.x & 63;
    const bool in = lane >= lo && lane < hi;
    const float x = wave_inclusive_sum(in ? a_tile[lane] : 0.f);
    const float end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
    Aw[lane] = x;
    Ew[lane] = in ? __expf(end - x) : 0.f;
    return end;
}

template <int DK, int NW>
__global__ __launch_bounds__(NW * 64) void k_prefill_job(PrefillParams p) {
    constexpr int DVW = NW * 16;
    constexpr int NDT = DK / 16;
    __shared__ __align__(16) bf16_t sK0[TC * DK];
    __shared__ __align__(16) bf16_t sK1[TC * DK];
    __shared__ __align__(16) bf16_t sV0[TC * DVW];
    __shared__ __align__(16) bf16_t sV1[TC * DVW];
    __shared__ __align__(16) float sa0[TC];
    __shared__ __align__(16) float sa1[TC];
    __shared__ __align__(16) float sAw[NW][TC];
    __shared__ __align__(16) float sEw[NW][TC];
    __shared__ float sred[NW];

    const int ncb = p.dv / DVW;
    int blk = blockIdx.x;
    const int cb = (blk % ncb) * DVW;
    blk /= ncb;
    const int job = blk % p.njobs;
    const int bh = blk / p.njobs;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, m16 = lane & 15, g = lane >> 4;
    const PrefillJob jb = prefill_job(p.T - 1, job);
    const size_t row0 = (size_t)bh * p.T;
    const bf16_t* kg = reinterpret_cast<const bf16_t*>(p.k);
    const bf16_t* vg = reinterpret_cast<const bf16_t*>(p.v);

    // decay from the end of the job to position T - 1 (read after a barrier):
    // 16-byte loads from the first 16-byte boundary on, eight in flight per
    // thread, the up to three floats before it and the rest after them one by one
    float part = 0.f;
    {
        constexpr int NT = NW * 64;
        const int n = p.T - jb.s1;
        const float* ap = p.a + row0 + jb.s1;
        const int head = min(n, (int)((16u - (uint32_t)(reinterpret_cast<uintptr_t>(ap) & 15u)) & 15u) / 4);
        const int n4 = (n - head) >> 2;
        const float4* ap4 = reinterpret_cast<const float4*>(ap + head);
        float4 ps[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ps[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        int r = threadIdx.x;
        for (; r + 7 * NT < n4; r += 8 * NT) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4 x = ap4[r + j * NT];
                ps[j].x += x.x; ps[j].y += x.y; ps[j].z += x.z; ps[j].w += x.w;
            }
        }
        for (; r < n4; r += NT) {
            const float4 x = ap4[r];
            ps[0].x += x.x; ps[0].y += x.y; ps[0].z += x.z; ps[0].w += x.w;
        }
        const int rest = n - head - 4 * n4;  // 0..3
        if ((int)threadIdx.x < head) ps[1].x += ap[threadIdx.x];
        if ((int)threadIdx.x < rest) ps[2].x += ap[head + 4 * n4 + threadIdx.x];
#pragma unroll
        for (int j = 0; j < 8; ++j) part += (ps[j].x + ps[j].y) + (ps[j].z + ps[j].w);
    }
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) sred[wave] = part;

    const int t0 = jb.s0 / TC, t1 = (jb.s1 - 1) / TC;  // the job's tiles
    // whole tiles by the forward's copy plan (one scalar base, precomputed
    // lane offsets), the sequence's partial last tile row by row
    TileCopy<DK, NW> ck;
    TileCopy<DVW, NW> cv;
    ck.init(DK, 0, wave);
    cv.init(p.dv, cb, wave);
    auto issue = [&](int tile, bf16_t* Kd, bf16_t* Vd, float* ad) __attribute__((always_inline)) {
        const int base = tile * TC;
        const int nvalid = min(TC, p.T - base);
        const size_t r = row0 + base;
        if (nvalid == TC) {
            ck.issue(kg + r * DK, Kd, wave);
            cv.issue(vg + r * p.dv, Vd, wave);
        } else {
            dma_tile<DK, NW>(kg + r * DK, DK, 0, nvalid, Kd, wave);
            dma_tile<DVW, NW>(vg + r * p.dv, p.dv, cb, nvalid, Vd, wave);
        }
        if (wave == 0) {
            if (lane < nvalid) dma4(p.a + r + lane, ad);
            else ad[lane] = 0.f;
        }
    };

    f32x4 u[NDT];
#pragma unroll
    for (int kt = 0; kt < NDT; ++kt) u[kt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto body = [&](int tile, const bf16_t* Kc, const bf16_t* Vc, const float* ac, bf16_t* Kn,
                    bf16_t* Vn, float* an) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tile + 1 <= t1) issue(tile + 1, Kn, Vn, an);
        const int base = tile * TC;
        const float tot = tile_decay_masked(ac, jb.s0 - base, jb.s1 - base, sAw[wave], sEw[wave]);
        const float f = __expf(tot);
#pragma unroll
        for (int kt = 0; kt < NDT; ++kt) {
            u[kt][0] *= f; u[kt][1] *= f; u[kt][2] *= f; u[kt][3] *= f;
        }
        bf16x8 vf[2];
        vf[0] = ld_tr8<DVW>(Vc, 0, 16 * wave);
        vf[1] = ld_tr8<DVW>(Vc, 32, 16 * wave);
        tile_state<DK, NDT, false>(u, 0, Kc, vf, sEw[wave]);
    };

    issue(t0, sK0, sV0, sa0);
    for (int tile = t0; tile <= t1; tile += 2) {
        body(tile, sK0, sV0, sa0, sK1, sV1, sa1);
        if (tile + 1 <= t1) body(tile + 1, sK1, sV1, sa1, sK0, sV0, sa0);
    }
    float carry = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) carry += sred[w];
    const float fin = __expf(carry);
    float* dst = (prefill_single(jb.level)
                      ? p.states + ((size_t)bh * p.Lmax + jb.level) * DK * p.dv
                      : p.ws + ((size_t)bh * p.njobs + job) * DK * p.dv) +
                 cb + wave * 16 + m16;
#pragma unroll
    for (int kt = 0; kt < NDT; ++kt) {
        // row of u[kt] (see tile_state): 32 (kt / 2) + 8g + 4 (kt % 2), or 4g for d_k = 16
        const int row = DK >= 32 ? 32 * (kt / 2) + 8 * g + 4 * (kt % 2) : 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(size_t)(row + i) * p.dv] = fin * u[kt][i];
    }
}

template <typename E>
__global__ __launch_bounds__(kThr) void k_prefill_part(PrefillParams p) {
    __shared__ float sk[kTile][129];  // K tile, fp32 (odd pitch: rows on distinct banks)
    __shared__ float4 sv[kTile][16];  // V tile, this block's columns (<= 64)
    __shared__ float se[kTile];       // per-token weights exp(A_{T-1} - A_s)
    __shared__ float sa[kTile];
    __shared__ float sred[kThr / 64];
    __shared__ float carry_s;

    const int dk = p.dk, dv = p.dv;
    const int dvw = dv < 64 ? dv : 64;
    const int ncb = dv / dvw;
    int blk = blockIdx.x;
    const int cb = blk % ncb;
    blk /= ncb;
    const int job = blk % p.njobs;
    const int bh = blk / p.njobs;
    const int tid = threadIdx.x;
    const int n = p.T - 1;
    const PrefillJob jb = prefill_job(n, job);

    const float* a = p.a + (size_t)bh * p.T;
    const E* k = static_cast<const E*>(p.k) + (size_t)bh * p.T * dk;
    const E* v = static_cast<const E*>(p.v) + (size_t)bh * p.T * dv + cb * dvw;

    // decay from the end of the job to position T - 1: sum of a over (s1 - 1, T - 1]
    float part = 0.f;
    for (int r = jb.s1 + tid; r < p.T; r += kThr) part += a[r];
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
    if ((tid & 63) == 0) sred[tid >> 6] = part;
    __syncthreads();
    if (tid == 0) {
        float c = 0.f;
        for (int w = 0; w < kThr / 64; ++w) c += sred[w];
        carry_s = c;
    }

    // output ownership: 4 consecutive columns and rows rg + nrg * i
    const int q4 = dvw / 4;          // column quads of the block
    const int cq = tid % q4;
    const int rg = tid / q4;
    const int nrg = kThr / q4;       // row groups
    const int nrow = (dk + nrg - 1) / nrg;
    float4 acc[8];                   // nrow <= 8 (dk <= 128, dvw >= 16 -> nrg <= 64)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);

    const int tfirst = jb.s0 / kTile, tlast = (jb.s1 - 1) / kTile;
    for (int tb = tlast; tb >= tfirst; --tb) {
        const int base = tb * kTile;
        __syncthreads();  // previous tile consumed; carry_s written
        if (tid < kTile) {
            const int s = base + tid;
            sa[tid] = (s >= jb.s0 && s < jb.s1) ? a[s] : 0.f;
        }
        for (int x = tid; x < kTile * dk; x += kThr) {
            const int s = x / dk, c = x % dk;
            const int g = base + s;
            sk[s][c] = g < p.T ? to_f32(k[(size_t)g * dk + c]) : 0.f;
        }
        for (int x = tid; x < kTile * q4; x += kThr) {
            const int s = x / q4, c4 = x % q4;
            const int g = base + s;
            float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
            if (g < p.T) {
                const E* vr = v + (size_t)g * dv + 4 * c4;
                y = make_float4(to_f32(vr[0]), to_f32(vr[1]), to_f32(vr[2]), to_f32(vr[3]));
            }
            sv[s][c4] = y;
        }
        __syncthreads();
        if (tid < kTile) {
            // tokens after s inside this tile and the job, then everything after it
            float suf = 0.f;
            for (int r = tid + 1; r < kTile; ++r) suf += sa[r];
            const int s = base + tid;
            se[tid] = (s >= jb.s0 && s < jb.s1) ? __expf(suf + carry_s) : 0.f;
        }
        __syncthreads();
        if (tid == 0) {
            float t = 0.f;
            for (int r = 0; r < kTile; ++r) t += sa[r];
            carry_s += t;
        }
        for (int s = 0; s < kTile; ++s) {
            const float e = se[s];
            if (e == 0.f) continue;  // uniform: outside the job
            const float4 vv = sv[s][cq];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i < nrow) {
                    const int r = rg + nrg * i;
                    if (r < dk) {
                        const float w = e * sk[s][r];
                        acc[i].x += w * vv.x;
                        acc[i].y += w * vv.y;
                        acc[i].z += w * vv.z;
                        acc[i].w += w * vv.w;
                    }
                }
            }
        }
    }
    // the level's state, or the partial [bh][job][dk][dv]
    float* dst = (prefill_single(jb.level) ? p.states + ((size_t)bh * p.Lmax + jb.level) * dk * dv
                                           : p.ws + ((size_t)bh * p.njobs + job) * dk * dv) +
                 cb * dvw + 4 * cq;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = rg + nrg * i;
        if (i < nrow && r < dk) *reinterpret_cast<float4*>(dst + (size_t)r * dv) = acc[i];
    }
}

__global__ __launch_bounds__(kThr) void k_prefill_sum(PrefillParams p) {
    // block: (bh, level, element chunk of kThr float4)
    const size_t n4 = (size_t)p.dk * p.dv / 4;
    const int nchunk = (int)((n4 + kThr - 1) / kThr);
    int blk = blockIdx.x;
    const int chunk = blk % nchunk;
    blk /= nchunk;
    const int level = blk % p.Lmax;
    const int bh = blk / p.Lmax;
    const size_t e = (size_t)chunk * kThr + threadIdx.x;
    if (e >= n4) return;
    const int n = p.T - 1;
    // n < 2^30, so no slot above level 31 is live (and the shift below
    // stays within the 32-bit word)
    const bool live = n >= 0 && (level == 0 || (level <= 31 && ((n >> (level - 1)) & 1)));
    if (live && prefill_single(level)) return;  // written by its job
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
        // the pieces of a long bucket are consecutive jobs from the first
        // piece: floor(s0 / kPrefillJobTokens) of the bucket's first token
        const float4* ws = reinterpret_cast<const float4*>(p.ws) + (size_t)bh * p.njobs * n4;
        const int first = ((n >> level) << level) / kPrefillJobTokens;
        const int count = (1 << (level - 1)) / kPrefillJobTokens;
        // four pieces' loads in flight at a time (the sum order is kept)
        int j = first;
        for (; j + 4 <= first + count; j += 4) {
            float4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = ws[(size_t)(j + u) * n4 + e];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                s.x += x[u].x; s.y += x[u].y; s.z += x[u].z; s.w += x[u].w;
            }
        }
        for (; j < first + count; ++j) {
            const float4 x = ws[(size_t)j * n4 + e];
            s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
        }
    }
    reinterpret_cast<float4*>(p.states)[((size_t)bh * p.Lmax + level) * n4 + e] = s;
}

}  // namespace

int prefill_jobs(int T) {
    if (T <= 0) return 0;
    const int n = T - 1;
    return n / kPrefillJobTokens + __builtin_popcount((unsigned)(n % kPrefillJobTokens)) + 1;
}

namespace {
template <int DK>
hipError_t launch_prefill_dk(const PrefillParams& p, hipStream_t stream) {
    const int dvw = p.dv >= 64 ? 64 : p.dv;
    const unsigned nb = (unsigned)((long)p.BH * p.njobs * (p.dv / dvw));
    switch (dvw) {
        case 16: hipLaunchKernelGGL((k_prefill_job<DK, 1>), dim3(nb), dim3(64), 0, stream, p); break;
        case 32: hipLaunchKernelGGL((k_prefill_job<DK, 2>), dim3(nb), dim3(128), 0, stream, p); break;
        case 64: hipLaunchKernelGGL((k_prefill_job<DK, 4>), dim3(nb), dim3(256), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill_jobs_bf16(const PrefillParams& p, hipStream_t stream) {
    switch (p.dk) {
        case 16: return launch_prefill_dk<16>(p, stream);
        case 32: return launch_prefill_dk<32>(p, stream);
        case 64: return launch_prefill_dk<64>(p, stream);
        case 128: return launch_prefill_dk<128>(p, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_states(const PrefillParams& p, bool bf16, hipStream_t stream) {
    const int dvw = p.dv < 64 ? p.dv : 64;
    if (p.njobs > 0) {
        hipError_t e;
        if (bf16) {
            e = launch_prefill_jobs_bf16(p, stream);
        } else {
            const unsigned nb = (unsigned)((long)p.BH * p.njobs * (p.dv / dvw));
            hipLaunchKernelGGL(k_prefill_part<float>, dim3(nb), dim3(kThr), 0, stream, p);
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
    }
    const size_t n4 = (size_t)p.dk * p.dv / 4;
    const unsigned nchunk = (unsigned)((n4 + kThr - 1) / kThr);
    hipLaunchKernelGGL(k_prefill_sum, dim3((unsigned)p.BH * p.Lmax * nchunk), dim3(kThr), 0, stream, p);
    return hipGetLastError();
}

}  // namespace loglin
