// Fenwick decode step, state export and level map on gfx950.
//
// "Log-linear attention, and what a logarithm buys", section 2: the decode
// recurrence is the Fenwick update.  At position t >= 1 with j = lssb(t), the
// new token's outer product enters level 0, levels 0..j (the old token and
// the buckets of the trailing one bits of t-1) are summed and promoted to
// level j+1, and, composing with the Mamba-2 scalar gate (sections 1 and 3),
// every carried state is decayed by alpha_t = exp(a_t).  The output reads
// o_t = sum_l lambda_t^(l) q_t^T S_t^(l) over the live levels.
//
// Storage: a level held as a matrix keeps an fp32 d_k x d_v matrix X and a
// log-scale sigma, the state being S = exp(sigma) X; decaying it only adds a_t
// to sigma.  Levels 0..6 are kept as the raw rows of the current 64-token
// window (see k_decode_step).  Slots that are not live are neither read nor
// written (their contents are stale; the export zeroes them, applies the
// scales and expands the window levels).
#include "common.hpp"
#include "kernels.hpp"

namespace loglin {

namespace {

constexpr int kThreads = 256;

// level matrices are streamed once per step: non-temporal 16-byte accesses
__device__ __forceinline__ float4 ld_stream(const float4* p) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void st_stream(float4* p, const float4& v) {
    const f32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}
constexpr int kMaxPer = 16;  // float4 elements per thread for a 128 x 128 state

// Storage of the scalar-gated mixer's state.  Levels 0..6 of query t hold
// exactly the tokens of t's 64-token window [t & ~63, t] (a level l <= 6
// bucket holds 2^(l-1) < 64 tokens next to t), so those levels are kept as
// the window's raw rows k_s, v_s with the running sum c_s of a from the window
// start: token s weighs exp(c_t - c_s) and its level is level(t, s).  A step
// inside a window moves no state at all; at a multiple of 64 the finished
// window (64 tokens) and the levels 7..j below the merge are summed into the
// level-j+1 matrix.  Levels 7 and up are fp32 matrices with log-scales.
// After a load the loaded levels 0..6 are matrices, so until the next
// multiple of 64 the step keeps every level as a matrix (level 0 as the last
// token's vectors) -- the "matrix" path below; the first window boundary
// merges them into a level >= 7 and the window path takes over.
constexpr int kWin = 64;
constexpr int kWinLevels = 7;  // levels 0..6 live inside the window
constexpr int kStageTok = 16;  // window tokens staged per pass of the merge

template <typename E>
__global__ __launch_bounds__(kThreads) void k_decode_step(DecodeParams p) {
    __shared__ float qs[128], ks[128], vs[128];
    __shared__ float k0[128], v0[128];  // the previous token: level 0 when raw0 (matrix path)
    __shared__ float sig_s[64];
    __shared__ float4 red[kThreads];
    __shared__ float sw[kWin];                        // window token weights
    __shared__ __align__(16) float stg[kStageTok * 256];  // window rows staged for the merge
    const int sh = blockIdx.x;  // sequence * H + head
    const int seq = sh / p.H;
    const int tid = threadIdx.x;
    const int64_t base = p.base_pos[seq];
    const int64_t t = base + p.step;
    const int64_t w0 = t & ~(int64_t)(kWin - 1);
    const bool window = p.window && w0 >= base;  // uniform over the block
    const int dk = p.dk, dv = p.dv;

    const E* q = static_cast<const E*>(p.q) + (size_t)sh * dk;
    const E* k = static_cast<const E*>(p.k) + (size_t)sh * dk;
    const E* v = static_cast<const E*>(p.v) + (size_t)sh * dv;
    float* sig = p.sigma + (size_t)sh * p.Lmax;
    if (tid < dk) {
        qs[tid] = to_f32(q[tid]);
        ks[tid] = to_f32(k[tid]);
    }
    if (tid < dv) vs[tid] = to_f32(v[tid]);
    if (tid < p.Lmax) sig_s[tid] = sig[tid];
    float* raw = p.raw + (size_t)sh * (dk + dv);
    if (p.raw0) {  // read by the matrix path and by a window boundary right after it
        if (tid < dk) k0[tid] = raw[tid];
        if (tid < dv) v0[tid] = raw[dk + tid];
    }
    __syncthreads();
    if (!window) {
        // this token becomes level 0 (every thread has read the previous one)
        if (tid < dk) raw[tid] = ks[tid];
        if (tid < dv) raw[dk + tid] = vs[tid];
    }

    const float a = p.a[sh];
    const float alpha = __expf(a);
    const float* lam = p.lam + (size_t)sh * p.Lmax;
    const size_t nst4 = (size_t)dk * dv / 4;
    float4* X = reinterpret_cast<float4*>(p.states) + (size_t)sh * p.Lmax * nst4;
    const int quads = dv / 4;
    const int col = (tid % quads) * 4;  // the same for every element of this thread

    // positions of this thread: e4 = tid + kThreads * u, in row r0 + u * rstep
    // (4 kThreads is a multiple of every supported dv)
    const int r0 = tid * 4 / dv, rstep = kThreads * 4 / dv;
    auto row = [&](int u) { return r0 + u * rstep; };
    auto valid = [&](int u) { return (size_t)(tid + kThreads * u) < nst4; };

    float4 part = make_float4(0.f, 0.f, 0.f, 0.f);
    auto accum = [&](float w, float qr, const float4& x) {
        const float f = w * qr;
        part.x += f * x.x;
        part.y += f * x.y;
        part.z += f * x.z;
        part.w += f * x.w;
    };
    auto add_scaled = [&](float4* acc, const float4* src, float w) {
        float4 x[kMaxPer];
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u)
            if (valid(u)) x[u] = ld_stream(src + tid + kThreads * u);
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u) {
            if (valid(u)) {
                acc[u].x += w * x[u].x;
                acc[u].y += w * x[u].y;
                acc[u].z += w * x[u].z;
                acc[u].w += w * x[u].w;
            }
        }
    };
    // live levels above j+1 (set bits of t there): decay through the scale, read
    auto carried = [&](int from) {
        for (uint64_t hb = (uint64_t)t >> (from - 1); hb; hb &= hb - 1) {
            const int l = from + __builtin_ctzll(hb);
            const float w = lam[l] * __expf(sig_s[l] + a);
            const float4* s = X + (size_t)l * nst4;
            float4 x[kMaxPer];
#pragma unroll
            for (int u = 0; u < kMaxPer; ++u)
                if (valid(u)) x[u] = ld_stream(s + tid + kThreads * u);
#pragma unroll
            for (int u = 0; u < kMaxPer; ++u)
                if (valid(u)) accum(w, qs[row(u)], x[u]);
        }
    };

    const int dw = dk + dv;  // floats per window row
    float* Wr = p.win + (size_t)sh * kWin * dw;
    float* Wc = p.wc + (size_t)sh * kWin;
    const int m = (int)(t - w0);  // slot of token t in its window
    float ct = 0.f;               // c_t: sum of a over the window up to t
    int j = -1;
    if (window) {
        ct = (m > 0 ? Wc[m - 1] : 0.f) + a;
        if (t >= 1 && m == 0) {
            // a window ends: its 64 tokens (levels 0..6) and the matrix levels
            // 7..j, decayed to t, become level j+1
            j = lssb((uint64_t)t);
            float4 acc[kMaxPer];
#pragma unroll
            for (int u = 0; u < kMaxPer; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t - kWin >= base) {
                const float clast = Wc[kWin - 1];
                for (int s0 = 0; s0 < kWin; s0 += kStageTok) {
                    __syncthreads();  // the previous pass is done with stg
                    for (int e = tid; e < kStageTok * dw; e += kThreads) {
                        const int s = e / dw, x = e - s * dw;
                        float val = Wr[(size_t)(s0 + s) * dw + x];
                        if (x >= dk) val *= __expf(a + clast - Wc[s0 + s]);
                        stg[s * dw + x] = val;
                    }
                    __syncthreads();
#pragma unroll 4
                    for (int s = 0; s < kStageTok; ++s) {
                        const float* kr = stg + s * dw;
                        const float4 vv = *reinterpret_cast<const float4*>(kr + dk + col);
#pragma unroll
                        for (int u = 0; u < kMaxPer; ++u) {
                            if (valid(u)) {
                                const float kk = kr[row(u)];
                                acc[u].x += kk * vv.x;
                                acc[u].y += kk * vv.y;
                                acc[u].z += kk * vv.z;
                                acc[u].w += kk * vv.w;
                            }
                        }
                    }
                }
                for (int l = kWinLevels; l <= j; ++l) add_scaled(acc, X + (size_t)l * nst4, __expf(a + sig_s[l]));
            } else {
                // the previous window began before the last load: its levels are
                // matrices (level 0 the previous token's vectors once a step ran)
                int lfirst = 0;
                if (p.raw0) {
                    const float w = alpha * __expf(sig_s[0]);
                    const float4 vv = make_float4(w * v0[col], w * v0[col + 1], w * v0[col + 2],
                                                  w * v0[col + 3]);
#pragma unroll
                    for (int u = 0; u < kMaxPer; ++u) {
                        if (valid(u)) {
                            const float kr = k0[row(u)];
                            acc[u].x += kr * vv.x;
                            acc[u].y += kr * vv.y;
                            acc[u].z += kr * vv.z;
                            acc[u].w += kr * vv.w;
                        }
                    }
                    lfirst = 1;
                }
                for (int l = lfirst; l <= j; ++l) add_scaled(acc, X + (size_t)l * nst4, alpha * __expf(sig_s[l]));
            }
            float4* dst = X + (size_t)(j + 1) * nst4;
            const float lj = lam[j + 1];
#pragma unroll
            for (int u = 0; u < kMaxPer; ++u) {
                if (valid(u)) {
                    st_stream(dst + tid + kThreads * u, acc[u]);
                    accum(lj, qs[row(u)], acc[u]);
                }
            }
            carried(j + 2);
        } else if (t >= 1) {
            carried(kWinLevels);  // inside a window only the matrix levels carry
        }
        // the window's tokens s <= t: weight lambda_t^(level) e^(c_t - c_s) (q . k_s)
        {
            const int s = tid >> 2, qu = tid & 3;
            const int per = dk / 4;
            float d = 0.f;
            if (s < m) {
                const float* kr = Wr + (size_t)s * dw + qu * per;
                for (int x = 0; x < per; x += 4) {
                    const float4 kk = *reinterpret_cast<const float4*>(kr + x);
                    const float* qq = qs + qu * per + x;
                    d += qq[0] * kk.x + qq[1] * kk.y + qq[2] * kk.z + qq[3] * kk.w;
                }
            } else if (s == m) {
                for (int x = qu * per; x < (qu + 1) * per; ++x) d += qs[x] * ks[x];
            }
            d += __shfl_xor(d, 1, kWave);
            d += __shfl_xor(d, 2, kWave);
            if (qu == 0 && s <= m) {
                const int lev = fenwick_level((uint32_t)m, (uint32_t)s);
                const float cs = s < m ? Wc[s] : ct;
                sw[s] = lam[lev] * __expf(ct - cs) * d;
            }
        }
        __syncthreads();
        {
            const int G = kThreads / quads;
            for (int s = tid / quads; s <= m; s += G) {
                const float w = sw[s];
                float4 vv;
                if (s < m)
                    vv = *reinterpret_cast<const float4*>(Wr + (size_t)s * dw + dk + col);
                else
                    vv = make_float4(vs[col], vs[col + 1], vs[col + 2], vs[col + 3]);
                part.x += w * vv.x;
                part.y += w * vv.y;
                part.z += w * vv.z;
                part.w += w * vv.w;
            }
        }
        // token t joins the window (every read of the old rows is behind the
        // barrier above)
        for (int x = tid; x < dw; x += kThreads) Wr[(size_t)m * dw + x] = x < dk ? ks[x] : vs[x - dk];
        if (tid == 0) Wc[m] = ct;
    } else {
        if (t >= 1) {
            j = lssb((uint64_t)t);
            // merge levels 0..j (decayed by their scales) into level j+1
            float4 acc[kMaxPer];
#pragma unroll
            for (int u = 0; u < kMaxPer; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            int lfirst = 0;
            if (p.raw0) {  // level 0 = k0 v0^T
                const float w = alpha * __expf(sig_s[0]);
                const float4 vv = make_float4(w * v0[col], w * v0[col + 1], w * v0[col + 2], w * v0[col + 3]);
#pragma unroll
                for (int u = 0; u < kMaxPer; ++u) {
                    if (valid(u)) {
                        const float kr = k0[row(u)];
                        acc[u].x += kr * vv.x;
                        acc[u].y += kr * vv.y;
                        acc[u].z += kr * vv.z;
                        acc[u].w += kr * vv.w;
                    }
                }
                lfirst = 1;
            }
            for (int l = lfirst; l <= j; ++l) add_scaled(acc, X + (size_t)l * nst4, alpha * __expf(sig_s[l]));
            float4* dst = X + (size_t)(j + 1) * nst4;
            const float lj = lam[j + 1];
#pragma unroll
            for (int u = 0; u < kMaxPer; ++u) {
                if (valid(u)) {
                    st_stream(dst + tid + kThreads * u, acc[u]);
                    accum(lj, qs[row(u)], acc[u]);
                }
            }
            carried(j + 2);
        }
        // level 0 holds the new token alone (kept as k, v above)
        const float l0 = lam[0];
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u) {
            if (valid(u)) {
                const float kr = ks[row(u)];
                const float4 y = make_float4(kr * vs[col], kr * vs[col + 1], kr * vs[col + 2],
                                             kr * vs[col + 3]);
                accum(l0, qs[row(u)], y);
            }
        }
    }

    __syncthreads();  // red is free
    red[tid] = part;
    __syncthreads();
    if (tid < quads) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int r = tid; r < kThreads; r += quads) {
            o.x += red[r].x;
            o.y += red[r].y;
            o.z += red[r].z;
            o.w += red[r].w;
        }
        *reinterpret_cast<float4*>(p.out + (size_t)sh * dv + col) = o;
    }
    // new scales: 0 for the rewritten levels, + a for the carried ones
    if (tid < p.Lmax) {
        float s = sig_s[tid];
        if (tid == 0 || tid == j + 1) s = 0.f;
        else if (t >= 1 && tid > j + 1 && (((uint64_t)t >> (tid - 1)) & 1)) s += a;
        sig[tid] = s;
    }
}

// Level states of the recurrence: the stored matrices with their scales, level
// 0 expanded from the last token's vectors, levels 0..6 of a window summed
// from its rows; slots that are not live are zero.
__global__ void k_state_export(DecodeParams p, float4* dst) {
    const size_t nst4 = (size_t)p.dk * p.dv / 4;
    const size_t total = (size_t)p.nseq * p.H * p.Lmax * nst4;
    const float4* src = reinterpret_cast<const float4*>(p.states);
    const int dw = p.dk + p.dv;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (size_t)gridDim.x * blockDim.x) {
        const size_t slot = e / nst4;  // (seq * H + h) * Lmax + l
        const int l = (int)(slot % p.Lmax);
        const size_t pair = slot / p.Lmax;
        const int seq = (int)(pair / p.H);
        const int64_t base = p.base_pos[seq];
        const int64_t n = base + p.step;  // tokens absorbed so far
        bool live = false;
        if (n >= 1) live = (l == 0) || (l <= 63 && (((uint64_t)(n - 1) >> (l - 1)) & 1));
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live) {
            const int64_t tl = n - 1;
            const int64_t w0 = tl & ~(int64_t)(kWin - 1);
            const size_t idx = (e % nst4) * 4;
            const int r = (int)(idx / p.dv), c = (int)(idx % p.dv);
            if (p.window && w0 >= base && l < kWinLevels) {
                // the bucket of level l of query tl, inside its window
                const int ml = (int)(tl - w0);
                const int s0 = l == 0 ? ml : ((ml >> l) << l);
                const int s1 = l == 0 ? ml + 1 : s0 + (1 << (l - 1));
                const float* Wr = p.win + pair * kWin * dw;
                const float* Wc = p.wc + pair * kWin;
                const float cl = Wc[ml];
                for (int s = s0; s < s1; ++s) {
                    const float w = __expf(cl - Wc[s]) * Wr[(size_t)s * dw + r];
                    const float* vr = Wr + (size_t)s * dw + p.dk + c;
                    x.x += w * vr[0];
                    x.y += w * vr[1];
                    x.z += w * vr[2];
                    x.w += w * vr[3];
                }
            } else {
                const float w = __expf(p.sigma[slot]);
                if (l == 0 && p.raw0) {  // k v^T of the newest token
                    const float* raw = p.raw + pair * (p.dk + p.dv);
                    const float kr = raw[r];
                    x = make_float4(kr * raw[p.dk + c], kr * raw[p.dk + c + 1], kr * raw[p.dk + c + 2],
                                    kr * raw[p.dk + c + 3]);
                } else {
                    x = src[e];
                }
                x.x *= w; x.y *= w; x.z *= w; x.w *= w;
            }
        }
        dst[e] = x;
    }
}

__global__ void k_level_map(int T, int8_t* out) {
    const size_t total = (size_t)T * T;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (size_t)gridDim.x * blockDim.x) {
        const int t = (int)(e / T), s = (int)(e % T);
        out[e] = s > t ? (int8_t)-1 : (int8_t)fenwick_level((uint32_t)t, (uint32_t)s);
    }
}

}  // namespace

hipError_t launch_decode_step(const DecodeParams& p, bool bf16, hipStream_t stream) {
    const unsigned nblk = (unsigned)p.nseq * p.H;
    if (bf16)
        hipLaunchKernelGGL(k_decode_step<bf16_t>, dim3(nblk), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(k_decode_step<float>, dim3(nblk), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_state_export(const DecodeParams& p, float* dst, hipStream_t stream) {
    const size_t total = (size_t)p.nseq * p.H * p.Lmax * p.dk * p.dv / 4;
    const unsigned nblk = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
    hipLaunchKernelGGL(k_state_export, dim3(nblk), dim3(256), 0, stream, p,
                       reinterpret_cast<float4*>(dst));
    return hipGetLastError();
}

hipError_t launch_level_map(int T, int8_t* out, hipStream_t stream) {
    const size_t total = (size_t)T * T;
    const unsigned nblk = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
    hipLaunchKernelGGL(k_level_map, dim3(nblk), dim3(256), 0, stream, T, out);
    return hipGetLastError();
}

}  // namespace loglin
