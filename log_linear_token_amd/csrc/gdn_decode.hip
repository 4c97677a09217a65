// Decode step of the log-linear Gated DeltaNet on gfx950.
//
// "Log-linear attention, and what a logarithm buys", section 2: the decode
// recurrence is the Fenwick update (levels 0..lssb(t) merged and promoted
// one level, the new token entering level 0); for the Gated DeltaNet lift
// (sections 1 and 3) every carried and merged state takes the gated
// delta-rule transition of the Gated DeltaNet paper (the page's source 3),
//     G_t = alpha_t (I - beta_t k_t k_t^T),  and the new token writes beta_t k_t v_t^T.
//
// Storage is the decode state of the scalar-gated mixer: each level an fp32
// d_k x d_v matrix X with a log-scale sigma (state exp(sigma) X), level 0 the
// newest token's k and (here beta-scaled) v.  The scalar part of G_t still
// goes into sigma; the rank-one part (I - beta k k^T) changes the matrix, so
// every live level is read, updated in registers and written back:
//     X <- X - beta k (k^T X),  sigma <- sigma + a_t.
// One block of 256 threads per (sequence, head); each thread holds 16 float4
// of a 128 x 128 level and the block reduces k^T X over the rows.
#include "common.hpp"
#include "kernels.hpp"

namespace loglin {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxPer = 16;  // float4 elements per thread for a 128 x 128 state

__device__ __forceinline__ float4 ld_stream(const float4* p) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void st_stream(float4* p, const float4& v) {
    const f32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

template <typename E>
__global__ __launch_bounds__(kThreads) void k_gdn_decode_step(DecodeParams p, const float* beta_in) {
    __shared__ float qs[128], ks[128], vs[128];
    __shared__ float k0[128], v0[128];  // the previous token (level 0 when raw0)
    __shared__ float sig_s[64];
    __shared__ float4 red[kThreads];
    __shared__ float4 wsum[32];         // k^T X of the level being updated, per column quad
    const int sh = blockIdx.x;
    const int seq = sh / p.H;
    const int tid = threadIdx.x;
    const int64_t t = p.base_pos[seq] + p.step;
    const int dk = p.dk, dv = p.dv;
    const float beta = beta_in[sh];

    const E* q = static_cast<const E*>(p.q) + (size_t)sh * dk;
    const E* k = static_cast<const E*>(p.k) + (size_t)sh * dk;
    const E* v = static_cast<const E*>(p.v) + (size_t)sh * dv;
    float* sig = p.sigma + (size_t)sh * p.Lmax;
    if (tid < dk) {
        qs[tid] = to_f32(q[tid]);
        ks[tid] = to_f32(k[tid]);
    }
    if (tid < dv) vs[tid] = beta * to_f32(v[tid]);  // the token writes beta k v^T
    if (tid < p.Lmax) sig_s[tid] = sig[tid];
    float* raw = p.raw + (size_t)sh * (dk + dv);
    if (p.raw0) {
        if (tid < dk) k0[tid] = raw[tid];
        if (tid < dv) v0[tid] = raw[dk + tid];
    }
    __syncthreads();
    if (tid < dk) raw[tid] = ks[tid];
    if (tid < dv) raw[dk + tid] = vs[tid];

    const float a = p.a[sh];
    const float alpha = __expf(a);
    const float* lam = p.lam + (size_t)sh * p.Lmax;
    const size_t nst4 = (size_t)dk * dv / 4;
    float4* X = reinterpret_cast<float4*>(p.states) + (size_t)sh * p.Lmax * nst4;
    const int quads = dv / 4;
    const int cq = tid % quads;
    const int col = cq * 4;
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
    // x <- s (x - beta k (k^T x)) for the level held in x (every thread)
    auto delta = [&](float4* x, float s) {
        float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u) {
            if (valid(u)) {
                const float kr = ks[row(u)];
                w.x += kr * x[u].x;
                w.y += kr * x[u].y;
                w.z += kr * x[u].z;
                w.w += kr * x[u].w;
            }
        }
        __syncthreads();  // red and wsum are free (previous level done)
        red[tid] = w;
        __syncthreads();
        if (tid < quads) {
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int r = tid; r < kThreads; r += quads) {
                o.x += red[r].x;
                o.y += red[r].y;
                o.z += red[r].z;
                o.w += red[r].w;
            }
            wsum[tid] = o;
        }
        __syncthreads();
        const float4 ww = wsum[cq];
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u) {
            if (valid(u)) {
                const float bk = beta * ks[row(u)];
                x[u].x = s * (x[u].x - bk * ww.x);
                x[u].y = s * (x[u].y - bk * ww.y);
                x[u].z = s * (x[u].z - bk * ww.z);
                x[u].w = s * (x[u].w - bk * ww.w);
            }
        }
    };

    int j = -1;
    if (t >= 1) {
        j = lssb((uint64_t)t);
        // levels 0..j (with their scales) summed, then taken through G_t
        float4 acc[kMaxPer];
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        int lfirst = 0;
        if (p.raw0) {
            const float w = __expf(sig_s[0]);
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
        for (int l = lfirst; l <= j; ++l) {
            const float w = __expf(sig_s[l]);
            const float4* src = X + (size_t)l * nst4;
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
        }
        delta(acc, alpha);
        float4* dst = X + (size_t)(j + 1) * nst4;
        const float lj = lam[j + 1];
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u) {
            if (valid(u)) {
                st_stream(dst + tid + kThreads * u, acc[u]);
                accum(lj, qs[row(u)], acc[u]);
            }
        }
        // live levels above j+1: the rank-one part on the matrix, alpha on the scale
        for (uint64_t hb = (uint64_t)t >> (j + 1); hb; hb &= hb - 1) {
            const int l = j + 2 + __builtin_ctzll(hb);
            float4* s = X + (size_t)l * nst4;
            float4 x[kMaxPer];
#pragma unroll
            for (int u = 0; u < kMaxPer; ++u)
                if (valid(u)) x[u] = ld_stream(s + tid + kThreads * u);
            delta(x, 1.f);
            const float w = lam[l] * __expf(sig_s[l] + a);
#pragma unroll
            for (int u = 0; u < kMaxPer; ++u) {
                if (valid(u)) {
                    st_stream(s + tid + kThreads * u, x[u]);
                    accum(w, qs[row(u)], x[u]);
                }
            }
        }
    }
    // level 0: the new token's beta k v^T alone
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

    __syncthreads();  // the last reduction's reads of red are done
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
    if (tid < p.Lmax) {
        float s = sig_s[tid];
        if (tid == 0 || tid == j + 1) s = 0.f;
        else if (t >= 1 && tid > j + 1 && (((uint64_t)t >> (tid - 1)) & 1)) s += a;
        sig[tid] = s;
    }
}

}  // namespace

hipError_t launch_gdn_decode_step(const DecodeParams& p, const float* beta, bool bf16,
                                  hipStream_t stream) {
    const unsigned nblk = (unsigned)p.nseq * p.H;
    if (bf16)
        hipLaunchKernelGGL(k_gdn_decode_step<bf16_t>, dim3(nblk), dim3(kThreads), 0, stream, p, beta);
    else
        hipLaunchKernelGGL(k_gdn_decode_step<float>, dim3(nblk), dim3(kThreads), 0, stream, p, beta);
    return hipGetLastError();
}

}  // namespace loglin
