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
// Storage: each level keeps an fp32 d_k x d_v matrix X and a log-scale sigma,
// the state being S = exp(sigma) X.  Decaying a level only adds a_t to its
// sigma.  Level 0 only ever holds the newest token's k v^T, so after the first
// step it is kept as the two vectors k and v (raw0) and expanded where it is
// used.  A step then writes one matrix (the merged level j+1) and reads the
// popcount(t-1) live levels above 0, which the output needs anyway.  Slots that
// are not live are neither read nor written (their contents are stale; the
// export zeroes them, applies the scales and expands level 0).
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

template <typename E>
__global__ __launch_bounds__(kThreads) void k_decode_step(DecodeParams p) {
    __shared__ float qs[128], ks[128], vs[128];
    __shared__ float k0[128], v0[128];  // the previous token: level 0 when raw0
    __shared__ float sig_s[64];
    __shared__ float4 red[kThreads];
    const int sh = blockIdx.x;  // sequence * H + head
    const int seq = sh / p.H;
    const int tid = threadIdx.x;
    const int64_t t = p.base_pos[seq] + p.step;
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
    if (p.raw0) {
        if (tid < dk) k0[tid] = raw[tid];
        if (tid < dv) v0[tid] = raw[dk + tid];
    }
    __syncthreads();
    // this token becomes level 0 (every thread has read the previous one)
    if (tid < dk) raw[tid] = ks[tid];
    if (tid < dv) raw[dk + tid] = vs[tid];

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

    int j = -1;
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
        for (int l = lfirst; l <= j; ++l) {
            const float w = alpha * __expf(sig_s[l]);
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
        float4* dst = X + (size_t)(j + 1) * nst4;
        const float lj = lam[j + 1];
#pragma unroll
        for (int u = 0; u < kMaxPer; ++u) {
            if (valid(u)) {
                st_stream(dst + tid + kThreads * u, acc[u]);
                accum(lj, qs[row(u)], acc[u]);
            }
        }
        // live levels above j+1: decay through the scale, read for the output
        for (uint64_t hb = (uint64_t)t >> (j + 1); hb; hb &= hb - 1) {
            const int l = j + 2 + __builtin_ctzll(hb);
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

__global__ void k_state_export(DecodeParams p, float4* dst) {
    const size_t nst4 = (size_t)p.dk * p.dv / 4;
    const size_t total = (size_t)p.nseq * p.H * p.Lmax * nst4;
    const float4* src = reinterpret_cast<const float4*>(p.states);
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (size_t)gridDim.x * blockDim.x) {
        const size_t slot = e / nst4;  // (seq * H + h) * Lmax + l
        const int l = (int)(slot % p.Lmax);
        const int seq = (int)(slot / ((size_t)p.Lmax * p.H));
        const int64_t n = p.base_pos[seq] + p.step;  // tokens absorbed so far
        bool live = false;
        if (n >= 1) live = (l == 0) || (((uint64_t)(n - 1) >> (l - 1)) & 1);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live) {
            const float w = __expf(p.sigma[slot]);
            if (l == 0 && p.raw0) {  // k v^T of the newest token
                const size_t idx = (e % nst4) * 4;
                const int r = (int)(idx / p.dv), c = (int)(idx % p.dv);
                const float* raw = p.raw + (slot / p.Lmax) * (p.dk + p.dv);
                const float kr = raw[r];
                x = make_float4(kr * raw[p.dk + c], kr * raw[p.dk + c + 1], kr * raw[p.dk + c + 2],
                                kr * raw[p.dk + c + 3]);
            } else {
                x = src[e];
            }
            x.x *= w; x.y *= w; x.z *= w; x.w *= w;
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
