// C ABI of libloglin.so: argument checks on the host, workspace carving,
// decode-state lifecycle, and the launches.  Declared in include/loglin.h.
#include "loglin.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "kernels.hpp"

using namespace loglin;

namespace {

thread_local char g_err[512] = "";

loglin_status fail(loglin_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

loglin_status ok() {
    g_err[0] = '\0';
    return LOGLIN_OK;
}

loglin_status hip_fail(hipError_t e, const char* where) {
    return fail(LOGLIN_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int bit_length(long x) {
    int n = 0;
    while (x > 0) {
        ++n;
        x >>= 1;
    }
    return n;
}

// levels a sequence of T tokens uses: level 0 and up to bit_length(T-1)
int levels_needed(long T) { return T <= 1 ? 1 : bit_length(T - 1) + 1; }

constexpr long kMaxChunks = 65536;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Checks shared by the workspace query and the forward; on failure sets the
// error text and returns the status.
loglin_status check_fwd_sizes(int B, int H, int T, int dk, int dv, int C) {
    if (B < 0 || H < 0 || T < 0)
        return fail(LOGLIN_EINVAL, "B, H, T must be >= 0 (got %d, %d, %d)", B, H, T);
    if (!supported_dim(C)) return fail(LOGLIN_EUNSUPPORTED, "chunk size C=%d not in {16,32,64,128}", C);
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LOGLIN_EUNSUPPORTED, "head dims dk=%d dv=%d must be in {16,32,64,128}", dk, dv);
    const long N = ((long)T + C - 1) / C;
    if (N > kMaxChunks)
        return fail(LOGLIN_EUNSUPPORTED, "T/C = %ld chunks exceeds %ld", N, kMaxChunks);
    if ((long)B * H * N > 0x7fffffffL)
        return fail(LOGLIN_EUNSUPPORTED, "B*H*ceil(T/C) = %ld blocks is too many", (long)B * H * N);
    return LOGLIN_OK;
}

}  // namespace

namespace loglin {
// the C ABI's error reporting for entry points defined in other sources
loglin_status api_fail(loglin_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

FwdWorkspace fwd_workspace_layout(long BH, long N, int dk, int dv, bool frags, int nsub) {
    FwdWorkspace w{};
    if (N <= 1 || BH == 0) return w;
    w.ust_off = 0;
    w.tot_off = align_up(w.ust_off + (size_t)BH * N * dv * dk * sizeof(float));
    w.cum_off = align_up(w.tot_off + (size_t)BH * N * sizeof(float));
    w.frag_off = align_up(w.cum_off + (size_t)BH * N * sizeof(double));
    w.upart_off = frags ? align_up(w.frag_off + (size_t)BH * N * dv * dk * 2) : w.frag_off;
    w.tpart_off = nsub > 1 ? align_up(w.upart_off + (size_t)BH * N * nsub * dv * dk * sizeof(float))
                           : w.upart_off;
    w.total = nsub > 1 ? align_up(w.tpart_off + (size_t)BH * N * nsub * sizeof(float)) : w.tpart_off;
    return w;
}
}  // namespace loglin

namespace {

enum Path { kPathChunked = 0, kPathFused = 1 };

// LOGLIN_FWD_PATH=chunked forces the three-kernel chunked path for bf16
// inputs as well (the fused path is the default where it applies).
bool force_chunked() {
    const char* e = getenv("LOGLIN_FWD_PATH");
    return e && strcmp(e, "chunked") == 0;
}

// LOGLIN_FUSED_SEGMENT=<tiles> (a power of two, 1..32) fixes the fused path's
// segment length; -1 when unset (the planner chooses).
int forced_segment_log2() {
    const char* e = getenv("LOGLIN_FUSED_SEGMENT");
    if (!e || !*e) return -1;
    const long n = strtol(e, nullptr, 10);
    for (int m = 0; m <= 5; ++m)
        if (n == (1L << m)) return m;
    return -1;
}

// LOGLIN_FUSED_SPLIT=<n> (a power of two, 1..8) fixes the number of sub-ranges
// the segment states are built in; -1 when unset (the planner chooses).
int forced_split_log2() {
    const char* e = getenv("LOGLIN_FUSED_SPLIT");
    if (!e || !*e) return -1;
    const long n = strtol(e, nullptr, 10);
    for (int k = 0; k <= 3; ++k)
        if (n == (1L << k)) return k;
    return -1;
}

struct Plan {
    Path path;
    FusedPlan fused;
    FwdWorkspace ws;  // layout of the workspace (chunked: per chunk; fused: per segment)
    long N;           // chunks (chunked) or segments (fused) per sequence
};

Plan make_plan(long BH, int T, int dk, int dv, int C, loglin_dtype dt) {
    Plan pl{};
    pl.path = kPathChunked;
    pl.N = ((long)T + C - 1) / C;
    if (dt == LOGLIN_BF16 && !force_chunked() && T > 0 && BH > 0) {
        FusedPlan f = plan_fused((int)BH, T, dk, dv, levels_needed(T), forced_segment_log2(), forced_split_log2());
        if (f.ok) {
            pl.path = kPathFused;
            pl.fused = f;
            pl.N = f.nseg;
        }
    }
    const int nsub = pl.path == kPathFused ? 1 << (pl.fused.m - pl.fused.msub) : 1;
    pl.ws = fwd_workspace_layout(BH, pl.N, dk, dv, pl.path == kPathFused, nsub);
    return pl;
}

// The fused path (segment states, their scan, the main kernel) for one
// problem: q, k, v bf16 [BH][T][dk|dk|dv], out fp32 [BH][T][dv].  qo and dlp
// select the backward's dq pass of the main kernel (nullptr for a forward).
hipError_t launch_fused_path(const FusedPlan& f, const FwdWorkspace& w, char* base, const void* q,
                             const void* k, const void* v, const float* log_decay,
                             const float* lambda, float* out, long BH, int T, int dk, int dv,
                             int L, int C, unsigned stage_mask, hipStream_t hs,
                             const void* qo = nullptr, float* dlp = nullptr,
                             float* dqd = nullptr, float* dlam_rows = nullptr,
                             double* ccum = nullptr) {
    FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.a = log_decay;
    p.lam = lambda;
    p.out = out;
    p.BH = (int)BH;
    p.T = T;
    p.dk = dk;
    p.dv = dv;
    p.L = L;
    p.C = C;
    p.N = f.nseg;
    p.nscan = f.nseg - 1;
    if (w.total > 0) {
        p.ust = reinterpret_cast<float*>(base + w.ust_off);
        p.tot = reinterpret_cast<float*>(base + w.tot_off);
        p.cum = reinterpret_cast<double*>(base + w.cum_off);
    }
    // the output kernel reads the nodes only as bf16 fragments: the scan
    // writes no fp32 copy (the segment states stay in place)
    p.nodes16_only = true;
    FusedParams fp{};
    fp.q = static_cast<const bf16_t_storage*>(q);
    fp.k = static_cast<const bf16_t_storage*>(k);
    fp.v = static_cast<const bf16_t_storage*>(v);
    fp.a = log_decay;
    fp.lam = lambda;
    fp.out = out;
    fp.BH = (int)BH;
    fp.T = T;
    fp.dk = dk;
    fp.dv = dv;
    fp.L = L;
    fp.LU = levels_needed(T);
    fp.ntiles = f.ntiles;
    fp.m = f.m;
    fp.nseg = f.nseg;
    fp.ntop = f.ntop;
    fp.dvw = f.dvw;
    fp.ndvb = f.ndvb;
    fp.useg = p.ust;
    fp.stot = p.tot;
    fp.scum = p.cum;
    fp.combo = f.combo;
    // lambda rows are copied whole when they fit the kernel's staging area
    // and every tile's rows start on a 16-byte boundary; otherwise the
    // levels in use are loaded element by element
    fp.lpitch = L <= kFusedMaxL ? L : fp.LU;
    fp.lam_dma = L <= kFusedMaxL && ((long)T * L) % 4 == 0 &&
                 reinterpret_cast<uintptr_t>(lambda) % 16 == 0;
    fp.a_dma = T % 4 == 0 && reinterpret_cast<uintptr_t>(log_decay) % 16 == 0;
    fp.msub = f.msub;
    fp.qo = static_cast<const bf16_t_storage*>(qo);
    fp.dlp = dlp;
    fp.dqd = dqd;
    fp.dlam_rows = dlam_rows;
    fp.ccum = ccum;
    if (w.total > 0) {
        p.gfrag = reinterpret_cast<bf16_t_storage*>(base + w.frag_off);
        fp.gfrag = p.gfrag;
        if (f.m > f.msub) {  // segment states come in sub-ranges
            fp.upart = reinterpret_cast<float*>(base + w.upart_off);
            fp.tpart = reinterpret_cast<float*>(base + w.tpart_off);
            p.upart = fp.upart;
            p.tpart = fp.tpart;
            p.nsub = 1 << (f.m - f.msub);
        }
    }
    return launch_fused_fwd(fp, p, stage_mask, hs);
}

}  // namespace

extern "C" {

const char* loglin_last_error(void) { return g_err; }

const char* loglin_status_string(loglin_status s) {
    switch (s) {
        case LOGLIN_OK: return "LOGLIN_OK";
        case LOGLIN_EINVAL: return "LOGLIN_EINVAL";
        case LOGLIN_EUNSUPPORTED: return "LOGLIN_EUNSUPPORTED";
        case LOGLIN_ENOMEM: return "LOGLIN_ENOMEM";
        case LOGLIN_ECAPACITY: return "LOGLIN_ECAPACITY";
        case LOGLIN_EHIP: return "LOGLIN_EHIP";
    }
    return "LOGLIN_<unknown>";
}

size_t loglin_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C, loglin_dtype in_dtype) {
    if (check_fwd_sizes(B, H, T, dk, dv, C) != LOGLIN_OK) return (size_t)-1;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16) {
        fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
        return (size_t)-1;
    }
    return make_plan((long)B * H, T, dk, dv, C, in_dtype).ws.total;
}

loglin_status loglin_fwd_plan(int B, int H, int T, int dk, int dv, int C, loglin_dtype in_dtype,
                              loglin_fwd_plan_t* out) {
    if (!out) return fail(LOGLIN_EINVAL, "null plan pointer");
    loglin_status s = check_fwd_sizes(B, H, T, dk, dv, C);
    if (s != LOGLIN_OK) return s;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16)
        return fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
    const Plan pl = make_plan((long)B * H, T, dk, dv, C, in_dtype);
    loglin_fwd_plan_t r{};
    r.path = pl.path;
    r.workspace_bytes = pl.ws.total;
    if (pl.path == kPathFused) {
        r.tile = 64;
        r.seg_tiles = 1 << pl.fused.m;
        r.nseg = pl.fused.nseg;
        r.col_block = pl.fused.dvw;
        r.coarse_levels = pl.fused.ntop;
        r.state_split = 1 << (pl.fused.m - pl.fused.msub);
    } else {
        r.tile = C;
        r.seg_tiles = 1;
        r.nseg = (int)pl.N;
        r.col_block = dv;
        r.state_split = 1;
        r.coarse_levels = 0;
        while ((1L << r.coarse_levels) < pl.N) ++r.coarse_levels;
    }
    *out = r;
    return ok();
}

loglin_status loglin_fwd_chunked_stages(const void* q, const void* k, const void* v,
                                        const float* log_decay, const float* lambda, float* out,
                                        int B, int H, int T, int dk, int dv, int L, int C,
                                        loglin_dtype in_dtype, void* workspace,
                                        size_t workspace_bytes, unsigned stage_mask,
                                        void* stream) {
    if (stage_mask & ~kStageAll) return fail(LOGLIN_EINVAL, "stage mask 0x%x has unknown bits", stage_mask);
    loglin_status s = check_fwd_sizes(B, H, T, dk, dv, C);
    if (s != LOGLIN_OK) return s;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16)
        return fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
    if ((long)B * H * T == 0) return ok();
    if (L < levels_needed(T) || L > 64)
        return fail(LOGLIN_EINVAL, "L=%d: T=%d needs %d levels (and L <= 64)", L, T, levels_needed(T));
    if (!q || !k || !v || !log_decay || !lambda || !out)
        return fail(LOGLIN_EINVAL, "null tensor pointer");
    const long BH = (long)B * H;
    const Plan pl = make_plan(BH, T, dk, dv, C, in_dtype);
    const FwdWorkspace& w = pl.ws;
    if (w.total > 0) {
        if (!workspace || workspace_bytes < w.total)
            return fail(LOGLIN_EINVAL, "workspace of %zu bytes needed, got %zu%s", w.total,
                        workspace_bytes, workspace ? "" : " (NULL)");
        if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
            return fail(LOGLIN_EINVAL, "workspace must be %zu-byte aligned", kAlign);
    }
    if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(k) % 16 ||
        reinterpret_cast<uintptr_t>(v) % 16 || reinterpret_cast<uintptr_t>(out) % 16)
        return fail(LOGLIN_EINVAL, "q, k, v and out must be 16-byte aligned");

    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (pl.path == kPathFused) {
        e = launch_fused_path(pl.fused, w, static_cast<char*>(workspace), q, k, v, log_decay, lambda,
                              out, BH, T, dk, dv, L, C, stage_mask, hs);
    } else {
        // the chunk state buffers of the chunked path
        FwdParams p{};
        p.q = q;
        p.k = k;
        p.v = v;
        p.a = log_decay;
        p.lam = lambda;
        p.out = out;
        p.BH = (int)BH;
        p.T = T;
        p.dk = dk;
        p.dv = dv;
        p.L = L;
        p.C = C;
        p.N = (int)pl.N;
        p.nscan = (int)pl.N - 1;
        if (w.total > 0) {
            char* base = static_cast<char*>(workspace);
            p.ust = reinterpret_cast<float*>(base + w.ust_off);
            p.tot = reinterpret_cast<float*>(base + w.tot_off);
            p.cum = reinterpret_cast<double*>(base + w.cum_off);
        }
        e = launch_fwd_chunked(p, in_dtype == LOGLIN_BF16, stage_mask, hs);
    }
    if (e != hipSuccess) return hip_fail(e, "loglin_fwd_chunked launch");
    return ok();
}

loglin_status loglin_fwd_chunked(const void* q, const void* k, const void* v,
                                 const float* log_decay, const float* lambda, float* out, int B,
                                 int H, int T, int dk, int dv, int L, int C, loglin_dtype in_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    return loglin_fwd_chunked_stages(q, k, v, log_decay, lambda, out, B, H, T, dk, dv, L, C,
                                     in_dtype, workspace, workspace_bytes, kStageAll, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// log-linear Gated DeltaNet: chunked forward

namespace {

struct GdnWorkspace {
    size_t f_off, q_off, u_off, total;
};

// one slot per chunk, a sequence's last chunk included: the bf16 chunk kernel
// writes q', F and U for every chunk (the walk reads them from chunk 1 on,
// and F, U up to the second-to-last chunk), so a single chunk needs them too
GdnWorkspace gdn_layout(long BH, int T, int dk, int dv) {
    GdnWorkspace w{};
    const long N = ((long)T + kGdnChunk - 1) / kGdnChunk;
    if (BH == 0 || N < 1) return w;
    w.f_off = 0;
    w.q_off = align_up(w.f_off + (size_t)BH * N * dk * dk * sizeof(float));
    w.u_off = align_up(w.q_off + (size_t)BH * N * kGdnChunk * dk * sizeof(float));
    w.total = align_up(w.u_off + (size_t)BH * N * dk * dv * sizeof(float));
    return w;
}

loglin_status check_gdn_sizes(int B, int H, int T, int dk, int dv, int C) {
    loglin_status s = check_fwd_sizes(B, H, T, dk, dv, C);
    if (s != LOGLIN_OK) return s;
    if (dk != 64 && dk != 128)
        return fail(LOGLIN_EUNSUPPORTED, "Gated DeltaNet forward: dk=%d must be 64 or 128", dk);
    if (dv != 16 && dv != 32 && dv != 64)
        return fail(LOGLIN_EUNSUPPORTED, "Gated DeltaNet forward: dv=%d must be 16, 32 or 64", dv);
    const long N = ((long)T + kGdnChunk - 1) / kGdnChunk;
    const int nlev = bit_length(N - 1);
    if (nlev > kGdnMaxWalkLevelsBf || gdn_levels_smem(dk, nlev) > kGdnLdsMax ||
        gdn_levels_smem_bf(dk, nlev) > kGdnLdsMax)
        return fail(LOGLIN_EUNSUPPORTED, "Gated DeltaNet forward: T=%d needs %d chunk levels, "
                    "more than one block holds", T, nlev);
    return LOGLIN_OK;
}

}  // namespace

extern "C" {

size_t loglin_gdn_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C,
                                      loglin_dtype in_dtype) {
    if (check_gdn_sizes(B, H, T, dk, dv, C) != LOGLIN_OK) return (size_t)-1;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16) {
        fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
        return (size_t)-1;
    }
    return gdn_layout((long)B * H, T, dk, dv).total;
}

loglin_status loglin_gdn_fwd_chunked_stages(const void* q, const void* k, const void* v,
                                            const float* log_decay, const float* beta,
                                            const float* lambda, float* out, int B, int H, int T,
                                            int dk, int dv, int L, int C, loglin_dtype in_dtype,
                                            void* workspace, size_t workspace_bytes,
                                            unsigned stage_mask, void* stream) {
    if (stage_mask & ~3u) return fail(LOGLIN_EINVAL, "stage mask 0x%x has unknown bits", stage_mask);
    loglin_status s = check_gdn_sizes(B, H, T, dk, dv, C);
    if (s != LOGLIN_OK) return s;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16)
        return fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
    if ((long)B * H * T == 0) return ok();
    if (L < levels_needed(T) || L > 64)
        return fail(LOGLIN_EINVAL, "L=%d: T=%d needs %d levels (and L <= 64)", L, T, levels_needed(T));
    if (!q || !k || !v || !log_decay || !beta || !lambda || !out)
        return fail(LOGLIN_EINVAL, "null tensor pointer");
    const long BH = (long)B * H;
    const GdnWorkspace w = gdn_layout(BH, T, dk, dv);
    if (w.total > 0) {
        if (!workspace || workspace_bytes < w.total)
            return fail(LOGLIN_EINVAL, "workspace of %zu bytes needed, got %zu%s", w.total,
                        workspace_bytes, workspace ? "" : " (NULL)");
        if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
            return fail(LOGLIN_EINVAL, "workspace must be %zu-byte aligned", kAlign);
    }
    GdnParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.a = log_decay;
    p.beta = beta;
    p.lam = lambda;
    p.out = out;
    p.BH = (int)BH;
    p.T = T;
    p.dk = dk;
    p.dv = dv;
    p.L = L;
    p.N = (int)(((long)T + kGdnChunk - 1) / kGdnChunk);
    p.nlev = bit_length(p.N - 1);
    if (w.total > 0) {
        char* base = static_cast<char*>(workspace);
        p.fmat = reinterpret_cast<float*>(base + w.f_off);
        p.qp = reinterpret_cast<float*>(base + w.q_off);
        p.ust = reinterpret_cast<float*>(base + w.u_off);
    }
    hipError_t e = launch_gdn_fwd(p, in_dtype == LOGLIN_BF16, stage_mask, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "loglin_gdn_fwd_chunked launch");
    return ok();
}

loglin_status loglin_gdn_fwd_chunked(const void* q, const void* k, const void* v,
                                     const float* log_decay, const float* beta, const float* lambda,
                                     float* out, int B, int H, int T, int dk, int dv, int L, int C,
                                     loglin_dtype in_dtype, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    return loglin_gdn_fwd_chunked_stages(q, k, v, log_decay, beta, lambda, out, B, H, T, dk, dv, L,
                                         C, in_dtype, workspace, workspace_bytes, 3u, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// backward pass

namespace {

// LOGLIN_BWD_DQ=chunked keeps the dq / dlambda stage of the backward on the
// chunk-state path for bf16 inputs too (the fused dq pass is the default
// where it applies).
bool force_bwd_dq_chunked() {
    const char* e = getenv("LOGLIN_BWD_DQ");
    return e && strcmp(e, "chunked") == 0;
}
// LOGLIN_BWD_DQ=fused64: the fused dq pass in two 64-column blocks even where
// the one-block kernel applies
bool force_bwd_dq_two_blocks() {
    const char* e = getenv("LOGLIN_BWD_DQ");
    return e && strcmp(e, "fused64") == 0;
}

// Workspace of the backward.  dq / dlambda either by the fused path run on
// the swapped problem (queries dO, keys v, values k; its segment states, the
// per-column-block dlambda rows, the chunk-level decay prefix) or from the
// Fenwick nodes of k v^T over chunks (the forward's chunk-state and scan
// buffers); then the block states R and R^T and the two per-token dot
// products that make up the decay gradient.
struct BwdWorkspace {
    bool fused_dq;
    FusedPlan fq;        // the fused dq pass's plan (fused_dq)
    FwdWorkspace nodes;  // its segment buffers, or the chunk nodes
    size_t dlp_off, dqd_off, ccum_off;
    size_t rst_off, rstT_off, da1_off, da2_off, total;
};

BwdWorkspace bwd_layout(long BH, int T, int dk, int dv, int C, loglin_dtype dt) {
    BwdWorkspace w{};
    const long N = ((long)T + C - 1) / C;
    size_t off = 0;
    if (dt == LOGLIN_BF16 && dv == 64 && (dk == 64 || dk == 128) && T > 0 && BH > 0 &&
        !force_bwd_dq_chunked()) {
        // d_v' = d_k = 128: one block of 128 columns (the score tile of dO v^T
        // computed once, dO, v, lambda and a read once) where the plan has
        // five register levels and two above the segment, the combination
        // that kernel is built for; two 64-column blocks otherwise
        FusedPlan f = plan_fused((int)BH, T, dv, dk, levels_needed(T), -1, -1);
        if (f.ok && dv == 64 && dk == 128 && !force_bwd_dq_two_blocks()) {
            const FusedPlan w1 = plan_fused((int)BH, T, dv, dk, levels_needed(T), -1, -1, 128);
            if (w1.ok && w1.ndvb == 1 && w1.combo == 2) f = w1;
        }
        if (f.ok) {
            w.fused_dq = true;
            w.fq = f;
            w.nodes = fwd_workspace_layout(BH, f.nseg, dv, dk, true, 1 << (f.m - f.msub));
            w.dlp_off = w.nodes.total;
            // per column block: dlambda rows [ndvb][BH][T][levels the sequence
            // uses] and the parts of q . dq [ndvb][BH][T]
            w.dqd_off = align_up(w.dlp_off + (size_t)f.ndvb * BH * T * levels_needed(T) * sizeof(float));
            w.ccum_off = align_up(w.dqd_off + (size_t)f.ndvb * BH * T * sizeof(float));
            off = align_up(w.ccum_off + (size_t)BH * N * sizeof(double));
        }
    }
    if (!w.fused_dq) {
        w.nodes = fwd_workspace_layout(BH, N, dk, dv, false, 1);
        off = w.nodes.total;
    }
    const size_t st = N > 1 ? (size_t)BH * N * dk * dv * sizeof(float) : 0;
    w.rst_off = off;
    off = align_up(off + st);
    w.rstT_off = off;
    off = align_up(off + st);
    w.da1_off = off;
    off = align_up(off + (size_t)BH * T * sizeof(float));
    w.da2_off = off;
    off = align_up(off + (size_t)BH * T * sizeof(float));
    w.total = BH * T > 0 ? off : 0;
    return w;
}

}  // namespace

extern "C" {

size_t loglin_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C, loglin_dtype in_dtype) {
    if (check_fwd_sizes(B, H, T, dk, dv, C) != LOGLIN_OK) return (size_t)-1;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16) {
        fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
        return (size_t)-1;
    }
    return bwd_layout((long)B * H, T, dk, dv, C, in_dtype).total;
}

loglin_status loglin_bwd_chunked(const void* q, const void* k, const void* v, const float* log_decay,
                                 const float* lambda, const void* dout, float* dq, float* dk_out,
                                 float* dv_out, float* dlog_decay, float* dlambda, int B, int H,
                                 int T, int dk, int dv, int L, int C, loglin_dtype in_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    loglin_status s = check_fwd_sizes(B, H, T, dk, dv, C);
    if (s != LOGLIN_OK) return s;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16)
        return fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
    if ((long)B * H * T == 0) return ok();
    if (L < levels_needed(T) || L > 64)
        return fail(LOGLIN_EINVAL, "L=%d: T=%d needs %d levels (and L <= 64)", L, T, levels_needed(T));
    if (!q || !k || !v || !log_decay || !lambda || !dout || !dq || !dk_out || !dv_out || !dlog_decay ||
        !dlambda)
        return fail(LOGLIN_EINVAL, "null tensor pointer");
    const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                         reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(dout) |
                         reinterpret_cast<uintptr_t>(dq) | reinterpret_cast<uintptr_t>(dk_out) |
                         reinterpret_cast<uintptr_t>(dv_out);
    if (al % 16) return fail(LOGLIN_EINVAL, "q, k, v, dout, dq, dk and dv must be 16-byte aligned");
    const long BH = (long)B * H;
    const BwdWorkspace w = bwd_layout(BH, T, dk, dv, C, in_dtype);
    if (!workspace || workspace_bytes < w.total)
        return fail(LOGLIN_EINVAL, "workspace of %zu bytes needed, got %zu%s", w.total, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
        return fail(LOGLIN_EINVAL, "workspace must be %zu-byte aligned", kAlign);
    char* base = static_cast<char*>(workspace);
    const int N = (int)(((long)T + C - 1) / C);
    hipStream_t hs = static_cast<hipStream_t>(stream);

    BwdParams bp{};
    bp.q = q;
    bp.k = k;
    bp.v = v;
    bp.dout = dout;
    bp.a = log_decay;
    bp.lam = lambda;
    bp.gq = dq;
    bp.gk = dk_out;
    bp.gv = dv_out;
    bp.ga = dlog_decay;
    bp.glam = dlambda;
    bp.BH = (int)BH;
    bp.T = T;
    bp.dk = dk;
    bp.dv = dv;
    bp.L = L;
    bp.C = C;
    bp.N = N;
    bp.nlev = bit_length(N - 1);
    bp.dA1 = reinterpret_cast<float*>(base + w.da1_off);
    bp.dA2 = reinterpret_cast<float*>(base + w.da2_off);
    if (w.fused_dq) {
        // dq = ((dO v^T) (.) M) k: the fused path over (dO, v, k), which also
        // leaves each column block's dlambda rows and part of q . dq; then
        // their sums
        float* dlp = reinterpret_cast<float*>(base + w.dlp_off);
        float* dqd = reinterpret_cast<float*>(base + w.dqd_off);
        // the one-block (128-column) pass with lambda rows that fit its LDS
        // tile writes dlambda rows and q . dq (dA1) itself; else the column
        // blocks' parts are summed and transposed by the dlambda kernel
        const bool rows = w.fq.dvw == 128 && L <= kFusedMaxL;
        // with 64-token chunks (the pass's tiles) the pass also leaves A at
        // the end of every chunk for the dk / dv stage
        double* ccum = reinterpret_cast<double*>(base + w.ccum_off);
        const bool cum_by_pass = C == 64 && N > 1;
        hipError_t e = launch_fused_path(w.fq, w.nodes, base, dout, v, k, log_decay, lambda, dq, BH, T,
                                         dv, dk, L, C, kStageAll, hs, q, dlp, rows ? bp.dA1 : dqd,
                                         rows ? dlambda : nullptr, cum_by_pass ? ccum : nullptr);
        if (e != hipSuccess) return hip_fail(e, "loglin_bwd_chunked dq launch");
        if (!rows) {
            e = launch_bwd_dlam_sum(bp, dlp, dqd, w.fq.ndvb, levels_needed(T), hs);
            if (e != hipSuccess) return hip_fail(e, "loglin_bwd_chunked dlambda launch");
        }
        bp.dq_done = 1;
        if (N > 1) {
            bp.cum = ccum;
            if (!cum_by_pass) {
                e = launch_bwd_chunk_cum(bp, hs);
                if (e != hipSuccess) return hip_fail(e, "loglin_bwd_chunked decay prefix launch");
            }
            bp.rst = reinterpret_cast<float*>(base + w.rst_off);
            bp.rstT = reinterpret_cast<float*>(base + w.rstT_off);
            bp.rst16 = reinterpret_cast<bf16_t_storage*>(base + w.rst_off);
        }
    } else if (N > 1) {
        // the forward's chunk states and node scan over k and v swapped: the
        // nodes come out as sum k v^T, [dk][dv]
        FwdParams fp{};
        fp.k = v;
        fp.v = k;
        fp.a = log_decay;
        fp.lam = lambda;
        fp.BH = (int)BH;
        fp.T = T;
        fp.dk = dv;
        fp.dv = dk;
        fp.L = L;
        fp.C = C;
        fp.N = N;
        fp.nscan = N - 1;
        fp.ust = reinterpret_cast<float*>(base + w.nodes.ust_off);
        fp.tot = reinterpret_cast<float*>(base + w.nodes.tot_off);
        fp.cum = reinterpret_cast<double*>(base + w.nodes.cum_off);
        if (in_dtype == LOGLIN_BF16) {
            // bf16 inputs: the nodes only as bf16 (the operand form the dq
            // kernel stages), in the region the fp32 R^T would use
            fp.gnode16 = reinterpret_cast<bf16_t_storage*>(base + w.rstT_off);
            fp.nodes16_only = true;
        }
        hipError_t e = launch_fwd_chunked(fp, in_dtype == LOGLIN_BF16, kStageChunkState | kStageScan, hs);
        if (e != hipSuccess) return hip_fail(e, "loglin_bwd_chunked node launch");
        bp.gnode = fp.ust;
        bp.gnode16 = fp.gnode16;
        bp.cum = fp.cum;
        bp.rst = reinterpret_cast<float*>(base + w.rst_off);
        bp.rstT = reinterpret_cast<float*>(base + w.rstT_off);
        bp.rst16 = reinterpret_cast<bf16_t_storage*>(base + w.rst_off);
    }
    hipError_t e = launch_bwd_chunked(bp, in_dtype == LOGLIN_BF16, hs);
    if (e != hipSuccess) return hip_fail(e, "loglin_bwd_chunked launch");
    return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// decode state

struct loglin_state {
    int nseq, H, dk, dv, Lmax;
    float* levels;               // device [nseq][H][Lmax][dk][dv] matrices X
    float* sigma;                // device [nseq][H][Lmax] log-scales (state = exp(sigma) X)
    float* raw;                  // device [nseq][H][dk + dv]: level 0 as k, v once a step ran
    float* win;                  // device [nseq][H][64][dk + dv]: the 64-token window's rows
    float* wc;                   // device [nseq][H][64]: running sums of a over the window
    int kind;                    // mixer stepping the state since the last load: 0 none,
                                 // 1 scalar-gated (levels 0..6 in the window), 2 Gated DeltaNet
    int64_t* base_pos;           // device [nseq]
    std::vector<int64_t> host_base;  // host mirror of base_pos
    int64_t step;                // steps since the last load
    int64_t max_base;
    uint32_t magic;
};

namespace {
constexpr uint32_t kMagic = 0x4c4f474cu;  // "LOGL"

loglin_status check_state(const loglin_state* st) {
    if (!st || st->magic != kMagic) return fail(LOGLIN_EINVAL, "invalid or freed state handle");
    return LOGLIN_OK;
}

DecodeParams decode_params(const loglin_state* st) {
    DecodeParams p{};
    p.states = st->levels;
    p.sigma = st->sigma;
    p.raw = st->raw;
    p.raw0 = st->step > 0;  // every step rewrites level 0 of every (sequence, head)
    p.win = st->win;
    p.wc = st->wc;
    p.window = st->kind == 1;
    p.base_pos = st->base_pos;
    p.step = st->step;
    p.nseq = st->nseq;
    p.H = st->H;
    p.dk = st->dk;
    p.dv = st->dv;
    p.Lmax = st->Lmax;
    return p;
}

bool alloc_fail_injected() {
    const char* e = getenv("LOGLIN_TEST_FAIL_ALLOC");
    return e && e[0] == '1';
}
}  // namespace

extern "C" {

loglin_status loglin_state_init(loglin_state** out, int nseq, int H, int dk, int dv, int Lmax,
                                void* stream) {
    if (!out) return fail(LOGLIN_EINVAL, "null output handle pointer");
    if (nseq < 1 || H < 1) return fail(LOGLIN_EINVAL, "nseq=%d and H=%d must be >= 1", nseq, H);
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LOGLIN_EUNSUPPORTED, "head dims dk=%d dv=%d must be in {16,32,64,128}", dk, dv);
    if (Lmax < 1 || Lmax > 48) return fail(LOGLIN_EINVAL, "Lmax=%d must be in [1, 48]", Lmax);
    if ((long)nseq * H > 0x7fffffffL) return fail(LOGLIN_EUNSUPPORTED, "nseq*H too large");
    loglin_state* st = new (std::nothrow) loglin_state();
    if (!st) return fail(LOGLIN_ENOMEM, "host allocation failed");
    st->nseq = nseq;
    st->H = H;
    st->dk = dk;
    st->dv = dv;
    st->Lmax = Lmax;
    st->step = 0;
    st->max_base = 0;
    st->host_base.assign(nseq, 0);
    const size_t bytes = (size_t)nseq * H * Lmax * dk * dv * sizeof(float);
    if (alloc_fail_injected()) {
        delete st;
        return fail(LOGLIN_ENOMEM, "device allocation of %zu bytes failed (injected)", bytes);
    }
    hipError_t e = hipMalloc(&st->levels, bytes);
    if (e != hipSuccess) {
        delete st;
        return fail(LOGLIN_ENOMEM, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
    }
    e = hipMalloc(&st->base_pos, (size_t)nseq * sizeof(int64_t));
    if (e != hipSuccess) {
        (void)hipFree(st->levels);
        delete st;
        return fail(LOGLIN_ENOMEM, "hipMalloc positions: %s", hipGetErrorString(e));
    }
    const size_t sbytes = (size_t)nseq * H * Lmax * sizeof(float);
    e = hipMalloc(&st->sigma, sbytes);
    if (e != hipSuccess) {
        (void)hipFree(st->levels);
        (void)hipFree(st->base_pos);
        delete st;
        return fail(LOGLIN_ENOMEM, "hipMalloc level scales: %s", hipGetErrorString(e));
    }
    e = hipMalloc(&st->raw, (size_t)nseq * H * (dk + dv) * sizeof(float));
    if (e != hipSuccess) {
        (void)hipFree(st->levels);
        (void)hipFree(st->base_pos);
        (void)hipFree(st->sigma);
        delete st;
        return fail(LOGLIN_ENOMEM, "hipMalloc level 0 vectors: %s", hipGetErrorString(e));
    }
    e = hipMalloc(&st->win, (size_t)nseq * H * 64 * (dk + dv) * sizeof(float));
    if (e == hipSuccess) {
        e = hipMalloc(&st->wc, (size_t)nseq * H * 64 * sizeof(float));
        if (e != hipSuccess) (void)hipFree(st->win);
    }
    if (e != hipSuccess) {
        (void)hipFree(st->levels);
        (void)hipFree(st->base_pos);
        (void)hipFree(st->sigma);
        (void)hipFree(st->raw);
        delete st;
        return fail(LOGLIN_ENOMEM, "hipMalloc window rows: %s", hipGetErrorString(e));
    }
    st->kind = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    e = hipMemsetAsync(st->levels, 0, bytes, s);
    if (e == hipSuccess) e = hipMemsetAsync(st->base_pos, 0, (size_t)nseq * sizeof(int64_t), s);
    if (e == hipSuccess) e = hipMemsetAsync(st->sigma, 0, sbytes, s);
    if (e != hipSuccess) {
        (void)hipFree(st->levels);
        (void)hipFree(st->base_pos);
        (void)hipFree(st->sigma);
        (void)hipFree(st->raw);
        (void)hipFree(st->win);
        (void)hipFree(st->wc);
        delete st;
        return hip_fail(e, "loglin_state_init");
    }
    st->magic = kMagic;
    *out = st;
    return ok();
}

loglin_status loglin_state_free(loglin_state* st) {
    if (!st) return ok();
    loglin_status s = check_state(st);
    if (s != LOGLIN_OK) return s;
    hipError_t e = hipDeviceSynchronize();
    st->magic = 0;
    hipError_t e1 = hipFree(st->levels);
    hipError_t e2 = hipFree(st->base_pos);
    hipError_t e3 = hipFree(st->sigma);
    hipError_t e4 = hipFree(st->raw);
    hipError_t e5 = hipFree(st->win);
    hipError_t e6 = hipFree(st->wc);
    if (e2 == hipSuccess) e2 = e3;
    if (e2 == hipSuccess) e2 = e4;
    if (e2 == hipSuccess) e2 = e5;
    if (e2 == hipSuccess) e2 = e6;
    delete st;
    if (e != hipSuccess) return hip_fail(e, "loglin_state_free (synchronize)");
    if (e1 != hipSuccess) return hip_fail(e1, "loglin_state_free");
    if (e2 != hipSuccess) return hip_fail(e2, "loglin_state_free");
    return ok();
}

loglin_status loglin_state_load(loglin_state* st, const int64_t* pos_host, const float* levels,
                                void* stream) {
    loglin_status s = check_state(st);
    if (s != LOGLIN_OK) return s;
    if (!pos_host) return fail(LOGLIN_EINVAL, "null positions");
    const int64_t cap = (int64_t)1 << (st->Lmax - 1);
    int64_t mx = 0;
    for (int i = 0; i < st->nseq; ++i) {
        if (pos_host[i] < 0) return fail(LOGLIN_EINVAL, "position %lld of sequence %d is negative",
                                         (long long)pos_host[i], i);
        if (pos_host[i] > cap)
            return fail(LOGLIN_ECAPACITY, "position %lld of sequence %d needs more than %d levels",
                        (long long)pos_host[i], i, st->Lmax);
        mx = pos_host[i] > mx ? pos_host[i] : mx;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t bytes = (size_t)st->nseq * st->H * st->Lmax * st->dk * st->dv * sizeof(float);
    hipError_t e = levels ? hipMemcpyAsync(st->levels, levels, bytes, hipMemcpyDeviceToDevice, hs)
                          : hipMemsetAsync(st->levels, 0, bytes, hs);
    if (e == hipSuccess)
        e = hipMemsetAsync(st->sigma, 0, (size_t)st->nseq * st->H * st->Lmax * sizeof(float), hs);
    if (e != hipSuccess) return hip_fail(e, "loglin_state_load (levels)");
    st->host_base.assign(pos_host, pos_host + st->nseq);
    // the host vector must outlive the asynchronous copy: it does, as it is
    // only replaced by the next load, which is ordered after this one only if
    // we wait here for the small copy to finish.
    e = hipMemcpyAsync(st->base_pos, st->host_base.data(), (size_t)st->nseq * sizeof(int64_t),
                       hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return hip_fail(e, "loglin_state_load (positions)");
    st->step = 0;
    st->max_base = mx;
    st->kind = 0;
    return ok();
}

loglin_status loglin_state_export(const loglin_state* st, int64_t* pos_host, float* levels,
                                  void* stream) {
    loglin_status s = check_state(st);
    if (s != LOGLIN_OK) return s;
    if (pos_host)
        for (int i = 0; i < st->nseq; ++i) pos_host[i] = st->host_base[i] + st->step;
    if (levels) {
        hipError_t e = launch_state_export(decode_params(st), levels, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "loglin_state_export");
    }
    return ok();
}

loglin_status loglin_decode_step(loglin_state* st, const void* q, const void* k, const void* v,
                                 const float* log_decay, const float* lambda, float* out,
                                 loglin_dtype in_dtype, void* stream) {
    loglin_status s = check_state(st);
    if (s != LOGLIN_OK) return s;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16)
        return fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
    if (!q || !k || !v || !log_decay || !lambda || !out)
        return fail(LOGLIN_EINVAL, "null tensor pointer");
    if (reinterpret_cast<uintptr_t>(out) % 16)
        return fail(LOGLIN_EINVAL, "out must be 16-byte aligned");
    const int64_t t = st->max_base + st->step;  // largest position decoded by this step
    if (t >= ((int64_t)1 << (st->Lmax - 1)))
        return fail(LOGLIN_ECAPACITY, "position %lld needs more than %d levels", (long long)t,
                    st->Lmax);
    if (st->kind == 2)
        return fail(LOGLIN_EINVAL, "the state was stepped by loglin_gdn_decode_step since its "
                    "last load; one state serves one mixer");
    st->kind = 1;
    DecodeParams p = decode_params(st);
    p.q = q;
    p.k = k;
    p.v = v;
    p.a = log_decay;
    p.lam = lambda;
    p.out = out;
    hipError_t e = launch_decode_step(p, in_dtype == LOGLIN_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "loglin_decode_step launch");
    st->step += 1;
    return ok();
}

loglin_status loglin_gdn_decode_step(loglin_state* st, const void* q, const void* k, const void* v,
                                     const float* log_decay, const float* beta, const float* lambda,
                                     float* out, loglin_dtype in_dtype, void* stream) {
    loglin_status s = check_state(st);
    if (s != LOGLIN_OK) return s;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16)
        return fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
    if (!q || !k || !v || !log_decay || !beta || !lambda || !out)
        return fail(LOGLIN_EINVAL, "null tensor pointer");
    if (reinterpret_cast<uintptr_t>(out) % 16)
        return fail(LOGLIN_EINVAL, "out must be 16-byte aligned");
    const int64_t t = st->max_base + st->step;
    if (t >= ((int64_t)1 << (st->Lmax - 1)))
        return fail(LOGLIN_ECAPACITY, "position %lld needs more than %d levels", (long long)t,
                    st->Lmax);
    if (st->kind == 1)
        return fail(LOGLIN_EINVAL, "the state was stepped by loglin_decode_step since its last "
                    "load; one state serves one mixer");
    st->kind = 2;
    DecodeParams p = decode_params(st);
    p.q = q;
    p.k = k;
    p.v = v;
    p.a = log_decay;
    p.lam = lambda;
    p.out = out;
    hipError_t e = launch_gdn_decode_step(p, beta, in_dtype == LOGLIN_BF16,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "loglin_gdn_decode_step launch");
    st->step += 1;
    return ok();
}

// ---------------------------------------------------------------------------
// prefill -> decode hand-over

namespace {
loglin_status check_prefill(int B, int H, int T, int dk, int dv, int Lmax) {
    if (B < 0 || H < 0 || T < 0)
        return fail(LOGLIN_EINVAL, "B, H, T must be >= 0 (got %d, %d, %d)", B, H, T);
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LOGLIN_EUNSUPPORTED, "head dims dk=%d dv=%d must be in {16,32,64,128}", dk, dv);
    if (Lmax < 1 || Lmax > 48) return fail(LOGLIN_EINVAL, "Lmax=%d must be in [1, 48]", Lmax);
    if (T > 0 && levels_needed(T) > Lmax)
        return fail(LOGLIN_ECAPACITY, "T=%d needs %d levels, Lmax=%d", T, levels_needed(T), Lmax);
    if ((long)T > ((long)1 << 30)) return fail(LOGLIN_EUNSUPPORTED, "T=%d too long", T);
    return LOGLIN_OK;
}
size_t prefill_ws_bytes(long BH, int T, int dk, int dv) {
    return align_up((size_t)BH * prefill_jobs(T) * dk * dv * sizeof(float));
}
}  // namespace

size_t loglin_prefill_workspace_bytes(int B, int H, int T, int dk, int dv, int Lmax) {
    if (check_prefill(B, H, T, dk, dv, Lmax) != LOGLIN_OK) return (size_t)-1;
    return prefill_ws_bytes((long)B * H, T, dk, dv);
}

loglin_status loglin_prefill_states(const void* k, const void* v, const float* log_decay,
                                    float* states, int B, int H, int T, int dk, int dv, int Lmax,
                                    loglin_dtype in_dtype, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    loglin_status s = check_prefill(B, H, T, dk, dv, Lmax);
    if (s != LOGLIN_OK) return s;
    if (in_dtype != LOGLIN_F32 && in_dtype != LOGLIN_BF16)
        return fail(LOGLIN_EINVAL, "in_dtype %d is neither LOGLIN_F32 nor LOGLIN_BF16", (int)in_dtype);
    const long BH = (long)B * H;
    if (BH == 0) return ok();
    if (!states) return fail(LOGLIN_EINVAL, "null states pointer");
    if (T > 0 && (!k || !v || !log_decay)) return fail(LOGLIN_EINVAL, "null tensor pointer");
    if (reinterpret_cast<uintptr_t>(states) % 16 || reinterpret_cast<uintptr_t>(k) % 16 ||
        reinterpret_cast<uintptr_t>(v) % 16)
        return fail(LOGLIN_EINVAL, "k, v and states must be 16-byte aligned");
    const size_t need = prefill_ws_bytes(BH, T, dk, dv);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(LOGLIN_EINVAL, "workspace of %zu bytes needed, got %zu%s", need,
                        workspace_bytes, workspace ? "" : " (NULL)");
        if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
            return fail(LOGLIN_EINVAL, "workspace must be %zu-byte aligned", kAlign);
    }
    if ((long)BH * Lmax > 0x7fffffffL / 64) return fail(LOGLIN_EUNSUPPORTED, "B*H*Lmax too large");
    PrefillParams p{};
    p.k = k;
    p.v = v;
    p.a = log_decay;
    p.states = states;
    p.ws = static_cast<float*>(workspace);
    p.BH = (int)BH;
    p.T = T;
    p.dk = dk;
    p.dv = dv;
    p.Lmax = Lmax;
    p.njobs = prefill_jobs(T);
    hipError_t e = launch_prefill_states(p, in_dtype == LOGLIN_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "loglin_prefill_states launch");
    return ok();
}

loglin_status loglin_debug_level_map(int T, int8_t* out, void* stream) {
    if (T < 1 || T > 16384) return fail(LOGLIN_EINVAL, "T=%d must be in [1, 16384]", T);
    if (!out) return fail(LOGLIN_EINVAL, "null output");
    hipError_t e = launch_level_map(T, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "loglin_debug_level_map");
    return ok();
}

}  // extern "C"
