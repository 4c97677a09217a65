// Internal launch interface between the C ABI (loglin_api.cpp) and the HIP
// kernels.  Not exported.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loglin {

typedef unsigned short bf16_t_storage;  // raw bf16 bits (same as bf16_t)

struct FwdParams {
    const void* q;       // [BH][T][dk]
    const void* k;       // [BH][T][dk]
    const void* v;       // [BH][T][dv]
    const float* a;      // [BH][T]
    const float* lam;    // [BH][T][L]
    float* out;          // [BH][T][dv]
    int BH, T, dk, dv, L, C, N;  // N = ceil(T / C): chunks per sequence (state stride)
    int nscan;           // Fenwick nodes the scan produces per sequence (N - 1)
    float* ust;          // workspace [BH][N][dv][dk]
    float* tot;          // workspace [BH][N]
    double* cum;         // workspace [BH][N]
    bf16_t_storage* gfrag;  // optional bf16 copy of the nodes in MFMA fragment order
    bf16_t_storage* gnode16;  // optional bf16 copy of the nodes in the order of ust
    bool nodes16_only;        // the fp32 nodes are not written back to ust (only the bf16
                              // copies: gnode16 and / or gfrag)
    const float* upart;  // optional [BH][N][nsub][dv][dk] states of sub-ranges (then tpart)
    const float* tpart;  // [BH][N][nsub] decay totals of the sub-ranges
    int nsub;            // sub-ranges per chunk (1, 2, 4 or 8) when upart is set
};

// workspace carving shared by the size query and the launch
struct FwdWorkspace {
    size_t ust_off, tot_off, cum_off, frag_off, upart_off, tpart_off, total;
};
// frags: bf16 node copies (fused path); nsub > 1: sub-range states per chunk
FwdWorkspace fwd_workspace_layout(long BH, long N, int dk, int dv, bool frags, int nsub);

enum : unsigned { kStageChunkState = 1u, kStageScan = 2u, kStageOutput = 4u, kStageAll = 7u };
hipError_t launch_fwd_chunked(const FwdParams& p, bool bf16, unsigned stages, hipStream_t stream);
// the Fenwick node scan over chunk (or segment) states, in place
hipError_t launch_fenwick_scan(const FwdParams& p, hipStream_t stream);

// Fused tile-recurrent forward (bf16 inputs): 64-token tiles, segments of
// 2^m tiles per block, Fenwick levels inside a segment held in registers.
constexpr int kFusedMaxL = 24;  // lambda levels staged per token (whole rows)
struct FusedParams {
    const bf16_t_storage* q;
    const bf16_t_storage* k;
    const bf16_t_storage* v;
    const float* a;
    const float* lam;
    float* out;
    int BH, T, dk, dv, L, LU;       // LU: levels the sequence uses
    int lpitch;                     // row pitch of lambda in LDS (L, or LU if L is too long)
    int ntiles, m, nseg, ntop, dvw, ndvb, combo;
    int lam_dma, a_dma;             // lambda / a rows of a whole tile are 16-byte aligned
    float* useg;                    // [BH][nseg][dv][dk] Fenwick nodes over segments
    float* upart;                   // [BH][nseg][nsub][dv][dk] states of segment sub-ranges
    float* tpart;                   // [BH][nseg][nsub] their decay totals
    int msub;                       // sub-ranges of 2^msub tiles (nsub = 2^(m - msub))
    float* stot;                    // [BH][nseg]
    double* scum;                   // [BH][nseg]
    const bf16_t_storage* gfrag;    // bf16 MFMA fragments of the nodes (written by the scan)
    // the backward's dq pass (q, k, v above are dO, v, k): the original q
    // ([BH][T][dv], dv here being the original d_k) and the partial dlambda
    // of each column block, level-major ([ndvb][BH][LU][T]); qo == nullptr otherwise
    const bf16_t_storage* qo;
    float* dlp;
    float* dqd;                     // [ndvb][BH][T] each column block's part of q_t . dq_t
    // one-block dq pass (ndvb = 1, L <= kFusedMaxL): dlambda written here as
    // whole [BH][T][L] rows (levels past LU zero) instead of dlp, and dqd is
    // then q_t . dq_t itself; nullptr otherwise
    float* dlam_rows;
    // dq pass with 64-token chunks: A at the end of every tile, fp64
    // ([BH][ntiles]; the segment scan's value before the segment plus the
    // tiles' totals in order), for the dk / dv stage; nullptr otherwise
    double* ccum;
};
struct FusedPlan {
    int ok, m, nseg, ntop, dvw, ndvb, ntiles, combo, msub;
};
// force_m >= 0 asks for segments of 2^force_m tiles (plan fails if that does not fit);
// max_dvw: widest column block (64, or 128 for the backward's dq pass, whose
// one-block kernel exists only for d_k = 64 with combination {5, 2})
FusedPlan plan_fused(int BH, int T, int dk, int dv, int lu, int force_m, int force_split,
                     int max_dvw = 64);
hipError_t launch_fused_fwd(const FusedParams& p, const FwdParams& scan, unsigned stages,
                            hipStream_t stream);

struct DecodeParams {
    float* states;            // [nseq][H][Lmax][dk][dv] matrices X (state = exp(sigma) X)
    float* sigma;             // [nseq][H][Lmax] per-level log-scales
    float* raw;               // [nseq][H][dk + dv]: k and v of the newest token (level 0)
    int raw0;                 // level 0 is raw's k v^T (else the matrix in states)
    float* win;               // [nseq][H][64][dk + dv]: the 64-token window's k, v rows
    float* wc;                // [nseq][H][64]: sum of a from the window start to each token
    int window;               // levels 0..6 live in the window (scalar-gated steps)
    const int64_t* base_pos;  // [nseq]: position of the first step after the last load
    int64_t step;             // steps taken since that load
    const void* q;            // [nseq][H][dk]
    const void* k;            // [nseq][H][dk]
    const void* v;            // [nseq][H][dv]
    const float* a;           // [nseq][H]
    const float* lam;         // [nseq][H][Lmax]
    float* out;               // [nseq][H][dv]
    int nseq, H, dk, dv, Lmax;
};

hipError_t launch_decode_step(const DecodeParams& p, bool bf16, hipStream_t stream);
// one step of the log-linear Gated DeltaNet (beta [nseq][H]) on the same state
hipError_t launch_gdn_decode_step(const DecodeParams& p, const float* beta, bool bf16,
                                  hipStream_t stream);

// Chunked forward of the log-linear Gated DeltaNet (csrc/gdn_fwd.hip)
constexpr int kGdnChunk = 64;                 // tokens per chunk
constexpr size_t kGdnLdsMax = 160 * 1024;     // LDS one block may use on gfx950
struct GdnParams {
    const void* q;       // [BH][T][dk]
    const void* k;       // [BH][T][dk]
    const void* v;       // [BH][T][dv]
    const float* a;      // [BH][T]
    const float* beta;   // [BH][T]
    const float* lam;    // [BH][T][L]
    float* out;          // [BH][T][dv]
    int BH, T, dk, dv, L;
    int N;               // chunks per sequence
    int nlev;            // chunk levels the walk holds: bit_length(N - 1)
    float* fmat;         // [BH][N][dk*dk] chunk transitions (MFMA operand order)
    float* qp;           // [BH][N][64*dk] read-out queries (MFMA operand order)
    float* ust;          // [BH][N][dk][dv] each chunk's own state at its end
};
// LDS bytes of the level walk for head dim dk holding nlev levels (fp32 and
// bf16 inputs); the bf16 walk holds at most 14 levels
size_t gdn_levels_smem(int dk, int nlev);
size_t gdn_levels_smem_bf(int dk, int nlev);
constexpr int kGdnMaxWalkLevelsBf = 14;
// stages: bit 0 the per-chunk kernel, bit 1 the level walk
hipError_t launch_gdn_fwd(const GdnParams& p, bool bf16, unsigned stages, hipStream_t stream);

// Backward pass of the chunked forward: gradients of sum(O (.) dO)
struct BwdParams {
    const void* q;            // [BH][T][dk]
    const void* k;            // [BH][T][dk]
    const void* v;            // [BH][T][dv]
    const void* dout;         // [BH][T][dv]
    const float* a;           // [BH][T]
    const float* lam;         // [BH][T][L]
    float* gq;                // [BH][T][dk]
    float* gk;                // [BH][T][dk]
    float* gv;                // [BH][T][dv]
    float* ga;                // [BH][T]
    float* glam;              // [BH][T][L]
    int BH, T, dk, dv, L, C, N, nlev;  // nlev = bit_length(N - 1)
    const float* gnode;       // [BH][N][dk][dv] Fenwick nodes of sum k v^T over chunks
    const bf16_t_storage* gnode16;  // the same in bf16 (bf16 inputs; gnode is then not written)
    const double* cum;        // [BH][N] A at the end of each chunk
    float* rst;               // [BH][N][dk][dv] block states R(j)
    float* rstT;              // [BH][N][dv][dk] the same, transposed (fp32 inputs)
    bf16_t_storage* rst16;    // [BH][N][dk][dv] R(j) in bf16 (bf16 inputs; in place of rst)
    float* dA1;               // [BH][T] q_t . dq_t
    float* dA2;               // [BH][T] k_t . dk_t
    int st_elems;             // bf16 elements of the LDS buffer that stages one carried state
    int rs_nbuf;              // copies of the staged chunk the R(j) kernel keeps (1 or 2)
    int dq_done;              // dq, dlambda and dA1 already written (fused dq pass)
};
hipError_t launch_bwd_chunked(const BwdParams& p, bool bf16, hipStream_t stream);
// R(j) of every block in one pass over the query chunks (bf16, C = 64,
// d_v = 64, d_k in {64, 128}, N <= 256): whether it applies, and the launch
bool bwd_rwalk_applies(const BwdParams& p);
// A at the end of every chunk ([BH][N] double, into p.cum) from a alone
hipError_t launch_bwd_chunk_cum(const BwdParams& p, hipStream_t stream);
// dlambda = the sum of the column blocks' parts dlp ([ndvb][BH][lu][T], the
// levels past lu zero), and dA1_t = q_t . dq_t, the sum of their parts dqd ([ndvb][BH][T])
hipError_t launch_bwd_dlam_sum(const BwdParams& p, const float* dlp, const float* dqd, int ndvb,
                               int lu, hipStream_t stream);
// coarse_only: only the blocks of levels >= m (those spanning segments), for
// the dk / dv walk, which builds the levels inside a segment itself
hipError_t launch_bwd_rwalk(const BwdParams& p, bool coarse_only, hipStream_t stream);
// dk, dv and k . dk in one reverse walk per segment (bf16, C = 64, d_k = 128,
// d_v = 64; after launch_bwd_rwalk with coarse_only): whether it applies, and the launch
bool bwd_kvwalk_applies(const BwdParams& p);
hipError_t launch_bwd_kvwalk(const BwdParams& p, hipStream_t stream);

// Fenwick level states after the T tokens of a prefill (the state a decode
// step at position T reads)
struct PrefillParams {
    const void* k;            // [BH][T][dk]
    const void* v;            // [BH][T][dv]
    const float* a;           // [BH][T]
    float* states;            // [BH][Lmax][dk][dv]
    float* ws;                // [BH][njobs][dk][dv] partial sums
    int BH, T, dk, dv, Lmax, njobs;
};
int prefill_jobs(int T);      // jobs the prefix of T tokens is cut into

// Job j of the prefix of T tokens (n = T - 1 >= 0): the prefix is cut into
// whole pieces of kPrefillJobTokens (512) tokens of the buckets of at least
// that many tokens (each such bucket is a whole number of aligned pieces),
// one job per smaller bucket (the set bits of n mod 512, largest first) and
// a last one for level 0 (the token n itself).  Token s < n lies in the
// bucket of level floor(log2(n xor s)) + 1.
constexpr int kPrefillJobLog = 9;
constexpr int kPrefillJobTokens = 1 << kPrefillJobLog;
struct PrefillJob {
    int level, s0, s1;  // tokens [s0, s1) of level `level`
};
__device__ __forceinline__ PrefillJob prefill_job(int n, int j) {
    const int nfull = n / kPrefillJobTokens;
    if (j < nfull) {
        const int s0 = j * kPrefillJobTokens;
        return PrefillJob{32 - __clz(n ^ s0), s0, s0 + kPrefillJobTokens};
    }
    int jj = j - nfull;
    const int low = n % kPrefillJobTokens;
    for (int p = kPrefillJobLog - 1; p >= 0; --p) {
        if ((low >> p) & 1) {
            if (jj == 0) {
                const int s0 = (n >> (p + 1)) << (p + 1);
                return PrefillJob{p + 1, s0, s0 + (1 << p)};
            }
            --jj;
        }
    }
    return PrefillJob{0, n, n + 1};
}
// A level whose bucket is at most one job long is written by its job
// directly; the pieces of longer buckets go to the workspace and are summed.
// (2^(level-1) <= 2^kPrefillJobLog, written without a shift so that every
// level index up to the state's 48 slots is defined)
__device__ __forceinline__ bool prefill_single(int level) {
    return level <= kPrefillJobLog + 1;
}
// bf16 inputs: each job's decayed sum on the matrix cores
hipError_t launch_prefill_jobs_bf16(const PrefillParams& p, hipStream_t stream);
hipError_t launch_prefill_states(const PrefillParams& p, bool bf16, hipStream_t stream);
// copy states to dst, zeroing every slot that is not live at the current position
hipError_t launch_state_export(const DecodeParams& p, float* dst, hipStream_t stream);
hipError_t launch_level_map(int T, int8_t* out, hipStream_t stream);

}  // namespace loglin
