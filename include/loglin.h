/*
 * loglin.h -- C ABI of libloglin.so, the log-linear (Fenwick-tree) token mixer
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation ("Log-linear attention, and what a logarithm buys"):
 *   section 1 writes a family of mixers as O = (Q K^T (.) M) V with a causal
 *   mask M; section 2 cuts the prefix of query t into Fenwick buckets
 *   (greedily the largest power of two first, bucket l >= 1 of 2^(l-1)
 *   tokens plus the query itself at level 0), gives each bucket a state
 *   S_t^(l) and reads o_t = sum_l lambda_t^(l) q_t^T S_t^(l); section 3
 *   composes this level mask elementwise with the Mamba-2 scalar-decay mask.
 * With 0-indexed positions, A_t = a_0 + ... + a_t and
 *   level(t, s) = 0 if s == t, else floor(log2(t XOR s)) + 1,
 * the mask is M[t, s] = lambda_t^(level(t, s)) * exp(A_t - A_s) for s <= t.
 *
 * Conventions for every entry point
 *  - Tensors are dense, row-major, caller-owned, and live in device memory
 *    unless a comment says "host".  The library never frees caller memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    All device work is enqueued on it and returns without waiting.
 *  - Every argument is checked on the host before anything is enqueued; a
 *    call that returns an error has enqueued nothing and changed nothing.
 *    The text of the last error of the calling thread is loglin_last_error().
 *  - Documented but not checked: lambda >= 0 and log_decay <= 0 (other values
 *    are computed as written, with the overflow that implies).
 *
 * Environment variables (read at each call; for tests and profiling, every
 * setting computes the same result by other kernels):
 *   LOGLIN_FWD_PATH=chunked       bf16 forward on the chunked path
 *   LOGLIN_FUSED_SEGMENT=<tiles>  fused path: segments of 1, 2, 4, 8, 16 or 32
 *                                 64-token tiles (else the planner chooses)
 *   LOGLIN_FUSED_SPLIT=<n>        fused path: segment states in 1, 2, 4 or 8
 *                                 sub-ranges (else the planner chooses)
 *   LOGLIN_BWD_DQ=chunked         backward dq by the chunk-state kernels
 *   LOGLIN_BWD_DQ=fused64         backward dq pass in 64-column blocks
 *   LOGLIN_BWD_RSTATE=blocks      backward R(j) states one block each
 *   LOGLIN_BWD_DKV=chunks         backward dk / dv one block per chunk
 *   LOGLIN_TEST_FAIL_ALLOC=1      loglin_state_init fails as if out of memory
 */
#ifndef LOGLIN_H
#define LOGLIN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define LOGLIN_API __attribute__((visibility("default")))
#else
#define LOGLIN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LOGLIN_OK = 0,
    LOGLIN_EINVAL = 1,       /* bad pointer, size, dtype or workspace */
    LOGLIN_EUNSUPPORTED = 2, /* chunk size or head dim not in {16,32,64,128}; too many chunks */
    LOGLIN_ENOMEM = 3,       /* device allocation failed (state init only) */
    LOGLIN_ECAPACITY = 4,    /* a position needs a level index >= the number of levels */
    LOGLIN_EHIP = 5          /* the HIP runtime reported an error (see loglin_last_error) */
} loglin_status;

/* Element type of q, k, v.  Any other value is answered with LOGLIN_EINVAL; the
 * last enumerator widens the type's value range to every int32 so that such a
 * value is well defined on the C++ side too. */
typedef enum {
    LOGLIN_F32 = 0,
    LOGLIN_BF16 = 1,
    LOGLIN_DTYPE_RANGE_ = 0x7fffffff /* not a dtype */
} loglin_dtype;

typedef struct loglin_state loglin_state; /* opaque, owned by the library */

/*
 * Bytes of device workspace loglin_fwd_chunked needs for these sizes and
 * input dtype (0 when no inter-chunk state is needed).  Returns (size_t)-1
 * for arguments that loglin_fwd_chunked would reject.
 */
LOGLIN_API size_t loglin_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C,
                                             loglin_dtype in_dtype);

/*
 * How loglin_fwd_chunked evaluates these sizes (for profiling and sizing).
 *  path 0, "chunked": three kernels over chunks of C tokens -- chunk states
 *    (MFMA), a Fenwick scan over chunks (HBM), and a fused intra-chunk plus
 *    coarse-level output kernel (MFMA).  Used for fp32 inputs.
 *  path 1, "fused": bf16 inputs.  One block walks a segment of seg_tiles
 *    64-token tiles in order with the Fenwick levels inside the segment held
 *    in registers; a segment-state kernel and the Fenwick scan over segments
 *    supply the coarse_levels levels above the segment.  The output does not
 *    depend on the tiling: every level of the mask is evaluated exactly, only
 *    the split between intra-tile blocks and carried states changes.
 */
typedef struct {
    int path;            /* 0 chunked, 1 fused */
    int tile;            /* tokens per intra block (C, or 64 on the fused path) */
    int seg_tiles;       /* tiles walked in order by one block (1 on the chunked path) */
    int nseg;            /* chunks (chunked) or segments (fused) per sequence */
    int col_block;       /* output columns per block */
    int coarse_levels;   /* levels carried between chunks / segments through the scan */
    int state_split;     /* fused path: each segment state is summed from this many
                            sub-range states (1 on the chunked path) */
    size_t workspace_bytes;
} loglin_fwd_plan_t;

LOGLIN_API loglin_status loglin_fwd_plan(int B, int H, int T, int dk, int dv, int C,
                                         loglin_dtype in_dtype, loglin_fwd_plan_t* out);

/*
 * Chunked forward O = (Q K^T (.) M) V over whole sequences.
 *
 * Section 3 of the page splits M into a block diagonal of T/C causal C x C
 * blocks (every level finer than the chunk) plus one term per coarser level,
 * each a decayed state passed between chunks; this entry point computes
 * exactly O, in that chunked form, on the GPU.
 *
 *   q          [B, H, T, dk]  in_dtype
 *   k          [B, H, T, dk]  in_dtype
 *   v          [B, H, T, dv]  in_dtype
 *   log_decay  [B, H, T]      fp32, a_t <= 0 (the gate is exp(a_t))
 *   lambda     [B, H, T, L]   fp32, lambda_t^(l) >= 0, indexed by query t
 *   out        [B, H, T, dv]  fp32, written (not accumulated)
 *   C          chunk size, one of 16, 32, 64, 128; T need not be a multiple
 *              of C (the last chunk is ragged)
 *   dk, dv     each one of 16, 32, 64, 128
 *   L          levels in lambda; must cover every level the sequence uses:
 *              L >= bit_length(T-1) + 1 (L >= 1 for T = 1), and L <= 64
 *   workspace  device buffer of at least loglin_fwd_workspace_bytes(...)
 *              bytes, 256-byte aligned (may be NULL when that is 0); its
 *              contents on entry are ignored and on return are unspecified
 * B, H or T equal to 0 is a no-op.  T / C may be at most 65536 chunks.
 * Numerics: in_dtype BF16 feeds bf16 matrix cores with fp32 accumulation
 * (scores, carried states and V are rounded to bf16 as MFMA operands);
 * in_dtype F32 uses fp32 matrix cores throughout.  Which kernels run is
 * reported by loglin_fwd_plan; the environment variable
 * LOGLIN_FWD_PATH=chunked selects the chunked path for bf16 too.
 */
LOGLIN_API loglin_status loglin_fwd_chunked(const void* q, const void* k, const void* v,
                                 const float* log_decay, const float* lambda, float* out,
                                 int B, int H, int T, int dk, int dv, int L, int C,
                                 loglin_dtype in_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Profiling variant of loglin_fwd_chunked: the same arguments plus a bit mask
 * of the kernels to enqueue, in their fixed order -- bit 0 chunk states,
 * bit 1 Fenwick node scan over chunks, bit 2 output (intra-chunk block plus
 * coarse levels).  Bits 0 and 1 do nothing when T <= C.  `out` is the
 * mixer's output only after all three ran, in order, on the same workspace;
 * running bit 2 alone again after that recomputes the same output.
 * stage_mask = 7 is loglin_fwd_chunked.  Other bits: LOGLIN_EINVAL.
 */
LOGLIN_API loglin_status loglin_fwd_chunked_stages(const void* q, const void* k, const void* v,
                                        const float* log_decay, const float* lambda, float* out,
                                        int B, int H, int T, int dk, int dv, int L, int C,
                                        loglin_dtype in_dtype, void* workspace,
                                        size_t workspace_bytes, unsigned stage_mask,
                                        void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It is loglin_fwd_chunked (same arguments, layouts, limits and
 * numerics; the same kernels, so the same output bit for bit) with the
 * workspace taken from a static device array inside the library instead of
 * an argument.  The caller still passes every input and the output.
 *  - The array holds LOGLIN_NOALLOC_SCRATCH_BYTES (64 MiB).  Sizes whose
 *    workspace (loglin_fwd_workspace_bytes) is larger are rejected with
 *    LOGLIN_EUNSUPPORTED before anything is enqueued.  The bf16 workloads
 *    B=2,H=8,T=2048,d=64 (14 MB), B=4,H=16,T=8192,dk=128,dv=64 (28 MB) and
 *    B=1,H=16,T=65536,d=128 (48 MB) fit.
 *  - Each GPU the library runs on holds its own copy of the array until the
 *    process ends.  The first call on a device looks up that copy's address
 *    (with the device current); no call allocates or frees device memory.
 *  - Every call on one GPU shares that GPU's array: calls that may overlap on
 *    one GPU (two streams, or two threads without ordering between their
 *    calls) race on it and may return wrong outputs.  Order such calls, e.g.
 *    on one stream.  The array needs no clearing between calls.
 */
#define LOGLIN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
LOGLIN_API loglin_status loglin_fwd_chunked_noalloc(const void* q, const void* k, const void* v,
                                                    const float* log_decay, const float* lambda,
                                                    float* out, int B, int H, int T, int dk,
                                                    int dv, int L, int C, loglin_dtype in_dtype,
                                                    void* stream);

/*
 * Log-linear Gated DeltaNet, chunked forward.  "Log-linear attention, and
 * what a logarithm buys": Gated DeltaNet changes the query-key interaction,
 * not the mask (section 1), and the log-linear lift composes its temporal mask
 * with the Fenwick level mask (section 3).  With the gated delta rule of the
 * Gated DeltaNet paper (the page's source 3), every bucket state takes the
 * transition G_t = exp(a_t) (I - beta_t k_t k_t^T) and token t writes
 * beta_t k_t v_t^T into level 0, so
 *   o_t = sum_{s <= t} lambda_t^(level(t,s)) beta_s (q_t^T G_t ... G_{s+1} k_s) v_s,
 * i.e. O = (A (.) M^S (.) M^H) V with
 * A = (Q K^T (.) L)(I + diag(beta)(K K^T (.) (L - I)))^-1 diag(beta).
 *
 *   q, k, v, log_decay, lambda, out, B, H, T, L, in_dtype
 *              as for loglin_fwd_chunked (same layouts)
 *   beta       [B, H, T] fp32, the writing strength, 0 <= beta_t <= 1
 *              (documented, not checked)
 *   dk         64 or 128;  dv  16, 32 or 64 (else LOGLIN_EUNSUPPORTED)
 *   C          validated as for loglin_fwd_chunked; the kernels always work
 *              on 64-token chunks (the result does not depend on the split)
 *   workspace  at least loglin_gdn_fwd_workspace_bytes(...) bytes, 256-byte
 *              aligned (NULL allowed when that is 0); contents on entry
 *              ignored, on return unspecified
 * T may be at most 2^20 (14 levels of 64-token chunks).
 * Numerics: fp32 inputs run on fp32 matrix cores throughout.  bf16 inputs
 * run on bf16 matrix cores with fp32 accumulation; the products whose
 * results carry from chunk to chunk (the chunk transitions and the level
 * states) take each fp32 operand as two bf16 pieces (about 16 significant
 * bits), the rest one piece.  The delta rule's triangular system is
 * inverted per chunk in fp32.  Keys of unit norm keep the transition
 * contractive; other keys are computed as written.  B, H or T equal to 0 is
 * a no-op.
 */
LOGLIN_API size_t loglin_gdn_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C,
                                                 loglin_dtype in_dtype);
LOGLIN_API loglin_status loglin_gdn_fwd_chunked(const void* q, const void* k, const void* v,
                                                const float* log_decay, const float* beta,
                                                const float* lambda, float* out, int B, int H,
                                                int T, int dk, int dv, int L, int C,
                                                loglin_dtype in_dtype, void* workspace,
                                                size_t workspace_bytes, void* stream);
/*
 * Profiling variant: bit 0 the per-chunk kernel (the chunk's own output, its
 * read-out queries, transition and state), bit 1 the walk over chunk levels
 * (adds the coarse levels to `out`).  `out` is the mixer's output only after
 * both ran in order on the same workspace.  Other bits: LOGLIN_EINVAL.
 */
LOGLIN_API loglin_status loglin_gdn_fwd_chunked_stages(const void* q, const void* k, const void* v,
                                                       const float* log_decay, const float* beta,
                                                       const float* lambda, float* out, int B,
                                                       int H, int T, int dk, int dv, int L, int C,
                                                       loglin_dtype in_dtype, void* workspace,
                                                       size_t workspace_bytes, unsigned stage_mask,
                                                       void* stream);

/*
 * Bytes of device workspace loglin_bwd_chunked needs for these sizes, or
 * (size_t)-1 (with the error text set) for sizes it would reject.
 */
LOGLIN_API size_t loglin_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C,
                                             loglin_dtype in_dtype);

/*
 * Backward pass of loglin_fwd_chunked: the gradients of sum(O (.) dO) with
 * respect to every input.  Section 3 of "Log-linear attention, and what a
 * logarithm buys" trains the mixer forward and backward with the same chunk
 * split; section 6 notes that the lambda gradients must be derived by hand.
 * With P = Q K^T (.) M and dP = dO V^T:
 *   dq = (dP (.) M) K,  dk = (dP (.) M)^T Q,  dv = P^T dO,
 *   dlambda_t^(l) = sum over the keys s of level l of dP[t,s] (q_t.k_s) e^(A_t - A_s),
 *   dlog_decay_j = sum_{t >= j} (q_t.dq_t - k_t.dk_t).
 *
 *   q, k, v, log_decay, lambda, B, H, T, dk, dv, L, C, in_dtype
 *              as for loglin_fwd_chunked (same layouts and limits)
 *   dout       [B, H, T, dv]  in_dtype: the gradient of the output
 *   dq, dk_out [B, H, T, dk]  fp32, written
 *   dv_out     [B, H, T, dv]  fp32, written
 *   dlog_decay [B, H, T]      fp32, written
 *   dlambda    [B, H, T, L]   fp32, written (zero at levels a row does not use)
 *   workspace  device buffer of at least loglin_bwd_workspace_bytes(...)
 *              bytes, 256-byte aligned; contents on entry ignored, on
 *              return unspecified
 * q, k, v, dout, dq, dk_out and dv_out must be 16-byte aligned; log_decay,
 * lambda, dlog_decay and dlambda need only 4-byte alignment.  B, H or T
 * equal to 0 is a no-op.  Errors as for loglin_fwd_chunked; nothing is
 * launched when an argument is rejected.  Numerics: bf16 in_dtype feeds
 * bf16 matrix cores with fp32 accumulation (32-deep steps in the fused dq
 * pass and the two walks, which cover C = 64, d_k = 128, d_v = 64; 16-deep
 * in the block-per-chunk kernels that serve the other shapes), the carried
 * states and the masked score tiles rounded to bf16 as operands; the decay
 * gradient's suffix sums run in fp64.
 */
LOGLIN_API loglin_status loglin_bwd_chunked(const void* q, const void* k, const void* v,
                                 const float* log_decay, const float* lambda, const void* dout,
                                 float* dq, float* dk_out, float* dv_out, float* dlog_decay,
                                 float* dlambda, int B, int H, int T, int dk, int dv, int L,
                                 int C, loglin_dtype in_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Decode state ("Log-linear attention, and what a logarithm buys", section 2:
 * every Fenwick bucket of the prefix keeps its own recurrent state, and the
 * live set holds at most ceil(log2 t + 1) + 1 of them): for nseq sequences x
 * H heads, Lmax level states of dk x dv (S = sum k v^T orientation) plus the
 * next position of each sequence.  Levels 7 and up are held as fp32 matrices
 * with a scalar log-scale (the state is the matrix times exp(scale)).  Levels
 * 0..6 of position t hold exactly the tokens of t's 64-token window
 * [t & ~63, t]; loglin_decode_step keeps them as those tokens' raw k, v rows
 * (with the running sum of a) and folds the window into a matrix level at
 * each multiple of 64, so a step inside a window writes one row and reads the
 * window and the matrix levels.  Loaded levels 0..6 are matrices and are kept
 * as such until the next multiple of 64.  loglin_gdn_decode_step keeps every
 * level as a matrix.  loglin_state_export returns the states themselves
 * (dk x dv matrices) either way.  Memory: nseq*H*(Lmax*dk*dv +
 * 64*(dk+dv+1) + dk+dv+Lmax) floats.
 * Allocates device memory (hipMalloc) and zeroes it on `stream`; every
 * sequence starts at position 0.  dk, dv in {16, 32, 64, 128};
 * 1 <= Lmax <= 48.  *st is set only on success.
 */
LOGLIN_API loglin_status loglin_state_init(loglin_state** st, int nseq, int H, int dk, int dv, int Lmax,
                                void* stream);

/*
 * Releases the state's device memory (after synchronising the device).  NULL
 * is a no-op.  The state is the section-2 level set described above.
 */
LOGLIN_API loglin_status loglin_state_free(loglin_state* st);

/*
 * Loads positions and level states (a checkpoint of the section-2 level set,
 * or the output of loglin_prefill_states).
 *   pos_host  [nseq] host int64: next position of each sequence (the state
 *             holds the buckets of tokens 0..pos-1); 0 <= pos <= 2^(Lmax-1)
 *   levels    [nseq, H, Lmax, dk, dv] device fp32, or NULL for all zeros.
 *             Slots that are not live for position pos-1 (slot 0 and slot
 *             p+1 for each set bit p of pos-1 are live) are ignored.
 * The level copy is enqueued on `stream` (`levels` must stay valid until it
 * ran); the call returns after the small position copy has completed.
 */
LOGLIN_API loglin_status loglin_state_load(loglin_state* st, const int64_t* pos_host, const float* levels,
                                void* stream);

/*
 * Exports positions (host, written before return) and the level states
 * [nseq, H, Lmax, dk, dv] (device fp32, enqueued on `stream`), with every
 * slot that is not live written as zero -- the states S_t^(l) of the
 * section-2 recurrence after tokens 0..pos-1 (slot 0 and slot p+1 for each
 * set bit p of pos-1 are live).  Either pointer may be NULL to skip that part.
 */
LOGLIN_API loglin_status loglin_state_export(const loglin_state* st, int64_t* pos_host, float* levels,
                                  void* stream);

/*
 * One Fenwick decode step for every (sequence, head), section 2 of the page:
 * at position t with j = lssb(t) (trailing zero bits of t), levels 0..j are
 * summed and promoted to level j+1, levels above decay by exp(a_t), v_t k_t^T
 * enters level 0 (at t = 0 only that), then o_t = sum_l lambda^(l) q^T S^(l).
 *   q, k   [nseq, H, dk] in_dtype;  v [nseq, H, dv] in_dtype
 *   log_decay [nseq, H] fp32;  lambda [nseq, H, Lmax] fp32
 *   out    [nseq, H, dv] fp32
 * Returns LOGLIN_ECAPACITY (and does nothing) if some sequence's position is
 * 2^(Lmax-1) or more.  Steps on one state must be ordered (same stream).
 */
LOGLIN_API loglin_status loglin_decode_step(loglin_state* st, const void* q, const void* k, const void* v,
                                 const float* log_decay, const float* lambda, float* out,
                                 loglin_dtype in_dtype, void* stream);

/*
 * One decode step of the log-linear Gated DeltaNet for every (sequence, head)
 * on a state from loglin_state_init (section 2's Fenwick update with the gated
 * delta-rule transition of loglin_gdn_fwd_chunked): at position t with
 * j = lssb(t), levels 0..j are summed, taken through
 * G_t = exp(a_t)(I - beta_t k_t k_t^T) and promoted to level j+1; every live
 * level above is taken through G_t; beta_t k_t v_t^T enters level 0 (at t = 0
 * only that); o_t = sum_l lambda^(l) q^T S^(l).
 *   q, k, v, log_decay, lambda, out, in_dtype  as for loglin_decode_step
 *   beta   [nseq, H] fp32
 * A state must be stepped by one mixer only (this call or
 * loglin_decode_step); export and load work the same for both.
 * LOGLIN_ECAPACITY as for loglin_decode_step.
 */
LOGLIN_API loglin_status loglin_gdn_decode_step(loglin_state* st, const void* q, const void* k,
                                                const void* v, const float* log_decay,
                                                const float* beta, const float* lambda, float* out,
                                                loglin_dtype in_dtype, void* stream);

/*
 * Prefill -> decode hand-over ("Log-linear attention, and what a logarithm
 * buys", section 2, with the scalar gate of sections 1 and 3): the Fenwick
 * level states after the T tokens 0..T-1 of each (batch, head) sequence, i.e.
 * the state a decode step at position T reads.  Level 0 holds the last
 * token's k v^T; level p+1, for each set bit p of T-1, the bucket of 2^p
 * tokens the greedy (oldest, largest first) decomposition of the prefix
 * assigns that bit; every token decayed to position T-1:
 *     S^(l) = sum over s in bucket l of exp(A_{T-1} - A_s) k_s v_s^T.
 * The result loads into a decode state with loglin_state_load(pos = T).
 *
 *   k          [B, H, T, dk]  in_dtype
 *   v          [B, H, T, dv]  in_dtype
 *   log_decay  [B, H, T]      fp32
 *   states     [B, H, Lmax, dk, dv] fp32, written; slots that are not live
 *              are zero.  k, v and states 16-byte aligned.
 *   Lmax       1..48 and at least bit_length(T-1) + 1 (else LOGLIN_ECAPACITY)
 *   workspace  device buffer of at least loglin_prefill_workspace_bytes(...)
 *              bytes, 256-byte aligned (NULL allowed when that is 0)
 * T = 0 writes zero states; B or H = 0 is a no-op.  Accumulates in fp32:
 * bf16 inputs on the matrix cores (k v^T products of bf16 operands, the
 * per-token decay rounded to bf16 with v), fp32 inputs with fp32 vector FMAs.
 * Asynchronous on `stream`.
 */
LOGLIN_API size_t loglin_prefill_workspace_bytes(int B, int H, int T, int dk, int dv, int Lmax);
LOGLIN_API loglin_status loglin_prefill_states(const void* k, const void* v, const float* log_decay,
                                               float* states, int B, int H, int T, int dk, int dv,
                                               int Lmax, loglin_dtype in_dtype, void* workspace,
                                               size_t workspace_bytes, void* stream);

/*
 * Level map used by the kernels, for checking: out[t * T + s] = level(t, s)
 * for s <= t and -1 for s > t, where level(t, s) is the Fenwick bucket of
 * key s in the prefix of query t ("Log-linear attention, and what a logarithm
 * buys", section 2: 0 for s = t, else one more than the highest bit in which
 * s and t differ).  out is [T, T] device int8; 1 <= T <= 16384.
 */
LOGLIN_API loglin_status loglin_debug_level_map(int T, int8_t* out, void* stream);

/* Text of the calling thread's last error ("" if none). */
LOGLIN_API const char* loglin_last_error(void);

/* Name of a status code. */
LOGLIN_API const char* loglin_status_string(loglin_status s);

#ifdef __cplusplus
}
#endif

#endif /* LOGLIN_H */
