/*
 * loglin_oracle.c -- plain, slow, fp64 CPU oracle for the log-linear
 * (Fenwick-tree) token mixer.  TEST INFRASTRUCTURE ONLY: it is loaded by the
 * test-suite, by the smoke check and by the CPU-baseline leg of the benchmark,
 * and by nothing on the product path.  It shares no code, header or constant
 * with the HIP library.
 *
 * What it computes follows "Log-linear attention, and what a logarithm buys":
 *
 *  - section 2 ("What structure buys the middle"): the prefix before position t
 *    is cut into Fenwick buckets by the least significant set bit of t; each
 *    bucket keeps its own state S^(l) (here d_k x d_v, S = sum k v^T); the
 *    output is o_t = sum_l lambda_t^(l) q_t^T S_t^(l); the decode recurrence
 *    puts the new outer product into level zero, merges every level up to
 *    lssb(t) and promotes the sum one level coarser.
 *  - section 1 ("The framing that makes the mechanism obvious"): Mamba-2's
 *    mask is 1-semiseparable, i.e. a scalar gate alpha_t = exp(a_t) per token;
 *    section 3 ("Where the log-linear cost is actually earned") composes that
 *    temporal mask with the level mask by an elementwise product, so every
 *    state is decayed by alpha_t at every step (the Mamba-2 recurrence
 *    S_t = alpha_t S_{t-1} + k_t v_t^T, applied to every bucket).
 *
 * Positions are 0-indexed.  At t = 0 only level 0 is written.  At t >= 1,
 * with j = number of trailing zero bits of t:
 *     S^(j+1) <- alpha_t * (S^(0) + ... + S^(j))
 *     S^(1..j) <- 0
 *     S^(l)   <- alpha_t * S^(l)          for l > j+1
 *     S^(0)   <- k_t v_t^T
 *     o_t      = sum_l lambda_t^(l) q_t^T S^(l)
 *
 * The set of live (possibly nonzero) levels is tracked as a bit mask by the
 * recurrence itself and checked against {0} U {p+1 : bit p of t} and against
 * the bucket bound ceil(log2 t + 1) + 1 that section 2 states; a violation is
 * reported as an error code, never silently ignored.
 *
 * The log-linear Gated DeltaNet (same page: section 1 says Gated DeltaNet
 * differs from Mamba-2 in how it structures A, not M, and section 3 lifts any
 * such layer by composing its temporal mask with the level mask) follows the
 * same Fenwick recurrence with the gated delta-rule transition of the Gated
 * DeltaNet paper (the page's source 3) in place of the scalar gate: every
 * carried (and merged) state is multiplied on the left by
 *     G_t = alpha_t (I - beta_t k_t k_t^T),
 * and the new token writes beta_t k_t v_t^T into level zero (gdn_step).
 *
 * Build:  gcc -O2 -shared -fPIC loglin_oracle.c -o liblloracle.so -lm -lpthread
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LLO_OK 0
#define LLO_EARG 1      /* bad argument */
#define LLO_ECAP 2      /* position needs a level index >= L */
#define LLO_ELIVE 3     /* live-set invariant violated */
#define LLO_ENOMEM 4

/* number of trailing zero bits of t (t >= 1), by repeated halving */
static int trailing_zeros(int64_t t) {
    int j = 0;
    while ((t % 2) == 0) {
        t /= 2;
        j++;
    }
    return j;
}

/* ceil(log2(t) + 1) + 1 for t >= 1, computed with doubles as the page writes it */
static int bucket_bound(int64_t t) {
    return (int)ceil(log2((double)t) + 1.0) + 1;
}

static int popcount64(uint64_t x) {
    int c = 0;
    while (x) {
        c += (int)(x & 1u);
        x >>= 1;
    }
    return c;
}

/*
 * One Fenwick step at position t for one (sequence, head).
 *   S      [L][dk][dv] states, updated in place
 *   live   bit mask of live levels, updated in place
 *   q,k    [dk]; v [dv]; a scalar log-decay; lam [L]; out [dv]
 */
static int fenwick_step(double* S, uint64_t* live, int64_t t, const double* q,
                        const double* k, const double* v, double a,
                        const double* lam, double* out, int dk, int dv, int L) {
    const size_t nst = (size_t)dk * dv;
    const double alpha = exp(a);
    if (t == 0) {
        memset(S, 0, sizeof(double) * nst * L);
        *live = 1;
    } else {
        const int j = trailing_zeros(t);
        if (j + 1 >= L) return LLO_ECAP;
        for (int l = j + 2; l < L; l++) {
            if ((*live >> l) & 1) {
                double* s = S + nst * l;
                for (size_t e = 0; e < nst; e++) s[e] *= alpha;
            }
        }
        double* dst = S + nst * (j + 1);
        /* level j+1 is not live before the merge (bit j of t-1 is zero) */
        for (size_t e = 0; e < nst; e++) {
            double acc = 0.0;
            for (int l = 0; l <= j; l++) acc += S[nst * l + e];
            dst[e] = alpha * acc;
        }
        for (int l = 1; l <= j; l++) memset(S + nst * l, 0, sizeof(double) * nst);
        uint64_t nl = *live;
        for (int l = 0; l <= j; l++) nl &= ~((uint64_t)1 << l);
        nl |= (uint64_t)1 << (j + 1);
        nl |= 1;
        *live = nl;
    }
    /* level zero holds the current token alone */
    for (int r = 0; r < dk; r++)
        for (int c = 0; c < dv; c++) S[(size_t)r * dv + c] = k[r] * v[c];

    if (t >= 1) {
        if (*live != (((uint64_t)t << 1) | 1)) return LLO_ELIVE;
        if (popcount64(*live) > bucket_bound(t)) return LLO_ELIVE;
    } else if (*live != 1) {
        return LLO_ELIVE;
    }

    for (int c = 0; c < dv; c++) out[c] = 0.0;
    for (int l = 0; l < L; l++) {
        if (!((*live >> l) & 1)) continue;
        const double* s = S + nst * l;
        for (int c = 0; c < dv; c++) {
            double dot = 0.0;
            for (int r = 0; r < dk; r++) dot += q[r] * s[(size_t)r * dv + c];
            out[c] += lam[l] * dot;
        }
    }
    return LLO_OK;
}

/* X <- alpha (I - beta k k^T) X for one d_k x d_v state; w is [dv] scratch */
static void delta_transition(double* X, const double* k, double alpha, double beta, double* w,
                             int dk, int dv) {
    for (int c = 0; c < dv; c++) {
        double acc = 0.0;
        for (int r = 0; r < dk; r++) acc += k[r] * X[(size_t)r * dv + c];
        w[c] = acc;
    }
    for (int r = 0; r < dk; r++)
        for (int c = 0; c < dv; c++)
            X[(size_t)r * dv + c] = alpha * (X[(size_t)r * dv + c] - beta * k[r] * w[c]);
}

/*
 * One Fenwick step of the log-linear Gated DeltaNet at position t: the step of
 * fenwick_step with every carried or merged state taken through
 * G_t = alpha_t (I - beta_t k_t k_t^T) instead of alpha_t, and beta_t k_t v_t^T
 * written to level zero.  w is [dv] scratch.
 */
static int gdn_step(double* S, uint64_t* live, int64_t t, const double* q, const double* k,
                    const double* v, double a, double beta, const double* lam, double* out,
                    double* w, int dk, int dv, int L) {
    const size_t nst = (size_t)dk * dv;
    const double alpha = exp(a);
    if (t == 0) {
        memset(S, 0, sizeof(double) * nst * L);
        *live = 1;
    } else {
        const int j = trailing_zeros(t);
        if (j + 1 >= L) return LLO_ECAP;
        for (int l = j + 2; l < L; l++)
            if ((*live >> l) & 1) delta_transition(S + nst * l, k, alpha, beta, w, dk, dv);
        double* dst = S + nst * (j + 1);
        /* level j+1 is not live before the merge (bit j of t-1 is zero) */
        for (size_t e = 0; e < nst; e++) {
            double acc = 0.0;
            for (int l = 0; l <= j; l++) acc += S[nst * l + e];
            dst[e] = acc;
        }
        delta_transition(dst, k, alpha, beta, w, dk, dv);
        for (int l = 1; l <= j; l++) memset(S + nst * l, 0, sizeof(double) * nst);
        uint64_t nl = *live;
        for (int l = 0; l <= j; l++) nl &= ~((uint64_t)1 << l);
        nl |= (uint64_t)1 << (j + 1);
        nl |= 1;
        *live = nl;
    }
    /* level zero holds the current token's write alone */
    for (int r = 0; r < dk; r++)
        for (int c = 0; c < dv; c++) S[(size_t)r * dv + c] = beta * k[r] * v[c];

    if (t >= 1) {
        if (*live != (((uint64_t)t << 1) | 1)) return LLO_ELIVE;
        if (popcount64(*live) > bucket_bound(t)) return LLO_ELIVE;
    } else if (*live != 1) {
        return LLO_ELIVE;
    }

    for (int c = 0; c < dv; c++) out[c] = 0.0;
    for (int l = 0; l < L; l++) {
        if (!((*live >> l) & 1)) continue;
        const double* s = S + nst * l;
        for (int c = 0; c < dv; c++) {
            double dot = 0.0;
            for (int r = 0; r < dk; r++) dot += q[r] * s[(size_t)r * dv + c];
            out[c] += lam[l] * dot;
        }
    }
    return LLO_OK;
}

/* ------------------------------------------------------------------------ */
/* forward over whole sequences                                              */

typedef struct {
    const double *q, *k, *v, *a, *lam;
    double *out, *states_out;
    long BH, T;
    int dk, dv, L;
    long next; /* next slice to take */
    pthread_mutex_t mu;
    int err;
    const double* beta; /* [BH][T] for the Gated DeltaNet recurrence, else NULL */
} fwd_job;

static void* fwd_worker(void* p) {
    fwd_job* J = (fwd_job*)p;
    const size_t nst = (size_t)J->dk * J->dv;
    double* S = (double*)malloc(sizeof(double) * (nst * J->L + J->dv));
    if (!S) {
        pthread_mutex_lock(&J->mu);
        J->err = LLO_ENOMEM;
        pthread_mutex_unlock(&J->mu);
        return NULL;
    }
    double* w = S + nst * J->L;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        long bh = J->next++;
        int stop = J->err != LLO_OK;
        pthread_mutex_unlock(&J->mu);
        if (stop || bh >= J->BH) break;
        uint64_t live = 0;
        for (long t = 0; t < J->T; t++) {
            const size_t row = (size_t)bh * J->T + t;
            int rc = J->beta
                ? gdn_step(S, &live, t, J->q + row * J->dk, J->k + row * J->dk,
                           J->v + row * J->dv, J->a[row], J->beta[row], J->lam + row * J->L,
                           J->out + row * J->dv, w, J->dk, J->dv, J->L)
                : fenwick_step(S, &live, t, J->q + row * J->dk, J->k + row * J->dk,
                               J->v + row * J->dv, J->a[row], J->lam + row * J->L,
                               J->out + row * J->dv, J->dk, J->dv, J->L);
            if (rc != LLO_OK) {
                pthread_mutex_lock(&J->mu);
                J->err = rc;
                pthread_mutex_unlock(&J->mu);
                break;
            }
        }
        if (J->states_out && J->err == LLO_OK)
            memcpy(J->states_out + (size_t)bh * nst * J->L, S, sizeof(double) * nst * J->L);
    }
    free(S);
    return NULL;
}

/*
 * Form B forward: o_t for every token of BH independent (batch, head) slices.
 *   q, k [BH][T][dk], v [BH][T][dv], a [BH][T], lam [BH][T][L]   (fp64)
 *   out [BH][T][dv]; states_out (may be NULL) [BH][L][dk][dv] = the states
 *   after the last token.
 * nthreads <= 0 means one thread.  Returns an LLO_* code.
 */
int llo_fwd_recurrent(const double* q, const double* k, const double* v, const double* a,
                      const double* lam, double* out, double* states_out, long BH, long T,
                      int dk, int dv, int L, int nthreads) {
    if (!q || !k || !v || !a || !lam || !out || BH < 0 || T < 0 || dk <= 0 || dv <= 0 ||
        L < 1 || L > 63)
        return LLO_EARG;
    fwd_job J = {q, k, v, a, lam, out, states_out, BH, T, dk, dv, L, 0,
                 PTHREAD_MUTEX_INITIALIZER, LLO_OK, NULL};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    for (int i = 0; i < nthreads; i++) pthread_create(&th[i], NULL, fwd_worker, &J);
    for (int i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
    return J.err;
}

/*
 * Log-linear Gated DeltaNet, Form B: as llo_fwd_recurrent with the per-token
 * writing strength beta [BH][T] (gdn_step).
 */
int llo_gdn_fwd_recurrent(const double* q, const double* k, const double* v, const double* a,
                          const double* beta, const double* lam, double* out, double* states_out,
                          long BH, long T, int dk, int dv, int L, int nthreads) {
    if (!q || !k || !v || !a || !beta || !lam || !out || BH < 0 || T < 0 || dk <= 0 ||
        dv <= 0 || L < 1 || L > 63)
        return LLO_EARG;
    fwd_job J = {q, k, v, a, lam, out, states_out, BH, T, dk, dv, L, 0,
                 PTHREAD_MUTEX_INITIALIZER, LLO_OK, beta};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    for (int i = 0; i < nthreads; i++) pthread_create(&th[i], NULL, fwd_worker, &J);
    for (int i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
    return J.err;
}

/* ------------------------------------------------------------------------ */
/* decode: continue independent (sequence, head) pairs from given states     */

typedef struct {
    double* states;
    int64_t* pos;
    const double *q, *k, *v, *a, *lam;
    double* out;
    long P;
    int steps, dk, dv, L;
    long next;
    pthread_mutex_t mu;
    int err;
    const double* beta; /* [steps][P] for the Gated DeltaNet recurrence, else NULL */
} dec_job;

static void* dec_worker(void* p) {
    dec_job* J = (dec_job*)p;
    const size_t nst = (size_t)J->dk * J->dv;
    double* w = (double*)malloc(sizeof(double) * J->dv);
    if (!w) {
        pthread_mutex_lock(&J->mu);
        J->err = LLO_ENOMEM;
        pthread_mutex_unlock(&J->mu);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&J->mu);
        long i = J->next++;
        int stop = J->err != LLO_OK;
        pthread_mutex_unlock(&J->mu);
        if (stop || i >= J->P) break;
        double* S = J->states + (size_t)i * nst * J->L;
        int64_t t = J->pos[i];
        /* live set implied by the position: levels of the buckets of t-1 */
        uint64_t live = t == 0 ? 0 : ((((uint64_t)(t - 1)) << 1) | 1);
        for (int st = 0; st < J->steps; st++, t++) {
            const size_t row = (size_t)st * J->P + i;
            int rc = J->beta
                ? gdn_step(S, &live, t, J->q + row * J->dk, J->k + row * J->dk,
                           J->v + row * J->dv, J->a[row], J->beta[row], J->lam + row * J->L,
                           J->out + row * J->dv, w, J->dk, J->dv, J->L)
                : fenwick_step(S, &live, t, J->q + row * J->dk, J->k + row * J->dk,
                               J->v + row * J->dv, J->a[row], J->lam + row * J->L,
                               J->out + row * J->dv, J->dk, J->dv, J->L);
            if (rc != LLO_OK) {
                pthread_mutex_lock(&J->mu);
                J->err = rc;
                pthread_mutex_unlock(&J->mu);
                break;
            }
        }
        J->pos[i] = t;
    }
    free(w);
    return NULL;
}

/*
 * Decode `steps` tokens for P independent (sequence, head) pairs.
 *   states [P][L][dk][dv] in/out; pos [P] in/out = next position to decode
 *   (the state holds the buckets of tokens 0..pos-1; levels that are not live
 *   for pos-1 must be zero and are ignored).
 *   q, k [steps][P][dk]; v [steps][P][dv]; a [steps][P]; lam [steps][P][L];
 *   out [steps][P][dv].
 */
int llo_decode(double* states, int64_t* pos, const double* q, const double* k,
               const double* v, const double* a, const double* lam, double* out, long P,
               int steps, int dk, int dv, int L, int nthreads) {
    if (!states || !pos || !q || !k || !v || !a || !lam || !out || P < 0 || steps < 0 ||
        dk <= 0 || dv <= 0 || L < 1 || L > 63)
        return LLO_EARG;
    for (long i = 0; i < P; i++)
        if (pos[i] < 0) return LLO_EARG;
    dec_job J = {states, pos, q, k, v, a, lam, out, P, steps, dk, dv, L, 0,
                 PTHREAD_MUTEX_INITIALIZER, LLO_OK, NULL};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    for (int i = 0; i < nthreads; i++) pthread_create(&th[i], NULL, dec_worker, &J);
    for (int i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
    return J.err;
}

/* Log-linear Gated DeltaNet decode: llo_decode with beta [steps][P] (gdn_step). */
int llo_gdn_decode(double* states, int64_t* pos, const double* q, const double* k,
                   const double* v, const double* a, const double* beta, const double* lam,
                   double* out, long P, int steps, int dk, int dv, int L, int nthreads) {
    if (!states || !pos || !q || !k || !v || !a || !beta || !lam || !out || P < 0 ||
        steps < 0 || dk <= 0 || dv <= 0 || L < 1 || L > 63)
        return LLO_EARG;
    for (long i = 0; i < P; i++)
        if (pos[i] < 0) return LLO_EARG;
    dec_job J = {states, pos, q, k, v, a, lam, out, P, steps, dk, dv, L, 0,
                 PTHREAD_MUTEX_INITIALIZER, LLO_OK, beta};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    for (int i = 0; i < nthreads; i++) pthread_create(&th[i], NULL, dec_worker, &J);
    for (int i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
    return J.err;
}
