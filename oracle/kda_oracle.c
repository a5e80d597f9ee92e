/*
 * kda_oracle.c -- plain, slow fp64 CPU oracle for the Kimi Delta Attention (KDA)
 * gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, helper or constant with the HIP
 * library.
 *
 * Sources (cited by page title and section):
 *  - "Kimi K3 ... 昇腾 day-0 adaptation" (hwcomputing.csdn.net), section
 *    "融合算子加速：KDA Prefill与Decode双路径": the order of the steps below (norms,
 *    gate, decay, delta rule, update, output, state back to its pool slot) and the
 *    64-token chunks of the prefill (kda_oracle_chunked).
 *  - "2.8倍性能提升！基于CANN实现Kimi K3高性能推理", section 04 ReplaySSM: the record
 *    {kh | alpha | u} kept per token by a verify pass, and the commit that applies a
 *    sequence's accepted prefix of records, in token order, to its committed state
 *    (kda_oracle_replay).
 *
 * The pages give the step list but no formula.  The formula used here, for one
 * sequence and one head, with state S (dk x dv, row c = key channel):
 *
 *     qh = q / sqrt(sum q^2 + eps),  kh = k / sqrt(sum k^2 + eps)   (Q/K L2 norm)
 *     alpha_c = exp(g_c)                                           (gate, per key channel)
 *     S <- diag(alpha) S                                           (state decay)
 *     delta = v - S^T kh                                           (delta rule)
 *     u = beta * delta                                             (beta processing)
 *     S <- S + kh u^T                                              (outer-product update)
 *     o = scale * S^T qh                                           (output, from the new state)
 *
 * Readings where the pages are silent: eps = 1e-6 inside the square root; the
 * output is taken from the updated state (the pages list the output after the
 * update); scale defaults to 1/sqrt(dk) and is passed in; an update record is
 * {kh, alpha, u}, so replay is S <- diag(alpha) S + kh u^T.
 *
 * Parity status: every function here is pinned by CPU tests (brute force with
 * dense transition matrices, exact rationals, closed forms and invariants); see
 * tests/test_oracle_pins.py.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   q, k, g  [T_total, H, dk]     v [T_total, H, dv]     beta [T_total, H]
 *   o        [T_total, H, dv]     h0, ht [num_seqs, H, dk, dv]
 *   records  [T_total, H, 2*dk + dv] = {kh | alpha | u}
 *   cu_seqlens int64 [num_seqs + 1], cu_seqlens[0] = 0, non-decreasing.
 * A batch of N sequences of T tokens each ([N, T, H, D]) is the same memory as
 * T_total = N*T with cu_seqlens = {0, T, 2T, ...}.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDA_ORACLE_OK 0
#define KDA_ORACLE_EINVAL -1
#define KDA_ORACLE_ENOMEM -2

typedef struct {
    const double *q, *k, *v, *g, *beta;
    const int64_t *cu_seqlens;
    int num_seqs, H, dk, dv;
    double scale, eps;
    int use_qk_l2norm;
    const double *h0;
    double *o, *ht, *records;
    int chunk;          /* 0 = token recurrence, >0 = chunk form with this chunk size */
    int nthreads, tid;
    int status;
} job_t;

/* ---------------------------------------------------------------------------
 * Q/K L2 normalisation of one head vector (section "KDA Prefill与Decode双路径":
 * "Q/K L2Norm").  x_hat = x / sqrt(sum x^2 + eps).
 * ------------------------------------------------------------------------- */
static void l2norm(const double *x, double *out, int d, int use, double eps)
{
    if (!use) {
        memcpy(out, x, sizeof(double) * (size_t)d);
        return;
    }
    double ss = 0.0;
    for (int c = 0; c < d; ++c) ss += x[c] * x[c];
    double inv = 1.0 / sqrt(ss + eps);
    for (int c = 0; c < d; ++c) out[c] = x[c] * inv;
}

/* ---------------------------------------------------------------------------
 * Token-by-token recurrence for one (sequence, head) chain.  Steps in the order
 * the decode kernel description lists them: L2 norm, gate, decay, delta rule,
 * beta, outer-product update, output.
 * ------------------------------------------------------------------------- */
static int run_chain_recurrent(const job_t *J, int n, int h)
{
    const int H = J->H, dk = J->dk, dv = J->dv;
    double *S = (double *)calloc((size_t)dk * dv, sizeof(double));
    double *qh = (double *)malloc(sizeof(double) * dk);
    double *kh = (double *)malloc(sizeof(double) * dk);
    double *al = (double *)malloc(sizeof(double) * dk);
    double *dl = (double *)malloc(sizeof(double) * dv);
    double *u = (double *)malloc(sizeof(double) * dv);
    if (!S || !qh || !kh || !al || !dl || !u) {
        free(S); free(qh); free(kh); free(al); free(dl); free(u);
        return KDA_ORACLE_ENOMEM;
    }
    if (J->h0) memcpy(S, J->h0 + ((size_t)n * H + h) * dk * dv, sizeof(double) * dk * dv);

    for (int64_t t = J->cu_seqlens[n]; t < J->cu_seqlens[n + 1]; ++t) {
        const size_t rk = ((size_t)t * H + h) * dk;   /* row of q, k, g */
        const size_t rv = ((size_t)t * H + h) * dv;   /* row of v, o    */
        const double b = J->beta[(size_t)t * H + h];
        l2norm(J->q + rk, qh, dk, J->use_qk_l2norm, J->eps);
        l2norm(J->k + rk, kh, dk, J->use_qk_l2norm, J->eps);
        for (int c = 0; c < dk; ++c) al[c] = exp(J->g[rk + c]);           /* gate   */
        for (int c = 0; c < dk; ++c)                                       /* decay  */
            for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= al[c];
        for (int j = 0; j < dv; ++j) {                                     /* delta  */
            double p = 0.0;
            for (int c = 0; c < dk; ++c) p += S[(size_t)c * dv + j] * kh[c];
            dl[j] = J->v[rv + j] - p;
            u[j] = b * dl[j];                                              /* beta   */
        }
        for (int c = 0; c < dk; ++c)                                       /* update */
            for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] += kh[c] * u[j];
        for (int j = 0; j < dv; ++j) {                                     /* output */
            double r = 0.0;
            for (int c = 0; c < dk; ++c) r += S[(size_t)c * dv + j] * qh[c];
            J->o[rv + j] = J->scale * r;
        }
        if (J->records) {
            double *rec = J->records + ((size_t)t * H + h) * (size_t)(2 * dk + dv);
            memcpy(rec, kh, sizeof(double) * dk);
            memcpy(rec + dk, al, sizeof(double) * dk);
            memcpy(rec + 2 * dk, u, sizeof(double) * dv);
        }
    }
    if (J->ht) memcpy(J->ht + ((size_t)n * H + h) * dk * dv, S, sizeof(double) * dk * dv);
    free(S); free(qh); free(kh); free(al); free(dl); free(u);
    return KDA_ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Chunk form of the same recurrence, for one (sequence, head) chain.
 *
 * The pages say only that prefill takes 64-token chunks and organises Q/K
 * normalisation, gate cumulation and "Chunk KDA" as batched work (section
 * "KDA Prefill与Decode双路径").  The chunk algebra below is derived from the
 * recurrence; the tests require it to equal the token recurrence to fp64
 * rounding.  For a chunk of L tokens with entering state S0:
 *
 *   G_t  = sum_{s<=t} g_s (inclusive cumulative gate, per key channel)
 *   A_ts = beta_t sum_c kh_tc kh_sc exp(G_tc - G_sc)   (s < t), else 0
 *   P_ts =        sum_c qh_tc kh_sc exp(G_tc - G_sc)   (s <= t), else 0
 *   (I + A) W  = beta (.) kh (.) exp(G)                (forward substitution)
 *   (I + A) Ut = beta (.) V
 *   U    = Ut - W S0                                    (row t is u_t)
 *   O    = scale ((qh (.) exp(G)) S0 + P U)
 *   S_L  = diag(exp(G_L)) S0 + (kh (.) exp(G_L - G))^T U
 *
 * exp(G_tc - G_sc) is evaluated directly from the difference; no factorisation.
 * ------------------------------------------------------------------------- */
static int run_chain_chunked(const job_t *J, int n, int h)
{
    const int H = J->H, dk = J->dk, dv = J->dv, C = J->chunk;
    double *S = (double *)calloc((size_t)dk * dv, sizeof(double));
    double *Sn = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *QH = (double *)malloc(sizeof(double) * (size_t)C * dk);
    double *KH = (double *)malloc(sizeof(double) * (size_t)C * dk);
    double *G = (double *)malloc(sizeof(double) * (size_t)C * dk);
    double *A = (double *)malloc(sizeof(double) * (size_t)C * C);
    double *P = (double *)malloc(sizeof(double) * (size_t)C * C);
    double *W = (double *)malloc(sizeof(double) * (size_t)C * dk);
    double *UT = (double *)malloc(sizeof(double) * (size_t)C * dv);
    double *U = (double *)malloc(sizeof(double) * (size_t)C * dv);
    double *B = (double *)malloc(sizeof(double) * (size_t)C);
    int st = KDA_ORACLE_OK;
    if (!S || !Sn || !QH || !KH || !G || !A || !P || !W || !UT || !U || !B) {
        st = KDA_ORACLE_ENOMEM;
        goto done;
    }
    if (J->h0) memcpy(S, J->h0 + ((size_t)n * H + h) * dk * dv, sizeof(double) * dk * dv);

    for (int64_t t0 = J->cu_seqlens[n]; t0 < J->cu_seqlens[n + 1]; t0 += C) {
        int64_t rem = J->cu_seqlens[n + 1] - t0;
        const int L = rem < C ? (int)rem : C;
        /* Q/K L2 norm, beta, gate cumulation */
        for (int t = 0; t < L; ++t) {
            const size_t rk = ((size_t)(t0 + t) * H + h) * dk;
            l2norm(J->q + rk, QH + (size_t)t * dk, dk, J->use_qk_l2norm, J->eps);
            l2norm(J->k + rk, KH + (size_t)t * dk, dk, J->use_qk_l2norm, J->eps);
            B[t] = J->beta[(size_t)(t0 + t) * H + h];
            for (int c = 0; c < dk; ++c)
                G[(size_t)t * dk + c] = J->g[rk + c] + (t ? G[(size_t)(t - 1) * dk + c] : 0.0);
        }
        /* A (strictly lower) and P (lower incl. diagonal) */
        for (int t = 0; t < L; ++t)
            for (int s = 0; s < L; ++s) {
                double a = 0.0, p = 0.0;
                if (s <= t)
                    for (int c = 0; c < dk; ++c) {
                        double e = exp(G[(size_t)t * dk + c] - G[(size_t)s * dk + c]);
                        a += KH[(size_t)t * dk + c] * KH[(size_t)s * dk + c] * e;
                        p += QH[(size_t)t * dk + c] * KH[(size_t)s * dk + c] * e;
                    }
                A[(size_t)t * C + s] = (s < t) ? B[t] * a : 0.0;
                P[(size_t)t * C + s] = (s <= t) ? p : 0.0;
            }
        /* (I + A) W = beta kh exp(G);  (I + A) Ut = beta V   -- forward substitution */
        for (int t = 0; t < L; ++t) {
            for (int c = 0; c < dk; ++c) {
                double x = B[t] * KH[(size_t)t * dk + c] * exp(G[(size_t)t * dk + c]);
                for (int s = 0; s < t; ++s) x -= A[(size_t)t * C + s] * W[(size_t)s * dk + c];
                W[(size_t)t * dk + c] = x;
            }
            const size_t rv = ((size_t)(t0 + t) * H + h) * dv;
            for (int j = 0; j < dv; ++j) {
                double x = B[t] * J->v[rv + j];
                for (int s = 0; s < t; ++s) x -= A[(size_t)t * C + s] * UT[(size_t)s * dv + j];
                UT[(size_t)t * dv + j] = x;
            }
        }
        /* U = Ut - W S0 */
        for (int t = 0; t < L; ++t)
            for (int j = 0; j < dv; ++j) {
                double x = UT[(size_t)t * dv + j];
                for (int c = 0; c < dk; ++c) x -= W[(size_t)t * dk + c] * S[(size_t)c * dv + j];
                U[(size_t)t * dv + j] = x;
            }
        /* O = scale ((qh exp(G)) S0 + P U) */
        for (int t = 0; t < L; ++t) {
            const size_t rv = ((size_t)(t0 + t) * H + h) * dv;
            for (int j = 0; j < dv; ++j) {
                double x = 0.0;
                for (int c = 0; c < dk; ++c)
                    x += QH[(size_t)t * dk + c] * exp(G[(size_t)t * dk + c]) * S[(size_t)c * dv + j];
                for (int s = 0; s <= t; ++s) x += P[(size_t)t * C + s] * U[(size_t)s * dv + j];
                J->o[rv + j] = J->scale * x;
            }
        }
        /* S_L = diag(exp(G_L)) S0 + (kh exp(G_L - G))^T U */
        const double *GL = G + (size_t)(L - 1) * dk;
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) {
                double x = exp(GL[c]) * S[(size_t)c * dv + j];
                for (int t = 0; t < L; ++t)
                    x += KH[(size_t)t * dk + c] * exp(GL[c] - G[(size_t)t * dk + c]) * U[(size_t)t * dv + j];
                Sn[(size_t)c * dv + j] = x;
            }
        memcpy(S, Sn, sizeof(double) * dk * dv);
    }
    if (J->ht) memcpy(J->ht + ((size_t)n * H + h) * dk * dv, S, sizeof(double) * dk * dv);
done:
    free(S); free(Sn); free(QH); free(KH); free(G); free(A); free(P);
    free(W); free(UT); free(U); free(B);
    return st;
}

/* Static round-robin split of the independent (sequence, head) chains. */
static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int nchains = J->num_seqs * J->H;
    for (int i = J->tid; i < nchains; i += J->nthreads) {
        int n = i / J->H, h = i % J->H;
        int st = J->chunk > 0 ? run_chain_chunked(J, n, h) : run_chain_recurrent(J, n, h);
        if (st != KDA_ORACLE_OK) J->status = st;
    }
    return NULL;
}

static int run_all(const job_t *proto)
{
    int nt = proto->nthreads < 1 ? 1 : proto->nthreads;
    const int nchains = proto->num_seqs * proto->H;
    if (nt > nchains) nt = nchains > 0 ? nchains : 1;
    job_t *jobs = (job_t *)calloc((size_t)nt, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs); free(th);
        return KDA_ORACLE_ENOMEM;
    }
    for (int i = 0; i < nt; ++i) {
        jobs[i] = *proto;
        jobs[i].nthreads = nt;
        jobs[i].tid = i;
        jobs[i].status = KDA_ORACLE_OK;
    }
    for (int i = 1; i < nt; ++i)
        if (pthread_create(&th[i], NULL, worker, &jobs[i]) != 0) {
            /* fall back to running this share on the calling thread */
            worker(&jobs[i]);
            th[i] = 0;
        }
    worker(&jobs[0]);
    int st = KDA_ORACLE_OK;
    for (int i = 1; i < nt; ++i)
        if (th[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < nt; ++i)
        if (jobs[i].status != KDA_ORACLE_OK) st = jobs[i].status;
    free(jobs); free(th);
    return st;
}

static int check_common(const double *q, const double *k, const double *v, const double *g,
                        const double *beta, const int64_t *cu, int num_seqs, int H, int dk,
                        int dv, const double *o)
{
    if (!q || !k || !v || !g || !beta || !cu || !o) return KDA_ORACLE_EINVAL;
    if (num_seqs < 0 || H < 1 || dk < 1 || dv < 1) return KDA_ORACLE_EINVAL;
    if (cu[0] != 0) return KDA_ORACLE_EINVAL;
    for (int i = 0; i < num_seqs; ++i)
        if (cu[i + 1] < cu[i]) return KDA_ORACLE_EINVAL;
    return KDA_ORACLE_OK;
}

/* Token recurrence over varlen sequences.  h0 may be NULL (zero state); ht and
 * records may be NULL.  Returns 0 on success. */
int kda_oracle_recurrent(const double *q, const double *k, const double *v, const double *g,
                         const double *beta, const int64_t *cu_seqlens, int num_seqs, int H,
                         int dk, int dv, double scale, int use_qk_l2norm, double eps,
                         const double *h0, double *o, double *ht, double *records, int nthreads)
{
    int st = check_common(q, k, v, g, beta, cu_seqlens, num_seqs, H, dk, dv, o);
    if (st) return st;
    job_t J = {q, k, v, g, beta, cu_seqlens, num_seqs, H, dk, dv, scale, eps, use_qk_l2norm,
               h0, o, ht, records, 0, nthreads, 0, 0};
    return run_all(&J);
}

/* Chunk form (chunk >= 1) over varlen sequences; chunks restart at every
 * sequence start and the last chunk of a sequence may be shorter. */
int kda_oracle_chunked(const double *q, const double *k, const double *v, const double *g,
                       const double *beta, const int64_t *cu_seqlens, int num_seqs, int H,
                       int dk, int dv, double scale, int use_qk_l2norm, double eps,
                       const double *h0, double *o, double *ht, int chunk, int nthreads)
{
    int st = check_common(q, k, v, g, beta, cu_seqlens, num_seqs, H, dk, dv, o);
    if (st) return st;
    if (chunk < 1) return KDA_ORACLE_EINVAL;
    job_t J = {q, k, v, g, beta, cu_seqlens, num_seqs, H, dk, dv, scale, eps, use_qk_l2norm,
               h0, o, ht, NULL, chunk, nthreads, 0, 0};
    return run_all(&J);
}

/* ReplaySSM commit (section 04): for each sequence n, starting from the committed
 * state[n] ([H, dk, dv]), apply the records of tokens 0 .. accepted[n]-1 in order:
 * S <- diag(alpha) S + kh u^T.  records [N, T, H, 2*dk + dv]. */
int kda_oracle_replay(double *state, const double *records, const int64_t *accepted, int N,
                      int T, int H, int dk, int dv)
{
    if (!state || !records || !accepted || N < 0 || T < 0 || H < 1 || dk < 1 || dv < 1)
        return KDA_ORACLE_EINVAL;
    const size_t R = (size_t)(2 * dk + dv);
    for (int n = 0; n < N; ++n) {
        if (accepted[n] < 0 || accepted[n] > T) return KDA_ORACLE_EINVAL;
        for (int h = 0; h < H; ++h) {
            double *S = state + ((size_t)n * H + h) * dk * dv;
            for (int t = 0; t < accepted[n]; ++t) {
                const double *rec = records + (((size_t)n * T + t) * H + h) * R;
                const double *kh = rec, *al = rec + dk, *u = rec + 2 * dk;
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j)
                        S[(size_t)c * dv + j] = al[c] * S[(size_t)c * dv + j] + kh[c] * u[j];
            }
        }
    }
    return KDA_ORACLE_OK;
}
