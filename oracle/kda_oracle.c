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

/* ---------------------------------------------------------------------------
 * Backward of the token recurrence (gradients of L = sum(do * o) + sum(dht * ht)),
 * one (sequence, head) chain per call.  The page's training section (the item on
 * linear-attention kernels built with Triton-Ascend, "基于昇腾实现Kimi K3训练基础功能适配
 * 与深度优化") names backward kernels but prints no formula; this is the chain rule
 * through the steps of run_chain_recurrent in reverse token order, with
 * D = dL/dS_t carried backwards (the same steps as oracle/kda_backward.py):
 *
 *   dqh_t = scale S_t do_t ;  D += scale qh_t do_t^T
 *   du_t = D^T kh_t ;  dkh_t = D u_t
 *   dbeta_t = du_t . (v_t - p_t) ;  dv_t = beta_t du_t ;  dp_t = -beta_t du_t
 *   D' = D + kh_t dp_t^T ;  dkh_t += S'_t dp_t
 *   dg_t = alpha_t * rowsum(D' * S_{t-1}) ;  D <- diag(alpha_t) D'
 *   dq_t = (dqh_t - qh_t (qh_t . dqh_t)) / sqrt(|q_t|^2 + eps)  (k likewise; identity
 *                                                                 without the norm)
 *   dh0 = D after the first token.
 *
 * The forward states are needed in reverse order: the forward pass keeps the state at
 * every 64-token boundary, and the backward recomputes the states of one 64-token span
 * at a time from its kept state with the same forward steps.
 * ------------------------------------------------------------------------- */
typedef struct {
    const double *q, *k, *v, *g, *beta, *h0, *dout, *dht;
    const int64_t *cu_seqlens;
    int num_seqs, H, dk, dv, use_qk_l2norm;
    double scale, eps;
    double *dq, *dk_, *dv_, *dg, *dbeta, *dh0;
    int nthreads, tid, status;
} bwd_job_t;

#define BWD_SPAN 64

/* One forward token step from S (dk x dv) into Sn, keeping S' = diag(alpha) S, p, u and
 * the normalised q and k. */
static void fwd_token(const bwd_job_t *J, int64_t t, int h, const double *S, double *Sp,
                      double *Sn, double *qh, double *kh, double *nq, double *nk, double *al,
                      double *p, double *u)
{
    const int H = J->H, dk = J->dk, dv = J->dv;
    const size_t rk = ((size_t)t * H + h) * dk, rv = ((size_t)t * H + h) * dv;
    double sq = 0.0, sk = 0.0;
    for (int c = 0; c < dk; ++c) {
        sq += J->q[rk + c] * J->q[rk + c];
        sk += J->k[rk + c] * J->k[rk + c];
    }
    *nq = J->use_qk_l2norm ? sqrt(sq + J->eps) : 1.0;
    *nk = J->use_qk_l2norm ? sqrt(sk + J->eps) : 1.0;
    for (int c = 0; c < dk; ++c) {
        qh[c] = J->q[rk + c] / *nq;
        kh[c] = J->k[rk + c] / *nk;
        al[c] = exp(J->g[rk + c]);
    }
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) Sp[(size_t)c * dv + j] = al[c] * S[(size_t)c * dv + j];
    const double b = J->beta[(size_t)t * H + h];
    for (int j = 0; j < dv; ++j) {
        double x = 0.0;
        for (int c = 0; c < dk; ++c) x += Sp[(size_t)c * dv + j] * kh[c];
        p[j] = x;
        u[j] = b * (J->v[rv + j] - x);
    }
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) Sn[(size_t)c * dv + j] = Sp[(size_t)c * dv + j] + kh[c] * u[j];
}

static int run_chain_backward(const bwd_job_t *J, int n, int h)
{
    const int H = J->H, dk = J->dk, dv = J->dv;
    const size_t SZ = (size_t)dk * dv;
    const int64_t bos = J->cu_seqlens[n], eos = J->cu_seqlens[n + 1];
    const int64_t nspan = (eos - bos + BWD_SPAN - 1) / BWD_SPAN;
    double *ck = (double *)malloc(sizeof(double) * SZ * (size_t)(nspan > 0 ? nspan : 1));
    double *Sprev = (double *)malloc(sizeof(double) * SZ * BWD_SPAN);
    double *Spv = (double *)malloc(sizeof(double) * SZ * BWD_SPAN);
    double *Snew = (double *)malloc(sizeof(double) * SZ * BWD_SPAN);
    double *D = (double *)malloc(sizeof(double) * SZ);
    double *Dp = (double *)malloc(sizeof(double) * SZ);
    double *QH = (double *)malloc(sizeof(double) * (size_t)dk * BWD_SPAN);
    double *KH = (double *)malloc(sizeof(double) * (size_t)dk * BWD_SPAN);
    double *AL = (double *)malloc(sizeof(double) * (size_t)dk * BWD_SPAN);
    double *PP = (double *)malloc(sizeof(double) * (size_t)dv * BWD_SPAN);
    double *UU = (double *)malloc(sizeof(double) * (size_t)dv * BWD_SPAN);
    double *NQ = (double *)malloc(sizeof(double) * BWD_SPAN);
    double *NK = (double *)malloc(sizeof(double) * BWD_SPAN);
    double *dqh = (double *)malloc(sizeof(double) * dk);
    double *dkh = (double *)malloc(sizeof(double) * dk);
    double *du = (double *)malloc(sizeof(double) * dv);
    int st = KDA_ORACLE_OK;
    if (!ck || !Sprev || !Spv || !Snew || !D || !Dp || !QH || !KH || !AL || !PP || !UU || !NQ ||
        !NK || !dqh || !dkh || !du) {
        st = KDA_ORACLE_ENOMEM;
        goto done;
    }
    /* forward: the state entering every 64-token span */
    {
        double *S = Sprev, *Sn = Snew;
        if (J->h0) memcpy(S, J->h0 + ((size_t)n * H + h) * SZ, sizeof(double) * SZ);
        else memset(S, 0, sizeof(double) * SZ);
        for (int64_t m = 0; m < nspan; ++m) {
            memcpy(ck + (size_t)m * SZ, S, sizeof(double) * SZ);
            const int64_t t1 = bos + (m + 1) * BWD_SPAN < eos ? bos + (m + 1) * BWD_SPAN : eos;
            for (int64_t t = bos + m * BWD_SPAN; t < t1; ++t) {
                fwd_token(J, t, h, S, Spv, Sn, QH, KH, NQ, NK, AL, PP, UU);
                double *x = S; S = Sn; Sn = x;
            }
        }
    }
    /* backward, one span at a time from the last */
    if (J->dht) memcpy(D, J->dht + ((size_t)n * H + h) * SZ, sizeof(double) * SZ);
    else memset(D, 0, sizeof(double) * SZ);
    for (int64_t m = nspan - 1; m >= 0; --m) {
        const int64_t t0 = bos + m * BWD_SPAN;
        const int L = (int)((t0 + BWD_SPAN < eos ? t0 + BWD_SPAN : eos) - t0);
        memcpy(Sprev, ck + (size_t)m * SZ, sizeof(double) * SZ);
        for (int i = 0; i < L; ++i) {
            if (i > 0) memcpy(Sprev + (size_t)i * SZ, Snew + (size_t)(i - 1) * SZ, sizeof(double) * SZ);
            fwd_token(J, t0 + i, h, Sprev + (size_t)i * SZ, Spv + (size_t)i * SZ, Snew + (size_t)i * SZ,
                      QH + (size_t)i * dk, KH + (size_t)i * dk, NQ + i, NK + i, AL + (size_t)i * dk,
                      PP + (size_t)i * dv, UU + (size_t)i * dv);
        }
        for (int i = L - 1; i >= 0; --i) {
            const int64_t t = t0 + i;
            const size_t rk = ((size_t)t * H + h) * dk, rv = ((size_t)t * H + h) * dv;
            const double *S1 = Snew + (size_t)i * SZ, *S0 = Sprev + (size_t)i * SZ;
            const double *Sp = Spv + (size_t)i * SZ;
            const double *qh = QH + (size_t)i * dk, *kh = KH + (size_t)i * dk, *al = AL + (size_t)i * dk;
            const double *p = PP + (size_t)i * dv, *u = UU + (size_t)i * dv;
            const double *dout = J->dout + rv;
            const double b = J->beta[(size_t)t * H + h];
            /* output: o = scale S_t^T qh */
            for (int c = 0; c < dk; ++c) {
                double x = 0.0;
                for (int j = 0; j < dv; ++j) x += S1[(size_t)c * dv + j] * dout[j];
                dqh[c] = J->scale * x;
            }
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j) D[(size_t)c * dv + j] += J->scale * qh[c] * dout[j];
            /* update S_t = S'_t + kh u^T */
            double db = 0.0;
            for (int j = 0; j < dv; ++j) {
                double x = 0.0;
                for (int c = 0; c < dk; ++c) x += D[(size_t)c * dv + j] * kh[c];
                du[j] = x;
                db += x * (J->v[rv + j] - p[j]);
            }
            for (int c = 0; c < dk; ++c) {
                double x = 0.0;
                for (int j = 0; j < dv; ++j) x += D[(size_t)c * dv + j] * u[j];
                dkh[c] = x;
            }
            /* u = beta (v - p), p = S'^T kh */
            J->dbeta[(size_t)t * H + h] = db;
            for (int j = 0; j < dv; ++j) J->dv_[rv + j] = b * du[j];
            for (int c = 0; c < dk; ++c) {
                double x = 0.0;
                for (int j = 0; j < dv; ++j) {
                    const double dp = -b * du[j];
                    Dp[(size_t)c * dv + j] = D[(size_t)c * dv + j] + kh[c] * dp;
                    x += Sp[(size_t)c * dv + j] * dp;
                }
                dkh[c] += x;
            }
            /* S' = diag(alpha) S_{t-1}, alpha = exp(g) */
            for (int c = 0; c < dk; ++c) {
                double x = 0.0;
                for (int j = 0; j < dv; ++j) x += Dp[(size_t)c * dv + j] * S0[(size_t)c * dv + j];
                J->dg[rk + c] = al[c] * x;
                for (int j = 0; j < dv; ++j) D[(size_t)c * dv + j] = al[c] * Dp[(size_t)c * dv + j];
            }
            /* L2 norms */
            double pq = 0.0, pk = 0.0;
            for (int c = 0; c < dk; ++c) {
                pq += qh[c] * dqh[c];
                pk += kh[c] * dkh[c];
            }
            for (int c = 0; c < dk; ++c) {
                if (J->use_qk_l2norm) {
                    J->dq[rk + c] = (dqh[c] - qh[c] * pq) / NQ[i];
                    J->dk_[rk + c] = (dkh[c] - kh[c] * pk) / NK[i];
                } else {
                    J->dq[rk + c] = dqh[c];
                    J->dk_[rk + c] = dkh[c];
                }
            }
        }
    }
    if (J->dh0) memcpy(J->dh0 + ((size_t)n * H + h) * SZ, D, sizeof(double) * SZ);
done:
    free(ck); free(Sprev); free(Spv); free(Snew); free(D); free(Dp); free(QH); free(KH);
    free(AL); free(PP); free(UU); free(NQ); free(NK); free(dqh); free(dkh); free(du);
    return st;
}

static void *bwd_worker(void *arg)
{
    bwd_job_t *J = (bwd_job_t *)arg;
    const int nchains = J->num_seqs * J->H;
    for (int i = J->tid; i < nchains; i += J->nthreads) {
        int st = run_chain_backward(J, i / J->H, i % J->H);
        if (st != KDA_ORACLE_OK) J->status = st;
    }
    return NULL;
}

/* Gradients of sum(do * o) + sum(dht * ht) of the varlen token recurrence with respect to
 * q, k, v, g, beta and h0.  h0 and dht may be NULL (zero); dh0 may be NULL.  Layouts as the
 * forward; do [T_total, H, dv]; dq, dk, dg [T_total, H, dk]; dv [T_total, H, dv]; dbeta
 * [T_total, H]; dh0 [num_seqs, H, dk, dv].  Returns 0 on success. */
int kda_oracle_backward(const double *q, const double *k, const double *v, const double *g,
                        const double *beta, const int64_t *cu_seqlens, int num_seqs, int H,
                        int dk, int dv, double scale, int use_qk_l2norm, double eps,
                        const double *h0, const double *dout, const double *dht, double *dq,
                        double *dk_, double *dv_, double *dg, double *dbeta, double *dh0,
                        int nthreads)
{
    int st = check_common(q, k, v, g, beta, cu_seqlens, num_seqs, H, dk, dv, dout);
    if (st) return st;
    if (!dq || !dk_ || !dv_ || !dg || !dbeta) return KDA_ORACLE_EINVAL;
    bwd_job_t proto = {q, k, v, g, beta, h0, dout, dht, cu_seqlens, num_seqs, H, dk, dv,
                       use_qk_l2norm, scale, eps, dq, dk_, dv_, dg, dbeta, dh0, 0, 0, 0};
    int nt = nthreads < 1 ? 1 : nthreads;
    const int nchains = num_seqs * H;
    if (nt > nchains) nt = nchains > 0 ? nchains : 1;
    bwd_job_t *jobs = (bwd_job_t *)calloc((size_t)nt, sizeof(bwd_job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs); free(th);
        return KDA_ORACLE_ENOMEM;
    }
    for (int i = 0; i < nt; ++i) {
        jobs[i] = proto;
        jobs[i].nthreads = nt;
        jobs[i].tid = i;
    }
    for (int i = 1; i < nt; ++i)
        if (pthread_create(&th[i], NULL, bwd_worker, &jobs[i]) != 0) {
            bwd_worker(&jobs[i]);
            th[i] = 0;
        }
    bwd_worker(&jobs[0]);
    for (int i = 1; i < nt; ++i)
        if (th[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < nt; ++i)
        if (jobs[i].status != KDA_ORACLE_OK) st = jobs[i].status;
    free(jobs); free(th);
    return st;
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
