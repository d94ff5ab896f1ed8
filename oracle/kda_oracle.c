/*
 * kda_oracle.c -- plain fp64 token-by-token KDA recurrence (CPU).
 *
 * TEST INFRASTRUCTURE ONLY (see kda_oracle.h).  Deliberately slow and
 * obvious: no chunking, no blocking, no reordering.  Each (sequence, head)
 * pair is independent; pairs are spread over POSIX threads.
 *
 * Per token t of sequence n, head h (the update rule of
 * "Kimi Linear：让长上下文大模型真正实用的线性注意力架构", section 三.5):
 *
 *   1. S <- Diag(alpha_t) S,   alpha_t[i] = exp(log_alpha[t,h,i])
 *        the per-channel forgetting gate (section 三.1) scales key rows.
 *   2. u = S^T k_t             what the memory currently returns for key k_t.
 *   3. e = beta_t (v_t - u)    one gradient step of size beta_t on
 *        1/2 || S^T k_t - v_t ||^2 (section 三.5 reads the update as online
 *        gradient descent with learning rate beta_t).
 *   4. S <- S + k_t e^T        equals (I - beta k k^T) Diag(alpha) S + beta k v^T.
 *   5. o_t = S^T q_t           read-out after the update.
 *
 * Sums run in ascending index order.
 */
#include "kda_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *q, *k, *v, *log_alpha, *beta;
    const double* S0;
    const int32_t* cu;
    int32_t N, H, dk, dv;
    const uint8_t* mask;
    double *o, *S_T;
    int32_t nthreads, tid;
    int status;
} job_t;

/* Runs the recurrence for one (sequence n, head h) pair. */
static int run_pair(const job_t* J, int32_t n, int32_t h) {
    const int32_t H = J->H, dk = J->dk, dv = J->dv;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!S || !u) {
        free(S);
        free(u);
        return -2;
    }
    const size_t sbase = ((size_t)n * H + h) * (size_t)dk * (size_t)dv;
    if (J->S0) {
        memcpy(S, J->S0 + sbase, sizeof(double) * (size_t)dk * (size_t)dv);
    } else {
        memset(S, 0, sizeof(double) * (size_t)dk * (size_t)dv);
    }
    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
        const size_t tk = ((size_t)t * H + h) * (size_t)dk;
        const size_t tv = ((size_t)t * H + h) * (size_t)dv;
        const float* qt = J->q + tk;
        const float* kt = J->k + tk;
        const float* vt = J->v + tv;
        const float* lat = J->log_alpha + tk;
        const double bt = (double)J->beta[(size_t)t * H + h];
        /* 1. decay: key row i of S is multiplied by alpha_t[i] */
        for (int32_t i = 0; i < dk; ++i) {
            const double a = exp((double)lat[i]);
            for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
        }
        /* 2. prediction u = S^T k_t */
        for (int32_t j = 0; j < dv; ++j) u[j] = 0.0;
        for (int32_t i = 0; i < dk; ++i) {
            const double ki = (double)kt[i];
            for (int32_t j = 0; j < dv; ++j) u[j] += ki * S[(size_t)i * dv + j];
        }
        /* 3. error scaled by the step size */
        for (int32_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - u[j]);
        /* 4. rank-1 correction k_t e^T */
        for (int32_t i = 0; i < dk; ++i) {
            const double ki = (double)kt[i];
            for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] += ki * u[j];
        }
        /* 5. read-out o_t = S^T q_t */
        double* ot = J->o + tv;
        for (int32_t j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int32_t i = 0; i < dk; ++i) {
            const double qi = (double)qt[i];
            for (int32_t j = 0; j < dv; ++j) ot[j] += qi * S[(size_t)i * dv + j];
        }
    }
    memcpy(J->S_T + sbase, S, sizeof(double) * (size_t)dk * (size_t)dv);
    free(S);
    free(u);
    return 0;
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int64_t npairs = (int64_t)J->N * J->H;
    for (int64_t p = J->tid; p < npairs; p += J->nthreads) {
        if (J->mask && !J->mask[p]) continue;
        const int rc = run_pair(J, (int32_t)(p / J->H), (int32_t)(p % J->H));
        if (rc) {
            J->status = rc;
            break;
        }
    }
    return NULL;
}

int kda_oracle_prefill(const float* q, const float* k, const float* v,
                       const float* log_alpha, const float* beta,
                       const double* S0, const int32_t* cu_seqlens,
                       int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                       const uint8_t* pair_mask, double* o, double* S_T, int32_t nthreads) {
    if (N < 1 || H < 1 || d_k < 1 || d_v < 1 || T_tot < 0) return -1;
    if (!cu_seqlens || !S_T || (T_tot > 0 && (!q || !k || !v || !log_alpha || !beta || !o)))
        return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T_tot) return -1;
    for (int32_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > (int64_t)N * H) nthreads = (int32_t)((int64_t)N * H);

    job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -2;
    }
    for (int32_t i = 0; i < nthreads; ++i) {
        job_t J = {q, k, v, log_alpha, beta, S0, cu_seqlens, N, H, d_k, d_v,
                   pair_mask, o, S_T, nthreads, i, 0};
        jobs[i] = J;
    }
    unsigned char* started = (unsigned char*)calloc((size_t)nthreads, 1);
    if (!started) {
        free(jobs);
        free(th);
        return -2;
    }
    for (int32_t i = 1; i < nthreads; ++i)
        started[i] = pthread_create(&th[i], NULL, worker, &jobs[i]) == 0;
    worker(&jobs[0]);
    int status = jobs[0].status;
    for (int32_t i = 1; i < nthreads; ++i) {
        if (started[i]) {
            pthread_join(th[i], NULL);
        } else {
            worker(&jobs[i]); /* could not start a thread: run its share here */
        }
        if (jobs[i].status) status = jobs[i].status;
    }
    free(started);
    free(jobs);
    free(th);
    return status;
}

int kda_oracle_decode_step(const float* q, const float* k, const float* v,
                           const float* log_alpha, const float* beta, double* S,
                           int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                           const uint8_t* pair_mask, double* o, int32_t nthreads) {
    if (N < 1 || !S) return -1;
    int32_t* cu = (int32_t*)malloc(sizeof(int32_t) * ((size_t)N + 1));
    if (!cu) return -2;
    for (int32_t n = 0; n <= N; ++n) cu[n] = n;
    /* one token per sequence; run_pair copies S0 before writing S_T, so the
     * state may be updated in place */
    const int rc = kda_oracle_prefill(q, k, v, log_alpha, beta, S, cu, N, (int64_t)N, H, d_k,
                                      d_v, pair_mask, o, S, nthreads);
    free(cu);
    return rc;
}

/* ------------------------------------------------------------------------
 * Backward pass: the gradient of a scalar loss L with respect to every input
 * of the recurrence above, given dL/do_t for every token and dL/dS_T for the
 * final states.  It is reverse-mode differentiation of steps 1-5, applied
 * token by token from the last token to the first, with G = dL/dS carried
 * backwards (G starts at dL/dS_T).  For token t, with S_p = S_{t-1},
 * a = alpha_t, S' = Diag(a) S_p, u = S'^T k, w = v - u, e = beta w and
 * S_t = S' + k e^T:
 *
 *   5. o_t = S_t^T q        dq = S_t do,           G += q do^T
 *   4. S_t = S' + k e^T     dk = G e,              de = G^T k,   dS' = G
 *   3. e = beta (v - u)     dv = beta de,          dbeta = de . w,  du = -beta de
 *   2. u = S'^T k           dk += S' du,           dS' += k du^T
 *   1. S' = Diag(a) S_p     da_i = sum_j dS'_ij S_p,ij,  dlog_alpha = a * da,
 *                           G <- Diag(a) dS'  (= dL/dS_{t-1})
 *
 * and dS0 = G after the first token.  The states S_{t-1} are recomputed by
 * the same forward steps from checkpoints taken every kBwdBlock tokens, so
 * they are bit-identical to those of the forward pass.
 * ------------------------------------------------------------------------ */
enum { kBwdBlock = 64 };

typedef struct {
    const float *q, *k, *v, *log_alpha, *beta;
    const double* S0;
    const int32_t* cu;
    int32_t N, H, dk, dv;
    const double *dO, *dST;
    const uint8_t* mask;
    double *dq, *dk_, *dv_, *dla, *dbeta, *dS0;
    int32_t nthreads, tid;
    int status;
} bjob_t;

/* steps 1-4 of the forward recurrence for token t: S_{t-1} -> S_t */
static void forward_token(const bjob_t* J, int64_t t, int32_t h, double* S, double* u) {
    const int32_t H = J->H, dk = J->dk, dv = J->dv;
    const size_t tk = ((size_t)t * H + h) * (size_t)dk;
    const size_t tv = ((size_t)t * H + h) * (size_t)dv;
    const double bt = (double)J->beta[(size_t)t * H + h];
    for (int32_t i = 0; i < dk; ++i) {
        const double a = exp((double)J->log_alpha[tk + i]);
        for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
    }
    for (int32_t j = 0; j < dv; ++j) u[j] = 0.0;
    for (int32_t i = 0; i < dk; ++i) {
        const double ki = (double)J->k[tk + i];
        for (int32_t j = 0; j < dv; ++j) u[j] += ki * S[(size_t)i * dv + j];
    }
    for (int32_t j = 0; j < dv; ++j) u[j] = bt * ((double)J->v[tv + j] - u[j]);
    for (int32_t i = 0; i < dk; ++i) {
        const double ki = (double)J->k[tk + i];
        for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] += ki * u[j];
    }
}

static int run_pair_bwd(const bjob_t* J, int32_t n, int32_t h) {
    const int32_t H = J->H, dk = J->dk, dv = J->dv;
    const size_t SS = (size_t)dk * (size_t)dv;
    const int64_t t0 = J->cu[n], t1 = J->cu[n + 1], len = t1 - t0;
    const int64_t nblk = (len + kBwdBlock - 1) / kBwdBlock;
    /* ckpt[b] = state entering block b; states[r] = S_{t-1} of row r of a block */
    double* ckpt = (double*)malloc(sizeof(double) * SS * (size_t)(nblk > 0 ? nblk : 1));
    double* states = (double*)malloc(sizeof(double) * SS * kBwdBlock);
    double* S = (double*)malloc(sizeof(double) * SS);
    double* G = (double*)malloc(sizeof(double) * SS);
    double* dSp = (double*)malloc(sizeof(double) * SS);
    double* vec = (double*)malloc(sizeof(double) * (size_t)(4 * dv + dk));
    if (!ckpt || !states || !S || !G || !dSp || !vec) {
        free(ckpt); free(states); free(S); free(G); free(dSp); free(vec);
        return -2;
    }
    double *u = vec, *w = vec + dv, *de = vec + 2 * dv, *du = vec + 3 * dv, *tmp = vec + 4 * dv;
    const size_t sbase = ((size_t)n * H + h) * SS;
    if (J->S0) memcpy(S, J->S0 + sbase, sizeof(double) * SS);
    else memset(S, 0, sizeof(double) * SS);
    for (int64_t b = 0; b < nblk; ++b) {
        memcpy(ckpt + (size_t)b * SS, S, sizeof(double) * SS);
        const int64_t te = t0 + (b + 1) * kBwdBlock < t1 ? t0 + (b + 1) * kBwdBlock : t1;
        for (int64_t t = t0 + b * kBwdBlock; t < te; ++t) forward_token(J, t, h, S, u);
    }
    if (J->dST) memcpy(G, J->dST + sbase, sizeof(double) * SS);
    else memset(G, 0, sizeof(double) * SS);
    for (int64_t b = nblk - 1; b >= 0; --b) {
        const int64_t tb = t0 + b * kBwdBlock;
        const int64_t te = tb + kBwdBlock < t1 ? tb + kBwdBlock : t1;
        memcpy(S, ckpt + (size_t)b * SS, sizeof(double) * SS);
        for (int64_t t = tb; t < te; ++t) {
            memcpy(states + (size_t)(t - tb) * SS, S, sizeof(double) * SS);
            forward_token(J, t, h, S, u);
        }
        for (int64_t t = te - 1; t >= tb; --t) {
            const double* Sp = states + (size_t)(t - tb) * SS;
            const size_t tk = ((size_t)t * H + h) * (size_t)dk;
            const size_t tv = ((size_t)t * H + h) * (size_t)dv;
            const float *qt = J->q + tk, *kt = J->k + tk, *vt = J->v + tv, *lat = J->log_alpha + tk;
            const double* dot = J->dO + tv;
            const double bt = (double)J->beta[(size_t)t * H + h];
            /* recompute S' (into S), u, w, e and S_t (into dSp) */
            for (int32_t i = 0; i < dk; ++i) {
                const double a = exp((double)lat[i]);
                for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] = a * Sp[(size_t)i * dv + j];
            }
            for (int32_t j = 0; j < dv; ++j) u[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j) u[j] += (double)kt[i] * S[(size_t)i * dv + j];
            for (int32_t j = 0; j < dv; ++j) w[j] = (double)vt[j] - u[j];
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j)
                    dSp[(size_t)i * dv + j] = S[(size_t)i * dv + j] + (double)kt[i] * (bt * w[j]);
            /* 5. read-out */
            for (int32_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += dSp[(size_t)i * dv + j] * dot[j];
                J->dq[tk + i] = acc;
            }
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j) G[(size_t)i * dv + j] += (double)qt[i] * dot[j];
            /* 4. rank-1 correction */
            for (int32_t j = 0; j < dv; ++j) de[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j) de[j] += G[(size_t)i * dv + j] * (double)kt[i];
            for (int32_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += G[(size_t)i * dv + j] * (bt * w[j]);
                tmp[i] = acc;
            }
            /* 3. error and step size */
            double db = 0.0;
            for (int32_t j = 0; j < dv; ++j) {
                J->dv_[tv + j] = bt * de[j];
                db += de[j] * w[j];
                du[j] = -bt * de[j];
            }
            J->dbeta[(size_t)t * H + h] = db;
            /* 2. prediction: dk += S' du, dS' = G + k du^T */
            for (int32_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += S[(size_t)i * dv + j] * du[j];
                J->dk_[tk + i] = tmp[i] + acc;
            }
            /* 1. decay */
            for (int32_t i = 0; i < dk; ++i) {
                const double a = exp((double)lat[i]);
                double da = 0.0;
                for (int32_t j = 0; j < dv; ++j) {
                    const double g = G[(size_t)i * dv + j] + (double)kt[i] * du[j];
                    da += g * Sp[(size_t)i * dv + j];
                    G[(size_t)i * dv + j] = a * g;
                }
                J->dla[tk + i] = a * da;
            }
        }
    }
    memcpy(J->dS0 + sbase, G, sizeof(double) * SS);
    free(ckpt); free(states); free(S); free(G); free(dSp); free(vec);
    return 0;
}

static void* bworker(void* arg) {
    bjob_t* J = (bjob_t*)arg;
    const int64_t npairs = (int64_t)J->N * J->H;
    for (int64_t p = J->tid; p < npairs; p += J->nthreads) {
        if (J->mask && !J->mask[p]) continue;
        const int rc = run_pair_bwd(J, (int32_t)(p / J->H), (int32_t)(p % J->H));
        if (rc) {
            J->status = rc;
            break;
        }
    }
    return NULL;
}

int kda_oracle_prefill_backward(const float* q, const float* k, const float* v,
                                const float* log_alpha, const float* beta,
                                const double* S0, const int32_t* cu_seqlens,
                                int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                                const double* dO, const double* dS_T, const uint8_t* pair_mask,
                                double* dq, double* dk, double* dv, double* dlog_alpha,
                                double* dbeta, double* dS0, int32_t nthreads) {
    if (N < 1 || H < 1 || d_k < 1 || d_v < 1 || T_tot < 0) return -1;
    if (!cu_seqlens || !dS0) return -1;
    if (T_tot > 0 && (!q || !k || !v || !log_alpha || !beta || !dO || !dq || !dk || !dv ||
                      !dlog_alpha || !dbeta))
        return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T_tot) return -1;
    for (int32_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > (int64_t)N * H) nthreads = (int32_t)((int64_t)N * H);
    bjob_t* jobs = (bjob_t*)calloc((size_t)nthreads, sizeof(bjob_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    unsigned char* started = (unsigned char*)calloc((size_t)nthreads, 1);
    if (!jobs || !th || !started) {
        free(jobs); free(th); free(started);
        return -2;
    }
    for (int32_t i = 0; i < nthreads; ++i) {
        bjob_t J = {q, k, v, log_alpha, beta, S0, cu_seqlens, N, H, d_k, d_v, dO, dS_T,
                    pair_mask, dq, dk, dv, dlog_alpha, dbeta, dS0, nthreads, i, 0};
        jobs[i] = J;
    }
    for (int32_t i = 1; i < nthreads; ++i)
        started[i] = pthread_create(&th[i], NULL, bworker, &jobs[i]) == 0;
    bworker(&jobs[0]);
    int status = jobs[0].status;
    for (int32_t i = 1; i < nthreads; ++i) {
        if (started[i]) pthread_join(th[i], NULL);
        else bworker(&jobs[i]);
        if (jobs[i].status) status = jobs[i].status;
    }
    free(started); free(jobs); free(th);
    return status;
}
