/*
 * mhla_oracle.c -- plain CPU reference of the MHLA forward pass, in float64.
 *
 * TEST INFRASTRUCTURE ONLY (see mhla_oracle.h).  Deliberately simple: scalar
 * loops, float64 accumulation in ascending token / block order; the forward
 * runs its blocks and (b, h) pairs on worker threads, each element summed in
 * the same order whatever the thread count.  No blocking, fusion or reordering beyond the
 * method's own blockwise reorganisation (paperlayer.ai summary of
 * arXiv 2601.07832, section 4 "Efficiency": summaries are formed once per
 * block and mixtures once per query block, then reused by every query).
 */
#define _POSIX_C_SOURCE 200809L
#include "mhla_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---- geometry (section 4 "Architecture": M non-overlapping token blocks on
 * a spatial / spatio-temporal grid; blocks and tokens both row-major) ---- */

typedef struct {
    int64_t N, M, T;     /* tokens, blocks, tokens per block */
    int32_t g[3], b[3], nb[3];  /* padded to 3 axes, slowest first */
} geom;

static int make_geom(const mhla_oracle_problem* p, geom* G) {
    if (!p || (p->ndim != 2 && p->ndim != 3)) return -1;
    if (p->batch < 0 || p->heads < 0 || p->head_dim <= 0) return -1;
    if (p->dtype != MHLA_ORACLE_F32 && p->dtype != MHLA_ORACLE_BF16) return -1;
    if (!(p->eps >= 0.0)) return -1;
    int off = 3 - p->ndim;
    for (int a = 0; a < 3; ++a) { G->g[a] = 1; G->b[a] = 1; }
    for (int a = 0; a < p->ndim; ++a) {
        if (p->grid[a] <= 0 || p->block[a] <= 0) return -1;
        if (p->grid[a] % p->block[a] != 0) return -1;
        G->g[off + a] = p->grid[a];
        G->b[off + a] = p->block[a];
    }
    G->N = 1; G->M = 1; G->T = 1;
    for (int a = 0; a < 3; ++a) {
        G->nb[a] = G->g[a] / G->b[a];
        G->N *= G->g[a];
        G->M *= G->nb[a];
        G->T *= G->b[a];
    }
    return 0;
}

/* Block id of raster token n: its per-axis coordinate divided by the block
 * extent gives the block coordinate; block ids are row-major over those. */
static int64_t block_of(const geom* G, int64_t n) {
    int64_t x2 = n % G->g[2];
    int64_t x1 = (n / G->g[2]) % G->g[1];
    int64_t x0 = n / ((int64_t)G->g[2] * G->g[1]);
    int64_t c0 = x0 / G->b[0], c1 = x1 / G->b[1], c2 = x2 / G->b[2];
    return (c0 * G->nb[1] + c1) * G->nb[2] + c2;
}

/* ---- element decoding and feature map ---- */

static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == MHLA_ORACLE_F32) {
        float f;
        memcpy(&f, (const char*)base + 4 * idx, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char*)base + 2 * idx, 2);
    uint32_t u = (uint32_t)h << 16;   /* bfloat16 is the top half of a float32 */
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* phi(x) = elu(x) + 1 (alpha = 1): x + 1 for x > 0, exp(x) otherwise.
 * Strictly positive, so every kernel weight phi(q).phi(k) is positive. */
double mhla_oracle_phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

int64_t mhla_oracle_num_blocks(const mhla_oracle_problem* p) {
    geom G;
    if (make_geom(p, &G) != 0) return -1;
    return G.M;
}

int mhla_oracle_token_blocks(const mhla_oracle_problem* p, int32_t* out) {
    geom G;
    if (make_geom(p, &G) != 0 || !out) return -1;
    for (int64_t n = 0; n < G.N; ++n) out[n] = (int32_t)block_of(&G, n);
    return 0;
}

/* ---- the blockwise form in three phases over (pair, block) units ----
 *
 * Pairs are taken in batches; within a batch every thread takes units
 * u = tid, tid + threads, ... of each phase, with a barrier between phases:
 *   phase 1, unit (s, j): S_j, z_j of pair s from block j's tokens, in
 *            ascending raster order;
 *   phase 2, unit (s, i): St_i, zt_i = sum_j W[i,j] S_j (z likewise), j ascending;
 *   phase 3, unit (s, i): outputs of the tokens of block i.
 * Every element is summed in the same order whatever the thread count. */

typedef struct {
    const void *q, *k, *v;
    const float* W;
    const mhla_oracle_problem* p;
    const geom* G;
    const int64_t* tok;     /* block j's tokens, ascending: tok[j*T .. j*T + T) */
    const int32_t* sel;     /* selected pairs (NULL: all, in order) */
    int32_t nsel, PB;       /* selected pairs, pairs per batch */
    double *out, *S_out, *z_out, *St_out, *zt_out;   /* caller's outputs (each may be NULL) */
    double *S, *z, *St, *zt;                         /* batch scratch, [PB][M][...] */
    int32_t nthreads;
    pthread_barrier_t* bar;
} fwd_shared;

typedef struct {
    const fwd_shared* F;
    int32_t tid;
} fwd_arg;

/* Local key-value summary of block j (repost section 5 item (2)):
 * S_j = sum phi(k_m) v_m^T and z_j = sum phi(k_m) over the block's tokens. */
static void summary_unit(const fwd_shared* F, int64_t base, int64_t j, double* S, double* z,
                         double* fk, double* vv) {
    const int64_t d = F->p->head_dim, row = (int64_t)F->p->heads * d, T = F->G->T;
    const int dt = F->p->dtype;
    double* Sj = S + j * d * d;
    double* zj = z + j * d;
    memset(Sj, 0, (size_t)(d * d) * sizeof(double));
    memset(zj, 0, (size_t)d * sizeof(double));
    for (int64_t r = 0; r < T; ++r) {
        const int64_t m = F->tok[j * T + r];
        for (int64_t c = 0; c < d; ++c) fk[c] = mhla_oracle_phi(load_elem(F->k, dt, base + m * row + c));
        for (int64_t e = 0; e < d; ++e) vv[e] = load_elem(F->v, dt, base + m * row + e);
        for (int64_t c = 0; c < d; ++c) {
            zj[c] += fk[c];
            for (int64_t e = 0; e < d; ++e) Sj[c * d + e] += fk[c] * vv[e];
        }
    }
}

/* Multi-head mixing (section 4 "Multi-Head Mixing"): query block i takes the
 * combination of all local summaries given by row i of W. */
static void mix_unit(const fwd_shared* F, int64_t i, const double* S, const double* z, double* St, double* zt) {
    const int64_t d = F->p->head_dim, M = F->G->M;
    double* Sti = St + i * d * d;
    double* zti = zt + i * d;
    memset(Sti, 0, (size_t)(d * d) * sizeof(double));
    memset(zti, 0, (size_t)d * sizeof(double));
    for (int64_t j = 0; j < M; ++j) {
        const double w = (double)F->W[i * M + j];
        for (int64_t t = 0; t < d * d; ++t) Sti[t] += w * S[j * d * d + t];
        for (int64_t c = 0; c < d; ++c) zti[c] += w * z[j * d + c];
    }
}

/* Every query of block i reads its block's mixed summary:
 * o_n = phi(q_n)^T St_i / (phi(q_n) . zt_i + eps). */
static void apply_unit(const fwd_shared* F, int64_t base, int64_t i, const double* St, const double* zt,
                       double* out, double* fq) {
    const int64_t d = F->p->head_dim, row = (int64_t)F->p->heads * d, T = F->G->T;
    const int dt = F->p->dtype;
    const double* Sti = St + i * d * d;
    const double* zti = zt + i * d;
    for (int64_t r = 0; r < T; ++r) {
        const int64_t n = F->tok[i * T + r];
        for (int64_t c = 0; c < d; ++c) fq[c] = mhla_oracle_phi(load_elem(F->q, dt, base + n * row + c));
        double den = 0.0;
        for (int64_t c = 0; c < d; ++c) den += fq[c] * zti[c];
        den += F->p->eps;
        for (int64_t e = 0; e < d; ++e) {
            double num = 0.0;
            for (int64_t c = 0; c < d; ++c) num += fq[c] * Sti[c * d + e];
            out[n * d + e] = num / den;
        }
    }
}

static void* fwd_worker(void* arg) {
    const fwd_arg* A = (const fwd_arg*)arg;
    const fwd_shared* F = A->F;
    const int64_t H = F->p->heads, d = F->p->head_dim, N = F->G->N, M = F->G->M;
    const int64_t rec = M * d * d, zrec = M * d;
    double* fk = malloc((size_t)d * sizeof(double));
    double* vv = malloc((size_t)d * sizeof(double));
    if (!fk || !vv) abort();
    for (int32_t s0 = 0; s0 < F->nsel; s0 += F->PB) {
        const int64_t npb = F->nsel - s0 < F->PB ? F->nsel - s0 : F->PB;
        const int64_t units = npb * M;
        for (int64_t u = A->tid; u < units; u += F->nthreads) {
            const int64_t sb = u / M, j = u % M, s = s0 + sb;
            const int64_t pair = F->sel ? F->sel[s] : s;
            const int64_t base = (pair / H) * N * H * d + (pair % H) * d;
            summary_unit(F, base, j, F->S + sb * rec, F->z + sb * zrec, fk, vv);
        }
        pthread_barrier_wait(F->bar);
        for (int64_t u = A->tid; u < units; u += F->nthreads) {
            const int64_t sb = u / M, i = u % M;
            mix_unit(F, i, F->S + sb * rec, F->z + sb * zrec, F->St + sb * rec, F->zt + sb * zrec);
        }
        pthread_barrier_wait(F->bar);
        for (int64_t u = A->tid; u < units; u += F->nthreads) {
            const int64_t sb = u / M, i = u % M, s = s0 + sb;
            const int64_t pair = F->sel ? F->sel[s] : s;
            const int64_t base = (pair / H) * N * H * d + (pair % H) * d;
            if (F->out) apply_unit(F, base, i, F->St + sb * rec, F->zt + sb * zrec, F->out + s * N * d, fk);
            if (F->S_out) memcpy(F->S_out + s * rec + i * d * d, F->S + sb * rec + i * d * d, (size_t)(d * d) * sizeof(double));
            if (F->z_out) memcpy(F->z_out + s * zrec + i * d, F->z + sb * zrec + i * d, (size_t)d * sizeof(double));
            if (F->St_out) memcpy(F->St_out + s * rec + i * d * d, F->St + sb * rec + i * d * d, (size_t)(d * d) * sizeof(double));
            if (F->zt_out) memcpy(F->zt_out + s * zrec + i * d, F->zt + sb * zrec + i * d, (size_t)d * sizeof(double));
        }
        pthread_barrier_wait(F->bar);   /* the batch scratch is reused by the next batch */
    }
    free(fk); free(vv);
    return NULL;
}

static int run_all(const void* q, const void* k, const void* v, const float* W,
                   const mhla_oracle_problem* p, const int32_t* sel, int32_t nsel,
                   double* out, double* S, double* z, double* St, double* zt,
                   int32_t threads, int32_t* threads_used) {
    geom G;
    if (make_geom(p, &G) != 0) return -1;
    int64_t pairs = (int64_t)p->batch * p->heads;
    if (!sel) nsel = (int32_t)pairs;
    if (nsel < 0) return -1;
    for (int32_t s = 0; sel && s < nsel; ++s)
        if (sel[s] < 0 || sel[s] >= pairs) return -1;
    if (nsel > 0 && (!k || !v || !W || (out && !q))) return -1;
    if (threads <= 0) threads = (int32_t)sysconf(_SC_NPROCESSORS_ONLN);
    if (threads < 1) threads = 1;
    /* Pairs per batch: enough (pair, block) units for every thread, at most all. */
    int64_t PB = (8 * (int64_t)threads + G.M - 1) / G.M;
    if (PB > nsel) PB = nsel > 0 ? nsel : 1;
    if (threads > PB * G.M) threads = (int32_t)(PB * G.M);
    if (threads_used) *threads_used = threads;
    if (nsel == 0) return 0;

    const int64_t d = p->head_dim, M = G.M, T = G.T;
    int64_t* tok = malloc((size_t)G.N * sizeof(int64_t));
    int64_t* fill = calloc((size_t)M, sizeof(int64_t));
    double* sS = malloc((size_t)(PB * M * d * d) * sizeof(double));
    double* sz = malloc((size_t)(PB * M * d) * sizeof(double));
    double* sSt = malloc((size_t)(PB * M * d * d) * sizeof(double));
    double* szt = malloc((size_t)(PB * M * d) * sizeof(double));
    pthread_t* tids = malloc(sizeof(pthread_t) * (size_t)threads);
    fwd_arg* args = malloc(sizeof(fwd_arg) * (size_t)threads);
    if (!tok || !fill || !sS || !sz || !sSt || !szt || !tids || !args) abort();
    /* Token lists: a scan in raster order leaves every block's list ascending. */
    for (int64_t n = 0; n < G.N; ++n) {
        const int64_t j = block_of(&G, n);
        tok[j * T + fill[j]++] = n;
    }
    pthread_barrier_t bar;
    pthread_barrier_init(&bar, NULL, (unsigned)threads);
    fwd_shared F = {q, k, v, W, p, &G, tok, sel, nsel, (int32_t)PB, out, S, z, St, zt,
                    sS, sz, sSt, szt, threads, &bar};
    for (int32_t t = 0; t < threads; ++t) {
        args[t].F = &F;
        args[t].tid = t;
    }
    for (int32_t t = 1; t < threads; ++t) pthread_create(&tids[t], NULL, fwd_worker, &args[t]);
    fwd_worker(&args[0]);
    for (int32_t t = 1; t < threads; ++t) pthread_join(tids[t], NULL);
    pthread_barrier_destroy(&bar);
    free(tok); free(fill); free(sS); free(sz); free(sSt); free(szt); free(tids); free(args);
    return 0;
}

int mhla_oracle_forward(const void* q, const void* k, const void* v, const float* W,
                        const mhla_oracle_problem* p, const int32_t* sel, int32_t nsel,
                        double* out, int32_t threads, int32_t* threads_used) {
    if (!out) return -1;
    return run_all(q, k, v, W, p, sel, nsel, out, NULL, NULL, NULL, NULL, threads, threads_used);
}

int mhla_oracle_summaries(const void* k, const void* v, const float* W,
                          const mhla_oracle_problem* p, const int32_t* sel, int32_t nsel,
                          double* S, double* z, double* St, double* zt, int32_t threads) {
    return run_all(NULL, k, v, W, p, sel, nsel, NULL, S, z, St, zt, threads, NULL);
}

/* =====================================================================
 * Backward pass (gradients of a scalar loss L with upstream gradient
 * g_n = dL/do_n).  The coefficient matrix W is a learned parameter of the
 * method (paperlayer.ai summary, section 4 "Multi-Head Mixing"), so the
 * gradient covers q, k, v and W.  Each step is the chain rule applied to the
 * forward definition above, in the forward's notation, u = phi(q), a = phi(k):
 *
 *   den_n = u_n . zt_i + eps,   o_n = St_i^T u_n / den_n
 *   dnum_n = g_n / den_n,       dden_n = -(g_n . o_n) / den_n
 *   du_n   = St_i dnum_n + zt_i dden_n,        dq_n = du_n * phi'(q_n)
 *   dSt_i  = sum_{n in i} u_n dnum_n^T,        dzt_i = sum_{n in i} u_n dden_n
 *   dS_j   = sum_i W[i,j] dSt_i,               dz_j  = sum_i W[i,j] dzt_i
 *   dW[i,j] = sum over (b, h) of <dSt_i, S_j> + <dzt_i, z_j>
 *   dv_m   = dS_j^T a_m,   da_m = dS_j v_m + dz_j,   dk_m = da_m * phi'(k_m)
 *
 * with phi'(x) = 1 for x > 0 and exp(x) otherwise.
 * ===================================================================== */

static double phi_grad(double x) { return x > 0.0 ? 1.0 : exp(x); }

typedef struct {
    const void *q, *k, *v, *dout;
    const float* W;
    const mhla_oracle_problem* p;
    const geom* G;
    double *dq, *dk, *dv;   /* [B][N][H][d] */
    double* dWp;            /* this pair's share of dW, [M][M] */
} bwd_job;

static void run_pair_backward(const bwd_job* J, int32_t b, int32_t h) {
    const geom* G = J->G;
    const int64_t H = J->p->heads, d = J->p->head_dim, N = G->N, M = G->M;
    const int dt = J->p->dtype;
    const int64_t row = H * d;
    const int64_t base = (int64_t)b * N * row + (int64_t)h * d;

    double* S = calloc((size_t)(M * d * d), sizeof(double));
    double* z = calloc((size_t)(M * d), sizeof(double));
    double* St = calloc((size_t)(M * d * d), sizeof(double));
    double* zt = calloc((size_t)(M * d), sizeof(double));
    double* dSt = calloc((size_t)(M * d * d), sizeof(double));
    double* dzt = calloc((size_t)(M * d), sizeof(double));
    double* dS = calloc((size_t)(M * d * d), sizeof(double));
    double* dz = calloc((size_t)(M * d), sizeof(double));
    double* x = malloc((size_t)d * sizeof(double));    /* raw q or k of one token */
    double* u = malloc((size_t)d * sizeof(double));    /* phi of it */
    double* y = malloc((size_t)d * sizeof(double));    /* v or g of one token */
    double* t1 = malloc((size_t)d * sizeof(double));
    if (!S || !z || !St || !zt || !dSt || !dzt || !dS || !dz || !x || !u || !y || !t1) abort();

    /* Forward summaries and their mixture, as in the forward pass. */
    for (int64_t m = 0; m < N; ++m) {
        int64_t j = block_of(G, m);
        for (int64_t c = 0; c < d; ++c) u[c] = mhla_oracle_phi(load_elem(J->k, dt, base + m * row + c));
        for (int64_t e = 0; e < d; ++e) y[e] = load_elem(J->v, dt, base + m * row + e);
        for (int64_t c = 0; c < d; ++c) {
            z[j * d + c] += u[c];
            for (int64_t e = 0; e < d; ++e) S[j * d * d + c * d + e] += u[c] * y[e];
        }
    }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < M; ++j) {
            double w = (double)J->W[i * M + j];
            for (int64_t t = 0; t < d * d; ++t) St[i * d * d + t] += w * S[j * d * d + t];
            for (int64_t c = 0; c < d; ++c) zt[i * d + c] += w * z[j * d + c];
        }

    /* Query side: gradient of q, and the gradients of the mixed summaries. */
    for (int64_t n = 0; n < N; ++n) {
        int64_t i = block_of(G, n);
        const double* Sti = St + i * d * d;
        const double* zti = zt + i * d;
        for (int64_t c = 0; c < d; ++c) {
            x[c] = load_elem(J->q, dt, base + n * row + c);
            u[c] = mhla_oracle_phi(x[c]);
        }
        for (int64_t e = 0; e < d; ++e) y[e] = load_elem(J->dout, dt, base + n * row + e);
        double den = J->p->eps;
        for (int64_t c = 0; c < d; ++c) den += u[c] * zti[c];
        double go = 0.0;   /* g . o */
        for (int64_t e = 0; e < d; ++e) {
            double num = 0.0;
            for (int64_t c = 0; c < d; ++c) num += u[c] * Sti[c * d + e];
            go += y[e] * (num / den);
        }
        const double dden = -go / den;
        for (int64_t e = 0; e < d; ++e) t1[e] = y[e] / den;   /* dnum */
        for (int64_t c = 0; c < d; ++c) {
            double du = zti[c] * dden;
            for (int64_t e = 0; e < d; ++e) du += Sti[c * d + e] * t1[e];
            J->dq[base + n * row + c] = du * phi_grad(x[c]);
            dzt[i * d + c] += u[c] * dden;
            for (int64_t e = 0; e < d; ++e) dSt[i * d * d + c * d + e] += u[c] * t1[e];
        }
    }

    /* Mixing, transposed: every source block collects the gradients of the
     * query blocks that read it; dW pairs each query block's gradient with
     * each source block's summary. */
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < M; ++j) {
            double w = (double)J->W[i * M + j];
            double acc = 0.0;
            for (int64_t t = 0; t < d * d; ++t) {
                dS[j * d * d + t] += w * dSt[i * d * d + t];
                acc += dSt[i * d * d + t] * S[j * d * d + t];
            }
            for (int64_t c = 0; c < d; ++c) {
                dz[j * d + c] += w * dzt[i * d + c];
                acc += dzt[i * d + c] * z[j * d + c];
            }
            J->dWp[i * M + j] = acc;
        }

    /* Key / value side. */
    for (int64_t m = 0; m < N; ++m) {
        int64_t j = block_of(G, m);
        const double* dSj = dS + j * d * d;
        for (int64_t c = 0; c < d; ++c) {
            x[c] = load_elem(J->k, dt, base + m * row + c);
            u[c] = mhla_oracle_phi(x[c]);
        }
        for (int64_t e = 0; e < d; ++e) y[e] = load_elem(J->v, dt, base + m * row + e);
        for (int64_t e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c) acc += u[c] * dSj[c * d + e];
            J->dv[base + m * row + e] = acc;
        }
        for (int64_t c = 0; c < d; ++c) {
            double acc = dz[j * d + c];
            for (int64_t e = 0; e < d; ++e) acc += dSj[c * d + e] * y[e];
            J->dk[base + m * row + c] = acc * phi_grad(x[c]);
        }
    }
    free(S); free(z); free(St); free(zt); free(dSt); free(dzt); free(dS); free(dz);
    free(x); free(u); free(y); free(t1);
}

typedef struct {
    bwd_job proto;
    double* dWparts;   /* [B*H][M][M] */
    int32_t pairs, nthreads, tid;
} bwd_worker_arg;

static void* bwd_worker(void* arg) {
    const bwd_worker_arg* A = (const bwd_worker_arg*)arg;
    const int64_t M = A->proto.G->M, H = A->proto.p->heads;
    for (int32_t s = A->tid; s < A->pairs; s += A->nthreads) {
        bwd_job J = A->proto;
        J.dWp = A->dWparts + (int64_t)s * M * M;
        run_pair_backward(&J, (int32_t)(s / H), (int32_t)(s % H));
    }
    return NULL;
}

int mhla_oracle_backward(const void* q, const void* k, const void* v, const float* W, const void* dout,
                         const mhla_oracle_problem* p, double* dq, double* dk, double* dv, double* dW,
                         int32_t threads, int32_t* threads_used) {
    geom G;
    if (make_geom(p, &G) != 0) return -1;
    const int64_t pairs = (int64_t)p->batch * p->heads, M = G.M;
    if (pairs > 0 && (!q || !k || !v || !W || !dout || !dq || !dk || !dv)) return -1;
    if (!dW) return -1;
    if (threads <= 0) threads = (int32_t)sysconf(_SC_NPROCESSORS_ONLN);
    if (threads < 1) threads = 1;
    if (threads > pairs) threads = pairs > 0 ? (int32_t)pairs : 1;
    if (threads_used) *threads_used = threads;
    for (int64_t t = 0; t < M * M; ++t) dW[t] = 0.0;
    if (pairs == 0) return 0;
    double* parts = malloc((size_t)(pairs * M * M) * sizeof(double));
    pthread_t* tids = malloc(sizeof(pthread_t) * (size_t)threads);
    bwd_worker_arg* args = malloc(sizeof(bwd_worker_arg) * (size_t)threads);
    if (!parts || !tids || !args) abort();
    for (int32_t t = 0; t < threads; ++t) {
        bwd_worker_arg a = {{q, k, v, dout, W, p, &G, dq, dk, dv, NULL}, parts, (int32_t)pairs, threads, t};
        args[t] = a;
    }
    for (int32_t t = 1; t < threads; ++t) pthread_create(&tids[t], NULL, bwd_worker, &args[t]);
    bwd_worker(&args[0]);
    for (int32_t t = 1; t < threads; ++t) pthread_join(tids[t], NULL);
    /* Sum the pairs' shares in pair order, so the result does not depend on
     * the thread count. */
    for (int64_t s = 0; s < pairs; ++s)
        for (int64_t t = 0; t < M * M; ++t) dW[t] += parts[s * M * M + t];
    free(parts); free(tids); free(args);
    return 0;
}

/* =====================================================================
 * Causal chunkwise form (paperlayer.ai summary, appendix B "Causal MHLA":
 * block-specific mixtures reused per block, causality preserved).  The
 * attention matrix is the MHLA matrix restricted to m <= n in raster order:
 *   A[n, m] = W[b(n), b(m)] phi(q_n) . phi(k_m)   for m <= n, else 0,
 *   o_n = sum_m A[n, m] v_m / (sum_m A[n, m] + eps).
 * For chunks that are contiguous in raster order this is, for query n in
 * chunk i: the mixture of the earlier chunks' summaries, sum_{j < i} W[i,j] S_j
 * (and z likewise), plus W[i,i] times the running summary of chunk i's own
 * tokens up to n.
 * ===================================================================== */

typedef struct {
    const void *q, *k, *v;
    const float* W;
    const mhla_oracle_problem* p;
    const geom* G;
    double* out;   /* this pair's [N][d] */
} causal_job;

static void run_pair_causal(const causal_job* J, int32_t b, int32_t h) {
    const geom* G = J->G;
    const int64_t H = J->p->heads, d = J->p->head_dim, N = G->N, M = G->M;
    const int dt = J->p->dtype;
    const int64_t row = H * d;
    const int64_t base = (int64_t)b * N * row + (int64_t)h * d;
    double* S = calloc((size_t)(M * d * d), sizeof(double));
    double* z = calloc((size_t)(M * d), sizeof(double));
    double* St = malloc((size_t)(d * d) * sizeof(double));   /* earlier chunks' mixture + own prefix */
    double* zt = malloc((size_t)d * sizeof(double));
    double* P = malloc((size_t)(d * d) * sizeof(double));    /* running summary of the own chunk */
    double* zP = malloc((size_t)d * sizeof(double));
    double* fk = malloc((size_t)d * sizeof(double));
    double* vv = malloc((size_t)d * sizeof(double));
    if (!S || !z || !St || !zt || !P || !zP || !fk || !vv) abort();
    for (int64_t m = 0; m < N; ++m) {
        int64_t j = block_of(G, m);
        for (int64_t c = 0; c < d; ++c) fk[c] = mhla_oracle_phi(load_elem(J->k, dt, base + m * row + c));
        for (int64_t e = 0; e < d; ++e) vv[e] = load_elem(J->v, dt, base + m * row + e);
        for (int64_t c = 0; c < d; ++c) {
            z[j * d + c] += fk[c];
            for (int64_t e = 0; e < d; ++e) S[j * d * d + c * d + e] += fk[c] * vv[e];
        }
    }
    /* Tokens in raster order; chunks are contiguous, so a chunk starts when
     * the block id changes. */
    int64_t cur = -1;
    double wii = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const int64_t i = block_of(G, n);
        if (i != cur) {
            cur = i;
            memset(P, 0, (size_t)(d * d) * sizeof(double));
            memset(zP, 0, (size_t)d * sizeof(double));
            memset(St, 0, (size_t)(d * d) * sizeof(double));
            memset(zt, 0, (size_t)d * sizeof(double));
            for (int64_t j = 0; j < i; ++j) {
                const double w = (double)J->W[i * M + j];
                for (int64_t t = 0; t < d * d; ++t) St[t] += w * S[j * d * d + t];
                for (int64_t c = 0; c < d; ++c) zt[c] += w * z[j * d + c];
            }
            wii = (double)J->W[i * M + i];
        }
        /* the own chunk's prefix grows by token n before n reads it (m <= n) */
        for (int64_t c = 0; c < d; ++c) fk[c] = mhla_oracle_phi(load_elem(J->k, dt, base + n * row + c));
        for (int64_t e = 0; e < d; ++e) vv[e] = load_elem(J->v, dt, base + n * row + e);
        for (int64_t c = 0; c < d; ++c) {
            zP[c] += fk[c];
            for (int64_t e = 0; e < d; ++e) P[c * d + e] += fk[c] * vv[e];
        }
        double* fq = fk;
        for (int64_t c = 0; c < d; ++c) fq[c] = mhla_oracle_phi(load_elem(J->q, dt, base + n * row + c));
        double den = J->p->eps;
        for (int64_t c = 0; c < d; ++c) den += fq[c] * (zt[c] + wii * zP[c]);
        for (int64_t e = 0; e < d; ++e) {
            double num = 0.0;
            for (int64_t c = 0; c < d; ++c) num += fq[c] * (St[c * d + e] + wii * P[c * d + e]);
            J->out[n * d + e] = num / den;
        }
    }
    free(S); free(z); free(St); free(zt); free(P); free(zP); free(fk); free(vv);
}

typedef struct {
    causal_job proto;
    const int32_t* sel;
    int32_t nsel, nthreads, tid;
} causal_worker_arg;

static void* causal_worker(void* arg) {
    const causal_worker_arg* A = (const causal_worker_arg*)arg;
    const int64_t N = A->proto.G->N, d = A->proto.p->head_dim, H = A->proto.p->heads;
    for (int32_t s = A->tid; s < A->nsel; s += A->nthreads) {
        const int32_t pair = A->sel ? A->sel[s] : s;
        causal_job J = A->proto;
        J.out = A->proto.out + (int64_t)s * N * d;
        run_pair_causal(&J, (int32_t)(pair / H), (int32_t)(pair % H));
    }
    return NULL;
}

int mhla_oracle_chunks_contiguous(const mhla_oracle_problem* p) {
    geom G;
    if (make_geom(p, &G) != 0) return -1;
    /* A block is one run of raster indices iff some axis a splits it while every
     * faster axis is covered whole and every slower axis has extent 1. */
    for (int a = 0; a < p->ndim; ++a) {
        int ok = 1;
        for (int x = 0; x < a; ++x) ok &= p->block[x] == 1;
        for (int x = a + 1; x < p->ndim; ++x) ok &= p->block[x] == p->grid[x];
        if (ok) return 1;
    }
    return 0;
}

int mhla_oracle_forward_causal(const void* q, const void* k, const void* v, const float* W,
                               const mhla_oracle_problem* p, const int32_t* sel, int32_t nsel, double* out,
                               int32_t threads) {
    geom G;
    if (make_geom(p, &G) != 0 || !out) return -1;
    if (mhla_oracle_chunks_contiguous(p) != 1) return -1;
    const int64_t pairs = (int64_t)p->batch * p->heads;
    if (!sel) nsel = (int32_t)pairs;
    if (nsel < 0) return -1;
    for (int32_t s = 0; sel && s < nsel; ++s)
        if (sel[s] < 0 || sel[s] >= pairs) return -1;
    if (nsel > 0 && (!q || !k || !v || !W)) return -1;
    if (threads <= 0) threads = (int32_t)sysconf(_SC_NPROCESSORS_ONLN);
    if (threads < 1) threads = 1;
    if (threads > nsel) threads = nsel > 0 ? nsel : 1;
    if (nsel == 0) return 0;
    pthread_t* tids = malloc(sizeof(pthread_t) * (size_t)threads);
    causal_worker_arg* args = malloc(sizeof(causal_worker_arg) * (size_t)threads);
    if (!tids || !args) abort();
    for (int32_t t = 0; t < threads; ++t) {
        causal_worker_arg a = {{q, k, v, W, p, &G, out}, sel, nsel, threads, t};
        args[t] = a;
    }
    for (int32_t t = 1; t < threads; ++t) pthread_create(&tids[t], NULL, causal_worker, &args[t]);
    causal_worker(&args[0]);
    for (int32_t t = 1; t < threads; ++t) pthread_join(tids[t], NULL);
    free(tids); free(args);
    return 0;
}
