/*
 * mhla_oracle.h -- plain CPU reference of the MHLA forward pass, in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this; only the test suite, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code with the HIP library.
 *
 * What it computes (MHLA: "Restoring Expressivity of Linear Attention via
 * Token-Level Multi-Head", arXiv 2601.07832; paperlayer.ai summary, section 4
 * "Architecture", "Multi-Head Mixing", "Efficiency"; 171host.com repost,
 * section 5 items (1)-(3)):
 *
 *   tokens on a 2D/3D grid are split into M non-overlapping blocks;
 *   per block j:  S_j = sum_{m in j} phi(k_m) v_m^T   (d x d)
 *                 z_j = sum_{m in j} phi(k_m)          (d)
 *   per query block i:  St_i = sum_j W[i,j] S_j,  zt_i = sum_j W[i,j] z_j
 *   per query token n in block i:
 *                 o_n = phi(q_n)^T St_i / (phi(q_n) . zt_i + eps)
 *   with phi(x) = elu(x) + 1 = (x > 0 ? x + 1 : exp(x)).
 *
 * Inputs q, k, v are [B, N, H, d] contiguous, N in raster order over the
 * grid (last axis fastest); elements are raw IEEE float32 or bfloat16 bit
 * patterns, decoded exactly.  W is float32 [M, M] row-major; blocks are
 * numbered row-major over the block grid.
 *
 * Return value of every function: 0 on success, -1 on an invalid problem.
 */
#ifndef MHLA_ORACLE_H
#define MHLA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MHLA_ORACLE_F32 = 0, MHLA_ORACLE_BF16 = 1 };

typedef struct mhla_oracle_problem {
    int32_t batch, heads, head_dim;
    int32_t dtype;      /* MHLA_ORACLE_F32 or MHLA_ORACLE_BF16 */
    int32_t ndim;       /* 2 or 3 */
    int32_t grid[3];    /* token-grid extents, slowest axis first; first ndim used */
    int32_t block[3];   /* block extents in tokens, same order */
    double eps;
} mhla_oracle_problem;

/* phi(x) = elu(x) + 1, exported so tests can pin it. */
double mhla_oracle_phi(double x);

/* Number of blocks M, or -1 if the problem is invalid (bad rank, extents,
 * or a grid extent not divisible by the block extent). */
int64_t mhla_oracle_num_blocks(const mhla_oracle_problem* p);

/* Block id of every token n in [0, N): out[n]. */
int mhla_oracle_token_blocks(const mhla_oracle_problem* p, int32_t* out);

/* Full forward for the selected (b, h) pairs.
 * sel: nsel indices s = b*H + h (NULL: all B*H pairs in order).
 * out: [nsel][N][d] float64.  threads <= 0: one per online CPU.
 * threads_used (may be NULL) receives the number of worker threads run. */
int mhla_oracle_forward(const void* q, const void* k, const void* v, const float* W,
                        const mhla_oracle_problem* p, const int32_t* sel, int32_t nsel,
                        double* out, int32_t threads, int32_t* threads_used);

/* Intermediates for the selected pairs: S [nsel][M][d][d] (index [c][e]),
 * z [nsel][M][d], St [nsel][M][d][d], zt [nsel][M][d].  Any output may be NULL. */
int mhla_oracle_summaries(const void* k, const void* v, const float* W,
                          const mhla_oracle_problem* p, const int32_t* sel, int32_t nsel,
                          double* S, double* z, double* St, double* zt, int32_t threads);

/* Gradients of a scalar loss with upstream gradient dout = dL/dout ([B, N,
 * H, d], same dtype and layout as q): dq, dk, dv [B, N, H, d] float64 and
 * dW [M, M] float64 (summed over every (b, h) pair in pair order).  Chain rule
 * on the forward above; W is a learned parameter of the method (section 4
 * "Multi-Head Mixing"). */
int mhla_oracle_backward(const void* q, const void* k, const void* v, const float* W, const void* dout,
                         const mhla_oracle_problem* p, double* dq, double* dk, double* dv, double* dW,
                         int32_t threads, int32_t* threads_used);

/* 1 if every block is one contiguous run of raster indices (some axis is
 * split while all faster axes are covered whole and all slower axes have
 * block extent 1), 0 if not, -1 for an invalid problem. */
int mhla_oracle_chunks_contiguous(const mhla_oracle_problem* p);

/* Causal chunkwise forward (appendix B "Causal MHLA"): the attention matrix
 * above restricted to m <= n in raster order.  Needs contiguous chunks.
 * Same selection and output conventions as mhla_oracle_forward. */
int mhla_oracle_forward_causal(const void* q, const void* k, const void* v, const float* W,
                               const mhla_oracle_problem* p, const int32_t* sel, int32_t nsel, double* out,
                               int32_t threads);

#ifdef __cplusplus
}
#endif
#endif
