/*
 * mhla.h -- libmhla: the MHLA forward pass on AMD Instinct MI355X (gfx950).
 *
 * MHLA ("Restoring Expressivity of Linear Attention via Token-Level
 * Multi-Head", arXiv 2601.07832; paperlayer.ai summary, section 4
 * "Architecture", "Multi-Head Mixing", "Efficiency"; 171host.com repost,
 * section 5 items (1)-(3)) splits the tokens of a 2D or 3D grid into M
 * non-overlapping blocks and computes, for every (batch b, head h):
 *
 *   S_j  = sum_{m in block j} phi(k_m) v_m^T          (d x d)
 *   z_j  = sum_{m in block j} phi(k_m)                (d)
 *   St_i = sum_j W[i,j] S_j,   zt_i = sum_j W[i,j] z_j
 *   o_n  = phi(q_n)^T St_i / (phi(q_n) . zt_i + eps)   for token n in block i
 *
 * with phi(x) = elu(x) + 1 and one M x M coefficient matrix W shared by all
 * batches and heads.  The work runs as hand-written HIP kernels on the
 * caller's stream; every call is asynchronous.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - q, k, v, out: device pointers to contiguous [B, N, H, d] tensors of the
 *   grid's dtype (IEEE float32 or bfloat16), N = prod(grid extents) in raster
 *   order over the grid (last axis fastest), channel index h*d + c.
 * - W: device pointer to a contiguous row-major float32 [M, M] matrix;
 *   W[i*M + j] weights source block j for query block i.  Blocks are
 *   numbered row-major over the block grid (slowest axis first).
 * - All pointers are owned by the caller; the library never frees or keeps
 *   them past the call's enqueued work.  q, k, v, W and out must be 16-byte
 *   aligned, and out must not overlap q, k, v or W.
 * - bfloat16 path: products in bf16 MFMA with fp32 accumulation; phi is
 *   evaluated in fp32; summaries and mixed summaries are stored in bf16,
 *   normalisers in fp32; output rounded to nearest even.  float32 path: all
 *   arithmetic in fp32 (fp32 MFMA), intermediates in fp32.
 * - B = 0 or H = 0 is an empty problem: the call validates and returns
 *   MHLA_OK without launching anything.
 * - Validation errors are returned before any HIP call; in that case nothing
 *   is enqueued.  Faults inside kernels surface at the caller's next
 *   synchronisation of `stream`.
 * - The library holds no global state (apart from mhla_forward_noalloc's
 *   scratch) and is safe to call from several threads; calls that share a
 *   workspace must not overlap in time.
 * - Fault injection for tests: with MHLA_FAIL_ALLOC=1 in the environment,
 *   every stream-ordered workspace allocation fails, so the entry points that
 *   allocate return MHLA_ERR_ALLOC without enqueueing anything.
 */
#ifndef MHLA_H
#define MHLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mhla_status {
    MHLA_OK = 0,
    MHLA_ERR_INVALID_ARG = 1,   /* null pointer, bad extents, grid % block != 0, eps < 0 or
                                   not finite, out overlapping an input, workspace too small */
    MHLA_ERR_UNSUPPORTED = 2,   /* head_dim not in {32, 64, 128}, unknown dtype, a tensor
                                   with 2^31 or more elements, or M * M >= 2^31 */
    MHLA_ERR_MISALIGNED = 3,    /* q, k, v, W, out or workspace not 16-byte aligned */
    MHLA_ERR_ALLOC = 4,         /* workspace allocation on the stream failed */
    MHLA_ERR_HIP = 5            /* a HIP launch or runtime call failed */
} mhla_status;

typedef enum mhla_dtype {
    MHLA_F32 = 0,
    MHLA_BF16 = 1
} mhla_dtype;

/* Problem shape.  extent[0..ndim-1] are the token-grid extents, slowest
 * axis first (2D: {Y, X}; 3D: {T, Y, X}); entries past ndim are ignored. */
typedef struct mhla_grid {
    int32_t batch;       /* B >= 0 */
    int32_t heads;       /* H >= 0 */
    int32_t head_dim;    /* d: 32, 64 or 128 */
    int32_t dtype;       /* mhla_dtype of q, k, v and out */
    int32_t ndim;        /* 2 or 3 */
    int32_t extent[3];
    float eps;           /* added once to every mixed normaliser; finite, >= 0 */
} mhla_grid;

/* Block shape in tokens, same axes and order as the grid; every grid extent
 * must be a multiple of the matching block extent (non-overlapping blocks
 * that tile the grid: section 4 "Architecture"). */
typedef struct mhla_block {
    int32_t extent[3];
} mhla_block;

/* Path selection for mhla_forward_ex. */
enum {
    MHLA_PATH_3KERNEL = 0,   /* block_kv_summary -> mix_summaries -> query_apply */
    MHLA_PATH_FUSED = 1,     /* block_kv_summary -> query_apply_fused (mixes per query
                                block on the fly, skipping zero W entries) */
    MHLA_PATH_CAUSAL = 2     /* causal chunkwise form (paperlayer.ai summary, appendix B
                                "Causal MHLA"): token n attends to tokens m <= n in raster
                                order, A[n,m] = W[b(n),b(m)] phi(q_n).phi(k_m); query block i
                                mixes the summaries of blocks j < i and adds W[i,i] times its
                                own block's tokens up to n.  block_kv_summary ->
                                mix_summaries (W restricted to j < i) -> query_apply_causal.
                                bfloat16 or fp32, any head_dim, and blocks that are contiguous
                                runs of raster indices (e.g. 1D chunks: grid {1, N}, block
                                {1, T}); MHLA_ERR_UNSUPPORTED otherwise. */
};

/* Kernel-variant flags, OR-ed into the path argument of mhla_forward_ex and
 * mhla_launch_plan.  They choose among kernels that compute the same result
 * (for tests and comparisons); problems a variant does not apply to ignore
 * it.  An unknown flag, or more than one mixing flag, gives MHLA_ERR_INVALID_ARG.
 * Without flags the library picks the variant for the problem. */
enum {
    MHLA_VARIANT_MIX_RESIDENT = 1 << 8,   /* bf16, at most 256 source records: persistent mixing
                                             kernel, one workgroup per compute unit, W in registers */
    MHLA_VARIANT_MIX_TILED = 1 << 9,      /* bf16: mixing with one workgroup per column tile of
                                             every query block (any M) */
    MHLA_VARIANT_NO_PAIR_HEADS = 1 << 10, /* bf16, head_dim 32, even head count: one head per wave
                                             in the summary kernel instead of head pairs */
    MHLA_VARIANT_MIX_SPLIT = 1 << 11,     /* bf16, at most 256 source records: mixing with one
                                             workgroup per (pair, column tile, query-block tile) */
    MHLA_VARIANT_APPLY_REGS = 1 << 12     /* bf16, head_dim 32 or 64: each apply wave holds St_i and
                                             zt_i operands in registers instead of reading them from
                                             the copy its head's waves stage in LDS */
};

/* Human-readable name of a status code (static storage, never NULL). */
const char* mhla_status_string(mhla_status status);

/* Validates grid and block alone (no pointers).  Returns MHLA_OK,
 * MHLA_ERR_INVALID_ARG or MHLA_ERR_UNSUPPORTED.  On success and if non-NULL,
 * *num_blocks receives M and *block_tokens receives T = N / M. */
mhla_status mhla_check_problem(const mhla_grid* grid, const mhla_block* block,
                               int64_t* num_blocks, int64_t* block_tokens);

/* The kernels a call with these arguments launches, in order: *num_kernels
 * receives 3 (MHLA_PATH_3KERNEL, MHLA_PATH_CAUSAL), 2 (MHLA_PATH_FUSED) or 0
 * (empty problem) and, if kernel_names is non-NULL, kernel_names[0..2]
 * receive static names of the kernels, NULL past the count:
 * "block_kv_summary", then "mix_summaries" and "query_apply" (or
 * "query_apply_causal"), or "query_apply_fused".  Returns the validation
 * status of grid, block and path; makes no HIP call. */
mhla_status mhla_launch_plan(const mhla_grid* grid, const mhla_block* block, int32_t path,
                             int32_t* num_kernels, const char** kernel_names);

/* Bytes of device workspace mhla_forward_ws / mhla_forward_ex need for this
 * problem (0 for an invalid problem or an empty one).  Layout, from the
 * start of the workspace, for P = B*H pairs ordered (b, h):
 *   region 0: summaries, P*M records of (d*d + d) elements of the compute
 *             type (bf16 for a bf16 problem, fp32 for fp32): S_j transposed
 *             ([e][c], c fastest: element (e, c) = sum phi(k)[c] v[e]),
 *             then z_j[c];
 *   region 1 (at a 256-byte boundary): mixed summaries St_i transposed,
 *             P*M records of d*d compute-type elements ([e][c]);
 *   region 2 (at a 256-byte boundary): mixed normalisers zt_i, P*M*d fp32;
 *   region 3 (at a 256-byte boundary, bf16 problems only): W rounded to
 *             bf16 and zero padded to roundup(M, 64) x roundup(M, 32), stored
 *             in the mixing kernel's operand order: 8-element unit
 *             (rt * roundup(M,32)/32 + kk) * 64 + l holds
 *             W[16*rt + l%16][32*kk + 8*(l/16) .. +7].
 * After a MHLA_PATH_3KERNEL call completes, regions 0-2 hold these
 * intermediates; the fused path fills region 0 only.
 * Token parts (bf16 problems with few blocks): let tasks = B*H*M and T the
 * tokens per block; tp starts at 1 and doubles while tasks*tp < 1536,
 * M*2*tp <= 256 and 2*tp*64 <= T.  With tp > 1 a MHLA_PATH_3KERNEL call
 * splits each block's 32-token steps into tp contiguous runs: region 0 then
 * holds P*M*tp records, record (pair, j*tp + t) summing part t of block j
 * (S_j and z_j are the sums over t), and region 3 holds W with each column
 * repeated tp times (roundup(M*tp, 32) columns).  The fused path writes
 * tp = 1 records.
 * Causal sub-chunks (bf16 problems with contiguous chunks): cp starts at 1
 * and doubles while the chunk's slowest axis of extent > 1 divides by 2*cp,
 * T/(2*cp) >= 256 and M*2*cp <= 256.  With cp > 1 a MHLA_PATH_CAUSAL call
 * runs the causal form on the M*cp sub-chunks (W between sub-chunks a and b
 * is W[a/cp][b/cp]), so its records in regions 0-2 are per sub-chunk and
 * region 3 holds that sub-chunk coefficient matrix.
 * Causal W parts (bf16 problems whose blocks are contiguous runs of raster
 * order): a MHLA_PATH_CAUSAL call takes W into its mixing as a bf16 high part
 * bf16(w) and a bf16 low part bf16(w - bf16(w)), so that the mixtures see W
 * to about 16 significant bits; region 3 then holds 2 columns per summary
 * record, the high part first.
 * Sizes: region 0 holds P*M*max(tp, cp) records, regions 1 and 2 P*M*cp,
 * region 3 roundup(M*cp, 64) x roundup(M*max(tp, k), 32) bf16 values, with
 * k = 2*cp when the blocks are contiguous runs of raster order, else k = cp. */
size_t mhla_workspace_bytes(const mhla_grid* grid, const mhla_block* block);

/* The MHLA forward pass: out = MHLA(q, k, v; W) for the whole problem,
 * enqueued on `stream` (0 = the null stream).  Allocates its workspace with
 * hipMallocAsync / hipFreeAsync on the same stream (MHLA_ERR_ALLOC if that
 * fails).  Uses the 3-kernel path. */
mhla_status mhla_forward(const void* q, const void* k, const void* v, const float* W,
                         const mhla_grid* grid, const mhla_block* block, void* out,
                         hipStream_t stream);

/* As mhla_forward, with a caller-provided device workspace of ws_bytes
 * >= mhla_workspace_bytes(grid, block) bytes (16-byte aligned).  Allocates
 * nothing. */
mhla_status mhla_forward_ws(const void* q, const void* k, const void* v, const float* W,
                            const mhla_grid* grid, const mhla_block* block, void* out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* As mhla_forward_ws, with a path choice (MHLA_PATH_*, optionally OR-ed with
 * MHLA_VARIANT_* flags) and optional stage
 * events.  If stage_events is non-NULL it points to 4 hipEvent_t handles
 * created by the caller; they are recorded on `stream` before the first
 * kernel, after the summary kernel, after the mixing kernel (right after
 * the summary kernel on the fused path) and after the last kernel, so the
 * caller can time each kernel with hipEventElapsedTime.  ws may be NULL
 * (with ws_bytes 0) to allocate on the stream as mhla_forward does. */
mhla_status mhla_forward_ex(const void* q, const void* k, const void* v, const float* W,
                            const mhla_grid* grid, const mhla_block* block, void* out,
                            void* ws, size_t ws_bytes, int32_t path,
                            const hipEvent_t* stage_events, hipStream_t stream);

/* ---------------------------------------------------------------- no allocation
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * mhla_forward_noalloc is mhla_forward (3-kernel path, same kernels, same
 * results) with its workspace taken from a fixed scratch array of
 * MHLA_NOALLOC_SCRATCH_BYTES bytes of device memory built into the library:
 * every GPU the library runs on holds its own copy from the first call on
 * that GPU until the process ends.  The call allocates nothing (no hipMalloc,
 * hipMallocAsync, hipFree or allocating library routine); the caller still
 * passes q, k, v, W and out as for mhla_forward.
 * - Problems whose workspace (mhla_workspace_bytes) exceeds
 *   MHLA_NOALLOC_SCRATCH_BYTES return MHLA_ERR_UNSUPPORTED before any HIP call
 *   (the metric workload, 256 x 256 tokens, H = 6, d = 64 bf16, needs 26 MB).
 * - `stream` (0 = the null stream) must belong to the current device, whose
 *   scratch is used (MHLA_ERR_INVALID_ARG otherwise).
 * - Every call on one GPU shares that GPU's scratch, which keeps the last
 *   call's contents (no part of it needs to start at zero).  Calls that
 *   overlap in time on one GPU (other threads, or other streams not ordered
 *   with this one) race on the scratch and give undefined results.
 * Other errors as for mhla_forward. */
#define MHLA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

mhla_status mhla_forward_noalloc(const void* q, const void* k, const void* v, const float* W,
                                 const mhla_grid* grid, const mhla_block* block, void* out,
                                 hipStream_t stream);

/* ---------------------------------------------------------------- backward
 *
 * Gradients of a scalar loss L through the forward pass above, given the
 * upstream gradient dout = dL/dout: dq, dk, dv (dL/dq, dL/dk, dL/dv) and dW
 * (dL/dW).  W is a learned parameter of the method (paperlayer.ai summary,
 * section 4 "Multi-Head Mixing").  With u = phi(q_n), a = phi(k_m), g = dout_n
 * and the forward's S_j, z_j, St_i, zt_i:
 *
 *   den = u . zt_i + eps,  dnum = g / den,  dden = -(g . o_n) / den
 *   dq_n   = (St_i dnum + zt_i dden) * phi'(q_n)
 *   dSt_i  = sum_{n in i} u dnum^T,  dzt_i = sum_{n in i} u dden
 *   dS_j   = sum_i W[i,j] dSt_i,     dz_j  = sum_i W[i,j] dzt_i
 *   dW[i,j] = sum over (b, h) of <dSt_i, S_j> + <dzt_i, z_j>
 *   dv_m   = dS_j^T a,  dk_m = (dS_j v_m + dz_j) * phi'(k_m)
 *
 * with phi'(x) = 1 for x > 0 and exp(x) otherwise.
 *
 * Every problem the forward accepts: q, k, v, dout, dq, dk, dv: [B, N, H, d]
 * in the grid's dtype as for the forward; W: fp32 [M, M] (read); dW: fp32
 * [M, M], overwritten (zero for an empty problem).  All device pointers,
 * 16-byte aligned, owned by the caller; no output may overlap an input or
 * another output.  bfloat16 problems with head_dim 32 or 64: products in bf16
 * MFMA with fp32 accumulation, gradients of the summaries kept in bf16.  Other
 * problems (fp32, or head_dim 128): fp32 arithmetic throughout, with fp32
 * records of the summaries and their gradients.  The forward summaries are
 * recomputed.  Asynchronous on `stream`. */

/* Bytes of device workspace mhla_backward needs (0 for an invalid or empty
 * problem).  bf16 with head_dim 32 or 64, from the start: the forward's
 * regions 0-3 (see mhla_workspace_bytes), then at 256-byte boundaries:
 * gradients of the mixed summaries as B*H*M bf16 records in the summaries'
 * layout; gradients of the summaries, B*H*M*d*d bf16 ([e][c] order); gradients
 * of the normalisers, B*H*M*d fp32; W^T in the mixing kernel's operand order;
 * dW partial sums; and when tokens are split into parts (ap > 1, where ap
 * starts at 1 and doubles while B*H*M*ap < 1536 and 2*ap*64 <= T), the query
 * side's fp32 partial records of the mixed summaries' gradients, B*H*M*ap
 * records of d*d + d values.  Other problems: four fp32 record arrays of B*H*M*(d*d + d)
 * values (summaries [c][e] then z, mixed summaries, their gradients, the
 * summaries' gradients), then dW partial sums. */
size_t mhla_backward_workspace_bytes(const mhla_grid* grid, const mhla_block* block);

/* The backward pass, enqueued on `stream`.  ws: workspace of ws_bytes >=
 * mhla_backward_workspace_bytes (16-byte aligned), or NULL with ws_bytes 0 to
 * allocate it on the stream (hipMallocAsync / hipFreeAsync).  stage_events:
 * NULL or 5 caller-created events recorded before the first kernel, after the
 * forward recompute (summary and mixing kernels), after the query-side kernel
 * (dq and the gradients of the mixed summaries), after the transposed mixing
 * and dW kernels, and after the key/value-side kernel (dk, dv).  Returns the
 * same codes as mhla_forward_ex. */
mhla_status mhla_backward(const void* q, const void* k, const void* v, const float* W, const void* dout,
                          const mhla_grid* grid, const mhla_block* block, void* dq, void* dk, void* dv,
                          float* dW, void* ws, size_t ws_bytes, const hipEvent_t* stage_events,
                          hipStream_t stream);

/* As mhla_backward, with kernel-variant flags: 0 or MHLA_VARIANT_NO_PAIR_HEADS
 * (head_dim 32, even head count: the key/value-side kernel takes one head per
 * wave instead of head pairs; same result).  Other flags give
 * MHLA_ERR_INVALID_ARG. */
mhla_status mhla_backward_ex(const void* q, const void* k, const void* v, const float* W, const void* dout,
                             const mhla_grid* grid, const mhla_block* block, void* dq, void* dk, void* dv,
                             float* dW, void* ws, size_t ws_bytes, int32_t variant,
                             const hipEvent_t* stage_events, hipStream_t stream);

/* ---------------------------------------------------------------- causal backward
 *
 * Gradients through the causal chunkwise form (MHLA_PATH_CAUSAL; paperlayer.ai
 * summary, appendix B "Causal MHLA"), for chunks contiguous in raster order.
 * Token n of chunk i sees C_n = St_i< + w P_n and zeta_n = zt_i< + w zp_n,
 * with St_i< = sum_{j<i} W[i,j] S_j, w = W[i,i] and P_n, zp_n the chunk's
 * prefix sums of a v^T and a over m <= n.  With den, dnum, dden as above:
 *
 *   dq_n     = (C_n dnum + zeta_n dden) * phi'(q_n)
 *   dSt_i<   = sum_{n in i} u dnum^T,  dzt_i< = sum_{n in i} u dden
 *   R_m, r_m = suffix sums over n >= m in the chunk of u dnum^T and u dden
 *   G_m      = sum_{k>i} W[k,i] dSt_k< + w R_m  (g_m likewise with dzt, r)
 *   dv_m     = G_m^T a,  dk_m = (G_m v_m + g_m) * phi'(k_m)
 *   dW[i,j]  = sum over (b, h) of <dSt_i<, S_j> + <dzt_i<, z_j>   (j < i)
 *   dW[i,i]  = sum over (b, h) and m in i of a . (R_m v_m + r_m), dW[i,j] = 0 (j > i)
 *
 * Arguments, layouts, ownership and aliasing rules as for mhla_backward; the
 * coefficients W[i,j] with j > i are never read.  bf16 or fp32, head_dim 32,
 * 64 or 128, fp32 arithmetic throughout.  MHLA_ERR_UNSUPPORTED when the
 * chunks are not contiguous in raster order (blocks spanning whole rows of
 * the grid, or any sequence). */

/* Bytes of device workspace mhla_causal_backward needs (0 for an invalid,
 * empty or unsupported problem): the four fp32 record arrays and dW partial
 * sums of the general backward path, then at 256-byte boundaries each token's
 * dnum (B*N*H*d fp32), each token's dden (B*N*H fp32) and the in-chunk terms
 * of dW's diagonal (B*H*M fp32). */
size_t mhla_causal_backward_workspace_bytes(const mhla_grid* grid, const mhla_block* block);

/* The causal backward pass, enqueued on `stream`; ws and stage_events as for
 * mhla_backward, except that the fourth event is recorded before the
 * key/value-side kernel and the dW reduction follows that kernel (it supplies
 * the diagonal). */
mhla_status mhla_causal_backward(const void* q, const void* k, const void* v, const float* W, const void* dout,
                                 const mhla_grid* grid, const mhla_block* block, void* dq, void* dk, void* dv,
                                 float* dW, void* ws, size_t ws_bytes, const hipEvent_t* stage_events,
                                 hipStream_t stream);

/* ---------------------------------------------------------------- causal streaming
 *
 * Stateful execution of the causal chunkwise form (the method keeps O(N) cost
 * and supports streaming or stateful execution: paperlayer.ai summary, key
 * points; appendix B "Causal MHLA").  A sequence arrives as calls of whole
 * chunks; a state of fp32 chunk summaries carries what later chunks need.
 * A call's grid and block describe its new tokens (chunks contiguous in
 * raster order, as for MHLA_PATH_CAUSAL); its chunks get the global indices
 * i = n_past .. n_past + M - 1.  For each new chunk i, with u = phi(q_n):
 *
 *   state[i] = [S_i | z_i] = [sum_{m in i} phi(k_m) v_m^T | sum_{m in i} phi(k_m)]
 *   o_n = u^T (St_i< + W[i,i] P_n) / (u . (zt_i< + W[i,i] zp_n) + eps)
 *   St_i< = sum_{j<i} W[i,j] S_j  (zt_i< likewise, over the state's slots j < i)
 *
 * P_n, zp_n the chunk's sums of phi(k_m) v_m^T and phi(k_m) over m <= n.  A
 * sequence streamed in any split into calls gives the outputs of one
 * MHLA_PATH_CAUSAL call on the whole sequence (chunk lengths may differ
 * between calls; the math is per chunk).
 *
 * state: fp32 [B*H][max_chunks][d*d + d] (pair b*H + h; per slot S as
 * [c][e], key channel c slowest, then z), device memory owned by the
 * caller; slots 0 .. n_past-1 must hold the summaries written by earlier
 * calls (or by the caller), slots n_past .. n_past + M - 1 are overwritten.
 * W: fp32 [w_dim][w_dim] row-major; only W[i][j] with j <= i for the new
 * rows i is read.  q, k, v, out: [B, N_new, H, d] in the grid's dtype.
 * Summaries and mixtures are formed in fp32; fp32 problems compute the
 * outputs in fp32 token by token, bf16 problems round the mixtures to bf16
 * operands and run the one-shot causal form's matrix-core apply (the
 * forward's bf16 accuracy).  Errors: MHLA_ERR_UNSUPPORTED for chunks that are not
 * contiguous; MHLA_ERR_INVALID_ARG for n_past < 0, n_past + M beyond
 * max_chunks or w_dim, null pointers, or overlaps between out, state, the
 * inputs and the workspace; MHLA_ERR_MISALIGNED for pointers not 16-byte
 * aligned.  An empty problem (B or H zero) does nothing. */

/* Bytes of the state for max_chunks chunks (0 for an invalid problem). */
size_t mhla_causal_state_bytes(const mhla_grid* grid, const mhla_block* block, int32_t max_chunks);

/* Bytes of workspace a call needs for the new chunks' mixtures: B*H*M
 * records of d*d + d fp32 for fp32 problems; for bf16 problems B*H*M*cp*d*d
 * bf16 (the mixed S, rounded) and B*H*M*cp*d fp32 (the mixed z), where cp is
 * the sub-chunk count of mhla_workspace_bytes' causal rule (long chunks run
 * as cp sub-chunks each), and with cp > 1 also B*H*M records of d*d + d fp32
 * (the chunks' mixtures) and B*H*M*cp such records (the sub-chunks'
 * summaries).  0 for an invalid, empty or unsupported problem. */
size_t mhla_causal_stream_workspace_bytes(const mhla_grid* grid, const mhla_block* block);

/* One call of the stream, enqueued on `stream`: summaries of the new chunks
 * into the state, their mixtures over earlier chunks, their outputs.  ws: at
 * least mhla_causal_stream_workspace_bytes (16-byte aligned), or NULL with
 * ws_bytes 0 to allocate it on the stream.  Calls on one state must be
 * ordered (same stream, or synchronised). */
mhla_status mhla_causal_stream(const void* q, const void* k, const void* v, const float* W, int32_t w_dim,
                               const mhla_grid* grid, const mhla_block* block, int32_t n_past, float* state,
                               int32_t max_chunks, void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- layer
 *
 * The layer around the core, after the plug-and-play module of the
 * 171host.com repost, section 七 (class MHLA, forward), on tokens in raster
 * order:
 *
 *   xn = LayerNorm(x) (biased variance over the C channels, ln_eps)
 *   [q | k | v] = xn w_qkv^T + b_qkv                   (w_qkv: [3C, C])
 *   q, k = RMSNorm(q; qn_w), RMSNorm(k; kn_w)          (only if qn_w != NULL)
 *   o = the core (mhla_forward, 3-kernel path) on q, k, v with feature map
 *       elu(x) + 1 (MHLA_PHI_ELU1) or relu(x) + phi_eps (MHLA_PHI_RELU_EPS)
 *   o += LePE(v): depthwise 5x5 convolution of v over the 2D token grid,
 *       zero padding 2, plus lepe_b     (only if lepe_w != NULL; 2D grids)
 *   y = o w_out^T + b_out                              (w_out: [C, C])
 *
 * C = heads * head_dim.  Dropout is the identity (inference).  Weight
 * matrices are bfloat16 laid out [output features, input features]; norm
 * weights, biases and the LePE kernels ([C][5][5], cross-correlation as in
 * convolution layers) are fp32.  Biases may be NULL (zero).  x, y: [B, N, C]
 * bfloat16.  Only bfloat16 grids (grid->dtype == MHLA_BF16). */

typedef enum mhla_phi {
    MHLA_PHI_ELU1 = 0,       /* elu(x) + 1, the core's feature map */
    MHLA_PHI_RELU_EPS = 1    /* relu(x) + phi_eps, as in the module's code */
} mhla_phi;

typedef struct mhla_layer_params {
    const float* ln_w;       /* [C] LayerNorm weight (required) */
    const float* ln_b;       /* [C] LayerNorm bias (required) */
    const void* w_qkv;       /* [3C][C] bfloat16 (required) */
    const float* b_qkv;      /* [3C] or NULL */
    const float* qn_w;       /* [C] q RMSNorm weight, or NULL for no q/k norm */
    const float* kn_w;       /* [C] k RMSNorm weight (required with qn_w, else NULL) */
    const float* lepe_w;     /* [C][5][5] or NULL for no LePE */
    const float* lepe_b;     /* [C] or NULL */
    const void* w_out;       /* [C][C] bfloat16 (required) */
    const float* b_out;      /* [C] or NULL */
    int32_t phi;             /* mhla_phi */
    float phi_eps;           /* >= 0, used by MHLA_PHI_RELU_EPS */
    float ln_eps;            /* > 0 */
    float rms_eps;           /* > 0 when q/k norms are used */
} mhla_layer_params;

/* Bytes of device workspace mhla_layer_forward needs (0 for an invalid or
 * empty problem).  Layout: q, k, v, o as [B, N, C] bfloat16, w_qkv scaled by
 * the LayerNorm weight ([3C][C] bfloat16), its column sums and folded bias
 * ([3C] fp32 each), the token means and inverse deviations of x ([B*N] fp32
 * each), then the core's workspace (mhla_workspace_bytes), each region at a
 * 256-byte boundary. */
size_t mhla_layer_workspace_bytes(const mhla_grid* grid, const mhla_block* block);

/* The layer forward, enqueued on `stream`.  x, y: device [B, N, C] bfloat16;
 * W: fp32 [M, M] as for mhla_forward; params: host struct of device pointers
 * (16-byte aligned).  ws: workspace of ws_bytes >= mhla_layer_workspace_bytes
 * (16-byte aligned) or NULL with ws_bytes 0 to allocate it on the stream.
 * stage_events: NULL or 5 caller-created events recorded before the first
 * kernel, after the QKV projection (and q/k norms), after the core, after
 * LePE and after the output projection.  y must not overlap x, W, a
 * parameter or the workspace.  Errors: MHLA_ERR_UNSUPPORTED for fp32 grids,
 * or LePE on a 3D grid; MHLA_ERR_INVALID_ARG for a missing required pointer,
 * an unknown phi, a negative or non-finite eps, overlaps or a short
 * workspace; otherwise as mhla_forward_ex. */
mhla_status mhla_layer_forward(const void* x, const float* W, const mhla_grid* grid, const mhla_block* block,
                               const mhla_layer_params* params, void* y, void* ws, size_t ws_bytes,
                               const hipEvent_t* stage_events, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MHLA_H */
