// launch.h -- internal launchers of the libmhla kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace mhla {

struct Tuning {
    int summary_waves;   // fp32 path: waves splitting the tokens of one block (1, 2, 4)
    int summary_pf;      // bf16 path: k-steps of K/V loads in flight per wave (1, 2)
    int d128_shared;     // bf16 path, head_dim 128: summary waves share K/V operands through LDS,
                         // this many heads (1, 2) per workgroup; 0 = quadrant waves loading their own
    int apply_waves;     // waves splitting the tokens of one block in query_apply (1, 2, 4)
    int apply_pf;        // bf16 path: 16-token groups of Q loads in flight per wave (1, 2, 4)
    int pair_heads;      // bf16 path, head_dim 32 with an even head count: summaries of head pairs
    int bwdq_heads;      // bf16 backward: heads per bwd_query workgroup (0: the kernel's maximum)
    int apply_maxw;      // bf16 path: waves per query_apply workgroup (4 or 8; heads grouped up to it)
    int apply_lds;       // bf16 path, d <= 64: query_apply reads St_i, zt_i operands from LDS (staged once per head)
    int nt_loads;        // bf16 path: non-temporal hint on the loads of k, v (summary kernel)
    int nt_apply;        // bf16 path: non-temporal hint on the loads of q (apply kernel)
    int nt_mix;          // bf16 persistent mixing kernel: 1 = non-temporal summary loads, 2 = non-temporal stores of St
    int mix_kind;        // bf16 path, M <= 256: 2 = mix_split (workgroup per tile), 1 = persistent
                         // mix_resident with W in registers, 0 = mix_summaries (any M)
    int mix_rows;        // mix_split: query blocks per wave / 16 (1 or 2; 0 = by M)
    int bwd_fuse;        // backward: W^T mixing of the gradient records and dW partials in one launch
    int num_cus;         // compute units of the current device (persistent grid size)
};

struct Launch {
    const void* q;
    const void* k;
    const void* v;
    const float* W;
    void* out;
    void* sz;      // summaries  [BH][M][D*D + D]   (compute type)
    void* st;      // mixed      [BH][M][D*D]       (compute type)
    float* zt;     // mixed normalisers [BH][M][D]  (fp32)
    void* wb;      // bf16 path: W as bf16 [roundup(M,64)][roundup(M,32)], zero padded
    void* wbt;     // bf16 path: W^T in the same form as well (backward), or nullptr
    Geo g;
    Tuning tune;
    int path;                     // MHLA_PATH_*
    int summaries_only;           // bf16: stop after the mixing kernel (backward recompute)
    const hipEvent_t* events;     // 4 events or nullptr
    hipStream_t stream;
};

// Enqueue the whole forward pass for one dtype.  Returns the first HIP error.
hipError_t run_bf16(const Launch& L);
hipError_t run_f32(const Launch& L);

// Backward pass (bf16, d = 32 or 64).  F holds the inputs q, k, v, W, the
// forward workspace regions (summaries, mixed summaries, normalisers, W in
// operand order) that the recompute fills, geometry, tuning and stream.
struct BwdLaunch {
    Launch F;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* dw;
    uint16_t* dst;    // gradients of the mixed summaries, records [BH][M][D*D + D] (bf16)
    uint16_t* ds;     // gradients of the summaries [BH][M][D*D] (bf16, record order)
    float* dz;        // gradients of the normalisers [BH][M][D]
    uint16_t* wbt;    // W^T in the mixing kernel's operand order
    float* part;      // dW partial sums [nsplit][M][M]
    int nsplit;
    int kv_parts;     // token parts of bwd_kv (1: one workgroup per block and head group)
    int q_parts;      // token parts of bwd_query (1: as above)
    float* dpart;     // q_parts > 1: fp32 partial records of dSt [BH][M][q_parts][D*D + D]
    uint16_t* sfold;  // recompute in token parts (F.g.TP > 1): S records folded to [BH][M][D*D + D]
    const hipEvent_t* events;   // 5 events or nullptr
};

// Summary and mixing kernels of the bf16 forward only (regions of F).
hipError_t run_bf16_summaries(const Launch& L);
hipError_t run_bwd_bf16(const BwdLaunch& B);
// The bf16 mixing product of records src (layout of the summaries) with W's
// operands wops (as converted by the summary launch) into dst (bf16) and
// zdst (fp32), on the kernel that suits g (L supplies tuning and stream).
hipError_t launch_mix_records_bf16(const Launch& L, const uint16_t* src, const uint16_t* wops, uint16_t* dst,
                                  float* zdst, const Geo& g);
// The piece of the bf16 backward shared with the causal form: the mixing of
// B.dst with W^T (B.wbt) into B.ds, B.dz, and the dW partial products of
// B.dst with the summary records srec into B.nsplit partial tiles at B.part
// (g: one record per block); one launch for 129..256 blocks, two otherwise.
hipError_t launch_mix_dw_bf16(const BwdLaunch& B, const Geo& g, const uint16_t* srec);

// The bf16 causal backward (d = 32 or 64, chunks contiguous in raster order,
// one sub-chunk per chunk).  B.F runs the recompute (path MHLA_PATH_CAUSAL,
// summaries_only, wbt set); B.dst, B.ds, B.dz, B.wbt, B.part, B.nsplit as in
// the non-causal backward; B.events: 5 events or nullptr.
struct CausalBwdLaunch {
    BwdLaunch B;
    float* tsc;       // [B][N][H][2]: per token 1 / den and dden = -(g . num) / den^2
    float* diag;      // [BH][M]: each pair's in-chunk terms of dW[i][i]
};
hipError_t run_causal_bwd_bf16(const CausalBwdLaunch& C);
// The causal chunkwise apply (bf16, d = 32 or 64) after the summary and
// mixing kernels have run with W restricted to earlier blocks.
// The causal apply kernel on the workspace's St, zt; W's diagonal entry of
// block i is read as L.W[iw * wld + iw], iw = i / g.WD (wld <= 0: g.WM, the
// one-shot form's square W).
hipError_t launch_causal_apply_bf16(const Launch& L, int wld = 0);

// The layer around the core: LayerNorm + QKV projection, optional q/k
// RMSNorm, the feature-map variant, the core (core.q/k/v/out point at q, k,
// v, o below), LePE added into o, output projection into y.
struct LayerLaunch {
    const uint16_t* x;      // [R][C] layer input
    uint16_t* y;            // [R][C] layer output
    uint16_t* q;            // workspace [R][C] each
    uint16_t* k;
    uint16_t* v;
    uint16_t* o;
    const uint16_t* w_qkv;  // [3C][C]
    uint16_t* wf;           // workspace: w_qkv scaled by the LayerNorm weight [3C][C]
    float* colsum;          // workspace [3C]
    float* biasf;           // workspace [3C]
    float* mean;            // workspace [R]: token means of x
    float* rstd;            // workspace [R]: token inverse deviations of x
    const float* ln_w;
    const float* ln_b;
    const float* b_qkv;     // or nullptr
    const float* qn_w;      // or nullptr (no q/k RMSNorm)
    const float* kn_w;
    const float* lepe_w;    // [C][5][5] or nullptr (no LePE)
    const float* lepe_b;    // or nullptr
    const uint16_t* w_out;  // [C][C]
    const float* b_out;     // or nullptr
    float ln_eps, rms_eps, phi_eps;
    int relu_phi;
    int R, C, B, Y, X;      // tokens (B N), channels, batch, 2D grid extents (LePE)
    Launch core;
    const hipEvent_t* events;   // 5 events or nullptr
    hipStream_t stream;
};
hipError_t run_layer_bf16(const LayerLaunch& L);

// Backward pass for the problems the bf16 MFMA kernels do not take (fp32
// inputs, or head_dim 128) and for the causal form: fp32 records [S | z] of
// L = d*d + d values.
struct GenericBwd {
    Geo g;
    int bf16;                 // inputs and gradients in bf16 (else fp32)
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* W;
    void* dq;
    void* dk;
    void* dv;
    float* dw;
    float* s;                 // [BH][M][L] summaries
    float* st;                // [BH][M][L] mixed summaries
    float* dst;               // [BH][M][L] their gradients
    float* ds;                // [BH][M][L] gradients of the summaries
    float* part;              // [nsplit][M][M] dW partial sums
    int nsplit;
    int causal;               // causal chunkwise form (chunks contiguous in raster order)
    float* dnum;              // causal: [B][N][H][d] per-token g / den
    float* dden;              // causal: [B][N][H] per-token -(g . o) / den
    float* diag;              // causal: [BH][M] in-chunk terms of dW[i][i]
    const hipEvent_t* events; // 5 events or nullptr
    hipStream_t stream;
};
hipError_t run_bwd_generic(const GenericBwd& B);

// Stateful causal execution: the new chunks of a sequence (Geo describes
// them), fp32 state records of every chunk [B*H][max_chunks][d*d + d].
struct StreamLaunch {
    Geo g;
    int bf16;                 // q, k, v, out in bf16 (else fp32)
    const void* q;
    const void* k;
    const void* v;
    const float* W;           // [w_dim][w_dim]
    int w_dim;
    int n_past;               // chunks already in the state
    float* state;
    int max_chunks;
    float* mixed;             // fp32 problems: mixtures [B*H][M][d*d + d] (workspace), else null
    uint16_t* st;             // bf16 problems: mixed St^T [B*H][M][d][d] (bf16, workspace), else null
    float* zt;                // bf16 problems: mixed zt [B*H][M][d] (fp32, workspace)
    // bf16 problems with long chunks: cp sub-chunks per chunk, their geometry
    // (WD = cp), their fp32 summaries [B*H][M*cp][d*d + d]; `mixed` then holds
    // the chunks' fp32 mixtures and st, zt the sub-chunks' operands.
    int cp;
    Geo gs;
    float* ssub;
    void* out;
    hipStream_t stream;
};
hipError_t run_causal_stream(const StreamLaunch& S);

// p[0 .. n) = 0 by a kernel (safe inside a captured graph).
hipError_t zero_f32(float* p, int n, hipStream_t stream);

}  // namespace mhla
