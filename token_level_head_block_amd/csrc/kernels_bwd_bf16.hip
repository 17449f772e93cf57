// kernels_bwd_bf16.hip -- gradients of the MHLA forward pass for bfloat16
// inputs on gfx950 (MI355X), d = 32 or 64.
//
// W is a learned parameter of the method (MHLA, arXiv 2601.07832;
// paperlayer.ai summary, section 4 "Multi-Head Mixing"), so the backward pass
// returns dq, dk, dv and dW.  With u = phi(q), a = phi(k), g = dL/do and the
// forward's S_j, z_j, St_i, zt_i (recomputed by the forward kernels):
//
//   den = u . zt_i + eps,  dnum = g / den,  dden = -(g . o) / den
//   dq  = (St_i dnum + zt_i dden) * phi'(q)
//   dSt_i = sum_{n in i} u dnum^T,  dzt_i = sum_{n in i} u dden        (bwd_query)
//   dS_j = sum_i W[i,j] dSt_i,  dz_j = sum_i W[i,j] dzt_i              (mixing with W^T)
//   dW[i,j] = sum over (b, h) of <dSt_i, S_j> + <dzt_i, z_j>          (dw_partial, then the sum of its partials)
//   dv = dS_j^T a,  dk = (dS_j v + dz_j) * phi'(k)                       (bwd_kv)
//
// with phi'(x) = 1 for x > 0 and exp(x) otherwise.  Products run on bf16
// MFMA with fp32 accumulation; the gradients of the summaries are kept as
// bf16 records in the summaries' own layout ([e][c] then the normaliser part),
// so dW is one GEMM over all (b, h) and record elements.
#include "launch.h"
#include "bf16_shared.h"

#include <mhla.h>

#include <algorithm>
#include <type_traits>

namespace mhla {
namespace {

// A x B operand rows for a d x d matrix held as [e][c] (c fastest), the way
// the summaries store S^T: row e, lane (t, gq) rows in the order that leaves
// each lane with 4*RT consecutive outputs, and the k-slots of lane group gq at
// c = 4 * RT * gq + 8 * kk + s: the 4 * RT channels that lane group also holds
// as output rows of a product whose A operand comes from rows_c_k_e.
template <int D>
__device__ __forceinline__ void rows_e_k_cl(const uint16_t* __restrict__ m, int t, int gq, u32x4 (&a)[D / 16][D / 32]) {
    constexpr int RT = D / 16, KS = D / 32;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int e = 4 * RT * (t >> 2) + 4 * r + (t & 3);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) a[r][kk] = *reinterpret_cast<const u32x4*>(m + e * D + 4 * RT * gq + 8 * kk);
    }
}

// The transposed operand of the same matrix: row c, k-slot s of k-step kk at
// e = ebase(gq) + 8 * kk + s, gathered element by element (once per block).
template <int D>
__device__ __forceinline__ void rows_c_k_e(const uint16_t* __restrict__ m, int t, int ebase,
                                           u32x4 (&a)[D / 16][D / 32]) {
    constexpr int RT = D / 16, KS = D / 32;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int c = 4 * RT * (t >> 2) + 4 * rt + (t & 3);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int e0 = ebase + 8 * kk + 2 * w;
                a[rt][kk][w] = (uint32_t)m[e0 * D + c] | ((uint32_t)m[(e0 + 1) * D + c] << 16);
            }
    }
}

// =====================================================================
// bwd_query: dq and the gradients of the mixed summaries, per query block.
// Workgroup = (b, block i, group of <= 8 heads), one wave per head over all of
// the block's tokens, 16 tokens per step (token t = lane % 16):
//   num = St^T u and den (as in the forward apply), then dnum = g / den, dden;
//   du  = (St g) / den (MFMA on the bf16 upstream gradient itself; k-slots of
//         lane group gq are its own 4*RT channels) + zt dden, dq = du * phi'(q);
//   dSt += u dnum^T, dzt += u dden on v_mfma_f32_16x16x16_bf16 with the 16
//   tokens as k, both operands read transposed from the wave's LDS slice.
// =====================================================================
// LOP = false: a wave keeps two operand copies of St in registers (at d = 64:
// 64 registers), zt's operand words and zt itself, and with the dSt
// accumulators (64) and a token group's working set that is more than 256
// registers at d = 64: one wave per SIMD.
// LOP = true (d = 64, blocks of >= 128 tokens): the transposed copy of St
// (rows c, k = e), zt's operand words and zt live in the wave's LDS slice and
// are read where used, so a wave fits in 256 registers: two waves per SIMD
// (dit-s2-256x256 bwd_query 73.5 -> 64.3 us; with 64-token blocks the extra
// staging per block costs more than it saves).
template <int D, bool LOP>
__global__ __launch_bounds__(D == 64 ? 256 : 512) __attribute__((amdgpu_waves_per_eu(LOP ? 2 : 1))) void bwd_query_bf16(const uint16_t* __restrict__ Q,
                                                      const uint16_t* __restrict__ dO,
                                                      const uint16_t* __restrict__ St,
                                                      const float* __restrict__ Zt, uint16_t* __restrict__ dQ,
                                                      uint16_t* __restrict__ dSt, float* __restrict__ dpart,
                                                      const Geo g) {
    constexpr int RT = D / 16, KS = D / 32, REC = D * D + D;
    constexpr int OSTR = D + 8, TS = 20;   // TS: transposed tile row, 16 tokens + 4 padding
    constexpr int A2U = LOP ? RT * KS * 64 * 8 : 0;   // bf16 values of the transposed operand copy
    constexpr int ZU = LOP ? 2 * KS * 64 * 8 : 0;     // bf16 values of zt's high and low operand words
    constexpr int SLICE = 16 * OSTR + 2 * D * TS + A2U + ZU + (LOP ? 2 * D : 0);   // + zt (fp32)
    constexpr int MAXW = D == 64 ? 4 : 8;
    __shared__ __attribute__((aligned(16))) uint16_t lds[MAXW * SLICE];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = lane & 15, gq = lane >> 4;
    // Workgroup = (b, block i, token part, head group); with g.AP > 1 part t
    // takes a contiguous run of the block's 16-token groups and leaves its
    // share of dSt, dzt as an fp32 partial record (fold_parts adds them).
    const WgCoordP wgc = wg_coord_parts(g, blockIdx.x, g.div_AP);
    const int hh = wgc.hg * g.G + wave;
    if (hh >= g.H) return;
    const int b = __builtin_amdgcn_readfirstlane(wgc.b);
    const int h = __builtin_amdgcn_readfirstlane(hh);
    const int i = __builtin_amdgcn_readfirstlane(wgc.j);
    const int ngr = (g.T + 15) >> 4, gper = (ngr + g.AP - 1) / g.AP;
    const int gr0 = __builtin_amdgcn_readfirstlane(min(ngr, gper * wgc.t));
    const int gr1 = min(ngr, gr0 + gper);
    const int bh = b * g.H + h, blk = bh * g.M + i;
    uint16_t* sout = lds + wave * SLICE;
    uint16_t* dnT = sout + 16 * OSTR;   // [e][token]
    uint16_t* uT = dnT + D * TS;        // [c][token]
    u32x4* a2l = reinterpret_cast<u32x4*>(uT + D * TS);   // [rt][kk][lane] operand words

    // ---- operands of this block's mixed summary
    const uint16_t* sb = St + (size_t)blk * (D * D);
    const float* zb = Zt + (size_t)blk * D;
    u32x4 a1[RT][KS], a2r[LOP ? 1 : RT][LOP ? 1 : KS], zhi[LOP ? 1 : KS], zlo[LOP ? 1 : KS];
    rows_e_k_cl<D>(sb, t, gq, a1);
    u32x4* zl2 = a2l + A2U / 8;   // [hi/lo][kk][lane] operand words of zt
    float* zl = reinterpret_cast<float*>(zl2 + ZU / 8);   // zt
    float zc[LOP ? 1 : 4 * RT];   // zt at this lane's output channels 4*RT*gq + ..
    if constexpr (LOP) {
        u32x4 a2[RT][KS];
        rows_c_k_e<D>(sb, t, 4 * RT * gq, a2);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) a2l[(rt * KS + kk) * 64 + lane] = a2[rt][kk];
    } else {
        rows_c_k_e<D>(sb, t, 4 * RT * gq, a2r);
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(zb + 4 * RT * gq + 8 * kk);
        const f32x4 y = *reinterpret_cast<const f32x4*>(zb + 4 * RT * gq + 8 * kk + 4);
        const float z[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
        if constexpr (LOP) {
            u32x4 hi, lo;
            split_zt(z, hi, lo);
            zl2[kk * 64 + lane] = hi;
            zl2[(KS + kk) * 64 + lane] = lo;
        } else {
            split_zt(z, zhi[kk], zlo[kk]);
        }
    }
    if constexpr (LOP) {
        if (lane < D / 4) *reinterpret_cast<f32x4*>(zl + 4 * lane) = *reinterpret_cast<const f32x4*>(zb + 4 * lane);
    } else {
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(zb + 4 * RT * gq + 4 * u);
            zc[4 * u] = x.x; zc[4 * u + 1] = x.y; zc[4 * u + 2] = x.z; zc[4 * u + 3] = x.w;
        }
    }

    const int row = g.H * D;
    const int origin = block_origin(g, i);
    const uint16_t* qb = Q + ((size_t)b * g.N * row + h * D);
    const uint16_t* gb = dO + ((size_t)b * g.N * row + h * D);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        dQ + (size_t)b * g.N * row, 0, g.N * row * 2, 0x00020000);
    const int olane = h * D * 2;

    f32x4 dsacc[RT][RT], dzacc[RT];
#pragma unroll
    for (int re = 0; re < RT; ++re) {
        dzacc[re] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rc = 0; rc < RT; ++rc) dsacc[re][rc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    struct Raw {
        u32x4 qv[KS], go[RT / 2];
        int off;
        bool ok;
    };
    auto load = [&](int it, Raw& R) {
        const int p = it * 16 + t;
        R.ok = p < g.T;
        R.off = (origin + in_block(g, R.ok ? p : g.T - 1)) * row;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) R.qv[kk] = *reinterpret_cast<const u32x4*>(qb + R.off + 4 * RT * gq + 8 * kk);
#pragma unroll
        for (int u = 0; u < RT / 2; ++u) R.go[u] = *reinterpret_cast<const u32x4*>(gb + R.off + 4 * RT * gq + 8 * u);
    };
    auto compute = [&](const Raw& R) {
        // u = phi(q) as the B operand (k = channel 4*RT*gq + 8*kk + s, column =
        // token t): the channels of this lane's dq.  With e = exp(min(x, 0)),
        // phi(x) = max(x, 0) + e and phi'(x) = e.
        u32x4 bq[KS];
        float pg[4 * RT];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float x0 = bf_lo(R.qv[kk][w]), x1 = bf_hi(R.qv[kk][w]);
                const float e0 = __expf(fminf(x0, 0.f)), e1 = __expf(fminf(x1, 0.f));
                bq[kk][w] = pack_bf16(fmaxf(x0, 0.f) + e0, fmaxf(x1, 0.f) + e1);
                pg[8 * kk + 2 * w] = e0;
                pg[8 * kk + 2 * w + 1] = e1;
            }
        // num = St^T u, den, and du' = St g: dnum = g / den, so du = du' / den with
        // the bf16 upstream gradient itself as the B operand (k-step kk of lane
        // group gq: e = 4*RT*gq + 8*kk + s, the words the lane loaded).
        f32x4 acc[RT], accd = f32x4{0.f, 0.f, 0.f, 0.f}, du[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = du[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
            for (int r = 0; r < RT; ++r) acc[r] = mfma_bf16(a1[r][kk], bq[kk], acc[r]);
            accd = mfma_bf16(LOP ? zl2[kk * 64 + lane] : zhi[LOP ? 0 : kk], bq[kk], accd);
            accd = mfma_bf16(LOP ? zl2[(KS + kk) * 64 + lane] : zlo[LOP ? 0 : kk], bq[kk], accd);
        }
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                du[rt] = mfma_bf16(LOP ? a2l[(rt * KS + kk) * 64 + lane] : a2r[LOP ? 0 : rt][LOP ? 0 : kk], R.go[kk],
                                   du[rt]);
        // 1 / den; zero for a token past the block (its row is a clamped copy of
        // a valid one), which zeroes its dnum, dden and so its dSt, dzt terms
        const float inv = R.ok ? 1.f / (accd[0] + g.eps) : 0.f;
        // Upstream gradient at this lane's channels e = 4*RT*gq + 4r + v.
        float gl[4 * RT];
#pragma unroll
        for (int u = 0; u < RT / 2; ++u) unpack8(R.go[u], gl + 8 * u);
        float dot = 0.f;   // g . num over this lane's channels
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int v = 0; v < 4; ++v) dot += gl[4 * r + v] * acc[r][v];
        dot += shfl_xor(dot, 16);
        dot += shfl_xor(dot, 32);
        const float dden = -dot * inv * inv;
        // dnum in bf16, transposed for the dSt product
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int e = 4 * RT * gq + 8 * kk + 2 * w;
                const uint32_t hw = pack_bf16(gl[8 * kk + 2 * w] * inv, gl[8 * kk + 2 * w + 1] * inv);
                dnT[e * TS + t] = (uint16_t)(hw & 0xffffu);
                dnT[(e + 1) * TS + t] = (uint16_t)(hw >> 16);
            }
        uint32_t wv[2 * RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float x[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int cl = 4 * rt + v;
                x[v] = (du[rt][v] * inv + (LOP ? zl[4 * RT * gq + cl] : zc[LOP ? 0 : cl]) * dden) * pg[cl];
            }
            wv[2 * rt] = pack_bf16(x[0], x[1]);
            wv[2 * rt + 1] = pack_bf16(x[2], x[3]);
        }
        store_rows<D>(sout, wv, lane, R.off, R.ok, rsrc, olane);

        // ---- dSt += u dnum^T and dzt += u dden over these 16 tokens.
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int c = 4 * RT * gq + 8 * kk + 2 * w;
                uT[c * TS + t] = (uint16_t)(bq[kk][w] & 0xffffu);
                uT[(c + 1) * TS + t] = (uint16_t)(bq[kk][w] >> 16);
            }
        float dd[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) dd[s] = __shfl(dden, 4 * gq + s, 64);
        const uint32_t d01 = pack_bf16(dd[0], dd[1]), d23 = pack_bf16(dd[2], dd[3]);
        const u32x2 dhi = u32x2{d01, d23};
        const u32x2 dlo = u32x2{pack_bf16(dd[0] - bf_lo(d01), dd[1] - bf_hi(d01)),
                                pack_bf16(dd[2] - bf_lo(d23), dd[3] - bf_hi(d23))};
        u32x2 bu[RT];
#pragma unroll
        for (int rc = 0; rc < RT; ++rc) bu[rc] = *reinterpret_cast<const u32x2*>(uT + (16 * rc + t) * TS + 4 * gq);
#pragma unroll
        for (int re = 0; re < RT; ++re) {
            const u32x2 an = *reinterpret_cast<const u32x2*>(dnT + (16 * re + t) * TS + 4 * gq);
#pragma unroll
            for (int rc = 0; rc < RT; ++rc) dsacc[re][rc] = mfma_k16(an, bu[rc], dsacc[re][rc]);
        }
#pragma unroll
        for (int rc = 0; rc < RT; ++rc) {
            dzacc[rc] = mfma_k16(dhi, bu[rc], dzacc[rc]);
            dzacc[rc] = mfma_k16(dlo, bu[rc], dzacc[rc]);
        }
    };
    // The next group's loads are in flight while this one is computed.
    // d = 32: two later groups in flight (sana-128x128 query side 164 -> 154 us).
    if (gr0 < gr1) pipelined<D == 32 ? 2 : 1, Raw>(gr0, 1, gr1, load, compute);

    if (g.AP > 1) {
        // ---- this part's fp32 partial record (zeros for an empty part)
        float* recf = dpart + ((size_t)blk * g.AP + wgc.t) * REC;
#pragma unroll
        for (int re = 0; re < RT; ++re)
#pragma unroll
            for (int rc = 0; rc < RT; ++rc)
#pragma unroll
                for (int v = 0; v < 4; ++v) recf[(16 * re + 4 * gq + v) * D + 16 * rc + t] = dsacc[re][rc][v];
        if (gq == 0) {
#pragma unroll
            for (int rc = 0; rc < RT; ++rc) recf[D * D + 16 * rc + t] = dzacc[rc][0];
        }
        return;
    }
    // ---- the block's record: dSt as [e][c] (element (c, e) at e*D + c), then dzt[c].
    uint16_t* rec = dSt + (size_t)blk * REC;
#pragma unroll
    for (int re = 0; re < RT; ++re)
#pragma unroll
        for (int rc = 0; rc < RT; ++rc)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int e = 16 * re + 4 * gq + v, c = 16 * rc + t;
                rec[e * D + c] = (uint16_t)(pack_bf16(dsacc[re][rc][v], 0.f) & 0xffffu);
            }
    if (gq == 0) {
#pragma unroll
        for (int rc = 0; rc < RT; ++rc) rec[D * D + 16 * rc + t] = (uint16_t)(pack_bf16(dzacc[rc][0], 0.f) & 0xffffu);
    }
}

// dW for M <= 64: one 64 x 64 tile; the workgroup's eight waves are four
// k-groups x two row halves (wave w: rows 32 (w & 1) .., all 64 columns), and
// the four k-groups' partial tiles are added in k-group order through LDS.
// The operands go through LDS four k-steps (128 record elements, two lines per
// record row) at a time, loaded by sixteen consecutive threads per row; in
// each stage k-group g multiplies its k-step g.  Rows past M load a valid row;
// their outputs are computed and not stored.
template <int D>
__global__ __launch_bounds__(512) void dw_partial_small_bf16(const uint16_t* __restrict__ dSt,
                                                             const uint16_t* __restrict__ SZ, float* __restrict__ part,
                                                             int M, int P, int nsplit) {
    constexpr int REC = D * D + D, KPR = REC / 32;
    constexpr int KST = 4;                 // k-steps per stage, one per k-group
    constexpr int SROW = 32 * KST + 8;     // LDS row: 128 elements + 8 padding (272 bytes)
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][64 * SROW];   // [buffer][dSt, S][row]: 68 KB
    __shared__ f32x4 red[3][2][2][4][64];   // k-groups 1..3 x row half x acc[2][4] x lane: 48 KB
    const int s = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, gq = lane >> 4;
    const int half = wave & 1, kg = wave >> 1;
    const int i0 = 32 * half;
    // staging role: rows srow and srow + 32 of both operands, 16-byte piece pc of the stage's 256 bytes
    const int srow = tid >> 4, pc = tid & 15;
    int rr[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) rr[p] = min(srow + 32 * p, M - 1) * REC;
    const int nks = P * KPR, per = (nks + nsplit - 1) / nsplit;
    const int k0 = min(nks, s * per), k1 = min(nks, k0 + per);
    const int nst = (k1 - k0 + KST - 1) / KST;

    struct Regs {
        u32x4 a[2], b[2];
    };
    // Stage st: k-steps k0 + KST st + (pc >> 2); a k-step past k1 stages zeros.
    auto load = [&](int st, Regs& r) {
        const int ks = k0 + KST * st + (pc >> 2);
        const bool ok = ks < k1;
        const int kc = ok ? ks : k0;
        const int bh = kc / KPR, col = (kc - bh * KPR) * 32 + (pc & 3) * 8;
        const size_t base = (size_t)bh * M * REC + col;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(dSt + base + rr[p]);
            const u32x4 y = *reinterpret_cast<const u32x4*>(SZ + base + rr[p]);
            r.a[p] = ok ? x : u32x4{0u, 0u, 0u, 0u};
            r.b[p] = ok ? y : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](int buf, const Regs& r) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            *reinterpret_cast<u32x4*>(&lds[buf][0][(srow + 32 * p) * SROW + pc * 8]) = r.a[p];
            *reinterpret_cast<u32x4*>(&lds[buf][1][(srow + 32 * p) * SROW + pc * 8]) = r.b[p];
        }
    };
    f32x4 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf) {
        const uint16_t* la = &lds[buf][0][(i0 + li) * SROW + 32 * kg + gq * 8];
        const uint16_t* lb = &lds[buf][1][li * SROW + 32 * kg + gq * 8];
        u32x4 A[2], B[4];
#pragma unroll
        for (int a = 0; a < 2; ++a) A[a] = *reinterpret_cast<const u32x4*>(la + 16 * a * SROW);
#pragma unroll
        for (int c = 0; c < 4; ++c) B[c] = *reinterpret_cast<const u32x4*>(lb + 16 * c * SROW);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[a][c] = mfma_bf16(A[a], B[c], acc[a][c]);
    };
    if (nst > 0) {
        Regs r0, r1;
        load(0, r0);
        if (nst > 1) load(1, r1);
        store(0, r0);
        __syncthreads();
        // Stage st is in buffer st & 1; the register set of stage st + 1 is
        // stored after stage st is multiplied, and stage st + 2 loads into the
        // set just freed.
        for (int st = 0; st < nst; st += 2) {
            if (st + 2 < nst) load(st + 2, r0);
            compute(0);
            if (st + 1 >= nst) break;
            store(1, r1);
            __syncthreads();
            if (st + 3 < nst) load(st + 3, r1);
            compute(1);
            if (st + 2 >= nst) break;
            store(0, r0);
            __syncthreads();
        }
    }
    if (kg > 0) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) red[kg - 1][half][a][c][lane] = acc[a][c];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[a][c] += red[q][half][a][c][lane];
    float* out = part + (size_t)s * M * M;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = i0 + 16 * a + 4 * gq + v, jj = 16 * c + li;
                if (i < M && jj < M) out[(size_t)i * M + jj] = acc[a][c][v];
            }
}

// The token parts' partial records [nrec][parts][rec] (fp32 or bf16) added in
// part order in fp32 and rounded to bf16 records [nrec][rec].
__device__ __forceinline__ float as_f32(float x) { return x; }
__device__ __forceinline__ float as_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
template <typename T>
__global__ __launch_bounds__(256) void fold_parts_bf16(const T* __restrict__ part, uint16_t* __restrict__ out,
                                                       int nrec, int parts, int rec) {
    const size_t x = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= (size_t)nrec * rec) return;
    const size_t r = x / rec, e = x - r * rec;
    const T* src = part + r * parts * rec + e;
    float sum = 0.f;
    for (int t = 0; t < parts; ++t) sum += as_f32(src[(size_t)t * rec]);
    out[x] = (uint16_t)(pack_bf16(sum, 0.f) & 0xffffu);
}

// dW[x] = the sum of the split partials part[0..nsplit)[x] in split order,
// eight loads in flight per thread.
__device__ __forceinline__ float dw_sum(const float* __restrict__ part, int x, int MM, int nsplit) {
    float s = 0.f;
    int k = 0;
    for (; k + 8 <= nsplit; k += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(k + u) * MM + x];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; k < nsplit; ++k) s += part[(size_t)k * MM + x];
    return s;
}

// =====================================================================
// bwd_kv: dv and dk per source block.  Workgroup = (b, block j, group of
// <= 8 heads), one wave per head over the block's tokens, 16 per step:
//   dv = dS^T a (rows e, k = c: the record's own layout),
//   dk = (dS v + dz) * phi'(k) (rows c, k = e: the transposed operand).
// =====================================================================
// PAIR (D = 64 only): the problem has head_dim 32 and an even head count; a
// wave takes heads 2p and 2p + 1 as one head of 64 channels whose dS is the
// block-diagonal matrix of the two heads' dS (zeros between the heads) and
// whose dz is the two heads' dz, which gives each head's dk and dv exactly.
template <int D, bool PAIR = false>
__global__ __launch_bounds__(512) void bwd_kv_bf16(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                   const uint16_t* __restrict__ dS, const float* __restrict__ dZ,
                                                   uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                                   const Geo g, const float* __restrict__ part,
                                                   float* __restrict__ dW, int MM, int nsplit, int nkv) {
    // Workgroups from nkv on reduce dW's split partials (independent of the
    // key/value gradients; they run beside them instead of in a launch of their own).
    if ((int)blockIdx.x >= nkv) {
        const int x = ((int)blockIdx.x - nkv) * (int)blockDim.x + (int)threadIdx.x;
        if (x < MM) dW[x] = dw_sum(part, x, MM, nsplit);
        return;
    }
    constexpr int RT = D / 16, KS = D / 32;
    constexpr int OSTR = D + 8;
    // per wave: the output staging of 16 token rows; first the summary tile [D][OSTR]
    constexpr int SLICE = PAIR ? 16 * OSTR : D * OSTR;
    __shared__ __attribute__((aligned(16))) uint16_t lds[8 * SLICE];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = lane & 15, gq = lane >> 4;
    // Workgroup = (b, block j, token part, head group): part t takes a
    // contiguous run of the block's 16-token groups (g.AP runs; one when the
    // problem has blocks enough).
    const WgCoordP wgc = wg_coord_parts(g, blockIdx.x, g.div_AP);
    const int hh = wgc.hg * g.G + wave;
    if (hh >= g.H) return;
    const int b = __builtin_amdgcn_readfirstlane(wgc.b);
    const int h = __builtin_amdgcn_readfirstlane(hh);
    const int j = __builtin_amdgcn_readfirstlane(wgc.j);
    const int ngr = (g.T + 15) >> 4, gper = (ngr + g.AP - 1) / g.AP;
    const int gr0 = __builtin_amdgcn_readfirstlane(min(ngr, gper * wgc.t));
    const int gr1 = min(ngr, gr0 + gper);
    if (gr0 >= gr1) return;
    const int blk = (b * g.H + h) * g.M + j;
    uint16_t* sout = lds + wave * SLICE;

    static_assert(!PAIR || D == 64, "paired heads run the 64-channel layout");
    const uint16_t* mb = dS + (size_t)blk * (D * D);
    u32x4 a3[RT][KS], a4[RT][KS];
    float dzc[4 * RT];
    if constexpr (PAIR) {
        // Records of the two heads (head_dim 32); channel x of the pair is
        // channel x % 32 of head x / 32.
        constexpr int DH = 32;
        const int Hr = 2 * g.H;
        const uint16_t* mp[2];
        const float* zp[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const size_t rec = (size_t)(b * Hr + 2 * h + s2) * g.M + j;
            mp[s2] = dS + rec * (DH * DH);
            zp[s2] = dZ + rec * DH;
        }
        // a3: row e, k = c (8 consecutive c of head kk per lane group)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int e = 4 * RT * (t >> 2) + 4 * r + (t & 3);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(mp[kk] + (e & 31) * DH + gq * 8);
                const uint32_t m = (e >> 5) == kk ? 0xffffffffu : 0u;
                a3[r][kk] = u32x4{x[0] & m, x[1] & m, x[2] & m, x[3] & m};
            }
        }
        // a4: row c, k-slot s of k-step kk at e = kk*32 + gq*8 + s (head kk)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int c = 4 * RT * (t >> 2) + 4 * rt + (t & 3);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const bool same = (c >> 5) == kk;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int e0 = gq * 8 + 2 * w;   // within head kk
                    const uint32_t lo = mp[kk][e0 * DH + (c & 31)], hi = mp[kk][(e0 + 1) * DH + (c & 31)];
                    a4[rt][kk][w] = same ? (lo | (hi << 16)) : 0u;
                }
            }
        }
        // dz of channels 4*RT*gq .. +4*RT-1 (all in head gq / 2)
        const float* zb = zp[gq >> 1] + 4 * RT * (gq & 1);
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(zb + 4 * u);
            dzc[4 * u] = x.x; dzc[4 * u + 1] = x.y; dzc[4 * u + 2] = x.z; dzc[4 * u + 3] = x.w;
        }
    } else {
    // The D x D tile read with whole-line loads into the wave's slice, then
    // gathered in both operand layouts (read straight in those layouts,
    // consecutive lanes would address rows D elements apart).
#pragma unroll
    for (int p = 0; p < D * D / 512; ++p) {
        const int x = p * 64 + lane, e = x / (D / 8), c8 = x % (D / 8);
        *reinterpret_cast<u32x4*>(sout + e * OSTR + 8 * c8) = *reinterpret_cast<const u32x4*>(mb + e * D + 8 * c8);
    }
    // a3: row e = 4*RT*(t/4) + 4r + t%4, k = c = 4*RT*gq + 8*kk + s
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int e = 4 * RT * (t >> 2) + 4 * r + (t & 3);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            a3[r][kk] = *reinterpret_cast<const u32x4*>(sout + e * OSTR + 4 * RT * gq + 8 * kk);
    }
    // a4: row c, k-slot s of k-step kk at e = kk*32 + gq*8 + s (the layout V is loaded in).
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int c = 4 * RT * (t >> 2) + 4 * rt + (t & 3);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int e0 = kk * 32 + gq * 8 + 2 * w;
                a4[rt][kk][w] = (uint32_t)sout[e0 * OSTR + c] | ((uint32_t)sout[(e0 + 1) * OSTR + c] << 16);
            }
    }
    // (the wave's LDS operations run in order: the tile is read before the output staging overwrites it)
    const float* zb = dZ + (size_t)blk * D;
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(zb + 4 * RT * gq + 4 * u);
        dzc[4 * u] = x.x; dzc[4 * u + 1] = x.y; dzc[4 * u + 2] = x.z; dzc[4 * u + 3] = x.w;
    }
    }

    const int row = g.H * D;
    const int origin = block_origin(g, j);
    const size_t bbase = (size_t)b * g.N * row + h * D;
    const uint16_t* kb = K + bbase;
    const uint16_t* vb = V + bbase;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(dK + (size_t)b * g.N * row, 0,
                                                                        g.N * row * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(dV + (size_t)b * g.N * row, 0,
                                                                        g.N * row * 2, 0x00020000);
    const int olane = h * D * 2;

    // Without head pairs phi(k) enters the dv product with k-slots c =
    // 4*RT*gq + 8*kk + s, the channels of this lane's dk, so phi'(k) there
    // shares its exponential and k is loaded once.  Head pairs keep k-slots
    // kk*32 + 8*gq + s (one head per k-step, the same sums as one head per
    // wave) and load k again at the dk channels.
    struct Raw {
        u32x4 kv[KS], vv[KS], ko[PAIR ? RT / 2 : 1];
        int off;
        bool ok;
    };
    auto load = [&](int it, Raw& R) {
        const int p = it * 16 + t;
        R.ok = p < g.T;
        R.off = (origin + in_block(g, R.ok ? p : g.T - 1)) * row;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            R.kv[kk] = *reinterpret_cast<const u32x4*>(kb + R.off + (PAIR ? kk * 32 + gq * 8 : 4 * RT * gq + 8 * kk));
            R.vv[kk] = *reinterpret_cast<const u32x4*>(vb + R.off + kk * 32 + gq * 8);
        }
        if constexpr (PAIR) {
#pragma unroll
            for (int u = 0; u < RT / 2; ++u)
                R.ko[u] = *reinterpret_cast<const u32x4*>(kb + R.off + 4 * RT * gq + 8 * u);
        }
    };
    auto compute = [&](const Raw& R) {
        // with e = exp(min(x, 0)): phi(x) = max(x, 0) + e, phi'(x) = e
        u32x4 ba[KS];
        float pg[4 * RT];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float x0 = bf_lo(R.kv[kk][w]), x1 = bf_hi(R.kv[kk][w]);
                const float e0 = __expf(fminf(x0, 0.f)), e1 = __expf(fminf(x1, 0.f));
                ba[kk][w] = pack_bf16(fmaxf(x0, 0.f) + e0, fmaxf(x1, 0.f) + e1);
                pg[8 * kk + 2 * w] = e0;
                pg[8 * kk + 2 * w + 1] = e1;
            }
        if constexpr (PAIR) {
            float kl[4 * RT];
#pragma unroll
            for (int u = 0; u < RT / 2; ++u) unpack8(R.ko[u], kl + 8 * u);
#pragma unroll
            for (int cl = 0; cl < 4 * RT; ++cl) pg[cl] = phi_grad(kl[cl]);
        }
        f32x4 accv[RT], acck[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            accv[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            acck[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                accv[r] = mfma_bf16(a3[r][kk], ba[kk], accv[r]);
                acck[r] = mfma_bf16(a4[r][kk], R.vv[kk], acck[r]);
            }
        uint32_t wv[2 * RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            wv[2 * r] = pack_bf16(accv[r][0], accv[r][1]);
            wv[2 * r + 1] = pack_bf16(accv[r][2], accv[r][3]);
        }
        store_rows<D>(sout, wv, lane, R.off, R.ok, rv, olane);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            float x[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int cl = 4 * r + v;
                x[v] = (acck[r][v] + dzc[cl]) * pg[cl];
            }
            wv[2 * r] = pack_bf16(x[0], x[1]);
            wv[2 * r + 1] = pack_bf16(x[2], x[3]);
        }
        store_rows<D>(sout, wv, lane, R.off, R.ok, rk, olane);
    };
    // The next group's loads are in flight while this one is computed.
    pipelined<1, Raw>(gr0, 1, gr1, load, compute);
}

// =====================================================================
// dW = sum over (b, h) and record elements of dSt_i[x] S_j[x]: a GEMM whose
// k runs over B*H*(d*d + d).  Workgroup = (split s of the k-steps, 128 x 128
// tile of dW); split s is a contiguous run of k-steps, and blockIdx.x = s puts
// every tile of one split on the same XCD (workgroups are dealt to the XCDs by
// linear index), where they share the records in L2.  The operands go through
// LDS two k-steps (64 record elements) at a time: eight consecutive threads
// load the 128 bytes of one record row, so the loads are whole lines that the
// L1 serves four lanes per access (loaded straight into the MFMA layout,
// consecutive lanes would read rows a record apart, one access per lane).  The
// loads of the next two stages are in flight while one is multiplied.  Wave
// (wi, wj) computes 32 i x 64 j.  Rows past M load a valid row; their outputs
// are computed and not stored (each output element depends only on its own
// rows).  Partial sums go to part[s]; dw_sum adds them in split order.
// =====================================================================
constexpr int DW_SROW = 72;                              // LDS row: 64 elements + 8 padding (144 bytes)
constexpr int DW_LDS_BYTES = 2 * 2 * 128 * DW_SROW * 2;  // [buffer][dSt, S][row]: 72 KB

template <int D>
__device__ __forceinline__ void dw_tile(int s, int tile, uint16_t* __restrict__ lds_raw,
                                        const uint16_t* __restrict__ dSt, const uint16_t* __restrict__ SZ,
                                        float* __restrict__ part, int M, int P, int nsplit, int ntj) {
    constexpr int REC = D * D + D, KPR = REC / 32;
    constexpr int KST = 2;                // k-steps per stage
    constexpr int SROW = DW_SROW;
    auto lds = reinterpret_cast<uint16_t (*)[2][128 * SROW]>(lds_raw);
    const int ti = tile / ntj, tj = tile - ti * ntj;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, gq = lane >> 4;
    const int i0 = ti * 128 + (wave >> 1) * 32, j0 = tj * 128 + (wave & 1) * 64;
    // staging role: rows srow and srow + 64 of both tiles, 16-byte piece pc of the stage's 128 bytes
    const int srow = tid >> 3, pc = tid & 7;
    int ra[2], rb[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        ra[p] = min(ti * 128 + srow + 64 * p, M - 1) * REC;
        rb[p] = min(tj * 128 + srow + 64 * p, M - 1) * REC;
    }
    const int nks = P * KPR, per = (nks + nsplit - 1) / nsplit;
    const int k0 = min(nks, s * per), k1 = min(nks, k0 + per);
    const int nst = (k1 - k0 + KST - 1) / KST;

    struct Regs {
        u32x4 a[2], b[2];
    };
    // Stage st: k-steps k0 + KST st + (pc >> 2); a k-step past k1 stages zeros.
    auto load = [&](int st, Regs& r) {
        const int ks = k0 + KST * st + (pc >> 2);
        const bool ok = ks < k1;
        const int kc = ok ? ks : k0;
        const int bh = kc / KPR, col = (kc - bh * KPR) * 32 + (pc & 3) * 8;
        const size_t base = (size_t)bh * M * REC + col;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(dSt + base + ra[p]);
            const u32x4 y = *reinterpret_cast<const u32x4*>(SZ + base + rb[p]);
            r.a[p] = ok ? x : u32x4{0u, 0u, 0u, 0u};
            r.b[p] = ok ? y : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](int buf, const Regs& r) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            *reinterpret_cast<u32x4*>(&lds[buf][0][(srow + 64 * p) * SROW + pc * 8]) = r.a[p];
            *reinterpret_cast<u32x4*>(&lds[buf][1][(srow + 64 * p) * SROW + pc * 8]) = r.b[p];
        }
    };
    f32x4 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf) {
        const uint16_t* la = &lds[buf][0][((wave >> 1) * 32 + li) * SROW + gq * 8];
        const uint16_t* lb = &lds[buf][1][((wave & 1) * 64 + li) * SROW + gq * 8];
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) {
            u32x4 A[2], B[4];
#pragma unroll
            for (int a = 0; a < 2; ++a) A[a] = *reinterpret_cast<const u32x4*>(la + 16 * a * SROW + 32 * kk);
#pragma unroll
            for (int c = 0; c < 4; ++c) B[c] = *reinterpret_cast<const u32x4*>(lb + 16 * c * SROW + 32 * kk);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[a][c] = mfma_bf16(A[a], B[c], acc[a][c]);
        }
    };
    if (nst > 0) {
        Regs r0, r1;
        load(0, r0);
        if (nst > 1) load(1, r1);
        store(0, r0);
        __syncthreads();
        // Stage st is in buffer st & 1; the register set of stage st + 1 is
        // stored after stage st is multiplied, and stage st + 2 loads into the
        // set just freed.
        for (int st = 0; st < nst; st += 2) {
            if (st + 2 < nst) load(st + 2, r0);
            compute(0);
            if (st + 1 >= nst) break;
            store(1, r1);
            __syncthreads();
            if (st + 3 < nst) load(st + 3, r1);
            compute(1);
            if (st + 2 >= nst) break;
            store(0, r0);
            __syncthreads();
        }
    }
    float* out = part + (size_t)s * M * M;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = i0 + 16 * a + 4 * gq + v, jj = j0 + 16 * c + li;
                if (i < M && jj < M) out[(size_t)i * M + jj] = acc[a][c][v];
            }
}

template <int D>
__global__ __launch_bounds__(512) void dw_partial_bf16(const uint16_t* __restrict__ dSt,
                                                       const uint16_t* __restrict__ SZ, float* __restrict__ part,
                                                       int M, int P, int nsplit, int ntj) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[DW_LDS_BYTES / 2];
    dw_tile<D>(blockIdx.x, blockIdx.y, lds, dSt, SZ, part, M, P, nsplit, ntj);
}

// The gradient records mixed with W^T (dS, dz of every block) and dW's partial
// products are independent, so one launch runs both: workgroups [0, ndw) are
// dW tiles (as dw_partial), the rest mix one column tile of 64 record
// elements of one (b, h) for all query blocks: wave w takes blocks 32 w ..
// 32 w + 31 with its W operands in registers, the column tile of every source
// record is staged once for the eight waves (the split mixing kernel's
// operand packing and output mapping).  At most 256 blocks.
template <int D, int NT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void mix_dw_bf16(
    const uint16_t* __restrict__ dSt, const uint16_t* __restrict__ SZ, float* __restrict__ part, int nsplit, int ntj,
    int ndw, const uint16_t* __restrict__ Wb, uint16_t* __restrict__ dS, float* __restrict__ dZ, const Geo g, int CT,
    int CW) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[DW_LDS_BYTES / 2];
    const int id = blockIdx.x;
    if (id < ndw) {
        dw_tile<D>(id % nsplit, id / nsplit, lds, dSt, SZ, part, g.M, g.BH, nsplit, ntj);
        return;
    }
    constexpr int REC = D * D + D, KMAX = 8, OROW = MIX_OROW, ROWS = 32;
    u32x4* sA = reinterpret_cast<u32x4*>(lds);   // [r][kk][lane] operands, 32 KB; then output staging
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, gq = lane >> 4;
    // this workgroup: column tiles ct0 .. ct0 + CW - 1 (those below CT) of pair bh
    const int CTP = (CT + CW - 1) / CW, c = id - ndw;
    const int bh = c / CTP, ct0 = (c - bh * CTP) * CW;
    const int M = g.M, NK = (M + 31) >> 5;
    const int i0 = wave * ROWS;
    const bool active = i0 < M;                  // then i0 + 32 <= roundup(M, 32): inside Wb's rows
    const int rt0 = active ? i0 >> 4 : 0;
    // W operands, loaded once for the workgroup's column tiles
    u32x4 bw[KMAX][2];
#pragma unroll
    for (int kk = 0; kk < KMAX; ++kk)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            bw[kk][t] = *reinterpret_cast<const u32x4*>(
                Wb + ((size_t)((rt0 + t) * NK + (kk < NK ? kk : NK - 1)) * 64 + lane) * 8);
    // staging of a column tile: unit (li', group of 8 source records) -> 4 packed operands, one per thread
    const int units = 16 * 4 * NK;
    const uint16_t* base = dSt + (size_t)bh * M * REC;
    auto load_raw = [&](int cp0, u32x2* raw) {
        const int u = tid;
        const int colp = cp0 + 4 * (u & 15);
        const bool ok = u < units && colp < REC;
        const int colc = ok ? colp : 0;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int jj = 8 * (u >> 4) + s;
            const u32x2 t = *reinterpret_cast<const u32x2*>(base + (size_t)(jj < M ? jj : M - 1) * REC + colc);
            const uint32_t m = (ok && jj < M) ? 0xffffffffu : 0u;
            raw[s] = u32x2{t.x & m, t.y & m};
        }
    };
    auto store_op = [&](const u32x2* raw) {
        const int u = tid;
        if (u < units) {
            const int jg = u >> 4, kk = jg >> 2, lanep = (jg & 3) * 16 + (u & 15);
            u32x4 op[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                op[0][w] = pack_lo(raw[2 * w].x, raw[2 * w + 1].x);
                op[1][w] = pack_hi(raw[2 * w].x, raw[2 * w + 1].x);
                op[2][w] = pack_lo(raw[2 * w].y, raw[2 * w + 1].y);
                op[3][w] = pack_hi(raw[2 * w].y, raw[2 * w + 1].y);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sA[(r * NK + kk) * 64 + lanep] = op[r];
        }
    };
    u32x2 raw[8];
    load_raw(ct0 * 64, raw);
    for (int q = 0; q < CW; ++q) {
        const int ct = ct0 + q;
        if (ct >= CT) break;                     // the same for the whole workgroup
        const int cp0 = ct * 64;
        if (q > 0) __syncthreads();              // the last tile's output staging (over sA) is done
        store_op(raw);
        if (q + 1 < CW && ct + 1 < CT) load_raw(cp0 + 64, raw);   // the next tile's records in flight
        __syncthreads();
        f32x4 acc[4][2];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][0] = acc[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (active) {
#pragma unroll
            for (int kk = 0; kk < KMAX; ++kk) {
                if (kk >= NK) break;
                u32x4 a[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] = sA[(r * NK + kk) * 64 + lane];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int t = 0; t < 2; ++t) acc[r][t] = mfma_bf16(a[r], bw[kk][t], acc[r][t]);
            }
        }
        __syncthreads();   // every wave is done with the A operands
        if (!active) continue;
        // Lane holds C[col' = cp0 + 16*gq + 4*v + r][i = i0 + 16*t + li].
        if (cp0 < D * D) {
            uint16_t* stage = lds + wave * (ROWS * OROW);   // this wave's slice only
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t wv[8];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    wv[2 * v] = pack_bf16(acc[0][t][v], acc[1][t][v]);
                    wv[2 * v + 1] = pack_bf16(acc[2][t][v], acc[3][t][v]);
                }
                uint16_t* dst = stage + (16 * t + li) * OROW + 16 * gq;
                *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
                *reinterpret_cast<u32x4*>(dst + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
            }
#pragma unroll
            for (int k = 0; k < ROWS / 8; ++k) {
                const int rl = 8 * k + (lane >> 3), chunk = lane & 7;
                const int i = i0 + rl;
                const u32x4 x = *reinterpret_cast<const u32x4*>(stage + rl * OROW + chunk * 8);
                u32x4* dst = reinterpret_cast<u32x4*>(dS + ((size_t)bh * M + i) * (D * D) + cp0 + chunk * 8);
                if (i < M) {
                    if constexpr ((NT & 2) != 0) __builtin_nontemporal_store(x, dst);
                    else *dst = x;
                }
            }
        } else if (cp0 + 16 * gq < REC) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int i = i0 + 16 * t + li;
                if (i >= M) continue;
                float* dst = dZ + ((size_t)bh * M + i) * D + (cp0 + 16 * gq - D * D);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    *reinterpret_cast<f32x4*>(dst + 4 * v) =
                        f32x4{acc[0][t][v], acc[1][t][v], acc[2][t][v], acc[3][t][v]};
            }
        }
    }
}

// dW from many split partials: a workgroup takes 16 entries, its 16 lane
// groups a sixteenth of the splits each (in split order), and the 16 group
// sums are added in group order, so each thread's chain of loads is nsplit / 16
// long instead of nsplit.
__global__ __launch_bounds__(256) void dw_reduce_wide(const float* __restrict__ part, float* __restrict__ dW, int MM,
                                                      int nsplit) {
    __shared__ float red[16][17];
    const int xl = threadIdx.x & 15, grp = threadIdx.x >> 4;
    const int x = blockIdx.x * 16 + xl;
    const int per = (nsplit + 15) >> 4;
    const int k0 = min(nsplit, grp * per), k1 = min(nsplit, k0 + per);
    float s = 0.f;
    if (x < MM) {
        int k = k0;
        for (; k + 8 <= k1; k += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(k + u) * MM + x];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; k < k1; ++k) s += part[(size_t)k * MM + x];
    }
    red[grp][xl] = s;
    __syncthreads();
    if (grp == 0 && x < MM) {
        float t = red[0][xl];
#pragma unroll
        for (int q = 1; q < 16; ++q) t += red[q][xl];
        dW[x] = t;
    }
}

inline void rec(const BwdLaunch& B, int k) {
    if (B.events) (void)hipEventRecord(B.events[k], B.F.stream);
}

template <int D>
hipError_t run_bwd_d(const BwdLaunch& B) {
    const Launch& L = B.F;
    const int tp = L.g.TP;   // the recompute's token parts
    // The gradient kernels see one record per block (token parts of the
    // query and key/value sides are set on their own launches below).
    Geo g = L.g;
    g.TP = g.AP = 1;
    g.div_TP = g.div_AP = make_fastdiv(1u);
    rec(B, 0);
    // Forward summaries and mixed summaries (regions 0-3 of the workspace).
    hipError_t err = run_bf16_summaries(L);
    if (err != hipSuccess) return err;
    // In token parts the summaries are partial records; dW reads them folded.
    const uint16_t* srec = static_cast<const uint16_t*>(L.sz);
    if (tp > 1 && B.sfold) {
        const size_t n = (size_t)g.BH * g.M * (D * D + D);
        fold_parts_bf16<uint16_t><<<(unsigned)((n + 255) / 256), 256, 0, L.stream>>>(
            static_cast<const uint16_t*>(L.sz), B.sfold, g.BH * g.M, tp, D * D + D);
        srec = B.sfold;
    }
    rec(B, 1);
    // Head groups: at most `maxw` heads (one wave each) per workgroup, balanced.
    auto heads = [&](int maxw) {
        Geo x = g;
        x.HG = (g.H + maxw - 1) / maxw;
        x.G = (g.H + x.HG - 1) / x.HG;
        x.div_HG = make_fastdiv((uint32_t)x.HG);
        return x;
    };
    // d = 64: one wave per SIMD.  With many (b, block, head) tasks, workgroups
    // of 2 waves keep every SIMD of a compute unit busy where groups of 3 idle
    // one (dit-s2-64x64, 12288 tasks: 188 -> 159 us); with few tasks the
    // larger groups' shared token rows win (dit-s2-256x256, 1536 tasks:
    // groups of 3 heads 73.6 us, of 2 heads 75-78 us).
    const int bq_max = D == 64 ? (g.H % 4 == 0 || g.B * g.M * g.H < 4096 ? 4 : 2) : 8;
    Geo gq = heads(L.tune.bwdq_heads > 0 ? L.tune.bwdq_heads : bq_max);
    gq.AP = B.q_parts > 1 && B.dpart ? B.q_parts : 1;
    gq.div_AP = make_fastdiv((uint32_t)gq.AP);
    if (D == 64 && g.T >= 128)
        bwd_query_bf16<D, true><<<gq.B * gq.M * gq.AP * gq.HG, 64 * gq.G, 0, L.stream>>>(
            static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(B.dout), static_cast<const uint16_t*>(L.st),
            L.zt, static_cast<uint16_t*>(B.dq), B.dst, B.dpart, gq);
    else
        bwd_query_bf16<D, false><<<gq.B * gq.M * gq.AP * gq.HG, 64 * gq.G, 0, L.stream>>>(
            static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(B.dout), static_cast<const uint16_t*>(L.st),
            L.zt, static_cast<uint16_t*>(B.dq), B.dst, B.dpart, gq);
    if (gq.AP > 1) {
        const size_t n = (size_t)g.BH * g.M * (D * D + D);
        fold_parts_bf16<float><<<(unsigned)((n + 255) / 256), 256, 0, L.stream>>>(B.dpart, B.dst, g.BH * g.M, gq.AP,
                                                                                  D * D + D);
    }
    Geo gh = heads(8);
    // bwd_kv: each block's tokens in token parts (dk, dv of a token depend only
    // on its block's dS, dz), as many as the forward's apply uses.
    gh.AP = B.kv_parts > 0 ? B.kv_parts : 1;
    gh.div_AP = make_fastdiv((uint32_t)gh.AP);
    const int grid_tok = gh.B * gh.M * gh.AP * gh.HG, block_tok = 64 * gh.G;
    rec(B, 2);
    err = launch_mix_dw_bf16(B, g, srec);
    if (err != hipSuccess) return err;
    // dW's split partials are summed by extra workgroups at the end of the
    // key/value launch while each thread's chain of loads is short (dit-s2-256x256,
    // 32 splits: 152.5 -> 150.1 us per step); a long chain (dit-s2-64x64, 256
    // splits of 4096 entries) would start last and outlast the key/value
    // workgroups, so it keeps a launch of its own.
    const int MM = g.M * g.M;
    const bool reduce_in_kv = B.nsplit <= 64;
    if (!reduce_in_kv) dw_reduce_wide<<<(MM + 15) / 16, 256, 0, L.stream>>>(B.part, B.dw, MM, B.nsplit);
    rec(B, 3);
    bool paired = false;
    if constexpr (D == 32) {
        if (g.H % 2 == 0 && L.tune.pair_heads) {
            // head pairs read as heads of 64 channels (whole 128-byte rows per lane group)
            Geo gp = g;
            gp.H = g.H / 2;
            gp.D = 64;
            gp.BH = g.B * gp.H;
            gp.HG = (gp.H + 7) / 8;
            gp.G = (gp.H + gp.HG - 1) / gp.HG;
            gp.div_HG = make_fastdiv((uint32_t)gp.HG);
            gp.AP = gh.AP;
            gp.div_AP = gh.div_AP;
            const int nkv = gp.B * gp.M * gp.AP * gp.HG, blk = 64 * gp.G;
            bwd_kv_bf16<64, true><<<nkv + (reduce_in_kv ? (MM + blk - 1) / blk : 0), blk, 0, L.stream>>>(
                static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v), B.ds, B.dz,
                static_cast<uint16_t*>(B.dk), static_cast<uint16_t*>(B.dv), gp, B.part, B.dw, MM, B.nsplit, nkv);
            paired = true;
        }
    }
    if (!paired)
        bwd_kv_bf16<D><<<grid_tok + (reduce_in_kv ? (MM + block_tok - 1) / block_tok : 0), block_tok, 0, L.stream>>>(
            static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v), B.ds, B.dz,
            static_cast<uint16_t*>(B.dk), static_cast<uint16_t*>(B.dv), gh, B.part, B.dw, MM, B.nsplit, grid_tok);
    rec(B, 4);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero(float* __restrict__ p, int n) {
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x < n) p[x] = 0.f;
}

}  // namespace

hipError_t launch_mix_dw_bf16(const BwdLaunch& B, const Geo& g, const uint16_t* srec) {
    const Launch& L = B.F;
    const int ntj = (g.M + 127) / 128;
    if (g.M > 128 && g.M <= 256 && L.tune.mix_kind != 0 && L.tune.bwd_fuse) {
        // the gradient records' W^T mixing and dW's partial products in one launch
        auto go = [&](auto d) {
            constexpr int D = decltype(d)::value;
            const int CT = (D * D + D + 63) / 64, ndw = B.nsplit * ntj * ntj;
            // Column tiles per mixing workgroup, which loads its W operands once for
            // them: with many tiles, fewer and longer workgroups (sana-128x128,
            // 2380 tiles: 1, 2, 3, 4, 6, 9 per workgroup 117.7, 116.0, 113.0,
            // 111.9, 115.3, 125.7 us for the stage); dit-s2-256x256's 396 the same.
            const int CW = std::max(1, std::min(4, g.BH * CT / 512));
            const int grid = ndw + g.BH * ((CT + CW - 1) / CW);
            if (L.tune.nt_mix & 2)
                mix_dw_bf16<D, 2><<<grid, 512, 0, L.stream>>>(B.dst, srec, B.part, B.nsplit, ntj, ndw, B.wbt, B.ds,
                                                               B.dz, g, CT, CW);
            else
                mix_dw_bf16<D, 0><<<grid, 512, 0, L.stream>>>(B.dst, srec, B.part, B.nsplit, ntj, ndw, B.wbt, B.ds,
                                                               B.dz, g, CT, CW);
        };
        switch (g.D) {
            case 32: go(std::integral_constant<int, 32>{}); break;
            case 64: go(std::integral_constant<int, 64>{}); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    // the gradient records mixed with W^T on the forward's mixing kernels, then dW's partials
    const hipError_t err = launch_mix_records_bf16(L, B.dst, B.wbt, B.ds, B.dz, g);
    if (err != hipSuccess) return err;
    auto go = [&](auto d) {
        constexpr int D = decltype(d)::value;
        if (g.M <= 64)
            dw_partial_small_bf16<D><<<B.nsplit, 512, 0, L.stream>>>(B.dst, srec, B.part, g.M, g.BH, B.nsplit);
        else
            dw_partial_bf16<D><<<dim3(B.nsplit, ntj * ntj), 512, 0, L.stream>>>(B.dst, srec, B.part, g.M, g.BH,
                                                                                B.nsplit, ntj);
    };
    switch (g.D) {
        case 32: go(std::integral_constant<int, 32>{}); break;
        case 64: go(std::integral_constant<int, 64>{}); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t zero_f32(float* p, int n, hipStream_t stream) {
    if (n > 0) fill_zero<<<(n + 255) / 256, 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

hipError_t run_bwd_bf16(const BwdLaunch& B) {
    switch (B.F.g.D) {
        case 32: return run_bwd_d<32>(B);
        case 64: return run_bwd_d<64>(B);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mhla
