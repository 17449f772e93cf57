// kernels_bf16.hip -- MHLA forward for bfloat16 inputs on gfx950 (MI355X).
//
// Three kernels follow the method's blockwise evaluation (MHLA,
// arXiv 2601.07832; paperlayer.ai summary, section 4 "Architecture",
// "Multi-Head Mixing", "Efficiency"):
//   block_kv_summary  S_j = phi(K_j)^T V_j and z_j = sum phi(k)   (one block per workgroup)
//   mix_summaries     [St|zt]_i = sum_j W[i,j] [S|z]_j            (a GEMM over blocks)
//   query_apply       o = phi(q) St_i / (phi(q) . zt_i + eps)      (one block per workgroup)
// plus query_apply_fused, which forms St_i inside the apply workgroup.
//
// All products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  The
// MFMA contracts over the k-slots each lane supplies; both operands of one
// instruction take the same (lane group, slot) -> k assignment, so any
// bijection between k and tokens (or blocks) is valid.  The kernels use that
// freedom to let every lane load a contiguous run of channels of 8 different
// tokens and transpose it in registers while converting to bf16 pairs, which
// keeps global loads coalesced without an LDS round trip.
//
// Output layout of a 16x16 MFMA tile (f32x4 per lane): lane l holds rows
// 4*(l/16) + v, v = 0..3, of column l % 16.
#include "launch.h"

#include <mhla.h>

namespace mhla {
namespace {

// =====================================================================
// block_kv_summary
// Workgroup = one (b, h, j) block, NQ x NWT waves.  A wave owns a 64x64
// (d = 128: one quadrant of S) or 32x32 (d = 32) tile of S and a 1/NWT share
// of the block's tokens; shares are summed through LDS in fixed order.
// Lane (li, gq): K channels CPL*li .. +CPL-1 for rows, V channels likewise
// for columns, tokens 32*ks + 8*gq + s (s = 0..7) as k-slots.
// =====================================================================
template <int D, int NWT>
__global__ __launch_bounds__(64 * NWT * (D == 128 ? 4 : 1)) void block_kv_summary_bf16(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, uint16_t* __restrict__ SZ,
    const Geo g) {
    constexpr int NQ = (D == 128) ? 4 : 1;
    constexpr int CPL = (D == 32) ? 2 : 4;   // channels per lane
    constexpr int CW = CPL / 2;              // 32-bit words per lane per token
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int quad = wave % NQ, tw = wave / NQ;
    const int li = lane & 15, gq = lane >> 4;
    const int blk = blockIdx.x;
    const int bh = (int)fdiv(blk, g.div_M);
    const int j = blk - bh * g.M;
    const int b = (int)fdiv(bh, g.div_H), h = bh - b * g.H;
    const int rowbase = (D == 128) ? (quad >> 1) * 64 : 0;
    const int colbase = (D == 128) ? (quad & 1) * 64 : 0;
    const int row = g.H * D;
    const int origin = block_origin(g, j);
    const uint16_t* kb = K + (b * g.N * row + h * D + rowbase + CPL * li);
    const uint16_t* vb = V + (b * g.N * row + h * D + colbase + CPL * li);

    f32x4 acc[CPL][CPL];
#pragma unroll
    for (int r = 0; r < CPL; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zacc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) zacc[c] = 0.f;

    struct Raw {
        uint32_t k[8][CW], v[8][CW];
        uint32_t valid;
    };
    auto load = [&](int ks, Raw& R) {
        R.valid = 0;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int p = ks * 32 + gq * 8 + s;
            const bool ok = p < g.T;
            const int off = (origin + in_block(g, ok ? p : g.T - 1)) * row;
            R.valid |= (ok ? 1u : 0u) << s;
            if constexpr (CW == 2) {
                const u32x2 a = *reinterpret_cast<const u32x2*>(kb + off);
                const u32x2 c = *reinterpret_cast<const u32x2*>(vb + off);
                R.k[s][0] = a.x; R.k[s][1] = a.y;
                R.v[s][0] = c.x; R.v[s][1] = c.y;
            } else {
                R.k[s][0] = *reinterpret_cast<const uint32_t*>(kb + off);
                R.v[s][0] = *reinterpret_cast<const uint32_t*>(vb + off);
            }
        }
    };
    auto compute = [&](const Raw& R) {
        u32x4 aw[CPL], bw[CPL];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const bool ok0 = (R.valid >> (2 * w)) & 1u, ok1 = (R.valid >> (2 * w + 1)) & 1u;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const uint32_t k0 = R.k[2 * w][c >> 1], k1 = R.k[2 * w + 1][c >> 1];
                const float x0 = (c & 1) ? bf_hi(k0) : bf_lo(k0);
                const float x1 = (c & 1) ? bf_hi(k1) : bf_lo(k1);
                const uint32_t pk = pack_bf16(ok0 ? phi_fast(x0) : 0.f, ok1 ? phi_fast(x1) : 0.f);
                aw[c][w] = pk;
                zacc[c] += bf_lo(pk) + bf_hi(pk);
                const uint32_t v0 = ok0 ? R.v[2 * w][c >> 1] : 0u;
                const uint32_t v1 = ok1 ? R.v[2 * w + 1][c >> 1] : 0u;
                bw[c][w] = (c & 1) ? pack_hi(v0, v1) : pack_lo(v0, v1);
            }
        }
#pragma unroll
        for (int r = 0; r < CPL; ++r)
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[r][c] = mfma_bf16(aw[r], bw[c], acc[r][c]);
    };

    const int nks = (g.T + 31) >> 5;
    Raw ra, rb;
    int ks = tw;
    if (ks < nks) load(ks, ra);
    while (ks < nks) {
        int kn = ks + NWT;
        if (kn < nks) load(kn, rb);
        compute(ra);
        ks = kn;
        if (ks >= nks) break;
        kn = ks + NWT;
        if (kn < nks) load(kn, ra);
        compute(rb);
        ks = kn;
    }

#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        zacc[c] += shfl_xor(zacc[c], 16);
        zacc[c] += shfl_xor(zacc[c], 32);
    }

    if constexpr (NWT > 1) {
        constexpr int NV = CPL * CPL * 4 + CPL;
        __shared__ float red[(NWT - 1) * NQ][NV][64];
        if (tw > 0) {
            float(*dst)[64] = red[(tw - 1) * NQ + quad];
#pragma unroll
            for (int r = 0; r < CPL; ++r)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int v = 0; v < 4; ++v) dst[(r * CPL + c) * 4 + v][lane] = acc[r][c][v];
#pragma unroll
            for (int c = 0; c < CPL; ++c) dst[CPL * CPL * 4 + c][lane] = zacc[c];
        }
        __syncthreads();
        if (tw > 0) return;
#pragma unroll
        for (int t = 0; t < NWT - 1; ++t) {
            float(*src)[64] = red[t * NQ + quad];
#pragma unroll
            for (int r = 0; r < CPL; ++r)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[r][c][v] += src[(r * CPL + c) * 4 + v][lane];
#pragma unroll
            for (int c = 0; c < CPL; ++c) zacc[c] += src[CPL * CPL * 4 + c][lane];
        }
    }

    // Record layout: S_j transposed ([e][c], c fastest), then z_j.
    // Lane holds S[c][e] for c = rowbase + 4*CPL*gq + CPL*v + r, e = colbase + CPL*li + c2.
    uint16_t* rec = SZ + (size_t)blk * (D * D + D);
#pragma unroll
    for (int c2 = 0; c2 < CPL; ++c2) {
        const int e = colbase + CPL * li + c2;
        uint32_t wv[2 * CPL];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int rp = 0; rp < CPL / 2; ++rp)
                wv[v * (CPL / 2) + rp] = pack_bf16(acc[2 * rp][c2][v], acc[2 * rp + 1][c2][v]);
        uint16_t* dst = rec + e * D + rowbase + 4 * CPL * gq;
        *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
        if constexpr (CPL == 4) *reinterpret_cast<u32x4*>(dst + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
    }
    if (gq == 0 && (quad & 1) == 0) {
        uint16_t* dst = rec + D * D + rowbase + CPL * li;
        if constexpr (CPL == 4)
            *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16(zacc[0], zacc[1]), pack_bf16(zacc[2], zacc[3])};
        else
            *reinterpret_cast<uint32_t*>(dst) = pack_bf16(zacc[0], zacc[1]);
    }
}

// =====================================================================
// mix_summaries:  C[col'][i] = sum_j [S|z]_j[col'] W[i][j]  per (b, h).
// A wave computes 64 columns col' of the (d*d + d)-long records for 64
// query blocks i; k runs over source blocks j.  Lane (li, gq): record
// elements 4*li .. +3 of 8 source blocks (rows), W row it*64 + 16*t + li
// (columns).  Mixed S goes out as bf16, mixed z as fp32.
// =====================================================================
template <int D>
__global__ __launch_bounds__(256) void mix_summaries_bf16(const uint16_t* __restrict__ SZ,
                                                          const float* __restrict__ W,
                                                          uint16_t* __restrict__ St,
                                                          float* __restrict__ Zt, const Geo g,
                                                          const FastDiv div_IT, const FastDiv div_CT) {
    constexpr int REC = D * D + D;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, gq = lane >> 4;
    const uint32_t tile = blockIdx.x * 4u + wave;
    const uint32_t rest = fdiv(tile, div_IT);
    const int it = (int)(tile - rest * div_IT.d);
    const uint32_t bh = fdiv(rest, div_CT);
    const int ct = (int)(rest - bh * div_CT.d);
    if ((int)bh >= g.BH) return;
    const int M = g.M;
    const int colp = ct * 64 + 4 * li;
    const bool colok = colp < REC;
    const uint16_t* abase = SZ + (size_t)bh * M * REC + colp;
    const bool wvec = (M & 7) == 0;

    f32x4 acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (M + 31) >> 5;
    for (int kk = 0; kk < nk; ++kk) {
        u32x2 raw[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int jj = kk * 32 + gq * 8 + s;
            raw[s] = (colok && jj < M) ? *reinterpret_cast<const u32x2*>(abase + (size_t)jj * REC)
                                       : u32x2{0u, 0u};
        }
        u32x4 aw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            aw[0][w] = pack_lo(raw[2 * w].x, raw[2 * w + 1].x);
            aw[1][w] = pack_hi(raw[2 * w].x, raw[2 * w + 1].x);
            aw[2][w] = pack_lo(raw[2 * w].y, raw[2 * w + 1].y);
            aw[3][w] = pack_hi(raw[2 * w].y, raw[2 * w + 1].y);
        }
        const int j0 = kk * 32 + gq * 8;
        u32x4 bw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            int i = it * 64 + 16 * t + li;
            i = i < M ? i : M - 1;
            const float* wr = W + (size_t)i * M;
            float wv[8];
            if (wvec) {
                f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f}, y = x;
                if (j0 < M) {
                    x = *reinterpret_cast<const f32x4*>(wr + j0);
                    y = *reinterpret_cast<const f32x4*>(wr + j0 + 4);
                }
                wv[0] = x.x; wv[1] = x.y; wv[2] = x.z; wv[3] = x.w;
                wv[4] = y.x; wv[5] = y.y; wv[6] = y.z; wv[7] = y.w;
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) wv[s] = (j0 + s < M) ? wr[j0 + s] : 0.f;
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) bw[t][w] = pack_bf16(wv[2 * w], wv[2 * w + 1]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[r][t] = mfma_bf16(aw[r], bw[t], acc[r][t]);
    }

    // Lane holds C[col' = ct*64 + 16*gq + 4*v + r][i = it*64 + 16*t + li].
    const int cp0 = ct * 64 + 16 * gq;
    if (cp0 >= REC) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = it * 64 + 16 * t + li;
        if (i >= M) continue;
        const size_t rec = (size_t)bh * M + i;
        if (cp0 < D * D) {
            uint32_t wv[8];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                wv[2 * v] = pack_bf16(acc[0][t][v], acc[1][t][v]);
                wv[2 * v + 1] = pack_bf16(acc[2][t][v], acc[3][t][v]);
            }
            uint16_t* dst = St + rec * (D * D) + cp0;
            *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
            *reinterpret_cast<u32x4*>(dst + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
        } else {
            float* dst = Zt + rec * D + (cp0 - D * D);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                *reinterpret_cast<f32x4*>(dst + 4 * v) = f32x4{acc[0][t][v], acc[1][t][v], acc[2][t][v], acc[3][t][v]};
        }
    }
}

// =====================================================================
// query_apply: O^T = St_i^T phi(Q)^T per 16-token group.
// A = St_i^T (rows e, k = c) stays in registers for the whole block; row ii of
// row-tile r is e = 4*RT*(ii/4) + 4r + ii%4, so each lane ends with 4*RT
// consecutive output channels of one token.  B = phi(q) of 16 tokens, loaded
// straight from Q (8 consecutive channels per lane).  The denominator is a
// per-lane partial dot product reduced over the 4 lane groups.
// =====================================================================
template <int D>
struct ApplyA {
    static constexpr int RT = D / 16, KS = D / 32;
    u32x4 a[RT][KS];
    float zt[KS][8];
};

template <int D, int NWA>
__device__ __forceinline__ void apply_tokens_bf16(const ApplyA<D>& A, const uint16_t* __restrict__ Q,
                                                  uint16_t* __restrict__ O, const Geo& g, int bh,
                                                  int i, int wave, int lane) {
    constexpr int RT = D / 16, KS = D / 32;
    const int t = lane & 15, gq = lane >> 4;
    const int b = (int)fdiv(bh, g.div_H), h = bh - b * g.H;
    const int row = g.H * D;
    const int origin = block_origin(g, i);
    const uint16_t* qb = Q + (b * g.N * row + h * D + gq * 8);
    uint16_t* ob = O + (b * g.N * row + h * D + 4 * RT * gq);
    const int nit = (g.T + 15) >> 4;

    struct Raw {
        u32x4 q[KS];
        int off;
        bool ok;
    };
    auto load = [&](int it, Raw& R) {
        const int p = it * 16 + t;
        R.ok = p < g.T;
        R.off = (origin + in_block(g, R.ok ? p : g.T - 1)) * row;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) R.q[kk] = *reinterpret_cast<const u32x4*>(qb + R.off + kk * 32);
    };
    auto compute = [&](const Raw& R) {
        u32x4 bq[KS];
        float den = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t pk = pack_bf16(phi_fast(bf_lo(R.q[kk][w])), phi_fast(bf_hi(R.q[kk][w])));
                bq[kk][w] = pk;
                den += bf_lo(pk) * A.zt[kk][2 * w] + bf_hi(pk) * A.zt[kk][2 * w + 1];
            }
        f32x4 acc[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int r = 0; r < RT; ++r) acc[r] = mfma_bf16(A.a[r][kk], bq[kk], acc[r]);
        den += shfl_xor(den, 16);
        den += shfl_xor(den, 32);
        const float inv = 1.f / (den + g.eps);
        if (R.ok) {
            uint32_t wv[2 * RT];
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                wv[2 * r] = pack_bf16(acc[r][0] * inv, acc[r][1] * inv);
                wv[2 * r + 1] = pack_bf16(acc[r][2] * inv, acc[r][3] * inv);
            }
#pragma unroll
            for (int u = 0; u < RT / 2; ++u)
                *reinterpret_cast<u32x4*>(ob + R.off + 8 * u) =
                    u32x4{wv[4 * u], wv[4 * u + 1], wv[4 * u + 2], wv[4 * u + 3]};
        }
    };

    Raw ra, rb;
    int it = wave;
    if (it < nit) load(it, ra);
    while (it < nit) {
        int in = it + NWA;
        if (in < nit) load(in, rb);
        compute(ra);
        it = in;
        if (it >= nit) break;
        in = it + NWA;
        if (in < nit) load(in, ra);
        compute(rb);
        it = in;
    }
}

template <int D, int NWA>
__global__ __launch_bounds__(64 * NWA) void query_apply_bf16(const uint16_t* __restrict__ Q,
                                                             const uint16_t* __restrict__ St,
                                                             const float* __restrict__ Zt,
                                                             uint16_t* __restrict__ O, const Geo g) {
    constexpr int RT = D / 16, KS = D / 32;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = lane & 15, gq = lane >> 4;
    const int blk = blockIdx.x;
    const int bh = (int)fdiv(blk, g.div_M);
    const int i = blk - bh * g.M;
    ApplyA<D> A;
    const uint16_t* sb = St + (size_t)blk * (D * D);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int e = 4 * RT * (t >> 2) + 4 * r + (t & 3);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) A.a[r][kk] = *reinterpret_cast<const u32x4*>(sb + e * D + kk * 32 + gq * 8);
    }
    const float* zb = Zt + (size_t)blk * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(zb + kk * 32 + gq * 8);
        const f32x4 y = *reinterpret_cast<const f32x4*>(zb + kk * 32 + gq * 8 + 4);
        A.zt[kk][0] = x.x; A.zt[kk][1] = x.y; A.zt[kk][2] = x.z; A.zt[kk][3] = x.w;
        A.zt[kk][4] = y.x; A.zt[kk][5] = y.y; A.zt[kk][6] = y.z; A.zt[kk][7] = y.w;
    }
    apply_tokens_bf16<D, NWA>(A, Q, O, g, bh, i, wave, lane);
}

// =====================================================================
// query_apply_fused: the workgroup first forms St_i, zt_i = sum_j W[i,j] [S|z]_j
// in fp32 (skipping zero weights, so a sparse local W costs only its
// non-zeros), stages them in LDS (St as bf16), then applies as query_apply.
// =====================================================================
template <int D>
__global__ __launch_bounds__(256) void query_apply_fused_bf16(const uint16_t* __restrict__ Q,
                                                              const uint16_t* __restrict__ SZ,
                                                              const float* __restrict__ W,
                                                              uint16_t* __restrict__ O, const Geo g) {
    constexpr int REC = D * D + D, NCH = REC / 8, NU = (NCH + 255) / 256;
    constexpr int RT = D / 16, KS = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t sSt[D * D];
    __shared__ __attribute__((aligned(16))) float sZt[D];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int blk = blockIdx.x;
    const int bh = (int)fdiv(blk, g.div_M);
    const int i = blk - bh * g.M;
    const int M = g.M;

    float acc[NU][8];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int s = 0; s < 8; ++s) acc[u][s] = 0.f;
    const float* wr = W + (size_t)i * M;
    const uint16_t* base = SZ + (size_t)bh * M * REC;
    for (int jj = 0; jj < M; ++jj) {
        const float w = wr[jj];
        if (w == 0.f) continue;
        const uint16_t* src = base + (size_t)jj * REC;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int ch = tid + 256 * u;
            if (ch < NCH) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(src + ch * 8);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    acc[u][2 * s] += w * bf_lo(x[s]);
                    acc[u][2 * s + 1] += w * bf_hi(x[s]);
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int ch = tid + 256 * u;
        if (ch < NCH) {
            if (ch * 8 < D * D) {
                *reinterpret_cast<u32x4*>(sSt + ch * 8) =
                    u32x4{pack_bf16(acc[u][0], acc[u][1]), pack_bf16(acc[u][2], acc[u][3]),
                          pack_bf16(acc[u][4], acc[u][5]), pack_bf16(acc[u][6], acc[u][7])};
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) sZt[ch * 8 - D * D + s] = acc[u][s];
            }
        }
    }
    __syncthreads();

    const int t = lane & 15, gq = lane >> 4;
    ApplyA<D> A;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int e = 4 * RT * (t >> 2) + 4 * r + (t & 3);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) A.a[r][kk] = *reinterpret_cast<const u32x4*>(sSt + e * D + kk * 32 + gq * 8);
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int s = 0; s < 8; ++s) A.zt[kk][s] = sZt[kk * 32 + gq * 8 + s];
    apply_tokens_bf16<D, 4>(A, Q, O, g, bh, i, wave, lane);
}

// =====================================================================
// launchers
// =====================================================================
inline void record(const Launch& L, int k) {
    if (L.events) (void)hipEventRecord(L.events[k], L.stream);
}

template <int D>
hipError_t run_d(const Launch& L) {
    const Geo& g = L.g;
    const int nblk = g.BH * g.M;
    const auto* q = static_cast<const uint16_t*>(L.q);
    const auto* k = static_cast<const uint16_t*>(L.k);
    const auto* v = static_cast<const uint16_t*>(L.v);
    auto* o = static_cast<uint16_t*>(L.out);
    auto* sz = static_cast<uint16_t*>(L.sz);
    auto* st = static_cast<uint16_t*>(L.st);

    record(L, 0);
    if constexpr (D == 128) {
        block_kv_summary_bf16<D, 1><<<nblk, 256, 0, L.stream>>>(k, v, sz, g);
    } else {
        switch (L.tune.summary_waves) {
            case 1: block_kv_summary_bf16<D, 1><<<nblk, 64, 0, L.stream>>>(k, v, sz, g); break;
            case 2: block_kv_summary_bf16<D, 2><<<nblk, 128, 0, L.stream>>>(k, v, sz, g); break;
            default: block_kv_summary_bf16<D, 4><<<nblk, 256, 0, L.stream>>>(k, v, sz, g); break;
        }
    }
    record(L, 1);
    if (L.path == MHLA_PATH_FUSED) {
        record(L, 2);
        query_apply_fused_bf16<D><<<nblk, 256, 0, L.stream>>>(q, sz, L.W, o, g);
    } else {
        const int CT = (D * D + D + 63) / 64, IT = (g.M + 63) / 64;
        const long tiles = (long)g.BH * CT * IT;
        mix_summaries_bf16<D><<<(unsigned)((tiles + 3) / 4), 256, 0, L.stream>>>(
            sz, L.W, st, L.zt, g, make_fastdiv(IT), make_fastdiv(CT));
        record(L, 2);
        switch (L.tune.apply_waves) {
            case 1: query_apply_bf16<D, 1><<<nblk, 64, 0, L.stream>>>(q, st, L.zt, o, g); break;
            case 2: query_apply_bf16<D, 2><<<nblk, 128, 0, L.stream>>>(q, st, L.zt, o, g); break;
            default: query_apply_bf16<D, 4><<<nblk, 256, 0, L.stream>>>(q, st, L.zt, o, g); break;
        }
    }
    record(L, 3);
    return hipGetLastError();
}

}  // namespace

hipError_t run_bf16(const Launch& L) {
    switch (L.g.D) {
        case 32: return run_d<32>(L);
        case 64: return run_d<64>(L);
        case 128: return run_d<128>(L);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mhla
