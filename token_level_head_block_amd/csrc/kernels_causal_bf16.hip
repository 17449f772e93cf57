// kernels_causal_bf16.hip -- the causal chunkwise form of MHLA (paperlayer.ai
// summary, appendix B "Causal MHLA": block-specific mixed summaries reused per
// block, causality preserved), bf16 inputs, d = 32 or 64, on gfx950.
//
// For chunks that are contiguous in raster order, query n of chunk i reads
//   the mixture of the earlier chunks,  St_i< = sum_{j < i} W[i,j] S_j  (z likewise),
// made by the ordinary summary and mixing kernels with W restricted to j < i,
// plus W[i,i] times its own chunk's keys and values up to n:
//   num_n = phi(q_n)^T St_i< + W[i,i] sum_{m in i, m <= n} (phi(q_n).phi(k_m)) v_m
//   den_n = phi(q_n) . zt_i< + W[i,i] sum_{m in i, m <= n} phi(q_n).phi(k_m) + eps.
// The second terms are the chunk's masked quadratic form, evaluated per
// 16-query group against each 16-key group of the chunk up to the diagonal.
#include "launch.h"
#include "bf16_shared.h"

#include <mhla.h>

namespace mhla {
namespace {

// Workgroup = (b, chunk i, group of heads) x NWA waves splitting the chunk's
// 16-token query groups (wave w takes groups w, w + NWA, ...).  Per query
// group: the forward apply's MFMAs against St_i< and zt_i<, then for each key
// group kg <= the query group
//   scores C[m][n] = phi(k_m) . phi(q_n) on v_mfma_f32_16x16x32_bf16 (A =
//   phi(K) with the key token as row, B = phi(Q) as in the apply), masked to
//   m <= n and scaled by W[i,i];  lane (n, gq) then holds keys 4*gq .. +3 of
//   query n, which is exactly the B operand of v_mfma_f32_16x16x16_bf16, so
//   num += V^T P needs no transpose of P; V^T comes from the wave's LDS slice.
template <int D, int NWA>
__global__ __launch_bounds__(512) void query_apply_causal_bf16(const uint16_t* __restrict__ Q,
                                                               const uint16_t* __restrict__ K,
                                                               const uint16_t* __restrict__ V,
                                                               const uint16_t* __restrict__ St,
                                                               const float* __restrict__ Zt,
                                                               const float* __restrict__ W,
                                                               uint16_t* __restrict__ O, const Geo g) {
    constexpr int RT = D / 16, KS = D / 32;
    constexpr int OSTR = D + 8, TS = 20;   // TS: rows of V^T, 16 keys + 4 padding
    constexpr int SLICE = 16 * OSTR + D * TS;
    __shared__ __attribute__((aligned(16))) uint16_t lds[8 * SLICE];
    const int wslot = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = lane & 15, gq = lane >> 4;
    const int wave = wslot % NWA;
    const WgCoord wgc = wg_coord(g, blockIdx.x);
    const int hh = wgc.hg * g.G + wslot / NWA;
    if (hh >= g.H) return;
    const int b = __builtin_amdgcn_readfirstlane(wgc.b);
    const int h = __builtin_amdgcn_readfirstlane(hh);
    const int i = __builtin_amdgcn_readfirstlane(wgc.j);
    const int blk = (b * g.H + h) * g.M + i;
    uint16_t* sout = lds + wslot * SLICE;
    uint16_t* vT = sout + 16 * OSTR;   // [channel][key]

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
        const float z[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
        split_zt(z, A.zhi[kk], A.zlo[kk]);
    }
    const float wii = W[(size_t)i * g.M + i];

    const int row = g.H * D;
    const int origin = block_origin(g, i);
    const size_t bb = (size_t)b * g.N * row + h * D;
    const uint16_t* qb = Q + bb;
    const uint16_t* kb = K + bb;
    const uint16_t* vb = V + bb;
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        O + (size_t)b * g.N * row, 0, g.N * row * 2, 0x00020000);
    const int olane = h * D * 2;
    auto token_off = [&](int p) { return (origin + in_block(g, p < g.T ? p : g.T - 1)) * row; };

    const int nit = (g.T + 15) >> 4;
    for (int it = wave; it < nit; it += NWA) {
        const int n_abs = it * 16 + t;
        const bool ok = n_abs < g.T;
        const int off = token_off(n_abs);
        u32x4 bq[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qb + off + kk * 32 + gq * 8);
#pragma unroll
            for (int w = 0; w < 4; ++w) bq[kk][w] = pack_bf16(phi_fast(bf_lo(x[w])), phi_fast(bf_hi(x[w])));
        }
        f32x4 acc[RT], accd = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
            for (int r = 0; r < RT; ++r) acc[r] = mfma_bf16(A.a[r][kk], bq[kk], acc[r]);
            accd = mfma_bf16(A.zhi[kk], bq[kk], accd);
            accd = mfma_bf16(A.zlo[kk], bq[kk], accd);
        }
        // The chunk's own keys up to this query group.
        float dpart = 0.f;
        for (int kg = 0; kg <= it; ++kg) {
            const int offk = token_off(kg * 16 + t);
            u32x4 ak[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(kb + offk + kk * 32 + gq * 8);
#pragma unroll
                for (int w = 0; w < 4; ++w) ak[kk][w] = pack_bf16(phi_fast(bf_lo(x[w])), phi_fast(bf_hi(x[w])));
            }
            // V of the 16 keys, transposed into vT: lane l takes key l / 4, channels (l % 4) * D/4 ..
            {
                const int key = lane >> 2, part = lane & 3;
                const int offv = token_off(kg * 16 + key);
#pragma unroll
                for (int u = 0; u < D / 32; ++u) {
                    const u32x4 x = *reinterpret_cast<const u32x4*>(vb + offv + part * (D / 4) + 8 * u);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const int c = part * (D / 4) + 8 * u + 2 * w;
                        vT[c * TS + key] = (uint16_t)(x[w] & 0xffffu);
                        vT[(c + 1) * TS + key] = (uint16_t)(x[w] >> 16);
                    }
                }
            }
            f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) sc = mfma_bf16(ak[kk], bq[kk], sc);
            float pv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m_abs = kg * 16 + 4 * gq + v;
                pv[v] = (m_abs <= n_abs && m_abs < g.T) ? wii * sc[v] : 0.f;
            }
            const u32x2 pb = u32x2{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
            // the denominator adds the same rounded weights the numerator uses
            dpart += bf_lo(pb.x) + bf_hi(pb.x) + bf_lo(pb.y) + bf_hi(pb.y);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int e = 4 * RT * (t >> 2) + 4 * r + (t & 3);
                const u32x2 av = *reinterpret_cast<const u32x2*>(vT + e * TS + 4 * gq);
                acc[r] = mfma_k16(av, pb, acc[r]);
            }
        }
        dpart += shfl_xor(dpart, 16);
        dpart += shfl_xor(dpart, 32);
        const float inv = 1.f / (accd[0] + dpart + g.eps);
        uint32_t wv[2 * RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            wv[2 * r] = pack_bf16(acc[r][0] * inv, acc[r][1] * inv);
            wv[2 * r + 1] = pack_bf16(acc[r][2] * inv, acc[r][3] * inv);
        }
        store_rows<D>(sout, wv, lane, off, ok, orsrc, olane);
    }
}

template <int D, int NWA>
void launch(const Launch& L) {
    Geo g = L.g;
    const int gmax = 8 / NWA;
    g.HG = (g.H + gmax - 1) / gmax;
    g.G = (g.H + g.HG - 1) / g.HG;
    g.div_HG = make_fastdiv((uint32_t)g.HG);
    query_apply_causal_bf16<D, NWA><<<g.B * g.M * g.HG, 64 * NWA * g.G, 0, L.stream>>>(
        static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v),
        static_cast<const uint16_t*>(L.st), L.zt, L.W, static_cast<uint16_t*>(L.out), g);
}

}  // namespace

hipError_t launch_causal_apply_bf16(const Launch& L) {
    const bool wide = L.g.T >= 128;   // four waves share a long chunk's query groups
    switch (L.g.D) {
        case 32: wide ? launch<32, 4>(L) : launch<32, 1>(L); break;
        case 64: wide ? launch<64, 4>(L) : launch<64, 1>(L); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mhla
