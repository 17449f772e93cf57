// kernels_f32.hip -- MHLA forward for float32 inputs on gfx950 (MI355X).
//
// Same three stages and fused variant as the bf16 path (MHLA, arXiv
// 2601.07832; paperlayer.ai summary, section 4), computed entirely in fp32 on
// v_mfma_f32_16x16x4_f32.  Each lane supplies one k-slot per instruction, so
// operands need no packing: a lane loads a contiguous run of channels of one
// token and feeds one channel to each row (or column) tile.
#include "launch.h"

#include <mhla.h>

namespace mhla {
namespace {

template <int N>
struct FVec {
    float x[N];
};

template <int N>
__device__ __forceinline__ FVec<N> load_f(const float* p) {
    FVec<N> r;
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int u = 0; u < N / 4; ++u) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(p + 4 * u);
            r.x[4 * u] = t.x; r.x[4 * u + 1] = t.y; r.x[4 * u + 2] = t.z; r.x[4 * u + 3] = t.w;
        }
    } else {
        static_assert(N == 2, "");
        const float2 t = *reinterpret_cast<const float2*>(p);
        r.x[0] = t.x; r.x[1] = t.y;
    }
    return r;
}

// =====================================================================
// block_kv_summary (fp32): k-step of 4 tokens, one token per lane group.
// Lane (li, gq): K channels CPL*li .. for rows, V channels for columns,
// token 32*it + 4*u + gq in sub-step u.
// =====================================================================
template <int D, int NWT>
__global__ __launch_bounds__(64 * NWT * (D == 128 ? 4 : 1)) void block_kv_summary_f32(
    const float* __restrict__ K, const float* __restrict__ V, float* __restrict__ SZ, const Geo g) {
    constexpr int NQ = (D == 128) ? 4 : 1;
    constexpr int CPL = (D == 32) ? 2 : 4;
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
    const float* kb = K + (b * g.N * row + h * D + rowbase + CPL * li);
    const float* vb = V + (b * g.N * row + h * D + colbase + CPL * li);

    f32x4 acc[CPL][CPL];
#pragma unroll
    for (int r = 0; r < CPL; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zacc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) zacc[c] = 0.f;

    const int nit = (g.T + 31) >> 5;
    for (int it = tw; it < nit; it += NWT) {
        FVec<CPL> kr[8], vr[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = it * 32 + 4 * u + gq;
            ok[u] = p < g.T;
            const int off = (origin + in_block(g, ok[u] ? p : g.T - 1)) * row;
            kr[u] = load_f<CPL>(kb + off);
            vr[u] = load_f<CPL>(vb + off);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            float fk[CPL], vv[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                fk[c] = ok[u] ? phi_exact(kr[u].x[c]) : 0.f;
                vv[c] = ok[u] ? vr[u].x[c] : 0.f;
                zacc[c] += fk[c];
            }
#pragma unroll
            for (int r = 0; r < CPL; ++r)
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[r][c] = mfma_f32(fk[r], vv[c], acc[r][c]);
        }
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

    // Lane holds S[c][e] for c = rowbase + 4*CPL*gq + CPL*v + r, e = colbase + CPL*li + c2.
    float* rec = SZ + (size_t)blk * (D * D + D);
#pragma unroll
    for (int c2 = 0; c2 < CPL; ++c2) {
        const int e = colbase + CPL * li + c2;
        float vals[4 * CPL];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int r = 0; r < CPL; ++r) vals[CPL * v + r] = acc[r][c2][v];
        float* dst = rec + e * D + rowbase + 4 * CPL * gq;
#pragma unroll
        for (int u = 0; u < CPL; ++u)
            *reinterpret_cast<f32x4*>(dst + 4 * u) = f32x4{vals[4 * u], vals[4 * u + 1], vals[4 * u + 2], vals[4 * u + 3]};
    }
    if (gq == 0 && (quad & 1) == 0) {
        float* dst = rec + D * D + rowbase + CPL * li;
#pragma unroll
        for (int c = 0; c < CPL; ++c) dst[c] = zacc[c];
    }
}

// =====================================================================
// mix_summaries (fp32): C[col'][i] = sum_j [S|z]_j[col'] W[i][j], k-step of
// 4 source blocks, one per lane group.
// =====================================================================
template <int D>
__global__ __launch_bounds__(256) void mix_summaries_f32(const float* __restrict__ SZ,
                                                         const float* __restrict__ W,
                                                         float* __restrict__ St, float* __restrict__ Zt,
                                                         const Geo g, const FastDiv div_IT,
                                                         const FastDiv div_CT, int causal) {
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
    const float* abase = SZ + (size_t)bh * M * REC + colp;

    f32x4 acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* wrow[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = it * 64 + 16 * t + li;
        wrow[t] = W + (size_t)(i < M ? i : M - 1) * M;
    }
    const int nk = (M + 3) >> 2;
    for (int kk = 0; kk < nk; ++kk) {
        const int jj = 4 * kk + gq;
        const bool ok = jj < M;
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
        if (ok && colok) a = *reinterpret_cast<const f32x4*>(abase + (size_t)jj * REC);
        float bw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // the causal form mixes only the blocks before query block i
            const bool keep = ok && !(causal && jj >= it * 64 + 16 * t + li);
            bw[t] = keep ? wrow[t][jj] : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[r][t] = mfma_f32(a[r], bw[t], acc[r][t]);
    }

    const int cp0 = ct * 64 + 16 * gq;
    if (cp0 >= REC) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = it * 64 + 16 * t + li;
        if (i >= M) continue;
        const size_t rec = (size_t)bh * M + i;
        float* dst = (cp0 < D * D) ? St + rec * (D * D) + cp0 : Zt + rec * D + (cp0 - D * D);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            *reinterpret_cast<f32x4*>(dst + 4 * v) = f32x4{acc[0][t][v], acc[1][t][v], acc[2][t][v], acc[3][t][v]};
    }
}

// =====================================================================
// query_apply (fp32): O^T = St_i^T phi(Q)^T per 16-token group.  k-step kk
// and lane group gq cover channel c = (D/4)*gq + kk, so each lane reads D/4
// consecutive channels of its token and of every St_i^T row it feeds.
// Output rows: e = 4*RT*(ii/4) + 4r + ii%4 (4*RT consecutive channels per lane).
// =====================================================================
template <int D, bool FROM_LDS>
__device__ __forceinline__ void apply_tokens_f32(const float* St_i, const float* zt_i,
                                                 const float* __restrict__ Q, float* __restrict__ O,
                                                 const Geo& g, int bh, int i, int wave, int nwaves,
                                                 int lane) {
    constexpr int RT = D / 16, NK = D / 4;
    const int t = lane & 15, gq = lane >> 4;
    const int b = (int)fdiv(bh, g.div_H), h = bh - b * g.H;
    const int row = g.H * D;
    const int origin = block_origin(g, i);
    const float* qb = Q + (b * g.N * row + h * D + NK * gq);
    float* ob = O + (b * g.N * row + h * D + 4 * RT * gq);
    float zt[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) zt[kk] = zt_i[NK * gq + kk];
    const int nit = (g.T + 15) >> 4;
    for (int it = wave; it < nit; it += nwaves) {
        const int p = it * 16 + t;
        const bool ok = p < g.T;
        const int off = (origin + in_block(g, ok ? p : g.T - 1)) * row;
        const FVec<NK> qv = load_f<NK>(qb + off);
        float fq[NK];
        float den = 0.f;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            fq[kk] = phi_exact(qv.x[kk]);
            den += fq[kk] * zt[kk];
        }
        f32x4 acc[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int e = 4 * RT * (t >> 2) + 4 * r + (t & 3);
            const FVec<NK> av = load_f<NK>(St_i + e * D + NK * gq);
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) acc[r] = mfma_f32(av.x[kk], fq[kk], acc[r]);
        }
        den += shfl_xor(den, 16);
        den += shfl_xor(den, 32);
        const float inv = 1.f / (den + g.eps);
        if (ok) {
#pragma unroll
            for (int r = 0; r < RT; ++r)
                *reinterpret_cast<f32x4*>(ob + off + 4 * r) =
                    f32x4{acc[r][0] * inv, acc[r][1] * inv, acc[r][2] * inv, acc[r][3] * inv};
        }
    }
}

template <int D, int NWA>
__global__ __launch_bounds__(64 * NWA) void query_apply_f32(const float* __restrict__ Q,
                                                            const float* __restrict__ St,
                                                            const float* __restrict__ Zt,
                                                            float* __restrict__ O, const Geo g) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int blk = blockIdx.x;
    const int bh = (int)fdiv(blk, g.div_M);
    const int i = blk - bh * g.M;
    apply_tokens_f32<D, false>(St + (size_t)blk * (D * D), Zt + (size_t)blk * D, Q, O, g, bh, i,
                               wave, NWA, lane);
}

// =====================================================================
// query_apply_fused (fp32): St_i, zt_i = sum_j W[i,j] [S|z]_j formed in the
// workgroup (zero weights skipped) and staged in LDS, then applied.
// =====================================================================
template <int D>
__global__ __launch_bounds__(256) void query_apply_fused_f32(const float* __restrict__ Q,
                                                             const float* __restrict__ SZ,
                                                             const float* __restrict__ W,
                                                             float* __restrict__ O, const Geo g) {
    constexpr int REC = D * D + D, NCH = REC / 4, NU = (NCH + 255) / 256;
    __shared__ __attribute__((aligned(16))) float sSt[D * D + D];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int blk = blockIdx.x;
    const int bh = (int)fdiv(blk, g.div_M);
    const int i = blk - bh * g.M;
    const int M = g.M;
    f32x4 acc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* wr = W + (size_t)i * M;
    const float* base = SZ + (size_t)bh * M * REC;
    __shared__ int s_idx[256], s_cnt[4];
    __shared__ float s_w[256];
    // Row i of W 256 entries at a time, nonzero weights listed first.
    for (int j0 = 0; j0 < M; j0 += 256) {
        const int n = compact_nonzero(wr, M, j0, s_idx, s_w, s_cnt);
        for (int t = 0; t < n; ++t) {
            const float w = s_w[t];
            const float* src = base + (size_t)s_idx[t] * REC;
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int ch = tid + 256 * u;
                if (ch < NCH) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(src + 4 * ch);
                    acc[u] += w * x;
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int ch = tid + 256 * u;
        if (ch < NCH) *reinterpret_cast<f32x4*>(sSt + 4 * ch) = acc[u];
    }
    __syncthreads();
    apply_tokens_f32<D, true>(sSt, sSt + D * D, Q, O, g, bh, i, wave, 4, lane);
}

inline void record(const Launch& L, int k) {
    if (L.events) (void)hipEventRecord(L.events[k], L.stream);
}

// =====================================================================
// query_apply_causal (fp32), chunks contiguous in raster order (paperlayer.ai
// summary, appendix B "Causal MHLA"): workgroup = (b, chunk i, head h) of D
// threads walking the chunk's tokens in order.  Thread e keeps column e of
// C = St_i< + W[i,i] sum_{m <= p} phi(k_m) v_m^T in registers and the mixed
// normaliser zt_i< + W[i,i] sum phi(k_m) lives in LDS, so query p reads
// num_e = phi(q_p) . C[:, e] and den = phi(q_p) . z + eps after its own token
// is added.
// =====================================================================
template <int D>
__global__ __launch_bounds__(D) void query_apply_causal_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                            const float* __restrict__ V, const float* __restrict__ St,
                                                            const float* __restrict__ Zt, const float* __restrict__ W,
                                                            float* __restrict__ O, const Geo g) {
    __shared__ float us[D], as[D], zs[D];
    const int e = threadIdx.x;
    const int blk = blockIdx.x;            // (b h) * M + i
    const int bh = blk / g.M, i = blk - bh * g.M;
    const int b = bh / g.H, h = bh - b * g.H;
    const float wii = W[(size_t)i * g.M + i];
    float col[D];
    const float* st = St + (size_t)blk * (D * D) + (size_t)e * D;   // stored as [e][c]
#pragma unroll
    for (int c = 0; c < D; ++c) col[c] = st[c];
    zs[e] = Zt[(size_t)blk * D + e];
    const size_t base = (((size_t)b * g.N + block_origin(g, i)) * g.H + h) * D + e;
    const size_t row = (size_t)g.H * D;
    for (int p = 0; p < g.T; ++p) {
        const size_t off = base + (size_t)p * row;   // contiguous chunk: raster index origin + p
        const float ve = V[off];
        us[e] = phi_exact(Q[off]);
        as[e] = phi_exact(K[off]);
        __syncthreads();
        float num = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            col[c] += wii * as[c] * ve;
            num += us[c] * col[c];
        }
        zs[e] += wii * as[e];
        __syncthreads();
        float den = g.eps;
#pragma unroll 8
        for (int c = 0; c < D; ++c) den += us[c] * zs[c];
        O[off] = num / den;
        __syncthreads();
    }
}

template <int D>
hipError_t run_d(const Launch& L) {
    const Geo& g = L.g;
    const int nblk = g.BH * g.M;
    const auto* q = static_cast<const float*>(L.q);
    const auto* k = static_cast<const float*>(L.k);
    const auto* v = static_cast<const float*>(L.v);
    auto* o = static_cast<float*>(L.out);
    auto* sz = static_cast<float*>(L.sz);
    auto* st = static_cast<float*>(L.st);

    record(L, 0);
    if constexpr (D == 128) {
        block_kv_summary_f32<D, 1><<<nblk, 256, 0, L.stream>>>(k, v, sz, g);
    } else {
        switch (L.tune.summary_waves) {
            case 1: block_kv_summary_f32<D, 1><<<nblk, 64, 0, L.stream>>>(k, v, sz, g); break;
            case 2: block_kv_summary_f32<D, 2><<<nblk, 128, 0, L.stream>>>(k, v, sz, g); break;
            default: block_kv_summary_f32<D, 4><<<nblk, 256, 0, L.stream>>>(k, v, sz, g); break;
        }
    }
    record(L, 1);
    if (L.path == MHLA_PATH_FUSED) {
        record(L, 2);
        query_apply_fused_f32<D><<<nblk, 256, 0, L.stream>>>(q, sz, L.W, o, g);
    } else {
        const int CT = (D * D + D + 63) / 64, IT = (g.M + 63) / 64;
        const long tiles = (long)g.BH * CT * IT;
        const bool causal = L.path == MHLA_PATH_CAUSAL;
        mix_summaries_f32<D><<<(unsigned)((tiles + 3) / 4), 256, 0, L.stream>>>(
            sz, L.W, st, L.zt, g, make_fastdiv(IT), make_fastdiv(CT), causal ? 1 : 0);
        record(L, 2);
        if (causal) {
            query_apply_causal_f32<D><<<nblk, D, 0, L.stream>>>(q, k, v, st, L.zt, L.W, o, g);
            record(L, 3);
            return hipGetLastError();
        }
        switch (L.tune.apply_waves) {
            case 1: query_apply_f32<D, 1><<<nblk, 64, 0, L.stream>>>(q, st, L.zt, o, g); break;
            case 2: query_apply_f32<D, 2><<<nblk, 128, 0, L.stream>>>(q, st, L.zt, o, g); break;
            default: query_apply_f32<D, 4><<<nblk, 256, 0, L.stream>>>(q, st, L.zt, o, g); break;
        }
    }
    record(L, 3);
    return hipGetLastError();
}

}  // namespace

hipError_t run_f32(const Launch& L) {
    switch (L.g.D) {
        case 32: return run_d<32>(L);
        case 64: return run_d<64>(L);
        case 128: return run_d<128>(L);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mhla
