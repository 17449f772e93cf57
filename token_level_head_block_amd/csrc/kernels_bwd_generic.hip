// kernels_bwd_generic.hip -- the backward pass of MHLA for the problems the
// bf16 MFMA kernels do not take: fp32 inputs (head_dim 32, 64, 128) and bf16
// inputs with head_dim 128.  Plain fp32 arithmetic with LDS tiling, no MFMA.
//
// The gradients are the chain rule on the forward definition (W is learned:
// paperlayer.ai summary, section 4 "Multi-Head Mixing"); with u = phi(q_n),
// a = phi(k_m), g = dout_n, and block records [S_j | z_j] (S as [c][e]):
//   den = u . zt_i + eps, dnum = g / den, dden = -(g . o_n) / den
//   dq = (St_i dnum + zt_i dden) * phi'(q),  dSt_i = sum u dnum^T, dzt_i = sum u dden
//   [dS | dz]_j = sum_i W[i,j] [dSt | dzt]_i,  dW[i,j] = sum over (b,h) of <[dSt|dzt]_i, [S|z]_j>
//   dv = dS_j^T a,  dk = (dS_j v + dz_j) * phi'(k)
// Every intermediate is an fp32 record of L = d*d + d values in workspace.
#include "launch.h"

#include <mhla.h>

namespace mhla {
namespace {

__device__ __forceinline__ float ld1(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ void st1(uint16_t* p, float x) { *p = (uint16_t)(pack_bf16(x, 0.f) & 0xffffu); }
__device__ __forceinline__ void st1(float* p, float x) { *p = x; }
__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : expf(x); }

__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += shfl_xor(x, o);
    return x;
}

// Raster token of position p of block j and the element offset of (b, n, h, 0).
__device__ __forceinline__ size_t tok_off(const Geo& g, int b, int h, int j, int p) {
    const int n = block_origin(g, j) + in_block(g, p);
    return (((size_t)b * g.N + n) * g.H + h) * g.D;
}

// ---- block summaries [S_j | z_j] in fp32: workgroup = (b h, block j), each
// thread owns d*d/256 entries of S and accumulates over batches of 16 tokens.
template <int D, typename T>
__global__ __launch_bounds__(256) void g_summary(const T* __restrict__ K, const T* __restrict__ V,
                                                 float* __restrict__ rec, const Geo g) {
    constexpr int E = D * D / 256, TB = 16, L = D * D + D;
    __shared__ float ka[TB][D], va[TB][D];
    const int tid = threadIdx.x, blk = blockIdx.x;
    const int bh = blk / g.M, j = blk - bh * g.M;
    const int b = bh / g.H, h = bh - b * g.H;
    float acc[E], zacc = 0.f;
#pragma unroll
    for (int r = 0; r < E; ++r) acc[r] = 0.f;
    for (int t0 = 0; t0 < g.T; t0 += TB) {
        __syncthreads();
        for (int u = tid; u < TB * D; u += 256) {
            const int tt = u / D, c = u - tt * D, p = t0 + tt;
            float kv = 0.f, vv = 0.f;   // tokens past the block contribute nothing
            if (p < g.T) {
                const size_t off = tok_off(g, b, h, j, p) + c;
                kv = phi_exact(ld1(K + off));
                vv = ld1(V + off);
            }
            ka[tt][c] = kv;
            va[tt][c] = vv;
        }
        __syncthreads();
#pragma unroll 4
        for (int tt = 0; tt < TB; ++tt) {
#pragma unroll
            for (int r = 0; r < E; ++r) {
                const int idx = tid + 256 * r, c = idx / D, e = idx - c * D;
                acc[r] += ka[tt][c] * va[tt][e];
            }
            if (tid < D) zacc += ka[tt][tid];
        }
    }
    float* out = rec + (size_t)blk * L;
#pragma unroll
    for (int r = 0; r < E; ++r) out[tid + 256 * r] = acc[r];
    if (tid < D) out[D * D + tid] = zacc;
}

// ---- record mixing: out[bh][i][x] = sum_j w(i, j) in[bh][j][x], with
// w(i, j) = W[i][j], or W[j][i] when transposed.  Causal: only earlier chunks
// feed a chunk (j < i), and in the transposed sum only later ones (j > i).
// Workgroup = (b h, 16 rows i, 256 record values); the W tile goes through LDS
// in chunks of 256 j.
__global__ __launch_bounds__(256) void g_mix(const float* __restrict__ W, const float* __restrict__ in,
                                             float* __restrict__ out, int M, int L, int transposed, int causal) {
    __shared__ float wt[16][257];
    const int tid = threadIdx.x;
    const int nxc = (L + 255) / 256, nit = (M + 15) / 16;
    int id = blockIdx.x;
    const int xc = id % nxc;
    id /= nxc;
    const int it = id % nit;
    const int bh = id / nit;
    const int x = xc * 256 + tid, i0 = it * 16;
    const bool xok = x < L;
    const float* src = in + (size_t)bh * M * L + (xok ? x : 0);
    float acc[16];
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) acc[ii] = 0.f;
    for (int j0 = 0; j0 < M; j0 += 256) {
        __syncthreads();
        for (int u = tid; u < 16 * 256; u += 256) {
            const int ii = u >> 8, jj = u & 255, i = i0 + ii, j = j0 + jj;
            float wv = 0.f;
            const bool masked = causal && (transposed ? j <= i : j >= i);
            if (i < M && j < M && !masked) wv = transposed ? W[(size_t)j * M + i] : W[(size_t)i * M + j];
            wt[ii][jj] = wv;
        }
        __syncthreads();
        const int jn = min(256, M - j0);
        for (int jj = 0; jj < jn; ++jj) {
            const float v = src[(size_t)(j0 + jj) * L];
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) acc[ii] += wt[ii][jj] * v;
        }
    }
    if (!xok) return;
#pragma unroll
    for (int ii = 0; ii < 16; ++ii)
        if (i0 + ii < M) out[((size_t)bh * M + i0 + ii) * L + x] = acc[ii];
}

// ---- query side: workgroup = (b h, block i), St_i and zt_i in LDS; the four
// waves take one token each per step (dq, and the token's u and dnum), then
// every thread adds the four tokens' u dnum^T into its d*d/256 entries of dSt_i.
template <int D, typename T>
__global__ __launch_bounds__(256) void g_query(const T* __restrict__ Q, const T* __restrict__ G,
                                               const float* __restrict__ strec, T* __restrict__ dQ,
                                               float* __restrict__ dstrec, const Geo g) {
    constexpr int DP = D + 1, E = D * D / 256, CPL = (D + 63) / 64, L = D * D + D;
    __shared__ float s[D * DP];
    __shared__ float zt[D];
    __shared__ float ub[4][D], dn[4][D], dd[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int blk = blockIdx.x;
    const int bh = blk / g.M, i = blk - bh * g.M;
    const int b = bh / g.H, h = bh - b * g.H;
    const float* src = strec + (size_t)blk * L;
    for (int u = tid; u < D * D; u += 256) s[(u / D) * DP + (u % D)] = src[u];
    if (tid < D) zt[tid] = src[D * D + tid];
    float acc[E], zacc = 0.f;
#pragma unroll
    for (int r = 0; r < E; ++r) acc[r] = 0.f;
    __syncthreads();
    for (int t0 = 0; t0 < g.T; t0 += 4) {
        const int p = t0 + w;
        if (p < g.T) {   // wave-uniform
            const size_t off = tok_off(g, b, h, i, p);
            float xq[CPL], uq[CPL];
            float dpart = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int c = lane + 64 * k;
                xq[k] = c < D ? ld1(Q + off + c) : 0.f;
                uq[k] = c < D ? phi_exact(xq[k]) : 0.f;
                if (c < D) {
                    ub[w][c] = uq[k];
                    dpart += uq[k] * zt[c];
                }
            }
            __builtin_amdgcn_wave_barrier();
            const float den = wave_sum64(dpart) + g.eps;
            float ge[CPL], oe[CPL], go = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int e = lane + 64 * k;
                float num = 0.f;
                if (e < D) {
#pragma unroll 8
                    for (int c = 0; c < D; ++c) num += ub[w][c] * s[c * DP + e];
                    ge[k] = ld1(G + off + e);
                } else {
                    ge[k] = 0.f;
                }
                oe[k] = num / den;
                go += ge[k] * oe[k];
            }
            const float dden = -wave_sum64(go) / den;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int e = lane + 64 * k;
                if (e < D) dn[w][e] = ge[k] / den;
            }
            if (lane == 0) dd[w] = dden;
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int c = lane + 64 * k;
                if (c >= D) continue;
                float t = zt[c] * dden;
#pragma unroll 8
                for (int e = 0; e < D; ++e) t += s[c * DP + e] * dn[w][e];
                st1(dQ + off + c, t * dphi(xq[k]));
            }
        } else {
            for (int c = lane; c < D; c += 64) {
                ub[w][c] = 0.f;
                dn[w][c] = 0.f;
            }
            if (lane == 0) dd[w] = 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const int idx = tid + 256 * r, c = idx / D, e = idx - c * D;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) acc[r] += ub[ww][c] * dn[ww][e];
        }
        if (tid < D)
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) zacc += ub[ww][tid] * dd[ww];
        __syncthreads();
    }
    float* out = dstrec + (size_t)blk * L;
#pragma unroll
    for (int r = 0; r < E; ++r) out[tid + 256 * r] = acc[r];
    if (tid < D) out[D * D + tid] = zacc;
}

// ---- key/value side: workgroup = (b h, block j), [dS | dz]_j in LDS, one
// token per wave and step: dv = dS^T a, dk = (dS v + dz) * phi'(k).
template <int D, typename T>
__global__ __launch_bounds__(256) void g_kv(const T* __restrict__ K, const T* __restrict__ V,
                                            const float* __restrict__ dsrec, T* __restrict__ dK, T* __restrict__ dV,
                                            const Geo g) {
    constexpr int DP = D + 1, CPL = (D + 63) / 64, L = D * D + D;
    __shared__ float s[D * DP];
    __shared__ float dz[D];
    __shared__ float ab[4][D], vb[4][D];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int blk = blockIdx.x;
    const int bh = blk / g.M, j = blk - bh * g.M;
    const int b = bh / g.H, h = bh - b * g.H;
    const float* src = dsrec + (size_t)blk * L;
    for (int u = tid; u < D * D; u += 256) s[(u / D) * DP + (u % D)] = src[u];
    if (tid < D) dz[tid] = src[D * D + tid];
    __syncthreads();
    for (int p = w; p < g.T; p += 4) {   // no cross-wave dependence
        const size_t off = tok_off(g, b, h, j, p);
        float xk[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int c = lane + 64 * k;
            xk[k] = c < D ? ld1(K + off + c) : 0.f;
            if (c < D) {
                ab[w][c] = phi_exact(xk[k]);
                vb[w][c] = ld1(V + off + c);
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int x = lane + 64 * k;
            if (x >= D) continue;
            float dvx = 0.f, dkx = dz[x];
            for (int y = 0; y < D; ++y) {
                dvx += s[y * DP + x] * ab[w][y];   // dv[e = x] = sum_c dS[c][e] a[c]
                dkx += s[x * DP + y] * vb[w][y];   // dk[c = x] = sum_e dS[c][e] v[e] + dz[c]
            }
            st1(dV + off + x, dvx);
            st1(dK + off + x, dkx * dphi(xk[k]));
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// ---- dW partial sums: partial[s][i][j] = sum over the s-th share of the
// 32-value chunks of all (b h) records of dst[bh][i][x] src[bh][j][x].
// Workgroup = (32 x 32 tile of (i, j), share s); each thread owns 4 outputs.
__global__ __launch_bounds__(256) void g_dw_partial(const float* __restrict__ dst, const float* __restrict__ src,
                                                    float* __restrict__ part, int BH, int M, int L, int nsplit) {
    constexpr int KC = 32;
    __shared__ float a[32][KC + 1], bt[32][KC + 1];
    const int tid = threadIdx.x;
    const int ntile = (M + 31) / 32;
    int id = blockIdx.x;
    const int sp = id % nsplit;
    id /= nsplit;
    const int tj = id % ntile, ti = id / ntile;
    const int i0 = ti * 32, j0 = tj * 32;
    const int cpr = L / KC;                       // chunks per record (L is a multiple of 32)
    const long total = (long)BH * cpr;
    const long c0 = total * sp / nsplit, c1 = total * (sp + 1) / nsplit;
    const int oi = tid >> 3, oj = (tid & 7) * 4;  // row oi, columns oj .. oj+3
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (long ch = c0; ch < c1; ++ch) {
        const int bh = (int)(ch / cpr), x0 = (int)(ch - (long)bh * cpr) * KC;
        __syncthreads();
        for (int u = tid; u < 32 * KC; u += 256) {
            const int r = u / KC, x = u - r * KC;
            const int i = i0 + r, j = j0 + r;
            a[r][x] = i < M ? dst[((size_t)bh * M + i) * L + x0 + x] : 0.f;
            bt[r][x] = j < M ? src[((size_t)bh * M + j) * L + x0 + x] : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int x = 0; x < KC; ++x) {
            const float av = a[oi][x];
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] += av * bt[oj + t][x];
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = i0 + oi, j = j0 + oj + t;
        if (i < M && j < M) part[((size_t)sp * M + i) * M + j] = acc[t];
    }
}

// dW = sum of the partials in share order (deterministic).  Causal (diag
// non-null): coefficients of later chunks get zero, and the diagonal is the
// in-chunk term diag[bh][i] summed over (b h) in order.
__global__ __launch_bounds__(256) void g_dw_reduce(const float* __restrict__ part, float* __restrict__ dW, int M,
                                                   int nsplit, const float* __restrict__ diag, int BH) {
    const int MM = M * M;
    const int x = blockIdx.x * 256 + threadIdx.x;
    if (x >= MM) return;
    const int i = x / M, j = x - i * M;
    float t = 0.f;
    if (!diag || j < i) {
        for (int s = 0; s < nsplit; ++s) t += part[(size_t)s * MM + x];
    } else if (j == i) {
        for (int bh = 0; bh < BH; ++bh) t += diag[(size_t)bh * M + i];
    }
    dW[x] = t;
}

// ---- causal query side (chunks contiguous in raster order; paperlayer.ai
// summary, appendix B "Causal MHLA").  Token n of chunk i sees
//   C_n = St_i< + w P_n,  zeta_n = zt_i< + w zp_n,  w = W[i][i],
// P_n, zp_n the chunk's prefix sums of a v^T and a over m <= n.  Workgroup =
// (b h, chunk i); LDS holds C and zeta at the start of the current step of four
// tokens (one per wave); each wave adds the in-step terms of the tokens before
// and at its own.  Writes dq, the record [dSt_i< | dzt_i<] (sums over the whole
// chunk, as in the non-causal case) and each token's dnum and dden for the
// key side.
template <int D, typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void g_query_causal(const T* __restrict__ Q, const T* __restrict__ K,
                                                      const T* __restrict__ V, const T* __restrict__ G,
                                                      const float* __restrict__ strec, const float* __restrict__ W,
                                                      T* __restrict__ dQ, float* __restrict__ dstrec,
                                                      float* __restrict__ dnum, float* __restrict__ dden,
                                                      const Geo g) {
    constexpr int DP = D + 1, E = D * D / 256, CPL = (D + 63) / 64, L = D * D + D;
    __shared__ float s[D * DP];
    __shared__ float da[D * D];   // dSt_i<, each entry owned by one thread
    __shared__ float zt[D];
    __shared__ float ub[4][D], ab[4][D], vb[4][D], dn[4][D], dd[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int blk = blockIdx.x;
    const int bh = blk / g.M, i = blk - bh * g.M;
    const int b = bh / g.H, h = bh - b * g.H;
    const float wii = W[(size_t)i * g.M + i];
    const float* src = strec + (size_t)blk * L;
    for (int u = tid; u < D * D; u += 256) s[(u / D) * DP + (u % D)] = src[u];
    if (tid < D) zt[tid] = src[D * D + tid];
    for (int r = 0; r < E; ++r) da[tid + 256 * r] = 0.f;
    float zacc = 0.f;
    for (int t0 = 0; t0 < g.T; t0 += 4) {
        const int p = t0 + w;
        const bool valid = p < g.T;   // wave-uniform
        const size_t off = valid ? tok_off(g, b, h, i, p) : 0;
        float xq[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int c = lane + 64 * k;
            xq[k] = 0.f;
            if (c >= D) continue;
            float uu = 0.f, aa = 0.f, vv = 0.f;
            if (valid) {
                xq[k] = ld1(Q + off + c);
                uu = phi_exact(xq[k]);
                aa = phi_exact(ld1(K + off + c));
                vv = ld1(V + off + c);
            }
            ub[w][c] = uu;
            ab[w][c] = aa;
            vb[w][c] = vv;
            dn[w][c] = 0.f;
        }
        if (lane == 0) dd[w] = 0.f;
        __syncthreads();
        if (valid) {
            float ua[4];
            float dpart = 0.f;
#pragma unroll
            for (int x = 0; x < 4; ++x) ua[x] = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int c = lane + 64 * k;
                if (c >= D) continue;
                dpart += ub[w][c] * zt[c];
#pragma unroll
                for (int x = 0; x < 4; ++x) ua[x] += ub[w][c] * ab[x][c];
            }
            float den = wave_sum64(dpart);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                ua[x] = x <= w ? wave_sum64(ua[x]) : 0.f;   // u_n . a_m for the in-step m <= n
                den += wii * ua[x];
            }
            den += g.eps;
            float ge[CPL], go = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int e = lane + 64 * k;
                ge[k] = 0.f;
                if (e >= D) continue;
                float num = 0.f, corr = 0.f;
#pragma unroll 8
                for (int c = 0; c < D; ++c) num += ub[w][c] * s[c * DP + e];
#pragma unroll
                for (int x = 0; x < 4; ++x) corr += ua[x] * vb[x][e];
                num += wii * corr;
                ge[k] = ld1(G + off + e);
                go += ge[k] * (num / den);
            }
            const float ddv = -wave_sum64(go) / den;
            const size_t toff = off / D;   // (b, n, h) index
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int e = lane + 64 * k;
                if (e >= D) continue;
                dn[w][e] = ge[k] / den;
                dnum[off + e] = ge[k] / den;
            }
            if (lane == 0) {
                dd[w] = ddv;
                dden[toff] = ddv;
            }
            __builtin_amdgcn_wave_barrier();
            float vd[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) vd[x] = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int e = lane + 64 * k;
                if (e >= D) continue;
#pragma unroll
                for (int x = 0; x < 4; ++x) vd[x] += vb[x][e] * dn[w][e];
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) vd[x] = x <= w ? wave_sum64(vd[x]) : 0.f;   // v_m . dnum_n
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int c = lane + 64 * k;
                if (c >= D) continue;
                float zc = zt[c], corr = 0.f;
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    if (x <= w) {
                        zc += wii * ab[x][c];
                        corr += ab[x][c] * vd[x];
                    }
                float t = zc * ddv + wii * corr;
#pragma unroll 8
                for (int e = 0; e < D; ++e) t += s[c * DP + e] * dn[w][e];
                st1(dQ + off + c, t * dphi(xq[k]));
            }
        }
        __syncthreads();
        for (int r = 0; r < E; ++r) {
            const int idx = tid + 256 * r, c = idx / D, e = idx - c * D;
            float av = 0.f, ud = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                ud += ub[ww][c] * dn[ww][e];
                av += ab[ww][c] * vb[ww][e];
            }
            da[idx] += ud;
            s[c * DP + e] += wii * av;
        }
        if (tid < D) {
            float za = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                zacc += ub[ww][tid] * dd[ww];
                za += ab[ww][tid];
            }
            zt[tid] += wii * za;
        }
        __syncthreads();
    }
    float* out = dstrec + (size_t)blk * L;
    for (int r = 0; r < E; ++r) out[tid + 256 * r] = da[tid + 256 * r];
    if (tid < D) out[D * D + tid] = zacc;
}

// ---- causal key/value side.  Key m of chunk i gets
//   G_m = Gx_i + w R_m,  gz_m = gzx_i + w r_m,
// Gx_i = sum_{k > i} W[k][i] dSt_k< (the transposed causal mixing, in dsrec),
// R_m, r_m the chunk's suffix sums of u dnum^T and u dden over n >= m.  Tokens
// go in reverse, four per step (one per wave), with R and r in LDS holding the
// sums over the tokens after the step.  dv = G_m^T a, dk = (G_m v + gz_m) phi'(k);
// the in-chunk share of dW[i][i], sum_m a . (R_m v_m + r_m), goes to diag[bh][i].
template <int D, typename T>
__global__ __launch_bounds__(256) void g_kv_causal(const T* __restrict__ Q, const T* __restrict__ K,
                                                   const T* __restrict__ V, const float* __restrict__ dsrec,
                                                   const float* __restrict__ dnum, const float* __restrict__ dden,
                                                   const float* __restrict__ W, T* __restrict__ dK,
                                                   T* __restrict__ dV, float* __restrict__ diag, const Geo g) {
    constexpr int DP = D + 1, E = D * D / 256, CPL = (D + 63) / 64, L = D * D + D;
    __shared__ float gx[D * DP];
    __shared__ float rr[D * DP];
    __shared__ float gz[D], rz[D];
    __shared__ float ub[4][D], ab[4][D], vb[4][D], dn[4][D], dd[4], dsum[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int blk = blockIdx.x;
    const int bh = blk / g.M, i = blk - bh * g.M;
    const int b = bh / g.H, h = bh - b * g.H;
    const float wii = W[(size_t)i * g.M + i];
    const float* src = dsrec + (size_t)blk * L;
    for (int u = tid; u < D * D; u += 256) {
        gx[(u / D) * DP + (u % D)] = src[u];
        rr[(u / D) * DP + (u % D)] = 0.f;
    }
    if (tid < D) {
        gz[tid] = src[D * D + tid];
        rz[tid] = 0.f;
    }
    float dacc = 0.f;
    for (int t0 = (g.T - 1) / 4 * 4; t0 >= 0; t0 -= 4) {
        const int p = t0 + w;
        const bool valid = p < g.T;   // wave-uniform
        const size_t off = valid ? tok_off(g, b, h, i, p) : 0;
        float xk[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int c = lane + 64 * k;
            xk[k] = 0.f;
            if (c >= D) continue;
            float uu = 0.f, aa = 0.f, vv = 0.f, gg = 0.f;
            if (valid) {
                xk[k] = ld1(K + off + c);
                aa = phi_exact(xk[k]);
                vv = ld1(V + off + c);
                uu = phi_exact(ld1(Q + off + c));
                gg = dnum[off + c];
            }
            ub[w][c] = uu;
            ab[w][c] = aa;
            vb[w][c] = vv;
            dn[w][c] = gg;
        }
        if (lane == 0) dd[w] = valid ? dden[off / D] : 0.f;
        __syncthreads();
        if (valid) {
            float ua[4], vd[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) ua[x] = vd[x] = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int c = lane + 64 * k;
                if (c >= D) continue;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    ua[x] += ub[x][c] * ab[w][c];
                    vd[x] += dn[x][c] * vb[w][c];
                }
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) {   // in-step n >= m
                ua[x] = x >= w ? wave_sum64(ua[x]) : 0.f;
                vd[x] = x >= w ? wave_sum64(vd[x]) : 0.f;
            }
            float part = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int x = lane + 64 * k;
                if (x >= D) continue;
                float dvx = 0.f, dvr = 0.f, dkx = gz[x], tr = rz[x];
#pragma unroll 8
                for (int y = 0; y < D; ++y) {
                    dvx += gx[y * DP + x] * ab[w][y];
                    dvr += rr[y * DP + x] * ab[w][y];
                    dkx += gx[x * DP + y] * vb[w][y];
                    tr += rr[x * DP + y] * vb[w][y];
                }
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    dvr += dn[n][x] * ua[n];
                    tr += ub[n][x] * (vd[n] + (n >= w ? dd[n] : 0.f));
                }
                part += ab[w][x] * tr;
                st1(dV + off + x, dvx + wii * dvr);
                st1(dK + off + x, (dkx + wii * tr) * dphi(xk[k]));
            }
            dacc += wave_sum64(part);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const int idx = tid + 256 * r, c = idx / D, e = idx - c * D;
            float t = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) t += ub[ww][c] * dn[ww][e];
            rr[c * DP + e] += t;
        }
        if (tid < D) {
            float t = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) t += ub[ww][tid] * dd[ww];
            rz[tid] += t;
        }
        __syncthreads();
    }
    if (lane == 0) dsum[w] = dacc;
    __syncthreads();
    if (tid == 0) diag[blk] = (dsum[0] + dsum[1]) + (dsum[2] + dsum[3]);
}

template <int D, typename T>
hipError_t run_generic(const GenericBwd& B) {
    const Geo& g = B.g;
    const int nblk = g.BH * g.M, L = D * D + D;
    const T* q = static_cast<const T*>(B.q);
    const T* k = static_cast<const T*>(B.k);
    const T* v = static_cast<const T*>(B.v);
    const T* dout = static_cast<const T*>(B.dout);
    const int causal = B.causal ? 1 : 0;
    auto rec = [&](int i) {
        if (B.events) (void)hipEventRecord(B.events[i], B.stream);
    };
    rec(0);
    g_summary<D, T><<<nblk, 256, 0, B.stream>>>(k, v, B.s, g);
    const int nxc = (L + 255) / 256, nit = (g.M + 15) / 16;
    g_mix<<<g.BH * nit * nxc, 256, 0, B.stream>>>(B.W, B.s, B.st, g.M, L, 0, causal);
    rec(1);
    if (causal)
        g_query_causal<D, T><<<nblk, 256, 0, B.stream>>>(q, k, v, dout, B.st, B.W, static_cast<T*>(B.dq), B.dst,
                                                         B.dnum, B.dden, g);
    else
        g_query<D, T><<<nblk, 256, 0, B.stream>>>(q, dout, B.st, static_cast<T*>(B.dq), B.dst, g);
    rec(2);
    g_mix<<<g.BH * nit * nxc, 256, 0, B.stream>>>(B.W, B.dst, B.ds, g.M, L, 1, causal);
    const int ntile = (g.M + 31) / 32;
    g_dw_partial<<<ntile * ntile * B.nsplit, 256, 0, B.stream>>>(B.dst, B.s, B.part, g.BH, g.M, L, B.nsplit);
    const int nred = (g.M * g.M + 255) / 256;
    if (!causal) {
        g_dw_reduce<<<nred, 256, 0, B.stream>>>(B.part, B.dw, g.M, B.nsplit, nullptr, g.BH);
        rec(3);
        g_kv<D, T><<<nblk, 256, 0, B.stream>>>(k, v, B.ds, static_cast<T*>(B.dk), static_cast<T*>(B.dv), g);
    } else {
        // the key/value side supplies the diagonal of dW, so the reduction follows it
        rec(3);
        g_kv_causal<D, T><<<nblk, 256, 0, B.stream>>>(q, k, v, B.ds, B.dnum, B.dden, B.W, static_cast<T*>(B.dk),
                                                      static_cast<T*>(B.dv), B.diag, g);
        g_dw_reduce<<<nred, 256, 0, B.stream>>>(B.part, B.dw, g.M, B.nsplit, B.diag, g.BH);
    }
    rec(4);
    return hipGetLastError();
}

}  // namespace

hipError_t run_bwd_generic(const GenericBwd& B) {
    if (B.bf16) {
        switch (B.g.D) {
            case 32: return run_generic<32, uint16_t>(B);
            case 64: return run_generic<64, uint16_t>(B);
            case 128: return run_generic<128, uint16_t>(B);
        }
    } else {
        switch (B.g.D) {
            case 32: return run_generic<32, float>(B);
            case 64: return run_generic<64, float>(B);
            case 128: return run_generic<128, float>(B);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace mhla
