// kernels_stream.hip -- stateful causal execution: a sequence arrives as calls
// of whole chunks, and a state of fp32 chunk summaries carries everything the
// later chunks need (the method keeps linear cost and supports streaming:
// paperlayer.ai summary, key points, and appendix B "Causal MHLA").
//
// A call with chunks r = 0 .. M_new-1 of the new tokens, global chunk indices
// i = n_past + r, state records [S_j | z_j] (S as [c][e]) of every chunk
// j < n_past, and coefficients W[i][j] (row-major, leading dimension w_dim):
//   1. the new chunks' summaries go to the state at slots n_past + r;
//   2. their mixtures over earlier chunks, St_i< = sum_{j<i} W[i][j] S_j and
//      zt_i< likewise, go to the workspace;
//   3. token n at position p of chunk i gets
//        o_n = u^T (St_i< + w P_p) / (u . (zt_i< + w zp_p) + eps),
//      u = phi(q_n), w = W[i][i], P_p, zp_p the chunk's sums of phi(k_m) v_m^T
//      and phi(k_m) over m <= p.
// fp32 arithmetic; q, k, v and o in bf16 or fp32.
#include "launch.h"

namespace mhla {
namespace {

__device__ __forceinline__ float ld1(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ void st1(uint16_t* p, float x) { *p = (uint16_t)(pack_bf16(x, 0.f) & 0xffffu); }
__device__ __forceinline__ void st1(float* p, float x) { *p = x; }

// Raster token of position p of chunk r and the element offset of (b, n, h, 0).
__device__ __forceinline__ size_t tok_off(const Geo& g, int b, int h, int r, int p) {
    const int n = block_origin(g, r) + in_block(g, p);
    return (((size_t)b * g.N + n) * g.H + h) * g.D;
}

// ---- summaries of the new chunks into the state: workgroup = (b h, chunk r),
// each thread owns d*d/256 entries of S; tokens in batches of 16 through LDS.
template <int D, typename T>
__global__ __launch_bounds__(256) void stream_summary(const T* __restrict__ K, const T* __restrict__ V,
                                                      float* __restrict__ state, int n_past, int max_chunks,
                                                      const Geo g) {
    constexpr int E = D * D / 256, TB = 16, L = D * D + D;
    __shared__ float ka[TB][D], va[TB][D];
    const int tid = threadIdx.x, blk = blockIdx.x;
    const int bh = blk / g.M, r = blk - bh * g.M;
    const int b = bh / g.H, h = bh - b * g.H;
    float acc[E], zacc = 0.f;
#pragma unroll
    for (int x = 0; x < E; ++x) acc[x] = 0.f;
    for (int t0 = 0; t0 < g.T; t0 += TB) {
        __syncthreads();
        for (int u = tid; u < TB * D; u += 256) {
            const int tt = u / D, c = u - tt * D, p = t0 + tt;
            float kv = 0.f, vv = 0.f;   // tokens past the chunk contribute nothing
            if (p < g.T) {
                const size_t off = tok_off(g, b, h, r, p) + c;
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
            for (int x = 0; x < E; ++x) {
                const int idx = tid + 256 * x, c = idx / D, e = idx - c * D;
                acc[x] += ka[tt][c] * va[tt][e];
            }
            if (tid < D) zacc += ka[tt][tid];
        }
    }
    float* out = state + ((size_t)bh * max_chunks + n_past + r) * L;
#pragma unroll
    for (int x = 0; x < E; ++x) out[tid + 256 * x] = acc[x];
    if (tid < D) out[D * D + tid] = zacc;
}

// ---- mixtures over earlier chunks: mixed[bh][r][x] = sum_{j < n_past + r}
// W[n_past + r][j] state[bh][j][x].  Workgroup = (b h, 16 new chunks, 256
// record values); W rows go through LDS in pieces of 256 source chunks.
__global__ __launch_bounds__(256) void stream_mix(const float* __restrict__ W, int w_dim,
                                                  const float* __restrict__ state, int max_chunks, int n_past,
                                                  int m_new, float* __restrict__ mixed, int L) {
    __shared__ float wt[16][257];
    const int tid = threadIdx.x;
    const int nxc = (L + 255) / 256, nrt = (m_new + 15) / 16;
    int id = blockIdx.x;
    const int xc = id % nxc;
    id /= nxc;
    const int rt = id % nrt;
    const int bh = id / nrt;
    const int x = xc * 256 + tid, r0 = rt * 16;
    const bool xok = x < L;
    const float* src = state + (size_t)bh * max_chunks * L + (xok ? x : 0);
    const int jend = n_past + min(r0 + 16, m_new) - 1;   // the last row's earlier chunks end here
    float acc[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) acc[rr] = 0.f;
    for (int j0 = 0; j0 < jend; j0 += 256) {
        __syncthreads();
        for (int u = tid; u < 16 * 256; u += 256) {
            const int rr = u >> 8, jj = u & 255, r = r0 + rr, j = j0 + jj;
            float wv = 0.f;
            if (r < m_new && j < n_past + r) wv = W[(size_t)(n_past + r) * w_dim + j];
            wt[rr][jj] = wv;
        }
        __syncthreads();
        const int jn = min(256, jend - j0);
        for (int jj = 0; jj < jn; ++jj) {
            const float v = src[(size_t)(j0 + jj) * L];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) acc[rr] += wt[rr][jj] * v;
        }
    }
    if (!xok) return;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
        if (r0 + rr < m_new) mixed[((size_t)bh * m_new + r0 + rr) * L + x] = acc[rr];
}

// ---- outputs of the new chunks: workgroup = (b h, chunk r) of D threads;
// thread e keeps column e of C = St_i< + w P in registers and walks the
// chunk's tokens in order, adding each token's phi(k) v^T before reading C
// for its query; zeta = zt_i< + w zp lives in LDS.
template <int D, typename T>
__global__ __launch_bounds__(D) void stream_apply(const T* __restrict__ Q, const T* __restrict__ K,
                                                  const T* __restrict__ V, const float* __restrict__ mixed,
                                                  const float* __restrict__ W, int w_dim, int n_past,
                                                  T* __restrict__ O, const Geo g) {
    constexpr int L = D * D + D;
    __shared__ float zs[D], ua[D], aa[D];
    const int e = threadIdx.x;
    const int blk = blockIdx.x;
    const int bh = blk / g.M, r = blk - bh * g.M;
    const int b = bh / g.H, h = bh - b * g.H;
    const int i = n_past + r;
    const float w = W[(size_t)i * w_dim + i];
    const float* rec = mixed + (size_t)blk * L;
    float col[D];
#pragma unroll
    for (int c = 0; c < D; ++c) col[c] = rec[c * D + e];
    zs[e] = rec[D * D + e];
    for (int p = 0; p < g.T; ++p) {
        const size_t off = tok_off(g, b, h, r, p);
        const float a = phi_exact(ld1(K + off + e));
        const float vv = ld1(V + off + e);
        __syncthreads();   // the previous token's reads of ua, aa and zs are done
        ua[e] = phi_exact(ld1(Q + off + e));
        aa[e] = a;
        zs[e] += w * a;
        __syncthreads();
        float num = 0.f, den = 0.f;   // every thread forms den = u . zeta itself, in the same order
#pragma unroll
        for (int c = 0; c < D; ++c) {
            col[c] += w * aa[c] * vv;
            num += ua[c] * col[c];
            den += ua[c] * zs[c];
        }
        st1(O + off + e, num / (den + g.eps));
    }
}

template <int D, typename T>
hipError_t run_stream(const StreamLaunch& S) {
    const Geo& g = S.g;
    const int L = D * D + D, nblk = g.BH * g.M;
    const T* q = static_cast<const T*>(S.q);
    const T* k = static_cast<const T*>(S.k);
    const T* v = static_cast<const T*>(S.v);
    stream_summary<D, T><<<nblk, 256, 0, S.stream>>>(k, v, S.state, S.n_past, S.max_chunks, g);
    const int nxc = (L + 255) / 256, nrt = (g.M + 15) / 16;
    stream_mix<<<g.BH * nrt * nxc, 256, 0, S.stream>>>(S.W, S.w_dim, S.state, S.max_chunks, S.n_past, g.M, S.mixed,
                                                        L);
    stream_apply<D, T><<<nblk, D, 0, S.stream>>>(q, k, v, S.mixed, S.W, S.w_dim, S.n_past, static_cast<T*>(S.out), g);
    return hipGetLastError();
}

}  // namespace

hipError_t run_causal_stream(const StreamLaunch& S) {
    if (S.bf16) {
        switch (S.g.D) {
            case 32: return run_stream<32, uint16_t>(S);
            case 64: return run_stream<64, uint16_t>(S);
            case 128: return run_stream<128, uint16_t>(S);
        }
    } else {
        switch (S.g.D) {
            case 32: return run_stream<32, float>(S);
            case 64: return run_stream<64, float>(S);
            case 128: return run_stream<128, float>(S);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace mhla
