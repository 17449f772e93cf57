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
//      zt_i< likewise, go to the workspace (fp32 records, or for bf16
//      problems St_i<^T rounded to bf16 and zt_i< in fp32);
//   3. token n at position p of chunk i gets
//        o_n = u^T (St_i< + w P_p) / (u . (zt_i< + w zp_p) + eps),
//      u = phi(q_n), w = W[i][i], P_p, zp_p the chunk's sums of phi(k_m) v_m^T
//      and phi(k_m) over m <= p.
// fp32 arithmetic for the summaries and mixtures; q, k, v and o in bf16 or
// fp32.  fp32 problems run step 3 token by token in fp32 (stream_apply);
// bf16 problems run the causal apply kernel of the one-shot form on the
// mixtures' bf16 operands.
#include "launch.h"

#include <mhla.h>

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

// ---- summaries of the new chunks into the state: workgroup = (b h, chunk r)
// of NG groups of 256 threads.  Group gi takes the chunk's 32-token batches
// gi, gi + NG, ... (the next one's raw loads in flight, in registers, while
// the current one is multiplied from the group's LDS slice); thread t of a
// group owns the TS x TS tile of S at rows TS (t / 16), columns TS (t % 16)
// (TS = d / 16), so each token costs it 2 TS LDS reads for TS^2 products.
// The groups' partial tiles are then added in group order (deterministic).
template <int D, int NG, typename T>
__global__ __launch_bounds__(256 * NG) void stream_summary(const T* __restrict__ K, const T* __restrict__ V,
                                                           float* __restrict__ state, int n_past, int max_chunks,
                                                           const Geo g) {
    // Record of block r: state[(b h) max_chunks + n_past + r] (for sub-chunks:
    // the workspace with max_chunks = the call's sub-chunks and n_past = 0).
    constexpr int TS = D / 16, TB = 32, L = D * D + D, NU = TB * D / 256;
    // staging of every group's batch, reused for the partial sums of groups 1 .. NG-1
    constexpr int NSTAGE = NG * 2 * TB * D, NPART = (NG - 1) * L;
    __shared__ __attribute__((aligned(16))) float lds[NSTAGE > NPART ? NSTAGE : NPART];
    const int tid = threadIdx.x & 255, gi = threadIdx.x >> 8, blk = blockIdx.x;
    float* ka = lds + gi * (2 * TB * D);   // [TB][D] phi(K), then [TB][D] V
    float* va = ka + TB * D;
    const int bh = blk / g.M, r = blk - bh * g.M;
    const int b = bh / g.H, h = bh - b * g.H;
    const int c0 = TS * (tid >> 4), e0 = TS * (tid & 15);
    float acc[TS][TS], zacc = 0.f;
#pragma unroll
    for (int a = 0; a < TS; ++a)
#pragma unroll
        for (int x = 0; x < TS; ++x) acc[a][x] = 0.f;
    T kr[NU], vr[NU];
    auto load = [&](int t0) {
#pragma unroll
        for (int s = 0; s < NU; ++s) {
            const int u = tid + 256 * s, tt = u / D, c = u - tt * D;
            const int p = min(t0 + tt, g.T - 1);   // clamped; tokens past the chunk are zeroed below
            const size_t off = tok_off(g, b, h, r, p) + c;
            kr[s] = K[off];
            vr[s] = V[off];
        }
    };
    // every group runs the same number of rounds (barriers are workgroup-wide)
    const int rounds = ((g.T + TB - 1) / TB + NG - 1) / NG;
    load(TB * gi);
    for (int it = 0; it < rounds; ++it) {
        const int t0 = TB * (gi + NG * it);
        __syncthreads();   // the previous batch's readers are done
#pragma unroll
        for (int s = 0; s < NU; ++s) {
            const int u = tid + 256 * s, tt = u / D, c = u - tt * D;
            const bool ok = t0 + tt < g.T;   // tokens past the chunk contribute nothing
            ka[tt * D + c] = ok ? phi_exact(ld1(&kr[s])) : 0.f;
            va[tt * D + c] = ok ? ld1(&vr[s]) : 0.f;
        }
        __syncthreads();
        if (it + 1 < rounds) load(t0 + TB * NG);
#pragma unroll 2
        for (int tt = 0; tt < TB; ++tt) {
            float kv[TS], vv[TS];
#pragma unroll
            for (int a = 0; a < TS; ++a) {
                kv[a] = ka[tt * D + c0 + a];
                vv[a] = va[tt * D + e0 + a];
            }
#pragma unroll
            for (int a = 0; a < TS; ++a)
#pragma unroll
                for (int x = 0; x < TS; ++x) acc[a][x] += kv[a] * vv[x];
            if (tid < D) zacc += ka[tt * D + tid];
        }
    }
    // groups 1 .. NG-1 leave their tiles (and z) in LDS; group 0 adds them in order
    __syncthreads();
    if (gi > 0) {
        float* part = lds + (gi - 1) * (D * D + D);
#pragma unroll
        for (int a = 0; a < TS; ++a)
#pragma unroll
            for (int x = 0; x < TS; ++x) part[(c0 + a) * D + e0 + x] = acc[a][x];
        if (tid < D) part[D * D + tid] = zacc;
    }
    __syncthreads();
    if (gi > 0) return;
    for (int q = 0; q < NG - 1; ++q) {
        const float* part = lds + q * (D * D + D);
#pragma unroll
        for (int a = 0; a < TS; ++a)
#pragma unroll
            for (int x = 0; x < TS; ++x) acc[a][x] += part[(c0 + a) * D + e0 + x];
        if (tid < D) zacc += part[D * D + tid];
    }
    float* out = state + ((size_t)bh * max_chunks + n_past + r) * L;
#pragma unroll
    for (int a = 0; a < TS; ++a)
#pragma unroll
        for (int x = 0; x < TS; ++x) out[(c0 + a) * D + e0 + x] = acc[a][x];
    if (tid < D) out[D * D + tid] = zacc;
}

// ---- mixtures over earlier chunks: mixed[bh][r][x] = sum_{j < n_past + r}
// W[n_past + r][j] state[bh][j][x].  Workgroup = (b h, 16 new chunks, 64
// record values); its four waves take every fourth earlier chunk, each lane
// one record value, eight chunks' loads in flight at a time; the four partial
// sums are added in wave order through LDS (deterministic).  W rows go
// through LDS in pieces of 256 source chunks.  With St non-null (bf16
// problems) the mixtures leave as the causal apply kernel's operands instead:
// St^T [bh][r][e][c] in bf16 (round to nearest even) and zt [bh][r][d] fp32.
__global__ __launch_bounds__(256) void stream_mix(const float* __restrict__ W, int w_dim,
                                                  const float* __restrict__ state, int max_chunks, int n_past,
                                                  int m_new, float* __restrict__ mixed, int L, int D,
                                                  uint16_t* __restrict__ St, float* __restrict__ Zt) {
    constexpr int XW = 64, RB = 16, UN = 16;
    __shared__ float wt[RB][257];
    __shared__ float part[4][RB][XW];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nxc = (L + XW - 1) / XW, nrt = (m_new + RB - 1) / RB;
    int id = blockIdx.x;
    const int xc = id % nxc;
    id /= nxc;
    const int rt = id % nrt;
    const int bh = id / nrt;
    const int x = xc * XW + lane, r0 = rt * RB;
    const bool xok = x < L;
    const float* src = state + (size_t)bh * max_chunks * L + (xok ? x : 0);
    const int jend = n_past + min(r0 + RB, m_new) - 1;   // the last row's earlier chunks end here
    float acc[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) acc[rr] = 0.f;
    for (int j0 = 0; j0 < jend; j0 += 256) {
        __syncthreads();
        for (int u = tid; u < RB * 256; u += 256) {
            const int rr = u >> 8, jj = u & 255, r = r0 + rr, j = j0 + jj;
            float wv = 0.f;
            if (r < m_new && j < n_past + r) wv = W[(size_t)(n_past + r) * w_dim + j];
            wt[rr][jj] = wv;
        }
        __syncthreads();
        const int jn = min(256, jend - j0);
        // chunks jj = wave, wave + 4, ...: UN loads issued before their products
        for (int jb = wave; jb < jn; jb += 4 * UN) {
            float v[UN];
#pragma unroll
            for (int t = 0; t < UN; ++t) {
                const int jj = jb + 4 * t;
                v[t] = src[(size_t)(j0 + (jj < jn ? jj : jn - 1)) * L];
            }
#pragma unroll
            for (int t = 0; t < UN; ++t) {
                const int jj = jb + 4 * t;
                if (jj < jn) {
#pragma unroll
                    for (int rr = 0; rr < RB; ++rr) acc[rr] += wt[rr][jj] * v[t];
                }
            }
        }
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) part[wave][rr][lane] = acc[rr];
    __syncthreads();
    // thread (rr, lane) for rr = wave, wave + 4, ...: sum of the four waves in order
    for (int rr = wave; rr < RB; rr += 4) {
        const float sum = ((part[0][rr][lane] + part[1][rr][lane]) + part[2][rr][lane]) + part[3][rr][lane];
        if (!xok || r0 + rr >= m_new) continue;
        const size_t rec = (size_t)bh * m_new + r0 + rr;
        if (!St) {
            mixed[rec * L + x] = sum;
        } else if (x < D * D) {
            const int c = x / D, e = x - c * D;
            St[rec * (D * D) + e * D + c] = (uint16_t)(pack_bf16(sum, 0.f) & 0xffffu);
        } else {
            Zt[rec * D + (x - D * D)] = sum;
        }
    }
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

// ---- long chunks in sub-chunks (bf16 problems): a chunk's state record is
// the sum of its cp sub-chunk summaries (added in sub-chunk order); sub-chunk
// t of new chunk r gets the operands of
//   St< = mixed[r] + W[i][i] sum_{t' < t} Ssub[r cp + t'],  i = n_past + r
// (zt< likewise), as St<^T in bf16 and zt< in fp32.
__global__ __launch_bounds__(256) void stream_fold(const float* __restrict__ ssub, float* __restrict__ state,
                                                   int m_new, int cp, int max_chunks, int n_past, int L, int nbh) {
    const size_t x = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= (size_t)nbh * m_new * L) return;
    const size_t rec = x / L, e = x - rec * L;
    const int bh = (int)(rec / m_new), r = (int)(rec - (size_t)bh * m_new);
    const float* src = ssub + ((size_t)bh * m_new * cp + (size_t)r * cp) * L + e;
    float sum = 0.f;
    for (int t = 0; t < cp; ++t) sum += src[(size_t)t * L];
    state[((size_t)bh * max_chunks + n_past + r) * L + e] = sum;
}

// Workgroup = (b h, chunk r, 256 record elements x); each thread walks the
// chunk's sub-chunks in order with the running prefix sum of their summaries.
template <int D>
__global__ __launch_bounds__(256) void stream_sub_operands(const float* __restrict__ mixed,
                                                           const float* __restrict__ ssub, const float* __restrict__ W,
                                                           int w_dim, int n_past, int m_new, int cp,
                                                           uint16_t* __restrict__ St, float* __restrict__ Zt) {
    constexpr int L = D * D + D, NXC = (L + 255) / 256;
    const int xc = blockIdx.x % NXC, br = blockIdx.x / NXC;   // br = (b h) m_new + r
    const int bh = br / m_new, r = br - bh * m_new;
    const int x = xc * 256 + threadIdx.x;
    if (x >= L) return;
    const float w = W[(size_t)(n_past + r) * (w_dim + 1)];
    const float m = mixed[(size_t)br * L + x];
    const float* sb = ssub + (size_t)br * cp * L + x;        // sub-chunk records r cp + t
    const int c = x / D, e = x - c * D;                       // S element (c, e) for x < D*D
    float prefix = 0.f;
    for (int t = 0; t < cp; ++t) {
        const size_t blk = (size_t)br * cp + t;               // (b h) (m_new cp) + r cp + t
        const float val = m + w * prefix;
        if (x < D * D) St[blk * (D * D) + e * D + c] = (uint16_t)(pack_bf16(val, 0.f) & 0xffffu);
        else Zt[blk * D + (x - D * D)] = val;
        prefix += sb[(size_t)t * L];
    }
}

template <int D, typename T>
hipError_t run_stream(const StreamLaunch& S) {
    const Geo& g = S.g;
    const int L = D * D + D, nblk = g.BH * g.M;
    const T* q = static_cast<const T*>(S.q);
    const T* k = static_cast<const T*>(S.k);
    const T* v = static_cast<const T*>(S.v);
    constexpr int NG = D == 128 ? 2 : 4;   // token groups per chunk (LDS: 64 KB)
    if constexpr (sizeof(T) == 2) {
        if (S.cp > 1) {
            // Long chunks: summaries per sub-chunk, folded into the state; the
            // chunks' mixtures over earlier chunks in fp32; operands per
            // sub-chunk; the causal apply on the sub-chunks.
            const Geo& gs = S.gs;
            const int nsub = gs.BH * gs.M;
            stream_summary<D, NG, T><<<nsub, 256 * NG, 0, S.stream>>>(k, v, S.ssub, 0, gs.M, gs);
            const size_t nf = (size_t)g.BH * g.M * L;
            stream_fold<<<(unsigned)((nf + 255) / 256), 256, 0, S.stream>>>(S.ssub, S.state, g.M, S.cp, S.max_chunks,
                                                                           S.n_past, L, g.BH);
            const int nxc = (L + 63) / 64, nrt = (g.M + 15) / 16;
            stream_mix<<<g.BH * nrt * nxc, 256, 0, S.stream>>>(S.W, S.w_dim, S.state, S.max_chunks, S.n_past, g.M,
                                                                S.mixed, L, D, nullptr, nullptr);
            stream_sub_operands<D><<<g.BH * g.M * ((L + 255) / 256), 256, 0, S.stream>>>(
                S.mixed, S.ssub, S.W, S.w_dim, S.n_past, g.M, S.cp, S.st, S.zt);
            Launch La{};
            La.q = q; La.k = k; La.v = v;
            La.W = S.W + (size_t)S.n_past * (S.w_dim + 1);
            La.out = S.out;
            La.st = S.st;
            La.zt = S.zt;
            La.g = gs;   // WD = cp: sub-chunk a reads W's diagonal of its chunk a / cp
            La.stream = S.stream;
            La.path = MHLA_PATH_CAUSAL;
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            return launch_causal_apply_bf16(La, S.w_dim);
        }
    }
    stream_summary<D, NG, T><<<nblk, 256 * NG, 0, S.stream>>>(k, v, S.state, S.n_past, S.max_chunks, g);
    const int nxc = (L + 63) / 64, nrt = (g.M + 15) / 16;
    constexpr bool BF = sizeof(T) == 2;
    stream_mix<<<g.BH * nrt * nxc, 256, 0, S.stream>>>(S.W, S.w_dim, S.state, S.max_chunks, S.n_past, g.M, S.mixed,
                                                        L, D, BF ? S.st : nullptr, BF ? S.zt : nullptr);
    if constexpr (sizeof(T) == 2) {
        // bf16: the causal apply kernel of the one-shot form (matrix cores,
        // whole chunks through LDS) on the mixtures, which stream_mix wrote
        // as bf16 operands; W[i][i]
        // of global chunk n_past + r is W0[r * w_dim + r], W0 = W + n_past (w_dim + 1).
        Launch L{};
        L.q = q; L.k = k; L.v = v;
        L.W = S.W + (size_t)S.n_past * (S.w_dim + 1);
        L.out = S.out;
        L.st = S.st;
        L.zt = S.zt;
        L.g = g;
        L.stream = S.stream;
        L.path = MHLA_PATH_CAUSAL;
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_causal_apply_bf16(L, S.w_dim);
    } else {
        stream_apply<D, T><<<nblk, D, 0, S.stream>>>(q, k, v, S.mixed, S.W, S.w_dim, S.n_past, static_cast<T*>(S.out), g);
        return hipGetLastError();
    }
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
