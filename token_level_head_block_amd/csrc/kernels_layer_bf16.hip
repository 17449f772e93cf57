// kernels_layer_bf16.hip -- the layer around the MHLA core (171host.com
// repost, section 七, class MHLA ``forward``): LayerNorm and QKV projection,
// optional q/k RMSNorm, the feature map variant, LePE (depthwise 5x5
// convolution of v over the 2D token grid) and the output projection, bf16
// activations with fp32 accumulation, on gfx950.
//
// Projection out[n][c] = sum_k x[n][k] Wt[c][k]: v_mfma_f32_16x16x32_bf16 with
// the weight rows as the A operand and the token rows as the B operand, so a
// lane's four accumulator values are four consecutive output channels of one
// token and leave as one 8-byte store.
//
// LayerNorm is folded into the QKV projection:
//   LN(x) Wt^T + b = rstd_n (x W'^T - mu_n colsum') + b',
//   W' = Wt * gamma (per input channel, bf16), b' = b + Wt beta, colsum'_c = sum_k W'_ck,
// so the MFMA loop streams raw x and the epilogue applies the token's mean
// and inverse deviation.  The products of bf16 values are exact in the fp32
// accumulators, so the subtraction loses accuracy only when |mean| is
// around 1e5 times the deviation.
#include "launch.h"

#include <type_traits>

#include <mhla.h>

namespace mhla {
namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += shfl_xor(x, o);
    return x;
}

// elu(y) + 1 = r for the feature map value r = relu(x) + eps > 0: the core
// then evaluates the relu feature map through its elu + 1.  r >= eps is a
// normal float, so the hardware log2 needs no denormal scaling.
__device__ __forceinline__ float relu_phi_preimage(float x, float eps) {
    const float r = fmaxf(x, 0.f) + eps;
    return r > 1.f ? r - 1.f : __builtin_amdgcn_logf(r) * 0.693147180559945309f;
}

// ---------------------------------------------------------------- weight folding
// One wave per output feature c of the QKV projection:
// W'[c][k] = bf16(Wt[c][k] gamma[k]), colsum'[c] = sum_k W'[c][k] (of the rounded
// values), b'[c] = b[c] + sum_k Wt[c][k] beta[k].
__device__ __forceinline__ void fold_ln_feature(const uint16_t* __restrict__ Wt, const float* __restrict__ gamma,
                                                const float* __restrict__ beta, const float* __restrict__ bias,
                                                uint16_t* __restrict__ Wf, float* __restrict__ colsum,
                                                float* __restrict__ biasf, int K, int c, int lane) {
    const uint16_t* wr = Wt + (size_t)c * K;
    uint16_t* fr = Wf + (size_t)c * K;
    float s = 0.f, t = 0.f;
    for (int k0 = 8 * lane; k0 < K; k0 += 512) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(wr + k0);
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + k0), g1 = *reinterpret_cast<const f32x4*>(gamma + k0 + 4);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(beta + k0), b1 = *reinterpret_cast<const f32x4*>(beta + k0 + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float be[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float w0 = bf_lo(w[j]), w1 = bf_hi(w[j]);
            o[j] = pack_bf16(w0 * g[2 * j], w1 * g[2 * j + 1]);
            s += bf_lo(o[j]) + bf_hi(o[j]);
            t += w0 * be[2 * j] + w1 * be[2 * j + 1];
        }
        *reinterpret_cast<u32x4*>(fr + k0) = o;
    }
    s = wave_sum(s);
    t = wave_sum(t);
    if (lane == 0) {
        colsum[c] = s;
        biasf[c] = (bias ? bias[c] : 0.f) + t;
    }
}

// ---------------------------------------------------------------- token statistics
// mean and 1 / sqrt(var + eps) of each token row of x (biased variance over the
// K channels), once per token: eight lanes per row, one pass of shifted sums
// (x - x0, x0 the row's first element, which keeps them accurate for a large
// mean).  Workgroup = 32 rows.
__device__ __forceinline__ void ln_stats_rows(const uint16_t* __restrict__ X, float* __restrict__ mean,
                                              float* __restrict__ rstd, int R, int K, float eps, int rg) {
    const int tid = threadIdx.x, part = tid & 7;
    const int n = rg * 32 + (tid >> 3);
    const int nc = n < R ? n : R - 1;
    const uint16_t* xr = X + (size_t)nc * K;
    float x0 = 0.f, s1 = 0.f, s2 = 0.f;
    // eight 16-byte pieces of the row per lane in flight at once (addresses
    // clamped inside the row, pieces past it skipped when summed)
    for (int kb = 0; kb < K; kb += 512) {
        u32x4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const u32x4*>(xr + min(kb + 64 * u + 8 * part, K - 8));
        // the row's first element, from the lane with part 0 (the row's lanes are consecutive)
        if (kb == 0) x0 = __shfl(bf_lo(x[0][0]), (tid & 63) & ~7, 64);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool in = kb + 64 * u + 8 * part < K;   // K is a multiple of 8
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float d0 = in ? bf_lo(x[u][j]) - x0 : 0.f, d1 = in ? bf_hi(x[u][j]) - x0 : 0.f;
                s1 += d0 + d1;
                s2 += d0 * d0 + d1 * d1;
            }
        }
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
        s1 += shfl_xor(s1, o);
        s2 += shfl_xor(s2, o);
    }
    if (part == 0 && n < R) {
        const float m1 = s1 / (float)K;
        mean[n] = x0 + m1;
        rstd[n] = 1.f / sqrtf(fmaxf(s2 / (float)K - m1 * m1, 0.f) + eps);
    }
}

// The weight folding and the token statistics in one launch (they are
// independent): workgroups [0, nfold) fold four features each (one per wave),
// the rest take 32 token rows each.
__global__ __launch_bounds__(256) void ln_prepare_bf16(const uint16_t* __restrict__ Wt, const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, const float* __restrict__ bias,
                                                       uint16_t* __restrict__ Wf, float* __restrict__ colsum,
                                                       float* __restrict__ biasf, int nfeat, int nfold,
                                                       const uint16_t* __restrict__ X, float* __restrict__ mean,
                                                       float* __restrict__ rstd, int R, int K, float eps) {
    if ((int)blockIdx.x < nfold) {
        const int c = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
        if (c < nfeat) fold_ln_feature(Wt, gamma, beta, bias, Wf, colsum, biasf, K, c, threadIdx.x & 63);
        return;
    }
    ln_stats_rows(X, mean, rstd, R, K, eps, (int)blockIdx.x - nfold);
}

// ---------------------------------------------------------------- projection GEMM
struct GemmArgs {
    const uint16_t* X;     // [R][K] token rows
    const uint16_t* Wt;    // [Nc][K] weight rows
    const float* bias;     // [Nc] or nullptr
    const float* colsum;   // [Nc] (LayerNorm mode)
    const float* mean;     // [R] token means (LayerNorm mode)
    const float* rstd;     // [R] token inverse deviations (LayerNorm mode)
    uint16_t* dst[3];      // output column ranges [0, split), [split, 2 split), [2 split, 3 split)
    int R, K, Nc, split;
    int phi_cols;          // columns [0, phi_cols) leave as the relu feature map's preimage
    float phi_eps;
};

// Workgroup: 4 waves, tile of 128 output features x 128 tokens, each wave
// 64 x 64 (4 x 4 MFMA tiles).  K in chunks of 64 through one LDS buffer per
// operand; the next chunk's global loads are in flight while the current one
// is multiplied.  36 KB of LDS and 128 registers let four workgroups share a
// compute unit, which hides more of the load latency than a second buffer.  Feature tiles of one token tile sit 8 workgroup ids apart, so
// they run on the same XCD and share its L2 copy of the token rows.
template <bool LN, bool WHOLE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WHOLE ? 4 : 3))) void layer_gemm_bf16(const GemmArgs a) {
    constexpr int TC = 128, TN = 128, KC = 64, STR = KC;
    // Rows of 128 bytes, the 16-byte piece c of row r at piece c ^ ((r / 2) % 8):
    // the sixteen rows of an operand read (and the two rows of eight pieces of a
    // staging write) cover every bank once.
    auto sw = [](int r, int c) { return r * STR + ((c ^ ((r >> 1) & 7)) << 3); };
    constexpr int ESTR = TC + 8;   // epilogue rows of 272 bytes
    constexpr int LDS_E = (TC * STR + TN * STR) > TN * ESTR ? (TC * STR + TN * STR) : TN * ESTR;
    __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_E];   // 34 KB: four workgroups per CU
    uint16_t* const la = lds;
    uint16_t* const lb = lds + TC * STR;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, gq = lane >> 4;
    const int nct = (a.Nc + TC - 1) / TC;
    const int ntt = (a.R + TN - 1) / TN;
    // blockIdx -> (token tile, feature tile) with the feature tiles of a token
    // tile on one XCD (ids congruent modulo 8)
    int ct, nt;
    {
        const int id = blockIdx.x;
        const int full = (ntt / 8) * 8 * nct;   // ids covered by whole groups of 8 token tiles
        if (id < full) {
            const int grp = id / (8 * nct), r = id % (8 * nct);
            nt = grp * 8 + r % 8;
            ct = r / 8;
        } else {
            const int r = id - full;
            nt = (ntt / 8) * 8 + r / nct;
            ct = r % nct;
        }
    }
    const int c0 = ct * TC, n0 = nt * TN;
    const int nk = (a.K + KC - 1) / KC;

    // ---- staging: unit u = (row, 8 k) of a 128 x 64 chunk, 4 per thread and operand,
    // through buffer descriptors.  WHOLE (Nc and R multiples of 128, K of 64:
    // every tile is whole): one lane offset, advanced by scalar offsets.
    // Otherwise the row and the k of every load are clamped so that each
    // address stays inside its tensor, and the values past K are zeroed when
    // the registers go to LDS after the MFMAs of the current chunk, so the
    // loads of the next chunk stay in flight.
    // Byte ranges and offsets are below 2^32 (tensors hold fewer than 2^31
    // elements): unsigned 32-bit arithmetic, passed as the bit patterns.
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.Wt, 0, (int)((uint32_t)a.Nc * (uint32_t)a.K * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.X, 0, (int)((uint32_t)a.R * (uint32_t)a.K * 2u), 0x00020000);
    const int r8 = tid >> 3, k8 = (tid & 7) * 8;
    const int offw = (int)(((uint32_t)(c0 + r8) * (uint32_t)a.K + (uint32_t)k8) * 2u);
    const int offx = (int)(((uint32_t)(n0 + r8) * (uint32_t)a.K + (uint32_t)k8) * 2u);
    u32x4 ra[4], rb[4];
    auto gload = [&](int kc) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if constexpr (WHOLE) {
                const int so = __builtin_amdgcn_readfirstlane((kc * KC + s * 32 * a.K) * 2);
                ra[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, offw, so, 0));
                rb[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, offx, so, 0));
            } else {
                const uint32_t kk = (uint32_t)min(kc * KC + k8, a.K - 8);   // K is a multiple of 8
                const uint32_t cw = (uint32_t)min(c0 + r8 + 32 * s, a.Nc - 1);
                const uint32_t cx = (uint32_t)min(n0 + r8 + 32 * s, a.R - 1);
                ra[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    rw, (int)((cw * (uint32_t)a.K + kk) * 2u), 0, 0));
                rb[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    rx, (int)((cx * (uint32_t)a.K + kk) * 2u), 0, 0));
            }
        }
    };
    const int soff = sw(tid >> 3, tid & 7);
    auto lstore = [&](int kc) {
        const bool partial = !WHOLE && (kc + 1) * KC > a.K;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int u = tid + 256 * s;
            const int off = soff + 32 * STR * s;   // sw(u >> 3, u & 7): rows 32 s apart share the swizzle
            u32x4 x = ra[s], y = rb[s];
            if (partial) {
                const uint32_t m = kc * KC + (u & 7) * 8 < a.K ? 0xffffffffu : 0u;
                x = u32x4{x[0] & m, x[1] & m, x[2] & m, x[3] & m};
                y = u32x4{y[0] & m, y[1] & m, y[2] & m, y[3] & m};
            }
            *reinterpret_cast<u32x4*>(&la[off]) = x;
            *reinterpret_cast<u32x4*>(&lb[off]) = y;
        }
    };

    const int wc = wave & 1, wn = wave >> 1;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < KC / 32; ++ks) {
            u32x4 fa[4], fb[4];
            // sw(16 m + li, c) = (16 m + li) STR + ((c ^ (li / 2 % 8)) << 3)
            const int po = ((ks * 4 + gq) ^ ((li >> 1) & 7)) << 3;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = *reinterpret_cast<const u32x4*>(&la[(64 * wc + 16 * i + li) * STR + po]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                fb[j] = *reinterpret_cast<const u32x4*>(&lb[(64 * wn + 16 * j + li) * STR + po]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
        }
    };
    // One LDS buffer: the next chunk waits in registers while the current one
    // is multiplied, then replaces it between two barriers.
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        if (kc + 1 < nk) gload(kc + 1);
        compute();
        __syncthreads();
        if (kc + 1 < nk) {
            lstore(kc + 1);
            __syncthreads();
        }
    }

    // ---- epilogue: lane (li, gq) holds features c .. c+3 of token n.  The
    // finished values go to LDS as [token][feature] (the staging buffers are
    // free after the last barrier), then every lane stores 16 bytes so that
    // eight lanes write one token's 128 features as whole 128-byte lines.
    uint16_t* et = lds;   // [token][ESTR]
    // PRE: 0 = no column of the tile takes the preimage, 1 = every column, 2 = per column
    auto epilogue = [&](auto pre_kind) {
        constexpr int PRE = decltype(pre_kind)::value;
        float mu[4], rs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = min(n0 + 64 * wn + 16 * j + li, a.R - 1);
            mu[j] = LN ? a.mean[n] : 0.f;
            rs[j] = LN ? a.rstd[n] : 1.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cl = 64 * wc + 16 * i + 4 * gq, c = c0 + cl;
            const int cb = c < a.Nc ? c : a.Nc - 4;   // Nc is a multiple of 4; columns past it are never stored
            const f32x4 bias = a.bias ? *reinterpret_cast<const f32x4*>(a.bias + cb) : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 cs = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (LN) cs = *reinterpret_cast<const f32x4*>(a.colsum + cb);
            const bool pre = PRE == 1 || (PRE == 2 && c < a.phi_cols);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int nl = 64 * wn + 16 * j + li;
                float o[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float x = acc[i][j][v];
                    if constexpr (LN) x = rs[j] * (x - mu[j] * cs[v]);
                    x += bias[v];
                    if constexpr (PRE == 1) o[v] = relu_phi_preimage(x, a.phi_eps);
                    else if constexpr (PRE == 2) o[v] = pre ? relu_phi_preimage(x, a.phi_eps) : x;
                    else o[v] = x;
                }
                *reinterpret_cast<u32x2*>(&et[nl * ESTR + cl]) = u32x2{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
            }
        }
    };
    if (c0 + TC <= a.phi_cols) epilogue(std::integral_constant<int, 1>{});
    else if (c0 >= a.phi_cols) epilogue(std::integral_constant<int, 0>{});
    else epilogue(std::integral_constant<int, 2>{});
    __syncthreads();
#pragma unroll
    for (int s = 0; s < TN * TC / 8 / 256; ++s) {
        const int u = tid + 256 * s;
        const int nl = u >> 4, cl = (u & 15) * 8;   // 16 lanes of 8 features per token
        const int n = n0 + nl, c = c0 + cl;
        if (n >= a.R || c >= a.Nc) continue;          // Nc is a multiple of 8
        const int which = c / a.split, cc = c - which * a.split;   // split is a multiple of 8
        uint16_t* d = which == 0 ? a.dst[0] : (which == 1 ? a.dst[1] : a.dst[2]);
        *reinterpret_cast<u32x4*>(d + (size_t)n * a.split + cc) = *reinterpret_cast<const u32x4*>(&et[nl * ESTR + cl]);
    }
}

// ---------------------------------------------------------------- q/k RMSNorm
// One wave per (token, tensor) row of C channels: x / sqrt(mean(x^2) + eps) * w,
// then the relu feature map's preimage when asked for.
__global__ __launch_bounds__(256) void rms_qk_bf16(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                                   const float* __restrict__ wq, const float* __restrict__ wk,
                                                   int R, int C, float eps, int relu_phi, float phi_eps) {
    const int lane = threadIdx.x & 63;
    const int rowid = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rowid >= 2 * R) return;
    const int which = rowid & 1, n = rowid >> 1;
    uint16_t* xr = (which ? k : q) + (size_t)n * C;
    const float* w = which ? wk : wq;
    float s = 0.f;
    for (int k0 = 8 * lane; k0 < C; k0 += 512) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(xr + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) s += bf_lo(x[j]) * bf_lo(x[j]) + bf_hi(x[j]) * bf_hi(x[j]);
    }
    s = wave_sum(s);
    const float r = 1.f / sqrtf(s / (float)C + eps);
    for (int k0 = 8 * lane; k0 < C; k0 += 512) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(xr + k0);
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + k0), w1 = *reinterpret_cast<const f32x4*>(w + k0 + 4);
        const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float y0 = bf_lo(x[j]) * r * ww[2 * j], y1 = bf_hi(x[j]) * r * ww[2 * j + 1];
            if (relu_phi) {
                y0 = relu_phi_preimage(y0, phi_eps);
                y1 = relu_phi_preimage(y1, phi_eps);
            }
            o[j] = pack_bf16(y0, y1);
        }
        *reinterpret_cast<u32x4*>(xr + k0) = o;
    }
}

// ---------------------------------------------------------------- LePE
// o[n][c] += b[c] + sum_{dy,dx} w[c][dy][dx] v[y+dy-2][x+dx-2][c] (zero outside
// the grid), per batch item on the Y x X grid.  Workgroup = (b, 8 rows x 16
// columns of tokens, 64 channels): a token's 64 channels are one 128-byte line,
// so v's 12 x 20 halo (in LDS) and the read-modify-write of o move whole lines.
// Thread (channel pair, pair of columns) keeps its two channels' 25 weights in
// registers and slides down the 12 input rows, feeding 8 x 2 outputs.
constexpr int LP_TY = 8, LP_TX = 16, LP_TCH = 64;

__global__ __launch_bounds__(256) void lepe_add_bf16(const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                                     const float* __restrict__ w, const float* __restrict__ bias,
                                                     int Y, int X, int C) {
    constexpr int HY = LP_TY + 4, HX = LP_TX + 4, PAIRS = LP_TCH / 2;
    __shared__ __attribute__((aligned(16))) uint32_t vt[HY * HX * PAIRS];   // bf16 channel pairs
    const int tid = threadIdx.x;
    const int ncg = (C + LP_TCH - 1) / LP_TCH, ntx = (X + LP_TX - 1) / LP_TX, nty = (Y + LP_TY - 1) / LP_TY;
    int id = blockIdx.x;
    const int cg = id % ncg; id /= ncg;
    const int tx = id % ntx; id /= ntx;
    const int ty = id % nty;
    const int b = id / nty;
    const int y0 = ty * LP_TY, x0 = tx * LP_TX, ch0 = cg * LP_TCH;
    const int nch = min(LP_TCH, C - ch0);   // 64, or 32 for the last group when C % 64 == 32
    const size_t img = (size_t)b * Y * X;
    const int p = tid & (PAIRS - 1), xg = tid / PAIRS;   // channel pair, pair of output columns
    const int c = ch0 + 2 * p;
    const bool cok = 2 * p < nch;
    const int cw = cok ? c : ch0;
    // halo of v: unit = (position, 8 channels).  Every load of the thread is
    // in flight before the first LDS write: unconditional loads from addresses
    // clamped inside the tensor, the units outside the image or the channels
    // zeroed afterwards.
    constexpr int NU = HY * HX * (LP_TCH / 8), NIT = (NU + 255) / 256;
    u32x4 hv[NIT];
    uint32_t inside = 0;
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
        const int u = min(tid + 256 * k, NU - 1);
        const int part = u % (LP_TCH / 8), pos = u / (LP_TCH / 8);
        const int hy = pos / HX, hx = pos % HX;
        const int yy = y0 + hy - 2, xx = x0 + hx - 2;
        if (yy >= 0 && yy < Y && xx >= 0 && xx < X && part * 8 < nch) inside |= 1u << k;
        const int yc = min(max(yy, 0), Y - 1), xc = min(max(xx, 0), X - 1), pc = min(part * 8, nch - 8);
        hv[k] = *reinterpret_cast<const u32x4*>(V + (img + (size_t)yc * X + xc) * C + ch0 + pc);
    }
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
        const int u = tid + 256 * k;
        const int part = u % (LP_TCH / 8), pos = u / (LP_TCH / 8);
        const uint32_t m = (inside >> k) & 1u ? 0xffffffffu : 0u;
        if (u < NU)
            *reinterpret_cast<u32x4*>(&vt[pos * PAIRS + part * 4]) =
                u32x4{hv[k][0] & m, hv[k][1] & m, hv[k][2] & m, hv[k][3] & m};
    }
    // Weights as bf16 pairs per tap row dy: (w0, w1), (w2, w3), (w4, 0), (0, w4),
    // for v_dot2_f32_bf16 (two products of bf16 values, exact in fp32, added
    // to an fp32 accumulator): three per output row instead of five FMAs.
    uint32_t wq[2][5][4];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int dy = 0; dy < 5; ++dy) {
            const float* wr = w + (size_t)(cw + ch) * 25 + dy * 5;
            wq[ch][dy][0] = pack_bf16(wr[0], wr[1]);
            wq[ch][dy][1] = pack_bf16(wr[2], wr[3]);
            wq[ch][dy][2] = pack_bf16(wr[4], 0.f);
            wq[ch][dy][3] = pack_bf16(0.f, wr[4]);
        }
    const float b0 = bias ? bias[cw] : 0.f, b1 = bias ? bias[cw + 1] : 0.f;
    __syncthreads();
    auto dot2 = [](uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
    };
    float acc[LP_TY][2][2];
#pragma unroll
    for (int oy = 0; oy < LP_TY; ++oy)
#pragma unroll
        for (int ox = 0; ox < 2; ++ox) acc[oy][ox][0] = acc[oy][ox][1] = 0.f;
#pragma unroll
    for (int iy = 0; iy < HY; ++iy) {
        // the window's six columns hold channel pairs (c, c + 1); q[ch][s] pairs
        // columns s and s + 1 of one channel
        uint32_t r[6], q[2][5];
#pragma unroll
        for (int s = 0; s < 6; ++s) r[s] = vt[(iy * HX + 2 * xg + s) * PAIRS + p];
#pragma unroll
        for (int s = 0; s < 5; ++s) {
            q[0][s] = pack_lo(r[s], r[s + 1]);
            q[1][s] = pack_hi(r[s], r[s + 1]);
        }
#pragma unroll
        for (int dy = 0; dy < 5; ++dy) {
            const int oy = iy - dy;
            if (oy < 0 || oy >= LP_TY) continue;
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                // column 0 of the pair: taps on columns 0..4; column 1: on columns 1..5
                float a0 = acc[oy][0][ch], a1 = acc[oy][1][ch];
                a0 = dot2(q[ch][0], wq[ch][dy][0], a0);
                a0 = dot2(q[ch][2], wq[ch][dy][1], a0);
                a0 = dot2(q[ch][4], wq[ch][dy][2], a0);
                a1 = dot2(q[ch][1], wq[ch][dy][0], a1);
                a1 = dot2(q[ch][3], wq[ch][dy][1], a1);
                a1 = dot2(q[ch][4], wq[ch][dy][3], a1);
                acc[oy][0][ch] = a0;
                acc[oy][1][ch] = a1;
            }
        }
    }
    if (!cok) return;
    // o's values at this thread's outputs, all requested before the first
    // store (O is read and written, so loads written between the stores
    // would each wait for the one before; addresses clamped inside the image)
    uint32_t prev[LP_TY][2];
#pragma unroll
    for (int oy = 0; oy < LP_TY; ++oy)
#pragma unroll
        for (int ox = 0; ox < 2; ++ox) {
            const int yy = min(y0 + oy, Y - 1), xx = min(x0 + 2 * xg + ox, X - 1);
            prev[oy][ox] = *reinterpret_cast<const uint32_t*>(O + (img + (size_t)yy * X + xx) * C + c);
        }
#pragma unroll
    for (int oy = 0; oy < LP_TY; ++oy)
#pragma unroll
        for (int ox = 0; ox < 2; ++ox) {
            const int yy = y0 + oy, xx = x0 + 2 * xg + ox;
            if (yy >= Y || xx >= X) continue;
            uint32_t* op = reinterpret_cast<uint32_t*>(O + (img + (size_t)yy * X + xx) * C + c);
            const uint32_t pv = prev[oy][ox];
            *op = pack_bf16(bf_lo(pv) + acc[oy][ox][0] + b0, bf_hi(pv) + acc[oy][ox][1] + b1);
        }
}

}  // namespace

hipError_t run_layer_bf16(const LayerLaunch& L) {
    const int R = L.R, C = L.C;
    auto rec = [&](int i) {
        if (L.events) (void)hipEventRecord(L.events[i], L.stream);
    };
    rec(0);
    // 1. LayerNorm folded into the QKV weights, then the projection
    const int nfold = (3 * C + 3) / 4;
    ln_prepare_bf16<<<nfold + (R + 31) / 32, 256, 0, L.stream>>>(L.w_qkv, L.ln_w, L.ln_b, L.b_qkv, L.wf, L.colsum,
                                                                   L.biasf, 3 * C, nfold, L.x, L.mean, L.rstd, R, C,
                                                                   L.ln_eps);
    GemmArgs a;
    a.X = L.x;
    a.Wt = L.wf;
    a.bias = L.biasf;
    a.colsum = L.colsum;
    a.mean = L.mean;
    a.rstd = L.rstd;
    a.dst[0] = L.q; a.dst[1] = L.k; a.dst[2] = L.v;
    a.R = R; a.K = C; a.Nc = 3 * C; a.split = C;
    a.phi_cols = (L.relu_phi && !L.qn_w) ? 2 * C : 0;
    a.phi_eps = L.phi_eps;
    const int ntt = (R + 127) / 128, nct = (3 * C + 127) / 128;
    if (a.Nc % 128 == 0 && R % 128 == 0 && C % 64 == 0)
        layer_gemm_bf16<true, true><<<ntt * nct, 256, 0, L.stream>>>(a);
    else
        layer_gemm_bf16<true, false><<<ntt * nct, 256, 0, L.stream>>>(a);
    if (L.qn_w)
        rms_qk_bf16<<<(2 * R + 3) / 4, 256, 0, L.stream>>>(L.q, L.k, L.qn_w, L.kn_w, R, C, L.rms_eps, L.relu_phi,
                                                           L.phi_eps);
    rec(1);
    // 2. the core on q, k, v -> o
    hipError_t e = run_bf16(L.core);
    if (e != hipSuccess) return e;
    rec(2);
    // 3. LePE added into o
    if (L.lepe_w) {
        const int nblk = L.B * ((L.Y + LP_TY - 1) / LP_TY) * ((L.X + LP_TX - 1) / LP_TX) * ((C + LP_TCH - 1) / LP_TCH);
        lepe_add_bf16<<<nblk, 256, 0, L.stream>>>(L.v, L.o, L.lepe_w, L.lepe_b, L.Y, L.X, C);
    }
    rec(3);
    // 4. output projection
    GemmArgs b;
    b.X = L.o;
    b.Wt = L.w_out;
    b.bias = L.b_out;
    b.colsum = nullptr;
    b.mean = nullptr;
    b.rstd = nullptr;
    b.dst[0] = L.y; b.dst[1] = L.y; b.dst[2] = L.y;
    b.R = R; b.K = C; b.Nc = C; b.split = C;
    b.phi_cols = 0;
    b.phi_eps = 0.f;
    if (C % 128 == 0 && R % 128 == 0)
        layer_gemm_bf16<false, true><<<ntt * ((C + 127) / 128), 256, 0, L.stream>>>(b);
    else
        layer_gemm_bf16<false, false><<<ntt * ((C + 127) / 128), 256, 0, L.stream>>>(b);
    rec(4);
    return hipGetLastError();
}

}  // namespace mhla
