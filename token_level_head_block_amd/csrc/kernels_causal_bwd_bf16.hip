// kernels_causal_bwd_bf16.hip -- gradients of the causal chunkwise form of
// MHLA (paperlayer.ai summary, appendix B "Causal MHLA"; W learned, section 4
// "Multi-Head Mixing") for bf16 inputs with d = 32 or 64, chunks contiguous in
// raster order, on the matrix cores of gfx950.
//
// Chunk i, w = W[i,i], u = phi(q), a = phi(k), g = dL/do; the mixtures of the
// earlier chunks St_i<, zt_i< come from the summary and causal mixing kernels.
// With P[n,m] = u_n . a_m and the mask m <= n inside the chunk:
//   num_n = St_i<^T u_n + w sum_m P[n,m] v_m,  den_n = u_n . zt_i< + w sum_m P[n,m] + eps
//   dnum_n = g_n / den_n,  dden_n = -(g_n . num_n) / den_n^2
//   X[n,m] = v_m . dnum_n + dden_n = (v_m . g_n) / den_n + dden_n
//   dq_n  = (St_i< dnum_n + zt_i< dden_n + w sum_m X[n,m] a_m) * phi'(q_n)
//   dSt_i< = sum_n u_n dnum_n^T,  dzt_i< = sum_n u_n dden_n
//   dW[i,i] (this pair's share) = sum_n,m P[n,m] X[n,m]
//           = sum_n dnum_n . (sum_m P[n,m] v_m) + dden_n sum_m P[n,m]
//   Gx_i = sum_{k > i} W[k,i] dSt_k<,  gzx_i likewise (transposed causal mixing)
//   dv_m = Gx_i^T a_m + w sum_{n >= m} P[n,m] dnum_n
//   dk_m = (Gx_i v_m + gzx_i + w sum_{n >= m} X[n,m] u_n) * phi'(k_m)
// The masked T x T products run per 16-token group pair on
// v_mfma_f32_16x16x32_bf16 (scores, contraction over channels) and
// v_mfma_f32_16x16x16_bf16 (contraction over 4 tokens per lane), as in the
// forward's causal apply.  dnum is never rounded: products take g itself (the
// exact bf16 input) and scale by 1 / den in fp32, so X, whose two terms
// cancel where v_m is close to o_n, is formed in fp32 from exact products;
// per token only 1 / den and dden pass from the query side to the key side.
#include "launch.h"
#include "bf16_shared.h"

#include <type_traits>

#include <mhla.h>

namespace mhla {
namespace {

// Channel of MFMA output row rho of row tile r: lane (t, gq) holds rows
// 4 gq + v of every tile, i.e. channels kk * 32 + 8 gq + s with kk = r / 2 and
// s = 4 (r % 2) + v -- exactly the k-slots that the same lane supplies in a
// 16x16x32 operand with k = channel, and eight consecutive channels per kk
// for 16-byte loads and stores.
__device__ __forceinline__ constexpr int och(int r, int rho) {
    return (r >> 1) * 32 + 8 * (rho >> 2) + 4 * (r & 1) + (rho & 3);
}

// XOR swizzle of the 8-byte pieces (4 tokens) in a row of a transposed tile:
// piece p of row c sits at p ^ tsw(c).  The staging writes (eight lanes on
// rows 8 apart) then fall on different banks, and the operand reads (rows
// och(r, li)) keep their spread.
__device__ __forceinline__ constexpr int tsw(int row) { return (row >> 3) & 7; }

// Element offset in a transposed tile of the operand piece 4 k + gq of row
// och(r, li) (k: 16-token group).  With d <= 64, tsw(och(r, li)) is
// 4 (r / 2) + li / 4, so the swizzle splits into a per-lane part and
// k ^ (r / 2).
__device__ __forceinline__ int tr_piece(int r, int li, int gq, int k, int vstr) {
    return och(r, li) * vstr + 4 * (gq ^ (li >> 2)) + 16 * (k ^ (r >> 1));
}

__device__ __forceinline__ u32x4 phi_words(const u32x4& x) {
    u32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = pack_bf16(phi_fast(bf_lo(x[j])), phi_fast(bf_hi(x[j])));
    return y;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

constexpr int kRF = 0x00020000;   // buffer descriptor flags (raw buffer, 32-bit offsets)

// One tile's global loads, held in registers: the rows source in 16-byte
// pieces of token rows, the transposed source as 4 tokens x 8 channels per
// unit.  Loading the next tile into them before the current one is
// multiplied keeps its loads in flight during the MFMAs.
template <int D, int NW>
struct TileRegs {
    static constexpr int NT = 64 * NW, KT = 32 * NW;
    static constexpr int KU = KT * D / 8 / NT;
    static constexpr int VU = (KT / 4 * (D / 8) + NT - 1) / NT;
    u32x4 kx[KU], vx[VU][4];
};

// Tokens at or past T read as the chunk's last token.
template <int D, int NW>
__device__ __forceinline__ void load_tile(TileRegs<D, NW>& R, __amdgpu_buffer_rsrc_t rr, __amdgpu_buffer_rsrc_t rt,
                                          int kt, int T, int rowb) {
    using TR = TileRegs<D, NW>;
    const int tid = threadIdx.x;
    auto tok = [&](int p) { return (p < T ? p : T - 1) * rowb; };
#pragma unroll
    for (int s = 0; s < TR::KU; ++s) {
        const int u = tid + TR::NT * s;
        R.kx[s] = ld16(rr, tok(kt * TR::KT + u / (D / 8)) + (u % (D / 8)) * 16);
    }
#pragma unroll
    for (int s = 0; s < TR::VU; ++s) {
        const int u = tid + TR::NT * s;
        const int kq = u / (D / 8), c8 = u % (D / 8);
        if (u < TR::KT / 4 * (D / 8)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) R.vx[s][j] = ld16(rt, tok(kt * TR::KT + 4 * kq + j) + c8 * 16);
        }
    }
}

// Writes a loaded tile of KT tokens (positions kt KT ..) of a chunk to LDS:
//   rows[key][channel] from the rows source, phi applied if PHI_R;
//   tr[channel][key]   from the transposed source, phi applied if PHI_T (row
//     stride KT + 4 and the pieces swizzled by tsw: the writes and the
//     operand reads share fewer banks);
// tokens past T as zeros where ZERO_R / ZERO_T ask for it (per-token
// gradients that must not count).
template <int D, int NW, bool PHI_R, bool ZERO_R, bool PHI_T, bool ZERO_T>
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ rows, uint16_t* __restrict__ tr,
                                           const TileRegs<D, NW>& R, int kt, int T) {
    using TR = TileRegs<D, NW>;
    constexpr int KSTR = D + 8, VSTR = TR::KT + 4;
    const int tid = threadIdx.x;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < TR::KU; ++s) {
        const int u = tid + TR::NT * s;
        const int key = u / (D / 8);
        u32x4 y = PHI_R ? phi_words(R.kx[s]) : R.kx[s];
        if (ZERO_R && kt * TR::KT + key >= T) y = zero;
        *reinterpret_cast<u32x4*>(rows + key * KSTR + (u % (D / 8)) * 8) = y;
    }
#pragma unroll
    for (int s = 0; s < TR::VU; ++s) {
        const int u = tid + TR::NT * s;
        const int kq = u / (D / 8), c8 = u % (D / 8);
        if (u < TR::KT / 4 * (D / 8)) {
            u32x4 y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                y[j] = PHI_T ? phi_words(R.vx[s][j]) : R.vx[s][j];
                if (ZERO_T && kt * TR::KT + 4 * kq + j >= T) y[j] = zero;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = c8 * 8 + 2 * j;   // rows row and row + 1 share tsw
                uint16_t* d0 = tr + row * VSTR + 4 * (kq ^ tsw(row));
                *reinterpret_cast<u32x2*>(d0) = u32x2{pack_lo(y[0][j], y[1][j]), pack_lo(y[2][j], y[3][j])};
                *reinterpret_cast<u32x2*>(d0 + VSTR) = u32x2{pack_hi(y[0][j], y[1][j]), pack_hi(y[2][j], y[3][j])};
            }
        }
    }
}

// Loads and writes one tile (store_tile's layouts).
template <int D, int NW, bool PHI_R, bool ZERO_R, bool PHI_T, bool ZERO_T>
__device__ __forceinline__ void stage_tile(uint16_t* __restrict__ rows, uint16_t* __restrict__ tr,
                                           __amdgpu_buffer_rsrc_t rr, __amdgpu_buffer_rsrc_t rt, int kt, int T,
                                           int rowb) {
    TileRegs<D, NW> R;
    load_tile<D, NW>(R, rr, rt, kt, T, rowb);
    store_tile<D, NW, PHI_R, ZERO_R, PHI_T, ZERO_T>(rows, tr, R, kt, T);
}

// A d x d record stored as [e][c] (element (c, e) at e d + c) -> LDS as
// [c][e] with row stride KSTR: the operand with rows c and k = e.
template <int D, int NT>
__device__ __forceinline__ void stage_transposed_record(uint16_t* __restrict__ dst, __amdgpu_buffer_rsrc_t r) {
    constexpr int KSTR = D + 8, SU = (D * D / 8 + NT - 1) / NT;
    const int tid = threadIdx.x;
    u32x4 x[SU];
#pragma unroll
    for (int s = 0; s < SU; ++s) {
        const int u = tid + NT * s;
        if (u < D * D / 8) x[s] = ld16(r, u * 16);
    }
#pragma unroll
    for (int s = 0; s < SU; ++s) {
        const int u = tid + NT * s;
        if (u < D * D / 8) {
            const int e = u / (D / 8), c0 = (u % (D / 8)) * 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dst[(c0 + 2 * j) * KSTR + e] = (uint16_t)(x[s][j] & 0xffffu);
                dst[(c0 + 2 * j + 1) * KSTR + e] = (uint16_t)(x[s][j] >> 16);
            }
        }
    }
}

// =====================================================================
// Query side.  Workgroup = (b, chunk i, head h) with NW waves; a tile is
// KT = 32 NW tokens and wave w takes the tile's 16-query groups w and
// 2 NW - 1 - w (equal masked work for every wave).  Per query tile:
//  phase 1: phi(K) rows and V^T of each key tile up to it in LDS; scores
//    phi(k) . phi(q) masked to m <= n, rounded to bf16 (unscaled), summed
//    into sum_m P v and sum_m P; then W[i,i], the mixture (St_i< from the
//    record, zt_i< as bf16 high and low parts), 1 / den and dden, which go
//    to HBM for the key/value side;
//  phase 2: V rows and phi(K)^T of each key tile in LDS; X = (v . g) / den +
//    dden, masked, times W[i,i], as bf16 high and low parts into du += X a;
//    (St_i< g) / den from the transposed record in LDS; dq = (du + zt_i<
//    dden) phi'(q);
//  then dSt_i< += u dnum^T and dzt_i< += u dden with the 16 tokens as k: an
//    MFMA against the identity turns each lane's token row into the
//    operand with 4 tokens per lane.
// The waves' partial dSt, dzt and dW[i,i] terms are added in a fixed order
// through LDS; the record [dSt_i< as [e][c] | dzt_i<] is stored in bf16.
// =====================================================================
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 1 ? 1 : 2))) void causal_bwd_query_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ St, const float* __restrict__ Zt,
    const float* __restrict__ W, uint16_t* __restrict__ dQ, float* __restrict__ tsc, uint16_t* __restrict__ dSt,
    float* __restrict__ diag, const Geo g) {
    constexpr int RT = D / 16, KS = D / 32, REC = D * D + D;
    constexpr int NT = 64 * NW, KT = 32 * NW, NKG = KT / 16;
    constexpr int KSTR = D + 8, VSTR = KT + 4;
    static_assert(D <= 64, "tr_piece assumes at most four row tiles");
    constexpr int STAGE_B = (KT * KSTR + D * VSTR) * 2;
    constexpr int SLOT = RT * RT * 4 * 64;   // floats of one wave's dSt partial
    constexpr int RED_B = ((NW / 2) * SLOT + NW * D) * 4;
    constexpr int UNION_B = STAGE_B > RED_B ? STAGE_B : RED_B;
    __shared__ __attribute__((aligned(16))) unsigned char smem[UNION_B];   // key tiles, then the reduction
    __shared__ __attribute__((aligned(16))) uint16_t stl[D * KSTR];   // St_i< as [c][e]
    __shared__ __attribute__((aligned(16))) float zl[D];
    __shared__ __attribute__((aligned(16))) float acl[SLOT];   // dSt_i< sums, in wave 0's lane order
    __shared__ float zacl[D];                                   // dzt_i< sums
    __shared__ float dr[NW];
    uint16_t* kl = reinterpret_cast<uint16_t*>(smem);
    uint16_t* vl = kl + KT * KSTR;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, gq = lane >> 4;
    const WgCoord wgc = wg_coord(g, blockIdx.x);
    const int b = __builtin_amdgcn_readfirstlane(wgc.b);
    const int h = __builtin_amdgcn_readfirstlane(wgc.hg);
    const int i = __builtin_amdgcn_readfirstlane(wgc.j);
    const int blk = (b * g.H + h) * g.M + i;
    const float wii = W[(size_t)i * g.M + i];

    const int row = g.H * D, T = g.T, rowb = row * 2;
    const int origin = block_origin(g, i);
    const int base = (b * g.N + origin) * row + h * D;
    const int crange = (T * row - h * D) * 2;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + base), 0, crange, kRF);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), 0, crange, kRF);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), 0, crange, kRF);
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc((void*)(dO + base), 0, crange, kRF);
    const __amdgpu_buffer_rsrc_t rdq = __builtin_amdgcn_make_buffer_rsrc((void*)(dQ + base), 0, crange, kRF);
    const int dbase = (b * g.N + origin) * g.H + h;   // (b, n, h) index of the chunk's first token
    const __amdgpu_buffer_rsrc_t rts =
        __builtin_amdgcn_make_buffer_rsrc((void*)(tsc + 2 * (size_t)dbase), 0, (T * g.H - h) * 8, kRF);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(St + (size_t)blk * (D * D)), 0, D * D * 2, kRF);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc((void*)(Zt + (size_t)blk * D), 0, D * 4, kRF);
    auto tok = [&](int p) { return (p < T ? p : T - 1) * rowb; };
    const u32x2 ones = u32x2{0x3f803f80u, 0x3f803f80u};
    const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
    // Identity operands: slot s of lane (li, gq) is 1 where 8 gq + s = 16 hf + li.
    u32x4 idb[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k0 = 8 * gq + 2 * j - 16 * hf;
            idb[hf][j] = (k0 == li ? 0x3f80u : 0u) | (k0 + 1 == li ? 0x3f800000u : 0u);
        }

    float dgacc = 0.f;   // this lane's share of the pair's dW[i,i] terms

    const int nit = (T + 15) >> 4;
    const int nqt = (T + KT - 1) / KT;
    for (int qt = 0; qt < nqt; ++qt) {
        const int ga = qt * NKG + w, gb = qt * NKG + NKG - 1 - w;
        const bool va = ga < nit, vb = gb < nit;   // gb > ga: vb implies va
        const int na = 16 * ga + li, nb = 16 * gb + li;
        u32x4 ua[KS], ub[KS];   // raw q, then phi(q): B operands, k = channel kk 32 + 8 gq + s
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            ua[kk] = ld16(rq, tok(na) + (kk * 32 + gq * 8) * 2);
            ub[kk] = ld16(rq, tok(nb) + (kk * 32 + gq * 8) * 2);
        }
        f32x4 acca[RT], accb[RT], pa = f32x4{0.f, 0.f, 0.f, 0.f}, pb = pa;
#pragma unroll
        for (int r = 0; r < RT; ++r) acca[r] = accb[r] = f32x4{0.f, 0.f, 0.f, 0.f};

        // ---- phase 1: sum_m P v and sum_m P over the key tiles up to this one
        for (int kt = 0; kt <= qt; ++kt) {
            __syncthreads();   // earlier readers of kl, vl are done
            stage_tile<D, NW, true, false, false, false>(kl, vl, rk, rv, kt, T, rowb);
            if (qt == 0 && kt == 0 && tid < D / 4)
                *reinterpret_cast<f32x4*>(zl + 4 * tid) = __builtin_bit_cast(f32x4, ld16(rz, 16 * tid));
            __syncthreads();
            if (kt == 0) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    ua[kk] = phi_words(ua[kk]);
                    ub[kk] = phi_words(ub[kk]);
                }
            }
            const int top = (vb ? gb : ga) - kt * NKG;
            const int nk = !va ? 0 : (top < NKG - 1 ? top + 1 : NKG);
            for (int kg = 0; kg < nk; ++kg) {
                u32x4 ak[KS];
                u32x2 av[RT];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    ak[kk] = *reinterpret_cast<const u32x4*>(kl + (16 * kg + li) * KSTR + kk * 32 + gq * 8);
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    av[r] = *reinterpret_cast<const u32x2*>(vl + tr_piece(r, li, gq, kg, VSTR));
                const int kgg = kt * NKG + kg;
                auto step = [&](const u32x4* bq, f32x4* acc, f32x4& ps, bool dg) {
                    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) sc = mfma_bf16(ak[kk], bq[kk], sc);
                    float pv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) pv[v] = (!dg || 4 * gq + v <= li) ? sc[v] : 0.f;
                    const u32x2 p = u32x2{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
                    ps = mfma_k16(ones, p, ps);
#pragma unroll
                    for (int r = 0; r < RT; ++r) acc[r] = mfma_k16(av[r], p, acc[r]);
                };
                if (kgg <= ga) step(ua, acca, pa, kgg == ga);
                if (vb) step(ub, accb, pb, kgg == gb);
            }
        }

        // ---- the mixture, den, dnum, dden and this group's dW[i,i] terms
        u32x4 gra[KS], grb[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const u32x4 x = ld16(rg, tok(na) + (kk * 32 + gq * 8) * 2);
            const u32x4 y = ld16(rg, tok(nb) + (kk * 32 + gq * 8) * 2);
            gra[kk] = (va && na < T) ? x : zero4;
            grb[kk] = (vb && nb < T) ? y : zero4;
        }
        // g . sum_m P v over this lane's channels, before the mixture joins the sums
        auto gdot = [&](const u32x4* gr, const f32x4* acc) {
            float x = 0.f;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                float gl[8];
                unpack8(gr[kk], gl);
#pragma unroll
                for (int s = 0; s < 8; ++s) x += gl[s] * acc[2 * kk + (s >> 2)][s & 3];
            }
            return x;
        };
        const float gia = gdot(gra, acca), gib = gdot(grb, accb);
        // num = w sum_m P v + St_i<^T u, den's u . zt_i< (zt as high and low parts);
        // St_i< with rows e = och(r, li) and k = c (the record's [e][c] rows), one k-step at a time
        f32x4 zaa = f32x4{0.f, 0.f, 0.f, 0.f}, zab = zaa;
        if (va) {
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                acca[r] = acca[r] * wii;
                accb[r] = accb[r] * wii;
            }
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                u32x4 am[RT];
#pragma unroll
                for (int r = 0; r < RT; ++r) am[r] = ld16(rs, (och(r, li) * D + kk * 32 + gq * 8) * 2);
                const f32x4 x = *reinterpret_cast<const f32x4*>(zl + kk * 32 + gq * 8);
                const f32x4 y = *reinterpret_cast<const f32x4*>(zl + kk * 32 + gq * 8 + 4);
                const float z[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
                u32x4 zhi, zlo;
                split_zt(z, zhi, zlo);
                zaa = mfma_bf16(zlo, ua[kk], mfma_bf16(zhi, ua[kk], zaa));
                if (vb) zab = mfma_bf16(zlo, ub[kk], mfma_bf16(zhi, ub[kk], zab));
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    acca[r] = mfma_bf16(am[r], ua[kk], acca[r]);
                    if (vb) accb[r] = mfma_bf16(am[r], ub[kk], accb[r]);
                }
            }
        }
        struct Grad {
            u32x4 g[KS];   // g as B operands, k = channel kk 32 + 8 gq + s (zero past the chunk)
            float inv, dden;
        };
        auto finish1 = [&](const f32x4* acc, const f32x4& ps, const f32x4& za, float gi, const u32x4* gr, int n,
                           Grad& G) {
            float gl[8 * KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) unpack8(gr[kk], gl + 8 * kk);
            float gn = 0.f;   // g . num
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int s = 0; s < 8; ++s) gn += gl[8 * kk + s] * acc[2 * kk + (s >> 2)][s & 3];
            gi += shfl_xor(gi, 16);
            gi += shfl_xor(gi, 32);
            gn += shfl_xor(gn, 16);
            gn += shfl_xor(gn, 32);
            const float den = za[0] + wii * ps[0] + g.eps;
            const float inv = n < T ? 1.f / den : 0.f;
            G.inv = inv;
            G.dden = -gn * inv * inv;
            dgacc += gq == 0 ? gi * inv + ps[0] * G.dden : 0.f;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) G.g[kk] = gr[kk];
            if (n < T && gq == 0)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(inv), __float_as_uint(G.dden)}, rts,
                                                      n * g.H * 8, 0, 0);
        };
        Grad Ga, Gb;
        if (va) finish1(acca, pa, zaa, gia, gra, na, Ga);
        if (vb) finish1(accb, pb, zab, gib, grb, nb, Gb);

        // ---- phase 2: du = St_i< dnum + w sum_m X a over the key tiles up to this one
        f32x4 dua[RT], dub[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) dua[r] = dub[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kt = 0; kt <= qt; ++kt) {
            __syncthreads();
            stage_tile<D, NW, false, false, true, false>(kl, vl, rv, rk, kt, T, rowb);
            if (qt == 0 && kt == 0) stage_transposed_record<D, NT>(stl, rs);
            __syncthreads();
            if (kt == 0 && va) {
                // (St_i< g) / den
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    f32x4 ta = f32x4{0.f, 0.f, 0.f, 0.f}, tb = ta;
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) {
                        const u32x4 a = *reinterpret_cast<const u32x4*>(stl + och(r, li) * KSTR + kk * 32 + gq * 8);
                        ta = mfma_bf16(a, Ga.g[kk], ta);
                        if (vb) tb = mfma_bf16(a, Gb.g[kk], tb);
                    }
                    dua[r] = ta * Ga.inv;
                    dub[r] = tb * Gb.inv;
                }
            }
            const int top = (vb ? gb : ga) - kt * NKG;
            const int nk = !va ? 0 : (top < NKG - 1 ? top + 1 : NKG);
            for (int kg = 0; kg < nk; ++kg) {
                u32x4 avr[KS];
                u32x2 akt[RT];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    avr[kk] = *reinterpret_cast<const u32x4*>(kl + (16 * kg + li) * KSTR + kk * 32 + gq * 8);
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    akt[r] = *reinterpret_cast<const u32x2*>(vl + tr_piece(r, li, gq, kg, VSTR));
                const int kgg = kt * NKG + kg;
                auto step = [&](const Grad& G, f32x4* du, bool dg) {
                    f32x4 xs = f32x4{0.f, 0.f, 0.f, 0.f};   // v . g
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) xs = mfma_bf16(avr[kk], G.g[kk], xs);
                    float xv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        xv[v] = (!dg || 4 * gq + v <= li) ? (xs[v] * G.inv + G.dden) * wii : 0.f;
                    const uint32_t x01 = pack_bf16(xv[0], xv[1]), x23 = pack_bf16(xv[2], xv[3]);
                    const u32x2 xh = u32x2{x01, x23};
                    const u32x2 xl = u32x2{pack_bf16(xv[0] - bf_lo(x01), xv[1] - bf_hi(x01)),
                                           pack_bf16(xv[2] - bf_lo(x23), xv[3] - bf_hi(x23))};
#pragma unroll
                    for (int r = 0; r < RT; ++r) du[r] = mfma_k16(akt[r], xl, mfma_k16(akt[r], xh, du[r]));
                };
                if (kgg <= ga) step(Ga, dua, kgg == ga);
                if (vb) step(Gb, dub, kgg == gb);
            }
        }

        // ---- dq, then this group's dSt_i<, dzt_i< terms
        auto finish2 = [&](const u32x4* bq, const Grad& G, f32x4* du, int n, f32x4 (*dsacc)[RT], f32x4* dzacc) {
            if (n < T) {
                u32x4 qr[KS];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) qr[kk] = ld16(rq, n * rowb + (kk * 32 + gq * 8) * 2);
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    float ql[8];
                    unpack8(qr[kk], ql);
                    u32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float x[2];
#pragma unroll
                        for (int t2 = 0; t2 < 2; ++t2) {
                            const int s = 2 * j + t2, r = 2 * kk + (s >> 2), v = s & 3;
                            x[t2] = (du[r][v] + zl[kk * 32 + 8 * gq + s] * G.dden) * phi_grad(ql[s]);
                        }
                        o[j] = pack_bf16(x[0], x[1]);
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(o, rdq, n * rowb + (kk * 32 + gq * 8) * 2, 0, 0);
                }
            }
            // token rows -> operands with 4 tokens per lane (exact: times 1.0)
            float iv[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) iv[s] = __shfl(G.inv, 4 * gq + s, 64);
            u32x2 tu[RT], tn[RT];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
                    const f32x4 x = mfma_bf16(bq[kk], idb[hf], z);
                    const f32x4 y = mfma_bf16(G.g[kk], idb[hf], z);
                    tu[2 * kk + hf] = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
                    // dnum = g / den of tokens 4 gq + v
                    tn[2 * kk + hf] = u32x2{pack_bf16(y[0] * iv[0], y[1] * iv[1]), pack_bf16(y[2] * iv[2], y[3] * iv[3])};
                }
#pragma unroll
            for (int rc = 0; rc < RT; ++rc)
#pragma unroll
                for (int re = 0; re < RT; ++re) dsacc[rc][re] = mfma_k16(tu[rc], tn[re], dsacc[rc][re]);
            float dd[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) dd[s] = __shfl(G.dden, 4 * gq + s, 64);
            const uint32_t d01 = pack_bf16(dd[0], dd[1]), d23 = pack_bf16(dd[2], dd[3]);
            const u32x2 dhi = u32x2{d01, d23};
            const u32x2 dlo = u32x2{pack_bf16(dd[0] - bf_lo(d01), dd[1] - bf_hi(d01)),
                                    pack_bf16(dd[2] - bf_lo(d23), dd[3] - bf_hi(d23))};
#pragma unroll
            for (int rc = 0; rc < RT; ++rc) dzacc[rc] = mfma_k16(tu[rc], dlo, mfma_k16(tu[rc], dhi, dzacc[rc]));
        };
        f32x4 dsacc[RT][RT], dzacc[RT];
#pragma unroll
        for (int rc = 0; rc < RT; ++rc) {
            dzacc[rc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int re = 0; re < RT; ++re) dsacc[rc][re] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (va) finish2(ua, Ga, dua, na, dsacc, dzacc);
        if (vb) finish2(ub, Gb, dub, nb, dsacc, dzacc);

        // ---- this tile's dSt_i<, dzt_i< terms: the waves' partials added in a
        // fixed order, then into the workgroup's fp32 sums in LDS
        float* red = reinterpret_cast<float*>(smem);
        float* zr = red + (NW / 2) * SLOT;
        __syncthreads();   // every wave is done with kl, vl
        if (li == 0) {
#pragma unroll
            for (int rc = 0; rc < RT; ++rc)
                *reinterpret_cast<f32x4*>(zr + w * D + 16 * rc + 4 * gq) = dzacc[rc];
        }
#pragma unroll
        for (int half = NW / 2; half >= 1; half >>= 1) {
            if (w >= half && w < 2 * half) {
                float* slot = red + (w - half) * SLOT;
#pragma unroll
                for (int rc = 0; rc < RT; ++rc)
#pragma unroll
                    for (int re = 0; re < RT; ++re)
#pragma unroll
                        for (int v = 0; v < 4; ++v) slot[((rc * RT + re) * 4 + v) * 64 + lane] = dsacc[rc][re][v];
            }
            __syncthreads();
            if (w < half) {
                const float* slot = red + w * SLOT;
#pragma unroll
                for (int rc = 0; rc < RT; ++rc)
#pragma unroll
                    for (int re = 0; re < RT; ++re)
#pragma unroll
                        for (int v = 0; v < 4; ++v) dsacc[rc][re][v] += slot[((rc * RT + re) * 4 + v) * 64 + lane];
            }
            __syncthreads();
        }
        if (NW == 1) __syncthreads();   // zr written by other lanes of the wave
        if (w == 0) {
#pragma unroll
            for (int rc = 0; rc < RT; ++rc)
#pragma unroll
                for (int re = 0; re < RT; ++re)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float* a = acl + ((rc * RT + re) * 4 + v) * 64 + lane;
                        *a = (qt == 0 ? 0.f : *a) + dsacc[rc][re][v];
                    }
            if (lane < D) {
                float z = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) z += zr[ww * D + lane];
                zacl[lane] = (qt == 0 ? 0.f : zacl[lane]) + z;
            }
        }
    }

    // ---- the record [dSt_i< as [e][c] | dzt_i<] and the pair's dW[i,i] terms
    const float dsum = wave_sum(dgacc);
    if (lane == 0) dr[w] = dsum;
    __syncthreads();
    if (w == 0) {
        uint16_t* rec = dSt + (size_t)blk * REC;
#pragma unroll
        for (int rc = 0; rc < RT; ++rc)
#pragma unroll
            for (int re = 0; re < RT; ++re) {
                const float* a = acl + (rc * RT + re) * 4 * 64 + lane;
                *reinterpret_cast<u32x2*>(rec + (16 * re + li) * D + 16 * rc + 4 * gq) =
                    u32x2{pack_bf16(a[0], a[64]), pack_bf16(a[128], a[192])};
            }
        if (lane < D) rec[D * D + lane] = (uint16_t)(pack_bf16(zacl[lane], 0.f) & 0xffffu);
        if (lane == 0) {
            float sd = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) sd += dr[ww];
            diag[blk] = sd;
        }
    }
}

// dW of the causal form: entries below the diagonal are sums over the
// partial products (split order), the diagonal is the pairs' in-chunk terms
// (pair order), entries above it are zero.
__device__ __forceinline__ float dw_causal_entry(const float* __restrict__ part, const float* __restrict__ dg, int x,
                                                 int M, int nsplit, int P) {
    const int i = x / M, j = x - i * M;
    const int MM = M * M;
    float s = 0.f;
    if (j < i) {
        int k = 0;
        for (; k + 8 <= nsplit; k += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(k + u) * MM + x];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; k < nsplit; ++k) s += part[(size_t)k * MM + x];
    } else if (j == i) {
        for (int p = 0; p < P; ++p) s += dg[(size_t)p * M + i];
    }
    return s;
}

__global__ __launch_bounds__(256) void dw_reduce_causal(const float* __restrict__ part, const float* __restrict__ dg,
                                                        float* __restrict__ dW, int M, int nsplit, int P) {
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x < M * M) dW[x] = dw_causal_entry(part, dg, x, M, nsplit, P);
}

// =====================================================================
// Key/value side.  Workgroup = (b, chunk i, head h) with NW waves; per key
// tile, wave w takes key groups w and 2 NW - 1 - w (phi(k) and v of its keys
// are the B operands, k = channel), over the query tiles from the key tile on:
//  pass 1: phi(Q) rows, g^T and 1 / den of the query tile in LDS; P^T
//    (queries as rows) masked to n >= m, times W[i,i] / den_n, into
//    dv += g^T P; then dv += Gx_i^T a (Gx_i from the transposed mixing's
//    record);
//  pass 2: g rows, phi(Q)^T, 1 / den and dden of the query tile in LDS;
//    X^T = (g . v) / den + dden masked, times W[i,i], as bf16 high and low
//    parts into du += u^T X; then du += Gx_i v (the record transposed in
//    LDS) + gzx_i and dk = du phi'(k).
// Queries past the chunk's end have g = 1 / den = dden = 0 in LDS, so they
// add nothing.
// =====================================================================
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 1 ? 1 : 2))) void causal_bwd_kv_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ tsc, const uint16_t* __restrict__ dS,
    const float* __restrict__ dZ, const float* __restrict__ W, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    const Geo g, const float* __restrict__ part, const float* __restrict__ dg, float* __restrict__ dW, int nsplit,
    int nkv) {
    // Workgroups from nkv on form dW from its split partials and the in-chunk
    // diagonal terms, beside the key/value gradients (which do not need it).
    if ((int)blockIdx.x >= nkv) {
        const int x = ((int)blockIdx.x - nkv) * (64 * NW) + (int)threadIdx.x;
        if (x < g.M * g.M) dW[x] = dw_causal_entry(part, dg, x, g.M, nsplit, g.BH);
        return;
    }
    constexpr int RT = D / 16, KS = D / 32;
    constexpr int NT = 64 * NW, KT = 32 * NW, NKG = KT / 16;
    constexpr int KSTR = D + 8, VSTR = KT + 4;
    static_assert(D <= 64, "tr_piece assumes at most four row tiles");
    __shared__ __attribute__((aligned(16))) uint16_t kl[KT * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vl[D * VSTR];
    __shared__ __attribute__((aligned(16))) uint16_t gxt[D * KSTR];   // Gx_i as [c][e]
    __shared__ __attribute__((aligned(16))) float ivl[KT];   // 1 / den of the query tile
    __shared__ __attribute__((aligned(16))) float ddl[KT];   // dden of the query tile

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, gq = lane >> 4;
    const WgCoord wgc = wg_coord(g, blockIdx.x);
    const int b = __builtin_amdgcn_readfirstlane(wgc.b);
    const int h = __builtin_amdgcn_readfirstlane(wgc.hg);
    const int i = __builtin_amdgcn_readfirstlane(wgc.j);
    const int blk = (b * g.H + h) * g.M + i;
    const float wii = W[(size_t)i * g.M + i];

    const int row = g.H * D, T = g.T, rowb = row * 2;
    const int origin = block_origin(g, i);
    const int base = (b * g.N + origin) * row + h * D;
    const int crange = (T * row - h * D) * 2;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + base), 0, crange, kRF);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), 0, crange, kRF);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), 0, crange, kRF);
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc((void*)(dO + base), 0, crange, kRF);
    const __amdgpu_buffer_rsrc_t rdk = __builtin_amdgcn_make_buffer_rsrc((void*)(dK + base), 0, crange, kRF);
    const __amdgpu_buffer_rsrc_t rdv = __builtin_amdgcn_make_buffer_rsrc((void*)(dV + base), 0, crange, kRF);
    const int dbase = (b * g.N + origin) * g.H + h;
    const __amdgpu_buffer_rsrc_t rts =
        __builtin_amdgcn_make_buffer_rsrc((void*)(tsc + 2 * (size_t)dbase), 0, (T * g.H - h) * 8, kRF);
    const __amdgpu_buffer_rsrc_t rds =
        __builtin_amdgcn_make_buffer_rsrc((void*)(dS + (size_t)blk * (D * D)), 0, D * D * 2, kRF);
    const __amdgpu_buffer_rsrc_t rdz = __builtin_amdgcn_make_buffer_rsrc((void*)(dZ + (size_t)blk * D), 0, D * 4, kRF);
    auto tok = [&](int p) { return (p < T ? p : T - 1) * rowb; };
    // 1 / den and dden of query tile qt (thread x < KT takes token x; zeros
    // past the chunk), loaded with the tile and written to LDS with it
    auto load_scalars = [&](int qt, u32x2& t) {
        const int p = qt * KT + tid;
        if (tid < KT)
            t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rts, (p < T ? p : 0) * g.H * 8, 0, 0));
    };
    auto store_scalars = [&](int qt, const u32x2& t) {
        const int p = qt * KT + tid;
        if (tid < KT) {
            ivl[tid] = p < T ? __uint_as_float(t[0]) : 0.f;
            ddl[tid] = p < T ? __uint_as_float(t[1]) : 0.f;
        }
    };
    // The stages run in the order (key tile kt: pass 1 over query tiles kt..,
    // then pass 2 over the same); each stage's loads are issued while the
    // stage before it is multiplied.  Pass 1 stages phi(Q) rows and g^T,
    // pass 2 g rows and phi(Q)^T: the same tokens, other layouts.
    TileRegs<D, NW> tr;
    u32x2 tsr = u32x2{0u, 0u};
    load_tile<D, NW>(tr, rq, rg, 0, T, rowb);
    load_scalars(0, tsr);

    const int nit = (T + 15) >> 4;
    const int nqt = (T + KT - 1) / KT;
    for (int kt = 0; kt < nqt; ++kt) {
        const int ga = kt * NKG + w, gb = kt * NKG + NKG - 1 - w;
        const bool va = ga < nit, vb = gb < nit;   // gb > ga: vb implies va
        const int ma = 16 * ga + li, mb = 16 * gb + li;
        u32x4 bka[KS], bkb[KS];   // phi(k) of the lane's key, k = channel kk 32 + 8 gq + s
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            bka[kk] = phi_words(ld16(rk, tok(ma) + (kk * 32 + gq * 8) * 2));
            bkb[kk] = phi_words(ld16(rk, tok(mb) + (kk * 32 + gq * 8) * 2));
        }
        f32x4 acca[RT], accb[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) acca[r] = accb[r] = f32x4{0.f, 0.f, 0.f, 0.f};

        // ---- pass 1: dv
        for (int qt = kt; qt < nqt; ++qt) {
            __syncthreads();
            store_tile<D, NW, true, false, false, true>(kl, vl, tr, qt, T);
            store_scalars(qt, tsr);
            if (kt == 0 && qt == 0) stage_transposed_record<D, NT>(gxt, rds);
            __syncthreads();
            // next stage: this pass's next query tile, else pass 2's first
            if (qt + 1 < nqt) {
                load_tile<D, NW>(tr, rq, rg, qt + 1, T, rowb);
                load_scalars(qt + 1, tsr);
            } else {
                load_tile<D, NW>(tr, rg, rq, kt, T, rowb);
                load_scalars(kt, tsr);
            }
            // local query groups [lq0, nlq) that either key group needs
            const int lq0 = qt == kt ? w : 0;
            const int nlq = min(NKG, nit - qt * NKG);
            for (int lq = va ? lq0 : nlq; lq < nlq; ++lq) {
                u32x4 aq[KS];
                u32x2 adn[RT];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    aq[kk] = *reinterpret_cast<const u32x4*>(kl + (16 * lq + li) * KSTR + kk * 32 + gq * 8);
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    adn[r] = *reinterpret_cast<const u32x2*>(vl + tr_piece(r, li, gq, lq, VSTR));
                const f32x4 iv = *reinterpret_cast<const f32x4*>(ivl + 16 * lq + 4 * gq);
                const int qg = qt * NKG + lq;
                auto step = [&](const u32x4* bk, f32x4* acc, bool dg) {
                    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) sc = mfma_bf16(aq[kk], bk[kk], sc);
                    float pv[4];   // W[i,i] P / den_n: the weights of dv += g^T p
#pragma unroll
                    for (int v = 0; v < 4; ++v) pv[v] = (!dg || 4 * gq + v >= li) ? sc[v] * (wii * iv[v]) : 0.f;
                    const u32x2 p = u32x2{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
#pragma unroll
                    for (int r = 0; r < RT; ++r) acc[r] = mfma_k16(adn[r], p, acc[r]);
                };
                if (qg >= ga) step(bka, acca, qg == ga);
                if (vb && qg >= gb) step(bkb, accb, qg == gb);
            }
        }
        // Gx_i^T a, then dv
        auto finish_v = [&](const u32x4* bk, f32x4* acc, int m) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    acc[r] = mfma_bf16(ld16(rds, (och(r, li) * D + kk * 32 + gq * 8) * 2), bk[kk], acc[r]);
            if (m < T) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const f32x4 x = acc[2 * kk], y = acc[2 * kk + 1];
                    const u32x4 o = u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(y[0], y[1]),
                                          pack_bf16(y[2], y[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(o, rdv, m * rowb + (kk * 32 + gq * 8) * 2, 0, 0);
                }
            }
        };
        if (va) finish_v(bka, acca, ma);
        if (vb) finish_v(bkb, accb, mb);

        // ---- pass 2: dk
        u32x4 bva[KS], bvb[KS];   // v of the lane's key
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            bva[kk] = ld16(rv, tok(ma) + (kk * 32 + gq * 8) * 2);
            bvb[kk] = ld16(rv, tok(mb) + (kk * 32 + gq * 8) * 2);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) acca[r] = accb[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int qt = kt; qt < nqt; ++qt) {
            __syncthreads();
            store_tile<D, NW, false, true, true, false>(kl, vl, tr, qt, T);
            store_scalars(qt, tsr);
            __syncthreads();
            // next stage: this pass's next query tile, else pass 1 of the next key tile
            if (qt + 1 < nqt) {
                load_tile<D, NW>(tr, rg, rq, qt + 1, T, rowb);
                load_scalars(qt + 1, tsr);
            } else if (kt + 1 < nqt) {
                load_tile<D, NW>(tr, rq, rg, kt + 1, T, rowb);
                load_scalars(kt + 1, tsr);
            }
            const int lq0 = qt == kt ? w : 0;
            const int nlq = min(NKG, nit - qt * NKG);
            for (int lq = va ? lq0 : nlq; lq < nlq; ++lq) {
                u32x4 adn[KS];
                u32x2 au[RT];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    adn[kk] = *reinterpret_cast<const u32x4*>(kl + (16 * lq + li) * KSTR + kk * 32 + gq * 8);
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    au[r] = *reinterpret_cast<const u32x2*>(vl + tr_piece(r, li, gq, lq, VSTR));
                const f32x4 dd = *reinterpret_cast<const f32x4*>(ddl + 16 * lq + 4 * gq);
                const f32x4 iv = *reinterpret_cast<const f32x4*>(ivl + 16 * lq + 4 * gq);
                const int qg = qt * NKG + lq;
                auto step = [&](const u32x4* bv, f32x4* acc, bool dg) {
                    f32x4 xs = f32x4{0.f, 0.f, 0.f, 0.f};   // g . v
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) xs = mfma_bf16(adn[kk], bv[kk], xs);
                    float xv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        xv[v] = (!dg || 4 * gq + v >= li) ? (xs[v] * iv[v] + dd[v]) * wii : 0.f;
                    const uint32_t x01 = pack_bf16(xv[0], xv[1]), x23 = pack_bf16(xv[2], xv[3]);
                    const u32x2 xh = u32x2{x01, x23};
                    const u32x2 xl = u32x2{pack_bf16(xv[0] - bf_lo(x01), xv[1] - bf_hi(x01)),
                                           pack_bf16(xv[2] - bf_lo(x23), xv[3] - bf_hi(x23))};
#pragma unroll
                    for (int r = 0; r < RT; ++r) acc[r] = mfma_k16(au[r], xl, mfma_k16(au[r], xh, acc[r]));
                };
                if (qg >= ga) step(bva, acca, qg == ga);
                if (vb && qg >= gb) step(bvb, accb, qg == gb);
            }
        }
        // Gx_i v + gzx_i, then dk = du phi'(k)
        auto finish_k = [&](const u32x4* bv, f32x4* acc, int m) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    acc[r] = mfma_bf16(*reinterpret_cast<const u32x4*>(gxt + och(r, li) * KSTR + kk * 32 + gq * 8),
                                       bv[kk], acc[r]);
            if (m < T) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const u32x4 kr = ld16(rk, m * rowb + (kk * 32 + gq * 8) * 2);
                    const f32x4 z0 = __builtin_bit_cast(f32x4, ld16(rdz, (kk * 32 + 8 * gq) * 4));
                    const f32x4 z1 = __builtin_bit_cast(f32x4, ld16(rdz, (kk * 32 + 8 * gq + 4) * 4));
                    float kl8[8];
                    unpack8(kr, kl8);
                    const f32x4 x = acc[2 * kk], y = acc[2 * kk + 1];
                    const float d8[8] = {x[0] + z0[0], x[1] + z0[1], x[2] + z0[2], x[3] + z0[3],
                                         y[0] + z1[0], y[1] + z1[1], y[2] + z1[2], y[3] + z1[3]};
                    u32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        o[j] = pack_bf16(d8[2 * j] * phi_grad(kl8[2 * j]), d8[2 * j + 1] * phi_grad(kl8[2 * j + 1]));
                    __builtin_amdgcn_raw_buffer_store_b128(o, rdk, m * rowb + (kk * 32 + gq * 8) * 2, 0, 0);
                }
            }
        };
        if (va) finish_k(bva, acca, ma);
        if (vb) finish_k(bvb, accb, mb);
    }
}

template <int D, int NW>
void launch_pair(const CausalBwdLaunch& C, const Geo& g) {
    const unsigned grid = (unsigned)(g.B * g.M * g.H);
    const Launch& L = C.B.F;
    causal_bwd_query_bf16<D, NW><<<grid, 64 * NW, 0, L.stream>>>(
        static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v),
        static_cast<const uint16_t*>(C.B.dout), static_cast<const uint16_t*>(L.st), L.zt, L.W,
        static_cast<uint16_t*>(C.B.dq), C.tsc, C.B.dst, C.diag, g);
}

template <int D, int NW>
void launch_kv(const CausalBwdLaunch& C, const Geo& g, bool with_reduce) {
    const int nkv = g.B * g.M * g.H, MM = g.M * g.M;
    const int nred = with_reduce ? (MM + 64 * NW - 1) / (64 * NW) : 0;
    const Launch& L = C.B.F;
    causal_bwd_kv_bf16<D, NW><<<(unsigned)(nkv + nred), 64 * NW, 0, L.stream>>>(
        static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v),
        static_cast<const uint16_t*>(C.B.dout), C.tsc, C.B.ds, C.B.dz, L.W, static_cast<uint16_t*>(C.B.dk),
        static_cast<uint16_t*>(C.B.dv), g, C.B.part, C.diag, C.B.dw, C.B.nsplit, nkv);
}

// Waves per workgroup: enough for two 16-token groups each, at most 4.  Two
// workgroups of 4 waves per compute unit overlap each other's staging and
// barriers; one of 8 waves (the register file allows no second) does not
// (dit-s2-256x256-causal-rows: query side 174 -> 167 us, key/value side
// 149 -> 137 us; workgroups of 2 waves: 211 and 199 us).
template <int D, bool KV>
void launch_nw(const CausalBwdLaunch& C, const Geo& g, bool with_reduce = false) {
    const int nit = (g.T + 15) / 16;
    auto go = [&](auto nw) {
        constexpr int NW = decltype(nw)::value;
        if constexpr (KV) launch_kv<D, NW>(C, g, with_reduce);
        else launch_pair<D, NW>(C, g);
    };
    if (nit > 4) go(std::integral_constant<int, 4>{});
    else if (nit > 2) go(std::integral_constant<int, 2>{});
    else go(std::integral_constant<int, 1>{});
}

inline void rec_event(const CausalBwdLaunch& C, int k) {
    if (C.B.events) (void)hipEventRecord(C.B.events[k], C.B.F.stream);
}

template <int D>
hipError_t run_cbwd_d(const CausalBwdLaunch& C) {
    const BwdLaunch& B = C.B;
    const Launch& L = B.F;
    rec_event(C, 0);
    // Summaries, the causal mixtures (W as bf16 high and low parts) and W^T
    // restricted to later chunks for the transposed mixing.
    hipError_t err = run_bf16(L);
    if (err != hipSuccess) return err;
    rec_event(C, 1);
    Geo g = L.g;
    g.HG = g.H;
    g.G = 1;
    g.div_HG = make_fastdiv((uint32_t)g.HG);
    g.TP = g.AP = 1;
    g.div_TP = g.div_AP = make_fastdiv(1u);
    g.RD = 1;
    launch_nw<D, false>(C, g);
    rec_event(C, 2);
    err = launch_mix_dw_bf16(B, g, static_cast<const uint16_t*>(L.sz));
    if (err != hipSuccess) return err;
    // dW's partials summed beside the key/value side while the chains are
    // short (as in the non-causal backward), else in a launch of their own
    const bool reduce_in_kv = B.nsplit <= 64;
    if (!reduce_in_kv)
        dw_reduce_causal<<<(g.M * g.M + 255) / 256, 256, 0, L.stream>>>(B.part, C.diag, B.dw, g.M, B.nsplit, g.BH);
    rec_event(C, 3);
    launch_nw<D, true>(C, g, reduce_in_kv);
    rec_event(C, 4);
    return hipGetLastError();
}

}  // namespace

hipError_t run_causal_bwd_bf16(const CausalBwdLaunch& C) {
    switch (C.B.F.g.D) {
        case 32: return run_cbwd_d<32>(C);
        case 64: return run_cbwd_d<64>(C);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mhla
