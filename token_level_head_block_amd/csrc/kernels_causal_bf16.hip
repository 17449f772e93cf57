// kernels_causal_bf16.hip -- the causal chunkwise form of MHLA (paperlayer.ai
// summary, appendix B "Causal MHLA": block-specific mixed summaries reused per
// block, causality preserved), bf16 inputs, d = 32, 64 or 128, on gfx950.
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

// Workgroup = (b, chunk i, head h) with NW waves; a tile is KT = 32 NW tokens.
// For each query tile of the chunk and each key tile up to it, the workgroup
// stages phi(K) ([key][channel]) and V^T ([channel][key]) of the key tile in
// LDS once; then every wave takes two 16-query groups of the query tile,
// local groups w and 2 NW - 1 - w, so that all waves do the same amount of
// masked work, and feeds both from each key group it reads from LDS.
//   scores C[m][n] = phi(k_m) . phi(q_n) on v_mfma_f32_16x16x32_bf16 (A =
//   phi(K), key as row; B = phi(Q)), masked to m <= n and scaled by W[i,i];
//   lane (n, gq) then holds keys 4 gq .. +3 of query n, exactly the B operand
//   of v_mfma_f32_16x16x16_bf16, so num += V^T P needs no transpose of P.
// The chunk's mixture St_i< and zt_i< go to LDS with the first key tile, so
// that a workgroup issues all of its first loads (Q, K, V, St, zt) in one
// burst and waits for memory once.
// Output row e of every MFMA is channel 16 r + e (the natural order), for
// the mixture's A operands as for V^T; lane (n, gq) ends with channels
// 16 r + 4 gq .. +3 of query n and stores them directly.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4))) void query_apply_causal_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ St, const float* __restrict__ Zt, const float* __restrict__ W,
    uint16_t* __restrict__ O, const Geo g, const int wld) {
    constexpr int RT = D / 16, KS = D / 32;
    constexpr int NT = 64 * NW;        // threads
    constexpr int KT = 32 * NW;        // tokens per query tile and per key tile
    constexpr int NKG = KT / 16;       // 16-key groups per key tile
    constexpr int KSTR = D + 8;        // row stride of phi(K) and St in LDS (bf16)
    constexpr int VSTR = KT + 4;       // V^T row stride in LDS (bf16): 264 bytes at KT = 128, rows 8 bytes apart in the banks
    constexpr int KU = KT * D / 8 / NT;                 // phi(K) units (key, 8 channels) per thread
    constexpr int VU = (KT / 4 * (D / 8) + NT - 1) / NT;   // V^T units (4 keys, 8 channels) per thread
    constexpr int SU = (D * D / 8 + NT - 1) / NT;          // St units (row, 8 channels) per thread
    __shared__ __attribute__((aligned(16))) uint16_t kl[KT * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vl[D * VSTR];
    __shared__ __attribute__((aligned(16))) uint16_t sl[D * KSTR];
    __shared__ __attribute__((aligned(16))) float zl[D];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, gq = lane >> 4;
    const WgCoord wgc = wg_coord(g, blockIdx.x);
    const int b = __builtin_amdgcn_readfirstlane(wgc.b);
    const int h = __builtin_amdgcn_readfirstlane(wgc.hg);
    const int i = __builtin_amdgcn_readfirstlane(wgc.j);
    const int blk = (b * g.H + h) * g.M + i;
    const int iw = i / g.WD;                     // W's index of this block (sub-chunks: WD per chunk)
    const float wii = W[(size_t)iw * wld + iw];  // W[iw][iw], leading dimension wld

    // Chunks are contiguous in raster order: position p of chunk i is raster
    // index origin + p.  Offsets fit in 32 bits: tensors hold fewer than 2^31
    // elements.
    // Loads and stores go through buffer descriptors with 32-bit byte offsets:
    // token rows of this chunk from channel h*D on (the range ends where the
    // chunk's last row does), and this block's St and zt records.
    const int row = g.H * D;
    const int T = g.T;
    const int base = (b * g.N + block_origin(g, i)) * row + h * D;
    const int crange = (T * row - h * D) * 2;
    constexpr int RF = 0x00020000;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + base), 0, crange, RF);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), 0, crange, RF);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), 0, crange, RF);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)(O + base), 0, crange, RF);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(St + (size_t)blk * (D * D)), 0, D * D * 2, RF);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc((void*)(Zt + (size_t)blk * D), 0, D * 4, RF);
    auto ld16 = [](__amdgpu_buffer_rsrc_t r, int off) {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    };
    auto tok = [&](int p) { return (p < T ? p : T - 1) * (row * 2); };   // byte offset of position p
    const u32x2 ones = u32x2{0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs: row sums of P on the MFMA

    const int nit = (T + 15) >> 4;               // 16-query groups of the chunk
    const int nqt = (T + KT - 1) / KT;           // query (and key) tiles
    for (int qt = 0; qt < nqt; ++qt) {
        const int ga = qt * NKG + w, gb = qt * NKG + NKG - 1 - w;
        const bool va = ga < nit, vb2 = gb < nit;
        const int na = 16 * ga + li, nb = 16 * gb + li;
        u32x4 bqa[KS], bqb[KS];    // raw Q, then phi(Q) as B operands
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            bqa[kk] = ld16(rq, tok(na) + (kk * 32 + gq * 8) * 2);
            bqb[kk] = ld16(rq, tok(nb) + (kk * 32 + gq * 8) * 2);
        }
        f32x4 acca[RT], accb[RT];
        float da = 0.f, db = 0.f;   // phi(q) . zt of the earlier chunks
        // sums of the rounded within-chunk weights, every row equal
        f32x4 pa = f32x4{0.f, 0.f, 0.f, 0.f}, pb_sum = pa;
#pragma unroll
        for (int r = 0; r < RT; ++r) acca[r] = accb[r] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kt = 0; kt <= qt; ++kt) {
            const bool first = qt == 0 && kt == 0;
            if (!first) __syncthreads();   // the previous tile's readers are done
            // ---- issue every load of this stage, then convert and write LDS
            u32x4 kx[KU], vx[VU][4], sx[SU];
            f32x4 zx = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KU; ++s) {
                const int u = tid + NT * s;
                kx[s] = ld16(rk, tok(kt * KT + u / (D / 8)) + (u % (D / 8)) * 16);
            }
#pragma unroll
            for (int s = 0; s < VU; ++s) {
                const int u = tid + NT * s;
                const int kq = u / (D / 8), c8 = u % (D / 8);
                if (u < KT / 4 * (D / 8)) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        vx[s][j] = ld16(rv, tok(kt * KT + 4 * kq + j) + c8 * 16);
                }
            }
            if (first) {
#pragma unroll
                for (int s = 0; s < SU; ++s) {
                    const int u = tid + NT * s;
                    if (u < D * D / 8) sx[s] = ld16(rs, u * 16);
                }
                if (tid < D / 4) zx = __builtin_bit_cast(f32x4, ld16(rz, 16 * tid));
            }
#pragma unroll
            for (int s = 0; s < KU; ++s) {
                const int u = tid + NT * s;
                u32x4 y;
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = pack_bf16(phi_fast(bf_lo(kx[s][j])), phi_fast(bf_hi(kx[s][j])));
                *reinterpret_cast<u32x4*>(kl + (u / (D / 8)) * KSTR + (u % (D / 8)) * 8) = y;
            }
#pragma unroll
            for (int s = 0; s < VU; ++s) {
                const int u = tid + NT * s;
                const int kq = u / (D / 8), c8 = u % (D / 8);
                if (u < KT / 4 * (D / 8)) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint16_t* d0 = vl + (c8 * 8 + 2 * j) * VSTR + 4 * kq;
                        *reinterpret_cast<u32x2*>(d0) =
                            u32x2{pack_lo(vx[s][0][j], vx[s][1][j]), pack_lo(vx[s][2][j], vx[s][3][j])};
                        *reinterpret_cast<u32x2*>(d0 + VSTR) =
                            u32x2{pack_hi(vx[s][0][j], vx[s][1][j]), pack_hi(vx[s][2][j], vx[s][3][j])};
                    }
                }
            }
            if (first) {
#pragma unroll
                for (int s = 0; s < SU; ++s) {
                    const int u = tid + NT * s;
                    if (u < D * D / 8) *reinterpret_cast<u32x4*>(sl + (u / (D / 8)) * KSTR + (u % (D / 8)) * 8) = sx[s];
                }
                if (tid < D / 4) *reinterpret_cast<f32x4*>(zl + 4 * tid) = zx;
            }
            __syncthreads();

            if (kt == 0) {
                // ---- phi(Q) of both groups, then the earlier chunks' mixture from LDS
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        bqa[kk][j] = pack_bf16(phi_fast(bf_lo(bqa[kk][j])), phi_fast(bf_hi(bqa[kk][j])));
                        bqb[kk][j] = pack_bf16(phi_fast(bf_lo(bqb[kk][j])), phi_fast(bf_hi(bqb[kk][j])));
                    }
                f32x4 za = f32x4{0.f, 0.f, 0.f, 0.f}, zb2 = za;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(zl + kk * 32 + gq * 8);
                    const f32x4 y = *reinterpret_cast<const f32x4*>(zl + kk * 32 + gq * 8 + 4);
                    const float z[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
                    u32x4 zhi, zlo;
                    split_zt(z, zhi, zlo);
                    za = mfma_bf16(zlo, bqa[kk], mfma_bf16(zhi, bqa[kk], za));
                    zb2 = mfma_bf16(zlo, bqb[kk], mfma_bf16(zhi, bqb[kk], zb2));
#pragma unroll
                    for (int r = 0; r < RT; ++r) {
                        const u32x4 a = *reinterpret_cast<const u32x4*>(sl + (16 * r + li) * KSTR + kk * 32 + gq * 8);
                        acca[r] = mfma_bf16(a, bqa[kk], acca[r]);
                        accb[r] = mfma_bf16(a, bqb[kk], accb[r]);
                    }
                }
                da = za[0];
                db = zb2[0];
            }

            // ---- key groups of this tile that either query group needs
            const int top = (vb2 ? gb : ga) - kt * NKG;   // last local key group needed
            const int nk = !va ? 0 : (top < NKG - 1 ? top + 1 : NKG);
            for (int kg = 0; kg < nk; ++kg) {
                u32x4 ak[KS];
                u32x2 av[RT];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    ak[kk] = *reinterpret_cast<const u32x4*>(kl + (16 * kg + li) * KSTR + kk * 32 + gq * 8);
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    av[r] = *reinterpret_cast<const u32x2*>(vl + (16 * r + li) * VSTR + 16 * kg + 4 * gq);
                const int kgg = kt * NKG + kg;
                // Key groups below a query group's own are complete and unmasked
                // (they lie before the query, inside the chunk); only the
                // diagonal group keeps keys 4 gq + v <= query li.
                auto step = [&](const u32x4* bq, f32x4* acc, f32x4& psum, bool diag) {
                    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) sc = mfma_bf16(ak[kk], bq[kk], sc);
                    float pv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) pv[v] = wii * sc[v];
                    if (diag) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) pv[v] = 4 * gq + v <= li ? pv[v] : 0.f;
                    }
                    const u32x2 p = u32x2{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
                    // the denominator adds the same rounded weights the numerator uses
                    psum = mfma_k16(ones, p, psum);
#pragma unroll
                    for (int r = 0; r < RT; ++r) acc[r] = mfma_k16(av[r], p, acc[r]);
                };
                if (kgg <= ga) step(bqa, acca, pa, kgg == ga);
                if (vb2) step(bqb, accb, pb_sum, kgg == gb);
            }
        }
        // ---- normalise and store: lane (n, gq) holds channels 16 r + 4 gq .. +3
        auto finish = [&](const f32x4* acc, float dd, const f32x4& psum, int n) {
            const float inv = 1.f / (dd + psum[0] + g.eps);
            if (n < T) {
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2{pack_bf16(acc[r][0] * inv, acc[r][1] * inv), pack_bf16(acc[r][2] * inv, acc[r][3] * inv)},
                        ro, n * (row * 2) + (16 * r + 4 * gq) * 2, 0, 0);
            }
        };
        if (va) finish(acca, da, pa, na);
        if (vb2) finish(accb, db, pb_sum, nb);
    }
}

template <int D, int NW>
void launch(const Launch& L, int wld) {
    Geo g = L.g;
    g.HG = g.H;
    g.G = 1;
    g.div_HG = make_fastdiv((uint32_t)g.HG);
    query_apply_causal_bf16<D, NW><<<g.B * g.M * g.H, 64 * NW, 0, L.stream>>>(
        static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v),
        static_cast<const uint16_t*>(L.st), L.zt, L.W, static_cast<uint16_t*>(L.out), g, wld);
}

template <int D>
void launch_d(const Launch& L, int wld) {
    // Waves per workgroup: enough for two query groups each, at most 8 (at
    // most 4 at d = 128, whose 256-token tile would not fit LDS).
    const int nit = (L.g.T + 15) / 16;
    if constexpr (D < 128) {
        if (nit > 8) {
            launch<D, 8>(L, wld);
            return;
        }
    }
    if (nit > 4) launch<D, 4>(L, wld);
    else if (nit > 2) launch<D, 2>(L, wld);
    else launch<D, 1>(L, wld);
}

}  // namespace

hipError_t launch_causal_apply_bf16(const Launch& L, int wld) {
    if (wld <= 0) wld = L.g.WM;
    switch (L.g.D) {
        case 32: launch_d<32>(L, wld); break;
        case 64: launch_d<64>(L, wld); break;
        case 128: launch_d<128>(L, wld); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mhla
