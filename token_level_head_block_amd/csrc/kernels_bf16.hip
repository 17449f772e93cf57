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

#include <type_traits>
#include "bf16_shared.h"

#include <mhla.h>

namespace mhla {
namespace {

// =====================================================================
// block_kv_summary
// Workgroup = one block j of one batch b for G consecutive heads; one wave per
// head (d = 128: four waves per head, one quadrant of S each), so together
// the waves read contiguous runs of every token's channels.  A wave owns a
// 64x64 (d = 32: 32x32) tile of S over all of the block's tokens.
// Lane (li, gq): K channels CPL*li .. +CPL-1 for rows, V channels likewise
// for columns, tokens 32*ks + 8*gq + s (s = 0..7) as k-slots.
// z_j = phi(K_j)^T 1 runs on the matrix cores too (one extra MFMA per row
// tile against an all-ones operand), which keeps the vector ALUs for phi.
// ROW8: block rows hold a multiple of 8 tokens, so the 8 tokens of a lane
// group are consecutive in raster order (one address computation).
// FULL: ROW8 and T a multiple of 32, so no token slot is ever padding.
// PAIR (D = 64 only): the problem has head_dim 32 and an even head count; a
// wave reads the 64 channels of heads 2p and 2p + 1 exactly as one head of
// 64 (whole 128-byte rows per lane group) and forms the 64 x 64 product,
// whose two diagonal 32 x 32 blocks are the two heads' S (the off-diagonal
// blocks are discarded); the records written are those of head_dim 32.
// =====================================================================

// NBW > 1 (whole blocks of at most 64 tokens, TP = 1): a wave walks NBW
// consecutive blocks as one pipeline, so the loads of the next block are in
// flight while one block's last step is multiplied and its record stored.
template <int D, int PF, bool ROW8, bool FULL, bool NTL, bool PAIR = false, int NBW = 1>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(PF == 1 && D <= 64 && FULL && NBW == 1 ? 3 : 2)))
void block_kv_summary_bf16(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                           uint16_t* __restrict__ SZ, const Geo g, const float* __restrict__ W,
                           uint16_t* __restrict__ Wb, const WConv wc) {
    static_assert(!FULL || ROW8, "FULL implies ROW8");
    static_assert(!PAIR || D == 64, "paired heads run the 64-channel layout");
    static_assert(NBW == 1 || (FULL && D <= 64), "several blocks per wave: whole blocks, d <= 64");
    constexpr int CPL = (D == 32) ? 2 : 4;   // channels per lane
    constexpr int CW = CPL / 2;              // 32-bit words per lane per token
    constexpr int NQ = (D == 128) ? 4 : 1;
    if ((int)blockIdx.x >= wc.first_wg) {
        convert_w(W, Wb, wc);
        return;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int quad = wave % NQ;
    const int li = lane & 15, gq = lane >> 4;
    WgCoordP wgc;
    if constexpr (NBW > 1) {
        // blocks NBW jg .. NBW jg + NBW - 1 (M is a multiple of NBW; TP = 1)
        const uint32_t bj = fdiv(blockIdx.x, g.div_HG);
        const int mg = g.M / NBW;
        wgc.hg = (int)(blockIdx.x - bj * g.div_HG.d);
        wgc.b = (int)bj / mg;
        wgc.j = ((int)bj - wgc.b * mg) * NBW;
        wgc.t = 0;
    } else {
        wgc = wg_coord_parts(g, blockIdx.x, g.div_TP);
    }
    const int b = wgc.b, j = wgc.j, h = wgc.hg * g.G + wave / NQ;
    if (h >= g.H) return;
    const int rowbase = (D == 128) ? (quad >> 1) * 64 : 0;
    const int colbase = (D == 128) ? (quad & 1) * 64 : 0;
    const bool do_z = (quad & 1) == 0;        // one wave per row range forms z
    const int row = g.H * D;
    int origin = block_origin(g, j);
    const uint16_t* kb = K + (b * g.N * row + h * D + rowbase + CPL * li);
    const uint16_t* vb = V + (b * g.N * row + h * D + colbase + CPL * li);
    const u32x4 ones = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs

    f32x4 acc[CPL][CPL], accz[CPL];
#pragma unroll
    for (int r = 0; r < CPL; ++r) {
        accz[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    struct Raw {
        uint32_t k[8][CW], v[8][CW];
        uint32_t valid;
        int it;                               // NBW > 1: the pipeline iteration
    };
    const int nks = (g.T + 31) >> 5;          // 32-token steps per block
    auto load = [&](int ks, Raw& R) {
        if constexpr (NBW > 1) {
            // iteration ks: step ks % nks of block j + ks / nks
            R.it = ks;
            const int jb = ks / nks;
            origin = block_origin(g, j + jb);
            ks -= jb * nks;
        }
        int offs[8];
        if constexpr (ROW8) {
            const int p0 = ks * 32 + gq * 8;
            const bool ok = FULL || p0 < g.T;
            const int off0 = (origin + in_block(g, ok ? p0 : 0)) * row;
            R.valid = ok ? 0xffu : 0u;
#pragma unroll
            for (int s = 0; s < 8; ++s) offs[s] = off0 + s * row;
        } else {
            R.valid = 0;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int p = ks * 32 + gq * 8 + s;
                const bool ok = p < g.T;
                offs[s] = (origin + in_block(g, ok ? p : g.T - 1)) * row;
                R.valid |= (ok ? 1u : 0u) << s;
            }
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if constexpr (CW == 2) {
                const u32x2 a = ld<NTL>(reinterpret_cast<const u32x2*>(kb + offs[s]));
                const u32x2 c = ld<NTL>(reinterpret_cast<const u32x2*>(vb + offs[s]));
                R.k[s][0] = a.x; R.k[s][1] = a.y;
                R.v[s][0] = c.x; R.v[s][1] = c.y;
            } else {
                R.k[s][0] = ld<NTL>(reinterpret_cast<const uint32_t*>(kb + offs[s]));
                R.v[s][0] = ld<NTL>(reinterpret_cast<const uint32_t*>(vb + offs[s]));
            }
        }
    };
    auto compute = [&](const Raw& R) {
        // V operands first (pure repacking), then one K row tile at a time:
        // phi, rounding to bf16 and that tile's MFMAs.  Padding token slots
        // (read from a real token) are zeroed in the K operand only, which
        // removes them from both S and z.
        u32x4 bw[CPL];
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const uint32_t v0 = R.v[2 * w][c >> 1], v1 = R.v[2 * w + 1][c >> 1];
                bw[c][w] = (c & 1) ? pack_hi(v0, v1) : pack_lo(v0, v1);
            }
#pragma unroll
        for (int r = 0; r < CPL; ++r) {
            u32x4 aw;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t k0 = R.k[2 * w][r >> 1], k1 = R.k[2 * w + 1][r >> 1];
                const float x0 = (r & 1) ? bf_hi(k0) : bf_lo(k0);
                const float x1 = (r & 1) ? bf_hi(k1) : bf_lo(k1);
                if constexpr (FULL) {
                    aw[w] = pack_bf16(phi_fast(x0), phi_fast(x1));
                } else if constexpr (ROW8) {
                    aw[w] = R.valid ? pack_bf16(phi_fast(x0), phi_fast(x1)) : 0u;
                } else {
                    const bool ok0 = (R.valid >> (2 * w)) & 1u, ok1 = (R.valid >> (2 * w + 1)) & 1u;
                    aw[w] = pack_bf16(ok0 ? phi_fast(x0) : 0.f, ok1 ? phi_fast(x1) : 0.f);
                }
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[r][c] = mfma_bf16(aw, bw[c], acc[r][c]);
            if (do_z) accz[r] = mfma_bf16(aw, ones, accz[r]);
        }
    };
    // Record layout: S_j transposed ([e][c], c fastest), then z_j.
    // Lane holds S[c][e] for c = rowbase + 4*CPL*gq + CPL*v + r, e = colbase + CPL*li + c2,
    // and z[c] (every column of accz is the same) for the same c.  The tile
    // goes through this wave's own LDS slice so that every store instruction
    // writes whole record rows (8 lanes x 16 bytes per 128 bytes).
    constexpr int TW = 16 * CPL;          // tile width: 64 (32 for d = 32)
    constexpr int TS = TW + 8;            // padded LDS row
    __shared__ __attribute__((aligned(16))) uint16_t stile_all[8 * TW * TS];
    uint16_t* stile = stile_all + wave * (TW * TS);
    // The record of block jr from acc, accz (through this wave's own LDS slice).
    auto store_record = [&](int jr) {
#pragma unroll
        for (int c2 = 0; c2 < CPL; ++c2) {
            uint32_t wv[2 * CPL];
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int rp = 0; rp < CPL / 2; ++rp)
                    wv[v * (CPL / 2) + rp] = pack_bf16(acc[2 * rp][c2][v], acc[2 * rp + 1][c2][v]);
            uint16_t* dst = stile + (CPL * li + c2) * TS + 4 * CPL * gq;
            *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
            if constexpr (CPL == 4) *reinterpret_cast<u32x4*>(dst + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
        }
        if constexpr (PAIR) {
            // Head 2h + s owns rows e and columns c in [32 s, 32 s + 32) of the
            // tile: each record row is 64 bytes, four lanes x 16 bytes.
            constexpr int DH = 32, RECH = DH * DH + DH;
            const int Hr = 2 * g.H;
#pragma unroll
            for (int k = 0; k < TW / 16; ++k) {
                const int er = k * 16 + (lane >> 2), chunk = lane & 3;
                const int s = er >> 5;
                const u32x4 x = *reinterpret_cast<const u32x4*>(stile + er * TS + DH * s + chunk * 8);
                uint16_t* rech = SZ + (((size_t)(b * Hr + 2 * h + s) * g.M + jr) * g.TP + wgc.t) * RECH;
                *reinterpret_cast<u32x4*>(rech + (er - DH * s) * DH + chunk * 8) = x;
            }
            if (li == 0) {
                // Lane group gq holds z for channels 16 gq .. 16 gq + 15 of the pair.
                uint32_t wv[8];
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int rp = 0; rp < 2; ++rp) wv[v * 2 + rp] = pack_bf16(accz[2 * rp][v], accz[2 * rp + 1][v]);
                const int s = gq >> 1;
                uint16_t* dst = SZ + (((size_t)(b * Hr + 2 * h + s) * g.M + jr) * g.TP + wgc.t) * RECH + DH * DH + 16 * (gq & 1);
                *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
                *reinterpret_cast<u32x4*>(dst + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
            }
            return;
        }
        uint16_t* rec = SZ + (size_t)(((b * g.H + h) * g.M + jr) * g.TP + wgc.t) * (D * D + D);
        constexpr int LPR = TW / 8;           // lanes per tile row (16 bytes each)
#pragma unroll
        for (int k = 0; k < TW / (64 / LPR); ++k) {
            const int er = k * (64 / LPR) + lane / LPR, chunk = lane % LPR;
            const u32x4 x = *reinterpret_cast<const u32x4*>(stile + er * TS + chunk * 8);
            *reinterpret_cast<u32x4*>(rec + (colbase + er) * D + rowbase + chunk * 8) = x;
        }
        if (do_z && li == 0) {
            uint32_t wv[2 * CPL];
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int rp = 0; rp < CPL / 2; ++rp)
                    wv[v * (CPL / 2) + rp] = pack_bf16(accz[2 * rp][v], accz[2 * rp + 1][v]);
            uint16_t* dst = rec + D * D + rowbase + 4 * CPL * gq;
            *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
            if constexpr (CPL == 4) *reinterpret_cast<u32x4*>(dst + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
        }
    };
    if constexpr (NBW > 1) {
        auto compute_nb = [&](const Raw& R) {
            compute(R);
            if (R.it % nks == nks - 1) {
                store_record(j + R.it / nks);
#pragma unroll
                for (int r = 0; r < CPL; ++r) {
                    accz[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        };
        pipelined<PF, Raw>(0, 1, NBW * nks, load, compute_nb);
    } else {
        // This part's run of the block's 32-token steps (all of them when TP = 1).
        const int per = (nks + g.TP - 1) / g.TP;
        const int ks0 = wgc.t * per, ks1 = min(nks, ks0 + per);
        if (ks0 < ks1) pipelined<PF, Raw>(ks0, 1, ks1, load, compute);
        store_record(j);
    }
}

// =====================================================================
// block_kv_summary at head_dim 128: four waves per head that share the
// step's operands through LDS, so every K and V element is read from memory
// once and phi is evaluated once.  Per 32-token step, wave q of a head loads
// one 64-channel half of one tensor (q = 0, 1: K channels 64q ..; q = 2, 3:
// V channels 64(q-2) ..), packs it into MFMA operands (phi for K) and writes
// them to one of two LDS buffers; after a workgroup barrier, wave q reads
// the K half q/2 and the V half q%2 and accumulates that 64 x 64 quadrant of
// S (and z for q%2 == 0).  Lane roles, operand packing, the output mapping
// and the record stores are those of block_kv_summary with rowbase = 64(q/2)
// and colbase = 64(q%2).  Waves of a head past H (odd head counts) load a
// valid head and take part in every barrier but store nothing.
// =====================================================================
template <int PF, bool ROW8, bool FULL, bool NTL, int HPW>
__global__ __launch_bounds__(256 * HPW) __attribute__((amdgpu_waves_per_eu(2)))
void block_kv_summary_d128_bf16(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                uint16_t* __restrict__ SZ, const Geo g, const float* __restrict__ W,
                                uint16_t* __restrict__ Wb, const WConv wc) {
    static_assert(!FULL || ROW8, "FULL implies ROW8");
    constexpr int D = 128, CPL = 4;
    constexpr int TW = 64, TS = TW + 8;                 // record tile width, padded LDS row
    constexpr int OPS = 4 * 64;                         // u32x4 operands of one (tensor, half): [r][lane]
    constexpr int HEADOPS = 4 * OPS;                    // one head: K halves 0, 1, V halves 0, 1
    constexpr int LDS_OPS = 2 * HPW * HEADOPS * 16;     // bytes: two buffers x HPW heads
    constexpr int LDS_TILE = 4 * HPW * TW * TS * 2;     // bytes: record tiles of the 4 HPW waves
    __shared__ u32x4 lds_raw[(LDS_OPS > LDS_TILE ? LDS_OPS : LDS_TILE) / 16];
    if ((int)blockIdx.x >= wc.first_wg) {
        convert_w(W, Wb, wc);
        return;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int quad = wave & 3, hl = wave >> 2;           // quadrant, head within the workgroup
    const int li = lane & 15, gq = lane >> 4;
    const WgCoordP wgc = wg_coord_parts(g, blockIdx.x, g.div_TP);
    const int b = wgc.b, j = wgc.j, h = wgc.hg * g.G + hl;
    const bool active = h < g.H;
    const int hv = active ? h : g.H - 1;                // inactive waves load a valid head
    const int rowbase = (quad >> 1) * 64, colbase = (quad & 1) * 64;
    const bool is_v = quad >= 2;                        // loader role: V half (quad - 2), else K half quad
    const bool do_z = (quad & 1) == 0;
    const int row = g.H * D;
    const int origin = block_origin(g, j);
    const uint16_t* src = (is_v ? V : K) + (b * g.N * row + hv * D + (quad & 1) * 64 + CPL * li);
    const u32x4 ones = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs

    f32x4 acc[CPL][CPL], accz[CPL];
#pragma unroll
    for (int r = 0; r < CPL; ++r) {
        accz[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    struct Raw {
        uint32_t x[8][2];
        uint32_t valid;
        int ks;
    };
    auto load = [&](int ks, Raw& R) {
        R.ks = ks;
        int offs[8];
        if constexpr (ROW8) {
            const int p0 = ks * 32 + gq * 8;
            const bool ok = FULL || p0 < g.T;
            const int off0 = (origin + in_block(g, ok ? p0 : 0)) * row;
            R.valid = ok ? 0xffu : 0u;
#pragma unroll
            for (int s = 0; s < 8; ++s) offs[s] = off0 + s * row;
        } else {
            R.valid = 0;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int p = ks * 32 + gq * 8 + s;
                const bool ok = p < g.T;
                offs[s] = (origin + in_block(g, ok ? p : g.T - 1)) * row;
                R.valid |= (ok ? 1u : 0u) << s;
            }
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x2 a = ld<NTL>(reinterpret_cast<const u32x2*>(src + offs[s]));
            R.x[s][0] = a.x;
            R.x[s][1] = a.y;
        }
    };
    u32x4* ops_head = lds_raw + hl * HEADOPS;           // + buffer * HPW * HEADOPS
    auto compute = [&](const Raw& R) {
        u32x4* buf = ops_head + (R.ks & 1) * (HPW * HEADOPS);
        // Pack this wave's half into operands: K (phi, padding slots zeroed) or V.
        u32x4 op[CPL];
#pragma unroll
        for (int r = 0; r < CPL; ++r)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a0 = R.x[2 * w][r >> 1], a1 = R.x[2 * w + 1][r >> 1];
                if (is_v) {
                    op[r][w] = (r & 1) ? pack_hi(a0, a1) : pack_lo(a0, a1);
                } else {
                    const float x0 = (r & 1) ? bf_hi(a0) : bf_lo(a0);
                    const float x1 = (r & 1) ? bf_hi(a1) : bf_lo(a1);
                    if constexpr (FULL) {
                        op[r][w] = pack_bf16(phi_fast(x0), phi_fast(x1));
                    } else if constexpr (ROW8) {
                        op[r][w] = R.valid ? pack_bf16(phi_fast(x0), phi_fast(x1)) : 0u;
                    } else {
                        const bool ok0 = (R.valid >> (2 * w)) & 1u, ok1 = (R.valid >> (2 * w + 1)) & 1u;
                        op[r][w] = pack_bf16(ok0 ? phi_fast(x0) : 0.f, ok1 ? phi_fast(x1) : 0.f);
                    }
                }
            }
#pragma unroll
        for (int r = 0; r < CPL; ++r) buf[(quad * CPL + r) * 64 + lane] = op[r];
        __syncthreads();
        // This wave's quadrant: K half quad/2 (slots 0, 1) and V half quad%2 (slots 2, 3).
        u32x4 bw[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) bw[c] = buf[((2 + (quad & 1)) * CPL + c) * 64 + lane];
#pragma unroll
        for (int r = 0; r < CPL; ++r) {
            const u32x4 aw = buf[((quad >> 1) * CPL + r) * 64 + lane];
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[r][c] = mfma_bf16(aw, bw[c], acc[r][c]);
            if (do_z) accz[r] = mfma_bf16(aw, ones, accz[r]);
        }
    };
    // This part's run of the block's 32-token steps (all of them when TP = 1).
    const int nks = (g.T + 31) >> 5, per = (nks + g.TP - 1) / g.TP;
    const int ks0 = wgc.t * per, ks1 = min(nks, ks0 + per);
    if (ks0 < ks1) pipelined<PF, Raw>(ks0, 1, ks1, load, compute);
    __syncthreads();   // every wave is done with the operand buffers; the LDS now holds record tiles

    // Record layout and stores as in block_kv_summary (S_j transposed, then z_j).
    uint16_t* stile = reinterpret_cast<uint16_t*>(lds_raw) + wave * (TW * TS);
#pragma unroll
    for (int c2 = 0; c2 < CPL; ++c2) {
        uint32_t wv[2 * CPL];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int rp = 0; rp < CPL / 2; ++rp)
                wv[v * (CPL / 2) + rp] = pack_bf16(acc[2 * rp][c2][v], acc[2 * rp + 1][c2][v]);
        uint16_t* dst = stile + (CPL * li + c2) * TS + 4 * CPL * gq;
        *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
        *reinterpret_cast<u32x4*>(dst + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
    }
    if (!active) return;
    const int blk = ((b * g.H + h) * g.M + j) * g.TP + wgc.t;   // record index (b, h, j, part)
    uint16_t* rec = SZ + (size_t)blk * (D * D + D);
    constexpr int LPR = TW / 8;           // lanes per tile row (16 bytes each)
#pragma unroll
    for (int k = 0; k < TW / (64 / LPR); ++k) {
        const int er = k * (64 / LPR) + lane / LPR, chunk = lane % LPR;
        const u32x4 x = *reinterpret_cast<const u32x4*>(stile + er * TS + chunk * 8);
        *reinterpret_cast<u32x4*>(rec + (colbase + er) * D + rowbase + chunk * 8) = x;
    }
    if (do_z && li == 0) {
        uint32_t wv[2 * CPL];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int rp = 0; rp < CPL / 2; ++rp)
                wv[v * (CPL / 2) + rp] = pack_bf16(accz[2 * rp][v], accz[2 * rp + 1][v]);
        uint16_t* dst = rec + D * D + rowbase + 4 * CPL * gq;
        *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
        *reinterpret_cast<u32x4*>(dst + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
    }
}

// =====================================================================
// mix_summaries (one workgroup per work unit), for any M.
// =====================================================================
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void mix_summaries_bf16(
    const uint16_t* __restrict__ SZ, const uint16_t* __restrict__ Wb, uint16_t* __restrict__ St,
    float* __restrict__ Zt, const Geo g, const MixGeo mg) {
    __shared__ u32x4 sA[MIX_LDS_UNITS];
    mix_tile_bf16<D>(blockIdx.x, SZ, Wb, St, Zt, g, mg, sA);
}

// =====================================================================
// mix_resident: the same product for M <= 256 as a persistent kernel.  One
// workgroup per compute unit; wave (c, it, th) loads its W operands (32 query
// blocks x all source blocks: at most 16 operand registers x 4) once and keeps
// them in registers, and the workgroup walks the work units (b*h, group of CPW
// column tiles) with a stride of the grid size.  The A operands of the next
// unit are loaded from memory while the current unit is multiplied and
// stored, with two LDS buffers for the packed operands.  Lane roles, operand
// packing and output mapping are those of mix_summaries.
// NT bit 0: summary records loaded with the non-temporal hint; bit 1: mixed
// summaries stored with it (they are read once, by the apply kernel).
// =====================================================================
template <int D, int NT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void mix_resident_bf16(
    const uint16_t* __restrict__ SZ, const uint16_t* __restrict__ Wb, uint16_t* __restrict__ St,
    float* __restrict__ Zt, const Geo g, const MixGeo mg) {
    constexpr int REC = D * D + D;
    constexpr int KMAX = 8;         // k-steps (32 source blocks each) held in registers
    constexpr int OROW = 72;        // output staging row: 64 bf16 + 8 padding
    __shared__ u32x4 sA[2][8 * 4 * 64];                                          // 2 x 32 KB
    __shared__ __attribute__((aligned(16))) uint16_t sOut[8 * 32 * OROW];       // 36 KB
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, gq = lane >> 4;
    const int M = g.M;                                // query blocks
    const int NR = g.M * g.TP;                        // source records (partial records of TP parts)
    const int MS = NR * g.RD;                         // k-slots: each record feeds RD of them
    const int NK = (MS + 31) >> 5;                    // <= KMAX (checked on the host)
    const int cpw = mg.CPW;
    const int itr = mg.IT;                            // <= 4 (checked on the host)
    const int th = wave & 1, w2 = wave >> 1;
    const int wc = w2 / itr, wit = w2 % itr;
    const bool wave_ok = w2 < cpw * itr;
    const int U = g.BH * mg.CTG;

    // ---- W operands of this wave, kept for the whole kernel.
    u32x4 bw[KMAX][2];
#pragma unroll
    for (int kk = 0; kk < KMAX; ++kk)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            bw[kk][t] = *reinterpret_cast<const u32x4*>(
                Wb + ((size_t)((wit * 4 + 2 * th + t) * NK + (kk < NK ? kk : NK - 1)) * 64 + lane) * 8);

    // ---- staging roles: thread -> (tile c, li', group of 8 source blocks).
    const int units = cpw * 16 * 4 * NK;              // <= 512
    const int lip = tid & 15;
    const int jg = (tid >> 4) % (4 * NK);
    const int sc = (tid >> 4) / (4 * NK);
    const bool srole = tid < units;
    u32x2 raw[8];
    auto load_a = [&](int unit) {
        const uint32_t bh = fdiv((uint32_t)unit, mg.div_CTG);
        const int ctg = unit - (int)(bh * mg.div_CTG.d);
        const int ct = ctg * cpw + sc;
        const int colp = ct * 64 + 4 * lip;
        const bool ok = srole && colp < REC && ct < mg.CT;
        const int colc = ok ? colp : 0;
        const uint16_t* base = SZ + (size_t)bh * NR * REC;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int jj = (jg >> 2) * 32 + (jg & 3) * 8 + s;
            const u32x2 t = ld<(NT & 1) != 0>(
                reinterpret_cast<const u32x2*>(base + (size_t)((jj < MS ? jj : MS - 1) / g.RD) * REC + colc));
            const uint32_t m = (ok && jj < MS) ? 0xffffffffu : 0u;
            raw[s] = u32x2{t.x & m, t.y & m};
        }
    };
    auto store_a = [&](u32x4* dst) {
        if (srole) {
            const int kk = jg >> 2, lanep = (jg & 3) * 16 + lip;
            u32x4 op[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                op[0][w] = pack_lo(raw[2 * w].x, raw[2 * w + 1].x);
                op[1][w] = pack_hi(raw[2 * w].x, raw[2 * w + 1].x);
                op[2][w] = pack_lo(raw[2 * w].y, raw[2 * w + 1].y);
                op[3][w] = pack_hi(raw[2 * w].y, raw[2 * w + 1].y);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[((sc * 4 + r) * NK + kk) * 64 + lanep] = op[r];
        }
    };

    uint16_t* stage = sOut + wave * (32 * OROW);
    int unit = blockIdx.x;
    load_a(unit);
    for (int buf = 0; unit < U; unit += gridDim.x, buf ^= 1) {
        u32x4* sAb = sA[buf];
        store_a(sAb);
        const int nxt = unit + (int)gridDim.x;
        load_a(nxt < U ? nxt : unit);     // next unit's operands (clamped: always valid)
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();                  // sAb complete; sA[buf ^ 1] free since the last barrier

        const uint32_t bh = fdiv((uint32_t)unit, mg.div_CTG);
        const int ctg = unit - (int)(bh * mg.div_CTG.d);
        const int ct = ctg * cpw + wc;
        const bool active = wave_ok && ct < mg.CT;
        if (!active) continue;
        f32x4 acc[4][2];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KMAX; ++kk) {
            if (kk >= NK) break;
            u32x4 a[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = sAb[((wc * 4 + r) * NK + kk) * 64 + lane];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[r][t] = mfma_bf16(a[r], bw[kk][t], acc[r][t]);
        }

        // ---- output.  Lane holds C[col' = cp0 + 16*gq + 4*v + r][i = it*64 + 32*th + 16*t + li].
        const int cp0 = ct * 64;
        const int it = wit;
        if (cp0 < D * D) {
            // The wave's own LDS slice: written and read back by this wave only.
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
            for (int k = 0; k < 4; ++k) {
                const int rl = 8 * k + (lane >> 3), chunk = lane & 7;
                const int i = it * 64 + 32 * th + rl;
                const u32x4 x = *reinterpret_cast<const u32x4*>(stage + rl * OROW + chunk * 8);
                u32x4* dst = reinterpret_cast<u32x4*>(St + ((size_t)bh * M + i) * (D * D) + cp0 + chunk * 8);
                if (i < M) {
                    if constexpr ((NT & 2) != 0) __builtin_nontemporal_store(x, dst);
                    else *dst = x;
                }
            }
        } else if (cp0 + 16 * gq < REC) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int i = it * 64 + 32 * th + 16 * t + li;
                if (i >= M) continue;
                float* dst = Zt + ((size_t)bh * M + i) * D + (cp0 + 16 * gq - D * D);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    *reinterpret_cast<f32x4*>(dst + 4 * v) = f32x4{acc[0][t][v], acc[1][t][v], acc[2][t][v], acc[3][t][v]};
            }
        }
    }
}

// =====================================================================
// mix_split: the same product with one workgroup of 4 waves per (pair,
// column tile of 64 record elements, tile of 64*TR query blocks), so that
// several workgroups share a compute unit and their load latencies overlap.
// Wave w computes query blocks 16*TR*w .. 16*TR*w + 16*TR - 1 of the tile
// with its W operands for every k-step held in registers; the A operand (the
// column tile of every source record) is staged once per workgroup in LDS,
// already packed as MFMA operands.  Workgroups are dealt to the XCDs
// round-robin, so tiles are numbered such that the query-block tiles of one
// column tile run back to back on one XCD and all but the first read the
// column tile from that XCD's L2.  Lane roles, operand packing and output
// mapping are those of mix_summaries.  At most 256 source records (NK <= 8).
// NT bit 1: mixed summaries stored with the non-temporal hint.
// =====================================================================
struct SplitGeo {
    int32_t CT;          // column tiles of 64 record elements per pair
    int32_t NC;          // column tiles over all pairs (BH * CT)
    FastDiv div_CT, div_NI;   // NI: query-block tiles per column tile
};

template <int D, int TR, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void mix_split_bf16(const uint16_t* __restrict__ SZ,
                                                      const uint16_t* __restrict__ Wb,
                                                      uint16_t* __restrict__ St, float* __restrict__ Zt,
                                                      const Geo g, const SplitGeo sg) {
    constexpr int REC = D * D + D;
    constexpr int KMAX = 8;            // k-steps (32 source records each)
    constexpr int OROW = MIX_OROW;
    constexpr int ROWS = 16 * TR;      // query blocks per wave
    __shared__ u32x4 sA[4 * KMAX * 64];   // A operands [r][kk][lane], 32 KB; then output staging
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, gq = lane >> 4;
    const uint32_t slot = blockIdx.x >> 3;
    const uint32_t cslot = fdiv(slot, sg.div_NI);
    const int itile = (int)(slot - cslot * sg.div_NI.d);
    const uint32_t c = cslot * 8u + (blockIdx.x & 7u);
    if (c >= (uint32_t)sg.NC) return;
    const uint32_t bh = fdiv(c, sg.div_CT);
    const int cp0 = (int)(c - bh * sg.div_CT.d) * 64;   // first record element of the tile
    const int M = g.M, NR = g.M * g.TP, MS = NR * g.RD, NK = (MS + 31) >> 5;
    const int i0 = itile * (4 * ROWS) + wave * ROWS;    // first query block of this wave
    const bool active = i0 < M;                         // then i0 + ROWS <= roundup(M, 32): inside Wb's rows
    const int rt0 = active ? i0 >> 4 : 0;

    // ---- W operands (B) of every k-step; positions past NK reload a valid step.
    u32x4 bw[KMAX][TR];
#pragma unroll
    for (int kk = 0; kk < KMAX; ++kk)
#pragma unroll
        for (int t = 0; t < TR; ++t)
            bw[kk][t] = *reinterpret_cast<const u32x4*>(
                Wb + ((size_t)((rt0 + t) * NK + (kk < NK ? kk : NK - 1)) * 64 + lane) * 8);

    // ---- stage A: unit (li', group of 8 source records) -> 4 packed operands.
    const int units = 16 * 4 * NK;                      // <= 512: at most two per thread
    const uint16_t* base = SZ + (size_t)bh * NR * REC;
    u32x2 raw[2][8];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int u = tid + 256 * p;
        const int colp = cp0 + 4 * (u & 15);
        const bool ok = u < units && colp < REC;
        const int colc = ok ? colp : 0;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            // Clamped address, then a mask: the load stays unconditional.
            const int jj = 8 * (u >> 4) + s;
            const u32x2 t = *reinterpret_cast<const u32x2*>(base + (size_t)((jj < MS ? jj : MS - 1) / g.RD) * REC + colc);
            const uint32_t m = (ok && jj < MS) ? 0xffffffffu : 0u;
            raw[p][s] = u32x2{t.x & m, t.y & m};
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int u = tid + 256 * p;
        if (u < units) {
            const int jg = u >> 4, kk = jg >> 2, lanep = (jg & 3) * 16 + (u & 15);
            u32x4 op[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                op[0][w] = pack_lo(raw[p][2 * w].x, raw[p][2 * w + 1].x);
                op[1][w] = pack_hi(raw[p][2 * w].x, raw[p][2 * w + 1].x);
                op[2][w] = pack_lo(raw[p][2 * w].y, raw[p][2 * w + 1].y);
                op[3][w] = pack_hi(raw[p][2 * w].y, raw[p][2 * w + 1].y);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sA[(r * NK + kk) * 64 + lanep] = op[r];
        }
    }
    __syncthreads();

    f32x4 acc[4][TR];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < TR; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
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
                for (int t = 0; t < TR; ++t) acc[r][t] = mfma_bf16(a[r], bw[kk][t], acc[r][t]);
        }
    }
    __syncthreads();   // every wave is done with the A operands
    if (!active) return;

    // ---- output.  Lane holds C[col' = cp0 + 16*gq + 4*v + r][i = i0 + 16*t + li].
    if (cp0 < D * D) {
        // The wave's own LDS slice: written and read back by this wave only.
        uint16_t* stage = reinterpret_cast<uint16_t*>(sA) + wave * (ROWS * OROW);
#pragma unroll
        for (int t = 0; t < TR; ++t) {
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
        // ROWS rows of 128 bytes: 8 lanes per row, 8 rows per instruction.
#pragma unroll
        for (int k = 0; k < ROWS / 8; ++k) {
            const int rl = 8 * k + (lane >> 3), chunk = lane & 7;
            const int i = i0 + rl;
            const u32x4 x = *reinterpret_cast<const u32x4*>(stage + rl * OROW + chunk * 8);
            u32x4* dst = reinterpret_cast<u32x4*>(St + ((size_t)bh * M + i) * (D * D) + cp0 + chunk * 8);
            if (i < M) {
                if constexpr ((NT & 2) != 0) __builtin_nontemporal_store(x, dst);
                else *dst = x;
            }
        }
    } else if (cp0 + 16 * gq < REC) {
#pragma unroll
        for (int t = 0; t < TR; ++t) {
            const int i = i0 + 16 * t + li;
            if (i >= M) continue;
            float* dst = Zt + ((size_t)bh * M + i) * D + (cp0 + 16 * gq - D * D);
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
// straight from Q (8 consecutive channels per lane).  The denominator also
// runs on the matrix cores: two extra row tiles whose every row is zt_i
// (split into a bf16 high part and the bf16 rounding of the remainder), so
// every lane receives its token's phi(q) . zt_i without cross-lane sums.
// =====================================================================
template <int D, int NWA, int PF, bool NTL, int MAXW, typename Ops, typename PrepLoad, typename PrepFinish>
__device__ __forceinline__ void apply_tokens_bf16(Ops A, PrepLoad&& prep_load, PrepFinish&& prep_finish,
                                                  const uint16_t* __restrict__ Q,
                                                  uint16_t* __restrict__ O, const Geo& g, int bh,
                                                  int i, int wave, int lane, int p0 = 0, int p1 = -1,
                                                  bool active = true) {
    // Tokens [p0, p1) of block i (p1 < 0: to the block's end).  A wave that is
    // not active (a head past the last, an empty part) only takes part in the
    // operands' preparation when that has a workgroup barrier (Ops::kShared).
    if (p1 < 0) p1 = g.T;
    constexpr int RT = D / 16, KS = D / 32;
    const int t = lane & 15, gq = lane >> 4;
    // bh and i are wave-uniform; say so, so that addresses and the buffer
    // descriptor below live in scalar registers.
    bh = __builtin_amdgcn_readfirstlane(bh);
    i = __builtin_amdgcn_readfirstlane(i);
    const int b = (int)fdiv(bh, g.div_H), h = bh - b * g.H;
    const int row = g.H * D;
    const int origin = block_origin(g, i);
    const uint16_t* qb = Q + (b * g.N * row + h * D);
    // Output of batch b as a raw buffer (at most 2^31 bytes: checked on the host);
    // the descriptor is wave-uniform, per-lane parts go in the offset.
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        O + (size_t)b * g.N * row, 0, g.N * row * 2, 0x00020000);
    const int olane = h * D * 2;
    const int nit = (p1 - p0 + 15) >> 4;
    // Output staging: 16 tokens x D channels per wave, rows padded by 8 elements.
    constexpr int OSTR = D + 8;
    constexpr int CPR = D / 8;   // 16-byte chunks per token row
    __shared__ __attribute__((aligned(16))) uint16_t sout_all[MAXW * 16 * OSTR];
    uint16_t* sout = sout_all + (threadIdx.x >> 6) * (16 * OSTR);

    // d <= 64: the group's q rows are loaded whole: load k brings tokens TPI k
    // .. TPI k + TPI - 1, CPR lanes per row (consecutive lanes, consecutive 16
    // bytes), and the rows go through the wave's LDS slice into the B-operand
    // layout (lane (t, gq): token t, channels kk*32 + 8 gq ..); read straight in
    // that layout, consecutive lanes would address different token rows
    // (dit-s2-256x256 apply 23.5 -> 22.1 us, dit-s2-64x64 53.3 -> 50.7 us,
    // sana-128x128 67.9 -> 65.2 us).  At d = 128 the direct loads stay
    // (video-16x64x64 apply 101.9 against 102.6 us).
    constexpr bool QROWS = D <= 64;
    constexpr int TPI = 64 / CPR;   // token rows per load instruction; 16 / TPI == KS
    struct Raw {
        u32x4 q[KS];
        int off;
        bool ok;
    };
    auto load = [&](int it, Raw& R) {
        const int p = p0 + it * 16 + t;
        R.ok = p < p1;   // false for padding lanes and for groups past the end
        R.off = (origin + in_block(g, R.ok ? p : p1 - 1)) * row;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            if constexpr (QROWS) {
                const int offk = __shfl(R.off, k * TPI + lane / CPR, 64);
                R.q[k] = ld<NTL>(reinterpret_cast<const u32x4*>(qb + offk + (lane % CPR) * 8));
            } else {
                R.q[k] = ld<NTL>(reinterpret_cast<const u32x4*>(qb + R.off + k * 32 + gq * 8));
            }
        }
    };
    auto compute = [&](const Ops& A, const Raw& R) {
        u32x4 qv[KS];
        if constexpr (QROWS) {
#pragma unroll
            for (int k = 0; k < KS; ++k)
                *reinterpret_cast<u32x4*>(sout + (k * TPI + lane / CPR) * OSTR + (lane % CPR) * 8) = R.q[k];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                qv[kk] = *reinterpret_cast<const u32x4*>(sout + t * OSTR + kk * 32 + gq * 8);
        } else {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) qv[kk] = R.q[kk];
        }
        u32x4 bq[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int w = 0; w < 4; ++w)
                bq[kk][w] = pack_bf16(phi_fast(bf_lo(qv[kk][w])), phi_fast(bf_hi(qv[kk][w])));
        f32x4 acc[RT], accd = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
            for (int r = 0; r < RT; ++r) acc[r] = mfma_bf16(A.op(r, kk, lane), bq[kk], acc[r]);
            accd = mfma_bf16(A.hi(kk, lane), bq[kk], accd);
            accd = mfma_bf16(A.lo(kk, lane), bq[kk], accd);
        }
        const float inv = 1.f / (accd[0] + g.eps);
        uint32_t wv[2 * RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            wv[2 * r] = pack_bf16(acc[r][0] * inv, acc[r][1] * inv);
            wv[2 * r + 1] = pack_bf16(acc[r][2] * inv, acc[r][3] * inv);
        }
        // The 16 x D output tile goes through this wave's LDS slice so that each
        // store instruction writes whole rows of 2*D bytes (8 lanes x 16 bytes per
        // 128-byte line) instead of interleaved 16-byte pieces of every row.
        uint16_t* srow = sout + t * OSTR + 4 * RT * gq;
#pragma unroll
        for (int u = 0; u < RT / 2; ++u)
            *reinterpret_cast<u32x4*>(srow + 8 * u) = u32x4{wv[4 * u], wv[4 * u + 1], wv[4 * u + 2], wv[4 * u + 3]};
        // Buffer stores: a lane past the block's last token gets an offset
        // beyond the buffer's range and the hardware drops its write, so the
        // store needs no branch.
#pragma unroll
        for (int k = 0; k < D / 32; ++k) {
            const int tt = k * (64 / CPR) + lane / CPR, chunk = lane % CPR;
            const int offk = __shfl(R.off, tt, 64);
            const int okk = __shfl((int)R.ok, tt, 64);
            const u32x4 x = *reinterpret_cast<const u32x4*>(sout + tt * OSTR + chunk * 8);
            const uint32_t bo = okk ? (uint32_t)(offk * 2 + olane + chunk * 16) : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b128(x, orsrc, bo, 0, 0);
        }
    };

    // Batches of PF token groups: all loads of a batch are issued together
    // (clamped past the end), then the groups are computed and stored.  No
    // buffer is carried across iterations, so every wait is exact.
    // Groups past the end load the block's last token and store nothing
    // (their lanes are all "not ok"), so the body has no branch the compiler
    // could sink the loads into.
    // Two batch buffers alternate: the next batch's loads are issued before the
    // current batch is computed and stored.  The first batch goes out before
    // the block's St / zt operands, the second right after them.
    const bool work = active && wave < nit;
    if (!Ops::kShared && !work) return;
    const int step = NWA * PF;
    Raw ra[PF], rb[PF];
    if (work) {
#pragma unroll
        for (int u = 0; u < PF; ++u) load(wave + u * NWA, ra[u]);
    }
    prep_load(A);
    if (!work) return;
    int it0 = wave;
#pragma unroll
    for (int u = 0; u < PF; ++u) load(it0 + step + u * NWA, rb[u]);
    // Keep the scheduler from sinking the batch's loads next to their uses.
    __builtin_amdgcn_sched_barrier(0);
    prep_finish(A);
    for (;;) {
#pragma unroll
        for (int u = 0; u < PF; ++u) compute(A, ra[u]);
        if (it0 + step >= nit) break;
#pragma unroll
        for (int u = 0; u < PF; ++u) load(it0 + 2 * step + u * NWA, ra[u]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < PF; ++u) compute(A, rb[u]);
        it0 += 2 * step;
        if (it0 >= nit) break;
#pragma unroll
        for (int u = 0; u < PF; ++u) load(it0 + step + u * NWA, rb[u]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Workgroup = query block i of batch b for G consecutive heads x NWA waves
// splitting the block's tokens, at most MAXW waves.
// LDSA: the NWA waves of each head first stage the head's operands (St_i^T
// row tiles and zt_i's high and low words) once in LDS and read them from
// there for every token group; each wave then holds about 30 fewer
// registers (d = 64: 97 -> 66, so 7 instead of 4 waves per SIMD) and St_i
// leaves L2 once per head instead of once per wave.  Otherwise each wave
// loads them into its own registers.
template <int D, int NWA, int PF, bool NTL, int MAXW, bool LDSA>
__global__ __launch_bounds__(64 * MAXW) void query_apply_bf16(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ St,
                                                        const float* __restrict__ Zt,
                                                        uint16_t* __restrict__ O, const Geo g) {
    constexpr int RT = D / 16, KS = D / 32;
    const int wave = (threadIdx.x >> 6) % NWA, lane = threadIdx.x & 63;
    const int t = lane & 15, gq = lane >> 4;
    const WgCoordP wgc = wg_coord_parts(g, blockIdx.x, g.div_AP);
    const int hs = (int)(threadIdx.x >> 6) / NWA;   // the head's slot in the workgroup
    const int h = wgc.hg * g.G + hs;
    const int i = wgc.j;
    // Part t of AP contiguous runs of the block's 16-token groups.
    const int ngr = (g.T + 15) >> 4, gper = (ngr + g.AP - 1) / g.AP;
    const int p0 = min(g.T, 16 * gper * wgc.t), p1 = min(g.T, p0 + 16 * gper);
    const int bh = wgc.b * g.H + h;
    const int blk = bh * g.M + i;
    const uint16_t* sb = St + (size_t)blk * (D * D);
    const float* zb = Zt + (size_t)blk * D;
    if constexpr (LDSA) {
        constexpr int WORDS = ApplyL<D>::WORDS;
        __shared__ u32x4 opw[(MAXW / NWA) * WORDS];
        u32x4* w = opw + hs * WORDS;
        const bool active = h < g.H && p0 < p1;
        auto stage = [&](ApplyL<D>&) {
            if (active) {
                const int x0 = (int)threadIdx.x - hs * 64 * NWA;
                for (int wi = x0; wi < WORDS; wi += 64 * NWA) {
                    const int ln = wi & 63, tl = ln & 15, gl = ln >> 4;
                    if (wi < RT * KS * 64) {
                        const int r = wi / (KS * 64), kk = (wi >> 6) % KS;
                        const int e = 4 * RT * (tl >> 2) + 4 * r + (tl & 3);
                        w[wi] = *reinterpret_cast<const u32x4*>(sb + e * D + kk * 32 + gl * 8);
                    } else {
                        const int zi = wi - RT * KS * 64, part = zi / (KS * 64), kk = (zi >> 6) % KS;
                        const f32x4 x = *reinterpret_cast<const f32x4*>(zb + kk * 32 + gl * 8);
                        const f32x4 y = *reinterpret_cast<const f32x4*>(zb + kk * 32 + gl * 8 + 4);
                        const float z[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
                        u32x4 hi, lo;
                        split_zt(z, hi, lo);
                        w[wi] = part == 0 ? hi : lo;
                    }
                }
            }
            __syncthreads();
        };
        auto none = [&](ApplyL<D>&) {};
        // The first batch of Q loads is in flight while the operands are staged.
        apply_tokens_bf16<D, NWA, PF, NTL, MAXW>(ApplyL<D>{w}, stage, none, Q, O, g, bh, i, wave, lane,
                                                  active ? p0 : 0, active ? p1 : 1, active);
    } else {
        if (h >= g.H || p0 >= p1) return;
        f32x4 zraw[KS][2];
        auto prep_load = [&](ApplyA<D>& A) {
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int e = 4 * RT * (t >> 2) + 4 * r + (t & 3);
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    A.a[r][kk] = *reinterpret_cast<const u32x4*>(sb + e * D + kk * 32 + gq * 8);
            }
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                zraw[kk][0] = *reinterpret_cast<const f32x4*>(zb + kk * 32 + gq * 8);
                zraw[kk][1] = *reinterpret_cast<const f32x4*>(zb + kk * 32 + gq * 8 + 4);
            }
        };
        auto prep_finish = [&](ApplyA<D>& A) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const f32x4 x = zraw[kk][0], y = zraw[kk][1];
                const float z[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
                split_zt(z, A.zhi[kk], A.zlo[kk]);
            }
        };
        apply_tokens_bf16<D, NWA, PF, NTL, MAXW>(ApplyA<D>{}, prep_load, prep_finish, Q, O, g, bh, i, wave, lane,
                                                  p0, p1);
    }
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
    __shared__ int s_idx[256], s_cnt[4];
    __shared__ float s_w[256];
    // Row i of W 256 entries at a time: the nonzero weights are listed first,
    // so a sparse row costs only its nonzeros.
    for (int j0 = 0; j0 < M; j0 += 256) {
        const int n = compact_nonzero(wr, M, j0, s_idx, s_w, s_cnt);
        for (int t = 0; t < n; ++t) {
            const float w = s_w[t];
            const uint16_t* src = base + (size_t)s_idx[t] * REC;
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
        __syncthreads();   // the list is rebuilt by the next pass
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
    auto prep_load = [&](ApplyA<D>& A) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int e = 4 * RT * (t >> 2) + 4 * r + (t & 3);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) A.a[r][kk] = *reinterpret_cast<const u32x4*>(sSt + e * D + kk * 32 + gq * 8);
        }
    };
    auto prep_finish = [&](ApplyA<D>& A) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float z[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) z[s] = sZt[kk * 32 + gq * 8 + s];
            split_zt(z, A.zhi[kk], A.zlo[kk]);
        }
    };
    apply_tokens_bf16<D, 4, 2, false, 4>(ApplyA<D>{}, prep_load, prep_finish, Q, O, g, bh, i, wave, lane);
}

// =====================================================================
// launchers
// =====================================================================
inline void record(const Launch& L, int k) {
    if (L.events) (void)hipEventRecord(L.events[k], L.stream);
}

// Head groups: G heads per workgroup with `per_head` waves each, at most 8
// waves, with the heads spread evenly over the groups.
inline Geo with_head_groups(Geo g, int per_head, int max_waves = 8) {
    const int gmax = max_waves / per_head;
    g.HG = (g.H + gmax - 1) / gmax;
    g.G = (g.H + g.HG - 1) / g.HG;
    g.div_HG = make_fastdiv((uint32_t)g.HG);
    return g;
}

template <int D, int PF, bool ROW8, bool FULL, bool PAIR = false>
void launch_summary(const Launch& L, const uint16_t* k, const uint16_t* v, uint16_t* sz,
                    const WConv& wc) {
    constexpr int NQ = D == 128 ? 4 : 1;
    Geo gp = L.g;
    if (PAIR) {   // head pairs of 32 channels read as heads of 64
        gp.H /= 2;
        gp.D = 64;
        gp.BH = gp.B * gp.H;
    }
    const Geo g = with_head_groups(gp, NQ);
    const int nsum = g.B * g.M * g.TP * g.HG, threads = 64 * NQ * g.G;
    WConv w = wc;
    const int nchunks = wc.nchunks + (wc.wbt ? wc.nchunks_t : 0);
    const int nconv = (nchunks + threads - 1) / threads;   // one chunk per thread
    w.first_wg = nsum;
    w.nconv = nconv;
    if constexpr (D == 128) {
        if (L.tune.d128_shared) {
            // HPW heads (4 waves each) per workgroup
            const Geo g1 = with_head_groups(gp, NQ, 4 * L.tune.d128_shared);
            const int ns1 = g1.B * g1.M * g1.TP * g1.HG, th1 = 64 * NQ * g1.G;
            WConv w1 = wc;
            w1.first_wg = ns1;
            w1.nconv = (nchunks + th1 - 1) / th1;
            auto* wbp = static_cast<uint16_t*>(L.wb);
            if (L.tune.d128_shared == 1) {
                if (L.tune.nt_loads)
                    block_kv_summary_d128_bf16<PF, ROW8, FULL, true, 1><<<ns1 + w1.nconv, th1, 0, L.stream>>>(k, v, sz, g1, L.W, wbp, w1);
                else
                    block_kv_summary_d128_bf16<PF, ROW8, FULL, false, 1><<<ns1 + w1.nconv, th1, 0, L.stream>>>(k, v, sz, g1, L.W, wbp, w1);
            } else {
                if (L.tune.nt_loads)
                    block_kv_summary_d128_bf16<PF, ROW8, FULL, true, 2><<<ns1 + w1.nconv, th1, 0, L.stream>>>(k, v, sz, g1, L.W, wbp, w1);
                else
                    block_kv_summary_d128_bf16<PF, ROW8, FULL, false, 2><<<ns1 + w1.nconv, th1, 0, L.stream>>>(k, v, sz, g1, L.W, wbp, w1);
            }
            return;
        }
    }
    if constexpr (FULL && D <= 64) {
        // Blocks of at most 64 tokens (one or two 32-token steps): each wave
        // walks four (else two) blocks, so the pipeline does not fill and
        // drain once per block (dit-s2-64x64 summary 65.0 -> 60.8 us with two,
        // 58.3 us with four; sana-128x128 80.8 -> 77.9 -> 77.5 us).
        auto go = [&](auto nbw) {
            constexpr int NBW = decltype(nbw)::value;
            const int nsb = g.B * (g.M / NBW) * g.HG;
            WConv wb = w;
            wb.first_wg = nsb;
            if (L.tune.nt_loads)
                block_kv_summary_bf16<D, PF, ROW8, FULL, true, PAIR, NBW><<<nsb + nconv, threads, 0, L.stream>>>(
                    k, v, sz, g, L.W, static_cast<uint16_t*>(L.wb), wb);
            else
                block_kv_summary_bf16<D, PF, ROW8, FULL, false, PAIR, NBW><<<nsb + nconv, threads, 0, L.stream>>>(
                    k, v, sz, g, L.W, static_cast<uint16_t*>(L.wb), wb);
        };
        if (g.TP == 1 && g.T <= 64 && g.M % 4 == 0) {
            go(std::integral_constant<int, 4>{});
            return;
        }
        if (g.TP == 1 && g.T <= 64 && g.M % 2 == 0) {
            go(std::integral_constant<int, 2>{});
            return;
        }
    }
    if (L.tune.nt_loads)
        block_kv_summary_bf16<D, PF, ROW8, FULL, true, PAIR><<<nsum + nconv, threads, 0, L.stream>>>(
            k, v, sz, g, L.W, static_cast<uint16_t*>(L.wb), w);
    else
        block_kv_summary_bf16<D, PF, ROW8, FULL, false, PAIR><<<nsum + nconv, threads, 0, L.stream>>>(
            k, v, sz, g, L.W, static_cast<uint16_t*>(L.wb), w);
}

// head_dim 32 with an even head count runs as head pairs of 64 channels.
template <int D, int PF, bool ROW8, bool FULL>
void launch_summary_any(const Launch& L, const uint16_t* k, const uint16_t* v, uint16_t* sz, const WConv& wc) {
    if constexpr (D == 32) {
        if (L.g.H % 2 == 0 && L.tune.pair_heads) {
            launch_summary<64, PF, ROW8, FULL, true>(L, k, v, sz, wc);
            return;
        }
    }
    launch_summary<D, PF, ROW8, FULL>(L, k, v, sz, wc);
}

template <int D, int NWA, int PF, int MAXW>
void launch_apply_pf(const Launch& L, const uint16_t* q, const uint16_t* st, uint16_t* o) {
    const Geo g = with_head_groups(L.g, NWA, MAXW);
    const int grid = g.B * g.M * g.AP * g.HG, block = 64 * NWA * g.G;
    if constexpr (D <= 64) {
        if (L.tune.apply_lds) {
            if (L.tune.nt_apply) query_apply_bf16<D, NWA, PF, true, MAXW, true><<<grid, block, 0, L.stream>>>(q, st, L.zt, o, g);
            else query_apply_bf16<D, NWA, PF, false, MAXW, true><<<grid, block, 0, L.stream>>>(q, st, L.zt, o, g);
            return;
        }
    }
    if (L.tune.nt_apply) query_apply_bf16<D, NWA, PF, true, MAXW, false><<<grid, block, 0, L.stream>>>(q, st, L.zt, o, g);
    else query_apply_bf16<D, NWA, PF, false, MAXW, false><<<grid, block, 0, L.stream>>>(q, st, L.zt, o, g);
}

template <int D, int NWA>
void launch_apply(const Launch& L, const uint16_t* q, const uint16_t* st, uint16_t* o) {
    if constexpr (NWA <= 2) {
        if (L.tune.apply_maxw == 2) {
            if (L.tune.apply_pf == 1) launch_apply_pf<D, NWA, 1, 2>(L, q, st, o);
            else if (L.tune.apply_pf == 2) launch_apply_pf<D, NWA, 2, 2>(L, q, st, o);
            else launch_apply_pf<D, NWA, 4, 2>(L, q, st, o);
            return;
        }
    }
    if (L.tune.apply_maxw == 4) {
        if (L.tune.apply_pf == 1) launch_apply_pf<D, NWA, 1, 4>(L, q, st, o);
        else launch_apply_pf<D, NWA, 2, 4>(L, q, st, o);
        return;
    }
    switch (L.tune.apply_pf) {
        case 1: launch_apply_pf<D, NWA, 1, 8>(L, q, st, o); break;
        case 2: launch_apply_pf<D, NWA, 2, 8>(L, q, st, o); break;
        default: launch_apply_pf<D, NWA, 4, 8>(L, q, st, o); break;
    }
}

// The mixing product of records with W's operands: out[i] = sum_j w(i, j) rec[j]
// over the M * TP * RD k-slots of g, for the forward's summaries (W) and the
// backward's gradient records (W^T, TP = RD = 1); outputs St-style bf16
// records and fp32 normalisers.  The kernel follows the problem: mix_split
// with at most 256 source k-slots, the persistent kernel when so tuned (at
// most 64 query blocks, head_dim 128, or head_dim 32 with many pairs by
// default), the per-tile kernel otherwise.
template <int D>
void launch_mixing(const Launch& L, const uint16_t* src, const uint16_t* wops, uint16_t* dst, float* zdst,
                   const Geo& g) {
    const int IT = (g.M + 63) / 64, NK = (g.M * g.TP * g.RD + 31) / 32;
    MixGeo mg;
    mg.CT = (D * D + D + 63) / 64;
    mg.IT = IT;
    // Column tiles per workgroup: its 8 waves cover CPW tiles x IT query
    // tiles x 2, and the A staging (one unit per thread) needs CPW * min(NK, 8) <= 8.
    const int nkp = NK < 8 ? NK : 8;
    mg.CPW = IT >= 4 ? 1 : 4 / IT;
    if (mg.CPW * nkp > 8) mg.CPW = 8 / nkp;
    mg.CTG = (mg.CT + mg.CPW - 1) / mg.CPW;
    mg.Jpad = NK * 32;
    mg.div_CTG = make_fastdiv(mg.CTG);
    if (L.tune.mix_kind == 2 && NK <= 8) {
        SplitGeo sg;
        sg.CT = mg.CT;
        sg.NC = g.BH * mg.CT;
        sg.div_CT = make_fastdiv((uint32_t)mg.CT);
        const int tr = (g.M <= 64 || L.tune.mix_rows == 1) ? 1 : 2;
        const int ni = (g.M + 64 * tr - 1) / (64 * tr);
        sg.div_NI = make_fastdiv((uint32_t)ni);
        const int grid = 8 * ni * ((sg.NC + 7) / 8);
        const bool nt = (L.tune.nt_mix & 2) != 0;
        if (tr == 1) {
            if (nt) mix_split_bf16<D, 1, 2><<<grid, 256, 0, L.stream>>>(src, wops, dst, zdst, g, sg);
            else mix_split_bf16<D, 1, 0><<<grid, 256, 0, L.stream>>>(src, wops, dst, zdst, g, sg);
        } else {
            if (nt) mix_split_bf16<D, 2, 2><<<grid, 256, 0, L.stream>>>(src, wops, dst, zdst, g, sg);
            else mix_split_bf16<D, 2, 0><<<grid, 256, 0, L.stream>>>(src, wops, dst, zdst, g, sg);
        }
    } else if (L.tune.mix_kind == 1 && IT <= 4 && NK <= 8) {
        // NK <= 8: at most 256 source records (M <= 256, M * TP <= 256).
        const int units = g.BH * mg.CTG;
        const int grid = units < L.tune.num_cus ? units : L.tune.num_cus;
        switch (L.tune.nt_mix) {
            case 1: mix_resident_bf16<D, 1><<<grid, 512, 0, L.stream>>>(src, wops, dst, zdst, g, mg); break;
            case 2: mix_resident_bf16<D, 2><<<grid, 512, 0, L.stream>>>(src, wops, dst, zdst, g, mg); break;
            case 3: mix_resident_bf16<D, 3><<<grid, 512, 0, L.stream>>>(src, wops, dst, zdst, g, mg); break;
            default: mix_resident_bf16<D, 0><<<grid, 512, 0, L.stream>>>(src, wops, dst, zdst, g, mg); break;
        }
    } else {
        mix_summaries_bf16<D><<<g.BH * mg.CTG, 512, 0, L.stream>>>(src, wops, dst, zdst, g, mg);
    }
}

template <int D>
hipError_t run_d(const Launch& L0) {
    // Token parts apply to the 3-kernel forward and the backward's recompute
    // (which folds the partial records itself); the fused and causal paths
    // read one record per block.
    Launch L = L0;
    if (L.path != MHLA_PATH_3KERNEL || L.g.TP < 1 || L.g.AP < 1) {
        L.g.TP = L.g.AP = 1;
        L.g.div_TP = L.g.div_AP = make_fastdiv(1u);
    }
    const Geo& g = L.g;
    const int nblk = g.BH * g.M;
    const auto* q = static_cast<const uint16_t*>(L.q);
    const auto* k = static_cast<const uint16_t*>(L.k);
    const auto* v = static_cast<const uint16_t*>(L.v);
    auto* o = static_cast<uint16_t*>(L.out);
    auto* sz = static_cast<uint16_t*>(L.sz);
    auto* st = static_cast<uint16_t*>(L.st);
    const bool fused = L.path == MHLA_PATH_FUSED;
    // IT: 64-block tiles of query blocks; NK: 32-record k-steps over the
    // M * TP source records.
    const int IT = (g.M + 63) / 64, NK = (g.M * g.TP * g.RD + 31) / 32;
    WConv wc;
    wc.M = g.M;
    wc.TP = g.TP;
    wc.NK = NK;
    wc.nchunks = fused ? 0 : IT * 64 * NK * 32 / 8;
    wc.NKt = (g.M + 31) / 32;
    wc.nchunks_t = IT * 64 * wc.NKt * 32 / 8;
    wc.WD = g.WD;
    wc.WM = g.WM;
    wc.RD = g.RD;
    wc.first_wg = 0;
    wc.nconv = 0;
    wc.wbt = static_cast<uint16_t*>(L.wbt);
    const bool causal = L.path == MHLA_PATH_CAUSAL;
    wc.causal = causal ? 1 : 0;   // mixed summaries of earlier blocks only
    const bool row8 = (g.bk2 % 8) == 0;

    record(L, 0);
    const bool full = row8 && (g.T % 32) == 0;
    if (L.tune.summary_pf == 1) {
        if (full) launch_summary_any<D, 1, true, true>(L, k, v, sz, wc);
        else if (row8) launch_summary_any<D, 1, true, false>(L, k, v, sz, wc);
        else launch_summary_any<D, 1, false, false>(L, k, v, sz, wc);
    } else {
        if (full) launch_summary_any<D, 2, true, true>(L, k, v, sz, wc);
        else if (row8) launch_summary_any<D, 2, true, false>(L, k, v, sz, wc);
        else launch_summary_any<D, 2, false, false>(L, k, v, sz, wc);
    }
    record(L, 1);
    if (fused) {
        record(L, 2);
        query_apply_fused_bf16<D><<<nblk, 256, 0, L.stream>>>(q, sz, L.W, o, g);
    } else {
        launch_mixing<D>(L, sz, static_cast<const uint16_t*>(L.wb), st, L.zt, g);
        record(L, 2);
        if (L.summaries_only) return hipGetLastError();
        if (causal) {
            const hipError_t e = launch_causal_apply_bf16(L);
            record(L, 3);
            return e;
        }
        switch (L.tune.apply_waves) {
            case 1: launch_apply<D, 1>(L, q, st, o); break;
            case 2: launch_apply<D, 2>(L, q, st, o); break;
            default: launch_apply<D, 4>(L, q, st, o); break;
        }
    }
    record(L, 3);
    return hipGetLastError();
}

}  // namespace

hipError_t run_bf16_summaries(const Launch& L) {
    Launch S = L;
    S.summaries_only = 1;
    S.path = MHLA_PATH_3KERNEL;
    S.events = nullptr;
    return run_bf16(S);
}

hipError_t launch_mix_records_bf16(const Launch& L, const uint16_t* src, const uint16_t* wops, uint16_t* dst,
                                  float* zdst, const Geo& g) {
    switch (g.D) {
        case 32: launch_mixing<32>(L, src, wops, dst, zdst, g); break;
        case 64: launch_mixing<64>(L, src, wops, dst, zdst, g); break;
        case 128: launch_mixing<128>(L, src, wops, dst, zdst, g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t run_bf16(const Launch& L) {
    switch (L.g.D) {
        case 32: return run_d<32>(L);
        case 64: return run_d<64>(L);
        case 128: return run_d<128>(L);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mhla
