// bf16_shared.h -- device code shared by the bf16 forward and backward kernels:
// load helpers, the software pipeline, the conversion of W to the mixing
// kernel's operand order, the mixing work unit, and the apply operands.
#pragma once

#include "common.h"

namespace mhla {
namespace {

// Loads of data read exactly once (q, k, v) may carry the non-temporal hint
// so they do not displace the summaries in the caches.
template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// =====================================================================
// Software pipeline: iterations first, first + step, ... < n (n >= 1), with
// the loads of PF later iterations in flight while one is computed.  Buffers
// rotate with compile-time indices so they stay in registers.  Every load is
// issued unconditionally (indices past the end are clamped to the last
// iteration and the data ignored): a load under a branch would make the
// compiler's wait counts conservative and drain the prefetched loads too.
// =====================================================================
template <int PF, typename Buf, typename LoadF, typename ComputeF>
__device__ __forceinline__ void pipelined(int first, int step, int n, LoadF&& load, ComputeF&& compute) {
    Buf buf[PF + 1];
    const int last = n - 1;
#pragma unroll
    for (int s = 0; s < PF; ++s) load(min(first + s * step, last), buf[s]);
    for (int base = first; base < n; base += step * (PF + 1)) {
#pragma unroll
        for (int u = 0; u <= PF; ++u) {
            const int it = base + u * step;
            if (it >= n) break;
            load(min(it + PF * step, last), buf[(u + PF) % (PF + 1)]);
            __builtin_amdgcn_sched_barrier(0);   // issue the prefetch before computing
            compute(buf[u]);
        }
    }
}

// W (fp32 [M][M]) -> bf16, zero padded to [Ipad = 64 * IT][Jpad = 32 * NK] and
// stored in the mixing kernel's B-operand order: 16-byte unit
// (rt * NK + kk) * 64 + lane holds W[16 * rt + lane % 16][32 * kk + 8 * (lane / 16) + 0..7],
// so each wave's operand loads are contiguous.  Done by extra workgroups at
// the end of the summary launch, one 16-byte unit per thread, so they start on
// the compute units the first summary workgroups leave and finish before the
// last ones (placed first, they would hold compute units that summary
// workgroups wait for).
struct WConv {
    int32_t M, NK, nchunks;   // NK = Jpad / 32; nchunks = Ipad * Jpad / 8; 0 = none
    int32_t first_wg, nconv;  // workgroups [first_wg, first_wg + nconv) of the launch convert
    uint16_t* wbt;            // if not null, W^T is converted to this buffer as well
    int32_t causal;           // nonzero: keep only W[i][j] with j < i (earlier blocks; in W^T, later ones)
    int32_t TP;               // token parts: column j' of the operand is W[i][j' / TP] (j' < M TP)
    int32_t NKt, nchunks_t;   // W^T (no token parts): NKt = roundup(M, 32) / 32, its 16-byte units
    int32_t WD, WM;           // causal sub-chunks: entry (i, j) is W[i / WD][j / WD], W is WM x WM
    int32_t RD;               // k-slots per source record: column j' is record j' / RD; with RD = 2
                              // the even slot takes bf16(w), the odd one bf16(w - bf16(w))
};

__device__ __forceinline__ void convert_w(const float* __restrict__ W, uint16_t* __restrict__ Wb,
                                          const WConv& wc) {
    const int nthr = wc.nconv * blockDim.x;
    const int total = wc.nchunks + (wc.wbt ? wc.nchunks_t : 0);
    for (int c0 = (blockIdx.x - wc.first_wg) * blockDim.x + threadIdx.x; c0 < total; c0 += nthr) {
        const bool tr = c0 >= wc.nchunks;   // the chunks of W^T follow those of W
        const int c = tr ? c0 - wc.nchunks : c0;
        const int lane = c & 63, rk = c >> 6;
        const int nk = tr ? wc.NKt : wc.NK;
        const int rt = rk / nk, kk = rk - rt * nk;
        const int i = 16 * rt + (lane & 15), j0 = 32 * kk + 8 * (lane >> 4);
        float x[8];
        if (tr) {
            // W^T; causal: later blocks only (source j0 + s > i)
#pragma unroll
            for (int s = 0; s < 8; ++s)
                x[s] = (i < wc.M && j0 + s < wc.M && (!wc.causal || j0 + s > i)) ? W[(size_t)(j0 + s) * wc.M + i] : 0.f;
        } else if (wc.TP > 1 || wc.WD > 1 || wc.RD > 1) {
            // token parts: source record r = j TP + t holds part t of block j;
            // causal sub-chunks: row and column indices are sub-chunks, WD per block of W;
            // RD k-slots per record: slot j' reads record j' / RD
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int jp = j0 + s, jr = jp / wc.RD;
                float w = (i < wc.M && jr < wc.M * wc.TP)
                              ? W[(size_t)(i / wc.WD) * wc.WM + jr / (wc.TP * wc.WD)] : 0.f;
                if (wc.causal && jr / wc.TP >= i) w = 0.f;   // earlier blocks only
                if (wc.RD > 1) {
                    const float hi = bf_lo(pack_bf16(w, 0.f));
                    w = (jp % wc.RD == 0) ? hi : w - hi;
                }
                x[s] = w;
            }
        } else if (i < wc.M && (wc.M & 7) == 0 && j0 < wc.M) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(W + (size_t)i * wc.M + j0);
            const f32x4 b = *reinterpret_cast<const f32x4*>(W + (size_t)i * wc.M + j0 + 4);
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) x[s] = (i < wc.M && j0 + s < wc.M) ? W[(size_t)i * wc.M + j0 + s] : 0.f;
        }
        if (wc.causal && !tr && wc.TP == 1 && wc.WD == 1 && wc.RD == 1) {
#pragma unroll
            for (int s = 0; s < 8; ++s) x[s] = j0 + s < i ? x[s] : 0.f;
        }
        *reinterpret_cast<u32x4*>((tr ? wc.wbt : Wb) + (size_t)c * 8) =
            u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
    }
}

// =====================================================================
// mixing:  C[col'][i] = sum_j [S|z]_j[col'] W[i][j]  per (b, h).
// Workgroup of 8 waves = CPW column tiles (64 record elements col' each) x
// all query blocks i.  The A operand (records of the CPW tiles, up to 256
// source blocks per pass) is staged once in LDS, already packed as MFMA
// operands; wave (c, it, th) computes 64 col' x 32 i (i = it*64 + 32*th + ..)
// with all of its W operands (bf16, padded and laid out in operand order by
// the summary kernel's extra workgroups) loaded from L2 around the staging.
// Lane (li, gq): A rows col' = 4*li + r, B column i = 16*t + li.
// Mixed S tiles leave through LDS so that every store writes whole 128-byte
// record rows; mixed z (fp32) is stored directly.
// =====================================================================
struct MixGeo {
    int32_t CT, IT, CPW, CTG, Jpad;   // column tiles, i tiles, column tiles per WG, WG per bh, padded j
    FastDiv div_CTG;
};

constexpr int MIX_OROW = 72;                           // output staging row: 64 bf16 + 8 padding
constexpr int MIX_LDS_UNITS = 8 * 32 * MIX_OROW / 8;   // 16-byte LDS units of one mixing workgroup

// Four consecutive record elements as two bf16 pairs (fp32 records round to
// nearest even).
__device__ __forceinline__ u32x2 load4_bf16(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ u32x2 load4_bf16(const float* p) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
    return u32x2{pack_bf16(x.x, x.y), pack_bf16(x.z, x.w)};
}

// One mixing work unit wg = (b*h, group of CPW column tiles) for a workgroup
// of 512 threads.  sA is the workgroup's LDS area of MIX_LDS_UNITS units: A
// operands [tile c][r][kk][lane] (cpw * nkp <= 8: 32 KB), reused for the
// output transpose (8 waves x 32 rows x MIX_OROW bf16 = 36 KB).  Records are
// bf16 or fp32 (rounded to bf16 as they are staged).
template <int D, typename RecT>
__device__ __forceinline__ void mix_tile_bf16(uint32_t wg, const RecT* __restrict__ SZ,
                                              const uint16_t* __restrict__ Wb, uint16_t* __restrict__ St,
                                              float* __restrict__ Zt, const Geo& g, const MixGeo& mg,
                                              u32x4* __restrict__ sA) {
    constexpr int REC = D * D + D;
    constexpr int KSP = 8;          // k-steps (32 source blocks) per staging pass
    constexpr int OROW = MIX_OROW;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, gq = lane >> 4;
    const uint32_t bh = fdiv(wg, mg.div_CTG);
    const int ctg = (int)(wg - bh * mg.div_CTG.d);
    const int M = g.M;                 // query blocks
    const int NR = g.M * g.TP;         // source records (partial records of TP parts)
    const int MS = NR * g.RD;          // k-slots: each record feeds RD of them
    const int NK = (MS + 31) >> 5;
    const int cpw = mg.CPW;
    const int itr = mg.IT < 4 ? mg.IT : 4;   // i tiles per round
    const RecT* base = SZ + (size_t)bh * NR * REC;
    const int th = wave & 1, w2 = wave >> 1;
    const int wc = w2 / itr, wit = w2 % itr;
    const int ct = ctg * cpw + wc;
    const bool wave_ok = (w2 < cpw * itr) && (ct < mg.CT);
    const int cp0 = ct * 64;   // first record element of this wave's column tile

    for (int iround = 0; iround * 4 < mg.IT; ++iround) {
        const int it = iround * 4 + wit;
        const bool active = wave_ok && it < mg.IT;
        const int itc = it < mg.IT ? it : mg.IT - 1;   // inactive waves load a valid tile too
        f32x4 acc[4][2];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int k0 = 0; k0 < NK; k0 += KSP) {
            const int nkp = min(KSP, NK - k0);
            // Workgroups visit the pass's k-steps in rotated order (step kr(kk)
            // at position kk), so that they do not all request the same W lines
            // from L2 at the same moment.
            const int rot = (int)(wg % (uint32_t)nkp);
            auto kr = [&](int kk) {
                const int x = kk + rot;
                return kk >= nkp ? nkp - 1 : (x >= nkp ? x - nkp : x);
            };
            // W operands (B) of this pass: the first half before the staging of A,
            // the second half after it; positions past nkp reload a valid step.
            u32x4 bw[KSP][2];
            auto load_w = [&](int kk) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    bw[kk][t] = *reinterpret_cast<const u32x4*>(
                        Wb + ((size_t)((itc * 4 + 2 * th + t) * NK + k0 + kr(kk)) * 64 + lane) * 8);
            };
#pragma unroll
            for (int kk = 0; kk < KSP / 2; ++kk) load_w(kk);
            __syncthreads();
            // ---- stage A: unit (tile c, li', j-group of 8) -> 4 packed operands.
            // cpw * nkp <= 8, so there are at most 512 units: one per thread.
            {
                const int units = cpw * 16 * 4 * nkp;
                const int u = tid;
                const int lip = u & 15;
                const int jg = (u >> 4) % (4 * nkp);
                const int c = (u >> 4) / (4 * nkp);
                const int colp = (ctg * cpw + c) * 64 + 4 * lip;
                const bool ok = u < units && colp < REC && (ctg * cpw + c) < mg.CT;
                const int colc = ok ? colp : 0;
                u32x2 raw[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    // Clamped address, then a mask: the load stays unconditional.
                    const int jj = (k0 + (jg >> 2)) * 32 + (jg & 3) * 8 + s;
                    const u32x2 t = load4_bf16(base + (size_t)((jj < MS ? jj : MS - 1) / g.RD) * REC + colc);
                    const uint32_t m = (ok && jj < MS) ? 0xffffffffu : 0u;
                    raw[s] = u32x2{t.x & m, t.y & m};
                }
                if (u < units) {
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
                    for (int r = 0; r < 4; ++r) sA[((c * 4 + r) * nkp + kk) * 64 + lanep] = op[r];
                }
            }
#pragma unroll
            for (int kk = KSP / 2; kk < KSP; ++kk) load_w(kk);
            __syncthreads();
            if (active) {
#pragma unroll
                for (int kk = 0; kk < KSP; ++kk) {
                    if (kk >= nkp) break;
                    u32x4 a[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) a[r] = sA[((wc * 4 + r) * nkp + kr(kk)) * 64 + lane];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int t = 0; t < 2; ++t) acc[r][t] = mfma_bf16(a[r], bw[kk][t], acc[r][t]);
                }
            }
        }

        // ---- output.  Lane holds C[col' = cp0 + 16*gq + 4*v + r][i = it*64 + 32*th + 16*t + li].
        const bool s_tile = active && cp0 < D * D;
        uint16_t* stage = reinterpret_cast<uint16_t*>(sA) + wave * (32 * OROW);
        __syncthreads();   // every wave is done with the A operands
        if (s_tile) {
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
        }
        __syncthreads();
        if (s_tile) {
            // 32 rows of 128 bytes: 8 lanes per row, 8 rows per instruction.
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int rl = 8 * k + (lane >> 3), chunk = lane & 7;
                const int i = it * 64 + 32 * th + rl;
                const u32x4 x = *reinterpret_cast<const u32x4*>(stage + rl * OROW + chunk * 8);
                if (i < M) *reinterpret_cast<u32x4*>(St + ((size_t)bh * M + i) * (D * D) + cp0 + chunk * 8) = x;
            }
        } else if (active && cp0 + 16 * gq < REC) {
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
        __syncthreads();   // the staging area is reused by the next round
    }
}

// The apply's A operands: St_i^T row tiles and zt_i's high and low words.
// ApplyA holds them in the wave's registers; ApplyL reads them from LDS
// operand words laid out [RT][KS][lane], then zt's high [KS][lane] and low
// [KS][lane] words (one 16-byte word per lane and operand: lane-linear,
// conflict-free reads).
template <int D>
struct ApplyA {
    static constexpr int RT = D / 16, KS = D / 32;
    static constexpr bool kShared = false;   // per wave: no workgroup barrier in its preparation
    u32x4 a[RT][KS];
    u32x4 zhi[KS], zlo[KS];
    __device__ __forceinline__ u32x4 op(int r, int kk, int) const { return a[r][kk]; }
    __device__ __forceinline__ u32x4 hi(int kk, int) const { return zhi[kk]; }
    __device__ __forceinline__ u32x4 lo(int kk, int) const { return zlo[kk]; }
};
template <int D>
struct ApplyL {
    static constexpr int RT = D / 16, KS = D / 32, WORDS = (RT + 2) * KS * 64;
    static constexpr bool kShared = true;    // staged by the workgroup: every wave reaches its barrier
    const u32x4* w;
    __device__ __forceinline__ u32x4 op(int r, int kk, int lane) const { return w[(r * KS + kk) * 64 + lane]; }
    __device__ __forceinline__ u32x4 hi(int kk, int lane) const { return w[(RT * KS + kk) * 64 + lane]; }
    __device__ __forceinline__ u32x4 lo(int kk, int lane) const { return w[((RT + 1) * KS + kk) * 64 + lane]; }
};

// zt (8 fp32 values of one k-slot group) -> hi/lo bf16 operand words.
__device__ __forceinline__ void split_zt(const float* z, u32x4& hi, u32x4& lo) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t h = pack_bf16(z[2 * w], z[2 * w + 1]);
        hi[w] = h;
        lo[w] = pack_bf16(z[2 * w] - bf_lo(h), z[2 * w + 1] - bf_hi(h));
    }
}

// prep_load(A) issues the loads of the block's A operands (and keeps zt raw);
// prep_finish(A) turns raw zt into operands.  Both run after the first batch of
// Q loads has been issued, so the latencies of St, zt and Q overlap.
typedef short s16x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x16_bf16: lane l supplies row (or column) l % 16 and
// k = 4 * (l / 16) + 0..3; output as for the 16x16x32 form.
__device__ __forceinline__ f32x4 mfma_k16(const u32x2& a, const u32x2& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                     c, 0, 0, 0);
}

__device__ __forceinline__ float phi_grad(float x) { return x > 0.f ? 1.f : __expf(x); }

// Unpack 8 channels (one 16-byte load) into fp32.
__device__ __forceinline__ void unpack8(const u32x4& w, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf_lo(w[k]);
        x[2 * k + 1] = bf_hi(w[k]);
    }
}

// A 16-token x D tile whose lane (t, gq) holds channels 4*RT*gq .. +4*RT-1 of
// token t as packed bf16 pairs leaves through the wave's LDS slice and is
// written as whole token rows by buffer stores; a token past the block's end
// gets an out-of-range offset, so the hardware drops its write.
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* sout, const uint32_t* wv, int lane, int off, bool ok,
                                           __amdgpu_buffer_rsrc_t rsrc, int olane) {
    constexpr int RT = D / 16, OSTR = D + 8, CPR = D / 8;
    const int t = lane & 15, gq = lane >> 4;
    uint16_t* srow = sout + t * OSTR + 4 * RT * gq;
#pragma unroll
    for (int u = 0; u < RT / 2; ++u)
        *reinterpret_cast<u32x4*>(srow + 8 * u) = u32x4{wv[4 * u], wv[4 * u + 1], wv[4 * u + 2], wv[4 * u + 3]};
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
        const int tt = k * (64 / CPR) + lane / CPR, chunk = lane % CPR;
        const int offk = __shfl(off, tt, 64);
        const int okk = __shfl((int)ok, tt, 64);
        const u32x4 x = *reinterpret_cast<const u32x4*>(sout + tt * OSTR + chunk * 8);
        const uint32_t bo = okk ? (uint32_t)(offk * 2 + olane + chunk * 16) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b128(x, rsrc, bo, 0, 0);
    }
}

}  // namespace
}  // namespace mhla
