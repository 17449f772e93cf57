// common.h -- shared device helpers and problem geometry for the libmhla kernels.
//
// Geometry follows the method's token-dimension partition (MHLA,
// arXiv 2601.07832; paperlayer.ai summary, section 4 "Architecture"): the
// token grid (up to 3 axes, slowest first, raster order) is tiled by
// non-overlapping blocks; blocks are numbered row-major over the block grid
// and the tokens of a block are visited row-major inside it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhla {

// ---------------------------------------------------------------- fast division
// Quotient n / d for 0 <= n < 2^31 and d >= 1 with one multiply-high, using
// the round-up multiplier of Granlund & Montgomery ("Division by invariant
// integers using multiplication", PLDI 1994): with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, n / d = (mulhi(n, m) + n) >> s.
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.s = s;
    f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (__umulhi(n, f.m) + n) >> f.s;
}

// ---------------------------------------------------------------- geometry
struct Geo {
    int32_t B, H, D, N, M, T;
    int32_t BH;           // B * H
    int32_t E1, E2;       // grid extents of the two fastest axes
    int32_t bk0, bk1, bk2;  // block extents (slowest first)
    FastDiv div_bk2, div_bk12;   // in-block position -> coordinates
    FastDiv div_nb2, div_nb12;   // block id -> block coordinates
    FastDiv div_M, div_H;
    // Head grouping of the bf16 kernels: a workgroup covers G consecutive heads
    // of one (b, block), so its waves read whole runs of each token's channels.
    int32_t G, HG;        // heads per workgroup, head groups per (b, block)
    FastDiv div_HG;
    // Token parts (bf16 3-kernel forward with few blocks): the summary kernel
    // sums each block's tokens in TP contiguous runs into TP partial records
    // (record (b h, j TP + t)), which the mixing kernel contracts as M TP source
    // records; the apply kernel splits each block's tokens into AP runs.
    int32_t TP, AP;
    FastDiv div_TP, div_AP;
    // W's index for this geometry's block i is i / WD (WD > 1: the bf16 causal
    // form run on sub-chunks, WD of them per chunk of the caller's problem);
    // WM is W's dimension (the caller's block count).
    int32_t WD, WM;
    // Every source record feeds RD consecutive k-slots of the mixing product
    // (RD = 2: the slots take W's bf16 high and low parts, so the mixture
    // sees W to about 16 significant bits; the bf16 causal form uses it).
    int32_t RD;
    float eps;
};

// Workgroup index -> (b, block, head group) for head-grouped launches:
// blockIdx = (b * M + j) * HG + hg.
struct WgCoord {
    int b, j, hg;
};
__device__ __forceinline__ WgCoord wg_coord(const Geo& g, uint32_t wg) {
    WgCoord c;
    const uint32_t bj = fdiv(wg, g.div_HG);
    c.hg = (int)(wg - bj * g.div_HG.d);
    c.b = (int)fdiv(bj, g.div_M);
    c.j = (int)(bj - (uint32_t)c.b * g.div_M.d);
    return c;
}

// Workgroup index -> (b, block, part, head group) for launches that also split
// each block's tokens into parts: blockIdx = ((b * M + j) * parts + t) * HG + hg.
struct WgCoordP {
    int b, j, t, hg;
};
__device__ __forceinline__ WgCoordP wg_coord_parts(const Geo& g, uint32_t wg, const FastDiv& div_parts) {
    WgCoordP c;
    const uint32_t bjt = fdiv(wg, g.div_HG);
    c.hg = (int)(wg - bjt * g.div_HG.d);
    const uint32_t bj = fdiv(bjt, div_parts);
    c.t = (int)(bjt - bj * div_parts.d);
    c.b = (int)fdiv(bj, g.div_M);
    c.j = (int)(bj - (uint32_t)c.b * g.div_M.d);
    return c;
}

// Raster index of the first token of block j.
__device__ __forceinline__ int32_t block_origin(const Geo& g, int32_t j) {
    uint32_t j0 = fdiv((uint32_t)j, g.div_nb12);
    uint32_t r = (uint32_t)j - j0 * g.div_nb12.d;
    uint32_t j1 = fdiv(r, g.div_nb2);
    uint32_t j2 = r - j1 * g.div_nb2.d;
    return (int32_t)(((j0 * g.bk0) * g.E1 + j1 * g.bk1) * g.E2 + j2 * g.bk2);
}

// Raster offset of in-block position p (row-major inside the block).
__device__ __forceinline__ int32_t in_block(const Geo& g, int32_t p) {
    uint32_t p0 = fdiv((uint32_t)p, g.div_bk12);
    uint32_t r = (uint32_t)p - p0 * g.div_bk12.d;
    uint32_t p1 = fdiv(r, g.div_bk2);
    uint32_t p2 = r - p1 * g.div_bk2.d;
    return (int32_t)((p0 * g.E1 + p1) * g.E2 + p2);
}

// ---------------------------------------------------------------- vector types
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 halves of a packed 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> packed bf16 pair (a in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2 p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, p);
}

// Low halves / high halves of two words, packed (first argument -> low half).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// Feature map phi(x) = elu(x) + 1: x + 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float phi_fast(float x) { return x > 0.f ? x + 1.f : __expf(x); }
__device__ __forceinline__ float phi_exact(float x) { return x > 0.f ? x + 1.f : expf(x); }

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// Nonzero weights of one row of W for a workgroup of 256 threads: entries
// [base, base + 256) of the row wr (length M) are scanned, and the nonzero
// ones are written in index order to idx[0..n) / wt[0..n) (LDS) by a wave
// ballot and a prefix count over the four waves; n is returned to every
// thread.  wcnt: 4 ints of LDS.  Ends with a workgroup barrier.
__device__ __forceinline__ int compact_nonzero(const float* __restrict__ wr, int M, int base, int* idx,
                                               float* wt, int* wcnt) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = base + tid;
    const float w = j < M ? wr[j] : 0.f;
    const bool nz = w != 0.f;
    const unsigned long long m = __ballot(nz);
    const int pre = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int off = 0, total = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = wcnt[k];
        off += k < wave ? c : 0;
        total += c;
    }
    if (nz) {
        idx[off + pre] = j;
        wt[off + pre] = w;
    }
    __syncthreads();
    return total;
}

}  // namespace mhla
