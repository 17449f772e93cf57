// mhla_api.cpp -- the C ABI of libmhla: validation, workspace layout and dispatch.
//
// The problem statement (token grid split into non-overlapping blocks, one
// M x M coefficient matrix mixing per-block key-value summaries) follows MHLA,
// arXiv 2601.07832 (paperlayer.ai summary, section 4 "Architecture" and
// "Multi-Head Mixing").  Everything here runs on the host; the kernels live
// in kernels_bf16.hip and kernels_f32.hip.
#include <mhla.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Shape {
    int64_t B, H, D, N, M, T;
    int64_t g[3], b[3], nb[3];   // padded to 3 axes, slowest first
    int dtype;
    size_t esz;                  // bytes per element of q/k/v/out and of intermediates
};

mhla_status check(const mhla_grid* grid, const mhla_block* block, Shape* s) {
    if (!grid || !block) return MHLA_ERR_INVALID_ARG;
    if (grid->dtype != MHLA_F32 && grid->dtype != MHLA_BF16) return MHLA_ERR_UNSUPPORTED;
    if (grid->head_dim != 32 && grid->head_dim != 64 && grid->head_dim != 128) return MHLA_ERR_UNSUPPORTED;
    if (grid->batch < 0 || grid->heads < 0) return MHLA_ERR_INVALID_ARG;
    if (grid->ndim != 2 && grid->ndim != 3) return MHLA_ERR_INVALID_ARG;
    if (!std::isfinite(grid->eps) || grid->eps < 0.f) return MHLA_ERR_INVALID_ARG;
    const int off = 3 - grid->ndim;
    for (int a = 0; a < 3; ++a) { s->g[a] = 1; s->b[a] = 1; }
    for (int a = 0; a < grid->ndim; ++a) {
        if (grid->extent[a] <= 0 || block->extent[a] <= 0) return MHLA_ERR_INVALID_ARG;
        if (grid->extent[a] % block->extent[a] != 0) return MHLA_ERR_INVALID_ARG;
        s->g[off + a] = grid->extent[a];
        s->b[off + a] = block->extent[a];
    }
    s->N = s->g[0] * s->g[1] * s->g[2];
    s->T = s->b[0] * s->b[1] * s->b[2];
    for (int a = 0; a < 3; ++a) s->nb[a] = s->g[a] / s->b[a];
    s->M = s->nb[0] * s->nb[1] * s->nb[2];
    s->B = grid->batch;
    s->H = grid->heads;
    s->D = grid->head_dim;
    s->dtype = grid->dtype;
    s->esz = grid->dtype == MHLA_F32 ? 4 : 2;
    // Kernels index with 32-bit offsets: every tensor (and every workspace
    // region, in elements) must stay below 2^31.
    const double lim = 2147483648.0;
    if ((double)s->B * (double)s->N * (double)s->H * (double)s->D >= lim) return MHLA_ERR_UNSUPPORTED;
    if ((double)s->B * (double)s->H * (double)s->M * (double)(s->D * s->D + s->D) >= lim)
        return MHLA_ERR_UNSUPPORTED;
    // W and dW hold M * M values, counted in 32-bit integers by the kernels.
    if ((double)s->M * (double)s->M >= lim) return MHLA_ERR_UNSUPPORTED;
    // One batch item's tensor must also fit a 2^31-byte buffer range.
    if ((double)s->N * (double)s->H * (double)s->D * (double)s->esz >= lim) return MHLA_ERR_UNSUPPORTED;
    return MHLA_OK;
}

// Blocks are single runs of raster indices: some axis is split while every
// faster axis is covered whole and every slower axis has block extent 1.
bool chunks_contiguous(const Shape& s) {
    for (int a = 0; a < 3; ++a) {
        bool ok = true;
        for (int x = 0; x < a; ++x) ok = ok && s.b[x] == 1;
        for (int x = a + 1; x < 3; ++x) ok = ok && s.b[x] == s.g[x];
        if (ok) return true;
    }
    return false;
}

bool causal_supported(const Shape& s) {
    return chunks_contiguous(s);   // bf16 or fp32, head_dim 32, 64 or 128
}

// Token parts of the bf16 3-kernel forward when the problem has few
// (b, block, head) tasks: each part is a contiguous run of at least 64 of a
// block's tokens, doubled until about 1536 tasks (six per compute unit) or
// the limits (the mixing kernel contracts at most 256 source records, so
// M * summary parts <= 256).
int summary_parts(const Shape& s) {
    if (s.dtype != MHLA_BF16) return 1;
    int64_t p = 1;
    while (s.B * s.M * s.H * p < 1536 && s.M * p * 2 <= 256 && p * 2 * 64 <= s.T) p *= 2;
    return (int)p;
}
// The bf16 causal form on long chunks runs on sub-chunks: a chunk (a run of
// raster order) is split along its slowest axis of extent > 1 into cp runs of
// at least 256 tokens (at most 256 sub-chunks in all).  The causal form over
// chunks with W equals the causal form over sub-chunks with coefficient
// W[a / cp][b / cp] between sub-chunks a and b: every pair of tokens keeps
// the weight of its chunks and the mask m <= n.
int causal_split_axis(const Shape& s) {
    for (int a = 0; a < 3; ++a)
        if (s.b[a] > 1) return a;
    return -1;
}
int causal_parts(const Shape& s) {
    if (s.dtype != MHLA_BF16 || !chunks_contiguous(s)) return 1;
    const int a = causal_split_axis(s);
    if (a < 0) return 1;
    int64_t cp = 1;
    while (s.b[a] % (cp * 2) == 0 && s.T / (cp * 2) >= 256 && s.M * cp * 2 <= 256) cp *= 2;
    return (int)cp;
}
Shape subchunk_shape(const Shape& s, int cp) {
    Shape t = s;
    const int a = causal_split_axis(s);
    t.b[a] = s.b[a] / cp;
    t.nb[a] = s.nb[a] * cp;
    t.M = s.M * cp;
    t.T = s.T / cp;
    return t;
}

int apply_parts(const Shape& s) {
    if (s.dtype != MHLA_BF16) return 1;
    int64_t p = 1;
    while (s.B * s.M * s.H * p < 1536 && p * 2 * 64 <= s.T) p *= 2;
    return (int)p;
}

// The 3-kernel forward's token parts in its geometry.
void set_token_parts(mhla::Geo& g, const Shape& s) {
    g.TP = summary_parts(s);
    g.AP = apply_parts(s);
    g.div_TP = mhla::make_fastdiv((uint32_t)g.TP);
    g.div_AP = mhla::make_fastdiv((uint32_t)g.AP);
}

// k-slots per summary record in the bf16 causal form's mixing: W's bf16
// high and low parts.
constexpr int kCausalWParts = 2;

struct Layout {
    size_t sz, st, zt, wb, total;   // byte offsets of the regions, total size
};

Layout layout(const Shape& s) {
    const size_t recs = (size_t)(s.B * s.H * s.M);
    const int tp = summary_parts(s), cp = causal_parts(s);
    const size_t r0 = recs * (size_t)(tp > cp ? tp : cp);   // summary records (parts or sub-chunks)
    const size_t r12 = recs * (size_t)cp;                     // mixed records (sub-chunks)
    Layout L;
    L.sz = 0;
    L.st = align_up(r0 * (size_t)(s.D * s.D + s.D) * s.esz);
    L.zt = L.st + align_up(r12 * (size_t)(s.D * s.D) * s.esz);
    L.wb = L.zt + align_up(r12 * (size_t)s.D * 4);
    // bf16 problems: W converted to bf16, rows padded to a multiple of 64 and
    // columns to a multiple of 32 (the mixing kernel's tile sizes).
    // columns: one per k-slot of the mixing product (token parts, or the causal
    // form's sub-chunks with W's high and low parts)
    const int64_t kslots = chunks_contiguous(s) ? (int64_t)cp * kCausalWParts : cp;
    const size_t wb = s.dtype == MHLA_BF16
                          ? (size_t)((s.M * cp + 63) / 64 * 64) *
                                (size_t)((s.M * (tp > kslots ? tp : kslots) + 31) / 32 * 32) * 2
                          : 0;
    L.total = L.wb + align_up(wb);
    return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Stream-ordered workspace allocation of the entry points that allocate.
// MHLA_FAIL_ALLOC=1 in the environment makes it fail without calling HIP (a
// fault-injection hook for testing the error path: the call then returns
// MHLA_ERR_ALLOC and enqueues nothing).
mhla_status alloc_workspace(void** ws, size_t bytes, hipStream_t stream) {
    const char* f = std::getenv("MHLA_FAIL_ALLOC");
    if (f && f[0] == '1' && f[1] == 0) return MHLA_ERR_ALLOC;
    if (hipMallocAsync(ws, bytes, stream) != hipSuccess || !*ws) {
        (void)hipGetLastError();
        return MHLA_ERR_ALLOC;
    }
    return MHLA_OK;
}

int env_int(const char* name, int dflt) {
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    return std::atoi(v);
}

mhla::Tuning choose_tuning(const Shape& s) {
    mhla::Tuning t;
    // Waves per block: enough token groups per wave to amortise the per-wave
    // setup, enough waves to keep loads in flight.
    t.summary_waves = 1;
    t.summary_pf = 1;
    // d = 128: every wave of a block holds all of St_i (32 KB of operands),
    // so two waves per head load it half as often as four (video-16x64x64
    // apply 118 -> 100 us; one wave per head 104 us).
    t.apply_waves = s.T >= 128 ? (s.D == 128 ? 2 : 4) : 1;
    // d = 128 keeps 32 operand registers per row tile live; with 4 waves per
    // block, one group in flight per wave is enough.
    t.apply_pf = (s.D == 128 || s.T >= 128) ? 1 : 2;
    // Overrides for launch-shape sweeps.
    const int sw = env_int("MHLA_SUMMARY_WAVES", 0), aw = env_int("MHLA_APPLY_WAVES", 0);
    const int sp = env_int("MHLA_SUMMARY_PF", 0), ap = env_int("MHLA_APPLY_PF", 0);
    if (sw == 1 || sw == 2 || sw == 4) t.summary_waves = sw;
    if (aw == 1 || aw == 2 || aw == 4) t.apply_waves = aw;
    if (sp == 1 || sp == 2) t.summary_pf = sp;
    if (ap == 1 || ap == 2 || ap == 4) t.apply_pf = ap;
    t.pair_heads = env_int("MHLA_PAIR_HEADS", 1) != 0;
    // head_dim 128: the summary kernel whose four waves per head share K/V
    // operands through LDS, one head per workgroup (video-16x64x64 summary
    // 136 -> 103 us; two heads per workgroup 122 us).
    t.d128_shared = env_int("MHLA_D128_SHARED", 1);
    if (t.d128_shared < 0 || t.d128_shared > 2) t.d128_shared = 1;
    t.apply_maxw = 8;
    // Apply operands staged once per head in LDS (d <= 64) when several waves
    // share a head: dit-s2-256x256 apply 25.9 -> 23.9 us, sana-128x128 (d = 32)
    // 75.1 -> 68.2 us; with one wave per head at d = 64 the 12 KB of operand
    // words per wave leave room for too few waves (dit-s2-64x64 53 -> 78 us).
    const int lds_default = s.D == 32 || (s.D == 64 && t.apply_waves >= 2);
    t.apply_lds = env_int("MHLA_APPLY_LDS", lds_default) != 0;
    t.bwdq_heads = env_int("MHLA_BWDQ_HEADS", 0);
    if (t.bwdq_heads < 0 || t.bwdq_heads > 4) t.bwdq_heads = 0;
    const int am = env_int("MHLA_APPLY_MAXW", 0);
    if (am == 4 || am == 8 || (am == 2 && t.apply_waves <= 2)) t.apply_maxw = am;
    // Non-temporal loads: faster for the summary kernel's k, v stream.  On
    // the apply kernel's q stream they cost the apply about 1 us at d <= 64
    // but the following summary launch runs 2-5 us faster, so a repeated
    // forward gains; at d = 128 the apply loses 6 us (measured on MI355X).
    t.nt_loads = env_int("MHLA_NT_LOADS", 1) != 0;
    t.nt_apply = env_int("MHLA_NT_APPLY", s.D <= 64 ? 1 : 0) != 0;
    // Mixing kernel: one workgroup per (pair, column tile, query-block tile)
    // by default; MHLA_MIX selects another for sweeps (flags of
    // mhla_forward_ex select one per call).
    // With at most 64 query blocks the per-tile workgroups are small (8 KB
    // of W and 8 KB of records each) and the persistent kernel, which loads W
    // once per compute unit, is faster (dit-s2-64x64 mixing 38.2 -> 33.7 us);
    // at head_dim 128 (258 column tiles per pair, each workgroup of the split
    // kernel reading 64 KB of W for 32 KB of records) too: video-16x64x64
    // step 254.4-255.5 -> 251.5-252.5 us over three alternating runs.
    // At head_dim 32 with many pairs (17 column tiles each; sana-128x128: 140
    // pairs, 4760 split workgroups) the persistent kernel wins as well:
    // mixing 38.0 -> 37.3 us, step 183.8 -> 180.7 us over two alternating runs.
    const bool many_d32 = s.D == 32 && s.M <= 256 && s.B * s.H >= 64;
    const int mix_default = (s.M <= 64 || s.D == 128 || many_d32) ? 1 : 2;
    t.mix_kind = env_int("MHLA_MIX", mix_default);
    if (t.mix_kind < 0 || t.mix_kind > 2) t.mix_kind = mix_default;
    t.mix_rows = env_int("MHLA_MIX_ROWS", 0);
    t.bwd_fuse = env_int("MHLA_BWD_FUSE", 1) != 0;
    // Non-temporal stores of the mixed summaries: mixing 12.7 -> 11.7 us at
    // dit-s2-256x256 (T = 256, the apply unchanged), video-16x64x64 307 us
    // per step against 308; at T = 64 the apply waits longer for St (one
    // wave per block and head reads all of St_i for 64 tokens): dit-s2-64x64
    // 153 -> 159 us, sana-128x128 201 -> 216 us.  Non-temporal summary
    // loads: 0.4 us slower at dit-s2-256x256.
    t.nt_mix = env_int("MHLA_NT_MIX", s.T >= 128 ? 2 : 0) & 3;
    t.num_cus = 256;
    return t;
}

mhla::Geo make_geo(const Shape& s, float eps) {
    mhla::Geo g;
    g.B = (int32_t)s.B; g.H = (int32_t)s.H; g.D = (int32_t)s.D;
    g.N = (int32_t)s.N; g.M = (int32_t)s.M; g.T = (int32_t)s.T;
    g.BH = (int32_t)(s.B * s.H);
    g.E1 = (int32_t)s.g[1]; g.E2 = (int32_t)s.g[2];
    g.bk0 = (int32_t)s.b[0]; g.bk1 = (int32_t)s.b[1]; g.bk2 = (int32_t)s.b[2];
    g.div_bk2 = mhla::make_fastdiv((uint32_t)s.b[2]);
    g.div_bk12 = mhla::make_fastdiv((uint32_t)(s.b[1] * s.b[2]));
    g.div_nb2 = mhla::make_fastdiv((uint32_t)s.nb[2]);
    g.div_nb12 = mhla::make_fastdiv((uint32_t)(s.nb[1] * s.nb[2]));
    g.div_M = mhla::make_fastdiv((uint32_t)s.M);
    g.div_H = mhla::make_fastdiv((uint32_t)(s.H > 0 ? s.H : 1));
    g.G = 1;
    g.HG = g.H;
    g.div_HG = mhla::make_fastdiv((uint32_t)(s.H > 0 ? s.H : 1));
    g.TP = g.AP = 1;
    g.div_TP = g.div_AP = mhla::make_fastdiv(1u);
    g.WD = 1;
    g.WM = g.M;
    g.RD = 1;
    g.eps = eps;
    return g;
}

// The path argument of mhla_forward_ex: a MHLA_PATH_* value in the low 8 bits
// and MHLA_VARIANT_* flags above them.
constexpr int32_t kMixFlags = MHLA_VARIANT_MIX_RESIDENT | MHLA_VARIANT_MIX_TILED | MHLA_VARIANT_MIX_SPLIT;
constexpr int32_t kVariantMask = kMixFlags | MHLA_VARIANT_NO_PAIR_HEADS | MHLA_VARIANT_APPLY_REGS;

bool split_path(int32_t arg, int32_t* path, int32_t* variant) {
    *path = arg & 0xff;
    *variant = arg & ~0xff;
    if (*variant & ~kVariantMask) return false;
    const int32_t mix = *variant & kMixFlags;
    if (mix & (mix - 1)) return false;   // at most one mixing kernel
    return *path == MHLA_PATH_3KERNEL || *path == MHLA_PATH_FUSED || *path == MHLA_PATH_CAUSAL;
}

void apply_variant(mhla::Tuning& t, int32_t variant) {
    if (variant & MHLA_VARIANT_MIX_RESIDENT) t.mix_kind = 1;
    if (variant & MHLA_VARIANT_MIX_TILED) t.mix_kind = 0;
    if (variant & MHLA_VARIANT_MIX_SPLIT) t.mix_kind = 2;
    if (variant & MHLA_VARIANT_NO_PAIR_HEADS) t.pair_heads = 0;
    if (variant & MHLA_VARIANT_APPLY_REGS) t.apply_lds = 0;
}

mhla_status forward_impl(const void* q, const void* k, const void* v, const float* W,
                         const mhla_grid* grid, const mhla_block* block, void* out, void* ws,
                         size_t ws_bytes, bool allow_alloc, int32_t path_arg,
                         const hipEvent_t* events, hipStream_t stream) {
    Shape s;
    mhla_status st = check(grid, block, &s);
    if (st != MHLA_OK) return st;
    int32_t path = 0, variant = 0;
    if (!split_path(path_arg, &path, &variant)) return MHLA_ERR_INVALID_ARG;
    if (path == MHLA_PATH_CAUSAL && !causal_supported(s)) return MHLA_ERR_UNSUPPORTED;
    if (s.B == 0 || s.H == 0) return MHLA_OK;
    if (!q || !k || !v || !W || !out) return MHLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(W) || !aligned16(out))
        return MHLA_ERR_MISALIGNED;
    const size_t tbytes = (size_t)(s.B * s.N * s.H * s.D) * s.esz;
    const size_t wbytes = (size_t)(s.M * s.M) * 4;
    if (overlaps(out, tbytes, q, tbytes) || overlaps(out, tbytes, k, tbytes) ||
        overlaps(out, tbytes, v, tbytes) || overlaps(out, tbytes, W, wbytes))
        return MHLA_ERR_INVALID_ARG;
    const Layout lay = layout(s);
    bool owned = false;
    if (ws) {
        if (ws_bytes < lay.total) return MHLA_ERR_INVALID_ARG;
        if (!aligned16(ws)) return MHLA_ERR_MISALIGNED;
        if (overlaps(ws, lay.total, out, tbytes) || overlaps(ws, lay.total, q, tbytes) ||
            overlaps(ws, lay.total, k, tbytes) || overlaps(ws, lay.total, v, tbytes) ||
            overlaps(ws, lay.total, W, wbytes))
            return MHLA_ERR_INVALID_ARG;
    } else {
        if (!allow_alloc || ws_bytes != 0) return MHLA_ERR_INVALID_ARG;
        const mhla_status as = alloc_workspace(&ws, lay.total, stream);
        if (as != MHLA_OK) return as;
        owned = true;
    }
    mhla::Launch L;
    L.q = q; L.k = k; L.v = v; L.W = W; L.out = out;
    char* base = static_cast<char*>(ws);
    L.sz = base + lay.sz;
    L.st = base + lay.st;
    L.zt = reinterpret_cast<float*>(base + lay.zt);
    L.wb = base + lay.wb;
    L.wbt = nullptr;
    L.g = make_geo(s, grid->eps);
    if (path == MHLA_PATH_3KERNEL) set_token_parts(L.g, s);
    if (path == MHLA_PATH_CAUSAL && s.dtype == MHLA_BF16) {
        const int cp = causal_parts(s);
        if (cp > 1) {
            L.g = make_geo(subchunk_shape(s, cp), grid->eps);
            L.g.WD = cp;
            L.g.WM = (int32_t)s.M;
        }
        // The causal mixtures take W as a bf16 high and low part: signed W can
        // make the partial row sums over earlier blocks cancel, and W rounded
        // to bf16 would then dominate the error.
        L.g.RD = kCausalWParts;
    }
    L.tune = choose_tuning(s);
    apply_variant(L.tune, variant);
    {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            L.tune.num_cus = cus;
        else
            (void)hipGetLastError();
    }
    L.path = path;
    L.summaries_only = 0;
    L.events = events;
    L.stream = stream;
    const hipError_t err = s.dtype == MHLA_BF16 ? mhla::run_bf16(L) : mhla::run_f32(L);
    if (owned) (void)hipFreeAsync(ws, stream);
    return err == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
}

// ---------------------------------------------------------------- backward

struct BwdLayout {
    Layout fwd;                                  // regions of the forward recompute
    size_t dst, ds, dz, wbt, part, dpart, sfold, total;
    int nsplit, q_parts, s_parts;
};

bool bwd_supported(const Shape& s) { return s.dtype == MHLA_BF16 && (s.D == 32 || s.D == 64); }

BwdLayout bwd_layout(const Shape& s) {
    BwdLayout L;
    L.fwd = layout(s);
    const size_t recs = (size_t)(s.B * s.H * s.M);
    const size_t wpad = (size_t)((s.M + 63) / 64 * 64) * (size_t)((s.M + 31) / 32 * 32) * 2;
    L.dst = L.fwd.total;
    L.ds = L.dst + align_up(recs * (size_t)(s.D * s.D + s.D) * 2);
    L.dz = L.ds + align_up(recs * (size_t)(s.D * s.D) * 2);
    L.wbt = L.dz + align_up(recs * (size_t)s.D * 4);
    L.part = L.wbt + align_up(wpad);
    // dW: k-steps of 32 record elements over all (b, h), split so that about
    // 256 workgroups share them.  Where the dW tiles run in one launch with
    // the W^T mixing (129..256 blocks), at least DW_KSTEPS k-steps per
    // workgroup: the mixing workgroups fill the rest of the GPU, and fewer
    // splits mean fewer fp32 partial tiles to write and reduce
    // (dit-s2-256x256: 64 -> 32 splits, the stage 31.0 -> 26.6 us).
    constexpr int64_t DW_KSTEPS = 24;
    const int64_t tiles = ((s.M + 127) / 128) * ((s.M + 127) / 128);
    const int64_t ksteps = s.B * s.H * ((s.D * s.D + s.D) / 32);
    int64_t ns = 256 / tiles;
    if (s.M > 128 && s.M <= 256 && ns > ksteps / DW_KSTEPS) ns = ksteps / DW_KSTEPS;
    if (ns < 1) ns = 1;
    if (ns > ksteps) ns = ksteps > 0 ? ksteps : 1;
    L.nsplit = (int)ns;
    // bwd_query's token parts: fp32 partial records of the mixed summaries' gradients.
    L.q_parts = apply_parts(s);
    L.dpart = L.part + align_up((size_t)ns * (size_t)(s.M * s.M) * 4);
    L.sfold = L.dpart + (L.q_parts > 1 ? align_up(recs * (size_t)L.q_parts * (size_t)(s.D * s.D + s.D) * 4) : 0);
    // The recompute's summaries in token parts, folded into one bf16 record per
    // block for the dW product.
    L.s_parts = summary_parts(s);
    L.total = L.sfold + (L.s_parts > 1 ? align_up(recs * (size_t)(s.D * s.D + s.D) * 2) : 0);
    return L;
}

// The bf16 causal backward on the matrix cores: d = 32 or 64 and chunks that
// the forward runs whole (no sub-chunks).  Its workspace: the backward's
// regions, then per-token 1 / den and dden (fp32 pairs), and the in-chunk dW terms.
bool cbwd_supported(const Shape& s) {
    return s.dtype == MHLA_BF16 && (s.D == 32 || s.D == 64) && chunks_contiguous(s) && causal_parts(s) == 1;
}

struct CbwdLayout {
    BwdLayout b;
    size_t tsc, diag, total;
};

CbwdLayout cbwd_layout(const Shape& s) {
    CbwdLayout L;
    L.b = bwd_layout(s);
    const size_t toks = (size_t)s.B * (size_t)s.N * (size_t)s.H;
    L.tsc = L.b.total;
    L.diag = L.tsc + align_up(toks * 8);
    L.total = L.diag + align_up((size_t)(s.B * s.H * s.M) * 4);
    return L;
}

// The general backward path (fp32 inputs, or head_dim 128): fp32 records.
struct GenLayout {
    size_t s, st, dst, ds, part, dnum, dden, diag, total;
    int nsplit;
};

GenLayout gen_layout(const Shape& s, bool causal = false) {
    GenLayout L;
    const size_t rec = (size_t)(s.B * s.H * s.M) * (size_t)(s.D * s.D + s.D) * 4;
    L.s = 0;
    L.st = align_up(rec);
    L.dst = L.st + align_up(rec);
    L.ds = L.dst + align_up(rec);
    L.part = L.ds + align_up(rec);
    // dW: 32 x 32 tiles, the (b h, 32-value chunk) pairs shared so that about
    // 1024 workgroups run
    const int64_t tiles = ((s.M + 31) / 32) * ((s.M + 31) / 32);
    const int64_t chunks = s.B * s.H * ((s.D * s.D + s.D) / 32);
    int64_t ns = 1024 / tiles;
    if (ns < 1) ns = 1;
    if (ns > chunks) ns = chunks > 0 ? chunks : 1;
    L.nsplit = (int)ns;
    L.total = L.part + align_up((size_t)ns * (size_t)(s.M * s.M) * 4);
    L.dnum = L.dden = L.diag = L.total;
    if (causal) {
        // per-token dnum and dden from the query side, per-chunk diagonal terms of dW
        const size_t toks = (size_t)s.B * (size_t)s.N * (size_t)s.H;
        L.dnum = L.total;
        L.dden = L.dnum + align_up(toks * (size_t)s.D * 4);
        L.diag = L.dden + align_up(toks * 4);
        L.total = L.diag + align_up((size_t)(s.B * s.H * s.M) * 4);
    }
    return L;
}

mhla_status backward_impl(const void* q, const void* k, const void* v, const float* W, const void* dout,
                          const mhla_grid* grid, const mhla_block* block, void* dq, void* dk, void* dv,
                          float* dW, void* ws, size_t ws_bytes, const hipEvent_t* events, hipStream_t stream,
                          bool causal, int32_t variant = 0) {
    Shape s;
    mhla_status st = check(grid, block, &s);
    if (st != MHLA_OK) return st;
    if (variant & ~MHLA_VARIANT_NO_PAIR_HEADS) return MHLA_ERR_INVALID_ARG;
    if (causal && !causal_supported(s)) return MHLA_ERR_UNSUPPORTED;
    const bool fast = !causal && bwd_supported(s);
    const bool cfast = causal && cbwd_supported(s);
    if (!dW) return MHLA_ERR_INVALID_ARG;
    if (!aligned16(dW)) return MHLA_ERR_MISALIGNED;
    const size_t wbytes = (size_t)(s.M * s.M) * 4;
    if (s.B == 0 || s.H == 0) {
        // No pair contributes: dW is zero.
        return mhla::zero_f32(dW, (int)(s.M * s.M), stream) == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
    }
    const void* ins[5] = {q, k, v, W, dout};
    void* outs[4] = {dq, dk, dv, dW};
    for (const void* x : ins)
        if (!x) return MHLA_ERR_INVALID_ARG;
    for (const void* x : outs)
        if (!x) return MHLA_ERR_INVALID_ARG;
    for (const void* x : ins)
        if (!aligned16(x)) return MHLA_ERR_MISALIGNED;
    for (const void* x : outs)
        if (!aligned16(x)) return MHLA_ERR_MISALIGNED;
    const size_t tbytes = (size_t)(s.B * s.N * s.H * s.D) * s.esz;
    const size_t insz[5] = {tbytes, tbytes, tbytes, wbytes, tbytes};
    const size_t outsz[4] = {tbytes, tbytes, tbytes, wbytes};
    for (int a = 0; a < 4; ++a) {
        for (int b = 0; b < 5; ++b)
            if (overlaps(outs[a], outsz[a], ins[b], insz[b])) return MHLA_ERR_INVALID_ARG;
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], outsz[a], outs[b], outsz[b])) return MHLA_ERR_INVALID_ARG;
    }
    const BwdLayout lay = bwd_layout(s);
    const GenLayout glay = gen_layout(s, causal);
    const CbwdLayout clay = cbwd_layout(s);
    const size_t need = fast ? lay.total : (cfast ? clay.total : glay.total);
    bool owned = false;
    if (ws) {
        if (ws_bytes < need) return MHLA_ERR_INVALID_ARG;
        if (!aligned16(ws)) return MHLA_ERR_MISALIGNED;
        for (int b = 0; b < 5; ++b)
            if (overlaps(ws, need, ins[b], insz[b])) return MHLA_ERR_INVALID_ARG;
        for (int a = 0; a < 4; ++a)
            if (overlaps(ws, need, outs[a], outsz[a])) return MHLA_ERR_INVALID_ARG;
    } else {
        if (ws_bytes != 0) return MHLA_ERR_INVALID_ARG;
        const mhla_status as = alloc_workspace(&ws, need, stream);
        if (as != MHLA_OK) return as;
        owned = true;
    }
    char* base = static_cast<char*>(ws);
    if (cfast) {
        mhla::CausalBwdLaunch C;
        mhla::BwdLaunch& B = C.B;
        mhla::Launch& L = B.F;
        L.q = q; L.k = k; L.v = v; L.W = W; L.out = nullptr;
        L.sz = base + clay.b.fwd.sz;
        L.st = base + clay.b.fwd.st;
        L.zt = reinterpret_cast<float*>(base + clay.b.fwd.zt);
        L.wb = base + clay.b.fwd.wb;
        L.wbt = base + clay.b.wbt;
        L.g = make_geo(s, grid->eps);
        L.g.RD = kCausalWParts;   // the causal mixtures take W as bf16 high and low parts
        L.tune = choose_tuning(s);
        apply_variant(L.tune, variant);
        L.path = MHLA_PATH_CAUSAL;
        L.summaries_only = 1;
        L.events = nullptr;
        L.stream = stream;
        {
            int dev = 0, cus = 0;
            if (hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
                L.tune.num_cus = cus;
            else
                (void)hipGetLastError();
        }
        B.dout = dout;
        B.dq = dq; B.dk = dk; B.dv = dv; B.dw = dW;
        B.dst = reinterpret_cast<uint16_t*>(base + clay.b.dst);
        B.ds = reinterpret_cast<uint16_t*>(base + clay.b.ds);
        B.dz = reinterpret_cast<float*>(base + clay.b.dz);
        B.wbt = reinterpret_cast<uint16_t*>(base + clay.b.wbt);
        B.part = reinterpret_cast<float*>(base + clay.b.part);
        B.nsplit = clay.b.nsplit;
        B.kv_parts = 1;
        B.q_parts = 1;
        B.dpart = nullptr;
        B.sfold = nullptr;
        B.events = events;
        C.tsc = reinterpret_cast<float*>(base + clay.tsc);
        C.diag = reinterpret_cast<float*>(base + clay.diag);
        const hipError_t err = mhla::run_causal_bwd_bf16(C);
        if (owned) (void)hipFreeAsync(ws, stream);
        return err == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
    }
    if (!fast) {
        mhla::GenericBwd G;
        G.g = make_geo(s, grid->eps);
        G.bf16 = s.dtype == MHLA_BF16;
        G.q = q; G.k = k; G.v = v; G.dout = dout; G.W = W;
        G.dq = dq; G.dk = dk; G.dv = dv; G.dw = dW;
        G.s = reinterpret_cast<float*>(base + glay.s);
        G.st = reinterpret_cast<float*>(base + glay.st);
        G.dst = reinterpret_cast<float*>(base + glay.dst);
        G.ds = reinterpret_cast<float*>(base + glay.ds);
        G.part = reinterpret_cast<float*>(base + glay.part);
        G.nsplit = glay.nsplit;
        G.causal = causal ? 1 : 0;
        G.dnum = reinterpret_cast<float*>(base + glay.dnum);
        G.dden = reinterpret_cast<float*>(base + glay.dden);
        G.diag = reinterpret_cast<float*>(base + glay.diag);
        G.events = events;
        G.stream = stream;
        const hipError_t err = mhla::run_bwd_generic(G);
        if (owned) (void)hipFreeAsync(ws, stream);
        return err == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
    }
    mhla::BwdLaunch B;
    mhla::Launch& L = B.F;
    L.q = q; L.k = k; L.v = v; L.W = W; L.out = nullptr;
    L.sz = base + lay.fwd.sz;
    L.st = base + lay.fwd.st;
    L.zt = reinterpret_cast<float*>(base + lay.fwd.zt);
    L.wb = base + lay.fwd.wb;
    L.wbt = base + lay.wbt;
    L.g = make_geo(s, grid->eps);
    set_token_parts(L.g, s);   // the recompute's summaries in token parts (regions sized for them)
    L.tune = choose_tuning(s);
    apply_variant(L.tune, variant);
    L.path = MHLA_PATH_3KERNEL;
    L.summaries_only = 1;
    L.events = nullptr;
    L.stream = stream;
    {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            L.tune.num_cus = cus;
        else
            (void)hipGetLastError();
    }
    B.dout = dout;
    B.dq = dq; B.dk = dk; B.dv = dv; B.dw = dW;
    B.dst = reinterpret_cast<uint16_t*>(base + lay.dst);
    B.ds = reinterpret_cast<uint16_t*>(base + lay.ds);
    B.dz = reinterpret_cast<float*>(base + lay.dz);
    B.wbt = reinterpret_cast<uint16_t*>(base + lay.wbt);
    B.part = reinterpret_cast<float*>(base + lay.part);
    B.nsplit = lay.nsplit;
    B.kv_parts = apply_parts(s);
    B.q_parts = lay.q_parts;
    B.dpart = lay.q_parts > 1 ? reinterpret_cast<float*>(base + lay.dpart) : nullptr;
    B.sfold = lay.s_parts > 1 ? reinterpret_cast<uint16_t*>(base + lay.sfold) : nullptr;
    B.events = events;
    const hipError_t err = mhla::run_bwd_bf16(B);
    if (owned) (void)hipFreeAsync(ws, stream);
    return err == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
}

// ---------------------------------------------------------------- layer

struct LayerLayout {
    size_t q, k, v, o, wf, colsum, biasf, mean, rstd, core, total;
};

LayerLayout layer_layout(const Shape& s) {
    const size_t C = (size_t)(s.H * s.D), R = (size_t)(s.B * s.N);
    const size_t act = align_up(R * C * 2);
    LayerLayout L;
    L.q = 0;
    L.k = L.q + act;
    L.v = L.k + act;
    L.o = L.v + act;
    L.wf = L.o + act;
    L.colsum = L.wf + align_up(3 * C * C * 2);
    L.biasf = L.colsum + align_up(3 * C * 4);
    L.mean = L.biasf + align_up(3 * C * 4);
    L.rstd = L.mean + align_up(R * 4);
    L.core = L.rstd + align_up(R * 4);
    L.total = L.core + layout(s).total;
    return L;
}

mhla_status layer_impl(const void* x, const float* W, const mhla_grid* grid, const mhla_block* block,
                       const mhla_layer_params* P, void* y, void* ws, size_t ws_bytes, const hipEvent_t* events,
                       hipStream_t stream) {
    Shape s;
    mhla_status st = check(grid, block, &s);
    if (st != MHLA_OK) return st;
    if (s.dtype != MHLA_BF16) return MHLA_ERR_UNSUPPORTED;
    if (!P) return MHLA_ERR_INVALID_ARG;
    if (P->phi != MHLA_PHI_ELU1 && P->phi != MHLA_PHI_RELU_EPS) return MHLA_ERR_INVALID_ARG;
    if (!std::isfinite(P->phi_eps) || P->phi_eps < 0.f) return MHLA_ERR_INVALID_ARG;
    if (!std::isfinite(P->ln_eps) || P->ln_eps <= 0.f) return MHLA_ERR_INVALID_ARG;
    if ((P->qn_w == nullptr) != (P->kn_w == nullptr)) return MHLA_ERR_INVALID_ARG;
    if (P->qn_w && (!std::isfinite(P->rms_eps) || P->rms_eps <= 0.f)) return MHLA_ERR_INVALID_ARG;
    if (P->lepe_w && grid->ndim != 2) return MHLA_ERR_UNSUPPORTED;
    if (!P->lepe_w && P->lepe_b) return MHLA_ERR_INVALID_ARG;
    const size_t C = (size_t)(s.H * s.D), R = (size_t)(s.B * s.N);
    // the layer's [3C, C] weight and its fold must also stay below 2^31 elements
    if ((double)(3 * C) * (double)C >= 2147483648.0) return MHLA_ERR_UNSUPPORTED;
    if (s.B == 0 || s.H == 0) return MHLA_OK;
    if (!x || !W || !y || !P->ln_w || !P->ln_b || !P->w_qkv || !P->w_out) return MHLA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, W, y, P->ln_w, P->ln_b, P->w_qkv, P->b_qkv, P->qn_w, P->kn_w,
                          P->lepe_w, P->lepe_b, P->w_out, P->b_out};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MHLA_ERR_MISALIGNED;
    const size_t tb = R * C * 2;
    struct Span { const void* p; size_t n; } spans[] = {
        {x, tb}, {W, (size_t)(s.M * s.M) * 4}, {P->ln_w, C * 4}, {P->ln_b, C * 4}, {P->w_qkv, 3 * C * C * 2},
        {P->b_qkv, 3 * C * 4}, {P->qn_w, C * 4}, {P->kn_w, C * 4}, {P->lepe_w, C * 25 * 4}, {P->lepe_b, C * 4},
        {P->w_out, C * C * 2}, {P->b_out, C * 4}};
    for (const Span& sp : spans)
        if (sp.p && overlaps(y, tb, sp.p, sp.n)) return MHLA_ERR_INVALID_ARG;
    const LayerLayout lay = layer_layout(s);
    bool owned = false;
    if (ws) {
        if (ws_bytes < lay.total) return MHLA_ERR_INVALID_ARG;
        if (!aligned16(ws)) return MHLA_ERR_MISALIGNED;
        if (overlaps(ws, lay.total, y, tb)) return MHLA_ERR_INVALID_ARG;
        for (const Span& sp : spans)
            if (sp.p && overlaps(ws, lay.total, sp.p, sp.n)) return MHLA_ERR_INVALID_ARG;
    } else {
        if (ws_bytes != 0) return MHLA_ERR_INVALID_ARG;
        const mhla_status as = alloc_workspace(&ws, lay.total, stream);
        if (as != MHLA_OK) return as;
        owned = true;
    }
    char* base = static_cast<char*>(ws);
    mhla::LayerLaunch L;
    L.x = static_cast<const uint16_t*>(x);
    L.y = static_cast<uint16_t*>(y);
    L.q = reinterpret_cast<uint16_t*>(base + lay.q);
    L.k = reinterpret_cast<uint16_t*>(base + lay.k);
    L.v = reinterpret_cast<uint16_t*>(base + lay.v);
    L.o = reinterpret_cast<uint16_t*>(base + lay.o);
    L.w_qkv = static_cast<const uint16_t*>(P->w_qkv);
    L.wf = reinterpret_cast<uint16_t*>(base + lay.wf);
    L.colsum = reinterpret_cast<float*>(base + lay.colsum);
    L.biasf = reinterpret_cast<float*>(base + lay.biasf);
    L.mean = reinterpret_cast<float*>(base + lay.mean);
    L.rstd = reinterpret_cast<float*>(base + lay.rstd);
    L.ln_w = P->ln_w; L.ln_b = P->ln_b; L.b_qkv = P->b_qkv;
    L.qn_w = P->qn_w; L.kn_w = P->kn_w;
    L.lepe_w = P->lepe_w; L.lepe_b = P->lepe_b;
    L.w_out = static_cast<const uint16_t*>(P->w_out); L.b_out = P->b_out;
    L.ln_eps = P->ln_eps; L.rms_eps = P->rms_eps; L.phi_eps = P->phi_eps;
    L.relu_phi = P->phi == MHLA_PHI_RELU_EPS;
    L.R = (int)R; L.C = (int)C; L.B = (int)s.B;
    L.Y = (int)s.g[1]; L.X = (int)s.g[2];   // 2D grids: the two fastest axes
    mhla::Launch& F = L.core;
    const Layout cl = layout(s);
    char* cb = base + lay.core;
    F.q = L.q; F.k = L.k; F.v = L.v; F.W = W; F.out = L.o;
    F.sz = cb + cl.sz;
    F.st = cb + cl.st;
    F.zt = reinterpret_cast<float*>(cb + cl.zt);
    F.wb = cb + cl.wb;
    F.wbt = nullptr;
    F.g = make_geo(s, grid->eps);
    set_token_parts(F.g, s);   // the core's workspace regions are sized for them
    F.tune = choose_tuning(s);
    {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            F.tune.num_cus = cus;
        else
            (void)hipGetLastError();
    }
    F.path = MHLA_PATH_3KERNEL;
    F.summaries_only = 0;
    F.events = nullptr;
    F.stream = stream;
    L.events = events;
    L.stream = stream;
    const hipError_t err = mhla::run_layer_bf16(L);
    if (owned) (void)hipFreeAsync(ws, stream);
    return err == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
}

// ---- stateful causal execution
size_t stream_state_bytes(const Shape& s, int64_t max_chunks) {
    return (size_t)(s.B * s.H) * (size_t)max_chunks * (size_t)(s.D * s.D + s.D) * 4;
}

// Stream workspace: fp32 problems, the mixtures [B*H][M][d*d + d] fp32;
// bf16 problems, the apply kernel's operands St^T [B*H][M*cp][d*d] bf16, then
// zt [B*H][M*cp][d] fp32, and with long chunks (cp > 1 sub-chunks per chunk,
// as for the one-shot causal form) the chunks' fp32 mixtures [B*H][M][d*d + d]
// and the sub-chunks' fp32 summaries [B*H][M*cp][d*d + d] (256-byte aligned).
struct StreamLayout {
    size_t st, zt, mixed, ssub, total;
    int cp;
};
StreamLayout stream_layout(const Shape& s) {
    const size_t recs = (size_t)(s.B * s.H * s.M), L1 = (size_t)(s.D * s.D + s.D);
    StreamLayout L;
    L.cp = s.dtype == MHLA_BF16 ? causal_parts(s) : 1;
    const size_t sub = recs * (size_t)L.cp;
    L.st = 0;
    L.zt = align_up(sub * (size_t)(s.D * s.D) * 2);
    L.mixed = L.zt + align_up(sub * (size_t)s.D * 4);
    L.ssub = L.mixed + align_up(recs * L1 * 4);
    if (s.dtype != MHLA_BF16) L.total = recs * L1 * 4;
    else if (L.cp == 1) L.total = L.mixed;
    else L.total = L.ssub + align_up(sub * L1 * 4);
    return L;
}
size_t stream_ws_bytes(const Shape& s) { return stream_layout(s).total; }

mhla_status stream_impl(const void* q, const void* k, const void* v, const float* W, int32_t w_dim,
                        const mhla_grid* grid, const mhla_block* block, int32_t n_past, float* state,
                        int32_t max_chunks, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    Shape s;
    mhla_status st = check(grid, block, &s);
    if (st != MHLA_OK) return st;
    if (!chunks_contiguous(s)) return MHLA_ERR_UNSUPPORTED;
    if (n_past < 0 || max_chunks <= 0 || w_dim <= 0) return MHLA_ERR_INVALID_ARG;
    if ((int64_t)n_past + s.M > (int64_t)max_chunks || (int64_t)n_past + s.M > (int64_t)w_dim)
        return MHLA_ERR_INVALID_ARG;
    if (s.B == 0 || s.H == 0) return MHLA_OK;   // no pair: nothing to read or write
    const void* ins[4] = {q, k, v, W};
    for (const void* x : ins)
        if (!x) return MHLA_ERR_INVALID_ARG;
    if (!state || !out) return MHLA_ERR_INVALID_ARG;
    for (const void* x : ins)
        if (!aligned16(x)) return MHLA_ERR_MISALIGNED;
    if (!aligned16(state) || !aligned16(out)) return MHLA_ERR_MISALIGNED;
    const size_t tbytes = (size_t)(s.B * s.N * s.H * s.D) * s.esz;
    const size_t wbytes = (size_t)w_dim * (size_t)w_dim * 4;
    const size_t sbytes = stream_state_bytes(s, max_chunks);
    const size_t insz[4] = {tbytes, tbytes, tbytes, wbytes};
    for (int b = 0; b < 4; ++b)
        if (overlaps(out, tbytes, ins[b], insz[b]) || overlaps(state, sbytes, ins[b], insz[b]))
            return MHLA_ERR_INVALID_ARG;
    if (overlaps(out, tbytes, state, sbytes)) return MHLA_ERR_INVALID_ARG;
    const size_t need = stream_ws_bytes(s);
    bool owned = false;
    if (ws) {
        if (ws_bytes < need) return MHLA_ERR_INVALID_ARG;
        if (!aligned16(ws)) return MHLA_ERR_MISALIGNED;
        for (int b = 0; b < 4; ++b)
            if (overlaps(ws, need, ins[b], insz[b])) return MHLA_ERR_INVALID_ARG;
        if (overlaps(ws, need, out, tbytes) || overlaps(ws, need, state, sbytes)) return MHLA_ERR_INVALID_ARG;
    } else {
        if (ws_bytes != 0) return MHLA_ERR_INVALID_ARG;
        const mhla_status as = alloc_workspace(&ws, need, stream);
        if (as != MHLA_OK) return as;
        owned = true;
    }
    mhla::StreamLaunch S;
    S.g = make_geo(s, grid->eps);
    S.bf16 = s.dtype == MHLA_BF16;
    S.q = q; S.k = k; S.v = v; S.W = W; S.w_dim = w_dim;
    S.n_past = n_past;
    S.state = state;
    S.max_chunks = max_chunks;
    const StreamLayout SL = stream_layout(s);
    char* wsb = static_cast<char*>(ws);
    S.cp = SL.cp;
    S.mixed = !S.bf16 ? static_cast<float*>(ws) : SL.cp > 1 ? reinterpret_cast<float*>(wsb + SL.mixed) : nullptr;
    S.st = S.bf16 ? reinterpret_cast<uint16_t*>(wsb + SL.st) : nullptr;
    S.zt = S.bf16 ? reinterpret_cast<float*>(wsb + SL.zt) : nullptr;
    S.ssub = SL.cp > 1 ? reinterpret_cast<float*>(wsb + SL.ssub) : nullptr;
    if (SL.cp > 1) {
        S.gs = make_geo(subchunk_shape(s, SL.cp), grid->eps);
        S.gs.WD = SL.cp;
        S.gs.WM = (int32_t)s.M;
    }
    S.out = out;
    S.stream = stream;
    const hipError_t err = mhla::run_causal_stream(S);
    if (owned) (void)hipFreeAsync(ws, stream);
    return err == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
}

// ---------------------------------------------------------------- no-alloc entry point
//
// mhla_forward_noalloc takes its workspace from `scratch`, a fixed array of
// device memory of which every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in;
// its device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device and kept in scratch_dev[].
constexpr size_t kScratchBytes = MHLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};

// Device address of the current GPU's scratch (looked up on the first call on
// that GPU, with it current).
mhla_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return MHLA_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return MHLA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return MHLA_ERR_HIP;
        }
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return MHLA_OK;
}

mhla_status forward_noalloc_impl(const void* q, const void* k, const void* v, const float* W,
                                 const mhla_grid* grid, const mhla_block* block, void* out,
                                 hipStream_t stream) {
    Shape s;
    const mhla_status st = check(grid, block, &s);
    if (st != MHLA_OK) return st;
    if (s.B == 0 || s.H == 0) return MHLA_OK;
    if (layout(s).total > kScratchBytes) return MHLA_ERR_UNSUPPORTED;
    if (stream) {
        // the scratch used is the current GPU's: the stream must run there
        int cur = -1, sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) {
            (void)hipGetLastError();
            return MHLA_ERR_HIP;
        }
        if (sdev != cur) return MHLA_ERR_INVALID_ARG;
    }
    void* ws = nullptr;
    const mhla_status sp = scratch_on_current_device(&ws);
    if (sp != MHLA_OK) return sp;
    return forward_impl(q, k, v, W, grid, block, out, ws, kScratchBytes, false, MHLA_PATH_3KERNEL, nullptr,
                        stream);
}

}  // namespace

extern "C" {

size_t mhla_backward_workspace_bytes(const mhla_grid* grid, const mhla_block* block) {
    Shape s;
    if (check(grid, block, &s) != MHLA_OK || s.B == 0 || s.H == 0) return 0;
    return bwd_supported(s) ? bwd_layout(s).total : gen_layout(s).total;
}

mhla_status mhla_backward(const void* q, const void* k, const void* v, const float* W, const void* dout,
                          const mhla_grid* grid, const mhla_block* block, void* dq, void* dk, void* dv,
                          float* dW, void* ws, size_t ws_bytes, const hipEvent_t* stage_events,
                          hipStream_t stream) {
    return backward_impl(q, k, v, W, dout, grid, block, dq, dk, dv, dW, ws, ws_bytes, stage_events, stream,
                         false);
}

mhla_status mhla_backward_ex(const void* q, const void* k, const void* v, const float* W, const void* dout,
                             const mhla_grid* grid, const mhla_block* block, void* dq, void* dk, void* dv,
                             float* dW, void* ws, size_t ws_bytes, int32_t variant,
                             const hipEvent_t* stage_events, hipStream_t stream) {
    return backward_impl(q, k, v, W, dout, grid, block, dq, dk, dv, dW, ws, ws_bytes, stage_events, stream,
                         false, variant);
}

size_t mhla_causal_backward_workspace_bytes(const mhla_grid* grid, const mhla_block* block) {
    Shape s;
    if (check(grid, block, &s) != MHLA_OK || s.B == 0 || s.H == 0 || !causal_supported(s)) return 0;
    return cbwd_supported(s) ? cbwd_layout(s).total : gen_layout(s, true).total;
}

mhla_status mhla_causal_backward(const void* q, const void* k, const void* v, const float* W, const void* dout,
                                 const mhla_grid* grid, const mhla_block* block, void* dq, void* dk, void* dv,
                                 float* dW, void* ws, size_t ws_bytes, const hipEvent_t* stage_events,
                                 hipStream_t stream) {
    return backward_impl(q, k, v, W, dout, grid, block, dq, dk, dv, dW, ws, ws_bytes, stage_events, stream,
                         true);
}

size_t mhla_layer_workspace_bytes(const mhla_grid* grid, const mhla_block* block) {
    Shape s;
    if (check(grid, block, &s) != MHLA_OK || s.dtype != MHLA_BF16 || s.B == 0 || s.H == 0) return 0;
    return layer_layout(s).total;
}

mhla_status mhla_layer_forward(const void* x, const float* W, const mhla_grid* grid, const mhla_block* block,
                               const mhla_layer_params* params, void* y, void* ws, size_t ws_bytes,
                               const hipEvent_t* stage_events, hipStream_t stream) {
    return layer_impl(x, W, grid, block, params, y, ws, ws_bytes, stage_events, stream);
}

const char* mhla_status_string(mhla_status status) {
    // C callers may pass any int: read it as one.
    static_assert(sizeof(mhla_status) == sizeof(int), "mhla_status is an int-sized enum");
    int code = 0;
    std::memcpy(&code, &status, sizeof(code));
    switch (code) {
        case MHLA_OK: return "MHLA_OK";
        case MHLA_ERR_INVALID_ARG: return "MHLA_ERR_INVALID_ARG: invalid argument";
        case MHLA_ERR_UNSUPPORTED: return "MHLA_ERR_UNSUPPORTED: unsupported head_dim, dtype or size";
        case MHLA_ERR_MISALIGNED: return "MHLA_ERR_MISALIGNED: pointer not 16-byte aligned";
        case MHLA_ERR_ALLOC: return "MHLA_ERR_ALLOC: workspace allocation failed";
        case MHLA_ERR_HIP: return "MHLA_ERR_HIP: HIP launch or runtime error";
    }
    return "unknown mhla_status";
}

mhla_status mhla_check_problem(const mhla_grid* grid, const mhla_block* block, int64_t* num_blocks,
                               int64_t* block_tokens) {
    Shape s;
    const mhla_status st = check(grid, block, &s);
    if (st == MHLA_OK) {
        if (num_blocks) *num_blocks = s.M;
        if (block_tokens) *block_tokens = s.T;
    }
    return st;
}

mhla_status mhla_launch_plan(const mhla_grid* grid, const mhla_block* block, int32_t path_arg,
                             int32_t* num_kernels, const char** kernel_names) {
    Shape s;
    const mhla_status st = check(grid, block, &s);
    if (st != MHLA_OK) return st;
    int32_t path = 0, variant = 0;
    if (!split_path(path_arg, &path, &variant)) return MHLA_ERR_INVALID_ARG;
    if (path == MHLA_PATH_CAUSAL && !causal_supported(s)) return MHLA_ERR_UNSUPPORTED;
    const char* names[3] = {nullptr, nullptr, nullptr};
    int n = 0;
    if (s.B != 0 && s.H != 0) {
        names[n++] = "block_kv_summary";
        if (path == MHLA_PATH_FUSED) {
            names[n++] = "query_apply_fused";
        } else if (path == MHLA_PATH_CAUSAL) {
            names[n++] = "mix_summaries";
            names[n++] = "query_apply_causal";
        } else {
            names[n++] = "mix_summaries";
            names[n++] = "query_apply";
        }
    }
    if (num_kernels) *num_kernels = n;
    if (kernel_names)
        for (int i = 0; i < 3; ++i) kernel_names[i] = names[i];
    return MHLA_OK;
}

size_t mhla_workspace_bytes(const mhla_grid* grid, const mhla_block* block) {
    Shape s;
    if (check(grid, block, &s) != MHLA_OK || s.B == 0 || s.H == 0) return 0;
    return layout(s).total;
}

mhla_status mhla_forward(const void* q, const void* k, const void* v, const float* W,
                         const mhla_grid* grid, const mhla_block* block, void* out,
                         hipStream_t stream) {
    return forward_impl(q, k, v, W, grid, block, out, nullptr, 0, true, MHLA_PATH_3KERNEL, nullptr,
                        stream);
}

mhla_status mhla_forward_ws(const void* q, const void* k, const void* v, const float* W,
                            const mhla_grid* grid, const mhla_block* block, void* out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
    if (!ws) {
        Shape s;
        const mhla_status st = check(grid, block, &s);
        if (st != MHLA_OK) return st;
        if (s.B != 0 && s.H != 0) return MHLA_ERR_INVALID_ARG;
    }
    return forward_impl(q, k, v, W, grid, block, out, ws, ws_bytes, false, MHLA_PATH_3KERNEL,
                        nullptr, stream);
}

mhla_status mhla_forward_ex(const void* q, const void* k, const void* v, const float* W,
                            const mhla_grid* grid, const mhla_block* block, void* out, void* ws,
                            size_t ws_bytes, int32_t path, const hipEvent_t* stage_events,
                            hipStream_t stream) {
    return forward_impl(q, k, v, W, grid, block, out, ws, ws_bytes, true, path, stage_events,
                        stream);
}

mhla_status mhla_forward_noalloc(const void* q, const void* k, const void* v, const float* W,
                                 const mhla_grid* grid, const mhla_block* block, void* out,
                                 hipStream_t stream) {
    return forward_noalloc_impl(q, k, v, W, grid, block, out, stream);
}

size_t mhla_causal_state_bytes(const mhla_grid* grid, const mhla_block* block, int32_t max_chunks) {
    Shape s;
    if (check(grid, block, &s) != MHLA_OK || max_chunks <= 0) return 0;
    return stream_state_bytes(s, max_chunks);
}

size_t mhla_causal_stream_workspace_bytes(const mhla_grid* grid, const mhla_block* block) {
    Shape s;
    if (check(grid, block, &s) != MHLA_OK || s.B == 0 || s.H == 0 || !chunks_contiguous(s)) return 0;
    return stream_ws_bytes(s);
}

mhla_status mhla_causal_stream(const void* q, const void* k, const void* v, const float* W, int32_t w_dim,
                               const mhla_grid* grid, const mhla_block* block, int32_t n_past, float* state,
                               int32_t max_chunks, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    return stream_impl(q, k, v, W, w_dim, grid, block, n_past, state, max_chunks, out, ws, ws_bytes, stream);
}

}  // extern "C"
