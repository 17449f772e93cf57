"""The C ABI without a GPU: exports, status strings, workspace arithmetic and
every validation error (all returned before any HIP call)."""
import ctypes
import math
import os
import re

import pytest

import token_level_head_block_amd as mh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "mhla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return mh.lib()


def test_every_declared_function_is_exported(L):
    names = header_functions()
    assert {"mhla_forward", "mhla_forward_ws", "mhla_forward_ex", "mhla_workspace_bytes",
            "mhla_status_string", "mhla_check_problem", "mhla_launch_plan"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(6):
        s = mh.mhla_status_string(code)
        assert s.startswith("MHLA_")
    assert mh.mhla_status_string(99) == "unknown mhla_status"


def cfg2():
    return mh.make_grid(1, 6, 64, mh.MHLA_BF16, (256, 256), 1e-6), mh.make_block((16, 16))


def test_workspace_bytes_layout(L):
    g, b = cfg2()
    st, M, T = mh.mhla_check_problem(g, b)
    assert (st, M, T) == (mh.MHLA_OK, 256, 256)
    recs = 6 * 256
    up = lambda x: (x + 255) // 256 * 256
    assert mh.mhla_workspace_bytes(g, b) == up(recs * (64 * 64 + 64) * 2) + up(recs * 64 * 64 * 2) + \
        up(recs * 64 * 4) + up(256 * 256 * 2)
    g32 = mh.make_grid(1, 1, 32, mh.MHLA_F32, (16, 16), 1e-6)
    assert mh.mhla_workspace_bytes(g32, mh.make_block((4, 4))) == \
        up(16 * (32 * 32 + 32) * 4) + up(16 * 32 * 32 * 4) + up(16 * 32 * 4)
    g3 = mh.make_grid(1, 12, 128, mh.MHLA_BF16, (16, 64, 64), 1e-6)
    assert mh.mhla_check_problem(g3, mh.make_block((4, 8, 8)))[1:] == (256, 256)
    assert mh.mhla_workspace_bytes(mh.make_grid(0, 6, 64, mh.MHLA_BF16, (256, 256)), b) == 0


@pytest.mark.parametrize("mut,code", [
    (lambda g, b: setattr(g, "head_dim", 48), mh.MHLA_ERR_UNSUPPORTED),
    (lambda g, b: setattr(g, "dtype", 7), mh.MHLA_ERR_UNSUPPORTED),
    (lambda g, b: setattr(g, "ndim", 4), mh.MHLA_ERR_INVALID_ARG),
    (lambda g, b: setattr(g, "ndim", 1), mh.MHLA_ERR_INVALID_ARG),
    (lambda g, b: setattr(g, "batch", -1), mh.MHLA_ERR_INVALID_ARG),
    (lambda g, b: setattr(g, "eps", -1e-6), mh.MHLA_ERR_INVALID_ARG),
    (lambda g, b: setattr(g, "eps", math.nan), mh.MHLA_ERR_INVALID_ARG),
    (lambda g, b: setattr(g, "eps", math.inf), mh.MHLA_ERR_INVALID_ARG),
    (lambda g, b: b.extent.__setitem__(0, 15), mh.MHLA_ERR_INVALID_ARG),      # 256 % 15 != 0
    (lambda g, b: b.extent.__setitem__(1, 0), mh.MHLA_ERR_INVALID_ARG),
    (lambda g, b: g.extent.__setitem__(0, -256), mh.MHLA_ERR_INVALID_ARG),
    (lambda g, b: setattr(g, "batch", 1 << 20), mh.MHLA_ERR_UNSUPPORTED),     # >= 2^31 elements
    (lambda g, b: (b.extent.__setitem__(0, 1), b.extent.__setitem__(1, 1)),  # M = 65536: M * M >= 2^31
     mh.MHLA_ERR_UNSUPPORTED),
], ids=["d48", "dtype", "ndim4", "ndim1", "neg-batch", "neg-eps", "nan-eps", "inf-eps",
        "not-divisible", "zero-block", "neg-extent", "too-large", "M-squared"])
def test_problem_validation(L, mut, code):
    g, b = cfg2()
    mut(g, b)
    assert mh.mhla_check_problem(g, b)[0] == code
    assert mh.mhla_workspace_bytes(g, b) == 0
    # the forward entry points return the same code before touching HIP
    fake = 1 << 20
    assert L.mhla_forward(fake, fake * 2, fake * 3, fake * 4, ctypes.byref(g), ctypes.byref(b),
                          fake * 5, None) == code


def test_null_structs(L):
    assert L.mhla_check_problem(None, None, None, None) == mh.MHLA_ERR_INVALID_ARG
    assert L.mhla_workspace_bytes(None, None) == 0


BIG = 1 << 36          # fake, 16-byte aligned, far apart: never dereferenced


def call_fwd(L, g, b, q=BIG, k=2 * BIG, v=3 * BIG, W=4 * BIG, out=5 * BIG, ws=None, ws_bytes=0, path=0,
             entry="ex"):
    if entry == "ex":
        return L.mhla_forward_ex(q, k, v, W, ctypes.byref(g), ctypes.byref(b), out, ws, ws_bytes, path,
                                 None, None)
    return L.mhla_forward_ws(q, k, v, W, ctypes.byref(g), ctypes.byref(b), out, ws, ws_bytes, None)


def test_pointer_validation(L):
    g, b = cfg2()
    need = mh.mhla_workspace_bytes(g, b)
    ws = 6 * BIG
    assert call_fwd(L, g, b, q=None, ws=ws, ws_bytes=need) == mh.MHLA_ERR_INVALID_ARG
    assert call_fwd(L, g, b, W=None, ws=ws, ws_bytes=need) == mh.MHLA_ERR_INVALID_ARG
    assert call_fwd(L, g, b, out=None, ws=ws, ws_bytes=need) == mh.MHLA_ERR_INVALID_ARG
    assert call_fwd(L, g, b, k=2 * BIG + 8, ws=ws, ws_bytes=need) == mh.MHLA_ERR_MISALIGNED
    assert call_fwd(L, g, b, out=5 * BIG + 2, ws=ws, ws_bytes=need) == mh.MHLA_ERR_MISALIGNED
    assert call_fwd(L, g, b, ws=ws + 4, ws_bytes=need) == mh.MHLA_ERR_MISALIGNED
    # out overlapping an input
    assert call_fwd(L, g, b, out=BIG + 4096, ws=ws, ws_bytes=need) == mh.MHLA_ERR_INVALID_ARG
    assert call_fwd(L, g, b, out=4 * BIG - 1024 * 16, ws=ws, ws_bytes=need) == mh.MHLA_ERR_INVALID_ARG
    # workspace too small / overlapping out
    assert call_fwd(L, g, b, ws=ws, ws_bytes=need - 16) == mh.MHLA_ERR_INVALID_ARG
    assert call_fwd(L, g, b, ws=5 * BIG, ws_bytes=need) == mh.MHLA_ERR_INVALID_ARG
    # unknown path
    assert call_fwd(L, g, b, ws=ws, ws_bytes=need, path=7) == mh.MHLA_ERR_INVALID_ARG
    # mhla_forward_ws requires a workspace
    assert call_fwd(L, g, b, ws=None, ws_bytes=0, entry="ws") == mh.MHLA_ERR_INVALID_ARG
    # ws NULL with nonzero size
    assert call_fwd(L, g, b, ws=None, ws_bytes=64) == mh.MHLA_ERR_INVALID_ARG


def test_empty_problem_is_a_no_op(L):
    for B, H in ((0, 6), (1, 0)):
        g = mh.make_grid(B, H, 64, mh.MHLA_BF16, (256, 256))
        b = mh.make_block((16, 16))
        assert call_fwd(L, g, b, q=None, k=None, v=None, W=None, out=None) == mh.MHLA_OK
        assert call_fwd(L, g, b, q=None, k=None, v=None, W=None, out=None, entry="ws") == mh.MHLA_OK
        assert L.mhla_forward(None, None, None, None, ctypes.byref(g), ctypes.byref(b), None, None) == mh.MHLA_OK


def test_variant_flags(L):
    """Kernel-variant flags ride in the path argument; unknown bits and both
    mixing flags at once are rejected before any HIP call."""
    g, b = cfg2()
    three = ["block_kv_summary", "mix_summaries", "query_apply"]
    for flag in (mh.MHLA_VARIANT_MIX_RESIDENT, mh.MHLA_VARIANT_MIX_TILED, mh.MHLA_VARIANT_MIX_SPLIT,
                 mh.MHLA_VARIANT_NO_PAIR_HEADS, mh.MHLA_VARIANT_MIX_SPLIT | mh.MHLA_VARIANT_NO_PAIR_HEADS,
                 mh.MHLA_VARIANT_APPLY_REGS):
        assert mh.mhla_launch_plan(g, b, mh.MHLA_PATH_3KERNEL | flag) == (mh.MHLA_OK, three)
    need = mh.mhla_workspace_bytes(g, b)
    for bad in (1 << 13, 1 << 30, mh.MHLA_VARIANT_MIX_RESIDENT | mh.MHLA_VARIANT_MIX_TILED,
                mh.MHLA_VARIANT_MIX_SPLIT | mh.MHLA_VARIANT_MIX_TILED):
        assert mh.mhla_launch_plan(g, b, bad)[0] == mh.MHLA_ERR_INVALID_ARG
        assert call_fwd(L, g, b, ws=6 * BIG, ws_bytes=need, path=bad) == mh.MHLA_ERR_INVALID_ARG
    # the backward takes only the head-pair flag
    bneed = mh.mhla_backward_workspace_bytes(g, b)
    for bad in (mh.MHLA_VARIANT_MIX_TILED, 1 << 12):
        assert L.mhla_backward_ex(BIG, 2 * BIG, 3 * BIG, 4 * BIG, 5 * BIG, ctypes.byref(g), ctypes.byref(b),
                                  6 * BIG, 7 * BIG, 8 * BIG, 9 * BIG, 10 * BIG, bneed, bad, None,
                                  None) == mh.MHLA_ERR_INVALID_ARG


def test_noalloc_validation(L):
    """mhla_forward_noalloc: the scratch size in the header and the binding
    agree; problems whose workspace exceeds it, invalid problems and empty
    problems return before any HIP call."""
    text = open(os.path.join(ROOT, "include", "mhla.h")).read()
    m = re.search(r"#define MHLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == mh.MHLA_NOALLOC_SCRATCH_BYTES
    g, b = cfg2()
    assert mh.mhla_workspace_bytes(g, b) <= mh.MHLA_NOALLOC_SCRATCH_BYTES
    call = lambda g_, b_: L.mhla_forward_noalloc(BIG, 2 * BIG, 3 * BIG, 4 * BIG, ctypes.byref(g_),
                                                 ctypes.byref(b_), 5 * BIG, None)
    g1 = mh.make_grid(32, 6, 64, mh.MHLA_BF16, (64, 64), 1e-6)      # 32 x 6 pairs, 64 blocks: ~205 MB
    b1 = mh.make_block((8, 8))
    assert mh.mhla_workspace_bytes(g1, b1) > mh.MHLA_NOALLOC_SCRATCH_BYTES
    assert call(g1, b1) == mh.MHLA_ERR_UNSUPPORTED
    bad = mh.make_block((15, 16))
    assert call(g, bad) == mh.MHLA_ERR_INVALID_ARG
    g0 = mh.make_grid(0, 6, 64, mh.MHLA_BF16, (256, 256))
    assert L.mhla_forward_noalloc(None, None, None, None, ctypes.byref(g0), ctypes.byref(b), None,
                                  None) == mh.MHLA_OK


def test_injected_allocation_failure(L, monkeypatch):
    """MHLA_FAIL_ALLOC=1 makes every entry point that allocates its workspace
    on the stream return MHLA_ERR_ALLOC before any HIP call (nothing is
    enqueued); entry points given a workspace do not allocate."""
    monkeypatch.setenv("MHLA_FAIL_ALLOC", "1")
    g, b = cfg2()
    assert L.mhla_forward(BIG, 2 * BIG, 3 * BIG, 4 * BIG, ctypes.byref(g), ctypes.byref(b), 5 * BIG,
                          None) == mh.MHLA_ERR_ALLOC
    assert call_fwd(L, g, b, ws=None, ws_bytes=0) == mh.MHLA_ERR_ALLOC
    for fn in (L.mhla_backward, L.mhla_causal_backward):
        gg, bb = (g, b) if fn is L.mhla_backward else (mh.make_grid(1, 6, 64, mh.MHLA_BF16, (1, 4096)),
                                                     mh.make_block((1, 256)))
        assert fn(BIG, 2 * BIG, 3 * BIG, 4 * BIG, 5 * BIG, ctypes.byref(gg), ctypes.byref(bb), 6 * BIG, 7 * BIG,
                  8 * BIG, 9 * BIG, None, 0, None, None) == mh.MHLA_ERR_ALLOC
    gs, bs = mh.make_grid(2, 3, 64, mh.MHLA_BF16, (1, 256)), mh.make_block((1, 64))
    assert L.mhla_causal_stream(BIG, 2 * BIG, 3 * BIG, 4 * BIG, 10, ctypes.byref(gs), ctypes.byref(bs), 0,
                                6 * BIG, 10, 7 * BIG, None, 0, None) == mh.MHLA_ERR_ALLOC
    # validation still comes first, and a caller workspace needs no allocation
    assert call_fwd(L, g, mh.make_block((15, 16)), ws=None, ws_bytes=0) == mh.MHLA_ERR_INVALID_ARG
    assert call_fwd(L, g, b, q=None, ws=None, ws_bytes=0) == mh.MHLA_ERR_INVALID_ARG
    # mhla_forward_noalloc allocates nothing: its rejection of a large problem is unchanged
    g1 = mh.make_grid(32, 6, 64, mh.MHLA_BF16, (64, 64), 1e-6)
    assert L.mhla_forward_noalloc(BIG, 2 * BIG, 3 * BIG, 4 * BIG, ctypes.byref(g1), ctypes.byref(mh.make_block((8, 8))),
                                  5 * BIG, None) == mh.MHLA_ERR_UNSUPPORTED


def test_launch_plan(L):
    g, b = cfg2()
    three = ["block_kv_summary", "mix_summaries", "query_apply"]
    assert mh.mhla_launch_plan(g, b, mh.MHLA_PATH_3KERNEL) == (mh.MHLA_OK, three)
    assert mh.mhla_launch_plan(g, b, mh.MHLA_PATH_FUSED) == (mh.MHLA_OK, ["block_kv_summary", "query_apply_fused"])
    g32 = mh.make_grid(1, 1, 32, mh.MHLA_F32, (16, 16))
    assert mh.mhla_launch_plan(g32, mh.make_block((4, 4)))[1] == three
    assert mh.mhla_launch_plan(mh.make_grid(0, 6, 64, mh.MHLA_BF16, (256, 256)), b) == (mh.MHLA_OK, [])
    assert mh.mhla_launch_plan(g, b, 7)[0] == mh.MHLA_ERR_INVALID_ARG
    assert mh.mhla_launch_plan(g, mh.make_block((15, 16)))[0] == mh.MHLA_ERR_INVALID_ARG


def test_backward_workspace_and_validation(L):
    g, b = cfg2()
    need = mh.mhla_backward_workspace_bytes(g, b)
    assert need > mh.mhla_workspace_bytes(g, b)
    # d = 128 and fp32 take the general path: fp32 records [S | z] four times, dW partials
    g128, b128 = mh.make_grid(1, 12, 128, mh.MHLA_BF16, (16, 64, 64)), mh.make_block((4, 8, 8))
    rec = 12 * 256 * (128 * 128 + 128) * 4
    assert mh.mhla_backward_workspace_bytes(g128, b128) >= 4 * rec + 256 * 256 * 4
    g32, b32 = mh.make_grid(1, 1, 32, mh.MHLA_F32, (16, 16)), mh.make_block((4, 4))
    assert mh.mhla_backward_workspace_bytes(g32, b32) >= 4 * 16 * (32 * 32 + 32) * 4

    def bwd(g_, b_, q=BIG, k=2 * BIG, v=3 * BIG, W=4 * BIG, dout=5 * BIG, dq=6 * BIG, dk=7 * BIG,
            dv=8 * BIG, dW=9 * BIG, ws=10 * BIG, ws_bytes=None):
        wsb = mh.mhla_backward_workspace_bytes(g_, b_) if ws_bytes is None else ws_bytes
        return L.mhla_backward(q, k, v, W, dout, ctypes.byref(g_), ctypes.byref(b_), dq, dk, dv, dW, ws, wsb,
                               None, None)

    assert bwd(g128, b128, ws_bytes=mh.mhla_backward_workspace_bytes(g128, b128) - 16) == mh.MHLA_ERR_INVALID_ARG
    assert bwd(g32, b32, dW=None) == mh.MHLA_ERR_INVALID_ARG
    assert bwd(g, b, dout=None) == mh.MHLA_ERR_INVALID_ARG
    assert bwd(g, b, dW=None) == mh.MHLA_ERR_INVALID_ARG
    assert bwd(g, b, dk=7 * BIG + 8) == mh.MHLA_ERR_MISALIGNED
    assert bwd(g, b, dq=BIG + 4096) == mh.MHLA_ERR_INVALID_ARG          # dq overlaps q
    assert bwd(g, b, dv=6 * BIG + 64) == mh.MHLA_ERR_INVALID_ARG        # dv overlaps dq
    assert bwd(g, b, ws_bytes=need - 16) == mh.MHLA_ERR_INVALID_ARG
    assert bwd(g, b, ws=9 * BIG) == mh.MHLA_ERR_INVALID_ARG             # workspace overlaps dW
    assert bwd(g, mh.make_block((15, 16))) == mh.MHLA_ERR_INVALID_ARG


def test_causal_path_validation(L):
    seq = mh.make_grid(1, 6, 64, mh.MHLA_BF16, (1, 65536))
    chunk = mh.make_block((1, 256))
    assert mh.mhla_launch_plan(seq, chunk, mh.MHLA_PATH_CAUSAL) == (
        mh.MHLA_OK, ["block_kv_summary", "mix_summaries", "query_apply_causal"])
    # 2D blocks are not contiguous runs of raster indices
    g, b = cfg2()
    assert mh.mhla_launch_plan(g, b, mh.MHLA_PATH_CAUSAL)[0] == mh.MHLA_ERR_UNSUPPORTED
    need = mh.mhla_workspace_bytes(g, b)
    assert call_fwd(L, g, b, ws=6 * BIG, ws_bytes=need, path=mh.MHLA_PATH_CAUSAL) == mh.MHLA_ERR_UNSUPPORTED
    # full rows are
    assert mh.mhla_launch_plan(mh.make_grid(1, 2, 32, mh.MHLA_BF16, (12, 20)), mh.make_block((3, 20)),
                               mh.MHLA_PATH_CAUSAL)[0] == mh.MHLA_OK
    # every head_dim, bf16 and fp32
    assert mh.mhla_launch_plan(mh.make_grid(1, 2, 128, mh.MHLA_BF16, (1, 256)), mh.make_block((1, 64)),
                               mh.MHLA_PATH_CAUSAL)[0] == mh.MHLA_OK
    assert mh.mhla_launch_plan(mh.make_grid(1, 2, 32, mh.MHLA_F32, (1, 256)), mh.make_block((1, 64)),
                               mh.MHLA_PATH_CAUSAL)[0] == mh.MHLA_OK



def test_causal_backward_workspace_and_validation(L):
    seq = mh.make_grid(1, 6, 64, mh.MHLA_BF16, (1, 65536))
    chunk = mh.make_block((1, 256))
    need = mh.mhla_causal_backward_workspace_bytes(seq, chunk)
    toks = 65536 * 6
    # bf16, d = 64, whole chunks: the matrix-core backward's regions plus per-token
    # 1 / den and dden (fp32 pairs) and the per-pair dW[i, i] terms
    assert need == mh.mhla_backward_workspace_bytes(seq, chunk) + toks * 8 + 6 * 256 * 4
    # d = 128: the general kernels' fp32 records (four kinds) and per-token dnum (fp32), dden
    s128 = mh.make_grid(1, 6, 128, mh.MHLA_BF16, (1, 65536))
    rec = 6 * 256 * (128 * 128 + 128) * 4
    assert mh.mhla_causal_backward_workspace_bytes(s128, chunk) >= 4 * rec + toks * 128 * 4 + toks * 4 + 6 * 256 * 4
    # 2D blocks are not contiguous runs of raster indices: no workspace, and the call says so
    g, b = cfg2()
    assert mh.mhla_causal_backward_workspace_bytes(g, b) == 0

    def bwd(g_, b_, ws_bytes, q=BIG, dW=9 * BIG):
        return L.mhla_causal_backward(q, 2 * BIG, 3 * BIG, 4 * BIG, 5 * BIG, ctypes.byref(g_), ctypes.byref(b_),
                                      6 * BIG, 7 * BIG, 8 * BIG, dW, 10 * BIG, ws_bytes, None, None)

    assert bwd(g, b, 1 << 30) == mh.MHLA_ERR_UNSUPPORTED
    assert bwd(seq, chunk, need - 16) == mh.MHLA_ERR_INVALID_ARG
    assert bwd(seq, chunk, need, dW=None) == mh.MHLA_ERR_INVALID_ARG
    assert bwd(seq, chunk, need, q=BIG + 8) == mh.MHLA_ERR_MISALIGNED
    assert bwd(seq, mh.make_block((1, 255)), need) == mh.MHLA_ERR_INVALID_ARG
    # fp32 and d = 128 too
    f32 = mh.make_grid(2, 1, 128, mh.MHLA_F32, (1, 400))
    assert mh.mhla_causal_backward_workspace_bytes(f32, mh.make_block((1, 100))) > 0



def test_causal_stream_state_and_validation(L):
    new = mh.make_grid(2, 3, 64, mh.MHLA_BF16, (1, 256))
    chunk = mh.make_block((1, 64))
    L_ = 64 * 64 + 64
    assert mh.mhla_causal_state_bytes(new, chunk, 10) == 2 * 3 * 10 * L_ * 4
    assert mh.mhla_causal_state_bytes(new, chunk, 0) == 0
    # bf16: the mixed S of the 2*3*4 new records as bf16, then their mixed z in fp32 (256-byte aligned)
    up = lambda x: (x + 255) // 256 * 256
    assert mh.mhla_causal_stream_workspace_bytes(new, chunk) == up(2 * 3 * 4 * 64 * 64 * 2) + up(2 * 3 * 4 * 64 * 4)
    # fp32: the mixtures as fp32 records
    new32 = mh.make_grid(2, 3, 64, mh.MHLA_F32, (1, 256))
    assert mh.mhla_causal_stream_workspace_bytes(new32, chunk) == 2 * 3 * 4 * L_ * 4
    g2d, b2d = cfg2()
    assert mh.mhla_causal_stream_workspace_bytes(g2d, b2d) == 0          # 2D tiles are not chunks
    sb = mh.mhla_causal_state_bytes(new, chunk, 10)

    def call(g=new, b=chunk, n_past=0, max_chunks=10, w_dim=10, q=BIG, state=6 * BIG, out=7 * BIG,
             ws=8 * BIG, ws_bytes=1 << 30):
        return L.mhla_causal_stream(q, 2 * BIG, 3 * BIG, 4 * BIG, w_dim, ctypes.byref(g), ctypes.byref(b), n_past,
                                    state, max_chunks, out, ws, ws_bytes, None)

    assert call(g=g2d, b=b2d) == mh.MHLA_ERR_UNSUPPORTED
    assert call(n_past=-1) == mh.MHLA_ERR_INVALID_ARG
    assert call(n_past=7) == mh.MHLA_ERR_INVALID_ARG                       # 7 + 4 chunks > max_chunks 10
    assert call(n_past=6, max_chunks=12, w_dim=9) == mh.MHLA_ERR_INVALID_ARG   # row 9 is past w_dim
    assert call(state=None) == mh.MHLA_ERR_INVALID_ARG
    assert call(out=6 * BIG + sb - 16) == mh.MHLA_ERR_INVALID_ARG          # out overlaps the state
    assert call(out=BIG + 64) == mh.MHLA_ERR_INVALID_ARG                   # out overlaps q
    assert call(ws_bytes=16) == mh.MHLA_ERR_INVALID_ARG
    assert call(q=BIG + 4) == mh.MHLA_ERR_MISALIGNED
    assert call(state=6 * BIG + 8) == mh.MHLA_ERR_MISALIGNED
    assert call(b=mh.make_block((1, 60))) == mh.MHLA_ERR_INVALID_ARG       # 256 is not a multiple of 60
    empty = mh.make_grid(0, 3, 64, mh.MHLA_BF16, (1, 256))
    assert call(g=empty, q=None, state=None, out=None) == mh.MHLA_OK        # nothing to do


def test_layer_workspace_and_validation(L):
    g, b = cfg2()
    C, R = 6 * 64, 65536
    need = mh.mhla_layer_workspace_bytes(g, b)
    assert need >= 4 * R * C * 2 + 3 * C * C * 2 + mh.mhla_workspace_bytes(g, b)
    assert mh.mhla_layer_workspace_bytes(mh.make_grid(1, 6, 64, mh.MHLA_F32, (256, 256)), b) == 0
    assert mh.mhla_layer_workspace_bytes(mh.make_grid(0, 6, 64, mh.MHLA_BF16, (256, 256)), b) == 0
    base = dict(ln_w=20 * BIG, ln_b=21 * BIG, w_qkv=22 * BIG, b_qkv=23 * BIG, lepe_w=26 * BIG,
                lepe_b=27 * BIG, w_out=28 * BIG, b_out=29 * BIG)

    def layer(g_=g, b_=b, x=BIG, W=2 * BIG, y=3 * BIG, ws=4 * BIG, ws_bytes=None, phi=0, phi_eps=1e-6,
              ln_eps=1e-5, rms_eps=1e-6, **kw):
        P = mh.mhla_layer_params()
        for k_, v_ in dict(base, **kw).items():
            setattr(P, k_, v_)
        P.phi, P.phi_eps, P.ln_eps, P.rms_eps = phi, phi_eps, ln_eps, rms_eps
        wsb = need if ws_bytes is None else ws_bytes
        return L.mhla_layer_forward(x, W, ctypes.byref(g_), ctypes.byref(b_), ctypes.byref(P), y, ws, wsb,
                                    None, None)

    assert L.mhla_layer_forward(BIG, 2 * BIG, ctypes.byref(g), ctypes.byref(b), None, 3 * BIG, 4 * BIG, need,
                                None, None) == mh.MHLA_ERR_INVALID_ARG
    assert layer(g_=mh.make_grid(1, 6, 64, mh.MHLA_F32, (256, 256))) == mh.MHLA_ERR_UNSUPPORTED
    assert layer(phi=5) == mh.MHLA_ERR_INVALID_ARG
    assert layer(phi_eps=-1.0) == mh.MHLA_ERR_INVALID_ARG
    assert layer(ln_eps=0.0) == mh.MHLA_ERR_INVALID_ARG
    assert layer(ln_eps=float("nan")) == mh.MHLA_ERR_INVALID_ARG
    assert layer(qn_w=24 * BIG) == mh.MHLA_ERR_INVALID_ARG                    # q norm without k norm
    assert layer(qn_w=24 * BIG, kn_w=25 * BIG, rms_eps=0.0) == mh.MHLA_ERR_INVALID_ARG
    assert layer(lepe_w=None) == mh.MHLA_ERR_INVALID_ARG                      # LePE bias without kernel
    for missing in ("ln_w", "ln_b", "w_qkv", "w_out"):
        assert layer(**{missing: None}) == mh.MHLA_ERR_INVALID_ARG, missing
    assert layer(x=None) == mh.MHLA_ERR_INVALID_ARG
    assert layer(y=None) == mh.MHLA_ERR_INVALID_ARG
    assert layer(w_qkv=22 * BIG + 8) == mh.MHLA_ERR_MISALIGNED
    assert layer(y=3 * BIG + 2) == mh.MHLA_ERR_MISALIGNED
    assert layer(y=BIG + 4096) == mh.MHLA_ERR_INVALID_ARG                     # y overlaps x
    assert layer(y=28 * BIG - 64) == mh.MHLA_ERR_INVALID_ARG                  # y overlaps w_out
    assert layer(ws_bytes=need - 16) == mh.MHLA_ERR_INVALID_ARG
    assert layer(ws=3 * BIG) == mh.MHLA_ERR_INVALID_ARG                       # workspace overlaps y
    assert layer(ws=None, ws_bytes=64) == mh.MHLA_ERR_INVALID_ARG
    # LePE needs a 2D grid
    g3, b3 = mh.make_grid(1, 12, 128, mh.MHLA_BF16, (16, 64, 64)), mh.make_block((4, 8, 8))
    assert layer(g_=g3, b_=b3, ws_bytes=1 << 40) == mh.MHLA_ERR_UNSUPPORTED
    # empty problem: nothing to do, no pointer needed
    g0 = mh.make_grid(0, 6, 64, mh.MHLA_BF16, (256, 256))
    assert layer(g_=g0, x=None, y=None, ws=None, ws_bytes=0) == mh.MHLA_OK


def test_workspace_sizes_with_token_parts(L):
    """The forward's workspace with token parts, by the rule the header states:
    tp doubles while B*H*M*tp < 1536, M*2*tp <= 256 and 2*tp*64 <= T; region 0
    holds P*M*tp records, region 3 W with roundup(M*max(tp, k), 32) columns, k = 2*cp
    where the blocks are contiguous runs of raster order (the causal form's W
    high and low parts) and cp otherwise."""
    up = lambda x: (x + 255) // 256 * 256

    def expected(B, H, d, M, T, split=None, bf16=True, contiguous=False):
        """split: extent of the chunk's slowest axis > 1 when chunks are contiguous."""
        tp = cp = 1
        if bf16:
            while B * H * M * tp < 1536 and M * 2 * tp <= 256 and 2 * tp * 64 <= T:
                tp *= 2
            while split and split % (2 * cp) == 0 and T // (2 * cp) >= 256 and M * 2 * cp <= 256:
                cp *= 2
        e = 2 if bf16 else 4
        P = B * H
        r0 = P * M * max(tp, cp)
        n = up(r0 * (d * d + d) * e) + up(P * M * cp * d * d * e) + up(P * M * cp * d * 4)
        if bf16:
            k = 2 * cp if contiguous else cp
            n += up((M * cp + 63) // 64 * 64 * ((M * max(tp, k) + 31) // 32 * 32) * 2)
        return n, tp, cp

    for (B, H, d, grid, block, split, contiguous) in [
            (1, 6, 64, (256, 256), (64, 64), None, False),     # M = 16, T = 4096: tp = 16 (tiles: no sub-chunks)
            (1, 6, 64, (256, 256), (32, 32), None, False),     # M = 64: tp = 4
            (1, 6, 64, (256, 256), (16, 16), None, False),     # M = 256: tp = 1
            (2, 3, 32, (64, 64), (32, 32), None, False),       # M = 4, T = 1024: tp = 16
            (1, 2, 128, (20, 40), (20, 40), 20, True),         # M = 1, T = 800: tp = 4, cp = 2 (20 rows of 40)
            (1, 6, 64, (256, 256), (16, 256), 16, True),       # chunks of 16 rows: tp = 16, cp = 16
            (1, 6, 64, (256, 256), (1, 256), None, True)]:     # chunks of one row: tp = cp = 1
        g, b = mh.make_grid(B, H, d, mh.MHLA_BF16, grid), mh.make_block(block)
        M = (grid[0] // block[0]) * (grid[1] // block[1])
        T = block[0] * block[1]
        n, tp, cp = expected(B, H, d, M, T, split, contiguous=contiguous)
        assert mh.mhla_workspace_bytes(g, b) == n, (grid, block, tp, cp)
    # fp32 problems never split
    g, b = mh.make_grid(1, 6, 64, mh.MHLA_F32, (256, 256)), mh.make_block((64, 64))
    assert mh.mhla_workspace_bytes(g, b) == expected(1, 6, 64, 16, 4096, bf16=False)[0]
