"""HIP path vs the float64 CPU oracle, through the C ABI.

Bar: max|d| / max|ref| <= 1e-5 for float32 problems and <= 1e-2 for bf16
(bf16 I/O with fp32 accumulation).  Small problems are compared element by
element over every output; the full-size workloads run in the benchmark's
launch configuration and are compared on every output of every (b, h) pair.
"""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_block_amd as mh
from token_level_head_block_amd import synth

from gpu_util import TOL, Run, rel_err, say, to_host64

pytestmark = pytest.mark.gpu

BF, F = synth.BF16, synth.F32

# name, B, H, d, grid, block, dtype, std  -- sizes the oracle finishes in seconds,
# spanning several tiles, ragged token / block tails, 2D and 3D.
SMALL = [
    ("bf-d64-M24", 2, 3, 64, (32, 48), (8, 8), BF, 1.0),
    ("bf-d32-T15", 1, 2, 32, (12, 20), (3, 5), BF, 1.0),
    ("bf-d128-3d", 1, 2, 128, (4, 12, 12), (2, 3, 4), BF, 1.0),
    ("bf-d64-T25-M64", 1, 2, 64, (40, 40), (5, 5), BF, 1.0),
    ("bf-d64-M1", 1, 2, 64, (7, 9), (7, 9), BF, 1.0),
    ("bf-d32-T1", 1, 1, 32, (6, 6), (1, 1), BF, 1.0),
    ("bf-d32-M10", 1, 3, 32, (15, 10), (3, 5), BF, 0.5),
    ("bf-d32-M360", 1, 1, 32, (36, 40), (2, 2), BF, 1.0),
    ("bf-d32-M1024", 1, 2, 32, (64, 64), (2, 2), BF, 1.0),
    ("bf-d128-T200", 1, 1, 128, (20, 40), (10, 20), BF, 1.0),
    ("bf-d128-H3-full", 2, 3, 128, (16, 32), (8, 8), BF, 1.0),   # odd head count: a half-empty head group
    ("bf-d128-row8", 1, 2, 128, (24, 16), (3, 8), BF, 1.0),     # rows of 8 tokens, T = 24: ragged last step
    # blocks of at most 64 tokens: summaries of four, two or one block per wave
    ("bf-d64-T64-M10-two-blocks", 1, 3, 64, (40, 16), (8, 8), BF, 1.0),
    ("bf-d64-T64-M5-one-block", 1, 2, 64, (40, 8), (8, 8), BF, 1.0),
    ("bf-d32-T32-M12-pairs", 2, 4, 32, (16, 24), (4, 8), BF, 1.0),
    ("f32-d32-T15", 1, 2, 32, (12, 20), (3, 5), F, 1.0),
    ("f32-d64-3d", 2, 1, 64, (8, 16, 8), (2, 4, 4), F, 1.0),
    ("f32-d128", 1, 2, 128, (16, 16), (4, 8), F, 1.0),
    ("f32-d64-M70", 1, 1, 64, (14, 20), (2, 2), F, 1.0),
]


def small_problem(case):
    name, B, H, d, grid, block, dt, std = case
    return synth.Problem(name, B, H, d, grid, block, dtype=dt, std=std)


@pytest.mark.parametrize("path", [mh.MHLA_PATH_3KERNEL, mh.MHLA_PATH_FUSED], ids=["3kernel", "fused"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_small_problems_all_outputs(case, path):
    p = small_problem(case)
    q, k, v, W = synth.make_inputs(p, seed=21)
    ref = oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)
    run = Run(p, q, k, v, W)
    out = to_host64(run.forward(path))
    err = rel_err(out, ref)
    say(f"  {p.name} path={path}: max|d|/max|ref| = {err:.3e}")
    assert np.isfinite(out).all()
    assert err <= TOL[p.dtype]


def test_tiny_fp32_workload_and_intermediates():
    p = synth.CONFIGS[0]
    q, k, v, W = synth.make_inputs(p, seed=0)
    run = Run(p, q, k, v, W)
    out = to_host64(run.forward())
    ref = oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)
    assert rel_err(out, ref) <= 1e-5
    S, z, St, zt = run.workspace()
    rS, rz, rSt, rzt = oracle.summaries(k, v, W, p.grid, p.block)
    for name, a, b in (("S", S, rS), ("z", z, rz), ("St", St, rSt), ("zt", zt, rzt)):
        e = rel_err(a, b)
        say(f"  {name}: {e:.2e}")
        assert e <= 1e-5, name


@pytest.mark.parametrize("case", [c for c in SMALL if c[6] == BF][:4], ids=lambda c: c[0])
def test_bf16_intermediates(case):
    """Per-kernel parity: summaries (bf16), mixed summaries (bf16) and mixed
    normalisers (fp32) against the oracle's float64 intermediates."""
    p = small_problem(case)
    q, k, v, W = synth.make_inputs(p, seed=22)
    run = Run(p, q, k, v, W)
    run.forward()
    S, z, St, zt = run.workspace()
    rS, rz, rSt, rzt = oracle.summaries(k, v, W, p.grid, p.block)
    for name, a, b in (("S", S, rS), ("z", z, rz), ("St", St, rSt), ("zt", zt, rzt)):
        e = rel_err(a, b)
        say(f"  {p.name} {name}: {e:.2e}")
        assert e <= 1e-2, name


MIX_CASES = [
    ("mix-d64-M16-units544", 4, 8, 64, (16, 16), (4, 4), BF, 1.0),     # 544 work units: several per workgroup
    ("mix-d32-M180", 1, 3, 32, (30, 24), (2, 2), BF, 1.0),              # 3 query-block tiles, ragged
    ("mix-d128-M96", 1, 2, 128, (24, 32), (2, 4), BF, 1.0),
    # more than three units per persistent workgroup
    ("mix-d64-M16-units1088", 8, 8, 64, (16, 16), (4, 4), BF, 1.0),
    ("mix-d128-M256-units774", 1, 3, 128, (32, 32), (2, 2), BF, 1.0),
    # 64 pairs, 144 blocks: 17 column tiles per pair, the last one ragged
    ("mix-d32-M144-H64-ragged-tile", 1, 64, 32, (48, 48), (4, 4), BF, 1.0),
]


MIX_VARIANTS = {   # path flags of each bf16 mixing variant
    "default": 0,
    "split": mh.MHLA_VARIANT_MIX_SPLIT,
    "resident": mh.MHLA_VARIANT_MIX_RESIDENT,
    "per-tile": mh.MHLA_VARIANT_MIX_TILED,
}


@pytest.mark.parametrize("case", MIX_CASES, ids=lambda c: c[0])
def test_mixing_kernels(case):
    """Every bf16 mixing kernel (a workgroup per column and query-block tile,
    persistent with W in registers, and a workgroup per column tile) against
    the oracle's mixed summaries, and the whole output of each against the
    oracle."""
    p = small_problem(case)
    q, k, v, W = synth.make_inputs(p, seed=25)
    ref = oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)
    _, _, rSt, rzt = oracle.summaries(k, v, W, p.grid, p.block)
    run = Run(p, q, k, v, W)
    for name, flag in MIX_VARIANTS.items():
        out = to_host64(run.forward(mh.MHLA_PATH_3KERNEL | flag))
        _, _, St, zt = run.workspace()
        e_out, e_st, e_zt = rel_err(out, ref), rel_err(St, rSt), rel_err(zt, rzt)
        say(f"  {p.name} {name}: out {e_out:.2e} St {e_st:.2e} zt {e_zt:.2e}")
        assert e_out <= TOL[p.dtype] and e_st <= 1e-2 and e_zt <= 1e-2


PAIR_CASES = [
    ("pair-d32-full-B2", 2, 4, 32, (32, 32), (8, 8), BF, 0.5),   # whole 32-token groups, two batch items
    ("pair-d32-row8", 1, 6, 32, (24, 16), (3, 8), BF, 1.0),      # rows of 8 tokens, T = 24
    ("pair-d32-ragged", 1, 2, 32, (12, 20), (3, 5), BF, 1.0),    # rows of 5 tokens
    ("pair-d32-odd-H", 1, 3, 32, (16, 16), (4, 4), BF, 1.0),     # odd head count: one head per wave
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=lambda c: c[0])
def test_d32_head_pairs(case):
    """head_dim 32 with an even head count: the summary kernel reads head
    pairs as 64-channel heads and keeps the diagonal blocks.  Summaries and
    outputs of the paired and the one-head-per-wave launch, each against the
    oracle; the two launches agree bit for bit (same products, same order)."""
    p = small_problem(case)
    q, k, v, W = synth.make_inputs(p, seed=26)
    ref = oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)
    rS, rz, _, _ = oracle.summaries(k, v, W, p.grid, p.block)
    run = Run(p, q, k, v, W)
    got = {}
    for flag in ("1", "0"):
        out = to_host64(run.forward(mh.MHLA_PATH_3KERNEL | (0 if flag == "1" else mh.MHLA_VARIANT_NO_PAIR_HEADS)))
        S, z, _, _ = run.workspace()
        e_out, e_s, e_z = rel_err(out, ref), rel_err(S, rS), rel_err(z, rz)
        say(f"  {p.name} pair={flag}: out {e_out:.2e} S {e_s:.2e} z {e_z:.2e}")
        assert np.isfinite(out).all()
        assert e_out <= TOL[p.dtype] and e_s <= 1e-2 and e_z <= 1e-2
        got[flag] = (out, S, z)
    for a, b in zip(got["1"], got["0"]):
        assert np.array_equal(a, b)


APPLY_CASES = [
    ("apply-d64-T256-H3", 1, 3, 64, (64, 64), (16, 16), BF, 1.0),        # two heads per workgroup: one slot idle
    ("apply-d32-T64-H5", 2, 5, 32, (32, 32), (8, 8), BF, 1.0),           # one wave per head, odd head count
    ("apply-d64-T200", 1, 2, 64, (20, 40), (10, 20), BF, 1.0),           # ragged last token group
    ("apply-d64-parts-empty", 1, 2, 64, (40, 52), (20, 26), BF, 1.0),    # 8 token parts, the last one empty
]


@pytest.mark.parametrize("case", APPLY_CASES, ids=lambda c: c[0])
def test_apply_operand_kernels(case):
    """query_apply with St_i, zt_i operands staged once per head in LDS (the
    default at d <= 64 with several waves per head, and at d = 32) and with
    each wave's own register copy (MHLA_VARIANT_APPLY_REGS): both against
    the oracle, and equal bit for bit (same operands, same products)."""
    p = small_problem(case)
    q, k, v, W = synth.make_inputs(p, seed=27)
    ref = oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)
    run = Run(p, q, k, v, W)
    outs = []
    for flag in (0, mh.MHLA_VARIANT_APPLY_REGS):
        out = run.forward(mh.MHLA_PATH_3KERNEL | flag)
        err = rel_err(to_host64(out), ref)
        say(f"  {p.name} variant={flag:#x}: max|d|/max|ref| = {err:.3e}")
        assert err <= TOL[p.dtype]
        outs.append(out.clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def token_parts(B, H, M, T, limit_sources):
    """Token parts of the bf16 3-kernel forward (the rule documented with
    mhla_workspace_bytes): doubled while B*M*H*parts < 1536, parts of at least
    64 tokens and, for the summaries, M*parts <= 256."""
    p = 1
    while B * M * H * p < 1536 and (not limit_sources or M * p * 2 <= 256) and p * 2 * 64 <= T:
        p *= 2
    return p


PART_CASES = [
    ("parts-d64-M16", 1, 6, 64, (128, 128), (32, 32), BF, 1.0),      # 16 parts of 64 tokens
    ("parts-d32-M4-3d", 1, 3, 32, (4, 32, 32), (4, 16, 16), BF, 1.0),  # odd H (no head pairs), 3D blocks
    ("parts-d128-M1", 1, 2, 128, (20, 40), (20, 40), BF, 1.0),       # one block, 25 token steps in 4 parts
    ("parts-d64-ragged", 1, 2, 64, (50, 60), (25, 30), BF, 1.0),     # rows of 30 tokens, ragged last step
    ("parts-d64-B2", 2, 3, 64, (64, 64), (32, 32), BF, 1.0),          # two batch items, 16 parts
]


@pytest.mark.parametrize("case", PART_CASES, ids=lambda c: c[0])
def test_token_parts(case):
    """Few blocks: the summary kernel sums each block's tokens in parts (one
    partial record per part), the mixing kernel contracts the partial records
    with W's columns repeated, the apply kernel splits each block's tokens.
    Every output against the oracle; the partial records of each block summed
    against the oracle's S and z."""
    p = small_problem(case)
    B, H, d, M, T = p.batch, p.heads, p.head_dim, p.n_blocks, p.n_tokens // p.n_blocks
    tp = token_parts(B, H, M, T, True)
    assert tp > 1
    q, k, v, W = synth.make_inputs(p, seed=27)
    ref = oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)
    run = Run(p, q, k, v, W)
    out_t = run.forward()
    out = to_host64(out_t)
    err = rel_err(out, ref)
    say(f"  {p.name} (summary parts {tp}, apply parts {token_parts(B, H, M, T, False)}): max|d|/max|ref| = {err:.3e}")
    assert np.isfinite(out).all()
    assert err <= TOL[p.dtype]
    rec = d * d + d
    raw = run.ws.cpu().numpy()[: 2 * B * H * M * tp * rec].view(np.uint16)
    parts = synth.bf16_to_f32(raw).astype(np.float64).reshape(B * H, M, tp, rec).sum(axis=2)
    S = parts[:, :, : d * d].reshape(B * H, M, d, d).transpose(0, 1, 3, 2)
    z = parts[:, :, d * d:]
    rS, rz, _, _ = oracle.summaries(k, v, W, p.grid, p.block)
    es, ez = rel_err(S, rS), rel_err(z, rz)
    say(f"  {p.name} summed partial records: S {es:.2e} z {ez:.2e}")
    assert es <= 1e-2 and ez <= 1e-2
    # deterministic: a second call is bitwise equal
    first = out_t.clone()
    out2 = run.forward()
    assert torch.equal(out2.view(torch.int16), first.view(torch.int16))


@pytest.mark.parametrize("cfg_index", [1, 2, 3, 4])
def test_full_workloads_all_outputs(cfg_index):
    """Full-size workload in the benchmark's launch configuration: every output
    of every (b, h) pair against the oracle, as one max|d|/max|ref| over the
    whole output, for the 3-kernel and the fused path; the 3-kernel output is
    bitwise equal over a second call."""
    p = synth.CONFIGS[cfg_index]
    q, k, v, W = synth.make_inputs(p, seed=cfg_index)
    ref = oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)
    run = Run(p, q, k, v, W)
    out = run.forward()
    got = to_host64(out)
    assert np.isfinite(got).all()
    err = rel_err(got, ref)
    pair_err = np.abs(got - ref).max(axis=(1, 3)) / np.abs(ref).max()   # [B, H]
    worst = np.unravel_index(int(np.argmax(pair_err)), pair_err.shape)
    say(f"  {p.name} 3kernel: max|d|/max|ref| = {err:.3e} over {p.batch * p.heads} pairs "
        f"(worst pair b={worst[0]} h={worst[1]})")
    assert err <= TOL[p.dtype]
    # determinism of the whole output over a second call
    out2 = run.forward()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    del out2
    got_f = to_host64(run.forward(mh.MHLA_PATH_FUSED))
    err_f = rel_err(got_f, ref)
    say(f"  {p.name} fused: max|d|/max|ref| = {err_f:.3e}")
    assert np.isfinite(got_f).all() and err_f <= TOL[p.dtype]


@pytest.mark.parametrize("w_kind", ["identity", "ones", "local", "linear", "cos", "exp", "gaussian-dmax"])
@pytest.mark.parametrize("path", [mh.MHLA_PATH_3KERNEL, mh.MHLA_PATH_FUSED], ids=["3kernel", "fused"])
@pytest.mark.parametrize("shape", [((64, 64), (8, 8)), ((64, 64), (2, 2))], ids=["M64", "M1024"])
def test_special_coefficient_matrices(w_kind, path, shape):
    """W = I (per-block attention), W = 1/M (global attention), sparse local W,
    and the module's linear, cos, exp and max-distance Gaussian transforms."""
    grid, block = shape
    p = synth.Problem("special", 1, 2, 64 if block[0] == 8 else 32, grid, block)
    q, k, v, W = synth.make_inputs(p, seed=23, w_kind=w_kind)
    ref = oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)
    out = to_host64(Run(p, q, k, v, W).forward(path))
    err = rel_err(out, ref)
    say(f"  W={w_kind} path={path}: {err:.3e}")
    assert err <= 1e-2


def test_alloc_entry_point_matches_workspace_entry_point():
    p = synth.CONFIGS[1].with_(batch=2)
    q, k, v, W = synth.make_inputs(p, seed=24)
    run = Run(p, q, k, v, W)
    a = run.forward()
    b = torch.empty_like(a)
    say("  [gpu] mhla_forward (stream-ordered workspace)")
    st = mh.mhla_forward(run.q, run.k, run.v, run.W, run.g, run.b, b)
    assert st == mh.MHLA_OK
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_side_stream_and_stage_events():
    p = synth.CONFIGS[2]
    q, k, v, W = synth.make_inputs(p, seed=2)
    run = Run(p, q, k, v, W)
    ref = run.forward()
    s = torch.cuda.Stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    with torch.cuda.stream(s):
        for e in ev:
            e.record(s)
        out = torch.empty_like(ref)
        say("  [gpu] mhla_forward_ex on a side stream with stage events")
        st = mh.mhla_forward_ex(run.q, run.k, run.v, run.W, run.g, run.b, out, run.ws, run.ws_bytes,
                                mh.MHLA_PATH_3KERNEL, ev, s)
        assert st == mh.MHLA_OK
    s.synchronize()
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
    say(f"  stage ms: {times}")
    assert all(t > 0 for t in times)


def test_injected_allocation_failure_enqueues_nothing(monkeypatch):
    """MHLA_FAIL_ALLOC=1: mhla_forward returns MHLA_ERR_ALLOC and the output
    keeps its contents (nothing ran); without it the same call succeeds."""
    p = synth.Problem("fail-alloc", 1, 2, 64, (32, 32), (8, 8))
    q, k, v, W = synth.make_inputs(p, seed=28)
    run = Run(p, q, k, v, W)
    out = torch.full_like(run.q, 7.0)
    monkeypatch.setenv("MHLA_FAIL_ALLOC", "1")
    say("  [gpu] mhla_forward with MHLA_FAIL_ALLOC=1")
    assert mh.mhla_forward(run.q, run.k, run.v, run.W, run.g, run.b, out) == mh.MHLA_ERR_ALLOC
    torch.cuda.synchronize()
    assert (out == 7.0).all().item()
    monkeypatch.delenv("MHLA_FAIL_ALLOC")
    assert mh.mhla_forward(run.q, run.k, run.v, run.W, run.g, run.b, out) == mh.MHLA_OK
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), run.forward().view(torch.int16))


def test_empty_problem_on_gpu():
    g = mh.make_grid(0, 6, 64, mh.MHLA_BF16, (256, 256))
    x = torch.empty(0, 65536, 6, 64, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    st = mh.mhla_forward(x, x, x, torch.empty(256, 256, device="cuda"), g, mh.make_block((16, 16)), y)
    torch.cuda.synchronize()
    assert st == mh.MHLA_OK
