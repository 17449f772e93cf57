"""The causal chunkwise path (MHLA_PATH_CAUSAL) against the float64 oracle's
causal form, through the C ABI.  Bar: max|d| / max|ref| <= 1e-2 (bf16) on
every output, including sequences whose signed W makes the partial row sums
over earlier chunks cancel (the cancellation factor of each query's
denominator is printed as a diagnostic)."""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_block_amd as mh
from token_level_head_block_amd import synth

from conditioning import BF16_U, causal_denominators
from gpu_util import Run, TOL, rel_err, say, to_host64

pytestmark = pytest.mark.gpu

BF = synth.BF16

# name, B, H, d, grid, block, std  (blocks are contiguous runs of raster indices)
CASES = [
    ("causal-1d-T64", 2, 3, 64, (1, 1024), (1, 64), 1.0),
    ("causal-1d-T256", 1, 2, 64, (1, 2048), (1, 256), 1.0),
    ("causal-1d-T15-d32", 1, 3, 32, (1, 240), (1, 15), 1.0),
    ("causal-1d-T1", 1, 1, 32, (1, 40), (1, 1), 1.0),
    ("causal-1d-M1", 1, 2, 64, (1, 200), (1, 200), 1.0),
    ("causal-rows-2d", 1, 2, 32, (12, 20), (3, 20), 0.5),
    ("causal-frames-3d", 1, 2, 64, (4, 6, 8), (1, 6, 8), 1.0),
    ("causal-d128-T256", 1, 2, 128, (1, 1024), (1, 256), 1.0),
    ("causal-d128-T40", 2, 1, 128, (1, 200), (1, 40), 1.0),
    ("causal-d128-M1", 1, 1, 128, (1, 300), (1, 300), 1.0),
    # long chunks run on sub-chunks of >= 256 tokens (W between sub-chunks from their chunks)
    ("causal-1d-T2048-sub", 1, 2, 64, (1, 8192), (1, 2048), 1.0),
    ("causal-rows-2d-sub", 1, 2, 32, (64, 64), (16, 64), 1.0),
    ("causal-frames-3d-sub", 1, 2, 64, (4, 32, 32), (1, 32, 32), 1.0),
    ("causal-d128-sub", 1, 2, 128, (1, 2048), (1, 1024), 1.0),
    ("causal-1d-T1000-sub", 1, 1, 64, (1, 3000), (1, 1000), 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_causal_small(case):
    name, B, H, d, grid, block, std = case
    p = synth.Problem(name, B, H, d, grid, block, dtype=BF, std=std)
    q, k, v, W = synth.make_inputs(p, seed=61)
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    out = to_host64(Run(p, q, k, v, W).forward(mh.MHLA_PATH_CAUSAL))
    err = rel_err(out, ref)
    say(f"  {name}: max|d|/max|ref| = {err:.3e}")
    assert np.isfinite(out).all()
    assert err <= TOL[BF]


# fp32 problems (bar 1e-5): name, B, H, d, grid, block
F32_CASES = [
    ("causal-f32-d32-T16", 1, 2, 32, (1, 256), (1, 16)),
    ("causal-f32-d64-T100", 2, 1, 64, (1, 400), (1, 100)),
    ("causal-f32-d128-M1", 1, 1, 128, (1, 96), (1, 96)),
    ("causal-f32-frames-3d", 1, 2, 64, (3, 4, 8), (1, 4, 8)),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: c[0])
def test_causal_f32(case):
    name, B, H, d, grid, block = case
    p = synth.Problem(name, B, H, d, grid, block, dtype=synth.F32)
    q, k, v, W = synth.make_inputs(p, seed=66)
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    out = to_host64(Run(p, q, k, v, W).forward(mh.MHLA_PATH_CAUSAL))
    err = rel_err(out, ref)
    say(f"  {name}: max|d|/max|ref| = {err:.3e}")
    assert err <= TOL[synth.F32]


def check_every_output(p, q, k, v, W, out, ref, kappa_max=16.0):
    """The bf16 bar on every output.  Diagnostic: the cancellation factor
    kappa of each query's causal denominator, and the error of the tokens above
    kappa_max against a rounding bound scaled by it (4 u kappa (max|v| + |o_n|),
    u = 2^-8), which the bar no longer needs."""
    den, absden = causal_denominators(q, k, W, p.grid, p.block, p.eps)
    kappa = absden / np.abs(den)                              # [B, N, H]
    dev = np.abs(out - ref).max(axis=3)
    scale = np.abs(ref).max()
    ill = kappa > kappa_max
    vmax = np.abs(oracle.decode(v)).max(axis=(1, 3))          # [B, H]
    bound = 4 * BF16_U * kappa * (vmax[:, None, :] + np.abs(ref).max(axis=3))
    err = dev.max() / scale
    say(f"  {p.name}: max|d|/max|ref| = {err:.3e}; kappa max {kappa.max():.1f}, {ill.mean():.4f} of tokens "
        f"above {kappa_max} (their max|d|/max|ref| {dev[ill].max() / scale if ill.any() else 0.0:.3e}), "
        f"worst d / bound = {(dev / bound).max():.3f}")
    assert np.isfinite(out).all()
    assert err <= TOL[BF]


def test_causal_sequence_workload():
    """65536 tokens as one sequence in chunks of 256 (the metric workload's size),
    every output of every pair against the bf16 bar; a second call is bitwise
    equal.  This signed W has partial row sums that cancel up to 145-fold; the
    mixing takes W as a bf16 high and low part, so the bar holds everywhere."""
    p = synth.Problem("seq-65536-chunk256", 1, 6, 64, (1, 65536), (1, 256), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=62)
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    run = Run(p, q, k, v, W)
    out = run.forward(mh.MHLA_PATH_CAUSAL)
    check_every_output(p, q, k, v, W, to_host64(out), ref)
    again = run.forward(mh.MHLA_PATH_CAUSAL)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))


def test_causal_sequence_d128():
    """16384 tokens in chunks of 256 at d = 128 (four heads): every output against the bf16 bar."""
    p = synth.Problem("seq-16384-chunk256-d128", 1, 4, 128, (1, 16384), (1, 256), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=65)
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    out = Run(p, q, k, v, W).forward(mh.MHLA_PATH_CAUSAL)
    check_every_output(p, q, k, v, W, to_host64(out), ref)


def test_causal_sequence_long_chunks_signed_w():
    """65536 tokens in 16 chunks of 4096 (the rows of a 256 x 256 grid, 16 per
    chunk), run as sub-chunks whose coefficients come from their chunks: every
    output against the bf16 bar with the jittered W."""
    p = synth.Problem("rows-65536-chunk4096", 1, 6, 64, (256, 256), (16, 256), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=67)
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    out = Run(p, q, k, v, W).forward(mh.MHLA_PATH_CAUSAL)
    check_every_output(p, q, k, v, W, to_host64(out), ref)


def test_causal_sequence_workload_local_w():
    """Same shape with the nonnegative local prior (kappa = 1): the bf16 bar on every output."""
    p = synth.Problem("seq-65536-chunk256-local", 1, 6, 64, (1, 65536), (1, 256), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=64, w_kind="local")
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    out = to_host64(Run(p, q, k, v, W).forward(mh.MHLA_PATH_CAUSAL))
    err = rel_err(out, ref)
    say(f"  {p.name}: max|d|/max|ref| = {err:.3e}")
    assert err <= TOL[BF]


def test_causal_ignores_later_coefficients_and_tokens():
    p = synth.Problem("causal-check", 1, 2, 64, (1, 512), (1, 64), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=63)
    base = Run(p, q, k, v, W).forward(mh.MHLA_PATH_CAUSAL)
    W2 = W.copy()
    W2[np.triu_indices(W.shape[0], 1)] = 3.0
    k2, v2 = k.copy(), v.copy()
    k2[:, -1] = synth.bf16_bits(np.full(k2[:, -1].shape, 2.0, dtype=np.float32))
    v2[:, -1] = synth.bf16_bits(np.full(v2[:, -1].shape, -5.0, dtype=np.float32))
    out = Run(p, q, k2, v2, W2).forward(mh.MHLA_PATH_CAUSAL)
    assert torch.equal(out[:, :-1].contiguous().view(torch.int16), base[:, :-1].contiguous().view(torch.int16))
