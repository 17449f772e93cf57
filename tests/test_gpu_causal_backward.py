"""Gradients through the causal chunkwise form (mhla_causal_backward) against
the float64 oracle's (oracle.backward_causal), through the C ABI.

Bar: max|d| / max|ref| <= 1e-2 for each of dq, dk, dv and dW with bf16
inputs and outputs, 1e-5 with fp32 (the forward's bars).  The kernels compute
in fp32 either way; the fp32 cases use the nonnegative local prior for W, so
no causal denominator cancels (with a signed W the fp32 rounding of a
denominator is amplified by its cancellation, and the 1e-5 bar would measure
W's conditioning rather than the kernels).  Every element is compared,
including a 65536-token sequence in chunks of 256.
"""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_block_amd as mh
from token_level_head_block_amd import synth

from conditioning import causal_denominators
from gpu_util import Run, rel_err, say, to_host64

pytestmark = pytest.mark.gpu

BF = synth.BF16
F32 = synth.F32
TOL = {BF: 1e-2, F32: 1e-5}

# name, B, H, d, grid, block, dtype, W kind (chunks are contiguous runs of raster indices)
CASES = [
    ("cbwd-d64-T64", 2, 3, 64, (1, 1024), (1, 64), BF, "gaussian"),
    ("cbwd-d32-T15", 1, 3, 32, (1, 240), (1, 15), BF, "gaussian"),
    ("cbwd-d32-T1", 1, 1, 32, (1, 40), (1, 1), BF, "gaussian"),
    ("cbwd-d64-M1", 1, 2, 64, (1, 200), (1, 200), BF, "gaussian"),
    ("cbwd-rows-2d", 1, 2, 32, (12, 20), (3, 20), BF, "gaussian"),
    ("cbwd-frames-3d", 1, 2, 64, (4, 6, 8), (1, 6, 8), BF, "gaussian"),
    ("cbwd-d128-T40", 2, 1, 128, (1, 200), (1, 40), BF, "gaussian"),
    ("cbwd-d128-T256", 1, 2, 128, (1, 1024), (1, 256), BF, "gaussian"),
    # long chunks on the matrix-core path (129 chunks: no sub-chunks): five
    # 128-token query tiles per chunk, the last one ragged
    ("cbwd-d32-T520-M129", 1, 1, 32, (1, 129 * 520), (1, 520), BF, "gaussian"),
    # 144 chunks of one pair: the transposed mixing and a single dW split in one launch
    ("cbwd-d32-M144-one-split", 1, 1, 32, (1, 144 * 8), (1, 8), BF, "gaussian"),
    ("cbwd-d64-M144-T16", 1, 1, 64, (1, 144 * 16), (1, 16), BF, "gaussian"),
    ("cbwd-f32-d32-T16", 1, 2, 32, (1, 256), (1, 16), F32, "local"),
    ("cbwd-f32-d64-T100", 2, 1, 64, (1, 400), (1, 100), F32, "local"),
    ("cbwd-f32-d128-T33", 1, 1, 128, (1, 99), (1, 33), F32, "local"),
    ("cbwd-f32-frames-3d", 1, 2, 64, (3, 4, 8), (1, 4, 8), F32, "local"),
    ("cbwd-f32-d64-M1", 1, 1, 64, (1, 64), (1, 64), F32, "local"),
]


def upstream(p, seed):
    g = np.random.default_rng(seed).standard_normal((p.batch, p.n_tokens, p.heads, p.head_dim)).astype(np.float32)
    return synth.bf16_bits(g) if p.dtype == BF else g


def check(p, q, k, v, W, seed):
    g = upstream(p, seed)
    ref = oracle.backward_causal(q, k, v, W, g, p.grid, p.block, eps=p.eps)
    run = Run(p, q, k, v, W)
    got = run.backward(g, causal=True)
    for name, a, r in zip(("dq", "dk", "dv", "dW"), got, ref):
        a = to_host64(a)
        assert np.isfinite(a).all(), name
        if name == "dW" and p.n_blocks == 1:
            # One chunk: o depends on W only through eps, so dW is a difference of
            # terms of size sum|g . o| / |W| that cancel to O(eps); its error is
            # measured against that size.
            o = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
            scale = float(np.sum(np.abs(oracle.decode(g) * o))) / abs(float(W[0, 0]))
            e = float(np.max(np.abs(a - r))) / scale
            say(f"  {p.name} dW (M = 1): max|d| / (sum|g.o| / |W|) = {e:.3e}")
        else:
            e = rel_err(a, r)
            say(f"  {p.name} {name}: max|d|/max|ref| = {e:.3e}")
        assert e <= TOL[p.dtype], name
        if name == "dW":
            assert np.all(a[np.triu_indices(p.n_blocks, 1)] == 0.0)   # later chunks get no gradient
    return run, g, got


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_causal_backward_small(case):
    name, B, H, d, grid, block, dt, wk = case
    p = synth.Problem(name, B, H, d, grid, block, dtype=dt)
    q, k, v, W = synth.make_inputs(p, seed=71, w_kind=wk)
    check(p, q, k, v, W, seed=72)


def test_causal_backward_sequence_workload():
    """65536 tokens as one sequence in chunks of 256 (six heads, d = 64): every
    gradient element, and a second call is bitwise equal (deterministic dW)."""
    p = synth.Problem("cbwd-seq-65536-chunk256", 1, 6, 64, (1, 65536), (1, 256), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=73)
    run, g, got = check(p, q, k, v, W, seed=74)
    again = run.backward(g, causal=True)
    for a, b in zip(got, again):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_causal_backward_f32_signed_w():
    """fp32 gradients with a signed W (the distance prior plus a jitter of
    standard deviation 0.15, so that some coefficients are negative) whose
    partial row sums over earlier chunks stay away from zero: every element
    against the fp32 bar; the denominators' cancellation factor is printed."""
    p = synth.Problem("cbwd-f32-signed", 1, 2, 64, (1, 640), (1, 80), dtype=F32)
    q, k, v, _ = synth.make_inputs(p, seed=77)
    M = p.n_blocks
    nb = [gx // bx for gx, bx in zip(p.grid, p.block)]
    W = (synth.distance_prior(nb, 3.0) + 0.15 * np.random.default_rng(78).standard_normal((M, M))).astype(np.float32)
    assert (np.tril(W) < 0).any()
    den, absden = causal_denominators(q, k, W, p.grid, p.block, p.eps)
    kappa = absden / np.abs(den)
    say(f"  {p.name}: {int((np.tril(W) < 0).sum())} negative coefficients on or below the diagonal, "
        f"kappa max {kappa.max():.2f}")
    assert kappa.max() < 4.0
    check(p, q, k, v, W, seed=79)


def test_causal_backward_ignores_later_coefficients():
    """W[i, j] with j > i is never read: changing it changes no gradient bit."""
    p = synth.Problem("cbwd-upper", 1, 2, 64, (1, 512), (1, 64), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=75)
    g = upstream(p, 76)
    base = Run(p, q, k, v, W).backward(g, causal=True)
    W2 = W.copy()
    W2[np.triu_indices(W.shape[0], 1)] = 7.0
    other = Run(p, q, k, v, W2).backward(g, causal=True)
    for a, b in zip(base, other):
        assert torch.equal(a, b)

