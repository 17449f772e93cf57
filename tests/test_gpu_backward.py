"""Gradients from the HIP backward pass against the float64 CPU oracle's,
through the C ABI.

Bar: max|d| / max|ref| <= 1e-2 for each of dq, dk, dv and dW with bf16
inputs and outputs, the forward's bf16 bar applied to each gradient; 1e-5,
the forward's fp32 bar, with fp32 inputs.  bf16 problems with d = 32 or 64
run on the MFMA kernels, the others (fp32, d = 128) on the general fp32 path.
Small problems compare every element; the full workloads compare every
element too (the oracle finishes them in seconds).
"""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_block_amd as mh
from token_level_head_block_amd import synth

from gpu_util import Run, rel_err, say, to_host64

pytestmark = pytest.mark.gpu

BF = synth.BF16
F32 = synth.F32
TOL = {BF: 1e-2, F32: 1e-5}

# name, B, H, d, grid, block, std
SMALL = [
    ("bwd-d64-M24", 2, 3, 64, (32, 48), (8, 8), 1.0),
    ("bwd-d32-T15", 1, 2, 32, (12, 20), (3, 5), 1.0),
    ("bwd-d64-3d", 1, 2, 64, (4, 12, 12), (2, 3, 4), 1.0),
    ("bwd-d64-T25", 1, 2, 64, (40, 40), (5, 5), 1.0),
    ("bwd-d64-M1", 1, 2, 64, (7, 9), (7, 9), 1.0),
    ("bwd-d32-T1", 1, 1, 32, (6, 6), (1, 1), 1.0),
    ("bwd-d32-M360", 1, 1, 32, (36, 40), (2, 2), 1.0),
    ("bwd-d32-H9-M180", 1, 9, 32, (30, 24), (2, 2), 0.5),
    ("bwd-d64-T256-M160", 1, 2, 64, (160, 256), (16, 16), 1.0),
    ("bwd-d64-B2-M196", 2, 3, 64, (56, 56), (4, 4), 1.0),
    # one pair, 144 blocks: the dW product runs as a single split beside the mixing
    ("bwd-d32-M144-one-split", 1, 1, 32, (48, 48), (4, 4), 1.0),
    # 64 pairs x 17 column tiles: two column tiles per mixing workgroup, the last one alone
    ("bwd-d32-H64-M144-two-tiles", 1, 64, 32, (48, 48), (4, 4), 1.0),
    # few blocks of many tokens: the key/value side runs in token parts
    ("bwd-d64-M4-parts", 1, 2, 64, (32, 32), (16, 16), 1.0),
    ("bwd-d32-M4-parts", 1, 4, 32, (32, 48), (16, 24), 1.0),
    ("bwd-d64-B2-parts", 2, 3, 64, (64, 64), (32, 32), 1.0),
    # enough (b, block, head) tasks for whole blocks per wave on the query side
    # (operand copies in LDS), 9 token groups with the last of 8 tokens
    ("bwd-d64-T136-one-part", 4, 6, 64, (64, 136), (8, 17), 1.0),
]

# the general path: name, B, H, d, grid, block, dtype
GENERAL = [
    ("bwd-f32-d32-M16", 1, 1, 32, (16, 16), (4, 4), F32),
    ("bwd-f32-d64-3d", 2, 2, 64, (4, 8, 8), (2, 4, 4), F32),
    ("bwd-f32-d128-T25", 1, 2, 128, (10, 10), (5, 5), F32),
    ("bwd-bf16-d128-M16", 1, 2, 128, (16, 16), (4, 4), BF),
    ("bwd-bf16-d128-T6-M42", 2, 1, 128, (14, 18), (2, 3), BF),
    ("bwd-bf16-d128-M1", 1, 1, 128, (8, 9), (8, 9), BF),
]


def upstream(p, seed):
    g = np.random.default_rng(seed).standard_normal((p.batch, p.n_tokens, p.heads, p.head_dim)).astype(np.float32)
    return synth.bf16_bits(g) if p.dtype == BF else g


def check(p, seed, variant=0):
    q, k, v, W = synth.make_inputs(p, seed=seed)
    g = upstream(p, seed + 1000)
    ref = oracle.backward(q, k, v, W, g, p.grid, p.block, eps=p.eps)
    run = Run(p, q, k, v, W)
    got = run.backward(g, variant=variant)
    for name, a, r in zip(("dq", "dk", "dv", "dW"), got, ref):
        a = to_host64(a)
        assert np.isfinite(a).all(), name
        if name == "dW" and p.n_blocks == 1:
            # One block: o depends on W only through eps, so dW = sum(g . o) eps / (W den)
            # is a difference of terms of size sum|g . o| / |W| that cancel to O(eps).
            # Its error is measured against that size.
            o = oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)
            scale = float(np.sum(np.abs(oracle.decode(g) * o))) / abs(float(W[0, 0]))
            e = float(np.max(np.abs(a - r))) / scale
            say(f"  {p.name} dW (M = 1): max|d| / (sum|g.o| / |W|) = {e:.3e}")
        else:
            e = rel_err(a, r)
            say(f"  {p.name} {name}: max|d|/max|ref| = {e:.3e}")
        assert e <= TOL[p.dtype], name
    return run, g, got


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_backward_small_problems(case):
    name, B, H, d, grid, block, std = case
    check(synth.Problem(name, B, H, d, grid, block, dtype=BF, std=std), seed=41)


@pytest.mark.parametrize("case", [("bwd-pairs-d32", 2, 4, 32, (16, 24), (4, 6), 1.0),
                                  ("bwd-pairs-d32-parts", 1, 6, 32, (32, 32), (16, 16), 0.5)],
                         ids=lambda c: c[0])
def test_backward_d32_head_pairs(case):
    """head_dim 32 with an even head count: the key/value side reads head pairs
    as heads of 64 channels with block-diagonal dS.  Each launch against the
    oracle, and the paired and one-head-per-wave launches bit for bit (the
    zero blocks add exact zeros to the same products)."""
    name, B, H, d, grid, block, std = case
    p = synth.Problem(name, B, H, d, grid, block, dtype=BF, std=std)
    outs = {}
    for flag in ("1", "0"):
        run, g, got = check(p, seed=46, variant=0 if flag == "1" else mh.MHLA_VARIANT_NO_PAIR_HEADS)
        outs[flag] = got
    for a, b in zip(outs["1"], outs["0"]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("case", GENERAL, ids=lambda c: c[0])
def test_backward_general_path(case):
    name, B, H, d, grid, block, dt = case
    check(synth.Problem(name, B, H, d, grid, block, dtype=dt), seed=45)


@pytest.mark.parametrize("cfg_index", [0, 1, 2, 3, 4])
def test_backward_full_workloads(cfg_index):
    """Every gradient element at full size; a second call is bitwise equal."""
    p = synth.CONFIGS[cfg_index]
    run, g, got = check(p, seed=cfg_index)
    again = run.backward(g)
    for a, b in zip(got, again):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_backward_stream_allocated_workspace_matches():
    p = synth.Problem("bwd-ws", 1, 3, 64, (32, 32), (8, 8), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=43)
    g = upstream(p, 44)
    run = Run(p, q, k, v, W)
    a = run.backward(g)
    b = run.backward(g, ws=False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_empty_problem_zeroes_dw():
    g = mh.make_grid(0, 6, 64, mh.MHLA_BF16, (32, 32))
    b = mh.make_block((8, 8))
    x = torch.empty(0, 1024, 6, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.ones(16, 16, device="cuda")
    dW = torch.full((16, 16), 7.0, device="cuda")
    say("  [gpu] mhla_backward on an empty problem")
    st = mh.mhla_backward(x, x, x, W, x, g, b, torch.empty_like(x), torch.empty_like(x), torch.empty_like(x), dW)
    torch.cuda.synchronize()
    assert st == mh.MHLA_OK
    assert (dW == 0).all().item()
