"""The layer around the core (mhla_layer_forward) against the float64 layer
oracle, every output, through the C ABI.  Bar: max|d| / max|ref| <= 1e-2
(bf16 activations and intermediates)."""
import numpy as np
import pytest
import torch

import token_level_head_block_amd as mh
from oracle import layer as L
from token_level_head_block_amd import synth

from gpu_util import LayerRun, TOL, rel_err, say, to_host64

pytestmark = pytest.mark.gpu

BF = synth.BF16
PHI = {mh.MHLA_PHI_ELU1: L.PHI_ELU1, mh.MHLA_PHI_RELU_EPS: L.PHI_RELU_EPS}

# name, B, H, d, grid, block, qk_norm, lepe, bias, phi
CASES = [
    ("layer-c64-ragged", 1, 2, 32, (16, 16), (4, 4), False, True, True, mh.MHLA_PHI_ELU1),
    ("layer-c96-qknorm-relu", 2, 3, 32, (12, 20), (3, 4), True, True, True, mh.MHLA_PHI_RELU_EPS),
    ("layer-3d-no-lepe", 1, 2, 64, (4, 8, 8), (2, 4, 4), False, False, False, mh.MHLA_PHI_ELU1),
    ("layer-d128", 1, 2, 128, (16, 16), (8, 8), False, True, True, mh.MHLA_PHI_RELU_EPS),
    ("layer-c384-rows", 2, 6, 64, (40, 36), (8, 12), True, True, False, mh.MHLA_PHI_ELU1),
    # 4 blocks of 256 tokens: the core runs with token parts (4 summary and 4 apply parts)
    ("layer-c64-token-parts", 1, 2, 32, (32, 32), (16, 16), False, True, True, mh.MHLA_PHI_ELU1),
    # relu feature map without q/k norm and 2C = 192: one projection tile holds
    # columns on both sides of the preimage boundary
    ("layer-c96-relu-split-tile", 1, 3, 32, (12, 16), (3, 4), False, True, True, mh.MHLA_PHI_RELU_EPS),
]


def check(p, x, P, W, phi, seed_note):
    ref = L.layer_forward(x, W, p.grid, p.block, p.heads, P, eps=p.eps, kind=PHI[phi])
    run = LayerRun(p, x, P, W)
    y = run.forward(phi)
    err = rel_err(to_host64(y), ref)
    say(f"  {p.name} {seed_note}: max|d|/max|ref| = {err:.3e}")
    assert np.isfinite(to_host64(y)).all()
    assert err <= TOL[BF]
    return run, y


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_layer_small(case):
    name, B, H, d, grid, block, qkn, lp, bias, phi = case
    p = synth.Problem(name, B, H, d, grid, block, dtype=BF)
    x, P, W = synth.make_layer_inputs(p, seed=71, qk_norm=qkn, lepe=lp, bias=bias)
    check(p, x, P, W, phi, "seed 71")


@pytest.mark.parametrize("phi", [mh.MHLA_PHI_ELU1, mh.MHLA_PHI_RELU_EPS])
def test_layer_metric_workload(phi):
    """The metric workload's shape (B=1, H=6, d=64, 256 x 256 grid, 16 x 16 blocks,
    C = 384) as a whole layer with LePE; a second call is bitwise equal."""
    p = synth.CONFIGS[2]
    x, P, W = synth.make_layer_inputs(p, seed=72)
    run, y = check(p, x, P, W, phi, "seed 72")
    again = run.forward(phi)
    assert torch.equal(y.view(torch.int16), again.view(torch.int16))


def test_layer_allocating_call_matches():
    p = synth.Problem("layer-alloc", 1, 2, 32, (16, 16), (4, 4), dtype=BF)
    x, P, W = synth.make_layer_inputs(p, seed=73)
    run = LayerRun(p, x, P, W)
    a = run.forward()
    b = run.forward(ws=False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
