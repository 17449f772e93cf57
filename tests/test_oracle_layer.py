"""Pins of the layer oracle (oracle/layer.py) against what is fixed outside it:
torch's own LayerNorm, RMSNorm, linear and grouped-convolution routines, the
C oracle of the core, the N x N definition of the core with either feature
map, and closed forms of the LePE convolution.  The module followed is the
171host.com repost's section 七 (class MHLA, ``forward``)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import layer as L
from token_level_head_block_amd import synth


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((3, 7, 48)) * 2 + 0.5
    w, b = rng.standard_normal(48), rng.standard_normal(48)
    ref = F.layer_norm(torch.from_numpy(X), (48,), torch.from_numpy(w), torch.from_numpy(b), eps=1e-5).numpy()
    assert rel_err(L.layer_norm(X, w, b, 1e-5), ref) < 1e-12
    # unit weight, zero bias: every token has mean 0 and mean square var / (var + eps)
    Y = L.layer_norm(X, np.ones(48), np.zeros(48), 1e-5)
    var = X.var(axis=-1)
    np.testing.assert_allclose(Y.mean(axis=-1), 0.0, atol=1e-13)
    np.testing.assert_allclose((Y * Y).mean(axis=-1), var / (var + 1e-5), rtol=1e-12)


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((2, 5, 32))
    w = rng.standard_normal(32)
    ref = F.rms_norm(torch.from_numpy(X), (32,), torch.from_numpy(w), eps=1e-6).numpy()
    assert rel_err(L.rms_norm(X, w, 1e-6), ref) < 1e-12


def test_phi_variants():
    x = np.array([-2.0, -0.5, 0.0, 0.5, 3.0])
    np.testing.assert_allclose(L.phi(x, L.PHI_ELU1), [np.exp(-2.0), np.exp(-0.5), 1.0, 1.5, 4.0], rtol=1e-15)
    np.testing.assert_allclose(L.phi(x, L.PHI_RELU_EPS, 1e-3), [1e-3, 1e-3, 1e-3, 0.501, 3.001], rtol=1e-15)
    with pytest.raises(ValueError):
        L.phi(x, "softplus")


def test_lepe_matches_torch_depthwise_conv():
    rng = np.random.default_rng(3)
    B, Y, X, C = 2, 9, 7, 6
    V = rng.standard_normal((B, Y, X, C))
    w, b = rng.standard_normal((C, 5, 5)), rng.standard_normal(C)
    ref = F.conv2d(torch.from_numpy(V).permute(0, 3, 1, 2), torch.from_numpy(w)[:, None], torch.from_numpy(b),
                   padding=2, groups=C).permute(0, 2, 3, 1).numpy()
    assert rel_err(L.lepe(V, w, b), ref) < 1e-12


def test_lepe_closed_forms():
    rng = np.random.default_rng(4)
    V = rng.standard_normal((1, 6, 8, 3))
    w = np.zeros((3, 5, 5))
    w[:, 2, 2] = 1.0
    np.testing.assert_array_equal(L.lepe(V, w), V)          # centre tap: identity
    w = np.zeros((3, 5, 5))
    w[:, 2, 4] = 1.0                                         # reads the token two to the right
    out = L.lepe(V, w)
    np.testing.assert_array_equal(out[:, :, :-2], V[:, :, 2:])
    np.testing.assert_array_equal(out[:, :, -2:], 0.0)       # zero padding at the border


@pytest.mark.parametrize("shape", [((1, 2, 8, (8, 8), (4, 4))), ((2, 1, 4, (2, 6, 4), (1, 3, 2)))])
def test_core_elu_matches_c_oracle(oracle_lib, shape):
    B, H, d, grid, block = shape
    p = synth.Problem("c", B, H, d, grid, block, dtype=synth.F32)
    q, k, v, W = synth.make_inputs(p, seed=5)
    got = L.core(*(oracle.decode(t) for t in (q, k, v)), W, grid, block, 1e-3, L.PHI_ELU1)
    ref = oracle.forward(q, k, v, W, grid, block, eps=1e-3)
    assert rel_err(got, ref) < 1e-12


def test_core_relu_matches_nxn_definition():
    p = synth.Problem("c", 1, 2, 8, (6, 8), (2, 4), dtype=synth.F32)
    q, k, v, W = synth.make_inputs(p, seed=6)
    Q, K, V = (oracle.decode(t) for t in (q, k, v))
    got = L.core(Q, K, V, W, p.grid, p.block, 1e-3, L.PHI_RELU_EPS, 1e-2)
    bid = oracle.token_blocks(p.grid, p.block)
    for h in range(p.heads):
        u = np.maximum(Q[0, :, h], 0) + 1e-2
        a = np.maximum(K[0, :, h], 0) + 1e-2
        A = W.astype(np.float64)[bid][:, bid] * (u @ a.T)
        ref = A @ V[0, :, h] / (A.sum(axis=1) + 1e-3)[:, None]
        assert rel_err(got[0, :, h], ref) < 1e-12


def torch_layer(x, W, p, P, kind, eps=1e-6):
    """The layer from torch's own routines, in float64, with the core as the
    materialised N x N attention."""
    X = torch.from_numpy(oracle.decode(x))
    t = lambda key: None if P.get(key) is None else torch.from_numpy(np.asarray(P[key], dtype=np.float64))
    tw = lambda key: torch.from_numpy(oracle.decode(P[key]))
    B, N, C = X.shape
    H, d = p.heads, p.head_dim
    xn = F.layer_norm(X, (C,), t("ln_w"), t("ln_b"), eps=1e-5)
    q, k, v = F.linear(xn, tw("w_qkv"), t("b_qkv")).split(C, dim=-1)
    if P.get("qn_w") is not None:
        q = F.rms_norm(q, (C,), t("qn_w"), eps=1e-6)
        k = F.rms_norm(k, (C,), t("kn_w"), eps=1e-6)
    fm = (lambda z: F.elu(z) + 1.0) if kind == L.PHI_ELU1 else (lambda z: F.relu(z) + 1e-6)
    bid = torch.from_numpy(oracle.token_blocks(p.grid, p.block))
    Wx = torch.from_numpy(W.astype(np.float64))[bid][:, bid]
    o = torch.empty(B, N, C, dtype=torch.float64)
    for b in range(B):
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            A = Wx * (fm(q[b, :, sl]) @ fm(k[b, :, sl]).T)
            o[b, :, sl] = A @ v[b, :, sl] / (A.sum(dim=1, keepdim=True) + eps)
    if P.get("lepe_w") is not None:
        img = v.reshape(B, p.grid[0], p.grid[1], C).permute(0, 3, 1, 2)
        o = o + F.conv2d(img, t("lepe_w")[:, None], t("lepe_b"), padding=2, groups=C).permute(0, 2, 3, 1).reshape(B, N, C)
    return F.linear(o, tw("w_out"), t("b_out")).numpy()


LAYER_CASES = [
    # name, B, H, d, grid, block, qk_norm, lepe, bias, phi
    ("plain", 1, 2, 8, (8, 8), (4, 4), False, True, True, L.PHI_ELU1),
    ("qknorm-relu", 2, 2, 8, (6, 4), (3, 2), True, True, True, L.PHI_RELU_EPS),
    ("no-lepe-no-bias", 1, 3, 4, (4, 8), (2, 4), False, False, False, L.PHI_ELU1),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: c[0])
def test_layer_matches_torch_composition(case):
    name, B, H, d, grid, block, qkn, lp, bias, kind = case
    p = synth.Problem(name, B, H, d, grid, block, dtype=synth.BF16)
    x, P, W = synth.make_layer_inputs(p, seed=7, qk_norm=qkn, lepe=lp, bias=bias)
    got = L.layer_forward(x, W, p.grid, p.block, p.heads, P, kind=kind)
    assert rel_err(got, torch_layer(x, W, p, P, kind)) < 1e-10


def test_layer_pins_catch_planted_mistakes():
    p = synth.Problem("plant", 1, 2, 8, (8, 8), (4, 4), dtype=synth.BF16)
    x, P, W = synth.make_layer_inputs(p, seed=8)
    ref = torch_layer(x, W, p, P, L.PHI_ELU1)
    run = lambda P_, **kw: L.layer_forward(x, W, p.grid, p.block, p.heads, P_, **kw)
    C = p.heads * p.head_dim
    flipped = dict(P, lepe_w=np.ascontiguousarray(P["lepe_w"][:, ::-1, ::-1]))      # convolution, not correlation
    wq = oracle.decode(P["w_qkv"])
    swapped = dict(P, w_qkv=synth.bf16_bits(np.concatenate([wq[C:2 * C], wq[:C], wq[2 * C:]]).astype(np.float32)))
    planted = {
        "flipped LePE kernel": run(flipped),
        "q and k projections swapped": run(swapped),
        "other feature map": run(P, kind=L.PHI_RELU_EPS),
        "no LayerNorm bias": run(dict(P, ln_b=np.zeros_like(P["ln_b"]))),
        "LePE dropped": run(dict(P, lepe_w=None)),
    }
    for name, out in planted.items():
        assert rel_err(out, ref) > 1e-3, name
