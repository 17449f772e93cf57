"""Pins of the CPU oracle against what the method and mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
closed forms, textbook special cases (vanilla / per-block linear attention),
the rank statements of the method, algebraic invariants, and the materialised
N x N definition evaluated by independent numpy code.  The last group plants
plausible mistakes into oracle calls and checks that the pins catch them.

Method: MHLA (arXiv 2601.07832), paperlayer.ai summary sections 3 and 4;
171host.com repost sections 5 and 6.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from token_level_head_block_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def load_examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def example_inputs(ex, dtype=None):
    dt = dtype or ex["dtype"]
    shape = (1, len(ex["q"]), 1, ex["head_dim"])
    arrs = []
    for key in ("q", "k", "v"):
        x = np.array(ex[key], dtype=np.float32).reshape(shape)
        arrs.append(synth.bf16_bits(x) if dt == "bf16" else x)
    W = np.array(ex["W"], dtype=np.float32)
    expected = np.array([[eval(s, {"__builtins__": {}}, {"e": math.exp(-1.0)}) for s in row]
                         for row in ex["expected"]], dtype=np.float64)
    return arrs[0], arrs[1], arrs[2], W, expected


# ---------------------------------------------------------------- feature map

def test_phi_closed_forms(oracle_lib):
    # elu(x) + 1: both branches give 1 at x = 0; x + 1 above, exp(x) below.
    assert oracle.phi(0.0) == 1.0
    assert oracle.phi(1.0) == 2.0
    assert oracle.phi(-1.0) == pytest.approx(math.exp(-1.0), rel=1e-15)
    assert oracle.phi(-50.0) > 0.0
    xs = np.linspace(-6, 6, 241)
    ref = torch.nn.functional.elu(torch.tensor(xs, dtype=torch.float64)).numpy() + 1.0
    got = np.array([oracle.phi(x) for x in xs])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=0)   # elu uses expm1
    np.testing.assert_allclose(oracle.phi_np(xs), ref, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- geometry

@pytest.mark.parametrize("grid,block", [((16, 16), (4, 4)), ((6, 10), (3, 5)), ((4, 6, 8), (2, 3, 4)),
                                        ((16, 64, 64), (4, 8, 8)), ((5, 7), (5, 7)), ((3, 4), (1, 1))])
def test_geometry_c_matches_numpy(oracle_lib, grid, block):
    np.testing.assert_array_equal(oracle.token_blocks_c(grid, block), oracle.token_blocks(grid, block))


def test_geometry_2d_closed_form(oracle_lib):
    Y, X, by, bx = 12, 20, 3, 5
    bid = oracle.token_blocks_c((Y, X), (by, bx))
    for n in range(Y * X):
        y, x = divmod(n, X)
        assert bid[n] == (y // by) * (X // bx) + x // bx
    assert oracle.num_blocks((Y, X), (by, bx)) == (Y // by) * (X // bx)
    assert oracle.num_blocks((12, 20), (5, 5)) == -1       # not divisible: rejected


# ---------------------------------------------------------------- hand-worked examples

@pytest.mark.parametrize("ex", load_examples(), ids=lambda e: e["name"])
def test_hand_worked_examples(oracle_lib, ex):
    q, k, v, W, expected = example_inputs(ex)
    out = oracle.forward(q, k, v, W, ex["grid"], ex["block"], eps=ex["eps"])[0, :, 0, :]
    np.testing.assert_allclose(out, expected, rtol=1e-14, atol=1e-15)
    brute = oracle.bruteforce(q, k, v, W, ex["grid"], ex["block"], eps=ex["eps"])[0, :, 0, :]
    np.testing.assert_allclose(brute, expected, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- definition (N x N) vs blockwise

CASES = [
    # grid, block, B, H, d, dtype, std
    ((16, 16), (4, 4), 1, 1, 32, synth.F32, 1.0),        # the tiny fp32 workload
    ((12, 10), (3, 5), 2, 3, 8, synth.BF16, 1.0),        # ragged 15-token blocks
    ((4, 6, 8), (2, 3, 4), 1, 2, 16, synth.BF16, 0.5),   # 3D blocks
    ((8, 8), (8, 8), 1, 2, 4, synth.F32, 1.0),           # M = 1
    ((6, 6), (1, 1), 1, 1, 4, synth.BF16, 1.0),          # T = 1
    ((4, 32), (2, 8), 1, 1, 64, synth.BF16, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-d{c[4]}")
def test_blockwise_equals_bruteforce(oracle_lib, case):
    grid, block, B, H, d, dt, std = case
    p = synth.Problem("t", B, H, d, grid, block, dtype=dt, std=std)
    q, k, v, W = synth.make_inputs(p, seed=11)
    out = oracle.forward(q, k, v, W, grid, block, eps=1e-6)
    ref = oracle.bruteforce(q, k, v, W, grid, block, eps=1e-6)
    assert rel_err(out, ref) < 1e-12


@pytest.mark.parametrize("cfg_index", [1, 2, 3, 4])
def test_row_sampled_bruteforce_on_workload_geometry(oracle_lib, cfg_index):
    """One head at each workload's full geometry; 128 random query rows by brute force."""
    cfg = synth.CONFIGS[cfg_index].with_(batch=1, heads=1)
    q, k, v, W = synth.make_inputs(cfg, seed=100 + cfg_index)
    out = oracle.forward(q, k, v, W, cfg.grid, cfg.block, eps=cfg.eps, pairs=[0])[0]
    rows = np.random.default_rng(cfg_index).choice(cfg.n_tokens, 128, replace=False)
    ref = oracle.bruteforce(q, k, v, W, cfg.grid, cfg.block, eps=cfg.eps, pairs=[0], rows=rows)[0]
    assert rel_err(out[rows], ref) < 1e-12


# ---------------------------------------------------------------- textbook special cases

def vanilla_linear_attention(Q, K, V, eps):
    """Global linear attention with a positive feature map (paperlayer.ai
    summary section 3, 'Linear Attention Formulation'), float64."""
    fq, fk = oracle.phi_np(Q), oracle.phi_np(K)
    kv = np.einsum("mc,me->ce", fk, V)
    ksum = fk.sum(axis=0)
    return (fq @ kv) / (fq @ ksum + eps)[:, None]


def test_m1_is_vanilla_linear_attention(oracle_lib):
    grid = (8, 12)
    p = synth.Problem("t", 2, 2, 16, grid, grid, dtype=synth.BF16)
    q, k, v, _ = synth.make_inputs(p, seed=3)
    for w in (1.0, 0.37):
        W = np.array([[w]], dtype=np.float32)
        out = oracle.forward(q, k, v, W, grid, grid, eps=1e-3)
        Q, K, V = (synth.as_float64(x, synth.BF16) for x in (q, k, v))
        for b in range(2):
            for h in range(2):
                ref = vanilla_linear_attention(Q[b, :, h], K[b, :, h], V[b, :, h], 1e-3 / np.float64(np.float32(w)))
                assert rel_err(out[b, :, h], ref) < 1e-12


def test_identity_w_is_per_block_linear_attention(oracle_lib):
    grid, block = (12, 10), (3, 5)
    p = synth.Problem("t", 1, 2, 8, grid, block, dtype=synth.F32)
    q, k, v, _ = synth.make_inputs(p, seed=4)
    W = np.eye(p.n_blocks, dtype=np.float32)
    out = oracle.forward(q, k, v, W, grid, block, eps=1e-4)
    Q, K, V = (synth.as_float64(x, synth.F32) for x in (q, k, v))
    # Gather each block by reshaping the raster grid: [Y,X] -> [Y/by, by, X/bx, bx].
    ny, nx = grid[0] // block[0], grid[1] // block[1]

    def blocks(a):   # a: [N, d] -> [M, T, d] and the token order inside
        g = a.reshape(ny, block[0], nx, block[1], -1).transpose(0, 2, 1, 3, 4)
        return g.reshape(ny * nx, block[0] * block[1], -1)
    idx = blocks(np.arange(p.n_tokens)[:, None])[..., 0]
    for h in range(2):
        Qb, Kb, Vb = blocks(Q[0, :, h]), blocks(K[0, :, h]), blocks(V[0, :, h])
        for j in range(p.n_blocks):
            ref = vanilla_linear_attention(Qb[j], Kb[j], Vb[j], 1e-4)
            assert rel_err(out[0, idx[j], h], ref) < 1e-12


def test_uniform_w_is_global_linear_attention(oracle_lib):
    """W = 1/M everywhere: St = S/M, zt = z/M, so eps acts as M*eps on the global form."""
    grid, block = (16, 16), (4, 4)
    p = synth.Problem("t", 1, 1, 32, grid, block, dtype=synth.F32)
    q, k, v, _ = synth.make_inputs(p, seed=5)
    M = p.n_blocks
    W = np.full((M, M), 1.0 / M, dtype=np.float32)
    w = np.float64(np.float32(1.0 / M))
    out = oracle.forward(q, k, v, W, grid, block, eps=1e-2)
    Q, K, V = (synth.as_float64(x, synth.F32) for x in (q, k, v))
    ref = vanilla_linear_attention(Q[0, :, 0], K[0, :, 0], V[0, :, 0], 1e-2 / w)
    assert rel_err(out[0, :, 0], ref) < 1e-12


# ---------------------------------------------------------------- rank statements

def normalised_attention(q, k, W, grid, block, eps=0.0):
    bid = oracle.token_blocks(grid, block)
    A = oracle.attention_matrix(synth.as_float64(q, synth.F32)[0, :, 0],
                                synth.as_float64(k, synth.F32)[0, :, 0], W, bid)
    return A / (A.sum(axis=1, keepdims=True) + eps)


def test_rank_global_linear_attention_bounded_by_d(oracle_lib):
    """Global (M = 1) linear attention has rank <= d (paperlayer.ai summary,
    section 3 'Global Context Collapse')."""
    d, grid = 4, (16, 16)
    p = synth.Problem("t", 1, 1, d, grid, grid, dtype=synth.F32)
    q, k, _, _ = synth.make_inputs(p, seed=6)
    A = normalised_attention(q, k, np.ones((1, 1)), grid, grid)
    assert np.linalg.matrix_rank(A) == d


def test_rank_grows_with_blocks(oracle_lib):
    """Block-diagonal W = I: rank = sum_b min(T, d); a generic mixing matrix
    reaches min(N, M*d) (section 4 'Rank Analysis')."""
    d, grid, block = 4, (16, 16), (4, 4)
    p = synth.Problem("t", 1, 1, d, grid, block, dtype=synth.F32)
    q, k, _, W = synth.make_inputs(p, seed=7)
    M, T, N = p.n_blocks, p.block_tokens, p.n_tokens
    A_id = normalised_attention(q, k, np.eye(M), grid, block)
    assert np.linalg.matrix_rank(A_id) == M * min(T, d)
    A_w = normalised_attention(q, k, W.astype(np.float64), grid, block)
    assert np.linalg.matrix_rank(A_w) == min(N, M * d)
    A_1 = normalised_attention(q, k, np.ones((M, M)), grid, block)
    assert np.linalg.matrix_rank(A_1) == d


# ---------------------------------------------------------------- algebraic invariants

def test_constant_values_give_constant_output(oracle_lib):
    """With eps = 0 every row is a convex combination (all weights > 0 for W > 0),
    so a constant V comes back unchanged."""
    grid, block = (12, 12), (4, 6)
    p = synth.Problem("t", 1, 2, 8, grid, block, dtype=synth.F32, jitter=0.0)
    q, k, v, W = synth.make_inputs(p, seed=8)
    c = np.linspace(-2, 3, 8).astype(np.float32)
    v[:] = c
    out = oracle.forward(q, k, v, W, grid, block, eps=0.0)
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=1e-13, atol=1e-13)


def test_linear_in_values(oracle_lib):
    grid, block = (8, 8), (2, 4)
    rng = np.random.default_rng(9)
    shape = (1, 64, 2, 8)
    q = rng.standard_normal(shape).astype(np.float32)
    k = rng.standard_normal(shape).astype(np.float32)
    v1 = rng.integers(-8, 8, shape).astype(np.float32)
    v2 = rng.integers(-8, 8, shape).astype(np.float32)
    W = synth.make_inputs(synth.Problem("t", 1, 2, 8, grid, block, dtype=synth.F32), 9)[3]
    f = lambda v: oracle.forward(q, k, v, W, grid, block, eps=1e-3)
    lhs = f((2 * v1 + v2).astype(np.float32))
    rhs = 2 * f(v1) + f(v2)
    assert rel_err(lhs, rhs) < 1e-12


def test_row_scaling_of_w_cancels_without_eps(oracle_lib):
    grid, block = (8, 8), (4, 4)
    p = synth.Problem("t", 1, 1, 8, grid, block, dtype=synth.F32, jitter=0.0)
    q, k, v, W = synth.make_inputs(p, seed=10)
    s = np.array([0.5, 2.0, 4.0, 0.25], dtype=np.float32)[:, None]
    a = oracle.forward(q, k, v, W, grid, block, eps=0.0)
    b = oracle.forward(q, k, v, (W * s).astype(np.float32), grid, block, eps=0.0)
    assert rel_err(b, a) < 1e-13


def test_summaries_match_definition(oracle_lib):
    """S_j = sum_{m in j} phi(k_m) v_m^T, z_j = sum phi(k_m), St = W S, zt = W z."""
    grid, block = (6, 10), (3, 5)
    p = synth.Problem("t", 2, 2, 8, grid, block, dtype=synth.BF16)
    q, k, v, W = synth.make_inputs(p, seed=12)
    S, z, St, zt = oracle.summaries(k, v, W, grid, block)
    bid = oracle.token_blocks(grid, block)
    K, V = oracle.decode(k), oracle.decode(v)
    for s in range(4):
        b, h = divmod(s, 2)
        fk = oracle.phi_np(K[b, :, h])
        for j in range(p.n_blocks):
            sel = bid == j
            np.testing.assert_allclose(S[s, j], fk[sel].T @ V[b, sel, h], rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(z[s, j], fk[sel].sum(0), rtol=1e-13)
        Wd = W.astype(np.float64)
        np.testing.assert_allclose(St[s], np.tensordot(Wd, S[s], axes=1), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(zt[s], Wd @ z[s], rtol=1e-12, atol=1e-12)


def test_pair_selection_and_threads(oracle_lib):
    p = synth.CONFIGS[0].with_(batch=2, heads=3)
    q, k, v, W = synth.make_inputs(p, seed=13)
    full = oracle.forward(q, k, v, W, p.grid, p.block, threads=1)
    sub, used = oracle.forward(q, k, v, W, p.grid, p.block, pairs=[5, 0, 3], threads=8,
                               return_threads=True)
    assert used == 8      # 3 pairs x 16 blocks: every thread has (pair, block) units
    for s, pair in enumerate([5, 0, 3]):
        b, h = divmod(pair, 3)
        np.testing.assert_array_equal(sub[s], full[b, :, h])
    # each element is summed in the same order whatever the thread count
    for t in (2, 5, 64):
        np.testing.assert_array_equal(oracle.forward(q, k, v, W, p.grid, p.block, threads=t), full)
    # one block: 6 (pair, block) units at most, so 6 threads
    p1 = p.with_(block=p.grid)
    q1, k1, v1, W1 = synth.make_inputs(p1, seed=14)
    _, used1 = oracle.forward(q1, k1, v1, W1, p1.grid, p1.block, threads=8, return_threads=True)
    assert used1 == 6



# ---------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes(oracle_lib):
    """Feed the oracle deliberately wrong operands; the hand-worked pins must fail."""
    ex = [e for e in load_examples() if e["name"] == "two-channel-negative-branch"][0]
    q, k, v, W, expected = example_inputs(ex)
    run = lambda q_, k_, v_, W_, eps: oracle.forward(q_, k_, v_, W_, ex["grid"], ex["block"], eps=eps)[0, :, 0]
    assert rel_err(run(q, k, v, W, ex["eps"]), expected) < 1e-14
    planted = {
        "transposed W": run(q, k, v, np.ascontiguousarray(W.T), ex["eps"]),
        "q and k swapped": run(k, q, v, W, ex["eps"]),
        "eps dropped": run(q, k, v, W, 0.0),
        "sign flip (other phi branch)": run(q, synth.bf16_bits(-synth.bf16_to_f32(k)), v, W, ex["eps"]),
        "channels transposed in values": run(q, k, np.ascontiguousarray(v[..., ::-1]), W, ex["eps"]),
    }
    for name, out in planted.items():
        assert rel_err(out, expected) > 1e-3, name
