"""Pins of the oracle's causal chunkwise form (paperlayer.ai summary,
appendix B "Causal MHLA": block-specific mixtures reused per block, causality
preserved), against what the definition fixes:

* the materialised N x N form with the causal mask m <= n (numpy);
* one block: textbook causal linear attention, written with prefix sums;
* the first token's closed form;
* causality itself: the output ignores the coefficients W[i, j] with j > i
  and the keys/values of later tokens.
"""
import numpy as np
import pytest

import oracle
from token_level_head_block_amd import synth


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# name, B, H, d, grid, block, dtype: chunks contiguous in raster order
CASES = [
    ("seq-1d", 1, 2, 8, (1, 48), (1, 8), synth.F32),
    ("rows-2d", 2, 1, 8, (6, 5), (2, 5), synth.BF16),
    ("frames-3d", 1, 2, 4, (4, 3, 4), (2, 3, 4), synth.F32),
    ("T1", 1, 1, 8, (1, 12), (1, 1), synth.BF16),
]


def make(case, seed, eps=1e-3):
    name, B, H, d, grid, block, dt = case
    p = synth.Problem(name, B, H, d, grid, block, dtype=dt, eps=eps)
    return p, synth.make_inputs(p, seed=seed)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_causal_blockwise_equals_masked_bruteforce(oracle_lib, case):
    p, (q, k, v, W) = make(case, seed=51)
    got = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    ref = oracle.bruteforce_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    assert rel_err(got, ref) < 1e-12


# chunks split along their slowest axis of extent > 1 into cp sub-chunks
SUBCHUNK_CASES = [
    ("seq-1d", 1, 2, 8, (1, 64), (1, 16), synth.F32, (1, 4), 4),
    ("rows-2d", 2, 1, 8, (8, 5), (4, 5), synth.BF16, (2, 5), 2),
    ("frames-3d", 1, 2, 4, (3, 4, 6), (1, 4, 6), synth.F32, (1, 1, 6), 4),
]


@pytest.mark.parametrize("case", SUBCHUNK_CASES, ids=lambda c: c[0])
def test_causal_form_over_subchunks_with_repeated_coefficients(oracle_lib, case):
    """The causal form over chunks with W equals the causal form over
    sub-chunks (each chunk split into cp contiguous runs) whose coefficient
    between sub-chunks a and b is W[a // cp][b // cp]: every pair of tokens
    keeps the weight of its chunks and the mask m <= n.  The library runs
    long chunks this way."""
    name, B, H, d, grid, block, dt, sub, cp = case
    p, (q, k, v, W) = make(case[:7], seed=55)
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    Wsub = W[np.arange(W.shape[0] * cp)[:, None] // cp, np.arange(W.shape[0] * cp)[None, :] // cp]
    got = oracle.forward_causal(q, k, v, np.ascontiguousarray(Wsub, dtype=np.float32), p.grid, sub, eps=p.eps)
    assert rel_err(got, ref) < 1e-12
    # and a W that differs between sub-chunks of one chunk changes the result
    Wbad = Wsub.copy()
    Wbad[1, 0] += 0.5
    bad = oracle.forward_causal(q, k, v, np.ascontiguousarray(Wbad, dtype=np.float32), p.grid, sub, eps=p.eps)
    assert rel_err(bad, ref) > 1e-6


def test_one_block_is_causal_linear_attention(oracle_lib):
    case = ("seq", 1, 2, 8, (1, 40), (1, 40), synth.F32)
    p, (q, k, v, _) = make(case, seed=52)
    W = np.array([[1.0]], dtype=np.float32)
    got = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    Q, K, V = (oracle.decode(x) for x in (q, k, v))
    for h in range(p.heads):
        u, a, vv = oracle.phi_np(Q[0, :, h]), oracle.phi_np(K[0, :, h]), V[0, :, h]
        S = np.cumsum(a[:, :, None] * vv[:, None, :], axis=0)     # sum_{m <= n} a_m v_m^T
        z = np.cumsum(a, axis=0)
        num = np.einsum("nc,nce->ne", u, S)
        den = np.einsum("nc,nc->n", u, z) + p.eps
        assert rel_err(got[0, :, h], num / den[:, None]) < 1e-12


def test_first_token_closed_form(oracle_lib):
    p, (q, k, v, W) = make(CASES[0], seed=53)
    got = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    Q, K, V = (oracle.decode(x) for x in (q, k, v))
    for h in range(p.heads):
        s = float(W[0, 0]) * float(oracle.phi_np(Q[0, 0, h]) @ oracle.phi_np(K[0, 0, h]))
        np.testing.assert_allclose(got[0, 0, h], s * V[0, 0, h] / (s + p.eps), rtol=1e-13)


def test_causality(oracle_lib):
    case = ("seq", 1, 2, 8, (1, 64), (1, 8), synth.F32)
    p, (q, k, v, W) = make(case, seed=54)
    base = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    # coefficients of later blocks are never read
    W2 = W.copy()
    W2[np.triu_indices(W.shape[0], 1)] = 7.0
    np.testing.assert_array_equal(oracle.forward_causal(q, k, v, W2, p.grid, p.block, eps=p.eps), base)
    # the last token's key and value reach no earlier output
    k2, v2 = k.copy(), v.copy()
    k2[:, -1] += 1.5
    v2[:, -1] -= 2.0
    out = oracle.forward_causal(q, k2, v2, W, p.grid, p.block, eps=p.eps)
    np.testing.assert_array_equal(out[:, :-1], base[:, :-1])
    assert rel_err(out[:, -1], base[:, -1]) > 1e-6
    # ... while the non-causal form depends on both
    assert rel_err(oracle.forward(q, k, v, W2, p.grid, p.block, eps=p.eps),
                   oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps)) > 1e-3


def test_causal_rejects_chunks_not_contiguous(oracle_lib):
    p = synth.Problem("blocks", 1, 1, 8, (8, 8), (4, 4), dtype=synth.F32)
    q, k, v, W = synth.make_inputs(p, seed=55)
    with pytest.raises(ValueError):
        oracle.forward_causal(q, k, v, W, p.grid, p.block)


def test_causal_pins_catch_planted_mistakes(oracle_lib):
    p, (q, k, v, W) = make(CASES[0], seed=56)
    ref = oracle.bruteforce_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    run = lambda q_, k_, v_, W_: oracle.forward_causal(q_, k_, v_, W_, p.grid, p.block, eps=p.eps)
    planted = {
        "transposed W": run(q, k, v, np.ascontiguousarray(W.T)),
        "q and k swapped": run(k, q, v, W),
        "no causal mask": oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps),
    }
    for name, out in planted.items():
        assert rel_err(out, ref) > 1e-3, name


def test_conditioning_helper_matches_masked_row_sums(oracle_lib):
    """The denominators the GPU tests use to measure cancellation equal the row
    sums of the masked N x N form plus eps, with W and with |W|."""
    from conditioning import causal_denominators
    for case in (("seq", 1, 2, 8, (1, 48), (1, 8), synth.F32), ("rows-2d", 2, 1, 8, (6, 5), (2, 5), synth.BF16)):
        p, (q, k, v, W) = make(case, seed=57)
        den, absden = causal_denominators(q, k, W, p.grid, p.block, p.eps)
        bid = oracle.token_blocks(p.grid, p.block)
        Q, K = oracle.decode(q), oracle.decode(k)
        N = bid.shape[0]
        mask = np.tril(np.ones((N, N)))
        for b in range(p.batch):
            for h in range(p.heads):
                S = oracle.phi_np(Q[b, :, h]) @ oracle.phi_np(K[b, :, h]).T * mask
                Wx = W.astype(np.float64)[bid][:, bid]
                np.testing.assert_allclose(den[b, :, h], (Wx * S).sum(1) + p.eps, rtol=1e-12)
                np.testing.assert_allclose(absden[b, :, h], (np.abs(Wx) * S).sum(1), rtol=1e-12)


def causal_autograd(p, q, k, v, W, g, eps):
    """Gradients of sum(g * o) by torch float64 autograd through the masked N x N form."""
    import torch
    bid = torch.from_numpy(oracle.token_blocks(p.grid, p.block))
    Q, K, V, G = (torch.from_numpy(oracle.decode(x)).requires_grad_(x is not g) for x in (q, k, v, g))
    Wt = torch.from_numpy(W.astype(np.float64)).requires_grad_(True)
    N = bid.shape[0]
    mask = torch.tril(torch.ones(N, N, dtype=torch.float64))
    phi = lambda x: torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))
    L = 0.0
    for b in range(p.batch):
        for h in range(p.heads):
            A = Wt[bid][:, bid] * (phi(Q[b, :, h]) @ phi(K[b, :, h]).T) * mask
            o = (A @ V[b, :, h]) / (A.sum(dim=1) + eps)[:, None]
            L = L + (o * G[b, :, h]).sum()
    L.backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy(), Wt.grad.numpy()


BWD_CASES = [
    ("seq", 1, 2, 4, (1, 24), (1, 6), synth.F32),
    ("rows-2d", 2, 1, 8, (6, 5), (2, 5), synth.BF16),
    ("frames-3d", 1, 1, 4, (3, 2, 4), (1, 2, 4), synth.F32),
    ("M1", 1, 2, 4, (1, 10), (1, 10), synth.F32),
    ("T1", 1, 1, 4, (1, 7), (1, 1), synth.F32),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: c[0])
def test_causal_gradients_match_autograd(oracle_lib, case):
    p, (q, k, v, W) = make(case, seed=58)
    rng = np.random.default_rng(59)
    g = rng.standard_normal(q.shape).astype(np.float32)
    g = synth.bf16_bits(g) if p.dtype == synth.BF16 else g
    got = oracle.backward_causal(q, k, v, W, g, p.grid, p.block, eps=p.eps)
    ref = causal_autograd(p, q, k, v, W, g, p.eps)
    for name, a, b in zip(("dq", "dk", "dv", "dW"), got, ref):
        assert rel_err(a, b) < 1e-10, name
    # coefficients of later blocks get no gradient
    assert np.all(got[3][np.triu_indices(W.shape[0], 1)] == 0.0)


def test_causal_gradient_directional_difference(oracle_lib):
    case = ("seq", 1, 1, 4, (1, 20), (1, 5), synth.F32)
    p, (q, k, v, W) = make(case, seed=60)
    g = np.random.default_rng(61).standard_normal(q.shape).astype(np.float32)
    grads = oracle.backward_causal(q, k, v, W, g, p.grid, p.block, eps=p.eps)
    X = [oracle.decode(x) for x in (q, k, v)] + [W.astype(np.float64)]
    G = oracle.decode(g)
    bid = oracle.token_blocks(p.grid, p.block)
    N = bid.shape[0]

    def loss(Qx, Kx, Vx, Wx):
        A = Wx[bid][:, bid] * (oracle.phi_np(Qx[0, :, 0]) @ oracle.phi_np(Kx[0, :, 0]).T) * np.tril(np.ones((N, N)))
        return float(np.sum((A @ Vx[0, :, 0]) / (A.sum(axis=1) + p.eps)[:, None] * G[0, :, 0]))

    rng = np.random.default_rng(62)
    for idx, gr in enumerate(grads):
        delta = rng.standard_normal(X[idx].shape)
        plus = [x.copy() for x in X]
        minus = [x.copy() for x in X]
        plus[idx] += 1e-5 * delta
        minus[idx] -= 1e-5 * delta
        fd = (loss(*plus) - loss(*minus)) / 2e-5
        assert abs(fd - float(np.sum(gr * delta))) <= 1e-6 * max(abs(fd), 1.0), idx


def test_causal_gradient_pins_catch_planted_mistakes(oracle_lib):
    p, (q, k, v, W) = make(BWD_CASES[0], seed=63)
    g = np.random.default_rng(64).standard_normal(q.shape).astype(np.float32)
    ref = causal_autograd(p, q, k, v, W, g, p.eps)
    run = lambda W_, g_, eps: oracle.backward_causal(q, k, v, W_, g_, p.grid, p.block, eps=eps)
    planted = {
        "transposed W": run(np.ascontiguousarray(W.T), g, p.eps),
        "upstream gradient negated": run(W, -g, p.eps),
        "eps dropped": run(W, g, 0.0),
        "non-causal gradients": oracle.backward(q, k, v, W, g, p.grid, p.block, eps=p.eps),
    }
    for name, got in planted.items():
        assert max(rel_err(a, b) for a, b in zip(got, ref)) > 1e-6, name
