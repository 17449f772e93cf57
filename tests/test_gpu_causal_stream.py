"""Stateful causal execution (mhla_causal_stream) against the float64 oracle,
through the C ABI: a sequence streamed in several calls of whole chunks gives
the oracle's one-shot causal outputs (oracle.forward_causal on the whole
sequence, or the masked N x N form when chunk lengths differ between calls),
and the state holds the oracle's chunk summaries.

Bar: max|d| / max|ref| <= 1e-2 with bf16 inputs and outputs, 1e-5 with fp32
(the forward's bars; fp32 cases use the nonnegative local W, as the causal
gradients' tests do, so that no denominator cancels).
"""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_block_amd as mh
from token_level_head_block_amd import synth

from gpu_util import rel_err, say, to_dev, to_host64

pytestmark = pytest.mark.gpu

BF = synth.BF16
F32 = synth.F32
TOL = {BF: 1e-2, F32: 1e-5}


def stream_calls(p, q, k, v, W, splits, T, max_chunks=None, w_pad=0, rows=None):
    """Run the stream: splits = chunks per call; chunks of T tokens along the
    last axis (rows = None: 1D sequence) or whole rows of width `rows`.
    Returns (outputs [B, N, H, d] float64, state [B*H, max_chunks, d*d + d])."""
    dt = mh.MHLA_BF16 if p.dtype == BF else mh.MHLA_F32
    total = sum(splits)
    max_chunks = max_chunks or total
    Wp = np.zeros((W.shape[0] + w_pad,) * 2, dtype=np.float32)
    Wp[:W.shape[0], :W.shape[0]] = W
    Wd = torch.from_numpy(Wp).cuda()
    qd, kd, vd = (to_dev(x, p.dtype) for x in (q, k, v))
    g0 = mh.make_grid(p.batch, p.heads, p.head_dim, dt, (1, T), p.eps)
    b0 = mh.make_block((1, T))
    state = torch.full((mh.mhla_causal_state_bytes(g0, b0, max_chunks) // 4,), float("nan"),
                       dtype=torch.float32, device="cuda")
    outs, n_past, tok = [], 0, 0
    for m in splits:
        n = m * T
        if rows is None:
            g, b = mh.make_grid(p.batch, p.heads, p.head_dim, dt, (1, n), p.eps), mh.make_block((1, T))
        else:
            g = mh.make_grid(p.batch, p.heads, p.head_dim, dt, (n // rows, rows), p.eps)
            b = mh.make_block((T // rows, rows))
        qs, ks, vs = (x[:, tok:tok + n].contiguous() for x in (qd, kd, vd))
        out = torch.empty_like(qs)
        wsb = mh.mhla_causal_stream_workspace_bytes(g, b)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        say(f"  [gpu] mhla_causal_stream {p.name} n_past={n_past} chunks={m} T={T}")
        st = mh.mhla_causal_stream(qs, ks, vs, Wd, g, b, n_past, state, max_chunks, out, ws, wsb)
        assert st == mh.MHLA_OK, mh.mhla_status_string(st)
        outs.append(out)
        n_past += m
        tok += n
    torch.cuda.synchronize()
    o = to_host64(torch.cat(outs, dim=1))
    L = p.head_dim * p.head_dim + p.head_dim
    return o, state.cpu().numpy().astype(np.float64).reshape(p.batch * p.heads, max_chunks, L)


# name, B, H, d, T (tokens per chunk), splits, dtype, W kind
CASES = [
    ("stream-d64", 2, 3, 64, 32, (1, 3, 2, 4), BF, "gaussian"),
    ("stream-d32-one-call", 1, 2, 32, 16, (6,), BF, "gaussian"),
    ("stream-d128", 1, 2, 128, 24, (2, 1, 3), BF, "gaussian"),
    ("stream-chunk-per-call", 1, 1, 64, 8, (1,) * 7, BF, "gaussian"),
    ("stream-f32-d64", 1, 2, 64, 20, (2, 1, 3), F32, "local"),
    ("stream-f32-d128", 1, 1, 128, 16, (1, 4), F32, "local"),
    ("stream-f32-d32-T1", 2, 1, 32, 1, (5, 1, 10), F32, "local"),
    # long chunks: each call runs its chunks as sub-chunks of >= 256 tokens
    ("stream-long-chunks", 1, 2, 64, 1024, (1, 2, 1), BF, "gaussian"),
    ("stream-d128-long", 1, 1, 128, 512, (2, 1), BF, "gaussian"),
    ("stream-d32-long-B2", 2, 3, 32, 768, (1, 1), BF, "local"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_stream_matches_one_shot(case):
    name, B, H, d, T, splits, dt, wk = case
    M = sum(splits)
    p = synth.Problem(name, B, H, d, (1, M * T), (1, T), dtype=dt)
    q, k, v, W = synth.make_inputs(p, seed=81, w_kind=wk)
    got, state = stream_calls(p, q, k, v, W, splits, T, max_chunks=M + 2, w_pad=3)
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    err = rel_err(got, ref)
    say(f"  {name}: max|d|/max|ref| = {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL[dt]
    # the state holds every chunk's summary [S as [c][e] | z]
    S, z, _, _ = oracle.summaries(k, v, W, p.grid, p.block)
    P = B * H
    rec = np.concatenate([S.reshape(P, M, d * d), z.reshape(P, M, d)], axis=2)
    assert rel_err(state[:, :M], rec) <= 1e-6
    assert np.isnan(state[:, M:]).all()          # slots past the stream are never written


def test_stream_chunk_length_may_change_between_calls():
    """Three chunks of 16 tokens, then two of 32: the masked N x N form with
    those block ids is the reference."""
    d, H = 64, 2
    n1, n2 = 3 * 16, 2 * 32
    p = synth.Problem("stream-mixed", 1, H, d, (1, n1 + n2), (1, 16), dtype=BF)
    q, k, v, _ = synth.make_inputs(p, seed=82)
    W = (0.3 + np.random.default_rng(83).random((5, 5))).astype(np.float32)
    dt = mh.MHLA_BF16
    qd, kd, vd = (to_dev(x, BF) for x in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    g1, b1 = mh.make_grid(1, H, d, dt, (1, n1), p.eps), mh.make_block((1, 16))
    g2, b2 = mh.make_grid(1, H, d, dt, (1, n2), p.eps), mh.make_block((1, 32))
    state = torch.empty(mh.mhla_causal_state_bytes(g1, b1, 5) // 4, dtype=torch.float32, device="cuda")
    o1 = torch.empty(1, n1, H, d, dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty(1, n2, H, d, dtype=torch.bfloat16, device="cuda")
    say("  [gpu] mhla_causal_stream stream-mixed: 3 chunks of 16, then 2 of 32")
    assert mh.mhla_causal_stream(qd[:, :n1].contiguous(), kd[:, :n1].contiguous(), vd[:, :n1].contiguous(), Wd,
                                 g1, b1, 0, state, 5, o1) == mh.MHLA_OK
    assert mh.mhla_causal_stream(qd[:, n1:].contiguous(), kd[:, n1:].contiguous(), vd[:, n1:].contiguous(), Wd,
                                 g2, b2, 3, state, 5, o2) == mh.MHLA_OK
    got = to_host64(torch.cat([o1, o2], dim=1))
    bid = np.concatenate([np.repeat(np.arange(3), 16), 3 + np.repeat(np.arange(2), 32)])
    Q, K, V = (oracle.decode(x) for x in (q, k, v))
    for h in range(H):
        ref = oracle.bruteforce_causal_head(Q[0, :, h], K[0, :, h], V[0, :, h], W, bid, p.eps)
        err = rel_err(got[0, :, h], ref)
        say(f"  stream-mixed head {h}: max|d|/max|ref| = {err:.3e}")
        assert err <= TOL[BF]


def test_stream_rows_of_an_image():
    """A 2D grid streamed two rows per chunk, in calls of 1, 2 and 3 chunks."""
    X, rows_per_chunk = 20, 2
    splits = (1, 2, 3)
    M = sum(splits)
    p = synth.Problem("stream-rows", 1, 2, 64, (M * rows_per_chunk, X), (rows_per_chunk, X), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=84)
    got, _ = stream_calls(p, q, k, v, W, splits, rows_per_chunk * X, rows=X)
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    err = rel_err(got, ref)
    say(f"  stream-rows: max|d|/max|ref| = {err:.3e}")
    assert err <= TOL[BF]


def test_stream_long_sequence_bf16():
    """16384 tokens in 64 chunks of 256 (six heads, d = 64), streamed in four
    calls of 16 chunks through the matrix-core apply, against the oracle's
    one-shot causal outputs: every output.  The nonnegative local W keeps
    every partial row sum of W positive, so no denominator cancels."""
    T, splits = 256, (16, 16, 16, 16)
    M = sum(splits)
    p = synth.Problem("stream-long", 1, 6, 64, (1, M * T), (1, T), dtype=BF)
    q, k, v, W = synth.make_inputs(p, seed=85, w_kind="local")
    got, state = stream_calls(p, q, k, v, W, splits, T)
    ref = oracle.forward_causal(q, k, v, W, p.grid, p.block, eps=p.eps)
    err = rel_err(got, ref)
    say(f"  stream-long: max|d|/max|ref| = {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL[BF]
