"""mhla_forward_noalloc (workspace in the library's fixed per-GPU scratch)
against mhla_forward_ex (caller workspace, same kernels) through the C ABI:
bit-for-bit equal outputs on consecutive calls, the second with a smaller
problem, and the oracle's bar on the small problem."""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_block_amd as mh
from token_level_head_block_amd import synth

from gpu_util import TOL, Run, rel_err, say, to_host64

pytestmark = pytest.mark.gpu


def noalloc(run: Run, stream=None):
    out = torch.empty_like(run.q)
    p = run.p
    say(f"  [gpu] mhla_forward_noalloc {p.name} B{p.batch} H{p.heads} d{p.head_dim} grid{p.grid} block{p.block}")
    st = mh.mhla_forward_noalloc(run.q, run.k, run.v, run.W, run.g, run.b, out, stream)
    assert st == mh.MHLA_OK, mh.mhla_status_string(st)
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    big = synth.CONFIGS[2]                                               # 26 MB of workspace
    small = synth.Problem("noalloc-small", 1, 3, 64, (40, 40), (5, 5))   # ragged: 25-token blocks
    gb = mh.make_grid(big.batch, big.heads, big.head_dim, mh.MHLA_BF16, big.grid, big.eps)
    assert mh.mhla_workspace_bytes(gb, mh.make_block(big.block)) <= mh.MHLA_NOALLOC_SCRATCH_BYTES
    for p, seed in ((big, 2), (small, 71)):
        q, k, v, W = synth.make_inputs(p, seed=seed)
        run = Run(p, q, k, v, W)
        ref = run.forward()                       # mhla_forward_ex, caller workspace
        got = noalloc(run)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), p.name
        if p is small:
            err = rel_err(to_host64(got), oracle.forward(q, k, v, W, p.grid, p.block, eps=p.eps))
            say(f"  {p.name}: max|d|/max|ref| = {err:.3e}")
            assert err <= TOL[p.dtype]


def test_noalloc_side_stream_and_repeat():
    p = synth.Problem("noalloc-d32", 1, 4, 32, (64, 64), (16, 16))       # head pairs, token parts
    q, k, v, W = synth.make_inputs(p, seed=72)
    run = Run(p, q, k, v, W)
    ref = run.forward()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = noalloc(run, s)
    b = noalloc(run)
    assert torch.equal(a.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(b.view(torch.int16), ref.view(torch.int16))
