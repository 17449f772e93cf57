"""Helpers shared by the GPU tests: device transfer and library calls through the C ABI."""
import sys

import numpy as np
import torch

import token_level_head_block_amd as mh
from token_level_head_block_amd import synth

TOL = {synth.F32: 1e-5, synth.BF16: 1e-2}   # max|d| / max|ref| against the float64 oracle


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: int) -> torch.Tensor:
    if dtype == synth.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def grid_block(p: synth.Problem, dtype=None):
    dt = p.dtype if dtype is None else dtype
    g = mh.make_grid(p.batch, p.heads, p.head_dim, mh.MHLA_BF16 if dt == synth.BF16 else mh.MHLA_F32,
                     p.grid, p.eps)
    return g, mh.make_block(p.block)


class Run:
    """Device inputs of one problem plus helpers to call the library."""

    def __init__(self, p: synth.Problem, q, k, v, W):
        self.p = p
        self.q, self.k, self.v = (to_dev(x, p.dtype) for x in (q, k, v))
        self.W = torch.from_numpy(W).cuda()
        self.g, self.b = grid_block(p)
        self.ws_bytes = mh.mhla_workspace_bytes(self.g, self.b)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def forward(self, path=mh.MHLA_PATH_3KERNEL, out=None, stream=None):
        if out is None:
            out = torch.empty_like(self.q)
        say(f"  [gpu] mhla_forward_ex path={path} {self.p.name} B{self.p.batch} H{self.p.heads} "
            f"d{self.p.head_dim} grid{self.p.grid} block{self.p.block}")
        st = mh.mhla_forward_ex(self.q, self.k, self.v, self.W, self.g, self.b, out, self.ws,
                                self.ws_bytes, path, None, stream)
        assert st == mh.MHLA_OK, mh.mhla_status_string(st)
        torch.cuda.synchronize()
        return out

    def backward(self, dout_host, stream=None, ws=True, causal=False, variant=0):
        """Gradients through mhla_backward (mhla_causal_backward if causal):
        (dq, dk, dv) device tensors like q and dW [M, M] fp32."""
        p = self.p
        dout = to_dev(dout_host, p.dtype)
        dq, dk, dv = (torch.empty_like(self.q) for _ in range(3))
        M = p.n_blocks
        dW = torch.empty(M, M, dtype=torch.float32, device="cuda")
        wsize = mh.mhla_causal_backward_workspace_bytes if causal else mh.mhla_backward_workspace_bytes
        call = mh.mhla_causal_backward if causal else mh.mhla_backward
        wsb = wsize(self.g, self.b)
        wst = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda") if ws else None
        say(f"  [gpu] {call.__name__} {p.name} B{p.batch} H{p.heads} d{p.head_dim} grid{p.grid} block{p.block}")
        if variant:
            say(f"  [gpu] mhla_backward_ex variant={variant:#x}")
            st = mh.mhla_backward_ex(self.q, self.k, self.v, self.W, dout, self.g, self.b, dq, dk, dv, dW,
                                     wst, wsb if ws else 0, variant, None, stream)
        else:
            st = call(self.q, self.k, self.v, self.W, dout, self.g, self.b, dq, dk, dv, dW,
                      wst, wsb if ws else 0, None, stream)
        assert st == mh.MHLA_OK, mh.mhla_status_string(st)
        torch.cuda.synchronize()
        return dq, dk, dv, dW

    def workspace(self):
        """Intermediates from the workspace after a 3-kernel call:
        (S [P,M,d,d] as [c][e], z [P,M,d], St [P,M,d,d] as [c][e], zt [P,M,d]) in float64."""
        p = self.p
        P, M, d = p.batch * p.heads, p.n_blocks, p.head_dim
        esz = 4 if p.dtype == synth.F32 else 2
        up = lambda x: (x + 255) // 256 * 256
        raw = self.ws.cpu().numpy()
        n0 = P * M * (d * d + d)
        o1 = up(n0 * esz)
        n1 = P * M * d * d
        o2 = o1 + up(n1 * esz)

        def dec(buf, n):
            if esz == 4:
                return buf[: 4 * n].view(np.float32).astype(np.float64)
            return synth.bf16_to_f32(buf[: 2 * n].view(np.uint16)).astype(np.float64)
        rec = dec(raw[:o1], n0).reshape(P, M, d * d + d)
        S = rec[:, :, : d * d].reshape(P, M, d, d).transpose(0, 1, 3, 2)
        z = rec[:, :, d * d:]
        St = dec(raw[o1:o2], n1).reshape(P, M, d, d).transpose(0, 1, 3, 2)
        zt = raw[o2: o2 + 4 * P * M * d].view(np.float32).astype(np.float64).reshape(P, M, d)
        return S, z, St, zt


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


class LayerRun:
    """Device inputs of one layer problem (bf16) and a call through mhla_layer_forward."""

    def __init__(self, p: synth.Problem, x, params: dict, W):
        self.p = p
        self.x = to_dev(x, synth.BF16)
        self.W = torch.from_numpy(W).cuda()
        self.params = {}
        for name, val in params.items():
            if val is None:
                continue
            if name.startswith("w_"):
                self.params[name] = to_dev(val, synth.BF16)
            else:
                self.params[name] = torch.from_numpy(np.ascontiguousarray(val, dtype=np.float32)).cuda()
        self.g, self.b = grid_block(p)
        self.ws_bytes = mh.mhla_layer_workspace_bytes(self.g, self.b)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def forward(self, phi=mh.MHLA_PHI_ELU1, ws=True, stream=None):
        y = torch.empty_like(self.x)
        say(f"  [gpu] mhla_layer_forward phi={phi} {self.p.name} B{self.p.batch} H{self.p.heads} "
            f"d{self.p.head_dim} grid{self.p.grid} block{self.p.block} params={sorted(self.params)}")
        st = mh.mhla_layer_forward(self.x, self.W, self.g, self.b, self.params, y,
                                   self.ws if ws else None, self.ws_bytes if ws else 0, phi=phi, stream=stream)
        assert st == mh.MHLA_OK, mh.mhla_status_string(st)
        torch.cuda.synchronize()
        return y
