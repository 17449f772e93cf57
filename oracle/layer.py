"""CPU oracle of the MHLA layer around the attention core (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library.

The layer follows the plug-and-play module of the 171host.com repost, section
七 (class MHLA, ``forward``), on tokens in raster order over a 2D grid:

    x -> LayerNorm -> QKV projection -> [RMSNorm on q and k] -> phi on q, k
      -> MHLA core -> + LePE(v) -> output projection.

Differences from that code, all stated where they occur: tokens are in raster
order [B, N, C] (the module takes pre-blocked tensors; the LePE convolution
works on the image either way); the normaliser is phi(q_n).zt_i + eps (the
module's form needs equal block sizes, reading R2); dropout is the identity
(inference).  The feature map is elu(x) + 1 (the core's workloads) or the
module's relu(x) + eps.

Every step is a plain formula; numpy matmul and einsum are the only library
primitives.  Inputs: x [B, N, C] bf16 bit patterns (uint16); weight matrices
bf16 bit patterns; norm weights, biases, the LePE kernel and W float32.
"""
from __future__ import annotations

import numpy as np

from . import decode, token_blocks

PHI_ELU1 = "elu1"
PHI_RELU_EPS = "relu_eps"


def layer_norm(X, w, b, eps):
    """LayerNorm over the channel axis ([repost] section 七: ``self.norm`` at the
    start of ``forward``): (x - mean) / sqrt(var + eps) * w + b, with the
    biased variance over the C channels of each token."""
    mu = X.mean(axis=-1, keepdims=True)
    var = ((X - mu) ** 2).mean(axis=-1, keepdims=True)
    return (X - mu) / np.sqrt(var + eps) * w + b


def linear(X, Wt, b=None):
    """y = x Wt^T + b with Wt laid out [out features, in features] ([repost]
    section 七: ``to_qkv`` and ``to_out``)."""
    y = X @ Wt.T
    return y if b is None else y + b


def rms_norm(X, w, eps):
    """RMSNorm over the channel axis ([repost] section 七: ``q_norm``,
    ``k_norm`` when qk_norm is set): x / sqrt(mean(x^2) + eps) * w."""
    return X / np.sqrt((X * X).mean(axis=-1, keepdims=True) + eps) * w


def phi(X, kind, phi_eps=1e-6):
    """Feature map: elu(x) + 1, or relu(x) + eps as in the module's
    ``_process_qkv_impl``."""
    if kind == PHI_ELU1:
        return np.where(X > 0, X + 1.0, np.exp(np.minimum(X, 0.0)))
    if kind == PHI_RELU_EPS:
        return np.maximum(X, 0.0) + phi_eps
    raise ValueError(f"unknown feature map {kind!r}")


def core(Q, K, V, W, grid, block, eps, kind, phi_eps=1e-6):
    """The MHLA core on float64 [B, N, H, d] arrays, blockwise
    (paperlayer.ai summary, section 4 "Architecture", "Multi-Head Mixing"):
    S_j = sum_{m in j} phi(k_m) v_m^T, z_j = sum phi(k_m), St_i = sum_j W[i,j] S_j,
    zt_i likewise, o_n = phi(q_n)^T St_i / (phi(q_n) . zt_i + eps)."""
    B, N, H, d = Q.shape
    bid = token_blocks(grid, block)
    M = W.shape[0]
    T = N // M
    order = np.argsort(bid, kind="stable")     # the tokens of block 0, then block 1, ...
    Wd = np.asarray(W, dtype=np.float64)
    out = np.empty_like(Q)
    for b in range(B):
        for h in range(H):
            u = phi(Q[b, :, h], kind, phi_eps)
            a = phi(K[b, :, h], kind, phi_eps)
            ab = a[order].reshape(M, T, d)
            vb = V[b, :, h][order].reshape(M, T, d)
            S = np.einsum("jtc,jte->jce", ab, vb)   # S_j = sum over the block's tokens
            z = ab.sum(axis=1)
            St = np.einsum("ij,jce->ice", Wd, S)
            zt = Wd @ z
            num = np.einsum("nc,nce->ne", u, St[bid])
            den = np.einsum("nc,nc->n", u, zt[bid]) + eps
            out[b, :, h] = num / den[:, None]
    return out


def lepe(Vimg, w, b=None):
    """Depthwise 5x5 convolution of v over the 2D token grid, zero padding 2,
    one 5x5 kernel per channel ([repost] section 七: ``self.lepe``, a Conv2d
    with groups = dim, applied to v laid out as an image).  Cross-correlation,
    as convolution layers compute it:
        out[y, x, c] = b[c] + sum_{dy, dx} w[c, dy, dx] v[y + dy - 2, x + dx - 2, c].
    Vimg: [B, Y, X, C]."""
    B, Y, X, C = Vimg.shape
    k = w.shape[-1]
    r = k // 2
    P = np.zeros((B, Y + 2 * r, X + 2 * r, C))
    P[:, r:r + Y, r:r + X] = Vimg
    out = np.zeros_like(Vimg)
    for dy in range(k):
        for dx in range(k):
            out += w[:, dy, dx] * P[:, dy:dy + Y, dx:dx + X]
    return out if b is None else out + b


def layer_forward(x, W, grid, block, heads, params, eps=1e-6, kind=PHI_ELU1, phi_eps=1e-6,
                  ln_eps=1e-5, rms_eps=1e-6, return_parts=False):
    """The whole layer in float64 ([repost] section 七, ``MHLA.forward``).

    params: dict with ln_w, ln_b [C]; w_qkv [3C, C] (bf16 bits); b_qkv [3C] or
    None; qn_w, kn_w [C] or None (no q/k norm); lepe_w [C, 5, 5] or None (no
    LePE); lepe_b [C] or None; w_out [C, C] (bf16 bits); b_out [C] or None.
    Returns y [B, N, C] (and the intermediates with return_parts)."""
    X = decode(x)
    B, N, C = X.shape
    d = C // heads
    f = lambda key: None if params.get(key) is None else np.asarray(params[key], dtype=np.float64)
    xn = layer_norm(X, f("ln_w"), f("ln_b"), ln_eps)
    qkv = linear(xn, decode(params["w_qkv"]), f("b_qkv"))
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    if params.get("qn_w") is not None:
        q = rms_norm(q, f("qn_w"), rms_eps)
        k = rms_norm(k, f("kn_w"), rms_eps)
    o = core(q.reshape(B, N, heads, d), k.reshape(B, N, heads, d), v.reshape(B, N, heads, d),
             W, grid, block, eps, kind, phi_eps).reshape(B, N, C)
    pe = None
    if params.get("lepe_w") is not None:
        if len(grid) != 2:
            raise ValueError("LePE is defined on 2D grids")
        pe = lepe(v.reshape(B, grid[0], grid[1], C), f("lepe_w"), f("lepe_b")).reshape(B, N, C)
        o = o + pe
    y = linear(o, decode(params["w_out"]), f("b_out"))
    if return_parts:
        return y, dict(xn=xn, q=q, k=k, v=v, o=o, lepe=pe)
    return y
