"""Conditioning of the causal chunkwise denominators, from the definition.

In the causal form (paperlayer.ai summary, appendix B "Causal MHLA") query n
of chunk i divides by
    den_n = sum_{j < i} W[i, j] phi(q_n).z_j + W[i, i] phi(q_n).sum_{m in i, m <= n} phi(k_m) + eps.
W is learned and may have negative entries, so the partial row sums
sum_{j < i} W[i, j] can nearly cancel even where the full rows do not.  Any
evaluation whose mixing operands carry a relative rounding of u (bf16 W and
block summaries) then errs by about u * kappa_n relative to o_n's scale, with
    kappa_n = (sum_{j < i} |W[i, j]| phi(q_n).z_j + |W[i, i]| phi(q_n).prefix_n) / |den_n|.
This module computes den and kappa in float64 with numpy; the GPU tests use
kappa to tell rounding amplified by cancellation from a wrong result.
"""
import numpy as np

import oracle

BF16_U = 2.0 ** -8   # unit roundoff of bfloat16 (8 significant bits)


def chunk_starts(bid: np.ndarray) -> np.ndarray:
    """First raster index of each token's chunk (chunks are runs of raster order)."""
    new = np.r_[True, bid[1:] != bid[:-1]]
    firsts = np.flatnonzero(new)
    return firsts[np.cumsum(new) - 1]


def causal_denominators(q, k, W, grid, block, eps):
    """(den, absden), each [B, N, H] float64: the signed causal denominator of
    every query and the same sum with |W| (eps left out)."""
    Q, K = oracle.decode(q), oracle.decode(k)
    bid = oracle.token_blocks(grid, block)
    B, N, H, d = Q.shape
    M = W.shape[0]
    Wd = W.astype(np.float64)
    Wrow = np.tril(Wd, -1)[bid]       # [N, M]: W[i(n), j] for j < i(n)
    diag = np.diag(Wd)[bid]           # [N]:    W[i(n), i(n)]
    start = chunk_starts(bid)
    den = np.empty((B, N, H))
    absden = np.empty((B, N, H))
    for b in range(B):
        for h in range(H):
            u = oracle.phi_np(Q[b, :, h])
            a = oracle.phi_np(K[b, :, h])
            Z = np.zeros((M, d))
            np.add.at(Z, bid, a)
            P = u @ Z.T                                    # phi(q_n) . z_j
            C = np.cumsum(a, axis=0)
            before = np.where((start > 0)[:, None], C[np.maximum(start - 1, 0)], 0.0)
            intra = np.einsum("nc,nc->n", u, C - before)   # phi(q_n) . own-chunk prefix
            den[b, :, h] = np.einsum("nm,nm->n", Wrow, P) + diag * intra + eps
            absden[b, :, h] = np.einsum("nm,nm->n", np.abs(Wrow), P) + np.abs(diag) * intra
    return den, absden
