"""Seeded synthetic inputs for the MHLA forward pass.

This module only draws and encodes inputs; it holds none of the method's
arithmetic.  It is the one piece of code shared by the HIP path's tests and
bench and by the CPU oracle's tests.

Workloads (shapes, value distributions and the distance-initialised mixing
matrix) follow the configurations the method is evaluated on: DiT-S/2-like
image grids, a SANA-like linear DiT layer and a spatio-temporal video latent
(paperlayer.ai summary of arXiv 2601.07832, sections 4 "Architecture" and 5
"Experiments"; 171host.com repost, section 7 code, class BlockDistanceConv,
for the block-centre distance initialisation of the coefficient matrix).

Conventions
-----------
* Q, K, V are [B, N, H, d] with N in raster order over the token grid (last
  axis fastest) and channel index h*d + c.
* bf16 tensors are returned as their raw 16-bit patterns (numpy uint16),
  produced from float32 draws by round-to-nearest-even.
* W is float32 [M, M]; W[i, j] weights source block j for query block i.
* Draw order from one generator: Q, K, V, then the W jitter.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass, field

import numpy as np

F32 = 0
BF16 = 1


@dataclass(frozen=True)
class Problem:
    """One MHLA forward problem: geometry, dtype and input distribution."""
    name: str
    batch: int
    heads: int
    head_dim: int
    grid: tuple            # token-grid extents, slowest axis first (2 or 3 axes)
    block: tuple           # block extents in tokens, same axis order
    dtype: int = BF16      # F32 or BF16 for q, k, v and out
    std: float = 1.0       # standard deviation of Q, K, V entries
    eps: float = 1e-6
    sigma: float = 3.0     # width of the distance prior, in block units
    jitter: float = 0.01   # std of the additive Gaussian jitter on W

    @property
    def ndim(self) -> int:
        return len(self.grid)

    @property
    def n_tokens(self) -> int:
        return int(np.prod(self.grid))

    @property
    def blocks_per_axis(self) -> tuple:
        return tuple(g // b for g, b in zip(self.grid, self.block))

    @property
    def n_blocks(self) -> int:
        return int(np.prod(self.blocks_per_axis))

    @property
    def block_tokens(self) -> int:
        return int(np.prod(self.block))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def with_(self, **kw) -> "Problem":
        d = dict(self.__dict__)
        d.update(kw)
        return Problem(**d)


# The five workloads.  Index k is also the default seed of its inputs.
CONFIGS = [
    Problem("tiny-fp32", 1, 1, 32, (16, 16), (4, 4), dtype=F32),
    Problem("dit-s2-64x64", 32, 6, 64, (64, 64), (8, 8)),
    Problem("dit-s2-256x256", 1, 6, 64, (256, 256), (16, 16)),
    Problem("sana-128x128", 2, 70, 32, (128, 128), (8, 8), std=0.5),
    Problem("video-16x64x64", 1, 12, 128, (16, 64, 64), (4, 8, 8)),
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def block_centres(blocks_per_axis) -> np.ndarray:
    """Centre of every block in block units, blocks in row-major order."""
    axes = [np.arange(n, dtype=np.float64) + 0.5 for n in blocks_per_axis]
    return np.array(list(itertools.product(*axes)), dtype=np.float64)


def distance_prior(blocks_per_axis, sigma: float) -> np.ndarray:
    """exp(-dist^2 / (2 sigma^2)) between block centres, each row scaled to sum to 1."""
    c = block_centres(blocks_per_axis)
    d2 = ((c[:, None, :] - c[None, :, :]) ** 2).sum(-1)
    g = np.exp(-d2 / (2.0 * sigma * sigma))
    return g / g.sum(axis=1, keepdims=True)


def local_prior(blocks_per_axis, thres: float = 1.5) -> np.ndarray:
    """Indicator of block-centre distance <= thres, each row scaled to sum to 1
    (a sparse, local coefficient matrix: at most 9 non-zeros per row in 2D)."""
    c = block_centres(blocks_per_axis)
    d = np.sqrt(((c[:, None, :] - c[None, :, :]) ** 2).sum(-1))
    g = (d <= thres).astype(np.float64)
    return g / g.sum(axis=1, keepdims=True)


def transform_prior(blocks_per_axis, kind: str, exp_sigma: float = 3.0) -> np.ndarray:
    """The module's distance transforms of the block-centre distance D
    (Euclidean, block units; 171host.com repost, section 七, BlockDistanceConv),
    each row scaled to sum to 1:
      "linear":      1 - D / max D
      "cos":         cos(D / max D * pi / 4)
      "exp":         exp(-D / exp_sigma)
      "gaussian-dmax": exp(-D^2 / (2 s^2)) with s = max D / 3
    A Gaussian of the Euclidean distance is separable, exp(-dy^2/2s^2) exp(-dx^2/2s^2),
    so the per-axis (separable) Gaussian is the same matrix as distance_prior."""
    c = block_centres(blocks_per_axis)
    D = np.sqrt(((c[:, None, :] - c[None, :, :]) ** 2).sum(-1))
    dmax = D.max() if D.max() > 0 else 1.0
    if kind == "linear":
        g = 1.0 - D / dmax
    elif kind == "cos":
        g = np.cos(D / dmax * np.pi / 4)
    elif kind == "exp":
        g = np.exp(-D / exp_sigma)
    elif kind == "gaussian-dmax":
        s = dmax / 3.0
        g = np.exp(-D * D / (2.0 * s * s))
    else:
        raise ValueError(f"unknown transform {kind!r}")
    return g / g.sum(axis=1, keepdims=True)


TRANSFORMS = ("linear", "cos", "exp", "gaussian-dmax")


def _rng(seed) -> np.random.Generator:
    return np.random.default_rng(seed)


def _draw(rng, shape, std, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x) if dtype == BF16 else x


def make_inputs(p: Problem, seed, w_kind: str = "gaussian"):
    """Seeded (q, k, v, W) for problem p.

    q, k, v: [B, N, H, d] (uint16 bf16 bits or float32); W: float32 [M, M].
    w_kind: "gaussian" (distance prior + jitter), "identity", "ones" (1/M),
    "local" (sparse local prior, no jitter), or one of TRANSFORMS (the
    module's other distance transforms, row-normalised, no jitter).
    """
    rng = _rng(seed)
    shape = (p.batch, p.n_tokens, p.heads, p.head_dim)
    q = _draw(rng, shape, p.std, p.dtype)
    k = _draw(rng, shape, p.std, p.dtype)
    v = _draw(rng, shape, p.std, p.dtype)
    M = p.n_blocks
    if w_kind == "gaussian":
        W = distance_prior(p.blocks_per_axis, p.sigma)
        W = W + p.jitter * rng.standard_normal((M, M))
    elif w_kind == "identity":
        W = np.eye(M)
    elif w_kind == "ones":
        W = np.full((M, M), 1.0 / M)
    elif w_kind == "local":
        W = local_prior(p.blocks_per_axis)
    elif w_kind in TRANSFORMS:
        W = transform_prior(p.blocks_per_axis, w_kind)
    else:
        raise ValueError(f"unknown w_kind {w_kind!r}")
    return q, k, v, np.ascontiguousarray(W, dtype=np.float32)


def as_float64(x: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float64 view of an input tensor given as bf16 bits or float32."""
    if dtype == BF16:
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def make_layer_inputs(p: Problem, seed, qk_norm: bool = False, lepe: bool = True, bias: bool = True,
                      w_kind: str = "gaussian"):
    """Seeded inputs of the whole layer around the core for problem p (bf16):
    x [B, N, C] (C = H * d) and a dict of parameters, scaled like freshly
    initialised layers: projection weights N(0, 1/C) in bf16 laid out
    [out features, in features]; norm weights 1 + 0.1 N(0, 1); biases
    0.02 N(0, 1); LePE kernels N(0, 1/25) per channel.  Plus W as in
    make_inputs.  Draw order: x, ln_w, ln_b, w_qkv, b_qkv, qn_w, kn_w, lepe_w,
    lepe_b, w_out, b_out, then W's jitter (each drawn whether used or not)."""
    if p.dtype != BF16:
        raise ValueError("the layer is bf16")
    rng = _rng(seed)
    C = p.heads * p.head_dim
    f32 = lambda shape, s=1.0: (rng.standard_normal(shape, dtype=np.float32) * np.float32(s))
    x = bf16_bits(f32((p.batch, p.n_tokens, C), p.std))
    params = {}
    params["ln_w"] = 1.0 + f32((C,), 0.1)
    params["ln_b"] = f32((C,), 0.1)
    params["w_qkv"] = bf16_bits(f32((3 * C, C), 1.0 / np.sqrt(C)))
    b_qkv = f32((3 * C,), 0.02)
    qn_w, kn_w = 1.0 + f32((C,), 0.1), 1.0 + f32((C,), 0.1)
    lepe_w, lepe_b = f32((C, 5, 5), 0.2), f32((C,), 0.02)
    params["w_out"] = bf16_bits(f32((C, C), 1.0 / np.sqrt(C)))
    b_out = f32((C,), 0.02)
    params["b_qkv"] = b_qkv if bias else None
    params["qn_w"] = qn_w if qk_norm else None
    params["kn_w"] = kn_w if qk_norm else None
    params["lepe_w"] = lepe_w if lepe else None
    params["lepe_b"] = lepe_b if lepe and bias else None
    params["b_out"] = b_out if bias else None
    M = p.n_blocks
    if w_kind == "gaussian":
        W = distance_prior(p.blocks_per_axis, p.sigma) + p.jitter * rng.standard_normal((M, M))
    elif w_kind == "local":
        W = local_prior(p.blocks_per_axis)
    else:
        raise ValueError(f"unknown w_kind {w_kind!r}")
    return x, params, np.ascontiguousarray(W, dtype=np.float32)
