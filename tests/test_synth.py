"""Seeded input synthesis: encoding, determinism and the W recipe."""
import numpy as np
import torch

from token_level_head_block_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -1e-40], np.float32)])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_inputs_are_deterministic_and_shaped():
    p = synth.CONFIGS[0]
    a = synth.make_inputs(p, seed=0)
    b = synth.make_inputs(p, seed=0)
    c = synth.make_inputs(p, seed=1)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    assert a[0].shape == (1, 256, 1, 32) and a[0].dtype == np.float32
    assert a[3].shape == (16, 16) and a[3].dtype == np.float32
    q = synth.make_inputs(synth.CONFIGS[1].with_(batch=1), seed=0)[0]
    assert q.dtype == np.uint16 and q.shape == (1, 4096, 6, 64)


def test_distance_prior():
    # 2x2 block grid: distances 0, 1, 1, sqrt(2); gaussian with sigma 3, rows sum to 1.
    W = synth.distance_prior((2, 2), 3.0)
    g = np.exp(-np.array([0.0, 1.0, 1.0, 2.0]) / 18.0)
    np.testing.assert_allclose(W[0], g / g.sum(), rtol=1e-15)
    np.testing.assert_allclose(W.sum(1), 1.0, rtol=1e-15)
    np.testing.assert_allclose(W, W.T, rtol=1e-15)   # equal row sums by symmetry of the 2x2 grid
    # 3D: centres in block units, slowest axis first.
    c = synth.block_centres((2, 1, 3))
    np.testing.assert_array_equal(c[4], [1.5, 0.5, 1.5])


def test_local_prior_is_sparse():
    W = synth.local_prior((16, 16))
    nnz = (W > 0).sum(1)
    assert nnz.max() == 9 and nnz.min() == 4
    np.testing.assert_allclose(W.sum(1), 1.0)


def test_jittered_w_row_sums_stay_positive():
    for p in synth.CONFIGS:
        W = synth.make_inputs(p.with_(batch=1, heads=1), seed=0)[3].astype(np.float64)
        assert W.sum(1).min() > 0.4


def test_transform_priors():
    """The module's other distance transforms on a 2x2 block grid (distances
    0, 1, 1, sqrt 2 from block 0; max distance sqrt 2), by hand, rows sum to 1."""
    r2 = np.sqrt(2.0)
    d = np.array([0.0, 1.0, 1.0, r2])
    expect = {
        "linear": 1.0 - d / r2,
        "cos": np.cos(d / r2 * np.pi / 4),
        "exp": np.exp(-d / 3.0),
        "gaussian-dmax": np.exp(-d * d / (2 * (r2 / 3) ** 2)),
    }
    for kind, g in expect.items():
        W = synth.transform_prior((2, 2), kind)
        np.testing.assert_allclose(W[0], g / g.sum(), rtol=1e-14)
        np.testing.assert_allclose(W.sum(1), 1.0, rtol=1e-14)
    # the linear transform gives the farthest block no weight; the separable
    # Gaussian equals the distance prior
    assert synth.transform_prior((2, 2), "linear")[0, 3] == 0.0
    sep = np.exp(-(np.subtract.outer(np.arange(3), np.arange(3)) ** 2) / 18.0)
    K = np.kron(sep, sep)
    np.testing.assert_allclose(K / K.sum(1, keepdims=True), synth.distance_prior((3, 3), 3.0), rtol=1e-14)
    p = synth.Problem("t", 1, 1, 32, (16, 16), (4, 4), dtype=synth.F32)
    for kind in synth.TRANSFORMS:
        W = synth.make_inputs(p, seed=0, w_kind=kind)[3]
        assert W.shape == (16, 16) and (W >= 0).all()
