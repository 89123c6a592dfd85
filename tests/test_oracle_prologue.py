"""Pins of the oracle's per-token prologue (RMSNorm with weights, ReLU, L2).

Checked against: rows of mean square 1 (unit weight, eps -> 0); invariance
under positive scaling of a token; the weight acting per channel; ReLU leaving
no negative entry; unit L2 norms, and an all-zero row staying zero; and the
bf16 rounding agreeing with torch's own conversion of the fp32 values.
"""
import numpy as np
import torch


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def test_unit_weight_rows_have_mean_square_one(oracle_mod):
    x = _rand((1, 2, 3, 5, 32), 1)
    y = oracle_mod.prologue(x, np.ones((2, 32), np.float32), eps=1e-30)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-12)


def test_positive_scaling_of_a_token_does_not_change_it(oracle_mod):
    x = _rand((1, 2, 3, 5, 16), 2)
    s = np.float32(4.0) ** np.random.default_rng(3).integers(-2, 3, size=(1, 2, 3, 5, 1)).astype(np.float32)
    w = _rand((2, 16), 4)
    np.testing.assert_allclose(oracle_mod.prologue(x * s, w, eps=1e-30), oracle_mod.prologue(x, w, eps=1e-30),
                               rtol=1e-12, atol=1e-14)


def test_weight_acts_per_channel(oracle_mod):
    x = _rand((2, 3, 2, 4, 8), 5)
    w = _rand((3, 8), 6)
    y1 = oracle_mod.prologue(x, np.ones((3, 8), np.float32))
    y2 = oracle_mod.prologue(x, w)
    np.testing.assert_allclose(y2, y1 * w[None, :, None, None, :].astype(np.float64), rtol=1e-14)


def test_relu_and_l2(oracle_mod):
    x = _rand((1, 2, 2, 6, 16), 7)
    x[0, 1, 1, 3] = 0.0
    y = oracle_mod.prologue(x, None, relu=True, l2=True)
    assert (y >= 0).all()
    nrm = np.sqrt(np.sum(y * y, axis=-1))
    live = np.any(x > 0, axis=-1)
    np.testing.assert_allclose(nrm[live], 1.0, rtol=1e-14)
    assert (y[0, 1, 1, 3] == 0).all()
    # without the norm, ReLU then L2 of x equals the plain formula
    r = np.maximum(x.astype(np.float64), 0)
    n = np.linalg.norm(r, axis=-1, keepdims=True)
    np.testing.assert_allclose(y, np.divide(r, n, out=np.zeros_like(r), where=n > 0), rtol=1e-14)


def test_bf16_rounding_matches_torch(oracle_mod):
    x = _rand((1, 1, 2, 7, 32), 8)
    w = _rand((1, 32), 9)
    y = oracle_mod.prologue(x, w)
    yb = oracle_mod.prologue(x, w, round_to="bf16")
    want = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(yb, want)
    assert np.max(np.abs(yb - y) / np.maximum(np.abs(y), 1e-30)) <= 2.0 ** -8
