"""Pins of the fp64 oracle's ReLU block-causal linear attention (CPU only).

Each test checks the oracle against something other than itself: hand-derived
values, the quadratic masked-sum form, special cases with closed forms, and
invariants (token permutation, linearity in v, chunking through the carried
state).
"""
import json
import os

import numpy as np
import pytest

from brute import relu, relu_masked_sum

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, positive_frac=None):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape).astype(np.float32)


def test_hand_values(oracle_mod):
    spec = json.load(open(os.path.join(GOLDEN, "relu_hand_values.json")))
    for case in spec["cases"]:
        shape = tuple(case["shape"])
        B, H, F, N, D = shape
        q = np.array(case["q"], np.float32).reshape(shape)
        k = np.array(case["k"], np.float32).reshape(shape)
        v = np.array(case["v"], np.float32).reshape(shape)
        o, S, z = oracle_mod.relu_block(q, k, v, block_frames=case["block_frames"], eps=spec["eps"])
        np.testing.assert_allclose(o.ravel(), case["o"], rtol=1e-13, atol=0, err_msg=case["name"])
        np.testing.assert_allclose(S.ravel(), case["S"], rtol=1e-13, atol=0, err_msg=case["name"])
        np.testing.assert_allclose(z.ravel(), case["z"], rtol=1e-13, atol=0, err_msg=case["name"])


@pytest.mark.parametrize("block_frames", [1, 2, 3, 5])
@pytest.mark.parametrize("with_state", [False, True])
def test_matches_quadratic_masked_sum(oracle_mod, block_frames, with_state):
    B, H, F, N, D = 2, 3, 5, 4, 6
    q, k, v = (_rand((B, H, F, N, D), s) for s in (1, 2, 3))
    S0 = z0 = None
    if with_state:
        rng = np.random.default_rng(9)
        S0 = rng.standard_normal((B, H, D, D))
        z0 = rng.uniform(0.5, 2.0, (B, H, D))
    o, S, z = oracle_mod.relu_block(q, k, v, S0, z0, block_frames=block_frames, eps=1e-6)
    ob, Sb, zb = relu_masked_sum(q, k, v, block_frames, 1e-6, S0, z0)
    np.testing.assert_allclose(o, ob, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, Sb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, zb, rtol=1e-12, atol=1e-12)


def test_single_frame_is_plain_linear_attention(oracle_mod):
    """F = 1: O = (A V) / (A 1 + eps) with A = phi(Q) phi(K)^T (non-causal)."""
    B, H, F, N, D = 1, 2, 1, 7, 5
    q, k, v = (_rand((B, H, F, N, D), s) for s in (4, 5, 6))
    o, _, _ = oracle_mod.relu_block(q, k, v, eps=1e-6)
    for h in range(H):
        A = relu(q[0, h, 0]) @ relu(k[0, h, 0]).T
        ref = (A @ v[0, h, 0].astype(np.float64)) / (A.sum(axis=1, keepdims=True) + 1e-6)
        np.testing.assert_allclose(o[0, h, 0], ref, rtol=1e-11, atol=1e-13)


def test_token_permutation_within_frame(oracle_mod):
    B, H, F, N, D = 1, 2, 3, 6, 4
    q, k, v = (_rand((B, H, F, N, D), s) for s in (7, 8, 9))
    perm = np.random.default_rng(1).permutation(N)
    o, S, z = oracle_mod.relu_block(q, k, v)
    op, Sp, zp = oracle_mod.relu_block(q[:, :, :, perm], k[:, :, :, perm], v[:, :, :, perm])
    np.testing.assert_allclose(op, o[:, :, :, perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sp, S, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(zp, z, rtol=1e-12, atol=1e-13)


def test_linear_in_values(oracle_mod):
    """O(v1 + v2) = O(v1) + O(v2) and O(-2 v) = -2 O(v); z does not depend on v.

    Small-integer values keep v1 + v2 exact in float32.
    """
    B, H, F, N, D = 1, 2, 3, 5, 4
    q, k = (_rand((B, H, F, N, D), s) for s in (10, 11))
    rng = np.random.default_rng(12)
    v1 = rng.integers(-8, 9, (B, H, F, N, D)).astype(np.float32)
    v2 = rng.integers(-8, 9, (B, H, F, N, D)).astype(np.float32)
    o1, S1, z1 = oracle_mod.relu_block(q, k, v1)
    o2, S2, z2 = oracle_mod.relu_block(q, k, v2)
    o12, S12, z12 = oracle_mod.relu_block(q, k, v1 + v2)
    np.testing.assert_allclose(o12, o1 + o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S12, S1 + S2, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(z12, z1)
    om, Sm, _ = oracle_mod.relu_block(q, k, -2 * v1)
    np.testing.assert_array_equal(om, -2 * o1)
    np.testing.assert_array_equal(Sm, -2 * S1)


@pytest.mark.parametrize("split", [[1, 1, 1, 1, 1, 1], [4, 2], [3, 3], [5, 1]])
def test_chunked_calls_equal_one_call(oracle_mod, split):
    """Carrying (S, z) between calls reproduces one call exactly (frame-causal)."""
    B, H, F, N, D = 1, 2, 6, 3, 4
    q, k, v = (_rand((B, H, F, N, D), s) for s in (13, 14, 15))
    o_all, S_all, z_all = oracle_mod.relu_block(q, k, v)
    S = z = None
    f0 = 0
    outs = []
    for nf in split:
        o, S, z = oracle_mod.relu_block(q[:, :, f0:f0 + nf], k[:, :, f0:f0 + nf],
                                        v[:, :, f0:f0 + nf], S, z)
        outs.append(o)
        f0 += nf
    np.testing.assert_array_equal(np.concatenate(outs, axis=2), o_all)
    np.testing.assert_array_equal(S, S_all)
    np.testing.assert_array_equal(z, z_all)


def test_state_only_mode_matches(oracle_mod):
    B, H, F, N, D = 1, 2, 3, 4, 4
    q, k, v = (_rand((B, H, F, N, D), s) for s in (16, 17, 18))
    _, S, z = oracle_mod.relu_block(q, k, v)
    o2, S2, z2 = oracle_mod.relu_block(None, k, v, with_output=False)
    assert o2 is None
    np.testing.assert_array_equal(S, S2)
    np.testing.assert_array_equal(z, z2)


def test_all_negative_queries_give_zero_outputs(oracle_mod):
    B, H, F, N, D = 1, 1, 2, 3, 4
    q = -np.abs(_rand((B, H, F, N, D), 19))
    k, v = (_rand((B, H, F, N, D), s) for s in (20, 21))
    o, _, _ = oracle_mod.relu_block(q, k, v)
    assert np.all(o == 0.0)
