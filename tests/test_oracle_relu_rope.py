"""Pins of the oracle's block-causal linear attention with separate numerator
and denominator features (the ReLU scan with a rotary embedding), CPU only.

Checked against: equal features reduce it to the ReLU oracle (the ReLU
features of q and k on both sides); a brute-force quadratic sum over the
visible tokens of every query for block sizes 1, 2 and 3, with an initial
state; the normaliser depending on the denominator features only (rotations
move S, never z); outputs unchanged when every position shifts by the same
number of frames (the rotated product depends on distances only); and chunked
calls through the carried (S, z) equalling one call.
"""
import numpy as np
import pytest

from block_causal_linear_attn_amd import inputs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _relu(x):
    x = np.asarray(x, np.float64)
    return np.where(np.signbit(x), 0.0, x)


@pytest.mark.parametrize("bf", [1, 3])
def test_equal_features_give_the_relu_scan(oracle_mod, bf):
    B, H, F, N, D = 1, 2, 5, 7, 8
    q, k, v = (_rand((B, H, F, N, D), s) for s in (1, 2, 3))
    S0 = np.random.default_rng(4).standard_normal((B, H, D, D))
    z0 = np.abs(np.random.default_rng(5).standard_normal((B, H, D)))
    o, S, z = oracle_mod.linear_block_split(_relu(q), _relu(k), _relu(q), _relu(k), v, S0, z0, block_frames=bf)
    ro, rS, rz = oracle_mod.relu_block(q, k, v, S0, z0, block_frames=bf)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, rS, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z, rz, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("bf", [1, 2, 3])
def test_brute_force_quadratic_sum(oracle_mod, bf):
    B, H, F, N, D = 1, 1, 5, 3, 4
    rng = np.random.default_rng(6)
    qn, kn = rng.standard_normal((2, B, H, F, N, D))
    qd, kd = np.abs(rng.standard_normal((2, B, H, F, N, D)))
    v = _rand((B, H, F, N, D), 7)
    S0 = rng.standard_normal((B, H, D, D))
    z0 = np.abs(rng.standard_normal((B, H, D)))
    o, S, z = oracle_mod.linear_block_split(qn, kn, qd, kd, v, S0, z0, block_frames=bf, eps=1e-3)
    for f in range(F):
        last = min(F, (f // bf + 1) * bf)     # the query's block ends here; every earlier frame is visible
        for n in range(N):
            num = S0[0, 0] @ qn[0, 0, f, n]
            den = z0[0, 0] @ qd[0, 0, f, n] + 1e-3
            for g in range(last):
                for m in range(N):
                    num = num + (kn[0, 0, g, m] @ qn[0, 0, f, n]) * v[0, 0, g, m].astype(np.float64)
                    den = den + kd[0, 0, g, m] @ qd[0, 0, f, n]
            np.testing.assert_allclose(o[0, 0, f, n], num / den, rtol=1e-11, atol=1e-12)


def test_rotations_move_the_state_not_the_normaliser(oracle_mod):
    B, H, F, N, D, P = 1, 2, 3, 6, 16, 4
    q, k, v = (_rand((B, H, F, N, D), s) for s in (8, 9, 10))
    f, t = inputs.rope_tables(F, N, 3, D, P)
    kn, kd = oracle_mod.relu_rope_features(k, rope=(f, t, P, 0))
    qn, qd = oracle_mod.relu_rope_features(q, rope=(f, t, P, 0))
    o, S, z = oracle_mod.linear_block_split(qn, kn, qd, kd, v)
    _, rS, rz = oracle_mod.relu_block(q, k, v)
    np.testing.assert_array_equal(z, oracle_mod.linear_block_split(_relu(q), _relu(k), _relu(q), _relu(k), v)[2])
    np.testing.assert_allclose(z, rz, rtol=1e-12)
    assert not np.allclose(S, rS)


@pytest.mark.parametrize("shift", [1, 7])
def test_a_common_shift_of_positions_leaves_outputs(oracle_mod, shift):
    """All pairs turn with the frame (frame_pairs = D/2): moving every frame's
    position by `shift` rows of the table leaves the outputs (and z) as they
    were, up to the fp32 tables' rounding."""
    B, H, F, N, D = 1, 1, 4, 5, 16
    q, k, v = (_rand((B, H, F, N, D), s) for s in (11, 12, 13))
    f, _ = inputs.rope_tables(F + shift, 1, 1, D, D // 2)
    outs = []
    for off in (0, shift):
        rope = (f, None, D // 2, off)
        kn, kd = oracle_mod.relu_rope_features(k, rope=rope)
        qn, qd = oracle_mod.relu_rope_features(q, rope=rope)
        outs.append(oracle_mod.linear_block_split(qn, kn, qd, kd, v, block_frames=2))
    np.testing.assert_allclose(outs[1][0], outs[0][0], rtol=2e-5, atol=2e-6 * np.abs(outs[0][0]).max())
    np.testing.assert_array_equal(outs[1][2], outs[0][2])


def test_chunked_calls_through_the_carry_equal_one_call(oracle_mod):
    B, H, F, N, D, P = 1, 2, 6, 4, 8, 0
    q, k, v = (_rand((B, H, F, N, D), s) for s in (14, 15, 16))
    f, t = inputs.rope_tables(F, N, 2, D, P)
    qn, qd = oracle_mod.relu_rope_features(q, rope=(f, t, P, 0))
    kn, kd = oracle_mod.relu_rope_features(k, rope=(f, t, P, 0))
    o, S, z = oracle_mod.linear_block_split(qn, kn, qd, kd, v, block_frames=2)
    S1, z1 = None, None
    for f0 in (0, 2, 4):
        sl = slice(f0, f0 + 2)
        part, S1, z1 = oracle_mod.linear_block_split(qn[:, :, sl], kn[:, :, sl], qd[:, :, sl], kd[:, :, sl],
                                                     v[:, :, sl], S1, z1, block_frames=2)
        np.testing.assert_allclose(part, o[:, :, sl], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S1, S, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z1, z, rtol=1e-12, atol=1e-13)
