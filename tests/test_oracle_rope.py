"""Pins of the oracle's rotary position embedding (CPU only).

Checked against: zero angles leaving tokens unchanged; a quarter turn sending
each channel pair (x0, x1) to (-x1, x0) exactly (the pairing of adjacent
channels and the sense of rotation); pairs routed to the frame or the token
table and the frame offset selecting rows; pair norms kept up to the tables'
cos^2 + sin^2; the product of a rotated query and key depending only on their
distance, equal to the closed form (q0 k0 + q1 k1) cos d + (q1 k0 - q0 k1) sin d
for the angle d between them; and the prologue rotating last (unit L2 rows
stay unit).
"""
import numpy as np
import pytest
import torch

from block_causal_linear_attn_amd import inputs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _const_tables(T, N, D, P, c, s):
    f = np.zeros((T, P, 2), np.float32)
    f[..., 0], f[..., 1] = c, s
    t = np.zeros((N, D // 2 - P, 2), np.float32)
    t[..., 0], t[..., 1] = c, s
    return f, t


def test_zero_angles_are_the_identity(oracle_mod):
    x = _rand((1, 2, 3, 5, 16), 1)
    f, t = _const_tables(3, 5, 16, 4, 1.0, 0.0)
    np.testing.assert_array_equal(oracle_mod.rope_rotate(x, f, t, 4), x.astype(np.float64))


def test_quarter_turn_moves_each_pair_exactly(oracle_mod):
    x = _rand((2, 1, 2, 3, 16), 2)
    f, t = _const_tables(2, 3, 16, 4, 0.0, 1.0)
    y = oracle_mod.rope_rotate(x, f, t, 4)
    np.testing.assert_array_equal(y[..., 0::2], -x[..., 1::2].astype(np.float64))
    np.testing.assert_array_equal(y[..., 1::2], x[..., 0::2].astype(np.float64))


def test_pairs_take_the_frame_or_the_token_table(oracle_mod):
    B, H, F, N, D, P = 1, 2, 3, 4, 32, 8
    x = _rand((B, H, F, N, D), 3)
    rng = np.random.default_rng(4)
    f = rng.standard_normal((F + 2, P, 2)).astype(np.float32)
    t = rng.standard_normal((N, D // 2 - P, 2)).astype(np.float32)
    base = oracle_mod.rope_rotate(x, f, t, P, 1)
    f2 = f.copy()
    f2[1:] += 1.0
    y = oracle_mod.rope_rotate(x, f2, t, P, 1)
    assert not np.allclose(y[..., :2 * P], base[..., :2 * P])
    np.testing.assert_array_equal(y[..., 2 * P:], base[..., 2 * P:])
    t2 = t + 1.0
    y = oracle_mod.rope_rotate(x, f, t2, P, 1)
    np.testing.assert_array_equal(y[..., :2 * P], base[..., :2 * P])
    assert not np.allclose(y[..., 2 * P:], base[..., 2 * P:])
    # the offset picks rows offset .. offset + F - 1 of the frame table
    np.testing.assert_array_equal(oracle_mod.rope_rotate(x, f[1:], t, P, 0), base)
    # frame f of the call turns by row offset + f
    one = oracle_mod.rope_rotate(x[:, :, 2:3], f[3:4], t, P, 0)
    np.testing.assert_array_equal(one, base[:, :, 2:3])


def test_pair_norms_are_kept(oracle_mod):
    B, H, F, N, D, P = 1, 1, 4, 30, 32, 4
    x = _rand((B, H, F, N, D), 5)
    f, t = inputs.rope_tables(F, N, 6, D, P)
    y = oracle_mod.rope_rotate(x, f, t, P)
    x64 = x.astype(np.float64)
    c2s2 = np.concatenate([np.broadcast_to(f.double().numpy()[None, :, None, :, :], (1, F, N, P, 2)),
                           np.broadcast_to(t.double().numpy()[None, None, :, :, :], (1, F, N, D // 2 - P, 2))],
                          axis=3)
    scale = (c2s2 ** 2).sum(-1)[:, None]                    # [1, 1, F, N, D/2]
    nx = x64[..., 0::2] ** 2 + x64[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx * scale, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("shift", [0, 3, 17])
def test_rotated_products_depend_on_the_distance_only(oracle_mod, shift):
    """Every pair turns with the frame index (frame_pairs = D/2): q at frame a
    and k at frame b give the closed form with angle (b - a) w_j."""
    D, T, base = 16, 40, 10000.0
    f, _ = inputs.rope_tables(T, 1, 1, D, D // 2, base=base)
    q = _rand((1, 1, T, 1, D), 6)
    k = _rand((1, 1, T, 1, D), 7)
    rq = oracle_mod.rope_rotate(q, f, None, D // 2)
    rk = oracle_mod.rope_rotate(k, f, None, D // 2)
    w = base ** (-np.arange(D // 2) / (D // 2))
    q64, k64 = q.astype(np.float64)[0, 0, :, 0], k.astype(np.float64)[0, 0, :, 0]
    for a, b in [(2, 5), (9, 4), (20, 20)]:
        a2, b2 = a + shift, b + shift
        got = rq[0, 0, a2, 0] @ rk[0, 0, b2, 0]
        d = (b2 - a2) * w
        q0, q1, k0, k1 = q64[a2, 0::2], q64[a2, 1::2], k64[b2, 0::2], k64[b2, 1::2]
        want = np.sum((q0 * k0 + q1 * k1) * np.cos(d) + (q1 * k0 - q0 * k1) * np.sin(d))
        assert abs(got - want) <= 1e-6 * (np.abs(q64[a2]).sum() * np.abs(k64[b2]).max() + 1)


def test_prologue_rotates_last(oracle_mod):
    B, H, F, N, D, P = 1, 2, 3, 12, 32, 4
    x = _rand((B, H, F, N, D), 8)
    w = _rand((H, D), 9)
    f, t = inputs.rope_tables(F, N, 4, D, P)
    rope = (f, t, P, 0)
    y = oracle_mod.prologue(x, w, eps=1e-5, relu=True, l2=True, rope=rope)
    plain = oracle_mod.prologue(x, w, eps=1e-5, relu=True, l2=True)
    np.testing.assert_array_equal(y, oracle_mod.rope_rotate(plain, *rope))
    nrm = np.sqrt((y * y).sum(-1))
    live = np.any(plain != 0, axis=-1)
    np.testing.assert_allclose(nrm[live], 1.0, rtol=2e-7)
