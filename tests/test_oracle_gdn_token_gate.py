"""Pins of the fp64 oracle's frame-wise Gated DeltaNet with a per-token update
gate (CPU only).

The gate of token n weights that token's terms of the frame's Gram and
value-key matrices.  The oracle is checked against: a scalar closed form; the
token-wise gated delta rule in its error-correcting form (one token per
frame); the per-frame-gate oracle when every token of a frame has the same
gate; tokens whose gate is zero dropping out of the frame; the invariance of
the update under (beta_n, k_n, v_n) -> (s beta_n, k_n / sqrt(s), v_n / sqrt(s));
and the additivity of gates over copies of one token.
"""
import numpy as np
import pytest

from brute import delta_rule_tokens


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _gates(shape, seed, mu=2.0):
    rng = np.random.default_rng(seed)
    return (1 / (1 + np.exp(-(mu + 0.5 * rng.standard_normal(shape))))).astype(np.float32)


def test_scalar_closed_form(oracle_mod):
    """D = 1, two tokens: s = alpha s0 (1 - c^2 (b1 k1^2 + b2 k2^2)) + c (b1 v1 k1 + b2 v2 k2)."""
    k = np.array([0.5, -2.0], np.float32).reshape(1, 1, 1, 2, 1)
    v = np.array([3.0, 1.5], np.float32).reshape(1, 1, 1, 2, 1)
    q = np.array([-1.0, 0.25], np.float32).reshape(1, 1, 1, 2, 1)
    a = np.array([0.75], np.float32).reshape(1, 1, 1)
    b = np.array([0.5, 0.125], np.float32).reshape(1, 1, 1, 2)
    s0 = 2.0
    c = 1 / np.sqrt(2.0)
    s = 0.75 * s0 * (1 - c * c * (0.5 * 0.25 + 0.125 * 4.0)) + c * (0.5 * 3.0 * 0.5 + 0.125 * 1.5 * -2.0)
    o, S = oracle_mod.gdn_frame_token_gate(q, k, v, a, b, np.full((1, 1, 1, 1), s0))
    assert abs(S.item() - s) < 1e-14
    np.testing.assert_allclose(o.ravel(), [-s, 0.25 * s], rtol=1e-14)


@pytest.mark.parametrize("D", [1, 4, 8])
def test_one_token_per_frame_is_the_token_wise_delta_rule(oracle_mod, D):
    F = 9
    q, k, v = (_rand((1, 1, F, 1, D), s) for s in (1, 2, 3))
    a = _gates((1, 1, F), 4)
    b = _gates((1, 1, F, 1), 5, mu=0.0)
    S0 = np.random.default_rng(6).standard_normal((1, 1, D, D))
    o, S = oracle_mod.gdn_frame_token_gate(q, k, v, a, b, S0)
    ob, Sb = delta_rule_tokens(q[0, 0, :, 0], k[0, 0, :, 0], v[0, 0, :, 0], a[0, 0], b[0, 0, :, 0], S0[0, 0])
    np.testing.assert_allclose(o[0, 0, :, 0], ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], Sb, rtol=1e-11, atol=1e-12)


def test_equal_gates_within_a_frame_match_the_frame_gate(oracle_mod):
    B, H, F, N, D = 2, 2, 4, 12, 6
    q, k, v = (_rand((B, H, F, N, D), s) for s in (7, 8, 9))
    a = _gates((B, H, F), 10)
    bf = _gates((B, H, F), 11, mu=0.0)
    bt = np.repeat(bf[..., None], N, axis=3)
    S0 = 0.3 * np.random.default_rng(12).standard_normal((B, H, D, D))
    o1, S1 = oracle_mod.gdn_frame(q, k, v, a, bf, S0)
    o2, S2 = oracle_mod.gdn_frame_token_gate(q, k, v, a, bt, S0)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)


def test_tokens_with_zero_gate_drop_out(oracle_mod):
    """Gate 0 on half of each frame's tokens equals the frame-gate scan over
    the other half (same key scale), for the state and the kept tokens' outputs."""
    B, H, F, N, D = 1, 2, 5, 10, 5
    q, k, v = (_rand((B, H, F, N, D), s) for s in (13, 14, 15))
    a = _gates((B, H, F), 16)
    bf = _gates((B, H, F), 17, mu=0.0)
    rng = np.random.default_rng(18)
    keep = np.stack([np.sort(rng.permutation(N)[: N // 2]) for _ in range(B * H * F)]).reshape(B, H, F, N // 2)
    bt = np.zeros((B, H, F, N), np.float32)
    take = lambda x: np.take_along_axis(x, keep[..., None], axis=3)
    np.put_along_axis(bt, keep, bf[..., None], axis=3)
    c = 1 / np.sqrt(D * N)
    o1, S1 = oracle_mod.gdn_frame(take(q), take(k), take(v), a, bf, None, key_scale=c)
    o2, S2 = oracle_mod.gdn_frame_token_gate(q, k, v, a, bt, None, key_scale=c)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(take(o2), o1, rtol=1e-12, atol=1e-13)


def test_gate_and_token_rescaling_leave_the_scan_unchanged(oracle_mod):
    """(beta_n, k_n, v_n) -> (s_n beta_n, k_n / sqrt(s_n), v_n / sqrt(s_n)) keeps
    both beta k k^T and beta v k^T; s_n powers of 4 keep every input exact."""
    B, H, F, N, D = 1, 2, 4, 9, 7
    q, k, v = (_rand((B, H, F, N, D), s) for s in (19, 20, 21))
    a = _gates((B, H, F), 22)
    bt = _gates((B, H, F, N), 23, mu=0.0) / 4  # gates up to 1/4, so s * beta <= 4
    m = np.random.default_rng(24).integers(-1, 2, size=(B, H, F, N)).astype(np.float32)  # s = 4^m
    s = np.power(4.0, m).astype(np.float32)
    r = np.power(2.0, m).astype(np.float32)[..., None]
    S0 = 0.2 * np.random.default_rng(25).standard_normal((B, H, D, D))
    o1, S1 = oracle_mod.gdn_frame_token_gate(q, k, v, a, bt, S0)
    o2, S2 = oracle_mod.gdn_frame_token_gate(q, k / r, v / r, a, bt * s, S0)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)


def test_gates_add_over_copies_of_a_token(oracle_mod):
    """A token given twice with gates x and beta - x equals it given once with beta."""
    B, H, F, N, D = 1, 1, 3, 6, 4
    q, k, v = (_rand((B, H, F, N, D), s) for s in (26, 27, 28))
    a = _gates((B, H, F), 29)
    rng = np.random.default_rng(30)
    bt = (rng.integers(1, 16, size=(B, H, F, N)) / 16).astype(np.float32)   # dyadic: sums exact
    x = np.floor(bt * 16 * rng.random((B, H, F, N))) / 16
    dup = lambda t: np.concatenate([t, t], axis=3)
    c = 1 / np.sqrt(D * N)
    o1, S1 = oracle_mod.gdn_frame_token_gate(q, k, v, a, bt, None, key_scale=c)
    o2, S2 = oracle_mod.gdn_frame_token_gate(dup(q), dup(k), dup(v), a,
                                             np.concatenate([x, bt - x], axis=3).astype(np.float32), None,
                                             key_scale=c)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o2[:, :, :, :N], o1, rtol=1e-12, atol=1e-13)
