"""Pins of the fp64 oracle's reversed frame-wise Gated DeltaNet that resets at
chunk boundaries (CPU only).

Checked against: the forward oracle run over the frame-reversed sequence (one
chunk covering every frame); the closed form for one-frame chunks (no
history: S = beta U); chunks being independent calls; and the direction of
the context (a frame's output depends on the later frames of its chunk and
on nothing earlier or outside the chunk).
"""
import numpy as np
import pytest


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _gates(B, H, F, seed):
    rng = np.random.default_rng(seed)
    a = 1 / (1 + np.exp(-(2.0 + 0.5 * rng.standard_normal((B, H, F)))))
    b = 1 / (1 + np.exp(-rng.standard_normal((B, H, F))))
    return a.astype(np.float32), b.astype(np.float32)


def _inputs(B, H, F, N, D, seed):
    q, k, v = (_rand((B, H, F, N, D), seed + i) for i in range(3))
    a, b = _gates(B, H, F, seed + 3)
    return q, k, v, a, b


@pytest.mark.parametrize("chunk", [5, 6, 50])
def test_one_chunk_is_the_forward_scan_of_the_reversed_frames(oracle_mod, chunk):
    B, H, F, N, D = 1, 2, 5, 7, 6
    q, k, v, a, b = _inputs(B, H, F, N, D, 1)
    rev = lambda t: np.ascontiguousarray(t[:, :, ::-1])
    o = oracle_mod.gdn_frame_reversed(q, k, v, a, b, chunk)
    of, _ = oracle_mod.gdn_frame(rev(q), rev(k), rev(v), rev(a), rev(b))
    np.testing.assert_allclose(o, rev(of), rtol=1e-12, atol=1e-13)


def test_one_frame_chunks_have_no_history(oracle_mod):
    """chunk = 1: S_f = beta_f U_f, so o_n = beta_f c sum_m v_m (k_m . q_n)."""
    B, H, F, N, D = 1, 1, 4, 5, 3
    q, k, v, a, b = _inputs(B, H, F, N, D, 2)
    o = oracle_mod.gdn_frame_reversed(q, k, v, a, b, 1)
    c = 1 / np.sqrt(D * N)
    for f in range(F):
        kf, vf, qf = (t[0, 0, f].astype(np.float64) for t in (k, v, q))
        want = b[0, 0, f] * c * (qf @ kf.T) @ vf        # [N, D]
        np.testing.assert_allclose(o[0, 0, f], want, rtol=1e-12, atol=1e-13)


def test_chunks_are_independent_calls(oracle_mod):
    B, H, F, N, D, C = 2, 1, 7, 4, 5, 3
    q, k, v, a, b = _inputs(B, H, F, N, D, 3)
    o = oracle_mod.gdn_frame_reversed(q, k, v, a, b, C)
    for c0 in range(0, F, C):
        sl = slice(c0, min(F, c0 + C))
        part = oracle_mod.gdn_frame_reversed(q[:, :, sl], k[:, :, sl], v[:, :, sl], a[:, :, sl], b[:, :, sl], F)
        np.testing.assert_allclose(o[:, :, sl], part, rtol=1e-12, atol=1e-13)


def test_context_comes_from_later_frames_of_the_chunk_only(oracle_mod):
    B, H, F, N, D, C = 1, 1, 8, 3, 4, 4
    q, k, v, a, b = _inputs(B, H, F, N, D, 4)
    base = oracle_mod.gdn_frame_reversed(q, k, v, a, b, C)
    for f in range(F):  # perturb frame f's values and keys
        k2, v2 = k.copy(), v.copy()
        k2[:, :, f] += 1.0
        v2[:, :, f] -= 2.0
        o = oracle_mod.gdn_frame_reversed(q, k2, v2, a, b, C)
        changed = [not np.allclose(o[:, :, g], base[:, :, g], rtol=0, atol=0) for g in range(F)]
        chunk0 = (f // C) * C
        assert changed == [chunk0 <= g <= f for g in range(F)], (f, changed)
