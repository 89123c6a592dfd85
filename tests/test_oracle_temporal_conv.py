"""Pins of the fp64 oracle's block-causal temporal convolution (kernel 3 along
frames, zero frame after each block, previous block's last frame carried in).

Checked against: numpy's correlation of each (token, channel) sequence padded
with the carried frame in front and a zero frame behind (one block); tap
vectors that give the identity and a one-frame shift; one-frame blocks, which
never see the next frame; and a call over several blocks equalling one call
per block chained through the carried frame.
"""
import numpy as np
import pytest


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("with_carry", [False, True])
def test_one_block_is_a_correlation_of_the_padded_sequence(oracle_mod, with_carry):
    B, H, F, N, D = 2, 3, 6, 4, 5
    x = _rand((B, H, F, N, D), 1)
    w = _rand((H, D, 3), 2)
    bias = _rand((H, D), 3)
    carry = _rand((B, H, N, D), 4) if with_carry else None
    y, co = oracle_mod.temporal_conv3(x, w, bias, carry, block_frames=F)
    for b in range(B):
        for h in range(H):
            for n in range(N):
                for d in range(D):
                    first = 0.0 if carry is None else float(carry[b, h, n, d])
                    seq = np.concatenate([[first], x[b, h, :, n, d].astype(np.float64), [0.0]])
                    want = np.correlate(seq, w[h, d].astype(np.float64), mode="valid") + bias[h, d]
                    np.testing.assert_allclose(y[b, h, :, n, d], want, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(co, x[:, :, F - 1])


def test_identity_and_shift_taps_are_exact(oracle_mod):
    B, H, F, N, D = 1, 2, 5, 3, 4
    x = _rand((B, H, F, N, D), 5)
    carry = _rand((B, H, N, D), 6)
    ident = np.tile(np.array([0, 1, 0], np.float32), (H, D, 1))
    y, _ = oracle_mod.temporal_conv3(x, ident, None, carry, block_frames=2)
    np.testing.assert_array_equal(y, x)
    shift = np.tile(np.array([1, 0, 0], np.float32), (H, D, 1))
    y, _ = oracle_mod.temporal_conv3(x, shift, None, carry, block_frames=2)
    np.testing.assert_array_equal(y[:, :, 0], carry)
    np.testing.assert_array_equal(y[:, :, 1:], x[:, :, :-1])


def test_one_frame_blocks_never_see_the_next_frame(oracle_mod):
    B, H, F, N, D = 1, 1, 5, 2, 3
    x = _rand((B, H, F, N, D), 7)
    w = _rand((H, D, 3), 8)
    y, _ = oracle_mod.temporal_conv3(x, w, None, None, block_frames=1)
    x64, w64 = x.astype(np.float64), w.astype(np.float64)
    prev = np.concatenate([np.zeros_like(x64[:, :, :1]), x64[:, :, :-1]], axis=2)
    want = w64[None, :, None, None, :, 0] * prev + w64[None, :, None, None, :, 1] * x64
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("block", [1, 2, 3])
def test_blocks_chain_through_the_carried_frame(oracle_mod, block):
    """One call over blocks of `block` frames equals one call per block, each
    taking the previous block's last frame as its carry."""
    B, H, F, N, D = 1, 2, 7, 3, 4
    x = _rand((B, H, F, N, D), 9)
    w = _rand((H, D, 3), 10)
    bias = _rand((H, D), 11)
    carry = _rand((B, H, N, D), 12)
    y, co = oracle_mod.temporal_conv3(x, w, bias, carry, block_frames=block)
    c = carry
    for f0 in range(0, F, block):
        sl = slice(f0, min(F, f0 + block))
        part, c_next = oracle_mod.temporal_conv3(x[:, :, sl], w, bias, c, block_frames=block)
        np.testing.assert_allclose(y[:, :, sl], part, rtol=1e-14, atol=1e-14)
        c = c_next.astype(np.float32)
    np.testing.assert_array_equal(co, c)
