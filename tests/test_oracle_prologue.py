"""Pins of the oracle's per-token prologue (RMSNorm with weights, ReLU, L2).

Checked against: rows of mean square 1 (unit weight, eps -> 0); invariance
under positive scaling of a token; the weight acting per channel; ReLU leaving
no negative entry; unit L2 norms, and an all-zero row staying zero; and the
bf16 rounding agreeing with torch's own conversion of values exact in fp32,
going to the nearer neighbour next to halfway points (one rounding, not
two), and staying within half a bf16 step.

The composed prologue is pinned by hand-derived rows
(tests/golden/prologue_hand_values.json): where eps sits (inside the square
root, at an eps large enough to matter), weights applied per channel after
the norm, the order RMSNorm -> ReLU -> L2 -> rotation with weights on, and the
bf16 rounding of the result.  Planted mistakes (eps outside the root, ReLU
before the norm, the rotation first, weights inside the mean) each fail them.
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


def test_bf16_rounding_of_fp32_values_matches_torch(oracle_mod):
    """On values that are exact in fp32, one rounding from fp64 is torch's
    fp32 -> bf16 conversion (round to nearest even)."""
    x = _rand((4096,), 8) * np.float32(3.0) ** np.random.default_rng(10).integers(-8, 9, 4096).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle_mod.round_bf16(x.astype(np.float64)), want)


def test_bf16_rounding_near_halfway_points(oracle_mod):
    """Near 1 the bf16 step is 2^-7: halfway points go to the even neighbour,
    and a value past one by less than fp32 resolves (2^-30) goes to the
    nearer neighbour (rounding through fp32 would land on the halfway point
    first and pick the even one)."""
    e = 2.0 ** -7
    cases = [
        (1 + e / 2, 1.0),                     # tie, 1.0 is even
        (1 + 3 * e / 2, 1 + 2 * e),           # tie, 1 + 2^-6 is even
        (1 + e / 2 + 2.0 ** -30, 1 + e),      # just past the tie
        (1 + e / 2 - 2.0 ** -30, 1.0),        # just before it
        (1 + 3 * e / 2 - 2.0 ** -30, 1 + e),
        (0.0, 0.0),
    ]
    y = np.array([c[0] for c in cases] + [-c[0] for c in cases])
    want = np.array([c[1] for c in cases] + [-c[1] for c in cases])
    np.testing.assert_array_equal(oracle_mod.round_bf16(y), want)
    via_fp32 = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert via_fp32[2] == 1.0  # the double rounding this avoids


def test_bf16_rounding_is_within_half_a_step(oracle_mod):
    x = _rand((1, 1, 2, 7, 32), 8)
    w = _rand((1, 32), 9)
    y = oracle_mod.prologue(x, w)
    yb = oracle_mod.prologue(x, w, round_to="bf16")
    np.testing.assert_array_equal(yb, oracle_mod.round_bf16(y))
    # bf16 values (fp32 with 16 zero low bits) within half a step of y
    assert (yb.astype(np.float32).view(np.uint32) & 0xFFFF == 0).all()
    assert np.array_equal(yb.astype(np.float32).astype(np.float64), yb)
    step = 2.0 ** (np.floor(np.log2(np.abs(y))) - 7)
    assert (np.abs(yb - y) <= step / 2).all()


# ---- hand-derived values (tests/golden/prologue_hand_values.json) ----------

import json
import math
import os
from fractions import Fraction

import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "prologue_hand_values.json")


def _value(s):
    """'p/q' -> the fraction; 'sqrt:p/q' -> its square root (as float64)."""
    if s.startswith("sqrt:"):
        return math.sqrt(Fraction(s[5:]))
    return float(Fraction(s))


def _cases():
    with open(GOLDEN) as fh:
        return json.load(fh)["cases"]


def _args(case):
    D = len(case["x"])
    x = np.array(case["x"], np.float32).reshape(1, 1, 1, 1, D)
    w = np.array(case["weight"], np.float32).reshape(1, D)
    rope = None
    if case["rope"] is not None:
        r = case["rope"]
        rope = (np.array(r["frame_cs"], np.float32), np.array(r["token_cs"], np.float32), r["frame_pairs"],
                r["frame_offset"])
    return x, w, rope


def _run(fn, case, round_to=None):
    x, w, rope = _args(case)
    return np.asarray(fn(x, w, eps=case["eps"], relu=case["relu"], l2=case["l2"], round_to=round_to,
                         rope=rope)).reshape(-1)


def _matches(fn, case):
    want = np.array([_value(s) for s in case["want"]])
    want_b = np.array([_value(s) for s in case["want_bf16"]])
    got = _run(fn, case)
    got_b = _run(fn, case, "bf16")
    return bool(np.allclose(got, want, rtol=1e-14, atol=1e-15) and np.array_equal(got_b, want_b))


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_prologue_hand_values(oracle_mod, case):
    want = np.array([_value(s) for s in case["want"]])
    np.testing.assert_allclose(_run(oracle_mod.prologue, case), want, rtol=1e-14, atol=1e-15)
    want_b = np.array([_value(s) for s in case["want_bf16"]])
    np.testing.assert_array_equal(_run(oracle_mod.prologue, case, "bf16"), want_b)


# Plausible mistakes, each the oracle's prologue with one change; the hand
# values must reject every one of them.
def _mutant(oracle_mod, eps_outside=False, relu_first=False, rope_first=False, weight_in_mean=False):
    def fn(x, weight=None, eps=1e-6, relu=False, l2=False, round_to=None, rope=None):
        y = np.asarray(x, np.float64)
        if rope_first and rope is not None:
            y = oracle_mod.rope_rotate(y, *rope)
        if relu_first and relu:
            y = np.maximum(y, 0.0)
        if weight is not None:
            w = np.asarray(weight, np.float64)[None, :, None, None, :]
            ms = np.mean((y * w if weight_in_mean else y) ** 2, axis=-1, keepdims=True)
            r = np.sqrt(ms) + eps if eps_outside else np.sqrt(ms + eps)
            y = y / r * w
        if relu and not relu_first:
            y = np.maximum(y, 0.0)
        if l2:
            n = np.sqrt(np.sum(y * y, axis=-1, keepdims=True))
            y = np.where(n > 0, y / np.where(n > 0, n, 1.0), 0.0)
        if rope is not None and not rope_first:
            y = oracle_mod.rope_rotate(y, *rope)
        return oracle_mod.round_bf16(y) if round_to == "bf16" else y
    return fn


def test_prologue_hand_values_reject_planted_mistakes(oracle_mod):
    cases = _cases()
    assert all(_matches(_mutant(oracle_mod), c) for c in cases)  # the mutant frame itself is faithful
    for kw in ({"eps_outside": True}, {"relu_first": True}, {"rope_first": True}, {"weight_in_mean": True}):
        assert not all(_matches(_mutant(oracle_mod, **kw), c) for c in cases), kw
