"""Error measures used by the parity tests.

max relative error: max_i |x_i - y_i| / max(|y_i|, tau) with tau = floor * max|y|
(y is the fp64 oracle).  The floor keeps elements that cancel to nearly zero
(ReLU numerators with zero-mean values) from dividing by ~0.

bf16 tokens use floor = 1e-3.  fp32 tokens use floor = 1 (the normwise error
max|x - y| / max|y|): a 1e-5 bar with a 1e-3 floor would ask near-zero
elements for an absolute error of 1e-8 * max|y|, below the resolution of the
fp32 sums that produce them.
"""
import numpy as np


def to_np(x):
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def max_rel_err(x, y, floor=1e-3):
    x = to_np(x)
    y = to_np(y)
    assert x.shape == y.shape, (x.shape, y.shape)
    if y.size == 0:
        return 0.0
    scale = float(np.max(np.abs(y)))
    if not np.all(np.isfinite(x)):
        return float("inf")
    if scale == 0.0:
        return float(np.max(np.abs(x)))
    tau = floor * scale
    return float(np.max(np.abs(x - y) / np.maximum(np.abs(y), tau)))


FLOOR = {"bf16": 1e-3, "fp32": 1.0}


def normwise_err(x, y):
    x = to_np(x)
    y = to_np(y)
    scale = float(np.max(np.abs(y))) if y.size else 0.0
    return float(np.max(np.abs(x - y))) / scale if scale else float(np.max(np.abs(x)))
