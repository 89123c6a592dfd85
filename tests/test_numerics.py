"""Why the GDN output product carries the state as two bf16 terms (CPU only).

The output o = S_f q sums D products that often cancel.  Under the parity
metric (relative error with a floor of 1e-3 of the largest output), rounding
S_f to bf16 alone leaves errors of about 2^-9 of the products' size in the
cancelled outputs, far above the 2e-2 bound, while S_f = hi + lo (two bf16
terms, 16 significant bits) keeps the product error well inside it.  States
come from the fp64 oracle on the 720p 60 s GDN inputs (two heads, twelve
frames).
"""
import numpy as np
import torch

from block_causal_linear_attn_amd import inputs as gen
from metrics import max_rel_err, FLOOR


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_bf16_state_breaks_output_bound_hi_lo_does_not(oracle_mod):
    x = gen.gdn_inputs(1, 2, 12, 920, 128, "bf16", seed=3, alpha_mu=3.0, l2_keys=True)
    q = x["q"].float().numpy()
    f = 11
    _, S = oracle_mod.gdn_frame(x["q"][:, :, :f + 1], x["k"][:, :, :f + 1], x["v"][:, :, :f + 1],
                                x["alpha"][:, :, :f + 1], x["beta"][:, :, :f + 1])
    S32 = S.astype(np.float32)
    hi = _bf16(S32)
    lo = _bf16(S32 - hi)
    qf = q[:, :, f].astype(np.float64)
    exact = np.einsum("bhij,bhnj->bhni", S, qf)
    one = np.einsum("bhij,bhnj->bhni", hi.astype(np.float64), qf)
    two = np.einsum("bhij,bhnj->bhni", hi.astype(np.float64) + lo.astype(np.float64), qf)
    e_one = max_rel_err(one, exact, FLOOR["bf16"])
    e_two = max_rel_err(two, exact, FLOOR["bf16"])
    print("output error, S as one bf16 term: %.3e, as hi + lo: %.3e" % (e_one, e_two))
    assert e_one > 2e-2
    assert e_two < 5e-3
