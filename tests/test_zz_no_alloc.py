"""ls_gdn_frame_forward_noalloc, the GDN scan for callers that cannot allocate
device memory, against ls_gdn_frame_forward (needs an MI355X).

Both run the same kernels on the same inputs, the first in the library's
static device scratch and the second in a caller workspace, so their results
must agree to the parity bar (and in fact bit for bit).  Two calls run in a
row, the second smaller than the first, so the second finds the first's
records, states and flags still in the scratch.
"""
import pytest
import torch

from metrics import max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def ls():
    assert torch.cuda.is_available()
    from block_causal_linear_attn_amd import binding
    return binding


def _pair(ls, gen, oracle_mod, B, H, F, N, seed, with_state):
    x = gen.gdn_inputs(B, H, F, N, 128, "bf16", seed=seed, device=DEV, l2_keys=True)
    S0 = 0.05 * torch.randn((B, H, 128, 128), generator=torch.Generator(DEV).manual_seed(seed), device=DEV) \
        if with_state else None
    out = torch.full_like(x["q"], float("nan"))
    so = torch.full((B, H, 128, 128), float("nan"), device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    ls.ls_gdn_frame_forward_noalloc(x["q"], x["k"], x["v"], x["alpha"], x["beta"], out, S0, so, fault=fault)
    ref_o, ref_S = ls.ls_gdn_frame_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0)
    torch.cuda.synchronize()
    assert int(fault.item()) == 0
    assert max_rel_err(out, ref_o) <= 2e-2 and max_rel_err(so, ref_S) <= 1e-2
    assert torch.equal(out, ref_o) and torch.equal(so, ref_S)
    return x, S0, out, so


def test_noalloc_matches_the_workspace_entry_point_twice(ls, oracle_mod):
    from block_causal_linear_attn_amd import inputs as gen
    # a single-frame step of 96 heads (phased launch, 19 MB of scratch) ...
    _pair(ls, gen, oracle_mod, 4, 24, 1, 920, 41, True)
    # ... then a smaller call (frame-interleaved launch) over what it left behind
    x, S0, out, so = _pair(ls, gen, oracle_mod, 1, 3, 5, 300, 42, True)
    ro, rS = oracle_mod.gdn_frame(*(x[n].float().cpu() for n in ("q", "k", "v", "alpha", "beta")), S0.cpu())
    assert max_rel_err(out, ro) <= 2e-2 and max_rel_err(so, rS) <= 1e-2


def test_noalloc_rejects_calls_beyond_the_scratch(ls):
    from block_causal_linear_attn_amd import inputs as gen
    B, H, F, N = 1, 24, 20, 64  # 20 frames of 24 heads: records and states need ~94 MB
    shp = ls.ls_shape(B, H, F, N, 128, ls.LS_DTYPE_BF16)
    assert ls.lib.ls_gdn_frame_workspace_size(ls.ctypes.byref(shp)) > ls.NOALLOC_SCRATCH_BYTES
    x = gen.gdn_inputs(B, H, F, N, 128, "bf16", seed=43, device=DEV, l2_keys=True)
    out = torch.full_like(x["q"], 7.0)
    with pytest.raises(ls.LinscanError) as e:
        ls.ls_gdn_frame_forward_noalloc(x["q"], x["k"], x["v"], x["alpha"], x["beta"], out)
    assert e.value.status == 6 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
