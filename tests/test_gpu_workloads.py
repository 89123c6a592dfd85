"""Full-size video workloads on the GPU, in the launch configuration the
benchmark times, checked against the fp64 oracle on sampled (batch, head)
pairs (needs an MI355X).

Every (batch, head) of the scan is independent, so the oracle recomputes a
few of them end to end from the same input values and compares every output
token and the final state of those heads.
"""
import numpy as np
import pytest
import torch

from metrics import max_rel_err

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"


@pytest.fixture(scope="module")
def ls():
    assert torch.cuda.is_available()
    from block_causal_linear_attn_amd import binding
    return binding


@pytest.fixture(scope="module")
def gen():
    from block_causal_linear_attn_amd import inputs
    return inputs


def check(name, got, want, tol):
    err = max_rel_err(got, want)
    print("%-44s max rel err %.3e (tol %.0e)" % (name, err, tol), flush=True)
    assert err <= tol, (name, err)


def _heads(t, hs):
    """[B, H, ...] device tensor -> CPU float32 copy of heads hs (batch 0)."""
    return t[:, hs].float().cpu()


def test_sana_video_480p_5s(ls, gen, oracle_mod):
    w = gen.WORKLOADS["sana_video_480p_5s"]
    x = gen.workload_call_inputs(w, 0, device=DEV)
    o, S, z = ls.ls_relu_block_forward(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    hs = [0, 37, 69]
    ro, rS, rz = oracle_mod.relu_block(_heads(x["q"], hs), _heads(x["k"], hs), _heads(x["v"], hs))
    check("480p-5s relu o (3 heads)", _heads(o, hs), ro, 2e-2)
    check("480p-5s relu S", _heads(S, hs), rS, 1e-2)
    check("480p-5s relu z", _heads(z, hs), rz, 1e-2)


def test_sana_video_720p_minute_rollout(ls, gen, oracle_mod):
    """241 frames in 25 calls of at most 10 frames chained through ls_state_carry."""
    w = gen.WORKLOADS["sana_video_720p_minute"]
    hs = [5, 52]
    cache = torch.zeros((w.B, w.H, w.D, w.D), device=DEV)
    ncache = torch.zeros((w.B, w.H, w.D), device=DEV)
    S_blk = torch.empty_like(cache)
    z_blk = torch.empty_like(ncache)
    qs, ks, vs, os_ = [], [], [], []
    for call in range(len(w.calls)):
        x = gen.workload_call_inputs(w, call, device=DEV)
        o, _, _ = ls.ls_relu_block_forward(x["q"], x["k"], x["v"], cache, ncache,
                                           state_out=S_blk, norm_out=z_blk)
        ls.ls_state_carry(S_blk, cache, z_blk, ncache)
        for lst, t in ((qs, x["q"]), (ks, x["k"]), (vs, x["v"]), (os_, o)):
            lst.append(_heads(t, hs))
        del x, o
    torch.cuda.synchronize()
    q, k, v, o = (torch.cat(l, dim=2) for l in (qs, ks, vs, os_))
    assert q.shape[2] == 241
    ro, rS, rz = oracle_mod.relu_block(q, k, v)
    check("720p-minute relu o (2 heads, 241 frames)", o, ro, 2e-2)
    check("720p-minute relu S", _heads(cache, hs), rS, 1e-2)
    check("720p-minute relu z", _heads(ncache, hs), rz, 1e-2)


def test_sana_video_720p_minute_rollout_d112(ls, gen, oracle_mod):
    """The rollout at head dim 112 (wide MFMA path), one sampled head over all 241 frames."""
    w = gen.WORKLOADS["sana_video_720p_minute_d112"]
    hs = [13]
    cache = torch.zeros((w.B, w.H, w.D, w.D), device=DEV)
    ncache = torch.zeros((w.B, w.H, w.D), device=DEV)
    S_blk = torch.empty_like(cache)
    z_blk = torch.empty_like(ncache)
    qs, ks, vs, os_ = [], [], [], []
    for call in range(len(w.calls)):
        x = gen.workload_call_inputs(w, call, device=DEV)
        o, _, _ = ls.ls_relu_block_forward(x["q"], x["k"], x["v"], cache, ncache,
                                           state_out=S_blk, norm_out=z_blk)
        ls.ls_state_carry(S_blk, cache, z_blk, ncache)
        for lst, t in ((qs, x["q"]), (ks, x["k"]), (vs, x["v"]), (os_, o)):
            lst.append(_heads(t, hs))
        del x, o
    torch.cuda.synchronize()
    q, k, v, o = (torch.cat(l, dim=2) for l in (qs, ks, vs, os_))
    ro, rS, rz = oracle_mod.relu_block(q, k, v)
    check("720p-minute D112 relu o (1 head, 241 frames)", o, ro, 2e-2)
    check("720p-minute D112 relu S", _heads(cache, hs), rS, 1e-2)
    check("720p-minute D112 relu z", _heads(ncache, hs), rz, 1e-2)


def test_sana_wm_720p_60s_d112(ls, gen, oracle_mod):
    w = gen.WORKLOADS["sana_wm_720p_60s_d112"]
    x = gen.workload_call_inputs(w, 0, device=DEV)
    o, S = ls.ls_gdn_frame_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    hs = [0, 27]
    ro, rS = oracle_mod.gdn_frame(*(_heads(x[n], hs) for n in ("q", "k", "v", "alpha", "beta")))
    check("wm-60s D112 gdn o (2 heads, 181 frames)", _heads(o, hs), ro, 2e-2)
    check("wm-60s D112 gdn S", _heads(S, hs), rS, 1e-2)


def test_sana_wm_720p_60s_token_gate(ls, gen, oracle_mod):
    """The 60 s GDN workload with one update gate per token (B1 H24 D128 F181 N920)."""
    w = gen.WORKLOADS["sana_wm_720p_60s"]
    x = gen.workload_call_inputs(w, 0, device=DEV)
    bt = gen.token_gates(w.B, w.H, w.F, w.N, seed=w.seed, device=DEV)
    o, S = ls.ls_gdn_frame_forward_token_gate(x["q"], x["k"], x["v"], x["alpha"], bt)
    torch.cuda.synchronize()
    hs = [7, 16]
    ro, rS = oracle_mod.gdn_frame_token_gate(*(_heads(t, hs) for t in (x["q"], x["k"], x["v"], x["alpha"], bt)))
    check("wm-60s gdn token-gate o (2 heads, 181 frames)", _heads(o, hs), ro, 2e-2)
    check("wm-60s gdn token-gate S", _heads(S, hs), rS, 1e-2)


def test_sana_wm_720p_60s_reversed(ls, gen, oracle_mod):
    """The 60 s GDN workload through the reversed scan in chunks of 8 frames."""
    w = gen.WORKLOADS["sana_wm_720p_60s"]
    x = gen.workload_call_inputs(w, 0, device=DEV)
    o = ls.ls_gdn_frame_forward_reversed(x["q"], x["k"], x["v"], x["alpha"], x["beta"], 8)
    torch.cuda.synchronize()
    hs = [2, 23]
    ro = oracle_mod.gdn_frame_reversed(*(_heads(x[n], hs) for n in ("q", "k", "v", "alpha", "beta")), 8)
    check("wm-60s gdn reversed c8 o (2 heads, 181 frames)", _heads(o, hs), ro, 2e-2)


def test_sana_wm_720p_60s(ls, gen, oracle_mod):
    w = gen.WORKLOADS["sana_wm_720p_60s"]
    x = gen.workload_call_inputs(w, 0, device=DEV)
    o, S = ls.ls_gdn_frame_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    hs = [3, 20]
    ro, rS = oracle_mod.gdn_frame(*(_heads(x[n], hs) for n in ("q", "k", "v", "alpha", "beta")))
    check("wm-60s gdn o (2 heads, 181 frames)", _heads(o, hs), ro, 2e-2)
    check("wm-60s gdn S", _heads(S, hs), rS, 1e-2)


def test_sana_wm_chunk_steps(ls, gen, oracle_mod):
    """50 single-frame calls re-reading one carried state built by the oracle
    from a 60-frame prefix; the cache itself is never written."""
    w = gen.WORKLOADS["sana_wm_chunk_step"]
    pre = gen.prefix_inputs(w, device="cpu")
    _, S_pre = oracle_mod.gdn_frame(None, pre["k"], pre["v"], pre["alpha"], pre["beta"], with_output=False)
    del pre
    cache = torch.from_numpy(S_pre.astype(np.float32)).to(DEV)
    cache_copy = cache.clone()
    state_out = torch.empty_like(cache)
    sample = [(0, 0), (3, 17)]
    for step in range(w.steps):
        x = gen.workload_call_inputs(w, step, device=DEV)
        o, _ = ls.ls_gdn_frame_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], cache,
                                       state_out=state_out)
        torch.cuda.synchronize()
        for b, h in sample:
            sl = lambda t: t[b:b + 1, h:h + 1].float().cpu()
            ro, rS = oracle_mod.gdn_frame(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["alpha"]),
                                          sl(x["beta"]), sl(cache))
            err_o = max_rel_err(sl(o), ro)
            err_s = max_rel_err(sl(state_out), rS)
            assert err_o <= 2e-2 and err_s <= 1e-2, (step, b, h, err_o, err_s)
        if step == w.steps - 1:
            # every head of the last step
            ro, rS = oracle_mod.gdn_frame(x["q"].float().cpu(), x["k"].float().cpu(),
                                          x["v"].float().cpu(), x["alpha"].cpu(), x["beta"].cpu(),
                                          cache.cpu())
            check("chunk-step gdn o (all 96 heads)", o, ro, 2e-2)
            check("chunk-step gdn S (all 96 heads)", state_out, rS, 1e-2)
    assert torch.equal(cache, cache_copy)
