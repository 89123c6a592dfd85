"""GPU parity of liblinscan against the fp64 oracle (needs an MI355X).

Bar (written here, applied per tensor with the floor-relative measure of
tests/metrics.py):
  bf16 tokens: outputs <= 2e-2, final state <= 1e-2 (floor 1e-3 * max|y|)
  fp32 tokens: outputs and state <= 1e-5 (normwise: floor max|y|)
Inputs come from block_causal_linear_attn_amd.inputs on the CPU (small cases)
or on the GPU (full-size workloads); the oracle sees exactly the values the
GPU library sees.
"""
import math

import numpy as np
import pytest
import torch

from metrics import FLOOR, max_rel_err

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-5, 1e-5)}
DEV = "cuda"


@pytest.fixture(scope="module")
def ls():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from block_causal_linear_attn_amd import binding
    return binding


@pytest.fixture(scope="module")
def gen():
    from block_causal_linear_attn_amd import inputs
    return inputs


def _dev(x):
    return {k: t.to(DEV) for k, t in x.items()}


def _rand_state(B, H, D, seed, scale=1.0, norm=False):
    g = torch.Generator().manual_seed(seed)
    S = scale * torch.randn((B, H, D, D), generator=g)
    if norm:
        z = torch.rand((B, H, D), generator=g) * scale * D
        return S, z
    return S


def check(name, got, want, tol, dt="bf16"):
    err = max_rel_err(got, want, FLOOR[dt])
    print("%-40s max rel err %.3e (tol %.0e, floor %g)" % (name, err, tol, FLOOR[dt]), flush=True)
    assert err <= tol, (name, err)


# --------------------------------------------------------------------------- ReLU
RELU_CASES = [
    # (B, H, F, N, D, dtype, block_frames, with_state)
    (1, 2, 4, 16, 16, "fp32", 1, False),        # the tiny workload's shape
    (1, 3, 5, 333, 32, "bf16", 1, True),        # MFMA path, ragged token count
    (2, 2, 3, 700, 32, "bf16", 1, False),       # several token chunks per frame
    (1, 2, 4, 200, 64, "bf16", 1, True),        # MFMA path, D = 64
    (1, 2, 2, 1500, 32, "bf16", 1, True),       # few items: each frame's summary in 2 token chunks
    (1, 2, 3, 2100, 64, "bf16", 2, True),       # D = 64, summaries in 4 token chunks, blocks of 2 frames
    (1, 2, 3, 97, 112, "bf16", 1, True),        # wide MFMA path at the pages' head dim (128 dims, zero-padded)
    (1, 2, 4, 2000, 112, "bf16", 1, False),     # wide path, two output chunks per frame, ragged tail
    (2, 10, 3, 200, 112, "bf16", 2, True),      # wide path, B*H = 20 (padding items, outputs spread over XCDs)
    (2, 8, 3, 300, 112, "bf16", 1, True),       # wide path, B*H = 16: every item on its head's XCD
    (1, 2, 1, 1, 112, "bf16", 1, True),         # wide path, single token, single frame
    (1, 2, 5, 300, 128, "bf16", 3, True),       # wide path at D = 128 (normaliser by MFMA), ragged block
    (1, 3, 3, 1000, 112, "bf16", 2, True),      # wide path, each frame's summary in 2 parts (ragged second)
    (1, 2, 2, 3121, 128, "bf16", 1, True),      # wide path at D = 128, summaries in 8 parts, the last one empty
    (1, 2, 3, 50, 16, "bf16", 1, False),        # generic bf16, D = 16
    (1, 2, 7, 40, 32, "bf16", 3, True),         # blocks of 3 frames (ragged last block)
    (1, 2, 3, 70, 48, "fp32", 2, True),         # generic fp32
    (1, 1, 2, 33, 128, "fp32", 1, True),        # generic fp32, D = 128
    (1, 2, 1, 1, 32, "bf16", 1, True),          # single token
]


@pytest.mark.parametrize("B,H,F,N,D,dt,bf,with_state", RELU_CASES)
def test_relu_parity(ls, gen, oracle_mod, B, H, F, N, D, dt, bf, with_state):
    x = gen.relu_inputs(B, H, F, N, D, dt, seed=11, part=N)
    S0 = z0 = None
    if with_state:
        S0, z0 = _rand_state(B, H, D, 5, scale=4.0, norm=True)
    xd = _dev(x)
    o, S, z = ls.ls_relu_block_forward(xd["q"], xd["k"], xd["v"],
                                       None if S0 is None else S0.to(DEV),
                                       None if z0 is None else z0.to(DEV), block_frames=bf)
    torch.cuda.synchronize()
    ro, rS, rz = oracle_mod.relu_block(x["q"], x["k"], x["v"], S0, z0, block_frames=bf)
    to, ts = TOL[dt]
    tag = "relu B%d H%d F%d N%d D%d %s bf%d" % (B, H, F, N, D, dt, bf)
    check(tag + " o", o, ro, to, dt)
    check(tag + " S", S, rS, ts, dt)
    check(tag + " z", z, rz, ts, dt)


# --------------------------------------------------------------------------- GDN
GDN_CASES = [
    # (B, H, F, N, D, dtype, l2_keys, with_state)
    (1, 2, 4, 16, 16, "fp32", False, False),    # the tiny workload's shape
    (1, 2, 6, 300, 128, "bf16", True, True),    # MFMA path, ragged token count
    (2, 1, 3, 920, 128, "bf16", True, False),   # the 720p token count
    (1, 2, 3, 97, 112, "bf16", True, True),     # the pages' head dim (MFMA path, 128 dims zero-padded)
    (2, 3, 5, 920, 112, "bf16", True, True),    # head dim 112, frame-interleaved launch
    (1, 2, 1, 300, 112, "bf16", True, True),    # head dim 112, phased launch, one frame
    (1, 40, 3, 130, 112, "bf16", True, True),   # head dim 112, phased launch, 40 heads
    (1, 2, 3, 80, 96, "bf16", True, True),      # generic bf16 kernels at a head dim without MFMA path
    (1, 2, 4, 64, 64, "bf16", True, False),     # generic bf16, D = 64
    (1, 2, 3, 40, 32, "fp32", False, True),     # generic fp32, raw keys
    (1, 1, 2, 45, 128, "fp32", True, True),     # generic fp32, D = 128
    (1, 2, 2, 1, 128, "bf16", True, True),      # single token per frame
    # single-launch phased path (gram, scan, output phases): one frame, or more heads than
    # the frame-interleaved launch takes
    (3, 24, 1, 920, 128, "bf16", True, True),   # the chunk-step shape at B = 3: chunked frames
    (1, 2, 1, 300, 128, "bf16", True, True),    # one frame, two token chunks
    (1, 70, 3, 130, 128, "bf16", True, True),   # 70 heads, a three-frame chain
    (1, 1, 1, 1, 128, "bf16", True, True),      # one token, one frame
    # single-frame step launch: four items per head swap their rows of beta*G and of the state
    (1, 37, 1, 257, 128, "bf16", True, True),   # odd head count (padded slots), ragged quarters
    (1, 5, 1, 3, 128, "bf16", True, True),      # fewer tokens than items: empty output quarters
    (2, 3, 1, 920, 112, "bf16", True, True),    # head dim 112
    (1, 9, 1, 130, 128, "bf16", False, True),   # raw keys (beta*G not small beside the identity)
]


@pytest.mark.parametrize("B,H,F,N,D,dt,l2,with_state", GDN_CASES)
def test_gdn_parity(ls, gen, oracle_mod, B, H, F, N, D, dt, l2, with_state):
    x = gen.gdn_inputs(B, H, F, N, D, dt, seed=13, part=N, alpha_mu=3.0 if l2 else 2.0, l2_keys=l2)
    S0 = _rand_state(B, H, D, 6, scale=0.5) if with_state else None
    xd = _dev(x)
    o, S = ls.ls_gdn_frame_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                   None if S0 is None else S0.to(DEV))
    torch.cuda.synchronize()
    ro, rS = oracle_mod.gdn_frame(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0)
    to, ts = TOL[dt]
    tag = "gdn B%d H%d F%d N%d D%d %s" % (B, H, F, N, D, dt)
    check(tag + " o", o, ro, to, dt)
    check(tag + " S", S, rS, ts, dt)


@pytest.mark.parametrize("H,F,N,D,dt", [(3, 4, 150, 128, "bf16"), (2, 3, 97, 112, "bf16"), (2, 3, 60, 64, "bf16")])
def test_gdn_camera_branch_shares_the_gates(ls, gen, oracle_mod, H, F, N, D, dt):
    """The coarse camera branch (SANA-WM summary, section 3, Dual-Branch Camera
    Control) has its own q, k, v and shares the frame-wise GDN gates with the
    main branch: the same scan with other token tensors.  Both branches stacked
    on the batch axis with the gates repeated equal the two calls bit for bit,
    and the camera branch driven by the main branch's alpha and beta matches
    the oracle."""
    main = gen.gdn_inputs(1, H, F, N, D, dt, seed=61, part=N, l2_keys=True)
    cam = gen.gdn_inputs(1, H, F, N, D, dt, seed=62, part=N, l2_keys=True)
    m, c = _dev(main), _dev(cam)
    o_m, S_m = ls.ls_gdn_frame_forward(m["q"], m["k"], m["v"], m["alpha"], m["beta"])
    o_c, S_c = ls.ls_gdn_frame_forward(c["q"], c["k"], c["v"], m["alpha"], m["beta"])
    st = {n: torch.cat([m[n], c[n]], dim=0) for n in ("q", "k", "v")}
    ga, gb = torch.cat([m["alpha"], m["alpha"]], dim=0), torch.cat([m["beta"], m["beta"]], dim=0)
    o_s, S_s = ls.ls_gdn_frame_forward(st["q"], st["k"], st["v"], ga, gb)
    torch.cuda.synchronize()
    assert torch.equal(o_s[:1], o_m) and torch.equal(o_s[1:], o_c)
    assert torch.equal(S_s[:1], S_m) and torch.equal(S_s[1:], S_c)
    ro, rS = oracle_mod.gdn_frame(cam["q"], cam["k"], cam["v"], main["alpha"], main["beta"])
    tag = "camera branch H%d F%d N%d D%d" % (H, F, N, D)
    check(tag + " o", o_c, ro, TOL[dt][0], dt)
    check(tag + " S", S_c, rS, TOL[dt][1], dt)


TG_CASES = [
    # (B, H, F, N, D, dtype, with_state): per-token update gates
    (1, 2, 4, 300, 128, "bf16", True),      # frame-interleaved launch, ragged token count
    (2, 3, 5, 920, 112, "bf16", True),      # head dim 112, frame-interleaved launch
    (1, 40, 3, 130, 128, "bf16", True),     # phased launch (40 heads)
    (1, 2, 1, 200, 112, "bf16", True),      # phased launch, one frame
    (3, 24, 1, 920, 128, "bf16", True),     # the chunk-step shape at B = 3
    (1, 2, 3, 80, 64, "bf16", True),        # generic bf16 kernels
    (1, 2, 3, 40, 32, "fp32", True),        # generic fp32 kernels
    (1, 1, 2, 1, 128, "bf16", False),       # one token per frame
    (1, 11, 1, 333, 128, "bf16", True),     # single-frame step launch, odd head count
]


@pytest.mark.parametrize("B,H,F,N,D,dt,with_state", TG_CASES)
def test_gdn_token_gate_parity(ls, gen, oracle_mod, B, H, F, N, D, dt, with_state):
    x = gen.gdn_inputs(B, H, F, N, D, dt, seed=15, part=N, l2_keys=True)
    bt = gen.token_gates(B, H, F, N, seed=15, part=N)
    S0 = _rand_state(B, H, D, 7, scale=0.5) if with_state else None
    xd = _dev(x)
    o, S = ls.ls_gdn_frame_forward_token_gate(xd["q"], xd["k"], xd["v"], xd["alpha"], bt.to(DEV),
                                              None if S0 is None else S0.to(DEV))
    torch.cuda.synchronize()
    ro, rS = oracle_mod.gdn_frame_token_gate(x["q"], x["k"], x["v"], x["alpha"], bt, S0)
    to, ts = TOL[dt]
    tag = "gdn token-gate B%d H%d F%d N%d D%d %s" % (B, H, F, N, D, dt)
    check(tag + " o", o, ro, to, dt)
    check(tag + " S", S, rS, ts, dt)


def test_gdn_token_gate_zero_gates_skip_tokens(ls, gen, oracle_mod):
    """Zero gates on half of each frame's tokens: matches the oracle, and the
    state equals the frame-gate path's over the other half (same key scale)."""
    B, H, F, N, D = 1, 4, 3, 256, 128
    x = gen.gdn_inputs(B, H, F, N, D, "bf16", seed=16, l2_keys=True)
    bt = torch.zeros((B, H, F, N))
    bt[..., 1::2] = x["beta"][..., None]
    xd = _dev(x)
    c = 1.0 / np.sqrt(D * N)
    o, S = ls.ls_gdn_frame_forward_token_gate(xd["q"], xd["k"], xd["v"], xd["alpha"], bt.to(DEV), key_scale=c)
    half = {n: xd[n][..., 1::2, :].contiguous() for n in ("q", "k", "v")}
    o2, S2 = ls.ls_gdn_frame_forward(half["q"], half["k"], half["v"], xd["alpha"], xd["beta"], key_scale=c)
    torch.cuda.synchronize()
    ro, rS = oracle_mod.gdn_frame_token_gate(x["q"], x["k"], x["v"], x["alpha"], bt, key_scale=np.float32(c))
    check("gdn token-gate zero-half o", o, ro, 2e-2)
    check("gdn token-gate zero-half S", S, rS, 1e-2)
    check("gdn token-gate zero-half S vs frame-gate half", S, S2.double().cpu().numpy(), 1e-2)


RV_CASES = [
    # (B, H, F, N, D, dtype, chunk_frames): reversed scan, reset at chunk boundaries
    (1, 2, 7, 300, 128, "bf16", 3),     # frame-interleaved launch, ragged last chunk
    (2, 3, 6, 920, 112, "bf16", 6),     # head dim 112, one chunk of all frames
    (1, 8, 20, 256, 128, "bf16", 16),   # chunks longer than the launch's default lag
    (1, 40, 5, 130, 128, "bf16", 2),    # phased launch (40 heads)
    (1, 2, 9, 200, 128, "bf16", 1),     # one-frame chunks: no history
    (1, 2, 5, 64, 64, "bf16", 2),       # generic bf16 kernels
    (1, 2, 5, 40, 32, "fp32", 4),       # generic fp32 kernels
    (1, 13, 1, 150, 128, "bf16", 1),    # a single frame: the step launch, S = beta U
    (2, 2, 1, 50, 112, "bf16", 4),      # a single frame shorter than its chunk, head dim 112
]


@pytest.mark.parametrize("B,H,F,N,D,dt,C", RV_CASES)
def test_gdn_reversed_parity(ls, gen, oracle_mod, B, H, F, N, D, dt, C):
    x = gen.gdn_inputs(B, H, F, N, D, dt, seed=17, part=N, l2_keys=True)
    xd = _dev(x)
    o = ls.ls_gdn_frame_forward_reversed(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], C)
    torch.cuda.synchronize()
    ro = oracle_mod.gdn_frame_reversed(x["q"], x["k"], x["v"], x["alpha"], x["beta"], C)
    check("gdn reversed B%d H%d F%d N%d D%d %s C%d o" % (B, H, F, N, D, dt, C), o, ro, TOL[dt][0], dt)


def test_gdn_explicit_key_scale(ls, gen, oracle_mod):
    x = gen.gdn_inputs(1, 2, 3, 64, 128, "bf16", seed=14, l2_keys=True)
    xd = _dev(x)
    o, S = ls.ls_gdn_frame_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], key_scale=0.01)
    torch.cuda.synchronize()
    ro, rS = oracle_mod.gdn_frame(x["q"], x["k"], x["v"], x["alpha"], x["beta"], key_scale=np.float32(0.01))
    check("gdn key_scale=0.01 o", o, ro, 2e-2)
    check("gdn key_scale=0.01 S", S, rS, 1e-2)


# --------------------------------------------------------------------------- edge cases
def test_zero_frames_copies_state(ls):
    S0 = torch.randn(1, 2, 32, 32, device=DEV)
    z0 = torch.rand(1, 2, 32, device=DEV)
    q = torch.empty((1, 2, 0, 16, 32), dtype=torch.bfloat16, device=DEV)
    o, S, z = ls.ls_relu_block_forward(q, q.clone(), q.clone(), S0, z0)
    o2, S2 = ls.ls_gdn_frame_forward(q, q.clone(), q.clone(), torch.empty(1, 2, 0, device=DEV),
                                     torch.empty(1, 2, 0, device=DEV), S0)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(z, z0) and torch.equal(S2, S0)
    _, S3, z3 = ls.ls_relu_block_forward(q, q.clone(), q.clone())
    torch.cuda.synchronize()
    assert torch.count_nonzero(S3) == 0 and torch.count_nonzero(z3) == 0


def test_zero_tokens(ls, oracle_mod):
    """N = 0: the ReLU state is unchanged, the GDN state only decays."""
    S0 = torch.randn(1, 2, 128, 128)
    a = torch.rand(1, 2, 3) * 0.5 + 0.5
    b = torch.rand(1, 2, 3)
    q = torch.empty((1, 2, 3, 0, 128), dtype=torch.bfloat16, device=DEV)
    _, S = ls.ls_gdn_frame_forward(q, q.clone(), q.clone(), a.to(DEV), b.to(DEV), S0.to(DEV))
    torch.cuda.synchronize()
    want = S0.double() * torch.prod(a.double(), dim=2)[:, :, None, None]
    check("gdn N=0 decay", S, want, 1e-5, "fp32")
    q32 = torch.empty((1, 2, 3, 0, 32), dtype=torch.bfloat16, device=DEV)
    S1 = torch.randn(1, 2, 32, 32, device=DEV)
    _, S2, _ = ls.ls_relu_block_forward(q32, q32.clone(), q32.clone(), S1, None)
    torch.cuda.synchronize()
    assert torch.equal(S2, S1)


def test_empty_batch_is_a_no_op(ls):
    q = torch.empty((0, 2, 3, 16, 32), dtype=torch.bfloat16, device=DEV)
    o, S, z = ls.ls_relu_block_forward(q, q.clone(), q.clone())
    torch.cuda.synchronize()
    assert o.numel() == 0 and S.numel() == 0


def test_in_place_state_and_poisoned_outputs(ls, gen, oracle_mod):
    """state_out == state_in works, and outputs prefilled with NaN are fully overwritten."""
    x = gen.relu_inputs(1, 2, 3, 130, 32, "bf16", seed=21)
    S0, z0 = _rand_state(1, 2, 32, 7, norm=True)
    xd = _dev(x)
    S = S0.to(DEV).clone()
    z = z0.to(DEV).clone()
    o = torch.full_like(xd["q"], float("nan"))
    ls.ls_relu_block_forward(xd["q"], xd["k"], xd["v"], S, z, out=o, state_out=S, norm_out=z)
    torch.cuda.synchronize()
    ro, rS, rz = oracle_mod.relu_block(x["q"], x["k"], x["v"], S0, z0)
    assert torch.isfinite(o).all()
    check("relu in-place o", o, ro, 2e-2)
    check("relu in-place S", S, rS, 1e-2)
    check("relu in-place z", z, rz, 1e-2)

    y = gen.gdn_inputs(1, 2, 3, 130, 128, "bf16", seed=22)
    G0 = _rand_state(1, 2, 128, 8, scale=0.3)
    yd = _dev(y)
    G = G0.to(DEV).clone()
    o = torch.full_like(yd["q"], float("nan"))
    ls.ls_gdn_frame_forward(yd["q"], yd["k"], yd["v"], yd["alpha"], yd["beta"], G, out=o, state_out=G)
    torch.cuda.synchronize()
    ro, rS = oracle_mod.gdn_frame(y["q"], y["k"], y["v"], y["alpha"], y["beta"], G0)
    assert torch.isfinite(o).all()
    check("gdn in-place o", o, ro, 2e-2)
    check("gdn in-place S", G, rS, 1e-2)


@pytest.mark.parametrize("F,D,N", [(1, 112, 150), (3, 112, 150), (1, 128, 150),
                                   (1, 112, 1000), (3, 128, 1000)])  # N = 1000: summaries in 2 parts
def test_relu_wide_in_place_state(ls, gen, oracle_mod, F, D, N):
    """Wide heads: state_out == state_in, also when one work item reads and writes it (F = 1)."""
    x = gen.relu_inputs(1, 2, F, N, D, "bf16", seed=28)
    S0, z0 = _rand_state(1, 2, D, 9, norm=True)
    xd = _dev(x)
    S = S0.to(DEV).clone()
    z = z0.to(DEV).clone()
    o = torch.full_like(xd["q"], float("nan"))
    ls.ls_relu_block_forward(xd["q"], xd["k"], xd["v"], S, z, out=o, state_out=S, norm_out=z)
    torch.cuda.synchronize()
    ro, rS, rz = oracle_mod.relu_block(x["q"], x["k"], x["v"], S0, z0)
    assert torch.isfinite(o).all()
    check("relu wide in-place o", o, ro, 2e-2)
    check("relu wide in-place S", S, rS, 1e-2)
    check("relu wide in-place z", z, rz, 1e-2)


def test_deterministic(ls, gen):
    x = _dev(gen.relu_inputs(1, 4, 4, 1000, 32, "bf16", seed=23))
    a = ls.ls_relu_block_forward(x["q"], x["k"], x["v"])
    b = ls.ls_relu_block_forward(x["q"], x["k"], x["v"])
    y = _dev(gen.gdn_inputs(1, 2, 5, 500, 128, "bf16", seed=24))
    c = ls.ls_gdn_frame_forward(y["q"], y["k"], y["v"], y["alpha"], y["beta"])
    d = ls.ls_gdn_frame_forward(y["q"], y["k"], y["v"], y["alpha"], y["beta"])
    # wide heads, each frame's summary in 2 parts (a fixed order of addition)
    w = _dev(gen.relu_inputs(1, 4, 3, 1000, 112, "bf16", seed=27))
    e = ls.ls_relu_block_forward(w["q"], w["k"], w["v"])
    f = ls.ls_relu_block_forward(w["q"], w["k"], w["v"])
    torch.cuda.synchronize()
    for s, t in zip(a + c + e, b + d + f):
        assert torch.equal(s, t)


def test_head_isolation(ls, gen):
    """A NaN in one head's values stays in that head."""
    x = _dev(gen.relu_inputs(1, 3, 2, 100, 32, "bf16", seed=25))
    x["v"][0, 1, 0, 5, 3] = float("nan")
    o, S, z = ls.ls_relu_block_forward(x["q"], x["k"], x["v"])
    y = _dev(gen.gdn_inputs(1, 3, 2, 100, 128, "bf16", seed=26))
    y["v"][0, 1, 1, 7, 0] = float("nan")
    o2, S2 = ls.ls_gdn_frame_forward(y["q"], y["k"], y["v"], y["alpha"], y["beta"])
    # wide heads with 2 summary parts per frame: the NaN sits in the second part's tokens
    w = _dev(gen.relu_inputs(1, 3, 2, 800, 128, "bf16", seed=28))
    w["v"][0, 1, 0, 600, 9] = float("nan")
    o3, S3, z3 = ls.ls_relu_block_forward(w["q"], w["k"], w["v"])
    torch.cuda.synchronize()
    for t in (o, S, o2, S2, o3, S3):
        assert torch.isfinite(t[:, 0]).all() and torch.isfinite(t[:, 2]).all()
        assert not torch.isfinite(t[:, 1]).all()
    assert torch.isfinite(z3).all()  # z takes no values


# --------------------------------------------------------------------------- carry
def test_state_carry_copy_and_reset(ls):
    S = torch.randn(2, 3, 32, 32, device=DEV)
    z = torch.randn(2, 3, 32, device=DEV)
    S2 = torch.empty_like(S)
    z2 = torch.empty_like(z)
    ls.ls_state_carry(S, S2, z, z2)
    torch.cuda.synchronize()
    assert torch.equal(S, S2) and torch.equal(z, z2)
    ls.ls_state_carry(None, S2, None, z2, reset=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S2) == 0 and torch.count_nonzero(z2) == 0


def test_chunked_rollout_through_carry_equals_one_call(ls, gen, oracle_mod):
    """Block-autoregressive rollout (calls of 3 frames chained by ls_state_carry)."""
    B, H, F, N, D = 1, 2, 8, 200, 32
    x = gen.relu_inputs(B, H, F, N, D, "bf16", seed=27)
    xd = _dev(x)
    o1, S1, z1 = ls.ls_relu_block_forward(xd["q"], xd["k"], xd["v"])
    cache = torch.zeros((B, H, D, D), device=DEV)
    ncache = torch.zeros((B, H, D), device=DEV)
    outs = []
    for f0 in range(0, F, 3):
        sl = slice(f0, min(F, f0 + 3))
        q, k, v = (xd[n][:, :, sl].contiguous() for n in "qkv")
        o, S, z = ls.ls_relu_block_forward(q, k, v, cache, ncache)
        ls.ls_state_carry(S, cache, z, ncache)
        outs.append(o)
    torch.cuda.synchronize()
    ro, rS, rz = oracle_mod.relu_block(x["q"], x["k"], x["v"])
    check("rollout o", torch.cat(outs, dim=2), ro, 2e-2)
    check("rollout S", cache, rS, 1e-2)
    check("rollout z", ncache, rz, 1e-2)
    check("rollout vs one call o", torch.cat(outs, dim=2).float(), o1.float().double().cpu().numpy(), 1e-2)
    assert torch.allclose(cache, S1, rtol=1e-5, atol=1e-5 * S1.abs().max().item())


# --------------------------------------------------------------------------- single-launch paths
@pytest.mark.parametrize("op", ["relu", "relu_wide", "gdn", "gdn_phased", "gdn_step", "gdn_token_gate",
                                "gdn_reversed"])
def test_single_launch_fault_word_stays_clear(ls, gen, oracle_mod, op):
    """The one-launch paths hand data between work items through flags with
    bounded waits; the workspace's fault word must stay zero and results match."""
    if op == "relu":
        x = gen.relu_inputs(1, 11, 9, 777, 32, "bf16", seed=31)   # B*H not a multiple of 8
        shp = ls.ls_shape(1, 11, 9, 777, 32, 1)
        need = ls.lib.ls_relu_block_workspace_size(ls.ctypes.byref(shp))
    elif op == "relu_wide":  # head dim 112: chained cumulative states
        x = gen.relu_inputs(1, 11, 9, 777, 112, "bf16", seed=34)
        shp = ls.ls_shape(1, 11, 9, 777, 112, 1)
        need = ls.lib.ls_relu_block_workspace_size(ls.ctypes.byref(shp))
    elif op == "gdn":
        x = gen.gdn_inputs(1, 5, 9, 333, 128, "bf16", seed=32)
        shp = ls.ls_shape(1, 5, 9, 333, 128, 1)
        need = ls.lib.ls_gdn_frame_workspace_size(ls.ctypes.byref(shp))
    elif op == "gdn_phased":  # 80 heads: the phased launch
        x = gen.gdn_inputs(2, 40, 2, 200, 128, "bf16", seed=33)
        shp = ls.ls_shape(2, 40, 2, 200, 128, 1)
        need = ls.lib.ls_gdn_frame_workspace_size(ls.ctypes.byref(shp))
    elif op == "gdn_step":  # one frame of 74 heads: the step launch, items waiting for their partners
        x = gen.gdn_inputs(2, 37, 1, 333, 128, "bf16", seed=37)
        shp = ls.ls_shape(2, 37, 1, 333, 128, 1)
        need = ls.lib.ls_gdn_frame_workspace_size(ls.ctypes.byref(shp))
    elif op == "gdn_reversed":  # reversed scan in chunks of 4, frame-interleaved launch
        x = gen.gdn_inputs(1, 5, 9, 333, 128, "bf16", seed=36)
        shp = ls.ls_shape(1, 5, 9, 333, 128, 1)
        need = ls.lib.ls_gdn_frame_workspace_size(ls.ctypes.byref(shp))
    else:  # per-token gates, frame-interleaved launch
        x = gen.gdn_inputs(1, 5, 9, 333, 112, "bf16", seed=35)
        x["beta_tok"] = gen.token_gates(1, 5, 9, 333, seed=35)
        shp = ls.ls_shape(1, 5, 9, 333, 112, 1)
        need = ls.lib.ls_gdn_frame_workspace_size(ls.ctypes.byref(shp))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    xd = _dev(x)
    for rep in range(3):  # reuse of a workspace across calls (fresh epochs)
        if op.startswith("relu"):
            o, S, z = ls.ls_relu_block_forward(xd["q"], xd["k"], xd["v"], block_frames=2, ws=ws)
        elif op == "gdn_token_gate":
            o, S = ls.ls_gdn_frame_forward_token_gate(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta_tok"], ws=ws)
        elif op == "gdn_reversed":
            o = ls.ls_gdn_frame_forward_reversed(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], 4, ws=ws)
        else:
            o, S = ls.ls_gdn_frame_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], ws=ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0
    if op.startswith("relu"):
        ro, rS, rz = oracle_mod.relu_block(x["q"], x["k"], x["v"], block_frames=2)
        check("single-launch relu o", o, ro, 2e-2)
        check("single-launch relu S", S, rS, 1e-2)
    elif op == "gdn_reversed":
        ro = oracle_mod.gdn_frame_reversed(x["q"], x["k"], x["v"], x["alpha"], x["beta"], 4)
        check("single-launch gdn reversed o", o, ro, 2e-2)
    elif op == "gdn_token_gate":
        ro, rS = oracle_mod.gdn_frame_token_gate(x["q"], x["k"], x["v"], x["alpha"], x["beta_tok"])
        check("single-launch gdn token-gate o", o, ro, 2e-2)
        check("single-launch gdn token-gate S", S, rS, 1e-2)
    else:
        ro, rS = oracle_mod.gdn_frame(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
        check("single-launch gdn o", o, ro, 2e-2)
        check("single-launch gdn S", S, rS, 1e-2)


def test_concurrent_streams_match_sequential(ls, gen):
    """Single-launch calls running at the same time on separate streams (three
    frame-interleaved GDN calls, one phased GDN call, two ReLU calls) give the
    same bits as when run one after another, and no wait times out."""
    jobs = []
    for i in range(3):  # frame-interleaved GDN launches (B*H <= 32)
        jobs.append(("gdn", _dev(gen.gdn_inputs(1, 8, 6, 300, 128, "bf16", seed=40 + i))))
    jobs.append(("gdn", _dev(gen.gdn_inputs(1, 40, 3, 200, 128, "bf16", seed=44))))  # phased launch
    for i in range(2):
        jobs.append(("relu", _dev(gen.relu_inputs(1, 12, 5, 700, 32, "bf16", seed=45 + i))))

    def run(kind, x, ws):
        if kind == "gdn":
            return ls.ls_gdn_frame_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], ws=ws)
        return ls.ls_relu_block_forward(x["q"], x["k"], x["v"], ws=ws)

    def workspace(kind, x):
        B, H, F, N, D = x["q"].shape
        shp = ls.ls_shape(B, H, F, N, D, 1)
        if kind == "gdn":
            need = ls.lib.ls_gdn_frame_workspace_size(ls.ctypes.byref(shp))
        else:
            need = ls.lib.ls_relu_block_workspace_size(ls.ctypes.byref(shp))
        return torch.zeros(need, dtype=torch.uint8, device=DEV)

    ref = [run(kind, x, workspace(kind, x)) for kind, x in jobs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in jobs]
    wss = [workspace(kind, x) for kind, x in jobs]
    torch.cuda.synchronize()
    out = []
    for (kind, x), st, ws in zip(jobs, streams, wss):
        with torch.cuda.stream(st):
            out.append(run(kind, x, ws))
    torch.cuda.synchronize()
    for i, (r, o, ws) in enumerate(zip(ref, out, wss)):
        assert int(ws[:4].view(torch.int32).item()) == 0, i
        for a, b in zip(r, o):
            assert torch.equal(a, b), i


# --------------------------------------------------------------------------- temporal conv
CONV_CASES = [
    # (B, H, F, N, D, dtype, block_frames, bias, carry)
    (1, 1, 10, 500, 2240, "bf16", 10, True, True),    # FFN-width channels, one 10-frame block
    (2, 3, 7, 33, 64, "bf16", 3, True, True),         # several blocks, ragged last block
    (1, 2, 5, 17, 40, "fp32", 1, False, True),        # fp32, one-frame blocks
    (1, 1, 1, 100, 128, "bf16", 1, True, False),      # a single frame, no carry
    (1, 70, 9, 50, 32, "bf16", 4, True, True),        # per-head channels of the attention layout
    (1, 1, 20, 64, 8, "bf16", 20, True, True),        # more frames than one register group, D = 8
    (1, 1, 17, 40, 16, "fp32", 5, True, True),
]


def _conv_params(H, D, seed):
    g = torch.Generator().manual_seed(seed)
    return 0.5 * torch.randn((H, D, 3), generator=g), 0.1 * torch.randn((H, D), generator=g)


@pytest.mark.parametrize("B,H,F,N,D,dt,bf,with_bias,with_carry", CONV_CASES)
def test_temporal_conv_parity(ls, gen, oracle_mod, B, H, F, N, D, dt, bf, with_bias, with_carry):
    x = gen.token_tensor(B, H, F, N, D, dt, seed=18, stream=0, part=N)
    carry = gen.token_tensor(B, H, 1, N, D, dt, seed=18, stream=1, part=N)[:, :, 0].contiguous() if with_carry else None
    w, b = _conv_params(H, D, 19)
    b = b if with_bias else None
    y, co = ls.ls_temporal_conv3(x.to(DEV), w.to(DEV), None if b is None else b.to(DEV),
                                 None if carry is None else carry.to(DEV), block_frames=bf)
    torch.cuda.synchronize()
    ry, rco = oracle_mod.temporal_conv3(x, w, b, carry, block_frames=bf)
    tag = "conv B%d H%d F%d N%d D%d %s bf%d" % (B, H, F, N, D, dt, bf)
    check(tag + " y", y, ry, 1e-2 if dt == "bf16" else 1e-5, dt)
    assert torch.equal(co.cpu().float(), torch.from_numpy(rco).float())


def test_temporal_conv_blocks_chain_through_the_carry(ls, gen):
    """Calls of one block each, carrying in place, equal one call over all blocks (bitwise)."""
    B, H, F, N, D, bf = 1, 4, 12, 300, 96, 3
    x = gen.token_tensor(B, H, F, N, D, "bf16", seed=20, stream=0).to(DEV)
    w, b = (t.to(DEV) for t in _conv_params(H, D, 21))
    carry0 = gen.token_tensor(B, H, 1, N, D, "bf16", seed=20, stream=1)[:, :, 0].contiguous().to(DEV)
    y1, co1 = ls.ls_temporal_conv3(x, w, b, carry0, block_frames=bf)
    carry = carry0.clone()
    parts = []
    for f0 in range(0, F, bf):
        yp, _ = ls.ls_temporal_conv3(x[:, :, f0:f0 + bf].contiguous(), w, b, carry, block_frames=bf,
                                     carry_out=carry)
        parts.append(yp)
    empty = torch.empty((B, H, 0, N, D), dtype=x.dtype, device=DEV)
    _, passed = ls.ls_temporal_conv3(empty, w, b, carry, block_frames=bf)  # F = 0: the carry passes through
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=2), y1)
    assert torch.equal(carry, co1) and torch.equal(passed, carry)


# --------------------------------------------------------------------------- strided token layouts
def _bshd(x):
    """A [B, H, F, N, D] view of a copy of x stored [B, F, N, H, D] (heads interleaved in each token)."""
    return x.permute(0, 2, 3, 1, 4).contiguous().permute(0, 3, 1, 2, 4)


@pytest.mark.parametrize("H,F,N,D,dt", [(5, 4, 333, 32, "bf16"), (3, 3, 200, 112, "bf16"), (2, 3, 300, 128, "bf16"),
                                        (4, 4, 333, 32, "bf16"),  # head dim 32 in pairs (even head count)
                                        (2, 3, 50, 16, "bf16"), (2, 3, 40, 48, "fp32")])
def test_relu_strided_layout(ls, gen, oracle_mod, H, F, N, D, dt):
    """[B, F, N, H, D] storage matches the oracle and, bit for bit, the packed call."""
    x = gen.relu_inputs(1, H, F, N, D, dt, seed=41, part=N)
    xd = _dev(x)
    o1, S1, z1 = ls.ls_relu_block_forward(xd["q"], xd["k"], xd["v"], block_frames=2)
    q, k, v = (_bshd(xd[n]) for n in ("q", "k", "v"))
    o2, S2, z2 = ls.ls_relu_block_forward_strided(q, k, v, block_frames=2)
    torch.cuda.synchronize()
    assert o2.stride() == q.stride()
    ro, rS, rz = oracle_mod.relu_block(x["q"], x["k"], x["v"], block_frames=2)
    tag = "relu strided H%d F%d N%d D%d %s" % (H, F, N, D, dt)
    check(tag + " o", o2, ro, TOL[dt][0], dt)
    check(tag + " S", S2, rS, TOL[dt][1], dt)
    assert torch.equal(o2.contiguous(), o1) and torch.equal(S2, S1) and torch.equal(z2, z1)


@pytest.mark.parametrize("B,H,F,N,D,bf", [(2, 6, 3, 700, 32, 1), (1, 70, 2, 130, 32, 2), (1, 2, 1, 1, 32, 1),
                                          (1, 4, 1, 1100, 32, 1)])  # pairs, summaries in 2 token chunks
def test_relu_head_pairs_with_state(ls, gen, oracle_mod, B, H, F, N, D, bf):
    """Head dim 32 stored [B, F, N, H, D] with an even head count runs heads in pairs: the carried state goes in
    and out per head (in place), and every output equals the packed call's bit for bit."""
    x = gen.relu_inputs(B, H, F, N, D, "bf16", seed=43, part=N)
    S0, z0 = _rand_state(B, H, D, 44, scale=4.0, norm=True)
    xd = _dev(x)
    o1, S1, z1 = ls.ls_relu_block_forward(xd["q"], xd["k"], xd["v"], S0.to(DEV), z0.to(DEV), block_frames=bf)
    q, k, v = (_bshd(xd[n]) for n in ("q", "k", "v"))
    S2, z2 = S0.to(DEV), z0.to(DEV)
    o2, _, _ = ls.ls_relu_block_forward_strided(q, k, v, S2, z2, block_frames=bf, state_out=S2, norm_out=z2)
    torch.cuda.synchronize()
    ro, rS, rz = oracle_mod.relu_block(x["q"], x["k"], x["v"], S0, z0, block_frames=bf)
    tag = "relu pairs B%d H%d F%d N%d" % (B, H, F, N)
    check(tag + " o", o2, ro, TOL["bf16"][0], "bf16")
    check(tag + " S", S2, rS, TOL["bf16"][1], "bf16")
    check(tag + " z", z2, rz, TOL["bf16"][1], "bf16")
    assert torch.equal(o2.contiguous(), o1) and torch.equal(S2, S1) and torch.equal(z2, z1)


@pytest.mark.parametrize("B,H,F,N,D,dt", [(1, 3, 4, 300, 128, "bf16"), (1, 40, 2, 130, 128, "bf16"),
                                          (2, 2, 3, 97, 112, "bf16"), (1, 2, 3, 80, 64, "bf16")])
def test_gdn_strided_layout(ls, gen, oracle_mod, B, H, F, N, D, dt):
    x = gen.gdn_inputs(B, H, F, N, D, dt, seed=42, part=N, l2_keys=True)
    xd = _dev(x)
    o1, S1 = ls.ls_gdn_frame_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"])
    q, k, v = (_bshd(xd[n]) for n in ("q", "k", "v"))
    o2, S2 = ls.ls_gdn_frame_forward_strided(q, k, v, xd["alpha"], xd["beta"])
    torch.cuda.synchronize()
    ro, rS = oracle_mod.gdn_frame(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    tag = "gdn strided B%d H%d F%d N%d D%d %s" % (B, H, F, N, D, dt)
    check(tag + " o", o2, ro, TOL[dt][0], dt)
    check(tag + " S", S2, rS, TOL[dt][1], dt)
    assert torch.equal(o2.contiguous(), o1) and torch.equal(S2, S1)


# --------------------------------------------------------------------------- fused per-token prologue
def _weights(H, D, seed):
    g = torch.Generator().manual_seed(seed)
    return 1.0 + 0.5 * torch.randn((H, D), generator=g), 1.0 + 0.5 * torch.randn((H, D), generator=g)


@pytest.mark.parametrize("H,F,N,D,dt,qw,kw", [(3, 4, 333, 32, "bf16", True, True), (2, 3, 200, 64, "bf16", True, True),
                                              (3, 3, 200, 112, "bf16", True, False), (2, 3, 150, 128, "bf16", False, True),
                                              (2, 2, 900, 128, "bf16", True, True),  # summaries in 2 parts
                                              (2, 3, 50, 16, "bf16", True, True), (2, 3, 40, 48, "fp32", True, True)])
def test_relu_prologue_parity(ls, gen, oracle_mod, H, F, N, D, dt, qw, kw):
    x = gen.relu_inputs(1, H, F, N, D, dt, seed=51, part=N)
    wq, wk = _weights(H, D, 52)
    wq, wk = (wq if qw else None), (wk if kw else None)
    xd = _dev(x)
    o, S, z = ls.ls_relu_block_forward_prologue(xd["q"], xd["k"], xd["v"], None if wq is None else wq.to(DEV),
                                                None if wk is None else wk.to(DEV), norm_eps=1e-5)
    torch.cuda.synchronize()
    rnd = "bf16" if dt == "bf16" else None
    qp = oracle_mod.prologue(x["q"], wq, eps=1e-5, round_to=rnd) if qw else x["q"]
    kp = oracle_mod.prologue(x["k"], wk, eps=1e-5, round_to=rnd) if kw else x["k"]
    ro, rS, rz = oracle_mod.relu_block(qp, kp, x["v"])
    tag = "relu prologue H%d F%d N%d D%d %s q%d k%d" % (H, F, N, D, dt, qw, kw)
    check(tag + " o", o, ro, TOL[dt][0], dt)
    check(tag + " S", S, rS, TOL[dt][1], dt)
    check(tag + " z", z, rz, TOL[dt][1], dt)


@pytest.mark.parametrize("B,H,F,N,D,dt,qw,kw,relu,l2", [
    (1, 3, 4, 300, 128, "bf16", True, True, True, True),      # frame-interleaved launch, the whole prologue
    (1, 40, 2, 130, 128, "bf16", True, True, True, False),    # phased launch
    (2, 2, 3, 97, 112, "bf16", False, True, False, True),     # head dim 112: RMSNorm + L2 of keys
    (1, 2, 3, 200, 128, "bf16", False, False, True, False),   # ReLU alone
    (1, 6, 1, 300, 128, "bf16", True, True, True, True),      # single-frame step launch, whole prologue
    (1, 2, 3, 80, 64, "bf16", True, True, True, True),        # generic bf16 kernels
    (1, 2, 3, 40, 32, "fp32", True, True, True, True),        # generic fp32 kernels
])
def test_gdn_prologue_parity(ls, gen, oracle_mod, B, H, F, N, D, dt, qw, kw, relu, l2):
    x = gen.gdn_inputs(B, H, F, N, D, dt, seed=53, part=N, l2_keys=False)
    wq, wk = _weights(H, D, 54)
    wq, wk = (wq if qw else None), (wk if kw else None)
    xd = _dev(x)
    o, S = ls.ls_gdn_frame_forward_prologue(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                            None if wq is None else wq.to(DEV), None if wk is None else wk.to(DEV),
                                            norm_eps=1e-5, relu=relu, l2_keys=l2)
    torch.cuda.synchronize()
    rnd = "bf16" if dt == "bf16" else None
    qp = oracle_mod.prologue(x["q"], wq, eps=1e-5, relu=relu, round_to=rnd) if (qw or relu) else x["q"]
    kp = oracle_mod.prologue(x["k"], wk, eps=1e-5, relu=relu, l2=l2, round_to=rnd) if (kw or relu or l2) else x["k"]
    ro, rS = oracle_mod.gdn_frame(qp, kp, x["v"], x["alpha"], x["beta"])
    tag = "gdn prologue B%d H%d F%d N%d D%d %s q%d k%d r%d l%d" % (B, H, F, N, D, dt, qw, kw, relu, l2)
    check(tag + " o", o, ro, TOL[dt][0], dt)
    check(tag + " S", S, rS, TOL[dt][1], dt)


def _as_tokens(a, dt):
    """Oracle values (already exact in the token precision) as a device token tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.float32)
    return (t.to(torch.bfloat16) if dt == "bf16" else t).to(DEV)


@pytest.mark.parametrize("H,F,N,D,dt", [(3, 4, 333, 32, "bf16"), (2, 3, 200, 64, "bf16"), (3, 3, 200, 112, "bf16"),
                                        (2, 3, 150, 128, "bf16"), (2, 3, 50, 16, "bf16"), (2, 3, 40, 48, "fp32")])
def test_relu_prologue_matches_plain_scan_bitwise(ls, gen, oracle_mod, H, F, N, D, dt):
    """The fused prologue rounds its fp64 result once to the token precision,
    as the oracle does: the scan of the fused call is then the plain scan of
    the oracle's prologue output, bit for bit."""
    x = gen.relu_inputs(1, H, F, N, D, dt, seed=55, part=N)
    wq, wk = _weights(H, D, 56)
    xd = _dev(x)
    o, S, z = ls.ls_relu_block_forward_prologue(xd["q"], xd["k"], xd["v"], wq.to(DEV), wk.to(DEV), norm_eps=1e-5)
    rnd = "bf16" if dt == "bf16" else None
    qp = oracle_mod.prologue(x["q"], wq, eps=1e-5, round_to=rnd)
    kp = oracle_mod.prologue(x["k"], wk, eps=1e-5, round_to=rnd)
    o2, S2, z2 = ls.ls_relu_block_forward(_as_tokens(qp, dt), _as_tokens(kp, dt), xd["v"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2) and torch.equal(z, z2)


@pytest.mark.parametrize("B,H,F,N,D,dt,relu,l2", [
    (1, 3, 4, 300, 128, "bf16", True, True), (1, 40, 2, 130, 128, "bf16", False, True),
    (1, 3, 4, 300, 128, "bf16", False, False), (2, 2, 3, 97, 112, "bf16", True, False),
    (1, 2, 3, 80, 64, "bf16", True, True), (1, 2, 3, 40, 32, "fp32", False, True)])
def test_gdn_prologue_matches_plain_scan_bitwise(ls, gen, oracle_mod, B, H, F, N, D, dt, relu, l2):
    x = gen.gdn_inputs(B, H, F, N, D, dt, seed=57, part=N, l2_keys=False)
    wq, wk = _weights(H, D, 58)
    xd = _dev(x)
    o, S = ls.ls_gdn_frame_forward_prologue(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], wq.to(DEV),
                                            wk.to(DEV), norm_eps=1e-5, relu=relu, l2_keys=l2)
    rnd = "bf16" if dt == "bf16" else None
    qp = oracle_mod.prologue(x["q"], wq, eps=1e-5, relu=relu, round_to=rnd)
    kp = oracle_mod.prologue(x["k"], wk, eps=1e-5, relu=relu, l2=l2, round_to=rnd)
    o2, S2 = ls.ls_gdn_frame_forward(_as_tokens(qp, dt), _as_tokens(kp, dt), xd["v"], xd["alpha"], xd["beta"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2)


@pytest.mark.parametrize("B,H,F,N,D,dt,qw,kw,relu,l2,P,off", [
    (1, 3, 4, 300, 128, "bf16", True, True, True, True, 16, 0),      # frame-interleaved launch, whole prologue
    (1, 40, 2, 130, 128, "bf16", False, False, False, False, 0, 0),  # phased launch, token table only
    (1, 2, 3, 200, 128, "bf16", False, True, False, True, 64, 5),    # frame table only, rows from 5
    (1, 5, 1, 230, 112, "bf16", True, True, True, True, 8, 3),       # single-frame step launch
    (2, 2, 3, 97, 112, "bf16", True, True, False, True, 8, 2),       # head dim 112
    (1, 2, 3, 80, 64, "bf16", True, True, True, True, 8, 1),         # generic bf16 kernels
    (1, 2, 3, 40, 32, "fp32", True, True, True, True, 4, 0),         # generic fp32 kernels
])
def test_gdn_rope_parity(ls, gen, oracle_mod, B, H, F, N, D, dt, qw, kw, relu, l2, P, off):
    """The rotary embedding at the end of the prologue: against the oracle, and
    bit for bit against the plain scan of the oracle's prologue output."""
    x = gen.gdn_inputs(B, H, F, N, D, dt, seed=59, part=N, l2_keys=False)
    wq, wk = _weights(H, D, 60)
    wq, wk = (wq if qw else None), (wk if kw else None)
    fcs, tcs = gen.rope_tables(off + F + 1, N, 20, D, P)
    xd = _dev(x)
    dev_rope = (None if fcs is None else fcs.to(DEV), None if tcs is None else tcs.to(DEV), P, off)
    o, S = ls.ls_gdn_frame_forward_prologue(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                            None if wq is None else wq.to(DEV), None if wk is None else wk.to(DEV),
                                            norm_eps=1e-5, relu=relu, l2_keys=l2, rope=dev_rope)
    rnd = "bf16" if dt == "bf16" else None
    rope = (fcs, tcs, P, off)
    qp = oracle_mod.prologue(x["q"], wq, eps=1e-5, relu=relu, round_to=rnd, rope=rope)
    kp = oracle_mod.prologue(x["k"], wk, eps=1e-5, relu=relu, l2=l2, round_to=rnd, rope=rope)
    o2, S2 = ls.ls_gdn_frame_forward(_as_tokens(qp, dt), _as_tokens(kp, dt), xd["v"], xd["alpha"], xd["beta"])
    torch.cuda.synchronize()
    ro, rS = oracle_mod.gdn_frame(qp, kp, x["v"], x["alpha"], x["beta"])
    tag = "gdn rope B%d H%d F%d N%d D%d %s q%d k%d r%d l%d P%d off%d" % (B, H, F, N, D, dt, qw, kw, relu, l2, P, off)
    check(tag + " o", o, ro, TOL[dt][0], dt)
    check(tag + " S", S, rS, TOL[dt][1], dt)
    assert torch.equal(o, o2) and torch.equal(S, S2)


@pytest.mark.parametrize("H,F,N,D,dt,qw,kw,P,off,bf", [
    (3, 4, 333, 32, "bf16", True, True, 4, 0, 1),      # narrow items, RMSNorm and RoPE
    (2, 3, 200, 64, "bf16", False, False, 0, 0, 2),    # narrow items, token table only, 2-frame blocks
    (3, 3, 200, 112, "bf16", True, True, 8, 2, 1),     # wide items, head dim 112
    (2, 3, 150, 128, "bf16", False, True, 64, 1, 1),   # wide items, frame table only
    (2, 2, 900, 112, "bf16", True, True, 8, 1, 1),     # wide items, each frame's summary in 2 parts
    (2, 3, 50, 16, "bf16", True, True, 4, 0, 1),       # generic bf16 kernels
    (2, 3, 40, 48, "fp32", True, True, 8, 0, 2),       # generic fp32 kernels
])
def test_relu_rope_parity(ls, gen, oracle_mod, H, F, N, D, dt, qw, kw, P, off, bf):
    """The ReLU scan with the rotary embedding: rotated features in the
    numerator, unrotated ones in the normaliser, against the oracle."""
    x = gen.relu_inputs(1, H, F, N, D, dt, seed=61, part=N)
    wq, wk = _weights(H, D, 62)
    wq, wk = (wq if qw else None), (wk if kw else None)
    fcs, tcs = gen.rope_tables(off + F + 1, N, 20, D, P)
    xd = _dev(x)
    dev_rope = (None if fcs is None else fcs.to(DEV), None if tcs is None else tcs.to(DEV), P, off)
    o, S, z = ls.ls_relu_block_forward_prologue(xd["q"], xd["k"], xd["v"], None if wq is None else wq.to(DEV),
                                                None if wk is None else wk.to(DEV), norm_eps=1e-5,
                                                block_frames=bf, rope=dev_rope)
    torch.cuda.synchronize()
    rnd = "bf16" if dt == "bf16" else None
    rope = (fcs, tcs, P, off)
    qn, qd = oracle_mod.relu_rope_features(x["q"], wq, eps=1e-5, rope=rope, round_to=rnd)
    kn, kd = oracle_mod.relu_rope_features(x["k"], wk, eps=1e-5, rope=rope, round_to=rnd)
    ro, rS, rz = oracle_mod.linear_block_split(qn, kn, qd, kd, x["v"], block_frames=bf)
    tag = "relu rope H%d F%d N%d D%d %s q%d k%d P%d off%d bf%d" % (H, F, N, D, dt, qw, kw, P, off, bf)
    check(tag + " o", o, ro, TOL[dt][0], dt)
    check(tag + " S", S, rS, TOL[dt][1], dt)
    check(tag + " z", z, rz, TOL[dt][1], dt)


# --------------------------------------------------------------------------- degenerate cases
@pytest.mark.parametrize("B,H,F,N,D,dt", [(1, 2, 10, 300, 128, "bf16"), (1, 40, 5, 130, 128, "bf16"),
                                          (1, 2, 10, 200, 112, "bf16"), (1, 2, 10, 40, 64, "bf16"),
                                          (1, 2, 10, 20, 32, "fp32")])
def test_gdn_degenerate_gates(ls, gen, oracle_mod, B, H, F, N, D, dt):
    """Frames with alpha = 0 (the state resets to beta U), beta = 0 (pure
    decay), alpha = 1 and beta = 0 (the state passes unchanged) and alpha =
    beta = 1, mixed in one call from a nonzero initial state."""
    x = gen.gdn_inputs(B, H, F, N, D, dt, seed=63, part=N, l2_keys=True)
    a, b = x["alpha"].clone(), x["beta"].clone()
    for f in range(F):
        if f % 5 == 1:
            a[:, :, f] = 0.0
        elif f % 5 == 2:
            b[:, :, f] = 0.0
        elif f % 5 == 3:
            a[:, :, f], b[:, :, f] = 1.0, 0.0
        elif f % 5 == 4:
            a[:, :, f], b[:, :, f] = 1.0, 1.0
    x["alpha"], x["beta"] = a.contiguous(), b.contiguous()
    S0 = _rand_state(B, H, D, 64, scale=0.5)
    xd = _dev(x)
    o, S = ls.ls_gdn_frame_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], S0.to(DEV))
    torch.cuda.synchronize()
    ro, rS = oracle_mod.gdn_frame(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0)
    tag = "gdn degenerate gates B%d H%d F%d N%d D%d %s" % (B, H, F, N, D, dt)
    check(tag + " o", o, ro, TOL[dt][0], dt)
    check(tag + " S", S, rS, TOL[dt][1], dt)


def test_gdn_more_frames_than_the_decay_window(ls, gen, oracle_mod):
    """2098 frames in one call: the scan items hold the decays of 2048 frames at
    a time, so the call crosses a window boundary (frame-interleaved launch)."""
    B, H, F, N, D, dt = 1, 2, 2098, 4, 128, "bf16"
    x = gen.gdn_inputs(B, H, F, N, D, dt, seed=65, part=N, l2_keys=True)
    xd = _dev(x)
    o, S = ls.ls_gdn_frame_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"])
    torch.cuda.synchronize()
    ro, rS = oracle_mod.gdn_frame(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    tag = "gdn long call F%d" % F
    check(tag + " o", o, ro, TOL[dt][0], dt)
    check(tag + " S", S, rS, TOL[dt][1], dt)


@pytest.mark.parametrize("H,F,N,D,dt", [(3, 4, 333, 32, "bf16"), (2, 3, 200, 64, "bf16"), (2, 3, 150, 112, "bf16"),
                                        (2, 3, 150, 128, "bf16"), (2, 3, 40, 48, "fp32")])
def test_relu_zero_features_give_zero_outputs(ls, gen, H, F, N, D, dt):
    """Queries with every entry negative have phi(q) = 0: the numerator is an
    empty sum and the output is exactly zero (denominator eps)."""
    x = gen.relu_inputs(1, H, F, N, D, dt, seed=67, part=N)
    q = -x["q"].abs()
    xd = _dev(x)
    o, S, z = ls.ls_relu_block_forward(q.to(DEV), xd["k"], xd["v"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
