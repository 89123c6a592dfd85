"""Seeded synthetic inputs for the block-causal linear-attention scan.

This module only draws random tensors of the shapes and distributions of the
video workloads; it holds none of the scan's arithmetic.  Both the GPU library
(through the tests and the benchmark) and the fp64 oracle consume what it
returns, so the two always see identical values.

Recipe (one torch.Generator per tensor):
  seed value = (1000 * workload_seed + stream) * 1000 + part
  streams: q=0, k=1, v=2, alpha=3, beta=4; the 60-frame state-building prefix
  of the chunk-step workload uses 10 + stream.  `part` numbers the call of a
  block-autoregressive rollout or the denoising step (0 for a single call).
  q, k, v ~ N(0, 1) drawn in float32 and rounded to the token dtype (bf16 by
  round-to-nearest-even, or kept as fp32).  For the Gated-DeltaNet workloads
  with `l2_keys`, each key token is divided by its float32 L2 norm before the
  rounding.  alpha = sigmoid(N(alpha_mu, 0.5)), beta = sigmoid(N(0, 1)) per
  (batch, head, frame), float32; per-token update gates (stream 5) are
  sigmoid(N(0, 1)) per (batch, head, frame, token), float32.

Large tensors are drawn frame-chunk by frame-chunk from one generator so that
peak temporary memory stays bounded; the chunking is fixed, so results depend
only on the seed and the device.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

Q, K, V, ALPHA, BETA, TOKEN_GATE = 0, 1, 2, 3, 4, 5
PREFIX = 10

_DTYPES = {"bf16": torch.bfloat16, "fp32": torch.float32}


@dataclass(frozen=True)
class Workload:
    """A named shape: B batch, H heads, F frames, N tokens per frame, D head dim."""
    name: str
    op: str                    # "relu" or "gdn" (the tiny case runs both)
    B: int
    H: int
    F: int
    N: int
    D: int
    dtype: str
    seed: int
    call_frames: int = 0       # frames per call of a block-autoregressive rollout (0 = one call)
    alpha_mu: float = 3.0
    l2_keys: bool = False
    steps: int = 0             # denoising steps re-reading one carried state
    prefix_frames: int = 0     # frames that build the carried state
    note: str = field(default="", compare=False)

    @property
    def calls(self):
        """Frame ranges [f0, f1) of the successive calls."""
        cf = self.call_frames or self.F
        return [(f0, min(self.F, f0 + cf)) for f0 in range(0, self.F, cf)]

    @property
    def tokens(self) -> int:
        """Scan tokens per pass, B * F * N (all heads of a token count once)."""
        return self.B * self.F * self.N * max(1, self.steps)


WORKLOADS = {
    # tiny correctness case: fp32, both ops, raw N(0,1) keys, alpha ~ sigmoid(N(2, .5))
    "tiny": Workload("tiny", "both", 1, 2, 4, 16, 16, "fp32", 0, alpha_mu=2.0, l2_keys=False,
                     note="B1 H2 D16 F4 N16 fp32"),
    # SANA-Video 480p, 5 s: 81 frames at 4x temporal stride -> 21 latent frames,
    # 480x832 / 8 (VAE) / 2 (patch) -> 30x52 tokens; 70 heads of 32 (hidden 2240)
    "sana_video_480p_5s": Workload("sana_video_480p_5s", "relu", 1, 70, 21, 1560, 32, "bf16", 1,
                                   note="B1 H70 D32 F21 N1560 bf16, one call"),
    # SANA-Video 720p minute-scale: 45x80 tokens, 241 latent frames in 10-frame calls
    "sana_video_720p_minute": Workload("sana_video_720p_minute", "relu", 1, 70, 241, 3600, 32,
                                       "bf16", 2, call_frames=10,
                                       note="B1 H70 D32 N3600, 241 frames as 24x10 + 1 calls"),
    # SANA-WM 720p 60 s frame-wise GDN: 23x40 tokens, 181 latent frames, 24 heads of 128
    "sana_wm_720p_60s": Workload("sana_wm_720p_60s", "gdn", 1, 24, 181, 920, 128, "bf16", 3,
                                 alpha_mu=3.0, l2_keys=True,
                                 note="B1 H24 D128 F181 N920 bf16, L2-normalised keys"),
    # the same two workloads at the pages' linear-attention head dim, 112, with
    # the hidden size kept (SANA-Video 20 x 112 = 2240) or the token bytes
    # kept within 2% (SANA-WM 28 x 112 = 3136 against 24 x 128 = 3072)
    "sana_video_720p_minute_d112": Workload("sana_video_720p_minute_d112", "relu", 1, 20, 241, 3600, 112,
                                            "bf16", 2, call_frames=10,
                                            note="B1 H20 D112 N3600, 241 frames as 24x10 + 1 calls"),
    "sana_wm_720p_60s_d112": Workload("sana_wm_720p_60s_d112", "gdn", 1, 28, 181, 920, 112, "bf16", 3,
                                      alpha_mu=3.0, l2_keys=True,
                                      note="B1 H28 D112 F181 N920 bf16, L2-normalised keys"),
    # SANA-WM chunk-causal inference: 50 single-frame calls re-reading one carried state
    "sana_wm_chunk_step": Workload("sana_wm_chunk_step", "gdn", 4, 24, 1, 920, 128, "bf16", 4,
                                   alpha_mu=3.0, l2_keys=True, steps=50, prefix_frames=60,
                                   note="B4 H24 D128 N920, F=1 x 50 steps on a 60-frame state"),
}


def _gen(seed: int, stream: int, part: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((1000 * seed + stream) * 1000 + part)
    return g


def token_tensor(B, H, F, N, D, dtype, seed, stream, part=0, device="cpu", l2=False,
                 chunk_elems: int = 1 << 27) -> torch.Tensor:
    """[B, H, F, N, D] tensor of N(0, 1) values (optionally unit-L2 per token)."""
    dt = _DTYPES[dtype] if isinstance(dtype, str) else dtype
    out = torch.empty((B, H, F, N, D), dtype=dt, device=device)
    g = _gen(seed, stream, part, device)
    flat = out.view(B * H * F, N, D)
    rows = max(1, chunk_elems // (N * D))
    for r0 in range(0, B * H * F, rows):
        r1 = min(B * H * F, r0 + rows)
        x = torch.randn((r1 - r0, N, D), generator=g, dtype=torch.float32, device=device)
        if l2:
            x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        flat[r0:r1].copy_(x)
        del x
    return out


def gates(B, H, F, seed, alpha_mu, part=0, device="cpu", prefix=False):
    """(alpha, beta), each [B, H, F] float32."""
    off = PREFIX if prefix else 0
    ga = _gen(seed, off + ALPHA, part, device)
    gb = _gen(seed, off + BETA, part, device)
    a = torch.sigmoid(alpha_mu + 0.5 * torch.randn((B, H, F), generator=ga, device=device))
    b = torch.sigmoid(torch.randn((B, H, F), generator=gb, device=device))
    return a.contiguous(), b.contiguous()


def token_gates(B, H, F, N, seed, part=0, device="cpu"):
    """Per-token update gates [B, H, F, N] float32, sigmoid(N(0, 1))."""
    g = _gen(seed, TOKEN_GATE, part, device)
    return torch.sigmoid(torch.randn((B, H, F, N), generator=g, device=device)).contiguous()


def rope_tables(T, N, W, D, frame_pairs, base=10000.0, device="cpu"):
    """(cos, sin) tables of a 3D rotary embedding at synthetic positions.

    Positions: frame t in [0, T); token n of a frame at row n // W, column
    n % W of the latent grid.  The first `frame_pairs` channel pairs turn with
    the frame index, the remaining pairs split between row (first half) and
    column; pair j of an axis group of m pairs has frequency base^(-j/m).
    Returns (frame_cs [T, frame_pairs, 2], token_cs [N, D/2 - frame_pairs, 2])
    float32, angles formed in float64 and rounded once.
    """
    half = D // 2
    sp = half - frame_pairs
    rows = sp // 2

    def table(pos, m):
        j = torch.arange(m, dtype=torch.float64)
        ang = pos[:, None].double() * base ** (-j / max(m, 1))[None, :]
        return torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1)

    frame_cs = table(torch.arange(T), frame_pairs) if frame_pairs > 0 else None
    token_cs = None
    if sp > 0:
        n = torch.arange(N)
        token_cs = torch.cat([table(n // W, rows), table(n % W, sp - rows)], dim=1)
    cast = lambda t: None if t is None else t.to(torch.float32).contiguous().to(device)
    return cast(frame_cs), cast(token_cs)


def relu_inputs(B, H, F, N, D, dtype="bf16", seed=0, part=0, device="cpu"):
    """q, k, v for the ReLU linear-attention scan."""
    return {
        "q": token_tensor(B, H, F, N, D, dtype, seed, Q, part, device),
        "k": token_tensor(B, H, F, N, D, dtype, seed, K, part, device),
        "v": token_tensor(B, H, F, N, D, dtype, seed, V, part, device),
    }


def gdn_inputs(B, H, F, N, D, dtype="bf16", seed=0, part=0, device="cpu", alpha_mu=3.0,
               l2_keys=True, prefix=False):
    """q, k, v, alpha, beta for the frame-wise Gated DeltaNet scan."""
    off = PREFIX if prefix else 0
    a, b = gates(B, H, F, seed, alpha_mu, part, device, prefix=prefix)
    return {
        "q": token_tensor(B, H, F, N, D, dtype, seed, off + Q, part, device),
        "k": token_tensor(B, H, F, N, D, dtype, seed, off + K, part, device, l2=l2_keys),
        "v": token_tensor(B, H, F, N, D, dtype, seed, off + V, part, device),
        "alpha": a,
        "beta": b,
    }


def workload_call_inputs(w: Workload, call: int, device="cpu", op=None):
    """Inputs of call `call` of workload `w` (a block of a rollout, or a step)."""
    op = op or w.op
    if op == "relu":
        f0, f1 = w.calls[call]
        return relu_inputs(w.B, w.H, f1 - f0, w.N, w.D, w.dtype, w.seed, call, device)
    if w.steps:
        return gdn_inputs(w.B, w.H, w.F, w.N, w.D, w.dtype, w.seed, call + 1, device,
                          w.alpha_mu, w.l2_keys)
    f0, f1 = w.calls[call]
    return gdn_inputs(w.B, w.H, f1 - f0, w.N, w.D, w.dtype, w.seed, call, device, w.alpha_mu,
                      w.l2_keys)


def prefix_inputs(w: Workload, device="cpu"):
    """Inputs of the frames that build the carried state of a chunk-step workload."""
    return gdn_inputs(w.B, w.H, w.prefix_frames, w.N, w.D, w.dtype, w.seed, 0, device,
                      w.alpha_mu, w.l2_keys, prefix=True)
