"""fp64 CPU oracle for the block-causal linear-attention scan.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It does not import, link or call the
GPU library and the GPU library never calls it.

The arithmetic lives in ``oracle.c`` (plain loops over frames and tokens in
double precision, each function citing the passage it follows).  This module
only builds that file with gcc, loads it with ctypes and marshals numpy arrays.

Inputs are taken as float32 arrays (bf16 and fp32 values widen to float32
exactly); states and outputs come back as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O3, OpenMP) into oracle/liboracle.so."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i = ctypes.c_int
    d = ctypes.c_double
    lib.oracle_relu_block.argtypes = [i, i, i, i, i, i, d, P, P, P, P, P, P, P, P, i]
    lib.oracle_relu_block.restype = i
    lib.oracle_gdn_frame.argtypes = [i, i, i, i, i, d, P, P, P, P, P, P, P, P, i]
    lib.oracle_gdn_frame.restype = i
    lib.oracle_gdn_frame_token_gate.argtypes = [i, i, i, i, i, d, P, P, P, P, P, P, P, P, i]
    lib.oracle_gdn_frame_token_gate.restype = i
    lib.oracle_gdn_frame_reversed.argtypes = [i, i, i, i, i, i, d, P, P, P, P, P, P, i]
    lib.oracle_gdn_frame_reversed.restype = i
    lib.oracle_temporal_conv3.argtypes = [i, i, i, i, i, i, P, P, P, P, P, P]
    lib.oracle_temporal_conv3.restype = i
    lib.oracle_linear_block_split.argtypes = [i, i, i, i, i, i, d, P, P, P, P, P, P, P, P, P, P, i]
    lib.oracle_linear_block_split.restype = i
    lib.oracle_max_threads.restype = i
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f32(x, shape=None):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: widen on the CPU (exact for bf16/fp32)
        x = x.detach().to("cpu").float().numpy()
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if shape is not None and a.shape != tuple(shape):
        a = a.reshape(shape)
    return a


def _f64(x, shape):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(shape))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def relu_block(q, k, v, state=None, norm=None, block_frames: int = 1, eps: float = 1e-6,
               with_output: bool = True, nthreads: int = 0):
    """ReLU block-causal linear attention, fp64.

    q, k, v: [B, H, F, N, D].  state: [B, H, D, D] or None (zeros);
    norm: [B, H, D] or None (zeros).  Returns (o or None, S, z) as float64.
    """
    k = _f32(k)
    B, H, F, N, D = k.shape
    v = _f32(v, k.shape)
    q = _f32(q, k.shape) if with_output else None
    S0 = _f64(state, (B, H, D, D))
    z0 = _f64(norm, (B, H, D))
    o = np.empty((B, H, F, N, D), np.float64) if with_output else None
    S = np.empty((B, H, D, D), np.float64)
    z = np.empty((B, H, D), np.float64)
    rc = _load().oracle_relu_block(B, H, F, N, D, int(block_frames), float(eps),
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0),
                                   _ptr(o), _ptr(S), _ptr(z), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_relu_block failed with code %d" % rc)
    return o, S, z


def linear_block_split(qn, kn, qd, kd, v, state=None, norm=None, block_frames: int = 1, eps: float = 1e-6,
                       nthreads: int = 0):
    """Block-causal linear attention with numerator features (qn, kn) and
    denominator features (qd, kd), fp64 (oracle.c, oracle_linear_block_split).

    Features: [B, H, F, N, D] (float64 kept exact); v as for relu_block.
    Returns (o, S, z) as float64.
    """
    kn = _f64(kn, np.shape(kn))
    B, H, F, N, D = kn.shape
    qn, qd, kd = (_f64(a, (B, H, F, N, D)) for a in (qn, qd, kd))
    v = _f32(v, (B, H, F, N, D))
    S0 = _f64(state, (B, H, D, D))
    z0 = _f64(norm, (B, H, D))
    o = np.empty((B, H, F, N, D), np.float64)
    S = np.empty((B, H, D, D), np.float64)
    z = np.empty((B, H, D), np.float64)
    rc = _load().oracle_linear_block_split(B, H, F, N, D, int(block_frames), float(eps), _ptr(qn), _ptr(kn),
                                           _ptr(qd), _ptr(kd), _ptr(v), _ptr(S0), _ptr(z0), _ptr(o), _ptr(S),
                                           _ptr(z), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_linear_block_split failed with code %d" % rc)
    return o, S, z


def relu_rope_features(x, weight=None, eps: float = 1e-6, rope=None, round_to=None):
    """Numerator and denominator features of the ReLU scan with the prologue.

    The denominator takes phi(x') = ReLU of the prologue's RMSNorm result x'
    (fp64, unrounded); the numerator takes the rotated phi(x'), rounded to the
    token precision (round_to) as the contractions consume it.  Without rope
    both are phi(x') (the numerator rounded).  Returns (numerator, denominator).
    """
    d = prologue(x, weight, eps=eps, relu=True)
    n = rope_rotate(d, *rope) if rope is not None else d
    if round_to == "bf16":
        n = round_bf16(n)
    return n, d


def gdn_frame(q, k, v, alpha, beta, state=None, key_scale=None, with_output: bool = True,
              nthreads: int = 0):
    """Frame-wise Gated DeltaNet, fp64.

    q, k, v: [B, H, F, N, D]; alpha, beta: [B, H, F]; state: [B, H, D, D] or
    None (zeros); key_scale None means 1/sqrt(D*N).  Returns (o or None, S).
    """
    k = _f32(k)
    B, H, F, N, D = k.shape
    v = _f32(v, k.shape)
    q = _f32(q, k.shape) if with_output else None
    a = _f32(alpha, (B, H, F))
    b = _f32(beta, (B, H, F))
    S0 = _f64(state, (B, H, D, D))
    o = np.empty((B, H, F, N, D), np.float64) if with_output else None
    S = np.empty((B, H, D, D), np.float64)
    c = -1.0 if key_scale is None else float(key_scale)
    rc = _load().oracle_gdn_frame(B, H, F, N, D, c, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                  _ptr(S0), _ptr(o), _ptr(S), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_gdn_frame failed with code %d" % rc)
    return o, S


def gdn_frame_token_gate(q, k, v, alpha, beta, state=None, key_scale=None, with_output: bool = True,
                         nthreads: int = 0):
    """Frame-wise Gated DeltaNet with a per-token update gate, fp64.

    As gdn_frame, but beta is [B, H, F, N]: token n's gate weights its terms
    of the frame's G and U (the transition is S <- alpha S (I - G) + U).
    """
    k = _f32(k)
    B, H, F, N, D = k.shape
    v = _f32(v, k.shape)
    q = _f32(q, k.shape) if with_output else None
    a = _f32(alpha, (B, H, F))
    b = _f32(beta, (B, H, F, N))
    S0 = _f64(state, (B, H, D, D))
    o = np.empty((B, H, F, N, D), np.float64) if with_output else None
    S = np.empty((B, H, D, D), np.float64)
    c = -1.0 if key_scale is None else float(key_scale)
    rc = _load().oracle_gdn_frame_token_gate(B, H, F, N, D, c, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                             _ptr(S0), _ptr(o), _ptr(S), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_gdn_frame_token_gate failed with code %d" % rc)
    return o, S


def gdn_frame_reversed(q, k, v, alpha, beta, chunk_frames: int, key_scale=None, nthreads: int = 0):
    """Reversed frame-wise Gated DeltaNet, reset at chunk boundaries, fp64.

    Frames are cut into chunks of chunk_frames from frame 0; each chunk is
    scanned from its last frame to its first, from a zero state.  Returns o.
    """
    k = _f32(k)
    B, H, F, N, D = k.shape
    v = _f32(v, k.shape)
    q = _f32(q, k.shape)
    a = _f32(alpha, (B, H, F))
    b = _f32(beta, (B, H, F))
    o = np.empty((B, H, F, N, D), np.float64)
    c = -1.0 if key_scale is None else float(key_scale)
    rc = _load().oracle_gdn_frame_reversed(B, H, F, N, D, int(chunk_frames), c, _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(a), _ptr(b), _ptr(o), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_gdn_frame_reversed failed with code %d" % rc)
    return o


def temporal_conv3(x, weight, bias=None, carry=None, block_frames: int = 1, with_carry: bool = True):
    """Block-causal temporal convolution of kernel 3 along frames, fp64.

    x: [B, H, F, N, D]; weight: [H, D, 3] (taps on frames f-1, f, f+1);
    bias: [H, D] or None; carry: [B, H, N, D] (frame -1) or None (zeros).
    Frame f's next-frame tap sees zero when f ends its block of block_frames.
    Returns (y, carry_out) with carry_out = x[:, :, F-1].
    """
    x = _f32(x)
    B, H, F, N, D = x.shape
    w = _f32(weight, (H, D, 3))
    b = _f32(bias, (H, D))
    c = _f32(carry, (B, H, N, D))
    y = np.empty((B, H, F, N, D), np.float64)
    co = np.empty((B, H, N, D), np.float64) if with_carry else None
    rc = _load().oracle_temporal_conv3(B, H, F, N, D, int(block_frames), _ptr(x), _ptr(w), _ptr(b), _ptr(c),
                                       _ptr(y), _ptr(co))
    if rc != 0:
        raise RuntimeError("oracle_temporal_conv3 failed with code %d" % rc)
    return y, co


def prologue(x, weight=None, eps: float = 1e-6, relu: bool = False, l2: bool = False, round_to=None, rope=None):
    """The per-token prologue fused into the scans' load stage, fp64.

    The SANA-WM digest (paragraph on context parallelism and the fused kernel)
    fuses RMSNorm, ReLU and the key scaling into the GDN scan; SANA-Video's
    linear attention normalises q and k (qk_norm) before its ReLU feature map.
    Per token row x (the D channels of one head):
      RMSNorm:  x <- x / sqrt(mean(x^2) + eps) * weight[h]   (when weight is given)
      ReLU:     x <- max(x, 0)                               (when relu)
      L2:       x <- x / |x|  (0 stays 0)                     (when l2)
      RoPE:     rope_rotate(x, *rope)                         (when rope is given)
    x: [B, H, F, N, D]; weight: [H, D] or None.  round_to = "bf16" rounds the
    result to bfloat16 (nearest even), the precision in which the scan
    consumes it for bf16 tokens.  Returns float64 (or the rounded values as
    float64).
    """
    x = np.asarray(_f32(x), dtype=np.float64)
    y = x
    if weight is not None:
        w = np.asarray(_f32(weight), dtype=np.float64)
        ms = np.mean(y * y, axis=-1, keepdims=True)
        y = y / np.sqrt(ms + eps) * w[None, :, None, None, :]
    if relu:
        y = np.where(np.signbit(y), 0.0, y)
    if l2:
        nrm = np.sqrt(np.sum(y * y, axis=-1, keepdims=True))
        y = np.where(nrm > 0, y / np.where(nrm > 0, nrm, 1.0), 0.0)
    if rope is not None:
        y = rope_rotate(y, *rope)
    if round_to == "bf16":
        y = round_bf16(y)
    return y


def rope_rotate(x, frame_cs, token_cs, frame_pairs: int, frame_offset: int = 0):
    """Rotary position embedding of the token rows, fp64.

    The SANA-WM digest (paragraph on context parallelism and the fused kernel)
    lists the positional encoding among the steps fused into the GDN scan, and
    SANA-Video's talk uses a 3D RoPE in its linear attention.  Each channel
    pair (x[2i], x[2i+1]) of the token of frame f (of the call) and index n
    turns by an angle whose (cos, sin) the caller tabulates:
        (x0, x1) <- (x0 cos - x1 sin, x0 sin + x1 cos)
    with (cos, sin) = frame_cs[frame_offset + f, i] for i < frame_pairs (the
    frame axis) and token_cs[n, i - frame_pairs] for the other pairs (the
    spatial axes).  x: [B, H, F, N, D]; frame_cs: [T, frame_pairs, 2];
    token_cs: [N, D/2 - frame_pairs, 2] (either None when it has no pairs).
    """
    y = np.asarray(_f32(x), dtype=np.float64) if not (isinstance(x, np.ndarray) and x.dtype == np.float64) else x
    B, H, F, N, D = y.shape
    half = D // 2
    cos = np.empty((F, N, half))
    sin = np.empty((F, N, half))
    if frame_pairs > 0:
        fc = np.asarray(_f32(frame_cs), dtype=np.float64)[frame_offset:frame_offset + F]
        cos[:, :, :frame_pairs] = fc[:, None, :, 0]
        sin[:, :, :frame_pairs] = fc[:, None, :, 1]
    if frame_pairs < half:
        tc = np.asarray(_f32(token_cs), dtype=np.float64)
        cos[:, :, frame_pairs:] = tc[None, :, :, 0]
        sin[:, :, frame_pairs:] = tc[None, :, :, 1]
    x0, x1 = y[..., 0::2], y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


def round_bf16(y):
    """Round float64 values to the nearest bfloat16 value, ties to the even one.

    One rounding from the exact float64 value: of the two bfloat16 neighbours
    (the value cut to its top 8 significant bits, and that plus one bfloat16
    step away from zero) take the nearer, and on a tie the one whose last kept
    bit is 0.  (Going through float32 first would round twice: a value just
    past a halfway point can land on it and then go to the even side.)
    Finite values in the normal float32 range.  Returns float64.
    """
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float64))
    bits = y.view(np.uint64)
    drop = np.uint64((1 << 45) - 1)                  # fraction bits below bfloat16's 7
    lo_bits = bits & ~drop
    lo = lo_bits.view(np.float64)                     # toward zero
    hi = (lo_bits + np.uint64(1 << 45)).view(np.float64)  # one step away from zero
    d_lo = np.abs(y - lo)                             # both differences are exact
    d_hi = np.abs(hi - y)
    odd = ((lo_bits >> np.uint64(45)) & np.uint64(1)) == 1
    return np.where((d_hi < d_lo) | ((d_hi == d_lo) & odd), hi, lo)
