"""Thin ctypes binding of liblinscan with the C entry points' names.

Only argument marshalling happens here: torch device tensors are checked for
dtype, shape, contiguity and device, and their data pointers, the workspace
and the current HIP stream are passed to the C ABI, where every step of the
scan runs in HIP kernels.  If liblinscan.so has not been built this module
raises on import: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes  # noqa: F401  (re-exported for callers building ls_shape)
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinscan.so")

LS_OK = 0
LS_ERR_HIP = 8
LS_DTYPE_FP32 = 0
LS_DTYPE_BF16 = 1
_DT = {torch.float32: LS_DTYPE_FP32, torch.bfloat16: LS_DTYPE_BF16}


class ls_strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong), ("frame", ctypes.c_longlong),
                ("token", ctypes.c_longlong)]


class ls_prologue(ctypes.Structure):
    _fields_ = [("q_weight", ctypes.c_void_p), ("k_weight", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("relu", ctypes.c_int), ("l2_keys", ctypes.c_int), ("rope_frame", ctypes.c_void_p),
                ("rope_token", ctypes.c_void_p), ("rope_frame_pairs", ctypes.c_int),
                ("rope_frame_offset", ctypes.c_int), ("rope_frames", ctypes.c_longlong)]


class LinscanError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("liblinscan status %d: %s" % (status, message))
        self.status = status


class ls_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("F", ctypes.c_int),
                ("N", ctypes.c_int), ("D", ctypes.c_int), ("dtype", ctypes.c_int)]


class ls_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblinscan.so is not built (%s); run "
                          "`python -m block_causal_linear_attn_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    SP = ctypes.POINTER(ls_shape)
    lib.ls_relu_block_workspace_size.argtypes = [SP]
    lib.ls_relu_block_workspace_size.restype = Z
    lib.ls_relu_block_forward.argtypes = [SP, I, F, P, P, P, P, P, P, P, P, P, Z, P]
    lib.ls_relu_block_forward.restype = I
    lib.ls_gdn_frame_workspace_size.argtypes = [SP]
    lib.ls_gdn_frame_workspace_size.restype = Z
    lib.ls_gdn_frame_forward.argtypes = [SP, F, P, P, P, P, P, P, P, P, P, Z, P]
    lib.ls_gdn_frame_forward.restype = I
    lib.ls_gdn_frame_forward_noalloc.argtypes = [SP, F, P, P, P, P, P, P, P, P, P, P]
    lib.ls_gdn_frame_forward_noalloc.restype = I
    ST = ctypes.POINTER(ls_strides)
    PR = ctypes.POINTER(ls_prologue)
    lib.ls_relu_block_forward_prologue.argtypes = [SP, PR, I, F, P, P, P, P, P, P, P, P, P, Z, P]
    lib.ls_relu_block_forward_prologue.restype = I
    lib.ls_gdn_frame_forward_prologue.argtypes = [SP, PR, F, P, P, P, P, P, P, P, P, P, Z, P]
    lib.ls_gdn_frame_forward_prologue.restype = I
    lib.ls_relu_block_forward_strided.argtypes = [SP, ST, I, F, P, P, P, P, P, P, P, P, P, Z, P]
    lib.ls_relu_block_forward_strided.restype = I
    lib.ls_gdn_frame_forward_strided.argtypes = [SP, ST, F, P, P, P, P, P, P, P, P, P, Z, P]
    lib.ls_gdn_frame_forward_strided.restype = I
    lib.ls_gdn_frame_forward_token_gate.argtypes = [SP, F, P, P, P, P, P, P, P, P, P, Z, P]
    lib.ls_gdn_frame_forward_token_gate.restype = I
    lib.ls_gdn_frame_forward_reversed.argtypes = [SP, I, F, P, P, P, P, P, P, P, Z, P]
    lib.ls_gdn_frame_forward_reversed.restype = I
    lib.ls_temporal_conv3.argtypes = [SP, I, P, P, P, P, P, P, P]
    lib.ls_temporal_conv3.restype = I
    lib.ls_state_carry.argtypes = [I, I, I, P, P, P, P, I, P]
    lib.ls_state_carry.restype = I
    lib.ls_status_string.argtypes = [I]
    lib.ls_status_string.restype = ctypes.c_char_p
    lib.ls_last_error.argtypes = []
    lib.ls_last_error.restype = ctypes.c_char_p
    lib.ls_version.argtypes = []
    lib.ls_version.restype = I
    lib.ls_profile_begin.argtypes = []
    lib.ls_profile_begin.restype = I
    lib.ls_profile_end.argtypes = [ctypes.POINTER(ls_kernel_stat), I]
    lib.ls_profile_end.restype = I
    return lib


lib = _load()

EXPORTS = ("ls_relu_block_workspace_size", "ls_relu_block_forward", "ls_gdn_frame_workspace_size",
           "ls_gdn_frame_forward", "ls_gdn_frame_forward_noalloc", "ls_gdn_frame_forward_token_gate",
           "ls_gdn_frame_forward_reversed", "ls_temporal_conv3", "ls_relu_block_forward_strided",
           "ls_gdn_frame_forward_strided", "ls_relu_block_forward_prologue", "ls_gdn_frame_forward_prologue",
           "ls_state_carry", "ls_status_string", "ls_last_error",
           "ls_version", "ls_profile_begin", "ls_profile_end")


def _check(status: int):
    if status != LS_OK:
        detail = lib.ls_last_error().decode() or lib.ls_status_string(status).decode()
        raise LinscanError(status, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _tokens(name, t, like=None):
    if not isinstance(t, torch.Tensor) or t.dim() != 5:
        raise ValueError("%s must be a 5-D [B, H, F, N, D] tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must live on a GPU (got %s)" % (name, t.device))
    if t.dtype not in _DT:
        raise ValueError("%s must be float32 or bfloat16 (got %s)" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if like is not None and (t.shape != like.shape or t.dtype != like.dtype or t.device != like.device):
        raise ValueError("%s must match q in shape, dtype and device" % name)
    return t


def _strided_tokens(name, t, like=None):
    """A 5-D [B, H, F, N, D] view with D contiguous (any other strides), matching `like`'s strides."""
    if not isinstance(t, torch.Tensor) or t.dim() != 5:
        raise ValueError("%s must be a 5-D [B, H, F, N, D] tensor (a view of any layout)" % name)
    if t.device.type != "cuda" or t.dtype not in _DT:
        raise ValueError("%s must be a float32 or bfloat16 GPU tensor" % name)
    if t.shape[4] > 1 and t.stride(4) != 1:
        raise ValueError("%s must have its last dimension contiguous" % name)
    if like is not None and (t.shape != like.shape or t.dtype != like.dtype or t.device != like.device
                             or t.stride() != like.stride()):
        raise ValueError("%s must match q in shape, dtype, device and strides" % name)
    return t


def _layout(t) -> ls_strides:
    return ls_strides(*t.stride()[:4])


def _f32(name, t, shape, device):
    if t is None:
        return None
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or t.device != device \
            or not t.is_contiguous():
        raise ValueError("%s must be a contiguous float32 tensor of shape %s on %s"
                         % (name, tuple(shape), device))
    return t


_ws_lock = threading.Lock()
_ws_cache: dict = {}


def workspace(nbytes: int, device) -> torch.Tensor:
    """A cached uint8 device buffer of at least nbytes (per device and stream).

    A new buffer starts zeroed, so its fault word (the first 4 bytes, which a
    bounded wait that gives up sets) reads 0; a buffer replaced by a larger
    one hands its fault word on, so no fault is lost.
    """
    key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            new = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            if buf is not None:
                new[:4].copy_(buf[:4])
            buf = new
            _ws_cache[key] = buf
        return buf


def _cached(device=None, ws=None):
    if ws is not None:
        return [ws]
    idx = None if device is None else torch.device(device).index
    with _ws_lock:
        return [b for (d, _), b in _ws_cache.items() if idx is None or d == idx]


def ls_fault_word(device=None, ws=None) -> int:
    """The fault word of `ws`, or the OR of the cached workspaces' words (all
    devices, or `device`'s): nonzero when a bounded wait of a single-launch
    call gave up, so that call's results are invalid.  Synchronises with the
    device (it reads device memory)."""
    word = 0
    for b in _cached(device, ws):
        word |= int(b[:4].view(torch.int32).item())
    return word


def ls_clear_fault_word(device=None, ws=None) -> None:
    """Zero the fault word of `ws`, or of every cached workspace (of `device`);
    the library only ever sets it."""
    for b in _cached(device, ws):
        b[:4].zero_()


def _shape(q) -> ls_shape:
    B, H, F, N, D = q.shape
    return ls_shape(B, H, F, N, D, _DT[q.dtype])


def ls_relu_block_forward(q, k, v, state=None, norm=None, block_frames: int = 1, eps: float = 1e-6,
                          out=None, state_out=None, norm_out=None, ws=None):
    """ReLU block-causal linear attention; returns (o, state_out, norm_out).

    q, k, v: [B, H, F, N, D] fp32 or bf16 on one GPU.  state [B, H, D, D] and
    norm [B, H, D] (fp32) seed the scan (zeros when None).  New output
    tensors are allocated unless given; pass state_out=state (and
    norm_out=norm) for an in-place update.
    """
    _tokens("q", q)
    _tokens("k", k, q)
    _tokens("v", v, q)
    B, H, F, N, D = q.shape
    dev = q.device
    _f32("state", state, (B, H, D, D), dev)
    _f32("norm", norm, (B, H, D), dev)
    o = out if out is not None else torch.empty_like(q)
    _tokens("out", o, q)
    so = state_out if state_out is not None else torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    no = norm_out if norm_out is not None else torch.empty((B, H, D), dtype=torch.float32, device=dev)
    _f32("state_out", so, (B, H, D, D), dev)
    _f32("norm_out", no, (B, H, D), dev)
    shp = _shape(q)
    need = lib.ls_relu_block_workspace_size(ctypes.byref(shp))
    w = ws if ws is not None else workspace(need, dev)
    _check(lib.ls_relu_block_forward(ctypes.byref(shp), int(block_frames), float(eps), _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(o), _ptr(state), _ptr(norm), _ptr(so), _ptr(no),
                                     _ptr(w), w.numel(), _stream(dev)))
    return o, so, no


def ls_gdn_frame_forward(q, k, v, alpha, beta, state=None, key_scale=None, out=None, state_out=None,
                         ws=None):
    """Frame-wise Gated DeltaNet; returns (o, state_out).

    alpha, beta: [B, H, F] fp32.  key_scale None means 1/sqrt(D*N).
    """
    _tokens("q", q)
    _tokens("k", k, q)
    _tokens("v", v, q)
    B, H, F, N, D = q.shape
    dev = q.device
    _f32("alpha", alpha, (B, H, F), dev)
    _f32("beta", beta, (B, H, F), dev)
    _f32("state", state, (B, H, D, D), dev)
    o = out if out is not None else torch.empty_like(q)
    _tokens("out", o, q)
    so = state_out if state_out is not None else torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    _f32("state_out", so, (B, H, D, D), dev)
    shp = _shape(q)
    need = lib.ls_gdn_frame_workspace_size(ctypes.byref(shp))
    w = ws if ws is not None else workspace(need, dev)
    scale = 0.0 if key_scale is None else float(key_scale)
    _check(lib.ls_gdn_frame_forward(ctypes.byref(shp), scale, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                    _ptr(beta), _ptr(o), _ptr(state), _ptr(so), _ptr(w), w.numel(),
                                    _stream(dev)))
    return o, so


NOALLOC_SCRATCH_BYTES = 64 << 20  # LS_NOALLOC_SCRATCH_BYTES


def ls_gdn_frame_forward_noalloc(q, k, v, alpha, beta, out, state=None, state_out=None, key_scale=None,
                                 fault=None):
    """ls_gdn_frame_forward without a workspace: the library's static device
    scratch (LS_NOALLOC_SCRATCH_BYTES per GPU) holds it, and nothing is
    allocated, here or in the library.  The caller passes every output: out
    like q, state_out [B, H, D, D] fp32 or None (not written), fault a
    one-element int32 device tensor the kernels set nonzero if a bounded wait
    gave up, or None.  Calls that overlap in time on one GPU race."""
    _tokens("q", q)
    _tokens("k", k, q)
    _tokens("v", v, q)
    _tokens("out", out, q)
    B, H, F, N, D = q.shape
    dev = q.device
    _f32("alpha", alpha, (B, H, F), dev)
    _f32("beta", beta, (B, H, F), dev)
    _f32("state", state, (B, H, D, D), dev)
    _f32("state_out", state_out, (B, H, D, D), dev)
    if fault is not None and (fault.dtype != torch.int32 or fault.numel() < 1 or fault.device != dev):
        raise ValueError("fault must be an int32 tensor on %s" % dev)
    shp = _shape(q)
    scale = 0.0 if key_scale is None else float(key_scale)
    _check(lib.ls_gdn_frame_forward_noalloc(ctypes.byref(shp), scale, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                            _ptr(beta), _ptr(out), _ptr(state), _ptr(state_out), _ptr(fault),
                                            _stream(dev)))
    return out, state_out


def ls_relu_block_forward_strided(q, k, v, state=None, norm=None, block_frames: int = 1, eps: float = 1e-6,
                                  out=None, state_out=None, norm_out=None, ws=None):
    """ls_relu_block_forward on [B, H, F, N, D] views of another layout.

    q, k, v (and out) share one set of strides, with D contiguous; for
    tensors stored [B, F, N, H, D] pass x.permute(0, 3, 1, 2, 4).  A new
    output gets q's strides.
    """
    _strided_tokens("q", q)
    _strided_tokens("k", k, q)
    _strided_tokens("v", v, q)
    B, H, F, N, D = q.shape
    dev = q.device
    _f32("state", state, (B, H, D, D), dev)
    _f32("norm", norm, (B, H, D), dev)
    o = out if out is not None else torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=dev)
    _strided_tokens("out", o, q)
    so = state_out if state_out is not None else torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    no = norm_out if norm_out is not None else torch.empty((B, H, D), dtype=torch.float32, device=dev)
    _f32("state_out", so, (B, H, D, D), dev)
    _f32("norm_out", no, (B, H, D), dev)
    shp = _shape(q)
    st = _layout(q)
    need = lib.ls_relu_block_workspace_size(ctypes.byref(shp))
    w = ws if ws is not None else workspace(need, dev)
    _check(lib.ls_relu_block_forward_strided(ctypes.byref(shp), ctypes.byref(st), int(block_frames), float(eps),
                                             _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(state), _ptr(norm), _ptr(so),
                                             _ptr(no), _ptr(w), w.numel(), _stream(dev)))
    return o, so, no


def ls_gdn_frame_forward_strided(q, k, v, alpha, beta, state=None, key_scale=None, out=None, state_out=None,
                                 ws=None):
    """ls_gdn_frame_forward on [B, H, F, N, D] views of another layout (see
    ls_relu_block_forward_strided)."""
    _strided_tokens("q", q)
    _strided_tokens("k", k, q)
    _strided_tokens("v", v, q)
    B, H, F, N, D = q.shape
    dev = q.device
    _f32("alpha", alpha, (B, H, F), dev)
    _f32("beta", beta, (B, H, F), dev)
    _f32("state", state, (B, H, D, D), dev)
    o = out if out is not None else torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=dev)
    _strided_tokens("out", o, q)
    so = state_out if state_out is not None else torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    _f32("state_out", so, (B, H, D, D), dev)
    shp = _shape(q)
    st = _layout(q)
    need = lib.ls_gdn_frame_workspace_size(ctypes.byref(shp))
    w = ws if ws is not None else workspace(need, dev)
    scale = 0.0 if key_scale is None else float(key_scale)
    _check(lib.ls_gdn_frame_forward_strided(ctypes.byref(shp), ctypes.byref(st), scale, _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(alpha), _ptr(beta), _ptr(o), _ptr(state), _ptr(so), _ptr(w),
                                            w.numel(), _stream(dev)))
    return o, so


def _prologue(q, q_weight, k_weight, eps, relu, l2_keys, rope=None):
    """rope: None, or (frame_cs, token_cs, frame_pairs, frame_offset) with frame_cs [T, frame_pairs, 2] and
    token_cs [N, D/2 - frame_pairs, 2] fp32 (cos, sin) tables on the device (either None when unused)."""
    B, H, F, N, D = q.shape
    _f32("q_weight", q_weight, (H, D), q.device)
    _f32("k_weight", k_weight, (H, D), q.device)
    pr = ls_prologue(None if q_weight is None else q_weight.data_ptr(),
                     None if k_weight is None else k_weight.data_ptr(), float(eps), int(relu), int(l2_keys))
    if rope is not None:
        frame_cs, token_cs, pf, off = rope
        if frame_cs is not None:
            if frame_cs.dim() != 3:
                raise ValueError("rope frame table must be [T, frame_pairs, 2]")
            _f32("rope frame table", frame_cs, (frame_cs.shape[0], pf, 2), q.device)
            pr.rope_frame, pr.rope_frames = frame_cs.data_ptr(), frame_cs.shape[0]
        _f32("rope token table", token_cs, (N, D // 2 - pf, 2), q.device)
        if token_cs is not None:
            pr.rope_token = token_cs.data_ptr()
        pr.rope_frame_pairs, pr.rope_frame_offset = int(pf), int(off)
    return pr


def ls_relu_block_forward_prologue(q, k, v, q_weight=None, k_weight=None, norm_eps: float = 1e-6, state=None,
                                   norm=None, block_frames: int = 1, eps: float = 1e-6, out=None, state_out=None,
                                   norm_out=None, ws=None, rope=None):
    """ls_relu_block_forward with RMSNorm of q and/or k (weights [H, D] fp32) and the rotary embedding (rope as
    for _prologue; numerator only) fused into the load."""
    _tokens("q", q)
    _tokens("k", k, q)
    _tokens("v", v, q)
    B, H, F, N, D = q.shape
    dev = q.device
    pr = _prologue(q, q_weight, k_weight, norm_eps, 0, 0, rope)
    _f32("state", state, (B, H, D, D), dev)
    _f32("norm", norm, (B, H, D), dev)
    o = out if out is not None else torch.empty_like(q)
    _tokens("out", o, q)
    so = state_out if state_out is not None else torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    no = norm_out if norm_out is not None else torch.empty((B, H, D), dtype=torch.float32, device=dev)
    _f32("state_out", so, (B, H, D, D), dev)
    _f32("norm_out", no, (B, H, D), dev)
    shp = _shape(q)
    need = lib.ls_relu_block_workspace_size(ctypes.byref(shp))
    w = ws if ws is not None else workspace(need, dev)
    _check(lib.ls_relu_block_forward_prologue(ctypes.byref(shp), ctypes.byref(pr), int(block_frames), float(eps),
                                              _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(state), _ptr(norm), _ptr(so),
                                              _ptr(no), _ptr(w), w.numel(), _stream(dev)))
    return o, so, no


def ls_gdn_frame_forward_prologue(q, k, v, alpha, beta, q_weight=None, k_weight=None, norm_eps: float = 1e-6,
                                  relu: bool = False, l2_keys: bool = False, state=None, key_scale=None, out=None,
                                  state_out=None, ws=None, rope=None):
    """ls_gdn_frame_forward with the per-token prologue (RMSNorm, ReLU, L2 of keys, rotary embedding) fused
    into the load; rope as for _prologue."""
    _tokens("q", q)
    _tokens("k", k, q)
    _tokens("v", v, q)
    B, H, F, N, D = q.shape
    dev = q.device
    pr = _prologue(q, q_weight, k_weight, norm_eps, relu, l2_keys, rope)
    _f32("alpha", alpha, (B, H, F), dev)
    _f32("beta", beta, (B, H, F), dev)
    _f32("state", state, (B, H, D, D), dev)
    o = out if out is not None else torch.empty_like(q)
    _tokens("out", o, q)
    so = state_out if state_out is not None else torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    _f32("state_out", so, (B, H, D, D), dev)
    shp = _shape(q)
    need = lib.ls_gdn_frame_workspace_size(ctypes.byref(shp))
    w = ws if ws is not None else workspace(need, dev)
    scale = 0.0 if key_scale is None else float(key_scale)
    _check(lib.ls_gdn_frame_forward_prologue(ctypes.byref(shp), ctypes.byref(pr), scale, _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(alpha), _ptr(beta), _ptr(o), _ptr(state), _ptr(so), _ptr(w),
                                             w.numel(), _stream(dev)))
    return o, so


def ls_gdn_frame_forward_token_gate(q, k, v, alpha, beta, state=None, key_scale=None, out=None,
                                    state_out=None, ws=None):
    """Frame-wise Gated DeltaNet with per-token update gates; returns (o, state_out).

    alpha: [B, H, F] fp32; beta: [B, H, F, N] fp32 (one gate per token).
    """
    _tokens("q", q)
    _tokens("k", k, q)
    _tokens("v", v, q)
    B, H, F, N, D = q.shape
    dev = q.device
    _f32("alpha", alpha, (B, H, F), dev)
    _f32("beta", beta, (B, H, F, N), dev)
    _f32("state", state, (B, H, D, D), dev)
    o = out if out is not None else torch.empty_like(q)
    _tokens("out", o, q)
    so = state_out if state_out is not None else torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    _f32("state_out", so, (B, H, D, D), dev)
    shp = _shape(q)
    need = lib.ls_gdn_frame_workspace_size(ctypes.byref(shp))
    w = ws if ws is not None else workspace(need, dev)
    scale = 0.0 if key_scale is None else float(key_scale)
    _check(lib.ls_gdn_frame_forward_token_gate(ctypes.byref(shp), scale, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                               _ptr(beta), _ptr(o), _ptr(state), _ptr(so), _ptr(w), w.numel(),
                                               _stream(dev)))
    return o, so


def ls_gdn_frame_forward_reversed(q, k, v, alpha, beta, chunk_frames: int, key_scale=None, out=None, ws=None):
    """Reversed frame-wise Gated DeltaNet that resets every chunk_frames frames; returns o.

    alpha, beta: [B, H, F] fp32.  Each chunk is scanned from its last frame to
    its first from a zero state.
    """
    _tokens("q", q)
    _tokens("k", k, q)
    _tokens("v", v, q)
    B, H, F, N, D = q.shape
    dev = q.device
    _f32("alpha", alpha, (B, H, F), dev)
    _f32("beta", beta, (B, H, F), dev)
    o = out if out is not None else torch.empty_like(q)
    _tokens("out", o, q)
    shp = _shape(q)
    need = lib.ls_gdn_frame_workspace_size(ctypes.byref(shp))
    w = ws if ws is not None else workspace(need, dev)
    scale = 0.0 if key_scale is None else float(key_scale)
    _check(lib.ls_gdn_frame_forward_reversed(ctypes.byref(shp), int(chunk_frames), scale, _ptr(q), _ptr(k),
                                             _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), _ptr(w), w.numel(),
                                             _stream(dev)))
    return o


def ls_temporal_conv3(x, weight, bias=None, carry=None, block_frames: int = 1, out=None, carry_out=None):
    """Block-causal temporal convolution of kernel 3 along frames; returns (y, carry_out).

    x: [B, H, F, N, D] fp32 or bf16; weight: [H, D, 3] fp32 (taps on frames
    f-1, f, f+1); bias: [H, D] fp32 or None; carry: [B, H, N, D] (x's dtype),
    the previous block's last frame, or None for zeros.  carry_out receives
    x's last frame (allocated unless given; may be `carry`).
    """
    if not isinstance(x, torch.Tensor) or x.dim() != 5 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 5-d GPU tensor [B, H, F, N, D]")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    B, H, F, N, D = x.shape
    dev = x.device
    _f32("weight", weight, (H, D, 3), dev)
    _f32("bias", bias, (H, D), dev)
    for name, t in (("carry", carry), ("carry_out", carry_out)):
        if t is not None and (t.dtype != x.dtype or tuple(t.shape) != (B, H, N, D) or t.device != dev
                              or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous %s tensor [B, H, N, D] on %s" % (name, x.dtype, dev))
    y = out if out is not None else torch.empty_like(x)
    if y.shape != x.shape or y.dtype != x.dtype or y.device != dev or not y.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    co = carry_out if carry_out is not None else torch.empty((B, H, N, D), dtype=x.dtype, device=dev)
    shp = _shape(x)
    _check(lib.ls_temporal_conv3(ctypes.byref(shp), int(block_frames), _ptr(x), _ptr(weight), _ptr(bias),
                                 _ptr(carry), _ptr(y), _ptr(co), _stream(dev)))
    return y, co


def ls_state_carry(state_src, state_dst, norm_src=None, norm_dst=None, reset: bool = False):
    """Commit a finished block's state to the carried cache (or zero the cache)."""
    B, H, D, _ = state_dst.shape
    dev = state_dst.device
    _f32("state_dst", state_dst, (B, H, D, D), dev)
    _f32("state_src", state_src, (B, H, D, D), dev)
    _f32("norm_src", norm_src, (B, H, D), dev)
    _f32("norm_dst", norm_dst, (B, H, D), dev)
    _check(lib.ls_state_carry(B, H, D, _ptr(state_src), _ptr(norm_src), _ptr(state_dst), _ptr(norm_dst),
                              int(bool(reset)), _stream(dev)))
    return state_dst


def ls_profile_begin():
    """Start timing every library kernel launch with HIP events."""
    _check(lib.ls_profile_begin())


def ls_profile_end():
    """Stop timing; returns {kernel: (launches, total_ms)} in first-launch order."""
    stats = (ls_kernel_stat * 64)()
    n = lib.ls_profile_end(stats, 64)
    if n < 0:
        raise LinscanError(LS_ERR_HIP, "profiling events failed")
    return {stats[i].name.decode(): (stats[i].launches, stats[i].total_ms) for i in range(min(n, 64))}


relu_block_forward = ls_relu_block_forward
gdn_frame_forward = ls_gdn_frame_forward
state_carry = ls_state_carry
