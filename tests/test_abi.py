"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/linscan.h declares, and rejects bad arguments on the host before any
HIP call (fake, never-dereferenced device addresses are enough for that)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linscan.h")


@pytest.fixture(scope="module")
def lib():
    from block_causal_linear_attn_amd import build as b
    srcs = b.sources() + [HEADER]
    if not os.path.exists(b.LIB) or os.path.getmtime(b.LIB) < max(os.path.getmtime(s) for s in srcs):
        b.build()
    from block_causal_linear_attn_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ls_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ls_relu_block_forward", "ls_gdn_frame_forward", "ls_state_carry",
              "ls_relu_block_workspace_size", "ls_gdn_frame_workspace_size",
              "ls_status_string", "ls_last_error", "ls_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(lib.EXPORTS) == set(declared_functions())
    assert lib.lib.ls_version() == 200


def test_status_codes_have_their_documented_values():
    """The status enum keeps the order and values of the boundary's specification (OK .. INTERNAL = 0 .. 9);
    the aliasing check added beside them takes the next free value."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef enum \{(.*?)\} ls_status;", text, flags=re.S).group(1)
    vals = {m.group(1): int(m.group(2)) for m in re.finditer(r"(LS_\w+)\s*=\s*(\d+)", body)}
    assert vals == {"LS_OK": 0, "LS_ERR_NULL_POINTER": 1, "LS_ERR_BAD_SHAPE": 2, "LS_ERR_UNSUPPORTED_HEAD_DIM": 3,
                    "LS_ERR_BAD_DTYPE": 4, "LS_ERR_MISALIGNED": 5, "LS_ERR_WORKSPACE_TOO_SMALL": 6,
                    "LS_ERR_BAD_PARAM": 7, "LS_ERR_HIP": 8, "LS_ERR_INTERNAL": 9, "LS_ERR_ALIASING": 10}
    assert re.search(r"size_t\s+ls_relu_block_workspace_size\(const ls_shape\* shape\);", text)


def _shape(lib, B=1, H=2, F=3, N=64, D=32, dtype=1):
    return lib.ls_shape(B, H, F, N, D, dtype)


A = 1 << 32  # fake 16-byte aligned device addresses, far apart
ALIASING = 10  # LS_ERR_ALIASING
P = [ctypes.c_void_p(A * (i + 1)) for i in range(16)]


def _relu(lib, shp, eps=1e-6, bf=1, q=P[0], k=P[1], v=P[2], o=P[3], si=None, ni=None, so=P[4],
          no=P[5], ws=P[6], wsb=1 << 40):
    return lib.lib.ls_relu_block_forward(ctypes.byref(shp), bf, eps, q, k, v, o, si, ni, so, no, ws,
                                         wsb, None)


def _gdn(lib, shp, scale=0.0, q=P[0], k=P[1], v=P[2], a=P[7], b=P[8], o=P[3], si=None, so=P[4],
         ws=P[6], wsb=1 << 40):
    return lib.lib.ls_gdn_frame_forward(ctypes.byref(shp), scale, q, k, v, a, b, o, si, so, ws, wsb, None)


def test_validation_errors_relu(lib):
    assert _relu(lib, _shape(lib, D=24)) == 3
    assert _relu(lib, _shape(lib, dtype=7)) == 4
    assert _relu(lib, _shape(lib, N=-1)) == 2
    assert _relu(lib, _shape(lib), eps=0.0) == 7
    assert _relu(lib, _shape(lib), eps=float("nan")) == 7
    assert _relu(lib, _shape(lib), bf=0) == 7
    assert _relu(lib, _shape(lib), q=None) == 1
    assert _relu(lib, _shape(lib), k=ctypes.c_void_p(A + 8)) == 5
    assert _relu(lib, _shape(lib), o=P[0]) == ALIASING                      # o aliases q
    assert _relu(lib, _shape(lib), so=P[1]) == ALIASING                     # state_out inside k
    assert _relu(lib, _shape(lib), ws=None) == 1
    shp = _shape(lib)
    need = lib.lib.ls_relu_block_workspace_size(ctypes.byref(shp))
    assert need > 0
    assert _relu(lib, shp, wsb=need - 1) == 6
    assert "workspace" in lib.lib.ls_last_error().decode()
    assert lib.lib.ls_relu_block_workspace_size(ctypes.byref(_shape(lib, D=24))) == 0


def test_relu_workspace_covers_head_pairs(lib):
    """Head dim 32 in bf16 with an even head count may run heads in pairs as head dim 64 (a layout the
    size query does not see), so its workspace covers that launch too; odd head counts never pair."""
    ws = lambda **kw: lib.lib.ls_relu_block_workspace_size(ctypes.byref(_shape(lib, **kw)))
    for H, F, N in ((2, 1, 1), (4, 3, 700), (70, 10, 3600), (6, 1, 1100)):
        assert ws(H=H, F=F, N=N, D=32) >= ws(H=H // 2, F=F, N=N, D=64) > 0
    assert ws(H=3, F=3, N=700, D=32) < ws(H=4, F=3, N=700, D=32)
    assert ws(H=4, F=3, N=700, D=32, dtype=0) > 0  # fp32: generic kernels, no pairs


def test_validation_errors_gdn(lib):
    assert _gdn(lib, _shape(lib, D=100)) == 3
    assert _gdn(lib, _shape(lib), scale=float("inf")) == 7
    assert _gdn(lib, _shape(lib), a=None) == 1
    assert _gdn(lib, _shape(lib), b=ctypes.c_void_p(A * 9 + 2)) == 5
    assert _gdn(lib, _shape(lib), o=P[2]) == ALIASING
    assert _gdn(lib, _shape(lib), so=P[7]) == ALIASING                      # state_out over alpha
    shp = _shape(lib, D=128)
    need = lib.lib.ls_gdn_frame_workspace_size(ctypes.byref(shp))
    assert need > 0
    assert _gdn(lib, shp, wsb=need - 1) == 6


def _gdn_tg(lib, shp, scale=0.0, q=P[0], k=P[1], v=P[2], a=P[7], b=P[8], o=P[3], si=None, so=P[4],
            ws=P[6], wsb=1 << 40):
    return lib.lib.ls_gdn_frame_forward_token_gate(ctypes.byref(shp), scale, q, k, v, a, b, o, si, so, ws, wsb,
                                                   None)


def test_validation_errors_gdn_token_gate(lib):
    assert _gdn_tg(lib, _shape(lib, D=100)) == 3
    assert _gdn_tg(lib, _shape(lib), b=None) == 1
    assert _gdn_tg(lib, _shape(lib), b=ctypes.c_void_p(A * 9 + 2)) == 5
    # beta holds B*H*F*N gates (1536 bytes here): a state 1 KiB past its start overlaps
    # it, while the per-frame entry point (24 bytes of beta) sees no overlap there
    inside = ctypes.c_void_p(A * 9 + 1024)
    assert _gdn_tg(lib, _shape(lib), so=inside) == ALIASING
    assert _gdn(lib, _shape(lib), so=inside, wsb=1) == 6
    shp = _shape(lib, D=112)
    need = lib.lib.ls_gdn_frame_workspace_size(ctypes.byref(shp))
    assert _gdn_tg(lib, shp, wsb=need - 1) == 6


def test_validation_errors_gdn_reversed(lib):
    r = lambda shp, C, **kw: lib.lib.ls_gdn_frame_forward_reversed(
        ctypes.byref(shp), C, 0.0, kw.get("q", P[0]), P[1], P[2], P[7], P[8], kw.get("o", P[3]), P[6],
        kw.get("wsb", 1 << 40), None)
    assert r(_shape(lib), 0) == 7
    assert r(_shape(lib, D=100), 2) == 3
    assert r(_shape(lib), 2, q=None) == 1
    assert r(_shape(lib), 2, o=P[1]) == ALIASING
    shp = _shape(lib, D=128)
    need = lib.lib.ls_gdn_frame_workspace_size(ctypes.byref(shp))
    assert r(shp, 2, wsb=need - 1) == 6


def test_validation_errors_temporal_conv(lib):
    def cv(shp, bf=1, x=P[0], w=P[1], b=None, ci=None, y=P[2], co=None):
        return lib.lib.ls_temporal_conv3(ctypes.byref(shp), bf, x, w, b, ci, y, co, None)
    assert cv(_shape(lib, D=12)) == 2                  # bf16 channels not a multiple of 8
    assert cv(_shape(lib, D=6, dtype=0)) == 2          # fp32 channels not a multiple of 4
    assert cv(_shape(lib, dtype=5)) == 4
    assert cv(_shape(lib), bf=0) == 7
    assert cv(_shape(lib), w=None) == 1
    assert cv(_shape(lib), x=ctypes.c_void_p(A + 8)) == 5
    assert cv(_shape(lib), y=P[0]) == ALIASING                # y over x
    assert cv(_shape(lib), co=P[0]) == ALIASING               # carry_out over x
    assert cv(_shape(lib, B=0)) == 0                   # nothing to do


def test_validation_errors_strided(lib):
    shp = _shape(lib, B=1, H=4, F=3, N=10, D=32)
    def rs(st, wsb=1):
        return lib.lib.ls_relu_block_forward_strided(ctypes.byref(shp), ctypes.byref(st), 1, 1e-6, P[0], P[1], P[2],
                                                     P[3], None, None, P[4], P[5], P[6], wsb, None)
    def gs(st, wsb=1):
        return lib.lib.ls_gdn_frame_forward_strided(ctypes.byref(shp), ctypes.byref(st), 0.0, P[0], P[1], P[2],
                                                    P[7], P[8], P[3], None, P[4], P[6], wsb, None)
    S = lib.ls_strides
    bshd = S(3 * 10 * 4 * 32, 32, 10 * 4 * 32, 4 * 32)          # [B][F][N][H][D]
    assert rs(bshd) == 6 and gs(bshd) == 6                        # valid: fails only on the workspace
    assert rs(S(3 * 10 * 4 * 32, 32, 10 * 4 * 32, 3 * 32)) == 7   # token stride too small for 4 heads
    assert gs(S(3 * 10 * 4 * 32, 16, 10 * 4 * 32, 4 * 32)) == 7   # head rows of 32 at stride 16 overlap
    assert rs(S(3 * 10 * 4 * 32, 36, 10 * 4 * 36, 4 * 36)) == 5   # 72-byte strides: rows not 16-byte aligned
    assert rs(S(-1, 32, 10 * 4 * 32, 4 * 32)) == 7


def test_validation_errors_prologue(lib):
    shp = _shape(lib, B=1, H=2, F=3, N=10, D=32)
    Pr = lib.ls_prologue
    def rp(pr):
        return lib.lib.ls_relu_block_forward_prologue(ctypes.byref(shp), ctypes.byref(pr), 1, 1e-6, P[0], P[1], P[2],
                                                      P[3], None, None, P[4], P[5], P[6], 1, None)
    def gp(pr):
        return lib.lib.ls_gdn_frame_forward_prologue(ctypes.byref(shp), ctypes.byref(pr), 0.0, P[0], P[1], P[2],
                                                     P[7], P[8], P[3], None, P[4], P[6], 1, None)
    w = P[10].value
    assert rp(Pr(w, w, 1e-6, 0, 0)) == 6 and gp(Pr(w, w, 1e-6, 1, 1)) == 6   # valid: workspace too small
    assert rp(Pr(w, None, 1e-6, 1, 0)) == 7                                  # no ReLU flag on the ReLU scan
    assert rp(Pr(None, None, 1e-6, 0, 1)) == 7
    assert gp(Pr(w, None, 0.0, 0, 0)) == 7                                   # eps must be > 0 with weights
    assert gp(Pr(None, None, 0.0, 2, 0)) == 7
    assert gp(Pr(w + 4, None, 1e-6, 0, 0)) == 5                              # misaligned weights
    assert gp(Pr(P[3].value, None, 1e-6, 0, 0)) == ALIASING                         # weights inside o
    # the rotary embedding: D/2 = 16 pairs, F = 3, N = 10
    rf, rt = P[11].value, P[12].value
    def rope(f=rf, t=rt, pf=8, off=0, T=3):
        return Pr(None, None, 1e-6, 0, 0, f, t, pf, off, T)
    assert gp(rope()) == 6 and gp(rope(f=None, pf=0)) == 6 and gp(rope(t=None, pf=16)) == 6
    assert gp(rope(off=2, T=5)) == 6
    assert rp(rope()) == 6                                                   # the ReLU scan takes it too
    assert gp(rope(pf=6)) == 7                                               # not a multiple of 4
    assert gp(rope(pf=20)) == 7                                              # more than D/2 pairs
    assert gp(rope(f=None)) == 1                                             # frame pairs need the frame table
    assert gp(rope(t=None)) == 1                                             # token pairs need the token table
    assert gp(rope(off=1, T=3)) == 7                                         # rows 1..3 of a 3-row table
    assert gp(rope(off=-1)) == 7
    assert gp(rope(t=rt + 8)) == 5                                           # misaligned table
    assert gp(rope(t=P[3].value)) == ALIASING                                       # table inside o


def test_in_place_state_is_not_an_aliasing_error(lib):
    """state_out == state_in is allowed; the call then fails only on the workspace check."""
    shp = _shape(lib)
    assert _relu(lib, shp, si=P[9], ni=P[10], so=P[9], no=P[10], wsb=1) == 6
    assert _gdn(lib, shp, si=P[9], so=P[9], wsb=1) == 6


def test_carry_validation(lib):
    c = lib.lib.ls_state_carry
    assert c(1, 1, 24, P[0], None, P[1], None, 0, None) == 3
    assert c(1, 1, 32, None, None, P[1], None, 0, None) == 1
    assert c(1, 1, 32, P[0], None, None, None, 0, None) == 1
    assert c(1, 1, 32, ctypes.c_void_p(A + 4), None, P[1], None, 0, None) == 5
    assert c(1, 1, 32, ctypes.c_void_p(A), None, ctypes.c_void_p(A + 16), None, 0, None) == ALIASING
    assert c(0, 1, 32, None, None, None, None, 0, None) == 0           # nothing to do


def test_empty_shapes_plan_on_the_host(lib):
    """Frames without tokens, calls without frames and empty batches are planned on the host and, when no
    output state is asked for, return without any HIP call (fake device addresses are never touched).  The
    F = 0 path once divided by zero on the host."""
    for D in (16, 32, 64, 112, 128):
        for dt in (0, 1):
            for B, H, F, N in ((1, 2, 0, 64), (1, 2, 3, 0), (1, 2, 0, 0), (0, 3, 4, 64), (2, 0, 4, 64)):
                shp = _shape(lib, B=B, H=H, F=F, N=N, D=D, dtype=dt)
                assert lib.lib.ls_relu_block_workspace_size(ctypes.byref(shp)) > 0
                assert lib.lib.ls_gdn_frame_workspace_size(ctypes.byref(shp)) > 0
                if F == 0 or B * H == 0:
                    assert _gdn(lib, shp, si=P[9], so=None, wsb=0, ws=None) == 0
                    assert lib.lib.ls_gdn_frame_forward_reversed(ctypes.byref(shp), 2, 0.0, P[0], P[1], P[2], P[7],
                                                                 P[8], P[3], None, 0, None) == 0
                if F * N == 0 or B * H == 0:
                    # no tokens: the state would pass through; with no output state nothing is enqueued
                    assert _relu(lib, shp, si=P[9], ni=P[10], so=None, no=None, wsb=0, ws=None) == 0
                    st = lib.ls_strides(0, 0, 0, 0)
                    assert lib.lib.ls_relu_block_forward_strided(ctypes.byref(shp), ctypes.byref(st), 1, 1e-6, P[0],
                                                                 P[1], P[2], P[3], None, None, None, None, None, 0,
                                                                 None) == 0
            # the checks still run first: a bad eps or block size is rejected even without tokens
            shp = _shape(lib, F=0, D=D, dtype=dt)
            assert _relu(lib, shp, eps=0.0, so=None, no=None) == 7
            assert _relu(lib, shp, bf=0, so=None, no=None) == 7
    cv = lambda shp: lib.lib.ls_temporal_conv3(ctypes.byref(shp), 1, P[0], P[1], None, None, P[2], None, None)
    assert cv(_shape(lib, F=0)) == 0 and cv(_shape(lib, N=0)) == 0


def test_noalloc_checks_its_scratch_size_on_the_host(lib):
    """The allocation-free GDN entry point rejects a call whose workspace would not fit its static scratch,
    and a bad shape, before any HIP call."""
    f = lambda shp: lib.lib.ls_gdn_frame_forward_noalloc(ctypes.byref(shp), 0.0, P[0], P[1], P[2], P[7], P[8], P[3],
                                                         None, P[4], None, None)
    big = _shape(lib, B=1, H=24, F=20, N=64, D=128)
    assert lib.lib.ls_gdn_frame_workspace_size(ctypes.byref(big)) > lib.NOALLOC_SCRATCH_BYTES
    assert f(big) == 6 and "scratch" in lib.lib.ls_last_error().decode()
    assert f(_shape(lib, D=24)) == 3
    assert lib.lib.ls_gdn_frame_forward_noalloc(ctypes.byref(_shape(lib)), 0.0, P[0], P[1], P[2], P[7], P[8], P[3],
                                                None, P[4], ctypes.c_void_p(A + 2), None) == 5
    # the chunk step (B4 H24 D128 N920, one frame) fits
    step = _shape(lib, B=4, H=24, F=1, N=920, D=128)
    assert lib.lib.ls_gdn_frame_workspace_size(ctypes.byref(step)) <= lib.NOALLOC_SCRATCH_BYTES


def test_status_strings(lib):
    for st in range(11):
        assert lib.lib.ls_status_string(st).decode()
