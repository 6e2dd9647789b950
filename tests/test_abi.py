"""The C ABI of libprism on the host: exported symbols and argument checks.

No kernel runs here: every call below fails validation on the host, before
anything is enqueued, so these tests need no GPU.
"""
import ctypes
import os

import pytest

import delta_rule_sequence_amd as prism

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(prism.LIB_PATH):
        pytest.fail("libprism.so is not built (run __graft_entry__.build())")
    return prism.load_library()


def test_exports_every_header_symbol(lib):
    names = prism.header_functions()
    assert {"prism_fwd", "prism_fwd_workspace_bytes", "prism_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in [OK, INVALID, UNSUPPORTED, WORKSPACE, HIP]:
        s = lib.prism_status_string(code).decode()
        assert s.startswith("PRISM_")
    assert lib.prism_version().decode().count(".") == 2


def test_workspace_bytes_valid_and_invalid(lib):
    f = lib.prism_fwd_workspace_bytes
    assert f(2, 4, 16384, 64, 64, 4, 64, 1) > 0
    assert f(1, 1, 64, 16, 16, 1, 16, 0) > 0
    assert f(1, 1, 1, 16, 16, 1, 16, 0) > 0           # a single token
    assert f(0, 1, 64, 16, 16, 1, 16, 0) == 0          # B <= 0
    assert f(1, 1, 0, 16, 16, 1, 16, 0) == 0           # T <= 0
    assert f(1, 1, 64, 48, 48, 1, 16, 0) == 0          # unsupported head dim
    assert f(1, 1, 64, 64, 32, 1, 16, 0) > 0           # dk != dv (generic kernels)
    assert f(1, 1, 64, 64, 48, 1, 16, 0) == 0          # unsupported value width
    assert f(1, 1, 64, 16, 16, 1, 8, 0) == 0           # chunk not in {16, 32, 64}
    assert f(1, 1, 64, 16, 16, 9, 16, 0) == 0          # L > 8
    assert f(1, 1, 64, 16, 16, 0, 16, 0) == 0          # L < 1
    assert f(1, 1, 64, 16, 16, 1, 16, 7) == 0          # unknown dtype
    assert f(1, 1, 64, 128, 128, 2, 64, 0) == 0        # fp32 tiles exceed LDS
    assert f(1 << 20, 1 << 12, 1 << 20, 128, 128, 8, 64, 1) == 0   # size overflow


# every (dk, dv) pair of the supported widths has a kernel at some chunk size; the pairs the
# GPU parity tests run (tests/test_parity_gpu.py, UNEQUAL) all have one
@pytest.mark.parametrize("dt", [0, 1])
@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_workspace_every_width_pair(lib, dt, dk, dv):
    f = lib.prism_fwd_workspace_bytes
    assert max(f(1, 2, 300, dk, dv, 3, c, dt) for c in (16, 32, 64)) > 0
    assert f(1, 2, 300, dk, dv, 3, 16, dt) > 0


def test_workspace_unequal_parity_cases(lib):
    from tests.test_parity_gpu import UNEQUAL
    for dt, dk, dv, chunk, L in UNEQUAL:
        code = 1 if dt == "bf16" else 0
        assert lib.prism_fwd_workspace_bytes(1, 2, 4 * chunk + 7, dk, dv, L, chunk, code) > 0, (dt, dk, dv, chunk)
        assert lib.prism_fwd_seg_workspace_bytes(1, 2, 4 * chunk + 7, dk, dv, L, chunk, code, 2) > 0


def test_workspace_grows_with_segments(lib):
    f = lib.prism_fwd_seg_workspace_bytes
    assert f(1, 2, 1024, 64, 64, 4, 64, 1, 1) > f(1, 2, 1024, 64, 64, 4, 64, 1, 16) > 0
    assert f(1, 2, 1024, 64, 64, 4, 64, 1, -1) == 0


def _call(lib, B=1, H=1, T=64, d=16, L=2, chunk=16, dt=1, ptr=1, null=(), ws_bytes=1 << 30, seg=None):
    p = ctypes.c_void_p(ptr)
    args = {n: p for n in ["q", "k", "v", "g", "beta", "u", "alpha", "gamma", "conv_w", "o", "S", "ws"]}
    for n in null:
        args[n] = None
    vals = [args["q"], args["k"], args["v"], args["g"], args["beta"], args["u"], args["alpha"],
            args["gamma"], args["conv_w"], B, H, T, d, d, L, chunk, dt, args["o"], args["S"], args["ws"], ws_bytes]
    if seg is None:
        return lib.prism_fwd(*vals, None)
    return lib.prism_fwd_seg(*vals, seg, None)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "o", "S"])
def test_null_required_pointer(lib, name):
    assert _call(lib, null=(name,)) == INVALID


@pytest.mark.parametrize("name", ["u", "alpha", "gamma", "conv_w"])
def test_null_rank_pointer_when_L_gt_1(lib, name):
    assert _call(lib, L=3, null=(name,)) == INVALID


def test_bad_shapes(lib):
    assert _call(lib, B=0) == INVALID
    assert _call(lib, H=-1) == INVALID
    assert _call(lib, T=0) == INVALID
    assert _call(lib, d=24) == UNSUPPORTED
    assert _call(lib, chunk=128) == UNSUPPORTED
    assert _call(lib, L=0) == UNSUPPORTED
    assert _call(lib, L=9) == UNSUPPORTED
    assert _call(lib, dt=5) == INVALID


def test_workspace_checks(lib):
    assert _call(lib, null=("ws",)) == WORKSPACE
    need = lib.prism_fwd_workspace_bytes(1, 1, 64, 16, 16, 2, 16, 1)
    assert _call(lib, ws_bytes=need - 1) == WORKSPACE
    assert _call(lib, seg=0) == INVALID
    assert _call(lib, seg=2, ws_bytes=lib.prism_fwd_seg_workspace_bytes(1, 1, 64, 16, 16, 2, 16, 1, 2) - 1) == WORKSPACE


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(prism, "_lib", None)
    monkeypatch.setattr(prism, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(prism.PrismError):
        prism.load_library()


def _call_state(lib, B=1, H=1, T=64, d=16, L=2, chunk=16, dt=1, null=(), ws_bytes=1 << 30):
    p = ctypes.c_void_p(1)
    args = {n: p for n in ["q", "k", "v", "g", "beta", "u", "alpha", "gamma", "conv_w", "S0", "cin",
                           "o", "S", "cout", "ws"]}
    for n in null:
        args[n] = None
    return lib.prism_fwd_state(args["q"], args["k"], args["v"], args["g"], args["beta"], args["u"],
                               args["alpha"], args["gamma"], args["conv_w"], B, H, T, d, d, L, chunk, dt,
                               args["S0"], args["cin"], args["o"], args["S"], args["cout"], args["ws"],
                               ws_bytes, None)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "o", "S"])
def test_fwd_state_null_required_pointer(lib, name):
    assert _call_state(lib, null=(name,)) == INVALID


def test_fwd_state_argument_checks(lib):
    assert _call_state(lib, T=0) == INVALID
    assert _call_state(lib, d=48) == UNSUPPORTED
    assert _call_state(lib, L=9) == UNSUPPORTED
    assert _call_state(lib, L=3, null=("conv_w",)) == INVALID
    assert _call_state(lib, ws_bytes=16) == WORKSPACE


def _call_decode(lib, B=1, H=1, dk=16, dv=16, L=2, dt=1, null=()):
    p = ctypes.c_void_p(1)
    args = {n: p for n in ["q", "k", "v", "g", "beta", "u", "alpha", "gamma", "conv_w", "S", "cs", "o"]}
    for n in null:
        args[n] = None
    return lib.prism_decode_step(args["q"], args["k"], args["v"], args["g"], args["beta"], args["u"],
                                 args["alpha"], args["gamma"], args["conv_w"], B, H, dk, dv, L, dt,
                                 args["S"], args["cs"], args["o"], None)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "S", "o"])
def test_decode_null_required_pointer(lib, name):
    assert _call_decode(lib, null=(name,)) == INVALID


@pytest.mark.parametrize("name", ["u", "alpha", "gamma", "conv_w", "cs"])
def test_decode_null_rank_pointer_when_L_gt_1(lib, name):
    assert _call_decode(lib, L=3, null=(name,)) == INVALID


def test_decode_argument_checks(lib):
    assert _call_decode(lib, B=0) == INVALID
    assert _call_decode(lib, dk=32, dv=16) == UNSUPPORTED
    assert _call_decode(lib, dk=48, dv=48) == UNSUPPORTED
    assert _call_decode(lib, L=0) == UNSUPPORTED
    assert _call_decode(lib, L=9) == UNSUPPORTED
    assert _call_decode(lib, dt=7) == UNSUPPORTED


def _bwd_call(lib, B=1, H=1, T=64, d=16, L=2, dt=1, null=(), ws_bytes=1 << 30):
    p = ctypes.c_void_p(1)
    names = ["q", "k", "v", "g", "beta", "u", "alpha", "gamma", "conv_w", "d_o", "dS",
             "dq", "dk", "dv", "dg", "dbeta", "du", "dalpha", "dgamma", "dconv_w", "ws"]
    args = {n: (None if n in null else p) for n in names}
    return lib.prism_bwd(args["q"], args["k"], args["v"], args["g"], args["beta"], args["u"], args["alpha"],
                         args["gamma"], args["conv_w"], B, H, T, d, d, L, dt, args["d_o"], args["dS"],
                         args["dq"], args["dk"], args["dv"], args["dg"], args["dbeta"], args["du"],
                         args["dalpha"], args["dgamma"], args["dconv_w"], args["ws"], ws_bytes, None)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "d_o", "dq", "dk", "dv", "dg", "dbeta"])
def test_bwd_null_required_pointer(lib, name):
    assert _bwd_call(lib, null=(name,)) == INVALID


@pytest.mark.parametrize("name", ["u", "alpha", "gamma", "conv_w", "du", "dalpha", "dgamma", "dconv_w"])
def test_bwd_null_rank_pointer_when_L_gt_1(lib, name):
    assert _bwd_call(lib, L=3, null=(name,)) == INVALID


def test_bwd_argument_checks(lib):
    assert _bwd_call(lib, B=0) == INVALID
    assert _bwd_call(lib, T=-1) == INVALID
    assert _bwd_call(lib, d=48) == UNSUPPORTED
    assert _bwd_call(lib, L=9) == UNSUPPORTED
    assert _bwd_call(lib, dt=3) == INVALID
    assert _bwd_call(lib, null=("ws",)) == WORKSPACE
    need = lib.prism_bwd_workspace_bytes(1, 1, 64, 16, 16, 2, 1)
    assert need > 0
    assert _bwd_call(lib, ws_bytes=need - 1) == WORKSPACE
    assert lib.prism_bwd_workspace_bytes(1, 1, 64, 16, 32, 2, 1) == 0
    # the low-memory form keeps one state per 64 tokens: one more once T passes a multiple of 64
    low = lib.prism_bwd_lowmem_workspace_bytes(1, 1, 64, 16, 16, 2, 1)
    assert 0 < low and lib.prism_bwd_lowmem_workspace_bytes(1, 1, 65, 16, 16, 2, 1) > low
    # the segment-parallel default holds per-segment matrices: one more segment once T
    # passes a multiple of the segment length (16 tokens at this size)
    assert lib.prism_bwd_workspace_bytes(1, 1, 65, 16, 16, 2, 1) > need
    assert lib.prism_bwd_workspace_bytes(1, 1, 4096, 64, 64, 4, 1) > lib.prism_bwd_lowmem_workspace_bytes(1, 1, 4096, 64, 64, 4, 1)


def _bwd_seg_call(lib, seg_len, T=64, d=16, L=2, ws_bytes=1 << 30):
    p = ctypes.c_void_p(1)
    return lib.prism_bwd_seg(p, p, p, p, p, p, p, p, p, 1, 1, T, d, d, L, 1, p, None,
                             p, p, p, p, p, p, p, p, p, seg_len, p, ws_bytes, None)


@pytest.mark.parametrize("seg_len", [0, -8, 8, 12, 20, 33])
def test_bwd_seg_refuses_bad_segment_length(lib, seg_len):
    """Segments are a multiple of the 8-token checkpoint spacing and at least 16 tokens (so
    that the anchor terms a segment owes reach only the segment before it)."""
    assert lib.prism_bwd_seg_workspace_bytes(1, 1, 64, 16, 16, 2, 1, seg_len) == 0
    assert _bwd_seg_call(lib, seg_len) == INVALID


def test_bwd_seg_workspace(lib):
    a = lib.prism_bwd_seg_workspace_bytes(1, 1, 64, 16, 16, 2, 1, 16)
    b = lib.prism_bwd_seg_workspace_bytes(1, 1, 64, 16, 16, 2, 1, 32)
    assert a > 0 and b > 0
    # five 16 x 16 float32 matrices per segment: four segments against two
    assert a - b >= 2 * 5 * 16 * 16 * 4
    assert _bwd_seg_call(lib, 16, ws_bytes=a - 1) == WORKSPACE
    assert lib.prism_bwd_seg_workspace_bytes(1, 1, 64, 16, 32, 2, 1, 16) == 0
    assert lib.prism_bwd_seg_workspace_bytes(1, 1, 64, 48, 48, 2, 1, 16) == 0


def _nl_gain_call(lib, B=1, H=1, T=64, dv=16, L=3, dt=1, null=()):
    p = ctypes.c_void_p(1)
    args = {n: (None if n in null else p) for n in ["v", "alpha", "p", "conv_w", "gamma"]}
    return lib.prism_nl_gain(args["v"], args["alpha"], args["p"], args["conv_w"], None, B, H, T, dv, L, dt,
                             args["gamma"], None)


@pytest.mark.parametrize("name", ["v", "alpha", "p", "conv_w", "gamma"])
def test_nl_gain_null_pointer(lib, name):
    assert _nl_gain_call(lib, null=(name,)) == INVALID


def test_nl_gain_argument_checks(lib):
    assert _nl_gain_call(lib, B=0) == INVALID
    assert _nl_gain_call(lib, T=0) == INVALID
    assert _nl_gain_call(lib, dv=24) == UNSUPPORTED
    assert _nl_gain_call(lib, L=9) == UNSUPPORTED
    assert _nl_gain_call(lib, dt=2) == INVALID
    # L = 1 has no factors: nothing to check beyond the sizes, nothing enqueued
    assert _nl_gain_call(lib, L=1, null=("v", "alpha", "p", "conv_w", "gamma")) == OK


def _fwd_nl_call(lib, B=1, H=1, T=64, d=16, L=2, chunk=16, dt=1, null=(), ws_bytes=1 << 30):
    p = ctypes.c_void_p(1)
    names = ["q", "k", "v", "g", "beta", "u", "alpha", "p", "conv_w", "o", "S", "ws"]
    a = {n: (None if n in null else p) for n in names}
    return lib.prism_fwd_nl(a["q"], a["k"], a["v"], a["g"], a["beta"], a["u"], a["alpha"], a["p"], a["conv_w"],
                            B, H, T, d, d, L, chunk, dt, a["o"], a["S"], a["ws"], ws_bytes, None)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "u", "alpha", "p", "conv_w", "o", "S"])
def test_fwd_nl_null_pointer(lib, name):
    assert _fwd_nl_call(lib, L=3, null=(name,)) == INVALID


def test_fwd_nl_workspace(lib):
    f = lib.prism_fwd_nl_workspace_bytes
    base = lib.prism_fwd_workspace_bytes(1, 1, 64, 16, 16, 3, 16, 1)
    # the factors (64 tokens x 2 slots x 16 channels of bf16) in front of the forward's workspace
    assert f(1, 1, 64, 16, 16, 3, 16, 1) == 4096 + base
    assert f(1, 1, 64, 16, 16, 1, 16, 1) == lib.prism_fwd_workspace_bytes(1, 1, 64, 16, 16, 1, 16, 1)
    assert f(1, 1, 64, 16, 32, 3, 16, 1) > 0           # dk != dv: factor pass + generic forward
    assert f(1, 1, 64, 16, 48, 3, 16, 1) == 0
    g = lib.prism_fwd_nl_seg_workspace_bytes
    assert g(1, 2, 600, 64, 64, 4, 64, 1, 2) > g(1, 2, 600, 64, 64, 4, 64, 1, 10) > 0
    assert g(1, 2, 600, 64, 64, 4, 64, 1, 0) == 0
    need = f(1, 1, 64, 16, 16, 2, 16, 1)
    assert _fwd_nl_call(lib, null=("ws",)) == WORKSPACE
    assert _fwd_nl_call(lib, ws_bytes=need - 1) == WORKSPACE
    assert _fwd_nl_call(lib, d=48) == UNSUPPORTED
    assert _fwd_nl_call(lib, T=0) == INVALID


def _pred_call(lib, B=1, H=1, T=64, dv=64, L=3, dt=1, null=()):
    p = ctypes.c_void_p(1)
    a = {n: (None if n in null else p) for n in ["v", "alpha", "W", "conv_w", "gamma"]}
    return lib.prism_nl_gain_pred(a["v"], a["alpha"], a["W"], a["conv_w"], None, B, H, T, dv, L, dt,
                                  a["gamma"], None)


@pytest.mark.parametrize("name", ["v", "alpha", "W", "conv_w", "gamma"])
def test_nl_gain_pred_null_pointer(lib, name):
    assert _pred_call(lib, null=(name,)) == INVALID


def test_nl_gain_pred_argument_checks(lib):
    assert _pred_call(lib, T=0) == INVALID
    assert _pred_call(lib, dt=0) == UNSUPPORTED       # bfloat16 only (MFMA operands)
    assert _pred_call(lib, dv=16) == UNSUPPORTED      # the contraction is 32 deep
    assert _pred_call(lib, L=9) == UNSUPPORTED
    assert _pred_call(lib, dt=4) == INVALID
    assert _pred_call(lib, L=1, null=("v", "alpha", "W", "conv_w", "gamma")) == OK


def test_fwd_nl_pred_checks(lib):
    p = ctypes.c_void_p(1)

    def call(d=64, L=3, dt=1, null=(), ws=1 << 30):
        a = {n: (None if n in null else p) for n in ["q", "k", "v", "g", "beta", "u", "alpha", "W", "cw", "o", "S",
                                                     "ws"]}
        return lib.prism_fwd_nl_pred(a["q"], a["k"], a["v"], a["g"], a["beta"], a["u"], a["alpha"], a["W"], a["cw"],
                                     1, 1, 64, d, d, L, 64, dt, a["o"], a["S"], a["ws"], ws, None)
    for n in ["q", "k", "v", "g", "beta", "u", "alpha", "W", "cw", "o", "S"]:
        assert call(null=(n,)) == INVALID, n
    assert call(dt=0) == UNSUPPORTED
    assert call(null=("ws",)) == WORKSPACE
    assert call(ws=lib.prism_fwd_nl_workspace_bytes(1, 1, 64, 64, 64, 3, 64, 1) - 1) == WORKSPACE


def test_noalloc_rejects_shapes_beyond_its_array(lib):
    """prism_fwd_noalloc checks the forward's workspace against its static array on the
    host and returns PRISM_ERR_WORKSPACE before looking up the array or launching."""
    cap = lib.prism_noalloc_scratch_bytes()
    assert cap == 64 << 20
    assert lib.prism_fwd_workspace_bytes(2, 4, 16384, 64, 64, 4, 64, 1) <= cap
    assert lib.prism_fwd_workspace_bytes(1, 8, 65536, 128, 128, 8, 64, 1) > cap
    f = lib.prism_fwd_noalloc
    f.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 8 + [ctypes.c_void_p] * 3
    f.restype = ctypes.c_int
    p = ctypes.c_void_p(1)
    assert f(*[p] * 9, 1, 8, 65536, 128, 128, 8, 64, 1, p, p, None) == WORKSPACE
    assert f(*[p] * 9, 1, 8, 64, 48, 48, 8, 64, 1, p, p, None) == UNSUPPORTED
    assert f(*[p] * 9, 0, 8, 64, 64, 64, 8, 64, 1, p, p, None) == INVALID


def test_delta_form_workspace_and_checks(lib):
    f = lib.prism_fwd_delta_workspace_bytes
    assert f(1, 1, 64, 16, 16, 3, 16, 1) == lib.prism_fwd_nl_workspace_bytes(1, 1, 64, 16, 16, 3, 16, 1)
    assert f(1, 1, 64, 16, 48, 3, 16, 1) == 0
    g = lib.prism_fwd_delta_seg_workspace_bytes
    assert g(1, 2, 600, 64, 64, 4, 64, 1, 2) > g(1, 2, 600, 64, 64, 4, 64, 1, 10) > 0
    p = lib.prism_fwd_delta_pred_workspace_bytes
    assert p(2, 4, 16384, 64, 64, 4, 64, 1) > f(2, 4, 16384, 64, 64, 4, 64, 1)
    assert p(1, 1, 64, 64, 64, 1, 64, 1) == 0          # L = 1: nothing to predict
    assert p(1, 1, 64, 64, 64, 4, 64, 0) == 0          # float32: no MFMA front end
    assert p(1, 1, 64, 64, 32, 4, 64, 1) == 0          # dk != dv
    assert p(1, 1, 64, 16, 16, 4, 16, 1) == 0          # d = 16
    v = ctypes.c_void_p(1)
    fwd = lambda **kw: lib.prism_fwd_delta(*[kw.get(n, v) for n in ("q", "k", "v", "g", "beta", "u", "alpha", "p",
                                                                     "w")],
                                           1, 1, 64, 16, 16, 3, 16, 1, v, v, kw.get("ws", v), 1 << 30, None)
    assert fwd(p=None) == INVALID
    assert fwd(alpha=None) == INVALID
    assert fwd(ws=None) == WORKSPACE
    ap = lib.prism_anchor_predict
    assert ap(v, v, v, v, v, None, 1, 1, 64, 64, 64, 3, 0, v, v, v, None) == UNSUPPORTED   # float32
    assert ap(v, v, v, v, v, None, 1, 1, 64, 64, 64, 1, 1, v, v, v, None) == UNSUPPORTED   # L = 1
    assert ap(v, v, v, v, v, None, 1, 1, 64, 64, 32, 3, 1, v, v, v, None) == UNSUPPORTED   # dk != dv
    assert ap(v, v, None, v, v, None, 1, 1, 64, 64, 64, 3, 1, v, v, v, None) == INVALID
    assert ap(v, v, v, v, v, None, 0, 1, 64, 64, 64, 3, 1, v, v, v, None) == INVALID
    dg = lib.prism_delta_gain
    assert dg(v, None, v, None, 1, 1, 64, 16, 3, 1, v, None) == INVALID
    assert dg(v, v, v, None, 1, 1, 64, 24, 3, 1, v, None) == UNSUPPORTED
    assert dg(None, None, None, None, 1, 1, 64, 16, 1, 1, None, None) == OK   # L = 1: nothing to do
