"""Python binding of libprism: the PRISM rank-L gated delta-rule forward on MI355X.

Argument marshalling only.  Every step of the forward (ShortConv anchor,
residual chain, chunked UT/WY delta rule, segment scan, output correction) runs
in the HIP kernels of libprism.so; PyTorch supplies device memory and the
stream.  There is no CPU path: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
# PRISM_LIB selects another build of the same library (the host-sanitized one of the ABI tests)
LIB_PATH = os.environ.get("PRISM_LIB") or os.path.join(HERE, "libprism.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "prism.h")

PRISM_F32, PRISM_BF16 = 0, 1
_lib = None


class PrismError(RuntimeError):
    pass


def load_library() -> ctypes.CDLL:
    """Load libprism.so (built by delta_rule_sequence_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise PrismError(f"{LIB_PATH} is missing: build it with `python -m delta_rule_sequence_amd.build` "
                         "(or __graft_entry__.build())")
    # torch first: the library then binds to the HIP runtime torch already loaded.  Opened
    # before torch, it would pull in a second runtime, whose launches fail with
    # hipErrorNoDevice once torch has brought up its own.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise PrismError("two HIP runtimes are loaded in this process (" + ", ".join(runtimes) + "): "
                         "libprism.so was opened before torch, so its kernels would run on a runtime that "
                         "sees no device.  Import torch (or delta_rule_sequence_amd) before opening libprism.so.")
    vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fwd_args = [vp, vp, vp, fp, fp, vp, fp, vp, fp, i, i, i, i, i, i, i, i, vp, fp, vp, sz]
    lib.prism_fwd.argtypes = fwd_args + [vp]
    lib.prism_fwd.restype = ctypes.c_int
    lib.prism_fwd_seg.argtypes = fwd_args + [i, vp]
    lib.prism_fwd_seg.restype = ctypes.c_int
    lib.prism_fwd_timed.argtypes = fwd_args + [vp, vp]
    lib.prism_fwd_timed.restype = ctypes.c_int
    lib.prism_fwd_state.argtypes = fwd_args[:17] + [fp, vp, vp, fp, vp, vp, sz, vp]
    lib.prism_fwd_state.restype = ctypes.c_int
    lib.prism_decode_step.argtypes = [vp, vp, vp, fp, fp, vp, fp, vp, fp, i, i, i, i, i, i, fp, vp, vp, vp]
    lib.prism_decode_step.restype = ctypes.c_int
    lib.prism_bwd.argtypes = fwd_args[:9] + [i] * 7 + [vp, fp] + [fp] * 9 + [vp, sz, vp]
    lib.prism_bwd.restype = ctypes.c_int
    lib.prism_bwd_workspace_bytes.argtypes = [i] * 7
    lib.prism_bwd_workspace_bytes.restype = sz
    lib.prism_bwd_lowmem.argtypes = lib.prism_bwd.argtypes
    lib.prism_bwd_seg.argtypes = fwd_args[:9] + [i] * 7 + [vp, fp] + [fp] * 9 + [i, vp, sz, vp]
    lib.prism_bwd_seg.restype = ctypes.c_int
    lib.prism_bwd_seg_workspace_bytes.argtypes = [i] * 8
    lib.prism_bwd_seg_workspace_bytes.restype = sz
    lib.prism_bwd_lowmem.restype = ctypes.c_int
    lib.prism_bwd_lowmem_workspace_bytes.argtypes = [i] * 7
    lib.prism_bwd_chunked.argtypes = lib.prism_bwd.argtypes
    lib.prism_bwd_chunked.restype = ctypes.c_int
    lib.prism_bwd_chunked_workspace_bytes.argtypes = [i] * 7
    lib.prism_bwd_chunked_workspace_bytes.restype = sz
    lib.prism_bwd_lowmem_workspace_bytes.restype = sz
    lib.prism_fwd_workspace_bytes.argtypes = [i] * 8
    lib.prism_fwd_workspace_bytes.restype = sz
    lib.prism_fwd_seg_workspace_bytes.argtypes = [i] * 9
    lib.prism_fwd_seg_workspace_bytes.restype = sz
    lib.prism_nl_gain.argtypes = [vp, fp, vp, fp, vp, i, i, i, i, i, i, vp, vp]
    lib.prism_nl_gain.restype = ctypes.c_int
    lib.prism_fwd_nl.argtypes = fwd_args + [vp]
    lib.prism_fwd_nl.restype = ctypes.c_int
    lib.prism_nl_gain_pred.argtypes = [vp, fp, vp, fp, vp, i, i, i, i, i, i, vp, vp]
    lib.prism_nl_gain_pred.restype = ctypes.c_int
    lib.prism_fwd_nl_pred.argtypes = fwd_args + [vp]
    lib.prism_fwd_nl_pred.restype = ctypes.c_int
    lib.prism_fwd_nl_workspace_bytes.argtypes = [i] * 8
    lib.prism_fwd_nl_workspace_bytes.restype = sz
    lib.prism_fwd_nl_seg.argtypes = fwd_args + [i, vp]
    lib.prism_fwd_nl_seg.restype = ctypes.c_int
    lib.prism_fwd_nl_seg_workspace_bytes.argtypes = [i] * 9
    lib.prism_fwd_nl_seg_workspace_bytes.restype = sz
    lib.prism_delta_gain.argtypes = [vp, vp, fp, vp, i, i, i, i, i, i, vp, vp]
    lib.prism_delta_gain.restype = ctypes.c_int
    lib.prism_fwd_delta.argtypes = fwd_args + [vp]
    lib.prism_fwd_delta.restype = ctypes.c_int
    lib.prism_fwd_delta_seg.argtypes = fwd_args + [i, vp]
    lib.prism_fwd_delta_seg.restype = ctypes.c_int
    lib.prism_fwd_delta_workspace_bytes.argtypes = [i] * 8
    lib.prism_fwd_delta_workspace_bytes.restype = sz
    lib.prism_fwd_delta_seg_workspace_bytes.argtypes = [i] * 9
    lib.prism_fwd_delta_seg_workspace_bytes.restype = sz
    lib.prism_anchor_predict.argtypes = [vp, fp, vp, vp, vp, vp] + [i] * 7 + [vp, vp, fp, vp]
    lib.prism_anchor_predict.restype = ctypes.c_int
    lib.prism_fwd_delta_pred.argtypes = [vp, vp, vp, fp, fp, vp, vp, vp, fp] + [i] * 8 + [vp, fp, vp, sz, vp]
    lib.prism_fwd_delta_pred.restype = ctypes.c_int
    lib.prism_fwd_delta_pred_workspace_bytes.argtypes = [i] * 8
    lib.prism_fwd_delta_pred_workspace_bytes.restype = sz
    lib.prism_fwd_noalloc.argtypes = fwd_args[:19] + [vp]
    lib.prism_fwd_noalloc.restype = ctypes.c_int
    lib.prism_noalloc_scratch_bytes.argtypes = []
    lib.prism_noalloc_scratch_bytes.restype = sz
    lib.prism_status_string.argtypes = [ctypes.c_int]
    lib.prism_status_string.restype = ctypes.c_char_p
    lib.prism_version.argtypes = []
    lib.prism_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _hip_runtimes_mapped() -> list:
    """Distinct files of the HIP runtime (libamdhip64) mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return []
    return sorted({os.path.realpath(p) for p in paths if p.startswith("/")})


def header_functions() -> list:
    """Names of the functions include/prism.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z_]+)\s*\(", text)))


def status_string(code: int) -> str:
    return load_library().prism_status_string(code).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return PRISM_BF16
    if t.dtype == torch.float32:
        return PRISM_F32
    raise PrismError(f"unsupported dtype {t.dtype}: q, k, v, u, gamma must be bfloat16 or float32")


def workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, L: int, chunk: int, dtype_code: int,
                    seg_chunks: Optional[int] = None) -> int:
    lib = load_library()
    if seg_chunks is None:
        return int(lib.prism_fwd_workspace_bytes(B, H, T, dk, dv, L, chunk, dtype_code))
    return int(lib.prism_fwd_seg_workspace_bytes(B, H, T, dk, dv, L, chunk, dtype_code, seg_chunks))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(named_vec, named_flt, shapes, dtype, dev):
    """Device, contiguity, dtype and shape checks of the tensor arguments."""
    import torch
    for name, t in named_vec + named_flt:
        if t is None:
            raise PrismError(f"{name} is required")
        if t.device != dev or not t.is_contiguous():
            raise PrismError(f"{name} must be a contiguous tensor on {dev}")
        if name in shapes and tuple(t.shape) != shapes[name]:
            raise PrismError(f"{name} has shape {tuple(t.shape)}, expected {shapes[name]}")
    for name, t in named_vec:
        if t.dtype != dtype:
            raise PrismError(f"{name} must have dtype {dtype}")
    for name, t in named_flt:
        if t.dtype != torch.float32:
            raise PrismError(f"{name} must be float32")


def _outputs(out, B, H, T, dk, dv, dtype, dev):
    """o and S_final: fresh tensors, or the caller's out=(o, S) after checking them."""
    import torch
    if out is None:
        return (torch.empty((B, H, T, dv), dtype=dtype, device=dev),
                torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev))
    if not isinstance(out, (tuple, list)) or len(out) != 2:
        raise PrismError("out must be a pair (o, S_final)")
    o, S = out
    for name, t, shape, dt in (("o", o, (B, H, T, dv), dtype), ("S_final", S, (B, H, dk, dv), torch.float32)):
        if not isinstance(t, torch.Tensor):
            raise PrismError(f"out {name} must be a tensor")
        if t.device != dev or not t.is_contiguous():
            raise PrismError(f"out {name} must be a contiguous tensor on {dev}")
        if tuple(t.shape) != shape or t.dtype != dt:
            raise PrismError(f"out {name} must have shape {shape} and dtype {dt}, "
                             f"got {tuple(t.shape)} {t.dtype}")
    return o, S


def _workspace(workspace, need: int, dev):
    """The caller's workspace after checking it, or a fresh one of `need` bytes."""
    import torch
    need = max(1, int(need))
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=dev)
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8:
        raise PrismError("workspace must be a uint8 tensor")
    if workspace.device != dev or not workspace.is_contiguous():
        raise PrismError(f"workspace must be a contiguous tensor on {dev}")
    if workspace.numel() < need:
        raise PrismError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    return workspace


def fwd_state(q, k, v, g, beta, u=None, alpha=None, gamma=None, conv_w=None, L: int = 1, chunk: int = 64,
              S0=None, conv_in=None, want_conv: bool = True, workspace=None, stream=None):
    """o, S_final, conv_out = fwd_state(..., S0, conv_in): the forward continued from a state.

    S0 [B,H,dk,dv] float32 (the S_final layout) and conv_in [B,H,3,dv] (the input dtype;
    values of the three tokens before the first) are optional (zero when None).  conv_out
    holds the values of the last three tokens of [conv_in; v] (None if want_conv is False);
    (S_final, conv_out) continue the sequence in the next call.
    """
    import torch
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    vec = [("q", q), ("k", k), ("v", v)] + ([("u", u), ("gamma", gamma)] if L > 1 else [])
    flt = [("g", g), ("beta", beta)] + ([("alpha", alpha), ("conv_w", conv_w)] if L > 1 else [])
    shapes = {"k": (B, H, T, dk), "v": (B, H, T, dv), "g": (B, H, T), "beta": (B, H, T),
              "u": (B, H, T, L - 1, dk), "gamma": (B, H, T, L - 1, dv), "alpha": (B, H, T, L),
              "conv_w": (H, 4, dv), "S0": (B, H, dk, dv), "conv_in": (B, H, 3, dv)}
    _check(vec + ([("conv_in", conv_in)] if conv_in is not None else []),
           flt + ([("S0", S0)] if S0 is not None else []), shapes, q.dtype, dev)
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    conv_out = torch.empty((B, H, 3, dv), dtype=q.dtype, device=dev) if want_conv else None
    workspace = _workspace(workspace, workspace_bytes(B, H, T, dk, dv, L, chunk, dt), dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    st = lib.prism_fwd_state(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(u) if L > 1 else None, _ptr(alpha) if L > 1 else None,
                             _ptr(gamma) if L > 1 else None, _ptr(conv_w) if L > 1 else None,
                             B, H, T, dk, dv, L, chunk, dt, _ptr(S0), _ptr(conv_in),
                             _ptr(o), _ptr(S), _ptr(conv_out),
                             ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_fwd_state failed: {status_string(st)}")
    return o, S, conv_out


def decode_step(S, conv_state, q, k, v, g, beta, u=None, alpha=None, gamma=None, conv_w=None, L: int = 1,
                stream=None):
    """o = decode_step(S, conv_state, q, k, v, g, beta, u, alpha, gamma, conv_w, L).

    One token for every (b, h) pair; S [B,H,dk,dv] float32 and conv_state [B,H,3,dv]
    (input dtype) are updated in place.  q, k [B,H,dk]; v [B,H,dv]; g, beta [B,H];
    u [B,H,L-1,dk]; alpha [B,H,L]; gamma [B,H,L-1,dv]; conv_w [H,4,dv].  Returns o [B,H,dv].
    """
    import torch
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    vec = [("q", q), ("k", k), ("v", v)] + ([("u", u), ("gamma", gamma), ("conv_state", conv_state)]
                                            if L > 1 else ([("conv_state", conv_state)] if conv_state is not None else []))
    flt = [("g", g), ("beta", beta), ("S", S)] + ([("alpha", alpha), ("conv_w", conv_w)] if L > 1 else [])
    shapes = {"k": (B, H, dk), "v": (B, H, dv), "g": (B, H), "beta": (B, H), "u": (B, H, L - 1, dk),
              "gamma": (B, H, L - 1, dv), "alpha": (B, H, L), "conv_w": (H, 4, dv), "S": (B, H, dk, dv),
              "conv_state": (B, H, 3, dv)}
    _check(vec, flt, shapes, q.dtype, dev)
    o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    st = lib.prism_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(u) if L > 1 else None, _ptr(alpha) if L > 1 else None,
                               _ptr(gamma) if L > 1 else None, _ptr(conv_w) if L > 1 else None,
                               B, H, dk, dv, L, dt, _ptr(S), _ptr(conv_state), _ptr(o), ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_decode_step failed: {status_string(st)}")
    return o


def fwd(q, k, v, g, beta, u=None, alpha=None, gamma=None, conv_w=None, L: int = 1, chunk: int = 64,
        seg_chunks: Optional[int] = None, out: Optional[Tuple] = None, workspace=None, stream=None):
    """o, S_final = fwd(q, k, v, g, beta, u, alpha, gamma, conv_w, L, chunk).

    q, k [B,H,T,dk]; v [B,H,T,dv]; u [B,H,T,L-1,dk]; gamma [B,H,T,L-1,dv] in
    bfloat16 or float32 (one dtype); g, beta [B,H,T], alpha [B,H,T,L], conv_w
    [H,4,dv] float32.  All on one GPU, contiguous.  Returns o [B,H,T,dv] (input
    dtype) and S_final [B,H,dk,dv] (float32, the transposed final state).
    """
    import torch
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    vec = [("q", q), ("k", k), ("v", v)] + ([("u", u), ("gamma", gamma)] if L > 1 else [])
    flt = [("g", g), ("beta", beta)] + ([("alpha", alpha), ("conv_w", conv_w)] if L > 1 else [])
    for name, t in vec + flt:
        if t is None:
            raise PrismError(f"{name} is required when L = {L}")
        if t.device != dev or not t.is_contiguous():
            raise PrismError(f"{name} must be a contiguous tensor on {dev}")
    for name, t in vec:
        if t.dtype != q.dtype:
            raise PrismError(f"{name} must have dtype {q.dtype}")
    for name, t in flt:
        if t.dtype != torch.float32:
            raise PrismError(f"{name} must be float32")
    shapes = {"k": (B, H, T, dk), "v": (B, H, T, dv), "g": (B, H, T), "beta": (B, H, T)}
    if L > 1:
        shapes.update({"u": (B, H, T, L - 1, dk), "gamma": (B, H, T, L - 1, dv),
                       "alpha": (B, H, T, L), "conv_w": (H, 4, dv)})
    for name, t in vec + flt:
        if name in shapes and tuple(t.shape) != shapes[name]:
            raise PrismError(f"{name} has shape {tuple(t.shape)}, expected {shapes[name]}")
    o, S = _outputs(out, B, H, T, dk, dv, q.dtype, dev)
    # a size of 0 (invalid arguments) lets the library report which argument is wrong
    workspace = _workspace(workspace, workspace_bytes(B, H, T, dk, dv, L, chunk, dt, seg_chunks), dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(u) if L > 1 else None, _ptr(alpha) if L > 1 else None,
            _ptr(gamma) if L > 1 else None, _ptr(conv_w) if L > 1 else None,
            B, H, T, dk, dv, L, chunk, dt, _ptr(o), _ptr(S),
            ctypes.c_void_p(workspace.data_ptr()), workspace.numel()]
    if seg_chunks is None:
        st = lib.prism_fwd(*args, ctypes.c_void_p(s))
    else:
        st = lib.prism_fwd_seg(*args, seg_chunks, ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_fwd failed: {status_string(st)}")
    return o, S


def bwd(q, k, v, g, beta, u=None, alpha=None, gamma=None, conv_w=None, L: int = 1, d_o=None,
        dS_final=None, workspace=None, stream=None, low_memory: bool = False, seg_len=None,
        chunked: bool = False):
    """Gradients of sum <d_o, o> + <dS_final, S_final> for fwd(q, ..., conv_w, L) (zero start).

    Inputs as fwd(); d_o [B,H,T,dv] in the input dtype; dS_final [B,H,dk,dv] float32 or None.
    low_memory: use prism_bwd_lowmem (the sequential form, states every 64 tokens only).
    seg_len: segment length of the segment-parallel form (prism_bwd_seg; a multiple of 8,
    at least 16); None: prism_bwd, which picks it.
    chunked: use prism_bwd_chunked (chunked form on MFMA; bfloat16, dk = dv = 64).
    Returns a dict of float32 tensors dq, dk, dv, dg, dbeta and, when L > 1, du, dalpha,
    dgamma, dconv_w (the shapes of the corresponding inputs; dconv_w summed over the batch).
    """
    import torch
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    if d_o is None:
        raise PrismError("d_o is required")
    vec = [("q", q), ("k", k), ("v", v), ("d_o", d_o)] + ([("u", u), ("gamma", gamma)] if L > 1 else [])
    flt = [("g", g), ("beta", beta)] + ([("alpha", alpha), ("conv_w", conv_w)] if L > 1 else []) + \
        ([("dS_final", dS_final)] if dS_final is not None else [])
    shapes = {"k": (B, H, T, dk), "v": (B, H, T, dv), "d_o": (B, H, T, dv), "g": (B, H, T), "beta": (B, H, T),
              "u": (B, H, T, L - 1, dk), "gamma": (B, H, T, L - 1, dv), "alpha": (B, H, T, L),
              "conv_w": (H, 4, dv), "dS_final": (B, H, dk, dv)}
    _check(vec, flt, shapes, q.dtype, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((B, H, T, dk), **f32), "dk": torch.empty((B, H, T, dk), **f32),
           "dv": torch.empty((B, H, T, dv), **f32), "dg": torch.empty((B, H, T), **f32),
           "dbeta": torch.empty((B, H, T), **f32)}
    if L > 1:
        out.update({"du": torch.empty((B, H, T, L - 1, dk), **f32), "dalpha": torch.empty((B, H, T, L), **f32),
                    "dgamma": torch.empty((B, H, T, L - 1, dv), **f32), "dconv_w": torch.empty((H, 4, dv), **f32)})
    if int(low_memory) + int(seg_len is not None) + int(chunked) > 1:
        raise PrismError("low_memory, seg_len and chunked select different forms")
    if chunked:
        name, need = "prism_bwd_chunked", lib.prism_bwd_chunked_workspace_bytes(B, H, T, dk, dv, L, dt)
    elif low_memory:
        name, need = "prism_bwd_lowmem", lib.prism_bwd_lowmem_workspace_bytes(B, H, T, dk, dv, L, dt)
    elif seg_len is not None:
        name, need = "prism_bwd_seg", lib.prism_bwd_seg_workspace_bytes(B, H, T, dk, dv, L, dt, seg_len)
    else:
        name, need = "prism_bwd", lib.prism_bwd_workspace_bytes(B, H, T, dk, dv, L, dt)
    if need == 0:
        raise PrismError(f"{name}: shape not supported")
    workspace = _workspace(workspace, need, dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(u) if L > 1 else None, _ptr(alpha) if L > 1 else None,
            _ptr(gamma) if L > 1 else None, _ptr(conv_w) if L > 1 else None,
            B, H, T, dk, dv, L, dt, _ptr(d_o), _ptr(dS_final),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
            _ptr(out.get("du")), _ptr(out.get("dalpha")), _ptr(out.get("dgamma")), _ptr(out.get("dconv_w"))]
    if seg_len is not None:
        args.append(seg_len)
    st = getattr(lib, name)(*args, ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"{name} failed: {status_string(st)}")
    return out


def nl_gain(v, alpha, p, conv_w, L: int, conv_in=None, stream=None):
    """gamma = nl_gain(v, alpha, p, conv_w, L, conv_in): the per-channel chain factors of the
    nonlinear refinement (GELU(p r) = gamma r along the chain), [B,H,T,L-1,dv] in the dtype of
    v.  v [B,H,T,dv]; alpha [B,H,T,L] float32; p [B,H,T,L-1,dv] (dtype of v); conv_w
    [H,4,dv] float32; conv_in [B,H,3,dv] optional.  None when L == 1."""
    import torch
    lib = load_library()
    B, H, T, dv = v.shape
    dev = v.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    if L == 1:
        return None
    shapes = {"alpha": (B, H, T, L), "p": (B, H, T, L - 1, dv), "conv_w": (H, 4, dv), "conv_in": (B, H, 3, dv)}
    _check([("v", v), ("p", p)] + ([("conv_in", conv_in)] if conv_in is not None else []),
           [("alpha", alpha), ("conv_w", conv_w)], shapes, v.dtype, dev)
    gamma = torch.empty((B, H, T, L - 1, dv), dtype=v.dtype, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    st = lib.prism_nl_gain(_ptr(v), _ptr(alpha), _ptr(p), _ptr(conv_w), _ptr(conv_in),
                           B, H, T, dv, L, _dtype_code(v), _ptr(gamma), ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_nl_gain failed: {status_string(st)}")
    return gamma


def fwd_nl(q, k, v, g, beta, u=None, alpha=None, p=None, conv_w=None, L: int = 1, chunk: int = 64,
           out: Optional[Tuple] = None, workspace=None, stream=None, seg_chunks: Optional[int] = None):
    """o, S_final = fwd_nl(q, k, v, g, beta, u, alpha, p, conv_w, L, chunk): the forward with
    the nonlinear refinement, gains p [B,H,T,L-1,dv] in place of gamma (see fwd).
    seg_chunks: an explicit segment length in chunks (prism_fwd_nl_seg)."""
    import torch
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    vec = [("q", q), ("k", k), ("v", v)] + ([("u", u), ("p", p)] if L > 1 else [])
    flt = [("g", g), ("beta", beta)] + ([("alpha", alpha), ("conv_w", conv_w)] if L > 1 else [])
    shapes = {"k": (B, H, T, dk), "v": (B, H, T, dv), "g": (B, H, T), "beta": (B, H, T),
              "u": (B, H, T, L - 1, dk), "p": (B, H, T, L - 1, dv), "alpha": (B, H, T, L),
              "conv_w": (H, 4, dv)}
    _check(vec, flt, shapes, q.dtype, dev)
    o, S = _outputs(out, B, H, T, dk, dv, q.dtype, dev)
    if seg_chunks is None:
        need = lib.prism_fwd_nl_workspace_bytes(B, H, T, dk, dv, L, chunk, dt)
    else:
        need = lib.prism_fwd_nl_seg_workspace_bytes(B, H, T, dk, dv, L, chunk, dt, seg_chunks)
    workspace = _workspace(workspace, need, dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(u) if L > 1 else None, _ptr(alpha) if L > 1 else None,
            _ptr(p) if L > 1 else None, _ptr(conv_w) if L > 1 else None,
            B, H, T, dk, dv, L, chunk, dt, _ptr(o), _ptr(S),
            ctypes.c_void_p(workspace.data_ptr()), workspace.numel()]
    if seg_chunks is None:
        st = lib.prism_fwd_nl(*args, ctypes.c_void_p(s))
    else:
        st = lib.prism_fwd_nl_seg(*args, seg_chunks, ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_fwd_nl failed: {status_string(st)}")
    return o, S


def nl_gain_pred(v, alpha, W_p, conv_w, L: int, conv_in=None, stream=None):
    """gamma = nl_gain_pred(v, alpha, W_p, conv_w, L, conv_in): the chain factors of the
    nonlinear refinement with the gains predicted from the anchor, p_l = W_p[h, l] anchor.
    v [B,H,T,dv] bfloat16; alpha [B,H,T,L] float32; W_p [H,L-1,dv,dv] bfloat16 (out, in);
    conv_w [H,4,dv] float32; conv_in [B,H,3,dv] optional.  None when L == 1."""
    import torch
    lib = load_library()
    B, H, T, dv = v.shape
    dev = v.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    if L == 1:
        return None
    shapes = {"alpha": (B, H, T, L), "W_p": (H, L - 1, dv, dv), "conv_w": (H, 4, dv), "conv_in": (B, H, 3, dv)}
    _check([("v", v), ("W_p", W_p)] + ([("conv_in", conv_in)] if conv_in is not None else []),
           [("alpha", alpha), ("conv_w", conv_w)], shapes, v.dtype, dev)
    gamma = torch.empty((B, H, T, L - 1, dv), dtype=v.dtype, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    st = lib.prism_nl_gain_pred(_ptr(v), _ptr(alpha), _ptr(W_p), _ptr(conv_w), _ptr(conv_in),
                                B, H, T, dv, L, _dtype_code(v), _ptr(gamma), ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_nl_gain_pred failed: {status_string(st)}")
    return gamma


def fwd_nl_pred(q, k, v, g, beta, u=None, alpha=None, W_p=None, conv_w=None, L: int = 1, chunk: int = 64,
                out: Optional[Tuple] = None, workspace=None, stream=None):
    """o, S_final = fwd_nl_pred(q, k, v, g, beta, u, alpha, W_p, conv_w, L, chunk): the
    nonlinear-refinement forward with gains predicted from the anchor (see nl_gain_pred)."""
    import torch
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    vec = [("q", q), ("k", k), ("v", v)] + ([("u", u), ("W_p", W_p)] if L > 1 else [])
    flt = [("g", g), ("beta", beta)] + ([("alpha", alpha), ("conv_w", conv_w)] if L > 1 else [])
    shapes = {"k": (B, H, T, dk), "v": (B, H, T, dv), "g": (B, H, T), "beta": (B, H, T),
              "u": (B, H, T, L - 1, dk), "W_p": (H, L - 1, dv, dv), "alpha": (B, H, T, L),
              "conv_w": (H, 4, dv)}
    _check(vec, flt, shapes, q.dtype, dev)
    o, S = _outputs(out, B, H, T, dk, dv, q.dtype, dev)
    workspace = _workspace(workspace, lib.prism_fwd_nl_workspace_bytes(B, H, T, dk, dv, L, chunk, dt), dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    st = lib.prism_fwd_nl_pred(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(u) if L > 1 else None, _ptr(alpha) if L > 1 else None,
                               _ptr(W_p) if L > 1 else None, _ptr(conv_w) if L > 1 else None,
                               B, H, T, dk, dv, L, chunk, dt, _ptr(o), _ptr(S),
                               ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_fwd_nl_pred failed: {status_string(st)}")
    return o, S


# ---- the written-correction form (each layer writes its GELU correction) ----------------------
def delta_gain(v, p, conv_w, L: int, conv_in=None, stream=None):
    """f = delta_gain(v, p, conv_w, L, conv_in): the per-channel factors of the written
    corrections, GELU(p r) = f r along the chain r <- r - f r; [B,H,T,L-1,dv] in the dtype of
    v.  v [B,H,T,dv]; p [B,H,T,L-1,dv] (dtype of v); conv_w [H,4,dv] float32; conv_in
    [B,H,3,dv] optional.  None when L == 1."""
    import torch
    lib = load_library()
    B, H, T, dv = v.shape
    dev = v.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    if L == 1:
        return None
    shapes = {"p": (B, H, T, L - 1, dv), "conv_w": (H, 4, dv), "conv_in": (B, H, 3, dv)}
    _check([("v", v), ("p", p)] + ([("conv_in", conv_in)] if conv_in is not None else []),
           [("conv_w", conv_w)], shapes, v.dtype, dev)
    fac = torch.empty((B, H, T, L - 1, dv), dtype=v.dtype, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    st = lib.prism_delta_gain(_ptr(v), _ptr(p), _ptr(conv_w), _ptr(conv_in), B, H, T, dv, L, _dtype_code(v),
                              _ptr(fac), ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_delta_gain failed: {status_string(st)}")
    return fac


def fwd_delta(q, k, v, g, beta, u=None, alpha=None, p=None, conv_w=None, L: int = 1, chunk: int = 64,
              out: Optional[Tuple] = None, workspace=None, stream=None, seg_chunks: Optional[int] = None):
    """o, S_final = fwd_delta(q, k, v, g, beta, u, alpha, p, conv_w, L, chunk): the forward of the
    written-correction form (layer l writes alpha_l GELU(p_{l-1} r_{l-1}) along u_l), gains p
    [B,H,T,L-1,dv] in place of gamma (see fwd).  seg_chunks: explicit segment length."""
    import torch
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    vec = [("q", q), ("k", k), ("v", v)] + ([("u", u), ("p", p)] if L > 1 else [])
    flt = [("g", g), ("beta", beta)] + ([("alpha", alpha), ("conv_w", conv_w)] if L > 1 else [])
    shapes = {"k": (B, H, T, dk), "v": (B, H, T, dv), "g": (B, H, T), "beta": (B, H, T),
              "u": (B, H, T, L - 1, dk), "p": (B, H, T, L - 1, dv), "alpha": (B, H, T, L),
              "conv_w": (H, 4, dv)}
    _check(vec, flt, shapes, q.dtype, dev)
    o, S = _outputs(out, B, H, T, dk, dv, q.dtype, dev)
    if seg_chunks is None:
        need = lib.prism_fwd_delta_workspace_bytes(B, H, T, dk, dv, L, chunk, dt)
    else:
        need = lib.prism_fwd_delta_seg_workspace_bytes(B, H, T, dk, dv, L, chunk, dt, seg_chunks)
    workspace = _workspace(workspace, need, dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(u) if L > 1 else None, _ptr(alpha) if L > 1 else None,
            _ptr(p) if L > 1 else None, _ptr(conv_w) if L > 1 else None,
            B, H, T, dk, dv, L, chunk, dt, _ptr(o), _ptr(S),
            ctypes.c_void_p(workspace.data_ptr()), workspace.numel()]
    if seg_chunks is None:
        st = lib.prism_fwd_delta(*args, ctypes.c_void_p(s))
    else:
        st = lib.prism_fwd_delta_seg(*args, seg_chunks, ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_fwd_delta failed: {status_string(st)}")
    return o, S


def anchor_predict(v, conv_w, W_p, W_k, W_b, L: int, conv_in=None, stream=None):
    """f, u, alpha = anchor_predict(v, conv_w, W_p, W_k, W_b, L, conv_in): the predictor front end
    of the written-correction form: correction factors [B,H,T,L-1,dv] and unit keys
    [B,H,T,L-1,dk] (bfloat16) and gates [B,H,T,L] (float32), from the anchor through
    W_p [H,L-1,dv,dv], W_k [H,L-1,dk,dv], W_b [H,L,dv] (bfloat16)."""
    import torch
    lib = load_library()
    B, H, T, dv = v.shape
    dk = W_k.shape[2]
    dev = v.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    shapes = {"W_p": (H, L - 1, dv, dv), "W_k": (H, L - 1, dk, dv), "W_b": (H, L, dv), "conv_w": (H, 4, dv),
              "conv_in": (B, H, 3, dv)}
    _check([("v", v), ("W_p", W_p), ("W_k", W_k), ("W_b", W_b)] +
           ([("conv_in", conv_in)] if conv_in is not None else []), [("conv_w", conv_w)], shapes, v.dtype, dev)
    fac = torch.empty((B, H, T, L - 1, dv), dtype=v.dtype, device=dev)
    uk = torch.empty((B, H, T, L - 1, dk), dtype=v.dtype, device=dev)
    al = torch.empty((B, H, T, L), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    st = lib.prism_anchor_predict(_ptr(v), _ptr(conv_w), _ptr(W_p), _ptr(W_k), _ptr(W_b), _ptr(conv_in),
                                  B, H, T, dk, dv, L, _dtype_code(v), _ptr(fac), _ptr(uk), _ptr(al),
                                  ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_anchor_predict failed: {status_string(st)}")
    return fac, uk, al


def fwd_delta_pred(q, k, v, g, beta, W_p, W_k, W_b, conv_w, L: int, chunk: int = 64,
                   out: Optional[Tuple] = None, workspace=None, stream=None):
    """o, S_final = fwd_delta_pred(q, k, v, g, beta, W_p, W_k, W_b, conv_w, L, chunk): the
    written-correction forward with gains, keys and gates predicted from the anchor."""
    import torch
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda":
        raise PrismError("inputs must be on a GPU")
    shapes = {"k": (B, H, T, dk), "v": (B, H, T, dv), "g": (B, H, T), "beta": (B, H, T),
              "W_p": (H, L - 1, dv, dv), "W_k": (H, L - 1, dk, dv), "W_b": (H, L, dv), "conv_w": (H, 4, dv)}
    _check([("q", q), ("k", k), ("v", v), ("W_p", W_p), ("W_k", W_k), ("W_b", W_b)],
           [("g", g), ("beta", beta), ("conv_w", conv_w)], shapes, q.dtype, dev)
    o, S = _outputs(out, B, H, T, dk, dv, q.dtype, dev)
    workspace = _workspace(workspace, lib.prism_fwd_delta_pred_workspace_bytes(B, H, T, dk, dv, L, chunk, dt), dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    st = lib.prism_fwd_delta_pred(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(W_p), _ptr(W_k),
                                  _ptr(W_b), _ptr(conv_w), B, H, T, dk, dv, L, chunk, dt, _ptr(o), _ptr(S),
                                  ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), ctypes.c_void_p(s))
    if st != 0:
        raise PrismError(f"prism_fwd_delta_pred failed: {status_string(st)}")
    return o, S
