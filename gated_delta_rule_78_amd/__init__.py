"""MI355X (gfx950) KDA / CKDA gated delta rule: thin Python binding of ``libkda.so``.

The arithmetic runs in the HIP library (``csrc/``); this module only checks
tensors, passes raw device pointers and the current HIP stream through the C
ABI declared in ``include/kda.h``, and raises on a non-zero status.  PyTorch
supplies device memory and streams.  There is no CPU fallback: without the
built library every call raises.

    o, S_T = chunk_fwd(q, k, v, alpha, beta, initial_state=None)   # prefill
    o      = decode_step(q, k, v, alpha, beta, state)               # state in place
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["chunk_fwd", "chunk_records", "chunk_apply_records", "chunk_fwd_debug", "decode_step",
           "gdn2_chunk_fwd", "gdn2_decode_step", "decode_tokens", "gdn2_decode_tokens", "chunk_fwd_varlen",
           "sfda_chunk_fwd", "sfda_decode_step", "sfda_decode_tokens", "chunk_bwd", "chunk_bwd_varlen",
           "gdn2_chunk_bwd", "bwd_workspace_size",
           "workspace_size", "pick_path", "chunk_fwd_noalloc", "lib", "version", "status_string",
           "LIB_PATH", "KdaError", "Shape", "BF16", "F32"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
BF16, F32 = 0, 1
_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int),
                ("dv", ctypes.c_int), ("chunk", ctypes.c_int), ("dtype", ctypes.c_int)]


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_78_amd.build` "
                               "(there is no CPU fallback)")
        # torch first: it carries its own HIP runtime, and libkda.so must bind to that
        # one.  Loaded before torch, the library would pull in the system runtime and
        # torch's the second one, and a launch on a torch stream then fails in the
        # library's runtime.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        SP = ctypes.POINTER(Shape)
        L.kda_chunk_fwd.argtypes = [SP, P, P, P, P, P, P, P, P, P]
        L.kda_chunk_fwd.restype = ctypes.c_int
        L.kda_chunk_fwd_debug.argtypes = [SP, P, P, P, P, P, P, P, P, P, P]
        L.kda_chunk_fwd_debug.restype = ctypes.c_int
        L.kda_chunk_fwd_ws.argtypes = [SP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kda_chunk_fwd_ws.restype = ctypes.c_int
        L.kda_chunk_fwd_noalloc.argtypes = [SP, P, P, P, P, P, P, P, P, P]
        L.kda_chunk_fwd_noalloc.restype = ctypes.c_int
        L.kda_chunk_fwd_workspace_size.argtypes = [SP]
        L.kda_chunk_fwd_workspace_size.restype = ctypes.c_size_t
        L.kda_chunk_records.argtypes = [SP, P, P, P, P, P, ctypes.c_size_t, P]
        L.kda_chunk_records.restype = ctypes.c_int
        L.kda_chunk_apply_records.argtypes = [SP, P, P, P, P, ctypes.c_size_t, P, P, P, P, P]
        L.kda_chunk_apply_records.restype = ctypes.c_int
        L.kda_decode_step.argtypes = [SP, P, P, P, P, P, P, P, P]
        L.kda_decode_step.restype = ctypes.c_int
        L.kda_gdn2_chunk_fwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kda_gdn2_chunk_fwd.restype = ctypes.c_int
        L.kda_gdn2_decode_step.argtypes = [SP, P, P, P, P, P, P, P, P, P]
        L.kda_gdn2_decode_step.restype = ctypes.c_int
        L.kda_chunk_fwd_varlen_workspace_size.argtypes = [SP, ctypes.c_int]
        L.kda_chunk_fwd_varlen_workspace_size.restype = ctypes.c_size_t
        L.kda_chunk_fwd_varlen.argtypes = [SP, P, ctypes.c_int, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kda_chunk_fwd_varlen.restype = ctypes.c_int
        L.kda_gdn2_chunk_fwd_varlen.argtypes = [SP, P, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t,
                                                P]
        L.kda_gdn2_chunk_fwd_varlen.restype = ctypes.c_int
        L.kda_decode_tokens.argtypes = [SP, P, P, P, P, P, P, P, P]
        L.kda_decode_tokens.restype = ctypes.c_int
        L.kda_gdn2_decode_tokens.argtypes = [SP, P, P, P, P, P, P, P, P, P]
        L.kda_gdn2_decode_tokens.restype = ctypes.c_int
        L.kda_sfda_chunk_fwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kda_sfda_chunk_fwd.restype = ctypes.c_int
        L.kda_sfda_chunk_fwd_varlen.argtypes = [SP, P, ctypes.c_int, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kda_sfda_chunk_fwd_varlen.restype = ctypes.c_int
        L.kda_sfda_decode_step.argtypes = [SP, P, P, P, P, P, P, P, P]
        L.kda_sfda_decode_step.restype = ctypes.c_int
        L.kda_sfda_decode_tokens.argtypes = [SP, P, P, P, P, P, P, P, P]
        L.kda_sfda_decode_tokens.restype = ctypes.c_int
        L.kda_chunk_bwd_workspace_size.argtypes = [SP]
        L.kda_chunk_bwd_workspace_size.restype = ctypes.c_size_t
        L.kda_chunk_bwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kda_chunk_bwd.restype = ctypes.c_int
        L.kda_chunk_bwd_varlen_workspace_size.argtypes = [SP, ctypes.c_int]
        L.kda_chunk_bwd_varlen_workspace_size.restype = ctypes.c_size_t
        L.kda_chunk_bwd_varlen.argtypes = [SP, P, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                           ctypes.c_size_t, P]
        L.kda_chunk_bwd_varlen.restype = ctypes.c_int
        L.kda_gdn2_chunk_bwd.argtypes = [SP] + [P] * 17 + [ctypes.c_size_t, P]
        L.kda_gdn2_chunk_bwd.restype = ctypes.c_int
        L.kda_gdn2_chunk_bwd_varlen.argtypes = [SP, P, ctypes.c_int] + [P] * 17 + [ctypes.c_size_t, P]
        L.kda_gdn2_chunk_bwd_varlen.restype = ctypes.c_int
        L.kda_sfda_chunk_bwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kda_sfda_chunk_bwd.restype = ctypes.c_int
        L.kda_sfda_chunk_bwd_varlen.argtypes = [SP, P, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                                ctypes.c_size_t, P]
        L.kda_sfda_chunk_bwd_varlen.restype = ctypes.c_int
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_version.argtypes = []
        L.kda_version.restype = ctypes.c_int
        _lib = L
    return _lib


def version() -> int:
    return lib().kda_version()


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"q/k/v/alpha/beta must be bfloat16 or float32, got {t.dtype}")


def _check(ts, names, dev):
    for t, nm in zip(ts, names):
        if t is None:
            continue
        if not t.is_cuda or t.device != dev:
            raise ValueError(f"{nm} must be on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def workspace_size(B, T, H, dk, dv, dtype="bf16") -> int:
    """Bytes of device workspace the two-pass chunk forward needs for this shape."""
    shape = Shape(B, T, H, dk, dv, 64, BF16 if dtype == "bf16" else F32)
    return int(lib().kda_chunk_fwd_workspace_size(ctypes.byref(shape)))


def pick_path(B, T, H, dk, dv):
    """The faster chunk-forward path for a shape on MI355X (measured): the two-pass path
    (parallel records, then the state walk) whenever there is more than one chunk -- about
    1.9x the fused single pass from B*H = 128 to 2048 heads at d = 128 -- and the fused
    kernel for a single chunk, where there is nothing to split."""
    return "twopass" if T > 64 else "fused"


def _chunk_call(debug, q, k, v, alpha, beta, initial_state, out, final_state, want_final, path="fused",
                workspace=None):
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    for t, nm in ((k, "k"), (alpha, "alpha"), (v, "v"), (beta, "beta")):
        if t.dtype != q.dtype:
            raise TypeError(f"{nm} must have the dtype of q")
    if k.shape != q.shape or alpha.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("shapes: q, k, alpha [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]")
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if final_state is None and want_final:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, H, dk, dv)):
            raise ValueError(f"{nm} must be float32 [B,H,dk,dv]")
    _check((q, k, v, alpha, beta, initial_state, out, final_state),
           ("q", "k", "v", "alpha", "beta", "initial_state", "out", "final_state"), dev)
    shape = Shape(B, T, H, dk, dv, 64, code)
    args = [ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state),
            _ptr(out), _ptr(final_state)]
    dbg = None
    if path == "auto":
        path = pick_path(B, T, H, dk, dv)
    if path == "twopass" and not debug:
        need = int(lib().kda_chunk_fwd_workspace_size(ctypes.byref(shape)))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace needs {need} bytes")
        _check((workspace,), ("workspace",), dev)
        rc = lib().kda_chunk_fwd_ws(*args, _ptr(workspace), ctypes.c_size_t(need), _stream(dev))
        if rc != 0:
            raise KdaError(rc, "kda_chunk_fwd_ws")
        return out, final_state, None
    if path not in ("fused", "twopass", "capi"):
        raise ValueError(f"unknown path {path!r}")
    if debug:
        nch = (T + 63) // 64
        dbg = torch.zeros((B * H, nch, 4, 64, 64), dtype=torch.float32, device=dev)
        rc = lib().kda_chunk_fwd_debug(*args, _ptr(dbg), _stream(dev))
    elif path == "capi":  # kda_chunk_fwd: the library picks the path and its workspace
        rc = lib().kda_chunk_fwd(*args, _stream(dev))
    else:  # the single-pass kernel (kda_chunk_fwd_ws without a workspace)
        rc = lib().kda_chunk_fwd_ws(*args, None, ctypes.c_size_t(0), _stream(dev))
    if rc != 0:
        raise KdaError(rc, "kda_chunk_fwd")
    return out, final_state, dbg


def chunk_fwd(q, k, v, alpha, beta, initial_state=None, out=None, final_state=None, want_final=True,
              path="auto", workspace=None):
    """Chunkwise WY forward.  q, k, alpha [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]
    (all bf16 or all fp32, contiguous, on one GPU); initial_state fp32 [B,H,dk,dv]
    or None.  path: "fused" (single pass), "twopass" (parallel per-chunk records in a
    workspace, then the state pass), "capi" (kda_chunk_fwd's own choice, with its
    workspace from the stream-ordered pool) or "auto".  workspace: optional uint8 device
    tensor of at least workspace_size(...) bytes for the two-pass path (allocated
    here when omitted).  Returns (o [B,T,H,dv], final_state fp32 [B,H,dk,dv] or None)."""
    o, s, _ = _chunk_call(False, q, k, v, alpha, beta, initial_state, out, final_state, want_final, path,
                          workspace)
    return o, s


def chunk_fwd_noalloc(q, k, v, alpha, beta, out, initial_state=None, final_state=None):
    """The two-pass chunk forward on the library's fixed per-GPU scratch (no device memory
    is allocated here or in the library): for callers that cannot allocate.  Layouts as
    chunk_fwd; `out` [B,T,H,dv] is required, `final_state` fp32 [B,H,dk,dv] is written
    when given.  Raises KdaError (KDA_ERR_SCRATCH) when the shape's workspace exceeds
    KDA_NOALLOC_SCRATCH_BYTES.  Calls that overlap in time on one GPU race on the scratch.
    Returns (out, final_state)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    for t, nm in ((k, "k"), (alpha, "alpha"), (v, "v"), (beta, "beta"), (out, "out")):
        if t.dtype != q.dtype:
            raise TypeError(f"{nm} must have the dtype of q")
    if k.shape != q.shape or alpha.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H) \
            or out.shape != (B, T, H, dv):
        raise ValueError("shapes: q, k, alpha [B,T,H,dk]; v, out [B,T,H,dv]; beta [B,T,H]")
    dev = q.device
    _check((q, k, v, alpha, beta, initial_state, out, final_state),
           ("q", "k", "v", "alpha", "beta", "initial_state", "out", "final_state"), dev)
    shape = Shape(B, T, H, dk, dv, 64, code)
    rc = lib().kda_chunk_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(initial_state), _ptr(out), _ptr(final_state), _stream(dev))
    if rc != 0:
        raise KdaError(rc, "kda_chunk_fwd_noalloc")
    return out, final_state


def chunk_records(q, k, alpha, beta, workspace=None, dv=None):
    """First pass of the two-pass forward alone: the per-chunk records of q, k, alpha,
    beta (layouts as chunk_fwd) into `workspace` (uint8 device tensor of at least
    workspace_size(...) bytes; allocated when None).  Returns the workspace."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = dk if dv is None else dv
    code = _dtype_code(q)
    for t, nm in ((k, "k"), (alpha, "alpha"), (beta, "beta")):
        if t.dtype != q.dtype:
            raise TypeError(f"{nm} must have the dtype of q")
    if k.shape != q.shape or alpha.shape != q.shape or beta.shape != (B, T, H):
        raise ValueError("shapes: q, k, alpha [B,T,H,dk]; beta [B,T,H]")
    dev = q.device
    shape = Shape(B, T, H, dk, dv, 64, code)
    need = int(lib().kda_chunk_fwd_workspace_size(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check((q, k, alpha, beta, workspace), ("q", "k", "alpha", "beta", "workspace"), dev)
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kda_chunk_records(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(alpha), _ptr(beta), _ptr(workspace),
                                 ctypes.c_size_t(nbytes), _stream(dev))
    if rc != 0:
        raise KdaError(rc, "kda_chunk_records")
    return workspace


def chunk_apply_records(workspace, q, k, alpha, v, initial_state=None, out=None, final_state=None, want_final=True):
    """Second pass alone: applies the records in `workspace` (made from q, k, alpha and
    beta by chunk_records) to v [B,T,H,dv] and the start state; q, k, alpha are the
    tensors the records were made from.  Returns (o [B,T,H,dv], final_state or None)."""
    torch = _torch()
    B, T, H, dv = v.shape
    dk = q.shape[-1]
    code = _dtype_code(v)
    for t, nm in ((q, "q"), (k, "k"), (alpha, "alpha")):
        if t.dtype != v.dtype:
            raise TypeError(f"{nm} must have the dtype of v")
        if t.shape != (B, T, H, dk):
            raise ValueError("shapes: q, k, alpha [B,T,H,dk]; v [B,T,H,dv]")
    dev = v.device
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=v.dtype, device=dev)
    if final_state is None and want_final:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, H, dk, dv)):
            raise ValueError(f"{nm} must be float32 [B,H,dk,dv]")
    _check((workspace, q, k, alpha, v, initial_state, out, final_state),
           ("workspace", "q", "k", "alpha", "v", "initial_state", "out", "final_state"), dev)
    shape = Shape(B, T, H, dk, dv, 64, code)
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kda_chunk_apply_records(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(alpha), _ptr(workspace),
                                       ctypes.c_size_t(nbytes), _ptr(v), _ptr(initial_state), _ptr(out),
                                       _ptr(final_state), _stream(dev))
    if rc != 0:
        raise KdaError(rc, "kda_chunk_apply_records")
    return out, final_state


def chunk_fwd_debug(q, k, v, alpha, beta, initial_state=None):
    """As chunk_fwd, also returning per-chunk intermediates [B*H, n_chunks, 4, 64, 64]
    (T, A, (I+T)^-1, W[:, :64]) for diagnosing parity failures."""
    return _chunk_call(True, q, k, v, alpha, beta, initial_state, None, None, True)


def decode_step(q, k, v, alpha, beta, state, out=None, _entry="kda_decode_step"):
    """One recurrent token for every (b, h).  q, k, alpha [B,H,dk]; v [B,H,dv];
    beta [B,H]; state fp32 [B,H,dk,dv] updated in place.  Returns o [B,H,dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    if k.shape != q.shape or alpha.shape != q.shape or v.shape != (B, H, dv) or beta.shape != (B, H):
        raise ValueError("shapes: q, k, alpha [B,H,dk]; v [B,H,dv]; beta [B,H]")
    if state.dtype != torch.float32 or state.shape != (B, H, dk, dv):
        raise ValueError("state must be float32 [B,H,dk,dv]")
    dev = q.device
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    _check((q, k, v, alpha, beta, state, out), ("q", "k", "v", "alpha", "beta", "state", "out"), dev)
    shape = Shape(B, 1, H, dk, dv, 0, code)
    rc = getattr(lib(), _entry)(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                _ptr(state), _ptr(out), _stream(dev))
    if rc != 0:
        raise KdaError(rc, _entry)
    return out


def gdn2_chunk_fwd(q, k, v, alpha, erase, write, initial_state=None, out=None, final_state=None, want_final=True,
                   workspace=None):
    """Gated DeltaNet-2 chunk forward: as chunk_fwd with beta replaced by the erase gate
    [B,T,H,dk] and the write gate [B,T,H,dv] (two-pass path; the workspace is allocated
    here when omitted).  Returns (o, final_state or None)."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    for t, nm in ((k, "k"), (alpha, "alpha"), (v, "v"), (erase, "erase"), (write, "write")):
        if t.dtype != q.dtype:
            raise TypeError(f"{nm} must have the dtype of q")
    if k.shape != q.shape or alpha.shape != q.shape or erase.shape != q.shape or v.shape != (B, T, H, dv) \
            or write.shape != v.shape:
        raise ValueError("shapes: q, k, alpha, erase [B,T,H,dk]; v, write [B,T,H,dv]")
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if final_state is None and want_final:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, H, dk, dv)):
            raise ValueError(f"{nm} must be float32 [B,H,dk,dv]")
    shape = Shape(B, T, H, dk, dv, 64, code)
    need = int(lib().kda_chunk_fwd_workspace_size(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check((q, k, v, alpha, erase, write, initial_state, out, final_state, workspace),
           ("q", "k", "v", "alpha", "erase", "write", "initial_state", "out", "final_state", "workspace"), dev)
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kda_gdn2_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase),
                                  _ptr(write), _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(workspace),
                                  ctypes.c_size_t(nbytes), _stream(dev))
    if rc != 0:
        raise KdaError(rc, "kda_gdn2_chunk_fwd")
    return out, final_state


def gdn2_decode_step(q, k, v, alpha, erase, write, state, out=None):
    """One Gated DeltaNet-2 token for every (b, h): q, k, alpha, erase [B,H,dk]; v, write
    [B,H,dv]; state fp32 [B,H,dk,dv] updated in place.  Returns o [B,H,dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    if k.shape != q.shape or alpha.shape != q.shape or erase.shape != q.shape or v.shape != (B, H, dv) \
            or write.shape != v.shape:
        raise ValueError("shapes: q, k, alpha, erase [B,H,dk]; v, write [B,H,dv]")
    if state.dtype != torch.float32 or state.shape != (B, H, dk, dv):
        raise ValueError("state must be float32 [B,H,dk,dv]")
    dev = q.device
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    _check((q, k, v, alpha, erase, write, state, out), ("q", "k", "v", "alpha", "erase", "write", "state", "out"),
           dev)
    shape = Shape(B, 1, H, dk, dv, 0, code)
    rc = lib().kda_gdn2_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase),
                                    _ptr(write), _ptr(state), _ptr(out), _stream(dev))
    if rc != 0:
        raise KdaError(rc, "kda_gdn2_decode_step")
    return out


def decode_tokens(q, k, v, alpha, beta, state, out=None, erase=None, write=None, _entry="kda_decode_tokens"):
    """Several tokens per (b, h) with the state read and written once: q, k, alpha
    [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H] (or, for Gated DeltaNet-2, beta=None with
    erase [B,T,H,dk] and write [B,T,H,dv]); state fp32 [B,H,dk,dv] in place.
    Returns o [B,T,H,dv]."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    g2 = erase is not None or write is not None
    if k.shape != q.shape or alpha.shape != q.shape or v.shape != (B, T, H, dv):
        raise ValueError("shapes: q, k, alpha [B,T,H,dk]; v [B,T,H,dv]")
    if g2 and (erase is None or write is None or erase.shape != q.shape or write.shape != v.shape):
        raise ValueError("Gated DeltaNet-2: erase [B,T,H,dk] and write [B,T,H,dv]")
    if not g2 and (beta is None or beta.shape != (B, T, H)):
        raise ValueError("beta [B,T,H]")
    if state.dtype != torch.float32 or state.shape != (B, H, dk, dv):
        raise ValueError("state must be float32 [B,H,dk,dv]")
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _check((q, k, v, alpha, beta, erase, write, state, out),
           ("q", "k", "v", "alpha", "beta", "erase", "write", "state", "out"), dev)
    shape = Shape(B, T, H, dk, dv, 0, code)
    if g2:
        rc = lib().kda_gdn2_decode_tokens(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase),
                                          _ptr(write), _ptr(state), _ptr(out), _stream(dev))
    else:
        rc = getattr(lib(), _entry)(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(state), _ptr(out), _stream(dev))
    if rc != 0:
        raise KdaError(rc, _entry)
    return out


def gdn2_decode_tokens(q, k, v, alpha, erase, write, state, out=None):
    """Gated DeltaNet-2 form of decode_tokens."""
    return decode_tokens(q, k, v, alpha, None, state, out=out, erase=erase, write=write)


def chunk_fwd_varlen(q, k, v, alpha, beta, cu_seqlens, initial_state=None, out=None, final_state=None,
                     want_final=True, workspace=None, erase=None, write=None, sfda=False):
    """Packed variable-length batch: q, k, alpha [1,T,H,dk]; v [1,T,H,dv]; beta [1,T,H]
    (or, for Gated DeltaNet-2, beta=None with erase [1,T,H,dk] and write [1,T,H,dv];
    sfda=True: alpha holds the SFDA complex gates); cu_seqlens int32 [N+1] on the
    device; states [N,H,dk,dv] fp32.
    Returns (o [1,T,H,dv], final_state [N,H,dk,dv] or None)."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if B != 1:
        raise ValueError("a packed batch has B == 1")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-D int32 tensor")
    N = cu_seqlens.numel() - 1
    code = _dtype_code(q)
    g2 = erase is not None or write is not None
    dev = q.device
    if out is None:
        out = torch.empty((1, T, H, dv), dtype=q.dtype, device=dev)
    if final_state is None and want_final:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None and (t.dtype != torch.float32 or t.shape != (N, H, dk, dv)):
            raise ValueError(f"{nm} must be float32 [N,H,dk,dv]")
    shape = Shape(1, T, H, dk, dv, 64, code)
    need = int(lib().kda_chunk_fwd_varlen_workspace_size(ctypes.byref(shape), N))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check((q, k, v, alpha, beta, erase, write, cu_seqlens, initial_state, out, final_state, workspace),
           ("q", "k", "v", "alpha", "beta", "erase", "write", "cu_seqlens", "initial_state", "out", "final_state",
            "workspace"), dev)
    nbytes = workspace.numel() * workspace.element_size()
    if sfda:
        rc = lib().kda_sfda_chunk_fwd_varlen(ctypes.byref(shape), _ptr(cu_seqlens), N, _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(out),
                                             _ptr(final_state), _ptr(workspace), ctypes.c_size_t(nbytes),
                                             _stream(dev))
    elif g2:
        rc = lib().kda_gdn2_chunk_fwd_varlen(ctypes.byref(shape), _ptr(cu_seqlens), N, _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(alpha), _ptr(erase), _ptr(write), _ptr(initial_state), _ptr(out),
                                             _ptr(final_state), _ptr(workspace), ctypes.c_size_t(nbytes),
                                             _stream(dev))
    else:
        rc = lib().kda_chunk_fwd_varlen(ctypes.byref(shape), _ptr(cu_seqlens), N, _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                        _ptr(workspace), ctypes.c_size_t(nbytes), _stream(dev))
    if rc != 0:
        raise KdaError(rc, "kda_chunk_fwd_varlen")
    return out, final_state


def sfda_chunk_fwd(q, k, v, lam, beta, initial_state=None, out=None, final_state=None, want_final=True,
                   workspace=None):
    """SFDA chunk forward with phase control: as chunk_fwd with the decay alpha replaced by
    the complex gates ``lam`` [B,T,H,dk] (channel 2p = Re, 2p+1 = Im of the gate of key
    pair p); two-pass path, bf16; the workspace is allocated here when omitted.
    Returns (o, final_state or None)."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    for t, nm in ((k, "k"), (lam, "lam"), (v, "v"), (beta, "beta")):
        if t.dtype != q.dtype:
            raise TypeError(f"{nm} must have the dtype of q")
    if k.shape != q.shape or lam.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("shapes: q, k, lam [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]")
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if final_state is None and want_final:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, H, dk, dv)):
            raise ValueError(f"{nm} must be float32 [B,H,dk,dv]")
    shape = Shape(B, T, H, dk, dv, 64, code)
    need = int(lib().kda_chunk_fwd_workspace_size(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check((q, k, v, lam, beta, initial_state, out, final_state, workspace),
           ("q", "k", "v", "lam", "beta", "initial_state", "out", "final_state", "workspace"), dev)
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kda_sfda_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(beta),
                                  _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(workspace),
                                  ctypes.c_size_t(nbytes), _stream(dev))
    if rc != 0:
        raise KdaError(rc, "kda_sfda_chunk_fwd")
    return out, final_state


def sfda_decode_step(q, k, v, lam, beta, state, out=None):
    """One SFDA token for every (b, h): lam [B,H,dk] complex gates in place of alpha;
    otherwise decode_step."""
    return decode_step(q, k, v, lam, beta, state, out=out, _entry="kda_sfda_decode_step")


def sfda_decode_tokens(q, k, v, lam, beta, state, out=None):
    """SFDA form of decode_tokens (lam [B,T,H,dk] complex gates in place of alpha)."""
    return decode_tokens(q, k, v, lam, beta, state, out=out, _entry="kda_sfda_decode_tokens")


def bwd_workspace_size(B, T, H, dk, dv, dtype="bf16") -> int:
    """Bytes of device workspace chunk_bwd needs for this shape (0 if invalid)."""
    shape = Shape(B, T, H, dk, dv, 64, BF16 if dtype == "bf16" else F32)
    return int(lib().kda_chunk_bwd_workspace_size(ctypes.byref(shape)))


def _bwd_call(q, k, v, alpha, gates, d_o, cu_seqlens, initial_state, d_final_state, want_d_initial, workspace,
              family="kda"):
    """Shared marshalling of the backward entry points; gates = (beta,) for KDA / CKDA and
    SFDA (family "sfda": complex gates in alpha) or (erase, write) for Gated DeltaNet-2.
    Returns the C call's output tensors."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    g2 = len(gates) == 2
    packed = cu_seqlens is not None
    if packed and B != 1:
        raise ValueError("a packed batch has B = 1")
    code = _dtype_code(q)
    named = (("k", k), ("alpha", alpha), ("v", v), ("d_o", d_o)) + (
        (("erase", gates[0]), ("write", gates[1])) if g2 else (("beta", gates[0]),))
    for nm, t in named:
        if t.dtype != q.dtype:
            raise TypeError(f"{nm} must have the dtype of q")
    if k.shape != q.shape or alpha.shape != q.shape or v.shape != (B, T, H, dv) or d_o.shape != (B, T, H, dv):
        raise ValueError("shapes: q, k, alpha [B,T,H,dk]; v, d_o [B,T,H,dv]")
    if g2 and (gates[0].shape != q.shape or gates[1].shape != v.shape):
        raise ValueError("shapes: erase [B,T,H,dk]; write [B,T,H,dv]")
    if not g2 and gates[0].shape != (B, T, H):
        raise ValueError("shape: beta [B,T,H]")
    if packed and (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1):
        raise TypeError("cu_seqlens must be a 1-d int32 tensor")
    n_states = cu_seqlens.numel() - 1 if packed else B
    for t, nm in ((initial_state, "initial_state"), (d_final_state, "d_final_state")):
        if t is not None and (t.dtype != torch.float32 or t.shape != (n_states, H, dk, dv)):
            raise ValueError(f"{nm} must be float32 [{'n_seqs' if packed else 'B'},H,dk,dv]")
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    new = torch.zeros if packed else torch.empty  # a packed call leaves tokens past the last offset
    dq, dkk, dal = (new((B, T, H, dk), **f32) for _ in range(3))
    dvv = new((B, T, H, dv), **f32)
    dgates = (new((B, T, H, dk), **f32), new((B, T, H, dv), **f32)) if g2 else (new((B, T, H), **f32),)
    ds0 = torch.empty((n_states, H, dk, dv), **f32) if want_d_initial else None
    shape = Shape(B, T, H, dk, dv, 64, code)
    if packed:
        need = int(lib().kda_chunk_bwd_varlen_workspace_size(ctypes.byref(shape), n_states))
    else:
        need = int(lib().kda_chunk_bwd_workspace_size(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check((q, k, v, alpha, d_o, cu_seqlens, initial_state, d_final_state, workspace) + tuple(gates),
           ("q", "k", "v", "alpha", "d_o", "cu_seqlens", "initial_state", "d_final_state", "workspace")
           + tuple(nm for nm, _ in named[4:]), dev)
    nbytes = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    head = [ctypes.byref(shape)] + ([_ptr(cu_seqlens), n_states] if packed else [])
    ins = [_ptr(q), _ptr(k), _ptr(v), _ptr(alpha)] + [_ptr(x) for x in gates]
    outs = [_ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dal)] + [_ptr(x) for x in dgates]
    if family == "sfda" and dk % 2:
        raise ValueError("SFDA gates pair the key channels: dk must be even")
    entry = ("kda_gdn2_chunk_bwd" if g2 else ("kda_sfda_chunk_bwd" if family == "sfda" else "kda_chunk_bwd")) + (
        "_varlen" if packed else "")
    rc = getattr(lib(), entry)(*head, *ins, _ptr(initial_state), _ptr(d_o), _ptr(d_final_state), *outs, _ptr(ds0),
                               _ptr(workspace), nbytes, _stream(dev))
    if rc != 0:
        raise KdaError(rc, entry)
    return (dq, dkk, dvv, dal) + dgates + (ds0,)


def chunk_bwd(q, k, v, alpha, beta, d_o, initial_state=None, d_final_state=None, want_d_initial=True,
              workspace=None):
    """Gradients of L = sum <d_o, o> + <d_final_state, S_T> through chunk_fwd (KDA / CKDA),
    the forward recomputed inside.  Inputs as chunk_fwd; d_o [B,T,H,dv] in the dtype of q;
    d_final_state fp32 [B,H,dk,dv] or None (zero).  workspace: optional uint8 device
    tensor of at least bwd_workspace_size(...) bytes (allocated here when omitted).
    Returns (dq, dk, dv, dalpha, dbeta, d_initial_state or None), all fp32."""
    return _bwd_call(q, k, v, alpha, (beta,), d_o, None, initial_state, d_final_state, want_d_initial, workspace)


def chunk_bwd_varlen(q, k, v, alpha, beta, d_o, cu_seqlens, initial_state=None, d_final_state=None,
                     want_d_initial=True, workspace=None):
    """Backward of chunk_fwd_varlen: a packed batch (B = 1) of len(cu_seqlens) - 1 sequences
    at the int32 device offsets cu_seqlens, each differentiated from its own start state.
    initial_state, d_final_state: fp32 [n_seqs, H, dk, dv] or None.  Returns (dq, dk, dv,
    dalpha, dbeta, d_initial_state [n_seqs, H, dk, dv] or None), all fp32; tokens after the
    last offset get zeros."""
    return _bwd_call(q, k, v, alpha, (beta,), d_o, cu_seqlens, initial_state, d_final_state, want_d_initial,
                     workspace)


def gdn2_chunk_bwd(q, k, v, alpha, erase, write, d_o, initial_state=None, d_final_state=None, want_d_initial=True,
                   workspace=None, cu_seqlens=None):
    """Gated DeltaNet-2 backward of gdn2_chunk_fwd (or, with cu_seqlens, of its packed form):
    erase [B,T,H,dk] and write [B,T,H,dv] in the dtype of q in place of beta.  Returns (dq,
    dk, dv, dalpha, d_erase, d_write, d_initial_state or None), all fp32."""
    return _bwd_call(q, k, v, alpha, (erase, write), d_o, cu_seqlens, initial_state, d_final_state, want_d_initial,
                     workspace)


def sfda_chunk_bwd(q, k, v, lam, beta, d_o, initial_state=None, d_final_state=None, want_d_initial=True,
                   workspace=None, cu_seqlens=None):
    """SFDA backward of sfda_chunk_fwd (or, with cu_seqlens, of its packed form): lam
    [B,T,H,dk] holds (Re, Im) of each key-channel pair's gate.  Returns (dq, dk, dv, dlam,
    dbeta, d_initial_state or None), all fp32; dlam holds d/dRe and d/dIm in the pair's
    channels."""
    return _bwd_call(q, k, v, lam, (beta,), d_o, cu_seqlens, initial_state, d_final_state, want_d_initial,
                     workspace, family="sfda")
