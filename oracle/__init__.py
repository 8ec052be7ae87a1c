"""fp64 CPU oracle for the KDA / CKDA gated delta rule -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  It is the parity reference for the HIP library and
shares no code with it; the product path never calls it.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, OpenMP): the token
recurrence

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t,

taken from the SFDA page ("Resumen Tecnico: Atencion Delta de Fourier
Semidirecta", section "Arquitectura Central", phases set to zero) and the
Gated DeltaNet-2 page (section 1, erase and write gates tied to beta).  This
module only marshals numpy arrays into that library.

Parity pins (all in ``tests/test_oracle*.py``): explicit products of the dense
transition matrices, alpha = 1 (plain delta rule), scalar alpha (Gated
DeltaNet), beta = 0 (pure decay), spectral norm <= 1, Frobenius-norm
preservation for alpha in {-1, 1} and beta in {0, 2} with zero writes, the d=2
reflection-pair rotation and its mod-5 counter, the affine block transfer and
split invariance, and a mutation test that plants mistakes in copies of the C
source and checks that the pins catch each one.  The SFDA recurrence (complex
rotation-decay gates on channel pairs; same page, section "Arquitectura Central")
has its own pins in ``tests/test_oracle_sfda.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_kda_oracle.so")
_lib = None

BF16, F32, F64 = 0, 1, 2


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the .so path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", src, "-o", out]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = _LIB_PATH):
    """Load (building first if absent) and return the ctypes library."""
    global _lib
    if path == _LIB_PATH and _lib is not None:
        return _lib
    if not os.path.exists(path) or (path == _LIB_PATH and os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build(out=path)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, I, I, I]
    lib.kda_oracle_fwd.restype = I
    lib.kda_oracle_decode.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, I, I]
    lib.kda_oracle_decode.restype = I
    lib.kda_oracle_fwd_gdn2.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, I, I, I]
    lib.kda_oracle_fwd_gdn2.restype = I
    lib.kda_oracle_decode_gdn2.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, I, I]
    lib.kda_oracle_decode_gdn2.restype = I
    lib.kda_oracle_fwd_sfda.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, I, I, I]
    lib.kda_oracle_fwd_sfda.restype = I
    lib.kda_oracle_decode_sfda.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, I, I]
    lib.kda_oracle_decode_sfda.restype = I
    lib.kda_oracle_bwd.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, I, I]
    lib.kda_oracle_bwd.restype = I
    lib.kda_oracle_bwd_gdn2.argtypes = [I, I, I, I, I, I] + [P] * 17 + [I, I]
    lib.kda_oracle_bwd_gdn2.restype = I
    lib.kda_oracle_bwd_sfda.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, I, I]
    lib.kda_oracle_bwd_sfda.restype = I
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16  # bf16 bit patterns
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs must be uint16 (bf16 bits), float32 or float64, got {a.dtype}")


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def fwd(q, k, v, alpha, beta, S0=None, heads=None, col_block=0, nthreads=0, lib=None,
        want_o=True):
    """Run the token recurrence over whole sequences.

    q, k, alpha: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H]; all the same
    dtype (uint16 = bf16 bits, float32 or float64).
    S0: None (zeros) or [n_sel, dk, dv] (any float dtype; widened to fp64).
    heads: None (all B*H pairs, in b*H + h order) or a list of flat indices.
    Returns (o [n_sel, T, dv] fp64 or None, S_T [n_sel, dk, dv] fp64).
    """
    return _fwd_impl("kda_oracle_fwd", q, k, v, alpha, beta, S0, heads, col_block, nthreads, lib, want_o)


def _fwd_impl(_entry, q, k, v, alpha, beta, S0, heads, col_block, nthreads, lib, want_o):
    lib = lib or load()
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, alpha, beta)]
    code = _dtype_code(arrs[0])
    for a in arrs[1:]:
        if _dtype_code(a) != code:
            raise TypeError("all oracle inputs must share one dtype")
    B, T, H, dk = arrs[0].shape
    dv = arrs[2].shape[-1]
    sel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    n_sel = B * H if sel is None else len(sel)
    S0d = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64)).reshape(n_sel, dk, dv)
    o = np.empty((n_sel, T, dv), np.float64) if want_o else None
    S = np.empty((n_sel, dk, dv), np.float64)
    rc = getattr(lib, _entry)(B, T, H, dk, dv, code, *[_ptr(a) for a in arrs], _ptr(S0d),
                              _ptr(o), _ptr(S), _ptr(sel), n_sel, int(col_block), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"{_entry} failed")
    return o, S


def decode(q, k, v, alpha, beta, state, heads=None, nthreads=0, lib=None):
    """One decode step; ``state`` ([n_sel, dk, dv] fp64) is updated in place.

    q, k, alpha: [B, H, dk]; v: [B, H, dv]; beta: [B, H].  Returns o [n_sel, dv].
    """
    return _decode_impl("kda_oracle_decode", q, k, v, alpha, beta, state, heads, nthreads, lib)


def _decode_impl(_entry, q, k, v, alpha, beta, state, heads, nthreads, lib):
    lib = lib or load()
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, alpha, beta)]
    code = _dtype_code(arrs[0])
    B, H, dk = arrs[0].shape
    dv = arrs[2].shape[-1]
    sel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    n_sel = B * H if sel is None else len(sel)
    if state.dtype != np.float64 or not state.flags.c_contiguous or state.shape != (n_sel, dk, dv):
        raise TypeError("state must be a C-contiguous float64 array of shape [n_sel, dk, dv]")
    o = np.empty((n_sel, dv), np.float64)
    rc = getattr(lib, _entry)(B, H, dk, dv, code, *[_ptr(a) for a in arrs], _ptr(state), _ptr(o),
                              _ptr(sel), n_sel, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"{_entry} failed")
    return o


def fwd_gdn2(q, k, v, alpha, erase, write, S0=None, heads=None, col_block=0, nthreads=0, lib=None,
             want_o=True):
    """Gated DeltaNet-2 recurrence over whole sequences: as fwd, with beta replaced by
    the erase gate [B, T, H, dk] and the write gate [B, T, H, dv]."""
    lib = lib or load()
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, alpha, erase, write)]
    code = _dtype_code(arrs[0])
    for a in arrs[1:]:
        if _dtype_code(a) != code:
            raise TypeError("all oracle inputs must share one dtype")
    B, T, H, dk = arrs[0].shape
    dv = arrs[2].shape[-1]
    if arrs[4].shape != arrs[0].shape or arrs[5].shape != arrs[2].shape:
        raise ValueError("erase gate [B,T,H,dk], write gate [B,T,H,dv]")
    sel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    n_sel = B * H if sel is None else len(sel)
    S0d = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64)).reshape(n_sel, dk, dv)
    o = np.empty((n_sel, T, dv), np.float64) if want_o else None
    S = np.empty((n_sel, dk, dv), np.float64)
    rc = lib.kda_oracle_fwd_gdn2(B, T, H, dk, dv, code, *[_ptr(a) for a in arrs], _ptr(S0d),
                                 _ptr(o), _ptr(S), _ptr(sel), n_sel, int(col_block), int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_fwd_gdn2 failed")
    return o, S


def decode_gdn2(q, k, v, alpha, erase, write, state, heads=None, nthreads=0, lib=None):
    """One Gated DeltaNet-2 decode step; ``state`` ([n_sel, dk, dv] fp64) in place.
    erase [B, H, dk], write [B, H, dv].  Returns o [n_sel, dv]."""
    lib = lib or load()
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, alpha, erase, write)]
    code = _dtype_code(arrs[0])
    B, H, dk = arrs[0].shape
    dv = arrs[2].shape[-1]
    sel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    n_sel = B * H if sel is None else len(sel)
    if state.dtype != np.float64 or not state.flags.c_contiguous or state.shape != (n_sel, dk, dv):
        raise TypeError("state must be a C-contiguous float64 array of shape [n_sel, dk, dv]")
    o = np.empty((n_sel, dv), np.float64)
    rc = lib.kda_oracle_decode_gdn2(B, H, dk, dv, code, *[_ptr(a) for a in arrs], _ptr(state), _ptr(o),
                                    _ptr(sel), n_sel, int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_decode_gdn2 failed")
    return o


def fwd_sfda(q, k, v, lam, beta, S0=None, heads=None, col_block=0, nthreads=0, lib=None, want_o=True):
    """SFDA recurrence (phase control) over whole sequences: as fwd, with the decay
    replaced by complex gates ``lam`` [B, T, H, dk] (channel 2p = Re, 2p+1 = Im of the
    gate of coordinate p, acting on rows 2p, 2p+1 of the state)."""
    return _fwd_impl("kda_oracle_fwd_sfda", q, k, v, lam, beta, S0, heads, col_block, nthreads, lib, want_o)


def decode_sfda(q, k, v, lam, beta, state, heads=None, nthreads=0, lib=None):
    """One SFDA decode step; lam [B, H, dk] complex gates as in fwd_sfda."""
    return _decode_impl("kda_oracle_decode_sfda", q, k, v, lam, beta, state, heads, nthreads, lib)


def bwd_gdn2(q, k, v, alpha, erase, write, dO, S0=None, dST=None, heads=None, nthreads=0, lib=None):
    """Gated DeltaNet-2 backward (GDN-2 page, section 3: the per-channel erase and write
    gates inside the gradients): as bwd with the erase gate [B, T, H, dk] and the write
    gate [B, T, H, dv] in place of beta.  Returns dq, dk, dalpha, derase [n_sel, T, dk];
    dv, dwrite [n_sel, T, dv]; dS0 [n_sel, dk, dv] (fp64)."""
    lib = lib or load()
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, alpha, erase, write)]
    code = _dtype_code(arrs[0])
    for a in arrs[1:]:
        if _dtype_code(a) != code:
            raise TypeError("all oracle inputs must share one dtype")
    B, T, H, dk = arrs[0].shape
    dv = arrs[2].shape[-1]
    sel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    n_sel = B * H if sel is None else len(sel)
    f64 = lambda x, shp: None if x is None else np.ascontiguousarray(np.asarray(x, dtype=np.float64)).reshape(shp)
    S0d, dSTd = f64(S0, (n_sel, dk, dv)), f64(dST, (n_sel, dk, dv))
    dOd = f64(dO, (n_sel, T, dv))
    out = {"dq": np.empty((n_sel, T, dk)), "dk": np.empty((n_sel, T, dk)), "dv": np.empty((n_sel, T, dv)),
           "dalpha": np.empty((n_sel, T, dk)), "derase": np.empty((n_sel, T, dk)),
           "dwrite": np.empty((n_sel, T, dv)), "dS0": np.empty((n_sel, dk, dv))}
    rc = lib.kda_oracle_bwd_gdn2(B, T, H, dk, dv, code, *[_ptr(a) for a in arrs], _ptr(S0d), _ptr(dOd),
                                 _ptr(dSTd), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                 _ptr(out["dalpha"]), _ptr(out["derase"]), _ptr(out["dwrite"]), _ptr(out["dS0"]),
                                 _ptr(sel), n_sel, int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_bwd_gdn2 failed")
    return out


def bwd(q, k, v, alpha, beta, dO, S0=None, dST=None, heads=None, nthreads=0, lib=None):
    """Gradients of L = sum <dO, o> + <dST, S_T> for the KDA / CKDA forward (reverse mode
    through the token recurrence).  Inputs as fwd; dO [n_sel, T, dv] and dST
    [n_sel, dk, dv] (or None) are widened to fp64.  Returns a dict of fp64 arrays:
    dq, dk, dalpha [n_sel, T, dk]; dv [n_sel, T, dv]; dbeta [n_sel, T]; dS0 [n_sel, dk, dv]."""
    return _bwd_impl("kda_oracle_bwd", q, k, v, alpha, beta, dO, S0, dST, heads, nthreads, lib)


def bwd_sfda(q, k, v, lam, beta, dO, S0=None, dST=None, heads=None, nthreads=0, lib=None):
    """SFDA backward (SFDA page, "Arquitectura Central": complex rotation-decay gates): as
    bwd with lam holding (Re, Im) of each key-channel pair's gate in channels (2p, 2p+1);
    the "dalpha" entry holds d/dRe in channel 2p and d/dIm in channel 2p+1."""
    return _bwd_impl("kda_oracle_bwd_sfda", q, k, v, lam, beta, dO, S0, dST, heads, nthreads, lib)


def _bwd_impl(_entry, q, k, v, alpha, beta, dO, S0, dST, heads, nthreads, lib):
    lib = lib or load()
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, alpha, beta)]
    code = _dtype_code(arrs[0])
    for a in arrs[1:]:
        if _dtype_code(a) != code:
            raise TypeError("all oracle inputs must share one dtype")
    B, T, H, dk = arrs[0].shape
    dv = arrs[2].shape[-1]
    sel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    n_sel = B * H if sel is None else len(sel)
    f64 = lambda x, shp: None if x is None else np.ascontiguousarray(np.asarray(x, dtype=np.float64)).reshape(shp)
    S0d, dSTd = f64(S0, (n_sel, dk, dv)), f64(dST, (n_sel, dk, dv))
    dOd = f64(dO, (n_sel, T, dv))
    out = {"dq": np.empty((n_sel, T, dk)), "dk": np.empty((n_sel, T, dk)), "dv": np.empty((n_sel, T, dv)),
           "dalpha": np.empty((n_sel, T, dk)), "dbeta": np.empty((n_sel, T)), "dS0": np.empty((n_sel, dk, dv))}
    rc = getattr(lib, _entry)(B, T, H, dk, dv, code, *[_ptr(a) for a in arrs], _ptr(S0d), _ptr(dOd), _ptr(dSTd),
                              _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]),
                              _ptr(out["dbeta"]), _ptr(out["dS0"]), _ptr(sel), n_sel, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"{_entry} failed")
    return out
