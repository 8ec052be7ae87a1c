"""Shared helpers for the GPU parity tests: seeded inputs -> device tensors, and the
per-(batch, head) max relative error used as the parity gate.

Parity gate (the pages fix no error measure; this is the reading used): for each
output tensor and each (b, h) slice, err = max|x - r| / max|r| (denominator
floored at 1e-30); the test takes the maximum over slices and requires it to be
<= 2e-2 for bf16 inputs with an fp32 state, <= 1e-4 for fp32 inputs.  Beside it the
tests print an elementwise diagnostic, max |x - r| / (|r| + 1e-3 rms(r)) per slice
(not gated: near-zero entries of r make it large without any error in the method).
"""
from __future__ import annotations

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-4}


def to_dev(x, dtype, dev="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def inputs_to_dev(inp, dev="cuda"):
    return [to_dev(x, inp.dtype, dev) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)]


def state_to_dev(S0, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(dev)


def rel_err_slices(x, r, axis_slices):
    """max over slices of max|x-r| / max|r|; x, r: arrays whose first axis indexes slices."""
    x = np.asarray(x, np.float64).reshape(axis_slices, -1)
    r = np.asarray(r, np.float64).reshape(axis_slices, -1)
    num = np.abs(x - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((num / den).max())


def heads_of(o_bthd, heads, H):
    """Select flat heads (b*H + h) from a [B, T, H, d] array -> [n, T, d]."""
    return np.stack([o_bthd[s // H, :, s % H] for s in heads])


def elem_err_slices(x, r, axis_slices):
    """Elementwise diagnostic: max over slices and entries of |x - r| / (|r| + 1e-3 rms(r))."""
    x = np.asarray(x, np.float64).reshape(axis_slices, -1)
    r = np.asarray(r, np.float64).reshape(axis_slices, -1)
    rms = np.sqrt((r * r).mean(axis=1, keepdims=True))
    return float((np.abs(x - r) / (np.abs(r) + 1e-3 * rms + 1e-300)).max())
