"""Seeded synthetic inputs for the KDA / CKDA workloads.

This module only draws random numbers and shapes them; it holds none of the
recurrence's arithmetic.  Both the HIP path (through the tests and the
benchmark) and the fp64 oracle consume exactly the arrays made here.

Recipe (one numpy PCG64 stream per tensor, from ``SeedSequence(seed).spawn(7)``
in the order q, k, v, alpha, beta, S0, mask; fp32 draws; bf16 workloads are
rounded to bf16 by round-to-nearest-even and handed over as uint16 bit
patterns, which both sides widen exactly):

* q, k   ~ N(0, 1), L2-normalised per (b, t, h) row (before bf16 rounding).
* v      ~ N(0, 1).
* KDA gates   : alpha = exp(-0.1 * softplus(x)), beta = sigmoid(x), x ~ N(0, 1).
* CKDA gates  : alpha = tanh(2x) in [-1, 1], beta = 2 * sigmoid(2x) in [0, 2];
  then a Bernoulli(0.05) mask over alpha entries sets each masked entry to a
  value drawn uniformly from {-1, 0, +1} (+0.0 for zero).
* GDN-2 gates : alpha as KDA; an erase gate b = sigmoid(x) per key channel and a
  write gate w = sigmoid(x) per value channel, x ~ N(0, 1) (two more streams,
  children 7 and 8 of the same SeedSequence, so the other tensors do not change);
  beta is drawn as for KDA and unused by GDN-2.
* SFDA gates : complex gates lambda = a e^{i theta} per key-channel pair p, stored
  as (Re, Im) in channels (2p, 2p+1) of the alpha tensor; magnitude
  a = exp(-0.1 * softplus(x)) from the even channels of the alpha stream, phase
  theta ~ U(-pi, pi) from a tenth stream (child 9); a Bernoulli(0.05) mask per pair
  sets lambda to one of {0, 1, -1, i, -i} (exact zeros and quarter turns); bf16
  gates whose rounded magnitude exceeds 1 are shrunk by 2^-8 and rounded again;
  beta = 2 * sigmoid(2x) in [0, 2] as for CKDA.
* S0     ~ N(0, std 0.02) in fp32, or zeros.

The five named workloads mirror the shapes the method is evaluated on: a tiny
fp32 KDA case, KDA and CKDA prefill at B=4, H=32, T=8192, d=128 (8K tokens is
the longest evaluated context on the Gated DeltaNet-2 page, RULER section), a
long-context CKDA prefill at T=131072 with H=16, and a batched CKDA decode of
B=256 sequences, H=32, for 64 steps.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20260


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str          # "bf16" or "f32"
    gates: str          # "kda", "ckda", "gdn2" or "sfda"
    zero_s0: bool
    decode_steps: int = 0   # > 0: decode workload, T is ignored
    index: int = 0


WORKLOADS = {
    "kda_tiny_f32": Workload("kda_tiny_f32", 1, 256, 2, 64, 64, "f32", "kda", True, index=0),
    "kda_prefill_8k": Workload("kda_prefill_8k", 4, 8192, 32, 128, 128, "bf16", "kda", False, index=1),
    "ckda_prefill_8k": Workload("ckda_prefill_8k", 4, 8192, 32, 128, 128, "bf16", "ckda", False, index=2),
    "ckda_prefill_128k": Workload("ckda_prefill_128k", 1, 131072, 16, 128, 128, "bf16", "ckda", False, index=3),
    "ckda_decode_b256": Workload("ckda_decode_b256", 256, 1, 32, 128, 128, "bf16", "ckda", False,
                                 decode_steps=64, index=4),
    "gdn2_prefill_8k": Workload("gdn2_prefill_8k", 4, 8192, 32, 128, 128, "bf16", "gdn2", False, index=5),
    "sfda_prefill_8k": Workload("sfda_prefill_8k", 4, 8192, 32, 128, 128, "bf16", "sfda", False, index=6),
    "sfda_decode_b256": Workload("sfda_decode_b256", 256, 1, 32, 128, 128, "bf16", "sfda", False,
                                 decode_steps=64, index=7),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _softplus(x):
    return np.logaddexp(0.0, x).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


@dataclass
class Inputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    S0: np.ndarray | None       # fp32 [B, H, dk, dv] or None (zeros)
    dtype: str                  # "bf16" (uint16 bit arrays) or "f32"
    meta: dict = field(default_factory=dict)
    erase: np.ndarray | None = None   # GDN-2 erase gate [.., dk]
    write: np.ndarray | None = None   # GDN-2 write gate [.., dv]


def make(B, T, H, dk, dv, dtype="bf16", gates="kda", zero_s0=False, seed=BASE_SEED,
         lead=None, force_mask_p=0.05):
    """Draw one workload.

    ``lead`` (optional) is an extra leading dimension (decode steps): tensors are
    then [lead, B, H, d] and beta [lead, B, H]; otherwise [B, T, H, d], [B, T, H].
    """
    ss = np.random.SeedSequence(seed).spawn(10)
    rq, rk, rv, ra, rb, rs, rm, re, rw, rt = [np.random.default_rng(s) for s in ss]
    shp = (lead, B, H) if lead else (B, T, H)
    f32 = np.float32
    q = _l2n(rq.standard_normal(shp + (dk,), dtype=f32))
    k = _l2n(rk.standard_normal(shp + (dk,), dtype=f32))
    v = rv.standard_normal(shp + (dv,), dtype=f32)
    xa = ra.standard_normal(shp + (dk,), dtype=f32)
    xb = rb.standard_normal(shp, dtype=f32)
    erase = write = None
    if gates in ("kda", "gdn2"):
        alpha = np.exp(-0.1 * _softplus(xa)).astype(f32)
        beta = _sigmoid(xb)
        if gates == "gdn2":
            erase = _sigmoid(re.standard_normal(shp + (dk,), dtype=f32))
            write = _sigmoid(rw.standard_normal(shp + (dv,), dtype=f32))
    elif gates == "ckda":
        alpha = np.tanh(2.0 * xa).astype(f32)
        beta = (2.0 * _sigmoid(2.0 * xb)).astype(f32)
        if force_mask_p > 0:
            m = rm.random(alpha.shape) < force_mask_p
            vals = np.array([-1.0, 0.0, 1.0], f32)[rm.integers(0, 3, size=int(m.sum()))]
            alpha[m] = vals
    elif gates == "sfda":
        if dk % 2:
            raise ValueError("SFDA gates pair the key channels: dk must be even")
        mag = np.exp(-0.1 * _softplus(xa[..., 0::2])).astype(np.float64)
        theta = rt.uniform(-np.pi, np.pi, size=mag.shape)
        re_, im_ = mag * np.cos(theta), mag * np.sin(theta)
        if force_mask_p > 0:
            m = rm.random(mag.shape) < force_mask_p
            pick = rm.integers(0, 5, size=int(m.sum()))
            re_[m] = np.array([0.0, 1.0, -1.0, 0.0, 0.0])[pick]
            im_[m] = np.array([0.0, 0.0, 0.0, 1.0, -1.0])[pick]
        alpha = np.empty(shp + (dk,), f32)
        alpha[..., 0::2], alpha[..., 1::2] = re_, im_
        if dtype == "bf16":
            for _ in range(4):  # keep |lambda| <= 1 after rounding to bf16
                r = bf16_to_f32(bf16_bits(alpha)).astype(np.float64)
                big = r[..., 0::2] ** 2 + r[..., 1::2] ** 2 > 1.0
                if not big.any():
                    break
                big2 = np.repeat(big, 2, axis=-1)
                alpha[big2] = (alpha[big2] * (1.0 - 2.0 ** -8)).astype(f32)
        beta = (2.0 * _sigmoid(2.0 * xb)).astype(f32)
    else:
        raise ValueError(gates)
    S0 = None if zero_s0 else (0.02 * rs.standard_normal((B, H, dk, dv), dtype=f32)).astype(f32)
    if dtype == "bf16":
        q, k, v, alpha, beta = (bf16_bits(x) for x in (q, k, v, alpha, beta))
        if erase is not None:
            erase, write = bf16_bits(erase), bf16_bits(write)
    elif dtype != "f32":
        raise ValueError(dtype)
    return Inputs(q, k, v, alpha, beta, S0, dtype,
                  dict(B=B, T=T, H=H, dk=dk, dv=dv, gates=gates, seed=seed, lead=lead), erase, write)


def make_upstream(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16", seed: int = BASE_SEED):
    """Upstream gradients for the backward: dO [B, T, H, dv] N(0, 1) in the input dtype
    (bf16 bits or fp32) and dS_T [B, H, dk, dv] fp32 N(0, 0.02), from their own seeded
    streams."""
    rd, rs = [np.random.default_rng(s) for s in np.random.SeedSequence([seed, 7]).spawn(2)]
    dO = rd.standard_normal((B, T, H, dv), dtype=np.float32)
    dST = (0.02 * rs.standard_normal((B, H, dk, dv), dtype=np.float32)).astype(np.float32)
    return (bf16_bits(dO) if dtype == "bf16" else dO), dST


def make_workload(name: str, T: int | None = None, B: int | None = None, H: int | None = None,
                  seed: int | None = None) -> Inputs:
    """Draw a named workload, optionally overriding B / T / H (tests use small T)."""
    w = WORKLOADS[name]
    s = BASE_SEED + w.index if seed is None else seed
    if w.decode_steps:
        return make(B or w.B, 1, H or w.H, w.dk, w.dv, w.dtype, w.gates, w.zero_s0, s,
                    lead=w.decode_steps)
    return make(B or w.B, T or w.T, H or w.H, w.dk, w.dv, w.dtype, w.gates, w.zero_s0, s)


def as_float(x: np.ndarray, dtype: str) -> np.ndarray:
    """The exact fp32 values behind an input array (bf16 bits widened)."""
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


def to_torch(inp: Inputs, device="cuda"):
    """Upload the exact input bytes: returns (q, k, v, alpha, beta, S0) torch tensors
    (bf16 inputs keep their bit patterns; S0 is fp32, or None)."""
    import torch

    def up(x):
        if inp.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

    s0 = None if inp.S0 is None else torch.from_numpy(np.ascontiguousarray(inp.S0, np.float32)).to(device)
    return (*[up(x) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)], s0)
