"""Inputs past 4 GiB on the GPU against the fp64 oracle (gpu).

Every kernel addresses the token tensors and the states through 64-bit offsets; these
tests run shapes whose tensors exceed 2^32 bytes (element indices past 2^31), so that a
32-bit index anywhere on the path would land in the wrong place.  Heads are independent,
so only the sampled heads carry inputs from the seeded generator (one single-head draw
each, which the oracle also reads); the other heads are filled on the device with draws
of the same distributions, so that they do real work, and are not checked.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_78_amd.inputs import make
from kda_testutil import TOL, rel_err_slices

pytestmark = pytest.mark.gpu


def _fill(shape, kind, gen):
    """Device filler for the unchecked heads: q, k unit rows; v normal; KDA gates."""
    import torch
    x = torch.randn(shape, dtype=torch.float32, device="cuda", generator=gen)
    if kind == "unit":
        x = x / x.norm(dim=-1, keepdim=True)
    elif kind == "alpha":
        x = torch.exp(-0.1 * torch.nn.functional.softplus(x))
    elif kind == "beta":
        x = torch.sigmoid(x)
    return x.to(torch.bfloat16)


def _bits_to_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def test_prefill_past_4gib():
    """B=1, T=2^18+37, H=64, d=128 bf16: each of q, k, v, alpha and o spans 4 GiB + 0.6 MB;
    the first and the last head (whose last rows sit past byte 2^32) are checked."""
    import gated_delta_rule_78_amd as kda
    import torch
    B, T, H, D = 1, (1 << 18) + 37, 64, 128
    assert T * H * D * 2 > (1 << 32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    print(f"max-size prefill: filling B={B} T={T} H={H} d={D}", flush=True)
    q = _fill((B, T, H, D), "unit", gen)
    k = _fill((B, T, H, D), "unit", gen)
    v = _fill((B, T, H, D), "normal", gen)
    a = _fill((B, T, H, D), "alpha", gen)
    b = _fill((B, T, H), "beta", gen)
    s0 = 0.02 * torch.randn((B, H, D, D), dtype=torch.float32, device="cuda", generator=gen)
    sel = [0, H - 1]
    host = {}
    for h in sel:
        inp = make(1, T, 1, D, D, "bf16", "kda", False, seed=7100 + h)
        host[h] = inp
        for dst, src in ((q, inp.q), (k, inp.k), (v, inp.v), (a, inp.alpha)):
            dst[0, :, h, :] = _bits_to_dev(src[0, :, 0, :])
        b[0, :, h] = _bits_to_dev(inp.beta[0, :, 0])
        s0[0, h] = torch.from_numpy(inp.S0[0, 0]).cuda()
    path = kda.pick_path(B, T, H, D, D)
    print(f"max-size prefill: running chunk_fwd ({path})", flush=True)
    o, sT = kda.chunk_fwd(q, k, v, a, b, initial_state=s0)
    torch.cuda.synchronize()
    for h in sel:
        inp = host[h]
        o_ref, s_ref = oracle.fwd(inp.q, inp.k, inp.v, inp.alpha, inp.beta, S0=inp.S0.reshape(1, D, D), col_block=16)
        o_gpu = o[0, :, h, :].float().cpu().numpy()[None]
        s_gpu = sT[0, h].cpu().numpy()[None]
        eo, es = rel_err_slices(o_gpu, o_ref, 1), rel_err_slices(s_gpu, s_ref, 1)
        print(f"   head {h}: err o {eo:.3e}  state {es:.3e}", flush=True)
        assert eo <= TOL["bf16"], (h, eo)
        assert es <= TOL["bf16"], (h, es)


def test_decode_state_past_2g_elements():
    """B=2100, H=64, d=128: the fp32 state holds 2.2e9 elements (8.8 GB); two decode steps
    on the first, a middle and the last (b, h), checked against the oracle."""
    import gated_delta_rule_78_amd as kda
    import torch
    B, H, D, steps = 2100, 64, 128, 2
    BH = B * H
    assert BH * D * D > (1 << 31)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4343)
    print(f"max-size decode: filling B={B} H={H} d={D}", flush=True)
    S = 0.02 * torch.randn((B, H, D, D), dtype=torch.float32, device="cuda", generator=gen)
    q = _fill((steps, B, H, D), "unit", gen)
    k = _fill((steps, B, H, D), "unit", gen)
    v = _fill((steps, B, H, D), "normal", gen)
    a = _fill((steps, B, H, D), "alpha", gen)
    bt = _fill((steps, B, H), "beta", gen)
    sel = [0, BH // 2 + 5, BH - 1]
    host = {}
    for s in sel:
        inp = make(1, 1, 1, D, D, "bf16", "ckda", False, seed=7300 + s % 997, lead=steps)
        host[s] = inp
        bi, hi = divmod(s, H)
        for dst, src in ((q, inp.q), (k, inp.k), (v, inp.v), (a, inp.alpha)):
            dst[:, bi, hi, :] = _bits_to_dev(src[:, 0, 0, :])
        bt[:, bi, hi] = _bits_to_dev(inp.beta[:, 0, 0])
        S[bi, hi] = torch.from_numpy(inp.S0[0, 0]).cuda()
    refs = {s: host[s].S0.reshape(1, D, D).astype(np.float64).copy() for s in sel}
    worst_o = 0.0
    for t in range(steps):
        print(f"max-size decode: step {t}", flush=True)
        o = kda.decode_step(q[t], k[t], v[t], a[t], bt[t], S)
        torch.cuda.synchronize()
        for s in sel:
            inp = host[s]
            o_ref = oracle.decode(inp.q[t], inp.k[t], inp.v[t], inp.alpha[t], inp.beta[t], refs[s])
            bi, hi = divmod(s, H)
            worst_o = max(worst_o, rel_err_slices(o[bi, hi].float().cpu().numpy()[None], o_ref, 1))
    errs = [rel_err_slices(S[divmod(s, H)].cpu().numpy()[None], refs[s], 1) for s in sel]
    print(f"   err o {worst_o:.3e}  state {max(errs):.3e}", flush=True)
    assert worst_o <= TOL["bf16"], worst_o
    assert max(errs) <= 1e-5, errs
