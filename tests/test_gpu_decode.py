"""Decode step on the GPU against the fp64 oracle (gpu)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_78_amd.inputs import make
from kda_testutil import TOL, inputs_to_dev, rel_err_slices, state_to_dev

pytestmark = pytest.mark.gpu


def _run(B, H, dk, dv, dtype, steps, seed, heads=None, gates="ckda"):
    import gated_delta_rule_78_amd as kda
    import torch
    inp = make(B, 1, H, dk, dv, dtype, gates, False, seed=seed, lead=steps)
    q, k, v, a, b = inputs_to_dev(inp)
    S = state_to_dev(inp.S0)
    sel = list(range(B * H)) if heads is None else list(heads)
    ref = inp.S0.reshape(B * H, dk, dv)[sel].astype(np.float64).copy()
    worst_o = 0.0
    for t in range(steps):
        print(f"decode B={B} H={H} dk={dk} dv={dv} {dtype} step {t}", flush=True)
        o = kda.decode_step(q[t], k[t], v[t], a[t], b[t], S)
        o_ref = oracle.decode(inp.q[t], inp.k[t], inp.v[t], inp.alpha[t], inp.beta[t], ref, heads=sel)
        o_gpu = o.float().cpu().numpy().reshape(B * H, dv)[sel]
        worst_o = max(worst_o, rel_err_slices(o_gpu, o_ref, len(sel)))
    torch.cuda.synchronize()
    S_gpu = S.cpu().numpy().reshape(B * H, dk, dv)[sel]
    return worst_o, rel_err_slices(S_gpu, ref, len(sel))


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_small(dk, dv, dtype):
    eo, es = _run(3, 2, dk, dv, dtype, 6, seed=31 + dk + dv)
    assert eo <= TOL[dtype], eo
    assert es <= 1e-5, es          # the state never passes through bf16


def test_decode_kda_gates():
    eo, es = _run(2, 4, 128, 128, "bf16", 8, seed=5, gates="kda")
    assert eo <= TOL["bf16"] and es <= 1e-5


def test_decode_full_batch_every_head():
    """The batched decode workload (B=256, H=32, d=128, 64 steps) on the GPU; the
    oracle follows all 8,192 (b, h) states through every step."""
    eo, es = _run(256, 32, 128, 128, "bf16", 64, seed=20264)
    assert eo <= TOL["bf16"], eo
    assert es <= 1e-5, es


def test_decode_tokens_equals_single_steps():
    """Several tokens per call (state read once) give exactly the single-step results:
    the same per-token arithmetic on an fp32 state that never leaves fp32."""
    import gated_delta_rule_78_amd as kda
    import torch
    B, H, T = 4, 3, 5
    inp = make(B, T, H, 128, 128, "bf16", "ckda", False, seed=61)
    q, k, v, a, b = inputs_to_dev(inp)
    S1 = state_to_dev(inp.S0)
    S2 = S1.clone()
    o_multi = kda.decode_tokens(q, k, v, a, b, S1)
    outs = [kda.decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                            a[:, t].contiguous(), b[:, t].contiguous(), S2) for t in range(T)]
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    assert torch.equal(o_multi, torch.stack(outs, dim=1))


@pytest.mark.parametrize("gates,T", [("ckda", 7), ("kda", 1), ("ckda", 0)])
def test_decode_tokens_against_oracle(gates, T):
    import gated_delta_rule_78_amd as kda
    import torch
    B, H, dk, dv = 3, 2, 128, 64
    inp = make(B, max(T, 1), H, dk, dv, "bf16", gates, False, seed=70 + T)
    q, k, v, a, b = (x[:, :T].contiguous() for x in inputs_to_dev(inp))
    S = state_to_dev(inp.S0)
    o = kda.decode_tokens(q, k, v, a, b, S)
    torch.cuda.synchronize()
    sl = lambda x: x[:, :T]
    o_ref, s_ref = oracle.fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.alpha), sl(inp.beta),
                              S0=inp.S0.reshape(B * H, dk, dv))
    if T:
        o_gpu = o.float().cpu().numpy().transpose(0, 2, 1, 3).reshape(B * H, T, dv)
        assert rel_err_slices(o_gpu, o_ref, B * H) <= TOL["bf16"]
    assert rel_err_slices(S.cpu().numpy().reshape(B * H, dk, dv), s_ref, B * H) <= 1e-5


def test_gdn2_decode_tokens_against_oracle():
    import gated_delta_rule_78_amd as kda
    import torch
    from kda_testutil import to_dev
    B, H, T, d = 2, 3, 6, 128
    inp = make(B, T, H, d, d, "bf16", "gdn2", False, seed=77)
    q, k, v, a, _ = inputs_to_dev(inp)
    e, w = to_dev(inp.erase, "bf16"), to_dev(inp.write, "bf16")
    S = state_to_dev(inp.S0)
    o = kda.gdn2_decode_tokens(q, k, v, a, e, w, S)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd_gdn2(inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write,
                                   S0=inp.S0.reshape(B * H, d, d))
    o_gpu = o.float().cpu().numpy().transpose(0, 2, 1, 3).reshape(B * H, T, d)
    assert rel_err_slices(o_gpu, o_ref, B * H) <= TOL["bf16"]
    assert rel_err_slices(S.cpu().numpy().reshape(B * H, d, d), s_ref, B * H) <= 1e-5
