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


def test_decode_full_batch_sampled_heads():
    """The batched decode workload (B=256, H=32, d=128, 64 steps) on the GPU; the
    oracle follows a sample of 24 (b, h) pairs through every step."""
    rng = np.random.default_rng(0)
    heads = sorted(rng.choice(256 * 32, size=24, replace=False).tolist()) + [0, 256 * 32 - 1]
    eo, es = _run(256, 32, 128, 128, "bf16", 64, seed=20264, heads=heads)
    assert eo <= TOL["bf16"], eo
    assert es <= 1e-5, es
