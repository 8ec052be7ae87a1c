"""kda_chunk_fwd_noalloc (the two-pass forward on the library's fixed per-GPU scratch)
against kda_chunk_fwd_ws on a caller-allocated workspace, both called through the C ABI
(gpu).  The two run the same kernels on the same inputs, so their outputs agree bit for
bit; three calls in a row reuse the one scratch array, each smaller than the one before,
so a call that read what an earlier, larger call left behind would show."""
import ctypes

import numpy as np
import pytest

from gated_delta_rule_78_amd.inputs import make
from kda_testutil import TOL, inputs_to_dev, rel_err_slices, state_to_dev

pytestmark = pytest.mark.gpu

KDA_ERR_SCRATCH = -9
SCRATCH_BYTES = 64 << 20


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _run_both(L, B, T, H, dk, dv, gates, seed):
    import torch
    import gated_delta_rule_78_amd as kda
    print(f"noalloc B={B} T={T} H={H} dk={dk} dv={dv} {gates} seed={seed}", flush=True)
    inp = make(B, T, H, dk, dv, "bf16", gates, False, seed=seed)
    q, k, v, a, b = inputs_to_dev(inp)
    s0 = state_to_dev(inp.S0)
    shape = kda.Shape(B, T, H, dk, dv, 64, kda.BF16)
    need = int(L.kda_chunk_fwd_workspace_size(ctypes.byref(shape)))
    assert 0 < need <= SCRATCH_BYTES
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    o1 = torch.full((B, T, H, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    s1 = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    rc = L.kda_chunk_fwd_noalloc(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(a), _p(b), _p(s0), _p(o1), _p(s1),
                                 stream)
    assert rc == 0, kda.status_string(rc)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    s2 = torch.empty_like(s1)
    rc = L.kda_chunk_fwd_ws(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(a), _p(b), _p(s0), _p(o2), _p(s2),
                            _p(ws), ctypes.c_size_t(need), stream)
    assert rc == 0, kda.status_string(rc)
    torch.cuda.synchronize()
    o1n, o2n = o1.float().cpu().numpy(), o2.float().cpu().numpy()
    s1n, s2n = s1.cpu().numpy(), s2.cpu().numpy()
    BH = B * H
    eo = rel_err_slices(o1n.transpose(0, 2, 1, 3).reshape(BH, -1), o2n.transpose(0, 2, 1, 3).reshape(BH, -1), BH)
    es = rel_err_slices(s1n.reshape(BH, -1), s2n.reshape(BH, -1), BH)
    print(f"   err o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert np.array_equal(o1n, o2n) and np.array_equal(s1n, s2n)


def test_noalloc_matches_workspace_entry_point():
    import gated_delta_rule_78_amd as kda
    L = kda.lib()
    # a split walk (few chains, 131 chunks each), then two plain walks, each call smaller
    _run_both(L, 1, 64 * 130 + 5, 2, 128, 128, "ckda", 301)
    _run_both(L, 2, 300, 4, 128, 128, "kda", 302)
    _run_both(L, 1, 130, 3, 64, 128, "ckda", 303)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """The B4 H32 T8192 workload needs 352 MB of records: refused before anything runs."""
    import torch
    import gated_delta_rule_78_amd as kda
    L = kda.lib()
    shape = kda.Shape(4, 8192, 32, 128, 128, 64, kda.BF16)
    assert int(L.kda_chunk_fwd_workspace_size(ctypes.byref(shape))) > SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")  # never read: the call returns first
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.kda_chunk_fwd_noalloc(ctypes.byref(shape), _p(x), _p(x), _p(x), _p(x), _p(x), None, _p(x), None, stream)
    assert rc == KDA_ERR_SCRATCH
    assert "KDA_NOALLOC_SCRATCH_BYTES" in kda.status_string(rc)
