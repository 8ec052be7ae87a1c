"""The split walks at forced segment counts, against the fp64 oracle (gpu).

The library takes the split from 8 segments on; KDA_STATE_SEG forces G segments for
tuning, which reaches the degenerate launch layouts: G = 2 (segment 0 walked in full, then
segment 1 from its end), G = 3 (segments 0, 1 and 2 each walked in full, no end-state or
transfer walks, no scan), G = 4 and 5 (one and two middle segments through the end-state
and transfer walks and the scan).  The setting is read once per process, so each count
runs in a child process of its own (one at a time).  Inputs follow the long-memory recipe
(gates in {1, 1 - 2^-8}, beta <= 0.05, S0 ~ N(0, 1)), where the start state carries into
every output, so a wrong segment start shows at O(1).  The backward's state and adjoint
walks (KDA_BWD_SEG) take the same counts: below 4 every segment goes through the end-state
and transfer walks, from 4 on the first two (the adjoint: the last two) are walked in full
beside them.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r"""
import ctypes, sys
import numpy as np
sys.path[:0] = [{root!r}, {here!r}]
import gated_delta_rule_78_amd as kda
from gated_delta_rule_78_amd import lib
from gated_delta_rule_78_amd.inputs import make, bf16_bits
from test_gpu_chunk import _check
G = {G}
T = 64 * 90 + 5
sh = kda.Shape(1, T, 2, 128, 128, 64, 0)
plain = kda.Shape(1, 64 * 15, 2, 128, 128, 64, 0)
rec = lambda s: (s.T + 63) // 64 * s.B * s.H
one = lib().kda_chunk_fwd_workspace_size(ctypes.byref(plain)) // rec(plain)
# the split is taken with G segments: its scratch is B, P and the start states per segment
assert lib().kda_chunk_fwd_workspace_size(ctypes.byref(sh)) == rec(sh) * one + 2 * G * 128 * (2 * 128 + 128) * 4
inp = make(1, T, 2, 128, 128, "bf16", "kda", False, seed=90 + G)
rng = np.random.default_rng(90 + G)
inp.alpha = bf16_bits(np.where(rng.random(inp.alpha.shape) < 0.5, 1.0, 1.0 - 2.0 ** -8).astype(np.float32))
inp.beta = bf16_bits((0.05 * rng.random(inp.beta.shape)).astype(np.float32))
S0 = rng.standard_normal(inp.S0.shape).astype(np.float32)
_check(inp, S0, label="split G=%d" % G, path="twopass")
_check(inp, S0, in_place=True, label="split G=%d in place" % G, path="twopass")
print("ok", flush=True)
"""


@pytest.mark.parametrize("G", [2, 3, 4, 5])
def test_split_walk_forced_segments(G):
    print(f"split walk with KDA_STATE_SEG={G} (child process)", flush=True)
    env = dict(os.environ, KDA_STATE_SEG=str(G))
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, here=HERE, G=G)], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=110)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0 and r.stdout.rstrip().endswith("ok")


CHILD_BWD = r"""
import sys
sys.path[:0] = [{root!r}, {here!r}]
from test_gpu_bwd import _split_inputs, _check
G = {G}
inp, dO, dST, S0 = _split_inputs("ckda", 80 + G, long_memory=True)
_check(inp, dO, dST, S0, label="bwd split G=%d" % G)
print("ok", flush=True)
"""


@pytest.mark.parametrize("G", [2, 3, 4, 5])
def test_bwd_split_walks_forced_segments(G):
    print(f"backward split walks with KDA_BWD_SEG={G} (child process)", flush=True)
    env = dict(os.environ, KDA_BWD_SEG=str(G))
    r = subprocess.run([sys.executable, "-c", CHILD_BWD.format(root=ROOT, here=HERE, G=G)], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=110)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0 and r.stdout.rstrip().endswith("ok")
