"""The binding loads libkda.so into torch's HIP runtime (CPU: loading only, no launches).

torch carries its own copy of the HIP runtime.  A library loaded before torch binds to the
system copy, and torch then loads its own: two runtimes in one process, and a kernel of
the library launched on a stream torch created fails.  The binding imports torch before it
loads the library, so calling it first (say for a workspace size) must still leave one
runtime mapped.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import gated_delta_rule_78_amd as kda
kda.workspace_size(1, 8325, 2, 128, 128)   # the library first
import torch                               # then torch
maps = sorted({{l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l}})
print(len(maps), maps)
assert len(maps) == 1, maps
"""


def test_library_binds_to_torchs_hip_runtime():
    if not os.path.exists(os.path.join(ROOT, "gated_delta_rule_78_amd", "libkda.so")):
        import pytest
        pytest.skip("libkda.so not built")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], capture_output=True, text=True, timeout=300)
    print(r.stdout, r.stderr[-2000:])
    assert r.returncode == 0
