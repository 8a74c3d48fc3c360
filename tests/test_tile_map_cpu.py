"""The prefill's block -> tile map, enumerated on the host.

`tests/tile_map_check.cpp` includes the kernels' own header
(`prefill_tiles.h`) and, for 1764 shapes (batch sizes 1..16, lengths 1..8205
with ragged last tiles, 1..24 groups, top-k 1..4), checks that every
(sequence, virtual group, tile) is produced by exactly one block, that blocks
come longest causal extent first on each XCD's list, and that with G a
multiple of 8 a group's routed tiles stay on one XCD. The GPU parity tests
read every output row of several shapes; this covers the index arithmetic of
many more.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def test_prefill_tile_map_host(tmp_path):
    exe = str(tmp_path / "tile_map_check")
    cmd = [_hipcc(), "--offload-host-only", "-x", "hip", "-std=c++17", "-O2",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sparse_query_gqa_amd", "csrc"),
           os.path.join(ROOT, "tests", "tile_map_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-2000:]
    assert "tile map ok: 1764 shapes" in r.stdout
