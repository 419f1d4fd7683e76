"""The grouped GEMM launches' workgroup -> tile mappings, built for the host from
the same header functions the kernels call (csrc/ffn_layout.h, csrc/bwd_layout.h)
and checked exhaustively over table sizes, shared-tile counts and run lengths:
every tile is computed by exactly one workgroup of the grid the launcher sizes
(a tile no workgroup takes would leave its outputs unwritten, silently)."""
import os
import shutil
import subprocess

import pytest

from biased_top_routing_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_every_tile_taken_exactly_once(tmp_path):
    if not (os.path.exists(B.HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not found")
    exe = tmp_path / "tile_mapping_check"
    cmd = [B.HIPCC, "-std=c++17", "-O2", "--cuda-host-only", "-x", "hip",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "biased_top_routing_amd", "csrc"),
           os.path.join(HERE, "tile_mapping_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
