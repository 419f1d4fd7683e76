"""Host logic of bench.py (runs without a GPU): the one-GPU guard, and the algorithmic
byte and FLOP counts its rates divide by, against totals worked out by hand from the
V3-like prefill shape (T = 16384 tokens, hidden 7168, 256 routed experts, top-8,
1 shared expert, intermediate 2048, bf16)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import V3_PREFILL  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stage_bytes_at_the_prefill_shape():
    c = V3_PREFILL
    b = bench.stage_bytes(c, gather=False, scores=True)
    # combine, per token: 8 routed rows + the shared row read (2 * 7168 bytes each), the
    # output row written, 8 (row, gate) pairs of 4 + 4 bytes: 143,424 bytes
    assert b["combine"] == 16384 * (9 * 14336 + 14336 + 64)
    assert abs(b["combine"] / 2.350e9 - 1) < 1e-3
    # dispatch with the row copy: x read once, 8 copies written, 16 bytes of indices per pair
    assert b["dispatch"] == 16384 * (14336 + 8 * 14336 + 8 * 16)
    assert abs(b["dispatch"] / 2.116e9 - 1) < 1e-3
    # top-k on stored affinities: 1 KB of fp32 scores per token, the bias, 64 bytes of idx + w out
    assert abs(b["topk"] / 17.83e6 - 1) < 1e-3
    # router GEMM: x (235 MB) and the 3.67 MB router weight in, the affinities out
    assert b["router"] == 16384 * 14336 + 256 * 14336 + 16384 * 256 * 4
    g = bench.stage_bytes(c, gather=True, scores=False)
    assert g["dispatch"] == 16384 * 8 * 16            # indices only: the GEMM gathers the rows
    assert g["router"] == 16384 * 14336 + 256 * 14336
    assert g["topk"] == 256 * 4 + 16384 * 64


def test_gemm_flops_at_the_prefill_shape():
    c = V3_PREFILL
    # 9 rows per token (8 routed + 1 shared), 6 * H * I flop per row: 12.99 TFLOP
    assert c.gate_up_flops() == 9 * 16384 * 4 * 7168 * 2048 == 8658654068736
    assert c.down_flops() * 2 == c.gate_up_flops()
    assert abs((c.gate_up_flops() + c.down_flops()) / 12.99e12 - 1) < 1e-3
    assert c.router_flops() == 2 * 16384 * 7168 * 256


@pytest.mark.parametrize("workload", ["v3_prefill_bf16", "mid_bf16"])
def test_traffic_summary_is_keyed_to_its_workload(workload):
    t = bench.measured_traffic(workload)
    if workload != "v3_prefill_bf16":
        assert t is None
    else:
        assert t is None or t > 0
