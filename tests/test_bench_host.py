"""The host side of bench.py on the CPU: the one-GPU refusal, the algorithmic
units and the oracle baseline record (no GPU involved)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_units():
    # packed codes + fp16 scale and zero per group of 128 + x + y, for the decode layer
    N, K = 11008, 4096
    assert bench.alg_bytes(1, N, K, 0) == N * K // 2 + N * (K // 128) * 4 + 2 * K + 2 * N == 23983616
    # the CSR adds 6 bytes per entry and 4 per row pointer
    assert bench.alg_bytes(16, 4096, 4096, 75497) - bench.alg_bytes(16, 4096, 4096, 0) == 6 * 75497 + 4 * 4097
    assert bench.alg_flops(2048, 14336, 4096, 0) == 2 * 2048 * 14336 * 4096
    assert bench.alg_flops(8, 8192, 28672, 117440) == 2 * 8 * 8192 * 28672 + 2 * 8 * 117440
    # a rank-r branch adds its two fp16 factors and 2 M r (K + N) flops; an
    # act-order layer adds its int32 channel permutation
    assert bench.alg_bytes(1, N, K, 0, rank=32) - bench.alg_bytes(1, N, K, 0) == 2 * 32 * (K + N)
    assert bench.alg_flops(2048, 14336, 4096, 0, rank=32) - bench.alg_flops(2048, 14336, 4096, 0) == \
        2 * 2048 * 32 * (4096 + 14336)
    assert bench.alg_bytes(1, N, K, 0, act_order=True) - bench.alg_bytes(1, N, K, 0) == 4 * K


def test_cpu_baseline_record():
    b = bench.cpu_baseline(budget_s=0.05)
    assert b["kind"] == "oracle" and b["unit"] == "GB/s"
    assert b["value"] > 0 and b["cores"] >= 1
    assert set(b["phases_ms"]) == {"quantize_fp32", "dequantize_fp64", "linear_ref"}
    assert "11008" in b["sample"] and "4096" in b["sample"]


def test_traffic_record_describes_the_current_decode_kernel():
    """The committed HBM-traffic record of the headline's decode kernel (which the
    bench reports as roofline.traffic) was measured on the kernel's current sources:
    a change to them needs the counters taken again."""
    t = bench.recorded_traffic()
    assert t is not None, "profiles/gemv_decode_7b_up_proj_traffic.txt describes other kernel sources"
    # within a few percent of the algorithmic bytes: every weight read from HBM once
    alg = bench.alg_bytes(1, 11008, 4096, 0)
    assert 0.99 * alg <= t <= 1.05 * alg
