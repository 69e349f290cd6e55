"""bench.py: its contract and its algorithmic counts.

Host tests: the multi-GPU request is refused with a message, and the byte
counts behind the preparation and GEMM rooflines are the algorithmic figures
of the path (per element of X: 2 B read, 0.9375 B written for MXFP4; the GEMM
reads both FP4 activation operands, their scales and W once and writes fp32 Y).
The GPU test runs a short bench and checks the JSON line's fields."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth_inputs as si  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_amd_smi_power_parser():
    """The power sampler's reading of `amd-smi metric -p -c --csv`: socket power
    and the mean of the XCD clocks; None when the tool printed no data line."""
    hdr = "gpu,socket_power,gfx_voltage," + ",".join(f"gfx_{i}_clk,gfx_{i}_min_clk" for i in range(8)) + ",mem_0_clk"
    row = "0,1381,N/A," + ",".join(f"{1700 + 10 * i},500" for i in range(8)) + ",2000"
    p, c = bench.parse_amd_smi_power(hdr + "\n" + row + "\n")
    assert p == 1381.0 and c == 1735.0
    assert bench.parse_amd_smi_power("WARNING: no data\n") is None
    assert bench.parse_amd_smi_power(hdr + "\n") is None
    assert bench.parse_amd_smi_power(hdr + "\n0,N/A,N/A," + ",".join("1700,500" for _ in range(8)) + ",2000") is None


def test_preparation_bytes_per_element():
    assert bench.prep_bytes_per_elem(si.MXFP4) == 2.9375
    assert bench.prep_bytes_per_elem(si.NVFP4) == 3.0
    w = si.WORKLOADS["qkv_prefill"]
    assert w.m * w.k * bench.prep_bytes_per_elem(w.fmt) == 24641536     # 24.64 MB


@pytest.mark.parametrize("name,mb", [("qkv_prefill", 71.6), ("down_prefill", 92.3),
                                     ("decode_gate_up", 64.3)])
def test_gemm_bytes(name, mb):
    """A (2:4 codes 1/4, meta 1/8, residual 1/2, two scale arrays 1/32 B per
    element), W (1/2 + 1/32 B per element) and Y (4 B per output)."""
    w = si.WORKLOADS[name]
    a = w.m * w.k * (0.25 + 0.125 + 0.5 + 2 / 32)
    wb = w.n * w.k * (0.5 + 1 / 32)
    assert bench.gemm_bytes(w) == pytest.approx(a + wb + 4 * w.m * w.n)
    assert round(bench.gemm_bytes(w) / 1e6, 1) == mb


def test_openmp_oracle_build_gives_the_same_values():
    """The CPU baseline's build (-O3 -march=native -fopenmp, rows on threads)
    computes exactly what the test build computes."""
    import numpy as np

    import oracle
    L = oracle.omp_lib_built()
    assert L.oracle_threads(4) == 4
    for fmt, name in ((oracle.MXFP4, "tiny"), (oracle.NVFP4, "tiny")):
        w = si.WORKLOADS[name]
        x, W = si.workload_x(w, m=37), si.workload_w(w, n=70)
        g = si.gamma(w.k, 3)
        a = oracle.prepare(fmt, x, g, dense_backbone=True)
        b = oracle.prepare(fmt, x, g, dense_backbone=True, L=L)
        for key in a:
            assert np.array_equal(a[key], b[key]), key
        q = oracle.quantize_weight(fmt, W)
        assert np.array_equal(oracle.dual_gemm(fmt, a, q).view(np.uint32),
                              oracle.dual_gemm(fmt, a, q, L=L).view(np.uint32))


@pytest.mark.gpu
def test_bench_line_contract():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "20", "--warmup", "5"],
                       capture_output=True, text=True, cwd=ROOT, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    b = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in b, key
    assert b["n_gpus"] == 1 and b["steps"] == 20 and b["warmup"] == 5
    assert b["value"] > 0 and b["ms_per_step"] > 0
    assert b["config"]["workload"]
    r = b["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert r["bound"] == "mfma" and r["peak"] == 10100.0 and 0 < r["frac"] < 1
    c = b["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]
    assert c["single_thread"]["threads"] == 1 and c["all_threads"]["threads"] == c["cores"]
    assert c["nproc"] >= 1 and c["cpu_model"]
