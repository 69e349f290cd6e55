"""Oracle against the hand-derived worked examples and the stored tiny fixture."""
import os

import numpy as np
import pytest

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            d[key] = val.split()
    return d


@pytest.mark.parametrize("name,fmt", [("worked_block_mxfp4.txt", oracle.MXFP4),
                                      ("worked_block_nvfp4.txt", oracle.NVFP4)])
def test_worked_example(name, fmt):
    d = _load(name)
    x = np.array([float(v) for v in d["x"]], np.float32)[None, :]
    xb = si.f32_to_bf16_bits(x)
    assert (si.bf16_bits_to_f32(xb) == x).all()       # exact in bf16
    p = oracle.prepare(fmt, xb, None)
    for key in ["meta", "s_codes", "s_scales", "r_codes", "r_scales"]:
        want = np.array([int(v, 16) for v in d[key]], np.uint8)
        assert (p[key][0] == want).all(), (key, p[key][0], want)
    if "tensor_scale" in d:
        assert p["tensor_scale"][0] == np.float32(float(d["tensor_scale"][0]))


def test_tiny_fixture_regression():
    ref = np.load(os.path.join(GOLDEN, "tiny_oracle.npz"))
    w = si.WORKLOADS["tiny"]
    x = si.workload_x(w)
    assert (x == ref["x"]).all() and (si.workload_w(w) == ref["w"]).all()
    p = oracle.prepare(oracle.MXFP4, x, si.workload_gamma(w), dense_backbone=True)
    for k, v in p.items():
        assert (v == ref["prep_" + k]).all(), k
    q = oracle.quantize_weight(oracle.MXFP4, ref["w"])
    for k, v in q.items():
        assert (v == ref["wq_" + k]).all(), k
    assert (oracle.dual_gemm(oracle.MXFP4, p, q) == ref["y"]).all()
