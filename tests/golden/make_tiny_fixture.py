"""Write tests/golden/tiny_oracle.npz from the oracle (no GPU code involved).

Run from the repository root: python tests/golden/make_tiny_fixture.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth_inputs as si  # noqa: E402


def main():
    w = si.WORKLOADS["tiny"]
    x = si.workload_x(w)
    W = si.workload_w(w)
    g = si.workload_gamma(w)
    p = oracle.prepare(oracle.MXFP4, x, g, dense_backbone=True)
    q = oracle.quantize_weight(oracle.MXFP4, W)
    y = oracle.dual_gemm(oracle.MXFP4, p, q)
    out = {"x": x, "w": W, "gamma": g, "y": y}
    out.update({"prep_" + k: v for k, v in p.items()})
    out.update({"wq_" + k: v for k, v in q.items()})
    np.savez_compressed(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.npz"), **out)


if __name__ == "__main__":
    main()
