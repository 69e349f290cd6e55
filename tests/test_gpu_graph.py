"""The preparation and the dual GEMM captured in a HIP graph (needs an MI355X).

The library allocates nothing, never synchronizes and clears nothing with a
memory-set command (the NVFP4 tensor amax is cleared by a kernel), so a
caller can capture its calls.  Both formats: the step (prepare, then the
dual GEMM) for two buffer sets is captured once through the bound calls on a
side stream and replayed several times, with eager work and a
synchronization between replays (each replay's outputs cleared first); every
replay must give exactly the eager outputs, and the eager outputs are the
oracle's (codes byte for byte, the GEMM within its bound) so that the graph is
checked against the pages' arithmetic, not only against itself.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from gemm_check import check_gemm
from test_gpu_parity import _compare_prep

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsity_fp4_quantized_amd as sq  # noqa: E402

DEV = "cuda:0"


def _arrays(sp, rs):
    out = {"codes": sp.codes, "meta": sp.meta, "scales": sp.scales, "dense": sp.dense_codes,
           "r_codes": rs.codes, "r_scales": rs.scales}
    if sp.fmt == sq.NVFP4:
        out["tensor_scale"] = sp.tensor_scale
    return out


@pytest.mark.parametrize("fmt", [sq.MXFP4, sq.NVFP4])
def test_prepare_and_dual_gemm_in_a_graph(fmt):
    m, k, n, sets = 200, 1024, 384, 2
    side = torch.cuda.Stream()
    cases = []
    for i in range(sets):
        x = si.activations("student_t4", m, k, 12, 40.0, 151 + i)
        g = si.gamma(k, 161 + i)
        W = si.weights(n, k, 171 + i)
        xt = torch.from_numpy(x.view(np.int16)).to(DEV)
        gt = torch.from_numpy(g.view(np.int16)).to(DEV)
        wq = sq.quantize_weight(torch.from_numpy(W.view(np.int16)).to(DEV), fmt)
        sp, rs = sq.alloc_prepared(fmt, m, k, DEV, dense_backbone=True)
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        calls = (sq.bind_prepare(xt, gt, 1e-5, sp, rs, stream=side), sq.bind_dual_gemm(sp, rs, wq, y, stream=side))
        cases.append((x, g, W, sp, rs, y, calls))
    torch.cuda.synchronize()

    def step():
        for (_, _, _, _, _, _, (prep, gemm)) in cases:
            prep()
            gemm()

    # eager reference, checked against the oracle
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    eager = []
    for (x, g, W, sp, rs, y, _) in cases:
        ref = oracle.prepare(fmt, x, g, dense_backbone=True)
        q = oracle.quantize_weight(fmt, W)
        _compare_prep(f"graph eager fmt {fmt}", sp, rs, ref)
        got = {name: t.cpu().numpy() for name, t in _arrays(sp, rs).items()}
        yref, yabs = oracle.dual_gemm_bound(fmt, ref, q)
        check_gemm(y.cpu().numpy(), yref, yabs, k, f"graph eager fmt {fmt}")
        eager.append((got, y.clone()))

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()

    for replay in range(3):
        for (_, _, _, sp, rs, y, _) in cases:      # eager work between replays
            for t in _arrays(sp, rs).values():
                t.zero_()
            y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (got0, y0), (_, _, _, sp, rs, y, _) in zip(eager, cases):
            for name, t in _arrays(sp, rs).items():
                assert np.array_equal(t.cpu().numpy(), got0[name]), (replay, name)
            assert torch.equal(y, y0), replay
