"""sharq_prepare_noalloc (the preparation for callers that cannot allocate)
against sharq_prepare, through the C ABI (needs an MI355X).

Two calls in a row, the second on a smaller input: every output byte and the
NVFP4 tensor scale must equal sharq_prepare's on the same input; the
caller's tensor_scale[1] is left untouched (the amax lives in the library's
static workspace), and the second call does not see the first call's amax.
"""
import numpy as np
import pytest

import synth_inputs as si

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsity_fp4_quantized_amd as sq  # noqa: E402

DEV = "cuda:0"


def _run(fmt, x, g, noalloc, layout):
    m, k = x.shape
    sp, rs = sq.alloc_prepared(fmt, m, k, DEV, dense_backbone=True, layout=layout)
    if fmt == sq.NVFP4:
        sp.tensor_scale.fill_(-7.0)            # a sentinel in both slots
        rs.tensor_scale = sp.tensor_scale
    xt = torch.from_numpy(x.view(np.int16)).to(DEV)
    gt = None if g is None else torch.from_numpy(g.view(np.int16)).to(DEV)
    sq.bind_prepare(xt, gt, 1e-5, sp, rs, noalloc=noalloc)()
    torch.cuda.synchronize()
    out = {name: t.cpu().numpy() for name, t in (("codes", sp.codes), ("meta", sp.meta), ("scales", sp.scales),
                                                  ("dense", sp.dense_codes), ("r_codes", rs.codes),
                                                  ("r_scales", rs.scales))}
    if fmt == sq.NVFP4:
        out["tensor_scale"] = sp.tensor_scale.cpu().numpy()
    return out


@pytest.mark.parametrize("fmt,norm", [(sq.NVFP4, True), (sq.NVFP4, False), (sq.MXFP4, True)])
@pytest.mark.parametrize("layout", [sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR])
def test_prepare_noalloc_matches_prepare(fmt, norm, layout):
    # the first input's amax is much larger than the second's: a workspace
    # left holding it would give the second call the wrong tensor scale
    big = si.activations("student_t4", 300, 1024, 10, 50.0, seed=71)
    small = si.activations("normal", 37, 512, 0, 1.0, seed=72)
    for step, x in enumerate((big, small)):
        k = x.shape[1]
        g = si.gamma(k, seed=k) if norm else None
        want = _run(fmt, x, g, False, layout)
        got = _run(fmt, x, g, True, layout)
        for name in want:
            if name == "tensor_scale":
                continue
            assert np.array_equal(got[name], want[name]), (step, name)
        if fmt == sq.NVFP4:
            assert got["tensor_scale"][0] == want["tensor_scale"][0], step
            assert got["tensor_scale"][1] == np.float32(-7.0), step      # not used as scratch
            assert want["tensor_scale"][1] != np.float32(-7.0), step     # sharq_prepare's amax slot
