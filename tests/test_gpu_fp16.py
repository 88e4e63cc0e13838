"""fp16 I/O: the same kernels instantiated for fp16 elements, against the fp64
oracle on fp16-rounded inputs (bar as for bf16: per tensor max|gpu - ref| <=
1e-2 * max|ref|; forward LSE within 1e-3)."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import parity as PT
from tests.test_gpu_forward import _check as check_forward

pytestmark = pytest.mark.gpu

F16 = torch.float16

CASES = {
    "dense_causal_ragged_gqa2_d64": lambda: W.make_inputs(
        W.custom("h1", 2, 4, 2, 200, 200, 64, True, seed=201), dtype=F16),
    "causal_sq_gt_sk_empty_rows_d128": lambda: W.make_inputs(
        W.custom("h2", 1, 4, 2, 300, 130, 128, True, seed=202), dtype=F16),
    "noncausal_mqa_d96": lambda: W.make_inputs(
        W.custom("h3", 1, 4, 1, 150, 260, 96, False, seed=203), dtype=F16),
    "varlen_unequal_and_empty_causal_d128": lambda: W.custom_varlen(
        "h4", [70, 0, 190, 33], [130, 50, 190, 0], 4, 2, 128, True, seed=204, dtype=F16),
}
MODES = {"separate": (False, False), "atomic": (True, False), "ordered": (True, True)}


def _flush(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", list(MODES))
def test_fp16_backward_parity(gpu_lib, name, mode):
    _flush("fp16 backward %s %s" % (name, mode))
    inp = CASES[name]()
    assert inp.q.dtype == F16
    pr = PT.Prepared(inp)
    acc, det = MODES[mode]
    res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    assert res["dq"].dtype == F16
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(inp.packed(res[key]), ref[key], "fp16 %s %s %s" % (name, mode, key))


@pytest.mark.parametrize("name", list(CASES))
def test_fp16_forward_parity(gpu_lib, name):
    _flush("fp16 forward %s" % name)
    inp = CASES[name]()
    out, lse = PT.run_gpu_fwd(inp)
    assert out.dtype == F16
    check_forward(inp, out, lse, "fp16 " + name)


def test_fp16_and_bf16_inputs_of_equal_values_agree(gpu_lib):
    """Inputs whose values are exact in both formats: the two instantiations
    compute the same quantities and agree to the output rounding."""
    inp = W.make_inputs(W.custom("h5", 1, 2, 2, 130, 130, 64, True, seed=205))
    inp16 = W.Inputs(inp.wl, inp.q.to(F16), inp.k.to(F16), inp.v.to(F16), inp.dout.to(F16),
                     inp.lens_q, inp.lens_k)
    o_b, l_b = PT.run_gpu_fwd(inp)
    o_h, l_h = PT.run_gpu_fwd(inp16)
    assert np.abs(PT.lse_rows(inp, l_b) - PT.lse_rows(inp16, l_h)).max() <= 1e-4
    scale = o_b.float().abs().max()
    assert (o_b.float() - o_h.float()).abs().max() <= 1e-2 * scale
