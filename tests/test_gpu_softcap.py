"""GPU parity of soft-capped scores: every scaled score x becomes c * tanh(x / c)
before the softmax and the gradients pass the cap by the chain rule (mha_bwd's
softcap on the backward call-trace page).  The HIP backward (three dQ modes)
and forward are compared with the fp64 CPU oracle on the same seeded inputs,
to the bars of the unwindowed parity tests (gradients and O within 1e-2 of
max|ref|, LSE within 1e-3), with caps small enough that tanh is far from
linear over the scores (N(0,1) inputs give scaled scores of about unit size).
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import parity as PT
from tests.test_gpu_forward import _check as check_forward
from tests.test_gpu_parity import MODES
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


CAPPED = {
    "causal_gqa2_d128_cap1": lambda: W.make_inputs(
        W.custom("s1", 2, 4, 2, 200, 200, 128, True, seed=301, softcap=1.0)),
    "noncausal_sq_lt_sk_d64_cap0.5": lambda: W.make_inputs(
        W.custom("s2", 1, 4, 1, 130, 300, 64, False, seed=302, softcap=0.5)),
    "causal_sq_gt_sk_empty_rows_d128_cap2": lambda: W.make_inputs(
        W.custom("s3", 1, 4, 2, 300, 130, 128, True, seed=303, softcap=2.0)),
    "headdim72_padded_noncausal_cap3": lambda: W.make_inputs(
        W.custom("s4", 1, 2, 2, 150, 150, 72, False, seed=304, softcap=3.0)),
    "varlen_causal_left64_d96_cap1.5": lambda: W.custom_varlen(
        "s5", [100, 257, 0, 64], [100, 257, 30, 64], 2, 2, 96, True, seed=305,
        window=(64, 0), softcap=1.5),
    "two_sided_window_d128_cap0.8": lambda: W.make_inputs(
        W.custom("s6", 1, 4, 2, 260, 260, 128, False, seed=306, window=(40, 30),
                 softcap=0.8)),
}


@pytest.fixture(scope="module")
def prepared():
    cache = {}

    def get(name):
        if name not in cache:
            cache[name] = PT.Prepared(CAPPED[name]())
        return cache[name]
    return get


@pytest.mark.parametrize("name", list(CAPPED))
@pytest.mark.parametrize("mode", list(MODES))
def test_softcap_backward_parity(gpu_lib, prepared, name, mode):
    _flush("softcap case %s mode=%s" % (name, mode))
    pr = prepared(name)
    acc, det = MODES[mode]
    res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(pr.inp.packed(res[key]), ref[key], "%s %s" % (name, key))
    flags = PT.ws_view(res, "flags", torch.int32, 4, (4,))
    assert int(flags[0]) == 0


@pytest.mark.parametrize("name", list(CAPPED))
def test_softcap_forward_parity(gpu_lib, name):
    _flush("softcap forward %s" % name)
    inp = CAPPED[name]()
    out, lse = PT.run_gpu_fwd(inp)
    check_forward(inp, out, lse, name)


def test_cap_changes_the_result(gpu_lib, prepared):
    """The capped gradients differ from the uncapped ones by far more than the
    parity bar, so the parity tests above could not pass without the cap."""
    pr = prepared("causal_gqa2_d128_cap1")
    ref_cap = PT.oracle_backward(pr)
    plain = O.backward(pr.q64, pr.k64, pr.v64, pr.do64, pr.cu_q, pr.cu_k,
                       pr.inp.wl.scale, True)
    for key in ("dq", "dk"):
        diff = np.abs(ref_cap[key] - plain[key]).max()
        assert diff > 0.2 * np.abs(ref_cap[key]).max(), key


def test_tiny_cap_is_uniform_attention(gpu_lib):
    """c = 1e-20: the kernels' tanh input factor saturates at the fp32 maximum,
    every capped score is 0 to within c, so each row attends uniformly to the
    keys it sees (O = their mean V), dQ = dK = 0 and dV = P^T dO; the oracle
    agrees on the same inputs."""
    _flush("softcap tiny cap")
    inp = W.make_inputs(W.custom("s7", 1, 2, 1, 140, 140, 64, True, seed=307, softcap=1e-20))
    out, lse = PT.run_gpu_fwd(inp)
    check_forward(inp, out, lse, "tiny cap")
    pr = PT.Prepared(inp)
    res = PT.run_gpu(pr)
    for key in ("dq", "dk"):
        got = res[key].float()
        assert torch.isfinite(got).all() and got.abs().max() <= 1e-3, key
    ref = PT.oracle_backward(pr)
    PT.compare(pr.inp.packed(res["dv"]), ref["dv"], "tiny cap dv")


@pytest.mark.parametrize("mode", ["separate", "ordered"])
def test_softcap_reproducible_modes_are_bit_identical(gpu_lib, prepared, mode):
    name = "two_sided_window_d128_cap0.8"
    _flush("softcap repeat %s mode=%s" % (name, mode))
    pr = prepared(name)
    acc, det = MODES[mode]
    a = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    b = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    for key in ("dq", "dk", "dv"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key


@pytest.mark.slow
def test_softcap_full_size_sampled_units(gpu_lib):
    """Batch 2, 32 query / 8 KV heads, 4096 x 4096, head_dim 128, causal, cap
    50 on the scores: GPU forward, then the GPU backward on its O and LSE, two
    (sequence, KV head) units against the oracle computed for them alone."""
    _flush("softcap full size sampled units")
    base = W.WORKLOADS[3]
    wl = W.Workload("gqa_b2_h32_hk8_s4096_d128_causal_cap50", base.batch, base.heads,
                    base.heads_k, base.seqlen_q, base.seqlen_k, base.head_dim, True,
                    seed=base.seed, softcap=50.0)
    inp = W.make_inputs(wl)
    # large scores so that a cap of 50 bends them: Q scaled by 30 (exact in bf16
    # up to rounding of the product, done on the CPU before the upload)
    inp = W.Inputs(wl, (inp.q.float() * 30).to(torch.bfloat16), inp.k, inp.v, inp.dout,
                   inp.lens_q, inp.lens_k)
    PT.check_full_size_units(inp)
