"""GPU parity at head dims above 128 (padded widths 192 and 256): the dQ and
forward kernels run four waves of 32 rows with two K/V buffers, the key-tile
kernel 64 keys per workgroup with each pair of waves splitting the head dim
of dK and dV.  Compared with the fp64 CPU oracle on the same seeded inputs to
the bars of the other parity tests (the default dQ pass; the fused dQ modes
are built for head_dim <= 128 only and are rejected above)."""
import numpy as np
import pytest
import torch

import attention_backward_fa2_amd as fa
import workloads as W
from tests import parity as PT
from tests.test_gpu_forward import _check as check_forward

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


BIGD = {
    "d256_causal_gqa2_ragged": lambda: W.make_inputs(
        W.custom("h1", 2, 4, 2, 200, 200, 256, True, seed=501)),
    "d192_noncausal_sq_lt_sk": lambda: W.make_inputs(
        W.custom("h2", 1, 2, 1, 130, 300, 192, False, seed=502)),
    "d160_padded_causal_sq_gt_sk_empty_rows": lambda: W.make_inputs(
        W.custom("h3", 1, 4, 2, 300, 130, 160, True, seed=503)),
    "d232_padded_noncausal": lambda: W.make_inputs(
        W.custom("h4", 1, 2, 2, 150, 150, 232, False, seed=504)),
    "d256_varlen_unequal_and_empty_causal": lambda: W.custom_varlen(
        "h5", [70, 0, 190, 33], [130, 50, 190, 0], 4, 2, 256, True, seed=505),
    "d256_window_cap_dropout": lambda: W.make_inputs(
        W.custom("h6", 1, 4, 2, 260, 260, 256, False, seed=506, window=(70, 20),
                 softcap=2.0, dropout=(0.25, 99, 4))),
    "d192_fp16_causal": lambda: W.make_inputs(
        W.custom("h7", 1, 4, 4, 192, 192, 192, True, seed=507), dtype=torch.float16),
}


@pytest.fixture(scope="module")
def prepared():
    cache = {}

    def get(name):
        if name not in cache:
            cache[name] = PT.Prepared(BIGD[name]())
        return cache[name]
    return get


@pytest.mark.parametrize("name", list(BIGD))
def test_big_head_dim_backward_parity(gpu_lib, prepared, name):
    _flush("head dim case %s" % name)
    pr = prepared(name)
    res = PT.run_gpu(pr)
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(pr.inp.packed(res[key]), ref[key], "%s %s" % (name, key))


@pytest.mark.parametrize("name", list(BIGD))
def test_big_head_dim_forward_parity(gpu_lib, name):
    _flush("head dim forward %s" % name)
    inp = BIGD[name]()
    out, lse = PT.run_gpu_fwd(inp)
    check_forward(inp, out, lse, name)


def test_big_head_dim_is_bit_reproducible(gpu_lib, prepared):
    pr = prepared("d256_causal_gqa2_ragged")
    a, b = PT.run_gpu(pr), PT.run_gpu(pr)
    for key in ("dq", "dk", "dv"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key


def test_columns_past_a_padded_head_dim_untouched(gpu_lib, prepared):
    """head_dim 232 runs at width 256: outputs with a wider row pitch keep
    their columns past 232 (they start as NaN)."""
    pr = prepared("d232_padded_noncausal")
    res = PT.run_gpu(pr, out_pad=24)
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        buf = res[key + "_buf"]
        assert torch.isnan(buf[..., 232:].float()).all(), key
        PT.compare(pr.inp.packed(res[key]), ref[key], "padded " + key)


@pytest.mark.slow
@pytest.mark.parametrize("head_dim", [256, 192])
def test_big_head_dim_full_size_sampled_units(gpu_lib, head_dim):
    """Batch 2, 32 query / 8 KV heads, 4096 x 4096, causal, head_dim 256 and
    192, in the launch configuration the benchmark times: GPU forward, then
    the GPU backward on its O and LSE, two (sequence, KV head) units against
    the oracle computed for them alone."""
    _flush("head_dim %d full size sampled units" % head_dim)
    base = W.WORKLOADS[3]
    wl = W.Workload("gqa_b2_h32_hk8_s4096_d%d_causal" % head_dim, base.batch, base.heads,
                    base.heads_k, base.seqlen_q, base.seqlen_k, head_dim, True,
                    seed=base.seed)
    PT.check_full_size_units(W.make_inputs(wl))
