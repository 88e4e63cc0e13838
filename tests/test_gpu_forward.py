"""GPU parity of the forward (O and LSE) against the fp64 CPU oracle's forward
on the same seeded inputs, through the C ABI.  Bar: max|O_gpu - O_ref| <=
1e-2 * max|O_ref| (bf16 output); LSE within 1e-3 absolute (fp32 sums of
exact products); rows without a visible key: O = 0 and LSE = -inf exactly;
repeated calls bit-identical; the GPU forward's outputs drive the GPU
backward to the backward's own parity bar."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import parity as PT
from tests.test_gpu_parity import SMALL
from oracle import oracle as O

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-3


def _flush(msg):
    print(msg, flush=True)


def _reference(inp):
    pk = lambda t: PT.to64(inp.packed(t))
    cu_q, cu_k = PT.cu_np(inp.lens_q), PT.cu_np(inp.lens_k)
    return O.forward(pk(inp.q), pk(inp.k), pk(inp.v), cu_q, cu_k, inp.wl.scale, inp.wl.causal,
                     window=inp.wl.window_sizes, softcap=inp.wl.softcap,
                     dropout=inp.wl.dropout_f32)


def _check(inp, out, lse, what):
    ref_o, ref_l = _reference(inp)
    got_o = PT.to64(inp.packed(out))
    got_l = PT.lse_rows(inp, lse)
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty), "%s: rows with -inf LSE differ" % what
    assert np.isfinite(got_l[~empty]).all(), "%s: non-finite LSE" % what
    if (~empty).any():
        err = np.abs(got_l[~empty] - ref_l[~empty]).max()
        assert err <= LSE_TOL, "%s: LSE max err %.3e" % (what, err)
    # rows without a visible key: O exactly 0
    assert (got_o[empty] == 0).all(), "%s: O of empty rows is not 0" % what
    PT.compare(inp.packed(out), ref_o, "%s O" % what)


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small_parity(gpu_lib, name):
    _flush("forward case %s" % name)
    inp = SMALL[name]()
    out, lse = PT.run_gpu_fwd(inp)
    _check(inp, out, lse, name)


@pytest.mark.parametrize("name", ["dense_causal_ragged_gqa2_d64", "varlen_d96_causal"])
def test_forward_is_bit_identical_across_calls(gpu_lib, name):
    _flush("forward repeat %s" % name)
    inp = SMALL[name]()
    a = PT.run_gpu_fwd(inp)
    b = PT.run_gpu_fwd(inp)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_forward_extreme_scores_stay_finite(gpu_lib):
    # Large scores (x30) and a row whose maximum grows late: the lazy
    # rescale must keep P bounded and the result exact.
    wl = W.custom("fx", 1, 2, 1, 200, 300, 64, False, seed=111)
    inp = W.make_inputs(wl)
    inp.q = (inp.q.float() * 30).to(torch.bfloat16)
    inp.k[0, 290:, 0, :] = (inp.k[0, 290:, 0, :].float() * 4).to(torch.bfloat16)
    out, lse = PT.run_gpu_fwd(inp)
    _check(inp, out, lse, "extreme")


@pytest.mark.parametrize("name", ["dense_causal_ragged_gqa2_d64", "varlen_unequal_and_empty_causal_d64",
                                  "noncausal_gqa4_d128"])
def test_gpu_forward_feeds_gpu_backward(gpu_lib, name):
    """O and LSE from the GPU forward as the backward's inputs: gradients
    to the backward's parity bar against the oracle."""
    _flush("forward->backward %s" % name)
    inp = SMALL[name]()
    out, lse = PT.run_gpu_fwd(inp)
    pr = PT.Prepared(inp)
    pr.o = out
    pr.o64 = PT.to64(inp.packed(out))
    pr.lse = torch.nan_to_num(lse, nan=float("-inf"))
    res = PT.run_gpu(pr)
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(pr.inp.packed(res[key]), ref[key], "%s %s" % (name, key))


@pytest.mark.slow
def test_forward_headline_size_sampled_heads(gpu_lib):
    """B=2, H=32, Hk=8, S=4096, D=128 causal, in the benchmark's launch
    configuration; the oracle checks two (batch, head) units."""
    wl = W.WORKLOADS[3]
    inp = W.make_inputs(wl)
    _flush("forward headline size")
    out, lse = PT.run_gpu_fwd(inp)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    for b, h in ((0, 5), (1, 30)):
        g = h // (wl.heads // wl.heads_k)
        q = PT.to64(inp.q[b, :, [h]])
        k = PT.to64(inp.k[b, :, [g]])
        v = PT.to64(inp.v[b, :, [g]])
        cu = np.array([0, wl.seqlen_q], np.int64)
        ref_o, ref_l = O.forward(q, k, v, cu, np.array([0, wl.seqlen_k], np.int64), wl.scale,
                                 wl.causal)
        PT.compare(out[b, :, [h]], ref_o, "headline O b%d h%d" % (b, h))
        err = np.abs(lse[b, h].numpy().astype(np.float64) - ref_l[:, 0]).max()
        assert err <= LSE_TOL, "headline LSE b%d h%d err %.3e" % (b, h, err)
