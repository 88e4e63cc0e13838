"""GPU parity of local (sliding-window) attention: key j is visible to query i
only if i + Lk - Lq - left <= j <= i + Lk - Lq + right (a negative size leaves
that side open; causal is right = 0), mha_bwd's window_size_left / _right on
the backward call-trace page.  The HIP backward (three dQ modes) and forward
are compared with the fp64 CPU oracle's windowed forward / backward on the
same seeded inputs, to the same bars as the unwindowed parity tests; windows
that reach every key are checked bit-for-bit against no window."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import parity as PT
from tests.test_gpu_forward import _check as check_forward
from tests.test_gpu_parity import MODES

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


# Windows narrower and wider than the 64- and 128-row tiles, one- and
# two-sided, with Sq != Sk (bottom-right alignment), GQA groups, rows that
# see no key, and packed sequences of unequal and zero length.
WINDOWED = {
    "causal_left100_gqa2_d64": lambda: W.make_inputs(
        W.custom("w1", 2, 4, 2, 300, 300, 64, True, seed=201, window=(100, 0))),
    "two_sided_37_53_sq_lt_sk_d128": lambda: W.make_inputs(
        W.custom("w2", 1, 4, 1, 257, 390, 128, False, seed=202, window=(37, 53))),
    "right_only_20_noncausal_d128": lambda: W.make_inputs(
        W.custom("w3", 1, 2, 2, 200, 200, 128, False, seed=203, window=(-1, 20))),
    "narrow_3_5_d96": lambda: W.make_inputs(
        W.custom("w4", 1, 2, 1, 260, 260, 96, False, seed=204, window=(3, 5))),
    "causal_left30_sq_gt_sk_empty_rows_d128": lambda: W.make_inputs(
        W.custom("w5", 1, 4, 2, 400, 150, 128, True, seed=205, window=(30, 0))),
    "diagonal_and_previous_1_0_d64": lambda: W.make_inputs(
        W.custom("w6", 1, 2, 2, 190, 190, 64, False, seed=206, window=(1, 0))),
    "left_only_200_noncausal_gqa4_d128": lambda: W.make_inputs(
        W.custom("w7", 1, 8, 2, 520, 520, 128, False, seed=207, window=(200, -1))),
    "varlen_64_16_unequal_and_empty_d64": lambda: W.custom_varlen(
        "w8", [70, 0, 190, 33, 300], [130, 50, 190, 0, 280], 4, 2, 64, False, seed=208,
        window=(64, 16)),
    "varlen_causal_left90_d96": lambda: W.custom_varlen(
        "w9", [100, 257, 64], [100, 257, 64], 2, 2, 96, True, seed=209, window=(90, 0)),
    # the dQ pass puts the heads of a KV group in one workgroup under a left
    # window: eight heads of 32 rows each (MQA, ragged), and a group of six
    # split into three sets of two heads of 128 rows
    "causal_left70_mqa8_ragged_d128": lambda: W.make_inputs(
        W.custom("w12", 1, 8, 1, 333, 333, 128, True, seed=212, window=(70, 0))),
    "left50_right10_gqa6_sq_lt_sk_d128": lambda: W.make_inputs(
        W.custom("w13", 1, 12, 2, 200, 260, 128, False, seed=213, window=(50, 10))),
}


@pytest.fixture(scope="module")
def prepared():
    cache = {}

    def get(name):
        if name not in cache:
            cache[name] = PT.Prepared(WINDOWED[name]())
        return cache[name]
    return get


@pytest.mark.parametrize("name", list(WINDOWED))
@pytest.mark.parametrize("mode", list(MODES))
def test_window_backward_parity(gpu_lib, prepared, name, mode):
    _flush("window case %s mode=%s" % (name, mode))
    pr = prepared(name)
    acc, det = MODES[mode]
    res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(pr.inp.packed(res[key]), ref[key], "%s %s" % (name, key))
    flags = PT.ws_view(res, "flags", torch.int32, 4, (4,))
    assert int(flags[0]) == 0


@pytest.mark.parametrize("name", list(WINDOWED))
def test_window_forward_parity(gpu_lib, name):
    _flush("window forward %s" % name)
    inp = WINDOWED[name]()
    out, lse = PT.run_gpu_fwd(inp)
    check_forward(inp, out, lse, name)


@pytest.mark.parametrize("mode", list(MODES))
def test_diagonal_only_window(gpu_lib, mode):
    """Window (0, 0): each query sees its own key only, so P = 1 there, O = V,
    dS = P (dP - rowdot) = 0 (dP and rowdot are both dO . V), dQ = dK = 0
    up to rounding and dV = dO."""
    _flush("window (0, 0) mode=%s" % mode)
    inp = W.make_inputs(W.custom("w11", 1, 2, 2, 190, 190, 64, False, seed=211,
                                 window=(0, 0)))
    pr = PT.Prepared(inp)
    acc, det = MODES[mode]
    res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    ref = PT.oracle_backward(pr)
    assert np.abs(ref["dq"]).max() == 0 and np.abs(ref["dk"]).max() == 0
    for key in ("dq", "dk"):
        got = res[key].float()
        assert torch.isfinite(got).all() and got.abs().max() <= 1e-3, key
    PT.compare(pr.inp.packed(res["dv"]), pr.do64, "dv = dO")


@pytest.mark.parametrize("mode", ["separate", "ordered"])
def test_window_reproducible_modes_are_bit_identical(gpu_lib, prepared, mode):
    name = "two_sided_37_53_sq_lt_sk_d128"
    _flush("window repeat %s mode=%s" % (name, mode))
    pr = prepared(name)
    acc, det = MODES[mode]
    a = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    b = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    for key in ("dq", "dk", "dv"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key


def _without_window(inp, causal):
    """The same tensors under a workload without a window."""
    wl = inp.wl
    plain = W.Workload(wl.name + "_plain", wl.batch, wl.heads, wl.heads_k, wl.seqlen_q,
                       wl.seqlen_k, wl.head_dim, causal, varlen=wl.varlen, seed=wl.seed)
    return W.Inputs(plain, inp.q, inp.k, inp.v, inp.dout, inp.lens_q, inp.lens_k)


@pytest.mark.parametrize("causal,window", [(False, (1 << 30, 1 << 30)), (True, (5000, 0)),
                                           (False, (-1, 0))])
def test_windows_reaching_every_key_equal_the_plain_rules_bit_for_bit(gpu_lib, causal, window):
    """A window past every key is no window; (-1, 0) is the causal rule.  The
    kernels take the same tiles and the same masks then, so the outputs match
    bit for bit (forward and all three backward modes)."""
    _flush("window identity causal=%s window=%s" % (causal, window))
    inp_w = W.make_inputs(W.custom("w10", 1, 4, 2, 333, 333, 128, causal, seed=210,
                                   window=window))
    inp_p = _without_window(inp_w, causal or window == (-1, 0))
    ow, lw = PT.run_gpu_fwd(inp_w)
    op, lp = PT.run_gpu_fwd(inp_p)
    assert torch.equal(ow.view(torch.int16), op.view(torch.int16))
    assert torch.equal(lw, lp)
    pw, pp = PT.Prepared(inp_w), PT.Prepared(inp_p)
    for mode, (acc, det) in MODES.items():
        if mode == "atomic":
            continue   # unordered fp32 adds: not bit-reproducible
        a = PT.run_gpu(pw, deterministic=det, dq_accumulate=acc)
        b = PT.run_gpu(pp, deterministic=det, dq_accumulate=acc)
        for key in ("dq", "dk", "dv"):
            assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), (mode, key)


@pytest.mark.slow
def test_window_full_size_sampled_units(gpu_lib):
    """Batch 2, 32 query / 8 KV heads, 4096 x 4096, head_dim 128, causal with
    a 1024-key left window, in the launch configuration of the full-size
    runs: forward and backward of two (sequence, KV head) units against the
    oracle computed for those units alone."""
    _flush("window full size sampled units")
    base = W.WORKLOADS[3]
    wl = W.Workload("gqa_b2_h32_hk8_s4096_d128_causal_left1024", base.batch, base.heads,
                    base.heads_k, base.seqlen_q, base.seqlen_k, base.head_dim, True,
                    seed=base.seed, window=(1024, 0))
    inp = W.make_inputs(wl)
    PT.check_full_size_units(inp)
