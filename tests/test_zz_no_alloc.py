"""fa_bwd_noalloc (the backward on the library's own scratch array, for
callers that cannot allocate) against fa_bwd with a caller-owned workspace:
the same kernels, so dQ, dK and dV must be bit-identical (and within the
oracle bar).  Two calls in a row, the second on a smaller input, so the
second runs on the scratch the first left behind."""
import ctypes

import pytest
import torch

import attention_backward_fa2_amd as fa
import workloads as W
from tests import parity as PT

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _run(pr, entry, dq_accumulate=False, deterministic=False):
    """Backward through the C ABI entry point `entry` ('all' = fa_bwd with a
    fresh NaN-filled workspace, 'noalloc' = fa_bwd_noalloc)."""
    inp, wl = pr.inp, pr.inp.wl
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.dout))
    o, lse = pr.o.to(dev).contiguous(), pr.lse.to(dev).contiguous()
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    kw = {}
    if wl.varlen:
        kw = dict(cu_seqlens_q=torch.tensor(pr.cu_q, dtype=torch.int32, device=dev),
                  cu_seqlens_k=torch.tensor(pr.cu_k, dtype=torch.int32, device=dev),
                  max_seqlen_q=max(inp.lens_q), max_seqlen_k=max(inp.lens_k))
    args = fa.make_args(do, q, k, v, o, lse, dq, dk, dv, wl.scale, wl.causal,
                        deterministic=deterministic, dq_accumulate=dq_accumulate,
                        window=wl.window, softcap=wl.softcap, dropout=wl.dropout, **kw)
    if entry == "all":
        ws = fa.alloc_workspace(args, dev)
        ws.fill_(0xA5)
    else:
        assert args.workspace is None or args.workspace == 0
    fa.run(args, entry)
    torch.cuda.synchronize()
    return {"dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}


CASES = [
    # (name, inputs, modes); each case is followed by a smaller one
    ("causal_gqa4_ragged_d128", lambda: W.make_inputs(
        W.custom("na1", 2, 8, 2, 700, 900, 128, True, seed=301))),
    ("varlen_unequal_and_empty_d64", lambda: W.custom_varlen(
        "na2", [70, 0, 190, 33], [130, 50, 190, 0], 4, 2, 64, True, seed=302)),
    ("dropout_window_d96", lambda: W.make_inputs(
        W.custom("na3", 1, 4, 4, 260, 300, 96, True, seed=303, window=(120, 0),
                 dropout=(0.2, 77, 5)))),
    ("small_noncausal_d64", lambda: W.make_inputs(
        W.custom("na4", 1, 2, 1, 65, 70, 64, False, seed=304))),
]
MODES = [("separate", False, False), ("ordered", True, True)]


def test_noalloc_matches_fa_bwd_on_calls_in_a_row(gpu_lib):
    """Each case in turn (largest first, then smaller ones) through both entry
    points and both reproducible dQ modes: bit-identical outputs."""
    lib = gpu_lib.load_library()
    assert hasattr(lib, "fa_bwd_noalloc")
    for name, make in CASES:
        pr = PT.Prepared(make())
        ref = PT.oracle_backward(pr)
        for mode, acc, det in MODES:
            if pr.inp.wl.dropout is not None and acc:
                continue   # (accumulate mode draws the keep bits in both entry points)
            _flush("noalloc case %s mode %s" % (name, mode))
            a = _run(pr, "all", acc, det)
            b = _run(pr, "noalloc", acc, det)
            for key in ("dq", "dk", "dv"):
                assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), (
                    name, mode, key)
                PT.compare(pr.inp.packed(b[key]), ref[key], "%s %s %s" % (name, mode, key))


def test_noalloc_rejects_a_workspace_beyond_its_scratch(gpu_lib):
    """A call that would need more than the scratch array is refused (and
    nothing is written)."""
    dev = torch.device("cuda")
    B, S, H, Hk, D = 4, 2048, 16, 4, 128   # accumulate mode: 4*2048*16*128*4 B > 64 MiB
    q = torch.zeros(B, S, H, D, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(B, S, Hk, D, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(B, H, S, dtype=torch.float32, device=dev)
    dq = torch.full_like(q, float("nan"))
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(k, float("nan"))
    args = fa.make_args(q, q, k, k, q, lse, dq, dk, dv, D ** -0.5, True, dq_accumulate=True)
    assert fa.workspace_size(args) > (64 << 20)
    lib = fa.load_library()
    assert lib.fa_bwd_noalloc(ctypes.byref(args), None) == fa.FA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(dq.float()).all() and torch.isnan(dk.float()).all()
