"""Helpers that run the HIP path and the CPU oracle on the same seeded inputs.

The oracle's fp64 forward supplies the backward's O (rounded to bf16) and LSE
(rounded to fp32); its fp64 backward supplies the expected gradients.  The
HIP path is called through the C ABI (python binding) only.
"""
import numpy as np
import torch

import attention_backward_fa2_amd as fa
import workloads as W
from oracle import oracle as O

# Parity bar for bf16 I/O: per gradient tensor, max |gpu - ref| <= TOL * max |ref|.
TOL = 1e-2


def to64(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp16 -> fp64, exact."""
    return t.float().numpy().astype(np.float64)


def cu_np(lens):
    return np.cumsum([0] + [int(x) for x in lens]).astype(np.int64)


class Prepared:
    """Inputs plus the oracle forward's O / LSE in the GPU's layouts."""

    def __init__(self, inp: W.Inputs):
        self.inp = inp
        wl = inp.wl
        self.cu_q, self.cu_k = cu_np(inp.lens_q), cu_np(inp.lens_k)
        self.q64 = to64(inp.packed(inp.q))
        self.k64 = to64(inp.packed(inp.k))
        self.v64 = to64(inp.packed(inp.v))
        self.do64 = to64(inp.packed(inp.dout))
        out, lse = O.forward(self.q64, self.k64, self.v64, self.cu_q, self.cu_k, wl.scale,
                             wl.causal, window=wl.window_sizes, softcap=wl.softcap,
                             dropout=wl.dropout_f32)
        self.o64_exact = out                      # [total_q, H, D] fp64
        self.lse_rows = lse                       # [total_q, H] fp64
        self.o = torch.from_numpy(out).to(inp.q.dtype).reshape(inp.q.shape)
        self.o64 = to64(inp.packed(self.o))
        nseq, H = len(inp.lens_q), wl.heads
        maxq = max(inp.lens_q) if inp.lens_q else 0
        L = np.full((nseq, H, maxq), -np.inf, np.float32)
        for s in range(nseq):
            L[s, :, :inp.lens_q[s]] = lse[self.cu_q[s]:self.cu_q[s + 1]].T
        self.lse = torch.from_numpy(L)            # (B|nseq, H, Sq|max) fp32

    @property
    def varlen(self):
        return self.inp.wl.varlen


def run_gpu(pr: Prepared, deterministic=False, out_pad=0, step_split=False, dq_accumulate=False,
            steps=None, keep_max=0, keep_words=None):
    """Backward on cuda:0.  Outputs start as NaN so unwritten elements show.
    out_pad > 0 gives dq/dk/dv a row pitch of head_dim + out_pad (strided
    views) to check that columns past head_dim are left alone.  keep_words:
    a forward call's dropout keep words (device tensor) for the backward to
    read."""
    inp, wl = pr.inp, pr.inp.wl
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.dout))
    o = pr.o.to(dev).contiguous()
    lse = pr.lse.to(dev).contiguous()

    def out_like(t):
        shp = list(t.shape)
        shp[-1] += out_pad
        buf = torch.full(shp, float("nan"), dtype=t.dtype, device=dev)
        return buf[..., :t.shape[-1]], buf

    (dq, dq_buf), (dk, dk_buf), (dv, dv_buf) = out_like(q), out_like(k), out_like(v)
    kw = {}
    if wl.varlen:
        kw = dict(cu_seqlens_q=torch.tensor(pr.cu_q, dtype=torch.int32, device=dev),
                  cu_seqlens_k=torch.tensor(pr.cu_k, dtype=torch.int32, device=dev),
                  max_seqlen_q=max(inp.lens_q), max_seqlen_k=max(inp.lens_k))
    args = fa.make_args(do, q, k, v, o, lse, dq, dk, dv, wl.scale, wl.causal,
                        deterministic=deterministic, dq_accumulate=dq_accumulate,
                        window=wl.window, softcap=wl.softcap, dropout=wl.dropout,
                        dropout_keep_max_bytes=keep_max, dropout_keep=keep_words, **kw)
    ws = fa.alloc_workspace(args, dev)
    ws.fill_(0xA5)   # garbage: the preprocess must clear what it uses
    if steps is not None:
        for step in steps:
            fa.run(args, step)
    elif step_split:
        # separate mode: dq before main (with dropout main reads the keep
        # bits dq writes)
        for step in (("preprocess", "main", "dq_convert") if dq_accumulate else
                     ("preprocess", "dq", "main")):
            fa.run(args, step)
    else:
        fa.run(args, "all")
    torch.cuda.synchronize()
    lay = fa.workspace_layout(args)
    return dict(dq=dq.cpu(), dk=dk.cpu(), dv=dv.cpu(), dq_buf=dq_buf.cpu(),
                dk_buf=dk_buf.cpu(), dv_buf=dv_buf.cpu(), ws=ws.cpu(), layout=lay,
                args=args)


def ws_view(res, name, dtype, count, shape):
    off = getattr(res["layout"], "off_" + name)
    raw = res["ws"][off:off + count * torch.tensor([], dtype=dtype).element_size()]
    return raw.view(dtype).reshape(shape)


def compare(gpu: torch.Tensor, ref: np.ndarray, what: str, tol=TOL):
    g = gpu.float().numpy().astype(np.float64).reshape(ref.shape)
    assert np.isfinite(g).all(), "%s: non-finite values (unwritten or NaN)" % what
    scale = np.abs(ref).max()
    err = np.abs(g - ref).max()
    assert err <= tol * scale, "%s: max err %.3e > %.0e * max|ref| (%.3e)" % (
        what, err, tol, scale)
    return err / scale if scale > 0 else 0.0


def oracle_backward(pr: Prepared):
    wl = pr.inp.wl
    return O.backward(pr.q64, pr.k64, pr.v64, pr.do64, pr.cu_q, pr.cu_k, wl.scale, wl.causal,
                      window=wl.window_sizes, softcap=wl.softcap, dropout=wl.dropout_f32)


def oracle_backward_unit(pr: Prepared, s: int, g: int):
    """Exact gradients of sequence s and KV head g alone (the query heads of
    its group), as (rows_q, heads, rows_k, ref) for sampled comparisons (with
    dropout, the unit replays the keep bits of its place in the whole call)."""
    wl = pr.inp.wl
    G = wl.heads // wl.heads_k
    heads = list(range(g * G, (g + 1) * G))
    qs, qe = pr.cu_q[s], pr.cu_q[s + 1]
    ks, ke = pr.cu_k[s], pr.cu_k[s + 1]
    ref = O.backward(pr.q64[qs:qe][:, heads], pr.k64[ks:ke][:, [g]], pr.v64[ks:ke][:, [g]],
                     pr.do64[qs:qe][:, heads], [0, qe - qs], [0, ke - ks], wl.scale,
                     wl.causal, window=wl.window_sizes, softcap=wl.softcap,
                     dropout=wl.dropout_f32, drop_base=(s, g * G, wl.heads))
    return (slice(qs, qe), heads, slice(ks, ke), ref)


def run_gpu_fwd(inp: W.Inputs, keep=False):
    """Forward on cuda:0 through the C ABI.  out and lse start as NaN so
    unwritten elements show.  Returns (out [same layout as q], lse
    (B|nseq, H, Sq|max_q) fp32), both on the CPU; with keep=True also the
    dropout keep words it wrote (a device int32 tensor that starts as a
    garbage pattern, so words the forward does not write hold it)."""
    wl = inp.wl
    dev = torch.device("cuda")
    q, k, v = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v))
    out = torch.full_like(q, float("nan"))
    nseq = len(inp.lens_q)
    maxq = max(inp.lens_q) if inp.lens_q else 0
    lse = torch.full((nseq, wl.heads, maxq), float("nan"), dtype=torch.float32, device=dev)
    kw = {}
    if wl.varlen:
        kw = dict(cu_seqlens_q=torch.tensor(cu_np(inp.lens_q), dtype=torch.int32, device=dev),
                  cu_seqlens_k=torch.tensor(cu_np(inp.lens_k), dtype=torch.int32, device=dev),
                  max_seqlen_q=maxq, max_seqlen_k=max(inp.lens_k))
    args = fa.make_fwd_args(q, k, v, out, lse, wl.scale, wl.causal, window=wl.window,
                            softcap=wl.softcap, dropout=wl.dropout, **kw)
    words = None
    if keep:
        n = fa.keep_bytes(args)
        assert n > 0
        words = torch.full(((n + 3) // 4,), 0x5A5AA5A5, dtype=torch.int32, device=dev)
        args.dropout_keep_out = words.data_ptr()
        args.dropout_keep_out_bytes = words.numel() * 4
    fa.run_fwd(args)
    torch.cuda.synchronize()
    if keep:
        return out.cpu(), lse.cpu(), words
    return out.cpu(), lse.cpu()


def lse_rows(inp: W.Inputs, lse: torch.Tensor) -> np.ndarray:
    """(B|nseq, H, Sq|max_q) -> [total_q, H] fp64 (valid rows only)."""
    cu = cu_np(inp.lens_q)
    L = lse.numpy().astype(np.float64)
    rows = np.empty((int(cu[-1]), inp.wl.heads), np.float64)
    for s in range(len(inp.lens_q)):
        rows[cu[s]:cu[s + 1]] = L[s, :, :inp.lens_q[s]].T
    return rows


class _Rows64:
    """fp64 rows of a packed (rows, H, D) tensor, converted when sliced (a
    whole fp64 copy of a multi-GB input would take that many GB again)."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, sl):
        return to64(self.t[sl])


def check_full_size_units(inp: W.Inputs, units=((0, 0), (1, 5))):
    """GPU forward, then the GPU backward on its O and LSE, at a size the
    oracle cannot take whole: each (sequence, KV head) unit's O, LSE and
    gradients against the oracle computed for that unit alone (with dropout,
    replaying the bits of the unit's place in the whole call)."""
    wl = inp.wl
    out, lse = run_gpu_fwd(inp)
    pr = Prepared.__new__(Prepared)
    pr.inp = inp
    pr.cu_q, pr.cu_k = cu_np(inp.lens_q), cu_np(inp.lens_k)
    pr.q64, pr.k64, pr.v64, pr.do64 = (_Rows64(inp.packed(t)) for t in
                                       (inp.q, inp.k, inp.v, inp.dout))
    pr.o, pr.lse = out, lse
    res = run_gpu(pr)
    lrows = lse_rows(inp, lse)
    G = wl.heads // wl.heads_k
    for s, g in units:
        qs, heads, ks, ref = oracle_backward_unit(pr, s, g)
        ro, rl = O.forward(pr.q64[qs][:, heads], pr.k64[ks][:, [g]], pr.v64[ks][:, [g]],
                           [0, qs.stop - qs.start], [0, ks.stop - ks.start], wl.scale,
                           wl.causal, window=wl.window_sizes, softcap=wl.softcap,
                           dropout=wl.dropout_f32, drop_base=(s, g * G, wl.heads))
        compare(inp.packed(out)[qs][:, heads], ro, "unit %d/%d O" % (s, g))
        assert np.abs(lrows[qs][:, heads] - rl).max() <= 1e-3
        compare(inp.packed(res["dq"])[qs][:, heads], ref["dq"], "unit %d/%d dq" % (s, g))
        compare(inp.packed(res["dk"])[ks][:, [g]], ref["dk"], "unit %d/%d dk" % (s, g))
        compare(inp.packed(res["dv"])[ks][:, [g]], ref["dv"], "unit %d/%d dv" % (s, g))
