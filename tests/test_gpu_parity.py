"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs.  Bar: per gradient tensor max|gpu - ref| <= 1e-2 *
max|ref| (bf16 I/O); ordered mode bit-identical across runs; preprocess and
dq_convert checked against their exact definitions."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import parity as PT
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


# Small cases: full oracle, several tiles, ragged tails.
SMALL = {
    "c1_mha_s128_d64": lambda: W.make_inputs(W.WORKLOADS[1]),
    "dense_causal_ragged_gqa2_d64": lambda: W.make_inputs(
        W.custom("r1", 2, 4, 2, 200, 200, 64, True, seed=101)),
    "causal_sq_lt_sk_mqa_d128": lambda: W.make_inputs(
        W.custom("r2", 1, 4, 1, 130, 300, 128, True, seed=102)),
    "causal_sq_gt_sk_empty_rows_d128": lambda: W.make_inputs(
        W.custom("r3", 1, 4, 2, 300, 130, 128, True, seed=103)),
    "noncausal_gqa4_d128": lambda: W.make_inputs(
        W.custom("r4", 1, 8, 2, 256, 192, 128, False, seed=104)),
    "headdim72_padded_noncausal": lambda: W.make_inputs(
        W.custom("r5", 1, 2, 2, 150, 150, 72, False, seed=105)),
    "varlen_d96_causal": lambda: W.make_inputs(
        W.Workload("r6", 3, 2, 2, 0, 0, 96, True, varlen=True, seed=106),
        lengths=[100, 257, 64]),
    "varlen_unequal_and_empty_causal_d64": lambda: W.custom_varlen(
        "r7", [70, 0, 190, 33], [130, 50, 190, 0], 4, 2, 64, True, seed=107),
    "varlen_unequal_noncausal_d128": lambda: W.custom_varlen(
        "r8", [70, 129, 1], [200, 64, 300], 2, 1, 128, False, seed=108),
}

# Row-vector cases above head dim 128 (not in the mode sweep above: the
# accumulate modes stop at 128).
BIG = {
    "causal_gqa2_d256_ragged": lambda: W.make_inputs(
        W.custom("r9", 1, 4, 2, 150, 170, 256, True, seed=109)),
    "varlen_d160_padded_causal": lambda: W.custom_varlen(
        "r10", [90, 0, 131], [120, 40, 131], 2, 1, 160, True, seed=110),
}


@pytest.fixture(scope="module")
def prepared():
    cache = {}

    def get(name):
        if name not in cache:
            cache[name] = PT.Prepared({**SMALL, **BIG}[name]())
        return cache[name]
    return get


# dQ strategies: (dq_accumulate, deterministic)
MODES = {"separate": (False, False), "atomic": (True, False), "ordered": (True, True)}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("mode", list(MODES))
def test_small_full_parity(gpu_lib, prepared, name, mode):
    _flush("case %s mode=%s" % (name, mode))
    pr = prepared(name)
    acc, det = MODES[mode]
    res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(pr.inp.packed(res[key]), ref[key], "%s %s" % (name, key))
    flags = PT.ws_view(res, "flags", torch.int32, 4, (4,))
    assert int(flags[0]) == 0


@pytest.mark.parametrize("name", ["dense_causal_ragged_gqa2_d64", "varlen_d96_causal",
                                  "causal_sq_gt_sk_empty_rows_d128"])
@pytest.mark.parametrize("mode", ["separate", "ordered"])
def test_reproducible_modes_are_bit_identical(gpu_lib, prepared, name, mode):
    _flush("case %s %s x3" % (name, mode))
    pr = prepared(name)
    acc, det = MODES[mode]
    runs = [PT.run_gpu(pr, deterministic=det, dq_accumulate=acc) for _ in range(3)]
    for key in ("dq", "dk", "dv"):
        for r in runs[1:]:
            assert torch.equal(r[key].view(torch.int16), runs[0][key].view(torch.int16)), key


def test_dk_dv_reproducible_in_atomic_mode(gpu_lib, prepared):
    pr = prepared("noncausal_gqa4_d128")
    a = PT.run_gpu(pr, dq_accumulate=True)
    b = PT.run_gpu(pr, dq_accumulate=True)
    for key in ("dk", "dv"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key


@pytest.mark.parametrize("name", ["headdim72_padded_noncausal",
                                  "varlen_unequal_and_empty_causal_d64"])
@pytest.mark.parametrize("mode", ["separate", "atomic"])
def test_columns_past_head_dim_untouched(gpu_lib, prepared, name, mode):
    pr = prepared(name)
    res = PT.run_gpu(pr, out_pad=8, dq_accumulate=MODES[mode][0])
    D = pr.inp.wl.head_dim
    for key in ("dq_buf", "dk_buf", "dv_buf"):
        assert torch.isnan(res[key][..., D:].float()).all(), key
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(pr.inp.packed(res[key]), ref[key], key)


@pytest.mark.parametrize("mode", ["separate", "ordered"])
def test_step_by_step_entry_points_match_whole_call(gpu_lib, prepared, mode):
    pr = prepared("dense_causal_ragged_gqa2_d64")
    acc, det = MODES[mode]
    a = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    b = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc, step_split=True)
    for key in ("dq", "dk", "dv"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key


@pytest.mark.parametrize("name", ["dense_causal_ragged_gqa2_d64", "varlen_d96_causal",
                                  "causal_sq_gt_sk_empty_rows_d128"])
def test_preprocess_rowdot_and_lse2(gpu_lib, prepared, name):
    """rowdot = sum_d dO*O with fp32 accumulation of exact bf16 products:
    within the summation bound (D+1) 2^-24 sum|dO*O| of the fp64 value;
    lse2 = LSE*log2(e) (+inf for rows without a visible key)."""
    pr = prepared(name)
    res = PT.run_gpu(pr)
    H, T, D = pr.inp.wl.heads, int(pr.cu_q[-1]), pr.inp.wl.head_dim
    rowdot = PT.ws_view(res, "rowdot", torch.float32, H * T, (H, T)).numpy().T
    lse2 = PT.ws_view(res, "lse2", torch.float32, H * T, (H, T)).numpy().T
    ref = O.rowdot(pr.do64, pr.o64)
    absum = O.rowdot(np.abs(pr.do64), np.abs(pr.o64))
    bound = (D + 1) * 2.0 ** -24 * absum + 1e-30
    assert np.all(np.abs(rowdot - ref) <= bound)
    lse32 = pr.lse_rows.astype(np.float32)
    empty = np.isneginf(lse32)
    assert np.all(np.isposinf(lse2[empty]))
    want = lse32[~empty].astype(np.float64) * np.log2(np.e)
    assert np.all(np.abs(lse2[~empty] - want) <= 2e-7 * np.maximum(1.0, np.abs(want)))


@pytest.mark.parametrize("name", ["dense_causal_ragged_gqa2_d64", "varlen_d96_causal",
                                  "causal_sq_gt_sk_empty_rows_d128", *BIG])
def test_dq_step_writes_the_preprocess_row_vectors_bit_for_bit(gpu_lib, prepared, name):
    """The separate dQ kernel forms lse2 and rowdot itself (the key-tile
    kernel then runs after it); they must equal the preprocess kernel's to
    the bit, so that every step order gives the same dK/dV."""
    pr = prepared(name)
    a = PT.run_gpu(pr, steps=["preprocess"])
    b = PT.run_gpu(pr, steps=["dq"])
    H, T = pr.inp.wl.heads, int(pr.cu_q[-1])
    for vec in ("lse2", "rowdot"):
        va = PT.ws_view(a, vec, torch.float32, H * T, (H, T)).view(torch.int32)
        vb = PT.ws_view(b, vec, torch.float32, H * T, (H, T)).view(torch.int32)
        assert torch.equal(va, vb), vec


@pytest.mark.parametrize("name", ["dense_causal_ragged_gqa2_d64", "varlen_unequal_and_empty_causal_d64",
                                  "causal_sq_gt_sk_empty_rows_d128", "causal_gqa2_d256_ragged"])
def test_debug_rowsum(gpu_lib, prepared, name):
    """fa_bwd_debug_rowsum writes D = rowsum(dO * O) in the lse layout:
    within the fp32 summation bound of the fp64 definition, equal to the
    workspace row sums the kernels use (bit for bit), packed rows past a
    sequence's length untouched; the backward afterwards is unchanged."""
    import attention_backward_fa2_amd as fa
    _flush("debug rowsum %s" % name)
    pr = prepared(name)
    inp, wl = pr.inp, pr.inp.wl
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.dout))
    o, lse = pr.o.to(dev).contiguous(), pr.lse.to(dev).contiguous()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = {}
    if wl.varlen:
        kw = dict(cu_seqlens_q=torch.tensor(pr.cu_q, dtype=torch.int32, device=dev),
                  cu_seqlens_k=torch.tensor(pr.cu_k, dtype=torch.int32, device=dev),
                  max_seqlen_q=max(inp.lens_q), max_seqlen_k=max(inp.lens_k))
    args = fa.make_args(do, q, k, v, o, lse, dq, dk, dv, wl.scale, wl.causal, **kw)
    ws = fa.alloc_workspace(args, dev)
    ws.fill_(0xA5)
    d_out = torch.full_like(lse, float("nan"))
    fa.debug_rowsum(args, d_out)
    torch.cuda.synchronize()
    H, T, D = wl.heads, int(pr.cu_q[-1]), wl.head_dim
    got = PT.lse_rows(inp, d_out.cpu())                      # [T, H]
    ref = O.rowdot(pr.do64, pr.o64)
    absum = O.rowdot(np.abs(pr.do64), np.abs(pr.o64))
    assert np.all(np.abs(got - ref) <= (D + 1) * 2.0 ** -24 * absum + 1e-30)
    lay = fa.workspace_layout(args)
    raw = ws.cpu()[lay.off_rowdot:lay.off_rowdot + 4 * H * T].view(torch.float32)
    wsrow = raw.reshape(H, T).numpy().T
    assert np.array_equal(got.astype(np.float32).view(np.int32), wsrow.view(np.int32))
    dc = d_out.cpu()
    for s_, n in enumerate(inp.lens_q):                     # padding rows untouched
        assert torch.isnan(dc[s_, :, n:]).all()
    fa.run(args, "all")
    torch.cuda.synchronize()
    ref_b = PT.oracle_backward(pr)
    for key, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        PT.compare(inp.packed(t.cpu()), ref_b[key], "%s after debug %s" % (name, key))


def test_dq_convert_is_exact_scaled_rne(gpu_lib, prepared):
    pr = prepared("varlen_unequal_noncausal_d128")
    res = PT.run_gpu(pr, dq_accumulate=True)
    lay = res["layout"]
    H, T, DP, D = pr.inp.wl.heads, int(pr.cu_q[-1]), lay.head_dim_pad, pr.inp.wl.head_dim
    acc = PT.ws_view(res, "dq_acc", torch.float32, H * T * DP, (H, T, DP))
    scale = torch.tensor(pr.inp.wl.scale, dtype=torch.float32)
    want = (acc[:, :, :D] * scale).to(torch.bfloat16).permute(1, 0, 2)
    got = pr.inp.packed(res["dq"])
    assert torch.equal(got.view(torch.int16), want.contiguous().view(torch.int16))


def test_dk_dv_column_sum_invariants(gpu_lib, prepared):
    """sum_j dK_j = 0 (softmax is invariant to shifting all keys) and
    sum_j dV_j = sum over rows with a visible key of dO_i, per KV head."""
    pr = prepared("causal_sq_lt_sk_mqa_d128")
    res = PT.run_gpu(pr)
    dk = pr.inp.packed(res["dk"]).double().numpy()
    dv = pr.inp.packed(res["dv"]).double().numpy()
    G = pr.inp.wl.heads // pr.inp.wl.heads_k
    vis = ~np.isneginf(pr.lse_rows)               # [T, H]
    for g in range(pr.inp.wl.heads_k):
        s_dk = dk[:, g].sum(0)
        assert np.abs(s_dk).max() <= 1e-2 * np.abs(dk[:, g]).sum(0).max()
        want = sum((pr.do64[:, h] * vis[:, h:h + 1]).sum(0) for h in range(g * G, (g + 1) * G))
        assert np.abs(dv[:, g].sum(0) - want).max() <= 1e-2 * np.abs(dv[:, g]).sum(0).max()


def test_zero_query_rows_write_zero_dk_dv(gpu_lib):
    """Dense seqlen_q == 0 with keys: dk and dv are written as zeros."""
    dev = torch.device("cuda")
    B, Sk, H, D = 1, 200, 2, 64
    q = torch.zeros(B, 0, H, D, dtype=torch.bfloat16, device=dev)
    k = torch.randn(B, Sk, H, D, device=dev).to(torch.bfloat16)
    v = torch.randn(B, Sk, H, D, device=dev).to(torch.bfloat16)
    lse = torch.zeros(B, H, 0, dtype=torch.float32, device=dev)
    dq = torch.empty_like(q)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    import attention_backward_fa2_amd as fa
    fa.fa_bwd(q, q, k, v, q, lse, dq, dk, dv, D ** -0.5, True)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


# ---------------- reference workloads at full size ----------------

def _full(cid):
    return PT.Prepared(W.make_inputs(W.WORKLOADS[cid]))


@pytest.mark.slow
def test_config2_full_parity(gpu_lib):
    _flush("config 2 full")
    pr = _full(2)
    ref = PT.oracle_backward(pr)
    for mode, (acc, det) in MODES.items():
        res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
        for key in ("dq", "dk", "dv"):
            PT.compare(pr.inp.packed(res[key]), ref[key], "c2 %s %s" % (key, mode))


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.slow
@pytest.mark.parametrize("cid", [3, 4, 5])
def test_full_size_parity(gpu_lib, cid):
    """Whole dQ, dK and dV at the full workload size, every element against
    the fp64 oracle (per tensor max|gpu - ref| <= 1e-2 max|ref|), in the
    three dQ modes; the separate mode in the launch configuration the
    benchmark times.  At the headline workload (3) the separate and ordered
    modes are also repeated three times and must be bit-identical, and the
    atomic mode's dK / dV (which do not depend on the dQ adds) must equal
    the separate mode's."""
    import time
    t0 = time.time()
    _flush("config %d full size: oracle forward" % cid)
    pr = _full(cid)
    _flush("config %d: oracle backward (%.1f s)" % (cid, time.time() - t0))
    ref = PT.oracle_backward(pr)
    _flush("config %d: oracle done (%.1f s)" % (cid, time.time() - t0))
    runs = {}
    for mode, (acc, det) in MODES.items():
        reps = 3 if cid == 3 and mode != "atomic" else 1
        runs[mode] = [PT.run_gpu(pr, deterministic=det, dq_accumulate=acc) for _ in range(reps)]
        res = runs[mode][0]
        errs = {key: PT.compare(pr.inp.packed(res[key]), ref[key], "c%d %s %s" % (cid, key, mode))
                for key in ("dq", "dk", "dv")}
        if acc:
            flags = PT.ws_view(res, "flags", torch.int32, 4, (4,))
            assert int(flags[0]) == 0, "ordered wait gave up"
        for r in runs[mode][1:]:
            for key in ("dq", "dk", "dv"):
                assert torch.equal(_bits(r[key]), _bits(res[key])), "c%d %s %s repeat" % (
                    cid, mode, key)
        _flush("config %d %s: max|err|/max|ref| %s (%.1f s)" % (
            cid, mode, {k: "%.2e" % v for k, v in errs.items()}, time.time() - t0))
    for key in ("dk", "dv"):   # the two dQ strategies share the dK/dV pass
        assert torch.equal(_bits(runs["atomic"][0][key]), _bits(runs["separate"][0][key])), key


@pytest.mark.slow
def test_tensors_beyond_2gib_sampled_units(gpu_lib):
    """B = 2112 sequences of 512 rows, 8 query / 2 KV heads, head_dim 128,
    causal: q, out, dout and dq are 2.2 GB each, so the rows of the last
    sequences start beyond 2^31 bytes (every kernel forms row addresses in
    64 bits and keeps 32-bit offsets within a tile).  GPU forward, then the
    GPU backward on its O and LSE; the first, a middle and the last
    (sequence, KV head) units against the oracle computed for them alone."""
    wl = W.custom("beyond_2gib", 2112, 8, 2, 512, 512, 128, True, seed=20261241)
    inp = W.make_inputs(wl)
    assert inp.q.numel() * inp.q.element_size() > 2 ** 31
    assert (2111 * 512 * 8 * 128) * 2 > 2 ** 31   # first row of the last sequence
    _flush("tensors beyond 2 GiB: inputs drawn")
    PT.check_full_size_units(inp, units=((0, 0), (1060, 1), (2111, 1)))


@pytest.mark.parametrize("shape", [
    # (B, H, Hk, S): standard dQ shape (8 waves, 256 rows) when the grid of
    # 256-row workgroups has at least 512 of them, else the small one (two
    # 128-row workgroups per CU)
    (2, 32, 8, 2048),   # 8 * 32 * 2 = 512 workgroups: standard
    (1, 4, 2, 600),     # 3 * 4 * 1 = 12: small
    (3, 6, 3, 1000),    # 4 * 6 * 3 = 72: small, ragged tail
])
def test_head_dim_64_both_dq_shapes(gpu_lib, shape):
    """Head dim 64, causal GQA: both dQ workgroup shapes against the oracle
    in the three dQ modes."""
    B, H, Hk, S = shape
    _flush("head dim 64 dq shapes %s" % (shape,))
    pr = PT.Prepared(W.make_inputs(W.custom("d64_%d_%d" % (B, S), B, H, Hk, S, S, 64, True,
                                            seed=20261250 + S)))
    ref = PT.oracle_backward(pr)
    for mode, (acc, det) in MODES.items():
        res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
        for key in ("dq", "dk", "dv"):
            PT.compare(pr.inp.packed(res[key]), ref[key], "d64 %s %s %s" % (shape, mode, key))
