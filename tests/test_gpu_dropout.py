"""GPU parity of dropout: keep bits Z from Philox4x32-10 (element (i, j) of
query head h of sequence b: word j % 4 at counter (j / 4, i, b*H + h, offset
lo), key (seed lo, seed hi ^ offset hi), kept iff >= floor(p * 2^32)), O =
(P Z / (1 - p)) V in the forward, the same bits replayed in the backward
(mha_bwd's p_dropout and rng_state on the backward call-trace page; the keep
test of the Triton FA2 teaching page's dropout_mask).

The keep bits are checked bit for bit against the oracle's through designs
that expose them: with Q = 0 every visible key has the same P, so one-hot V
rows make O_ij nonzero exactly where Z_ij = 1 (forward), one-hot dO rows do
the same for dV (key-tile kernel), and one-hot K rows give dQ two distinct
values by Z (dQ kernel).  Random-input cases then compare all outputs with
the fp64 oracle to the usual bars in the three dQ modes.
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


SEED = 0x243F6A8885A308D3
DROPPED = {
    "causal_gqa2_d128_p0.25": lambda: W.make_inputs(
        W.custom("d1", 2, 4, 2, 200, 200, 128, True, seed=401, dropout=(0.25, SEED, 0))),
    "noncausal_sq_lt_sk_d64_p0.5": lambda: W.make_inputs(
        W.custom("d2", 1, 4, 1, 130, 300, 64, False, seed=402, dropout=(0.5, SEED, 12))),
    "causal_sq_gt_sk_empty_rows_d128_p0.125": lambda: W.make_inputs(
        W.custom("d3", 1, 4, 2, 300, 130, 128, True, seed=403,
                 dropout=(0.125, SEED, (7 << 32) + 5))),
    "headdim72_noncausal_p0.375": lambda: W.make_inputs(
        W.custom("d4", 1, 2, 2, 150, 150, 72, False, seed=404, dropout=(0.375, 17, 3))),
    "varlen_causal_left64_cap1.5_d96_p0.25": lambda: W.custom_varlen(
        "d5", [100, 257, 0, 64], [100, 257, 30, 64], 2, 2, 96, True, seed=405,
        window=(64, 0), softcap=1.5, dropout=(0.25, SEED, 99)),
    "two_sided_window_d128_p0.1": lambda: W.make_inputs(
        W.custom("d6", 1, 4, 2, 260, 260, 128, False, seed=406, window=(40, 30),
                 dropout=(0.1, 5, 1))),
}
# Cases for the forward's keep words only (above head_dim 128 the forward and
# dQ kernels take 128 query rows per workgroup).
KEEP_EXTRA = {
    "causal_gqa2_d256_p0.25": lambda: W.make_inputs(
        W.custom("d7", 1, 4, 2, 300, 300, 256, True, seed=407, dropout=(0.25, SEED, 3))),
    "varlen_noncausal_d192_p0.5": lambda: W.custom_varlen(
        "d8", [70, 0, 200], [90, 40, 130], 4, 4, 192, False, seed=408, dropout=(0.5, 9, 2)),
}


@pytest.fixture(scope="module")
def prepared():
    cache = {}

    def get(name):
        if name not in cache:
            cache[name] = PT.Prepared(DROPPED[name]())
        return cache[name]
    return get


@pytest.mark.parametrize("name", list(DROPPED))
@pytest.mark.parametrize("mode", list(MODES))
def test_dropout_backward_parity(gpu_lib, prepared, name, mode):
    _flush("dropout case %s mode=%s" % (name, mode))
    pr = prepared(name)
    acc, det = MODES[mode]
    res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(pr.inp.packed(res[key]), ref[key], "%s %s" % (name, key))
    flags = PT.ws_view(res, "flags", torch.int32, 4, (4,))
    assert int(flags[0]) == 0


@pytest.mark.parametrize("name", list(DROPPED))
def test_dropout_forward_parity(gpu_lib, name):
    _flush("dropout forward %s" % name)
    inp = DROPPED[name]()
    out, lse = PT.run_gpu_fwd(inp)
    check_forward(inp, out, lse, name)


def _uniform_design(name, B, H, Hk, Sq, Sk, D, causal, drop, onehot):
    """Q = 0 (every visible key has the same P); `onehot` in {"v", "do", "k"}
    sets that tensor's rows to unit vectors (row r -> e_r) and the rest to
    N(0, 1) draws of the workload's generator."""
    inp = W.make_inputs(W.custom(name, B, H, Hk, Sq, Sk, D, causal, seed=410, dropout=drop))
    q = torch.zeros_like(inp.q)
    k, v, do = inp.k, inp.v, inp.dout

    def eye_rows(t, n_rows_dim):
        e = torch.zeros_like(t)
        n = t.shape[1]
        idx = torch.arange(n)
        e[:, idx, :, idx % t.shape[-1]] = 1.0
        return e
    if onehot == "v":
        v = eye_rows(v, 1)
    elif onehot == "do":
        do = eye_rows(do, 1)
    elif onehot == "k":
        k = eye_rows(k, 1)
        v = torch.ones_like(v)
        do = eye_rows(do, 1)
    return W.Inputs(inp.wl, q, k, v, do, inp.lens_q, inp.lens_k)


def _visible(Sq, Sk, causal):
    i = np.arange(Sq)[:, None] + (Sk - Sq)
    j = np.arange(Sk)[None, :]
    return (j <= i) if causal else np.ones((Sq, Sk), bool)


DESIGN = [(2, 3, 3, 200, 128, 128, True), (1, 2, 1, 100, 128, 128, False)]


@pytest.mark.parametrize("shape", DESIGN)
def test_forward_keep_bits_are_the_oracles(gpu_lib, shape):
    """O_ij = Z_ij / (n_i (1 - p)) with one-hot V: the nonzero pattern of O is
    the keep mask (times visibility), bit for bit."""
    B, H, Hk, Sq, Sk, D, causal = shape
    drop = (0.375, SEED, 21)
    _flush("forward keep bits %s" % (shape,))
    inp = _uniform_design("dk_v", B, H, Hk, Sq, Sk, D, causal, drop, "v")
    out, _ = PT.run_gpu_fwd(inp)
    vis = _visible(Sq, Sk, causal)
    for b in range(B):
        for h in range(H):
            z = O.dropout_mask(drop[0], drop[1], drop[2], b, h, H, Sq, Sk).astype(bool)
            got = out[b, :, h, :Sk].float().numpy() != 0
            assert np.array_equal(got, z & vis), (b, h, int((got != (z & vis)).sum()))


@pytest.mark.parametrize("mode", list(MODES))
def test_backward_dv_keep_bits_are_the_oracles(gpu_lib, mode):
    """dV_j = sum_i P_ij Z_ij / (1 - p) dO_i with one-hot dO rows: dV_jd is
    nonzero exactly where row i = d keeps key j (summed over the group's
    heads, so the check is per KV head over the union of its query heads'
    bits with G = 1 here)."""
    B, H, Hk, Sq, Sk, D, causal = 2, 2, 2, 128, 200, 128, True
    drop = (0.25, SEED, 5)
    _flush("dV keep bits mode=%s" % mode)
    inp = _uniform_design("dk_do", B, H, Hk, Sq, Sk, D, causal, drop, "do")
    pr = PT.Prepared(inp)
    acc, det = MODES[mode]
    res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    vis = _visible(Sq, Sk, causal)
    for b in range(B):
        for h in range(H):
            z = O.dropout_mask(drop[0], drop[1], drop[2], b, h, H, Sq, Sk).astype(bool)
            got = res["dv"][b, :, h, :Sq].float().numpy() != 0     # [key j, row i]
            assert np.array_equal(got, (z & vis).T), (b, h, int((got != (z & vis).T).sum()))


def test_backward_dq_keep_bits_are_the_oracles(gpu_lib):
    """K_j = e_j, V = 1, dO_i = e_i, Q = 0: dP_ij = 1, so dS_ij = P_ij
    (Z_ij / (1 - p) - D_i) and dQ_ij = scale dS_ij takes two values per row,
    one for kept and one for dropped keys; the GPU dQ must match the
    oracle's element by element far inside the gap between the two."""
    B, H, Hk, Sq, Sk, D, causal = 1, 2, 1, 120, 128, 128, True
    drop = (0.5, SEED, 8)
    _flush("dQ keep bits")
    inp = _uniform_design("dk_k", B, H, Hk, Sq, Sk, D, causal, drop, "k")
    pr = PT.Prepared(inp)
    ref = PT.oracle_backward(pr)
    for mode, (acc, det) in MODES.items():
        res = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
        got = pr.inp.packed(res["dq"]).float().numpy().astype(np.float64)
        want = ref["dq"]
        # the two values of a row differ by scale * P / (1 - p) >= scale * 2 / Sk
        gap = inp.wl.scale * 2.0 / Sk
        assert np.abs(got - want).max() < 0.25 * gap, mode


@pytest.mark.parametrize("mode", ["separate", "ordered"])
def test_dropout_reproducible_and_offset_sensitive(gpu_lib, prepared, mode):
    """Same rng state: bit-identical; another offset: other keep bits."""
    name = "causal_gqa2_d128_p0.25"
    _flush("dropout repeat mode=%s" % mode)
    pr = prepared(name)
    acc, det = MODES[mode]
    a = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    b = PT.run_gpu(pr, deterministic=det, dq_accumulate=acc)
    for key in ("dq", "dk", "dv"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key
    wl = pr.inp.wl
    other = W.Workload(wl.name, wl.batch, wl.heads, wl.heads_k, wl.seqlen_q, wl.seqlen_k,
                       wl.head_dim, wl.causal, seed=wl.seed,
                       dropout=(wl.dropout[0], wl.dropout[1], wl.dropout[2] + 1))
    pr2 = PT.Prepared(W.Inputs(other, pr.inp.q, pr.inp.k, pr.inp.v, pr.inp.dout,
                               pr.inp.lens_q, pr.inp.lens_k))
    c = PT.run_gpu(pr2, deterministic=det, dq_accumulate=acc)
    assert not torch.equal(a["dv"], c["dv"])


def test_forward_then_backward_with_dropout(gpu_lib):
    """The GPU forward's O and LSE (dropout applied) drive the GPU backward
    with the same rng state; gradients against the oracle."""
    _flush("dropout forward -> backward")
    inp = DROPPED["causal_gqa2_d128_p0.25"]()
    out, lse = PT.run_gpu_fwd(inp)
    pr = PT.Prepared(inp)
    pr.o, pr.lse = out, lse
    res = PT.run_gpu(pr)
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(pr.inp.packed(res[key]), ref[key], "fwd->bwd %s" % key)


@pytest.mark.slow
def test_dropout_full_size_sampled_units(gpu_lib):
    """Batch 2, 32 query / 8 KV heads, 4096 x 4096, head_dim 128, causal,
    p = 0.1 with the benchmark's seed: GPU forward, then the GPU backward on
    its O and LSE; two (sequence, KV head) units against the oracle computed
    for them alone, replaying the keep bits of their place in the whole call
    (so the counters of the last sequence and of heads past 32 are covered)."""
    _flush("dropout full size sampled units")
    base = W.WORKLOADS[3]
    wl = W.Workload("gqa_b2_h32_hk8_s4096_d128_causal_dropout0.1", base.batch, base.heads,
                    base.heads_k, base.seqlen_q, base.seqlen_k, base.head_dim, True,
                    seed=base.seed, dropout=(0.1, SEED, 0))
    PT.check_full_size_units(W.make_inputs(wl), units=((0, 0), (1, 7)))


@pytest.mark.parametrize("name", ["causal_gqa2_d128_p0.25", "varlen_causal_left64_cap1.5_d96_p0.25",
                                  "causal_sq_gt_sk_empty_rows_d128_p0.125",
                                  "two_sided_window_d128_p0.1"])
def test_dq_pass_writes_the_oracles_keep_bits(gpu_lib, prepared, name):
    """The separate-dQ backward hands the key-tile kernel the keep bits
    through the workspace (word w of a row: keys 32w .. 32w+31); on every
    element a row sees, the word's bit equals the oracle's keep bit."""
    _flush("dropout keep words %s" % name)
    pr = prepared(name)
    wl = pr.inp.wl
    res = PT.run_gpu(pr)
    lay = res["layout"]
    kwn, H, rows = lay.keep_words, wl.heads, lay.rows
    assert kwn == 2 * ((max(pr.inp.lens_k) + 63) // 64)
    words = res["ws"][lay.off_keep:lay.off_keep + kwn * H * rows * 4].view(torch.int32)
    _check_words_against_oracle(pr.inp, words.numpy().view(np.uint32).reshape(kwn, H, rows))


def _check_words_against_oracle(inp, words):
    """words[w, h, row]: on every element a row sees, bit j % 32 of word
    j // 32 equals the oracle's keep bit."""
    wl = inp.wl
    H = wl.heads
    cu_q = PT.cu_np(inp.lens_q)
    p, seed, offset = wl.dropout_f32
    lw, rw = wl.window_sizes
    checked = 0
    for s, (lq, lk) in enumerate(zip(inp.lens_q, inp.lens_k)):
        if lq == 0 or lk == 0:
            continue
        r0 = int(cu_q[s]) if wl.varlen else s * wl.seqlen_q
        i = np.arange(lq)[:, None]
        j = np.arange(lk)[None, :]
        d = i + lk - lq
        vis = np.ones((lq, lk), bool)
        if wl.causal:
            vis &= j <= d
        if rw >= 0:
            vis &= j <= d + rw
        if lw >= 0:
            vis &= j >= d - lw
        for h in range(H):
            ref = O.dropout_mask(p, seed, offset, s, h, H, lq, lk)
            got = (words[j // 32, h, r0 + i] >> (j % 32).astype(np.uint32)) & 1
            assert np.array_equal(got[vis], ref[vis]), (s, h)
            checked += int(vis.sum())
    assert checked > 0


KEEP_CASES = ["causal_gqa2_d128_p0.25", "varlen_causal_left64_cap1.5_d96_p0.25",
              "causal_sq_gt_sk_empty_rows_d128_p0.125", "two_sided_window_d128_p0.1",
              "noncausal_sq_lt_sk_d64_p0.5"] + list(KEEP_EXTRA)


def _keep_inputs(prepared, name):
    return prepared(name) if name in DROPPED else PT.Prepared(KEEP_EXTRA[name]())


@pytest.mark.parametrize("name", KEEP_CASES)
def test_forward_writes_the_oracles_keep_bits(gpu_lib, prepared, name):
    """fa_fwd with dropout_keep_out writes the keep words in the workspace
    layout: on every element a row sees, the bit equals the oracle's."""
    _flush("forward keep words %s" % name)
    pr = _keep_inputs(prepared, name)
    wl = pr.inp.wl
    _, _, words = PT.run_gpu_fwd(pr.inp, keep=True)
    kwn = 2 * ((max(pr.inp.lens_k) + 63) // 64)
    rows = sum(pr.inp.lens_q) if wl.varlen else wl.batch * wl.seqlen_q
    assert words.numel() == kwn * wl.heads * rows
    _check_words_against_oracle(pr.inp, words.cpu().numpy().view(np.uint32).reshape(
        kwn, wl.heads, rows))


@pytest.mark.parametrize("name", KEEP_CASES)
def test_backward_reading_the_forwards_keep_words(gpu_lib, prepared, name):
    """The backward given the forward's words (dropout_keep) reads the bits
    instead of drawing them: no keep region in the workspace, dq / dk / dv
    bit-identical to the drawing backward's, also as separate steps."""
    _flush("backward from forward keep words %s" % name)
    pr = _keep_inputs(prepared, name)
    _, _, words = PT.run_gpu_fwd(pr.inp, keep=True)
    a = PT.run_gpu(pr)
    b = PT.run_gpu(pr, keep_words=words)
    c = PT.run_gpu(pr, keep_words=words, step_split=True)
    assert b["layout"].keep_words == 0 and c["layout"].keep_words == 0
    for key in ("dq", "dk", "dv"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key
        assert torch.equal(a[key].view(torch.int16), c[key].view(torch.int16)), key
    if name in KEEP_EXTRA:
        ref = PT.oracle_backward(pr)
        for key in ("dq", "dk", "dv"):
            PT.compare(pr.inp.packed(b[key]), ref[key], "%s %s" % (name, key))


def test_dropout_step_by_step_equals_whole_call(gpu_lib, prepared):
    """preprocess, dq, main as separate calls (main reading the keep bits the
    dq step wrote) give the whole call's gradients bit for bit."""
    _flush("dropout step by step")
    pr = prepared("causal_gqa2_d128_p0.25")
    a = PT.run_gpu(pr)
    b = PT.run_gpu(pr, step_split=True)
    for key in ("dq", "dk", "dv"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key


@pytest.mark.parametrize("name", ["causal_gqa2_d128_p0.25", "varlen_causal_left64_cap1.5_d96_p0.25"])
def test_key_tile_kernel_drawing_its_own_bits_when_the_keep_region_is_bounded(gpu_lib, prepared,
                                                                               name):
    """With the keep region bounded below its size (1 byte) the workspace has
    none and the key-tile kernel draws the bits itself: same bits, so the
    gradients equal those of the default path bit for bit (and the oracle)."""
    _flush("dropout without keep words %s" % name)
    pr = prepared(name)
    a = PT.run_gpu(pr)
    b = PT.run_gpu(pr, keep_max=1)
    assert a["layout"].keep_words > 0 and b["layout"].keep_words == 0
    for key in ("dq", "dk", "dv"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key
    ref = PT.oracle_backward(pr)
    for key in ("dq", "dk", "dv"):
        PT.compare(pr.inp.packed(b[key]), ref[key], "%s %s" % (name, key))
