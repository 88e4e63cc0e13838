"""Pins of the fp64 CPU oracle against things other than itself.

Each test fixes the oracle to mathematics it cannot share code with:
central finite differences of its own forward (the gradient definition),
hand-derived closed forms (tests/golden), invariants of the softmax
Jacobian, a library softmax (scipy) for the forward, and structural
identities of the method (GQA = repeated-KV MHA, causal = explicit -inf mask,
packed = per-sequence).  CPU only.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _problem(seed, lens_q, lens_k, H, Hk, D, zero_q=False, equal_k=False):
    rng = np.random.default_rng(seed)
    Tq, Tk = sum(lens_q), sum(lens_k)
    q = np.zeros((Tq, H, D)) if zero_q else rng.standard_normal((Tq, H, D))
    k = rng.standard_normal((Tk, Hk, D))
    if equal_k:
        k[:] = k[:1]
    v = rng.standard_normal((Tk, Hk, D))
    do = rng.standard_normal((Tq, H, D))
    cu_q = np.cumsum([0] + list(lens_q))
    cu_k = np.cumsum([0] + list(lens_k))
    return q, k, v, do, cu_q, cu_k


def _loss(q, k, v, do, cu_q, cu_k, scale, causal):
    out, _ = O.forward(q, k, v, cu_q, cu_k, scale, causal)
    return float(np.sum(do * out))


def _central_diff(x, f, h=1e-5):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


FD_CASES = [
    # (name, lens_q, lens_k, H, Hk, D, causal)
    ("dense_noncausal", [5], [7], 2, 1, 3, False),
    ("dense_causal_sq_lt_sk", [5], [7], 2, 1, 3, True),
    ("causal_sq_gt_sk_empty_rows", [7], [5], 2, 1, 3, True),
    ("varlen_two_seqs_causal", [3, 5], [4, 2], 2, 1, 3, True),
    ("varlen_two_seqs_noncausal_d5", [3, 5], [4, 2], 2, 2, 5, False),
]


@pytest.mark.parametrize("case", FD_CASES, ids=[c[0] for c in FD_CASES])
@pytest.mark.parametrize("mode", ["contracted", "explicit"])
def test_gradient_matches_central_differences(case, mode):
    name, lq, lk, H, Hk, D, causal = case
    q, k, v, do, cu_q, cu_k = _problem(11, lq, lk, H, Hk, D)
    scale = 0.7
    g = O.backward(q, k, v, do, cu_q, cu_k, scale, causal, mode=mode)
    f = lambda: _loss(q, k, v, do, cu_q, cu_k, scale, causal)  # noqa: E731
    for key, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = _central_diff(x, f)
        err = np.abs(g[key] - fd)
        assert np.all(err <= 1e-7 * np.maximum(1.0, np.abs(g[key]))), (key, err.max())


@pytest.mark.parametrize("fname", ["closed_form_one_query_two_keys.json",
                                   "closed_form_causal_bottom_right_2x3.json",
                                   "closed_form_softcap_one_query_two_keys.json"])
@pytest.mark.parametrize("mode", ["contracted", "explicit"])
def test_hand_derived_closed_forms(fname, mode):
    gd = json.load(open(os.path.join(GOLDEN, fname)))
    A = {k: np.array(gd[k], dtype=np.float64)
         for k in ("q", "k", "v", "dout", "out", "lse", "dq", "dk", "dv")}
    cu_q = [0, gd["shape"]["Sq"]]
    cu_k = [0, gd["shape"]["Sk"]]
    cap = gd.get("softcap", 0.0)
    out, lse = O.forward(A["q"], A["k"], A["v"], cu_q, cu_k, gd["scale"], gd["causal"],
                         softcap=cap)
    np.testing.assert_allclose(out, A["out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, A["lse"], rtol=0, atol=1e-14)
    g = O.backward(A["q"], A["k"], A["v"], A["dout"], cu_q, cu_k, gd["scale"],
                   gd["causal"], mode=mode, softcap=cap)
    for key in ("dq", "dk", "dv"):
        np.testing.assert_allclose(g[key], A[key], rtol=0, atol=1e-14, err_msg=key)


@pytest.mark.parametrize("causal,lq,lk", [(False, 9, 13), (True, 9, 13), (True, 13, 9),
                                           (True, 12, 12)])
def test_forward_matches_library_softmax(causal, lq, lk):
    q, k, v, _, cu_q, cu_k = _problem(5, [lq], [lk], 4, 2, 8)
    scale = 0.35
    out, lse = O.forward(q, k, v, cu_q, cu_k, scale, causal)
    for h in range(4):
        g = h // 2
        S = scale * (q[:, h, :] @ k[:, g, :].T)
        if causal:
            i = np.arange(lq)[:, None]
            j = np.arange(lk)[None, :]
            S = np.where(j <= i + lk - lq, S, -np.inf)
        empty = np.all(np.isinf(S), axis=1)
        Sf = np.where(empty[:, None], 0.0, S)
        ref_lse = np.where(empty, -np.inf, scipy.special.logsumexp(Sf, axis=1))
        P = np.where(empty[:, None], 0.0, scipy.special.softmax(Sf, axis=1))
        P = np.where(np.isinf(S), 0.0, P)
        np.testing.assert_allclose(out[:, h, :], P @ v[:, g, :], rtol=1e-12, atol=1e-13)
        fin = ~empty
        np.testing.assert_allclose(lse[fin, h], ref_lse[fin], rtol=1e-13, atol=1e-13)
        assert np.all(lse[empty, h] == -np.inf)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_jacobian_rows_sum_to_zero(causal):
    q, k, v, do, cu_q, cu_k = _problem(3, [16], [24], 2, 1, 8)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.5, causal, mode="explicit", want_ds=True)
    ds = g["ds"]
    tol = 1e-12 * ds.shape[-1] * np.abs(ds).max()
    assert np.abs(ds.sum(axis=-1)).max() <= tol


@pytest.mark.parametrize("causal,lq,lk", [(False, 17, 23), (True, 17, 23), (True, 23, 17),
                                           (True, 20, 20)])
def test_explicit_jacobian_equals_contracted(causal, lq, lk):
    q, k, v, do, cu_q, cu_k = _problem(7, [lq], [lk], 4, 2, 16)
    a = O.backward(q, k, v, do, cu_q, cu_k, 0.25, causal, mode="explicit")
    b = O.backward(q, k, v, do, cu_q, cu_k, 0.25, causal, mode="contracted")
    for key in ("dq", "dk", "dv", "dj"):
        scale = max(1.0, np.abs(a[key]).max())
        assert np.abs(a[key] - b[key]).max() <= 1e-12 * scale, key


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha_with_repeated_kv(causal):
    G = 3
    q, k, v, do, cu_q, cu_k = _problem(9, [11, 6], [13, 6], 6, 2, 8)
    gq = O.backward(q, k, v, do, cu_q, cu_k, 0.3, causal)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    mh = O.backward(q, kr, vr, do, cu_q, cu_k, 0.3, causal)
    assert np.array_equal(gq["dq"], mh["dq"])
    for key in ("dk", "dv"):
        summed = np.zeros_like(gq[key])
        for g in range(2):
            acc = np.zeros_like(summed[:, g])
            for h in range(g * G, (g + 1) * G):   # ascending head order
                acc = acc + mh[key][:, h]
            summed[:, g] = acc
        assert np.array_equal(gq[key], summed), key


@pytest.mark.parametrize("lq,lk", [(5, 9), (8, 8), (9, 5)])
@pytest.mark.parametrize("mode", ["contracted", "explicit"])
def test_causal_equals_explicit_minus_inf_mask(lq, lk, mode):
    q, k, v, do, cu_q, cu_k = _problem(13, [lq], [lk], 2, 1, 4)
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    mask = np.where(j <= i + lk - lq, 0.0, -np.inf)
    a = O.backward(q, k, v, do, cu_q, cu_k, 0.6, True, mode=mode)
    b = O.backward(q, k, v, do, cu_q, cu_k, 0.6, False, mask=mask, mode=mode)
    for key in ("dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key]), key
    oa, la = O.forward(q, k, v, cu_q, cu_k, 0.6, True)
    ob, lb = O.forward(q, k, v, cu_q, cu_k, 0.6, False, mask=mask)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


@pytest.mark.parametrize("causal", [False, True])
def test_row_contraction_equals_rowdot_of_output(causal):
    """sum_k P_ik dP_ik == sum_d dO_id O_id: the identity the GPU preprocess
    relies on, checked on the oracle's own fp64 O."""
    q, k, v, do, cu_q, cu_k = _problem(21, [10, 19], [14, 19], 4, 4, 12)
    out, _ = O.forward(q, k, v, cu_q, cu_k, 0.4, causal)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.4, causal)
    rd = O.rowdot(do, out)
    np.testing.assert_allclose(g["dj"], rd, rtol=1e-12, atol=1e-12)


def test_rowdot_is_plain_sum():
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal((7, 3, 10)), rng.standard_normal((7, 3, 10))
    np.testing.assert_allclose(O.rowdot(a, b), np.einsum("thd,thd->th", a, b),
                               rtol=1e-14, atol=1e-14)


def test_single_key_gives_zero_dq_dk_and_summed_dv():
    q, k, v, do, cu_q, cu_k = _problem(4, [6], [1], 4, 2, 5)
    out, _ = O.forward(q, k, v, cu_q, cu_k, 0.5, False)
    for h in range(4):
        np.testing.assert_array_equal(out[:, h], np.repeat(v[:, h // 2], 6, axis=0))
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.5, False)
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    for gk in range(2):
        ref = do[:, 2 * gk].sum(0) + do[:, 2 * gk + 1].sum(0)
        np.testing.assert_allclose(g["dv"][0, gk], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_keys_give_uniform_softmax_and_zero_dq(causal):
    q, k, v, do, cu_q, cu_k = _problem(8, [9], [12], 2, 1, 6, equal_k=True)
    out, _ = O.forward(q, k, v, cu_q, cu_k, 0.5, causal)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.5, causal)
    assert np.abs(g["dq"]).max() <= 1e-13
    for i in range(9):
        nvis = min(12, i + 12 - 9 + 1) if causal else 12
        np.testing.assert_allclose(out[i, 0], v[:nvis, 0].mean(0), rtol=1e-13, atol=1e-13)


def test_causal_first_row_of_aligned_square_has_zero_dq():
    q, k, v, do, cu_q, cu_k = _problem(10, [8], [8], 2, 2, 4)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.5, True)
    assert np.all(g["dq"][0] == 0)


def test_zero_queries_give_uniform_attention():
    Sq, Sk = 7, 5
    q, k, v, do, cu_q, cu_k = _problem(12, [Sq], [Sk], 2, 1, 4, zero_q=True)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.9, False)
    assert np.all(g["dk"] == 0)
    ref = (do[:, 0].sum(0) + do[:, 1].sum(0)) / Sk
    for j in range(Sk):
        np.testing.assert_allclose(g["dv"][j, 0], ref, rtol=1e-13, atol=1e-13)


def test_gradient_is_linear_in_dout():
    q, k, v, do1, cu_q, cu_k = _problem(14, [8], [10], 2, 1, 4)
    do2 = np.random.default_rng(15).standard_normal(do1.shape)
    a = 1.75
    g1 = O.backward(q, k, v, do1, cu_q, cu_k, 0.5, True)
    g2 = O.backward(q, k, v, do2, cu_q, cu_k, 0.5, True)
    g3 = O.backward(q, k, v, a * do1 + do2, cu_q, cu_k, 0.5, True)
    for key in ("dq", "dk", "dv"):
        np.testing.assert_allclose(g3[key], a * g1[key] + g2[key], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_equals_per_sequence(causal):
    lq, lk = [5, 9, 3], [7, 9, 2]
    q, k, v, do, cu_q, cu_k = _problem(16, lq, lk, 4, 2, 6)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.5, causal)
    out, lse = O.forward(q, k, v, cu_q, cu_k, 0.5, causal)
    for s in range(3):
        qs, qe, ks, ke = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        gs = O.backward(q[qs:qe], k[ks:ke], v[ks:ke], do[qs:qe], [0, qe - qs], [0, ke - ks],
                        0.5, causal)
        os_, ls = O.forward(q[qs:qe], k[ks:ke], v[ks:ke], [0, qe - qs], [0, ke - ks], 0.5,
                            causal)
        assert np.array_equal(g["dq"][qs:qe], gs["dq"])
        assert np.array_equal(g["dk"][ks:ke], gs["dk"])
        assert np.array_equal(g["dv"][ks:ke], gs["dv"])
        assert np.array_equal(out[qs:qe], os_) and np.array_equal(lse[qs:qe], ls)


def test_empty_rows_have_zero_gradient_and_minus_inf_lse():
    q, k, v, do, cu_q, cu_k = _problem(17, [6], [3], 2, 1, 4)
    out, lse = O.forward(q, k, v, cu_q, cu_k, 0.5, True)
    # key limit of row i is i + 3 - 6 = i - 3: rows 0..2 see nothing
    assert np.all(lse[:3] == -np.inf) and np.all(out[:3] == 0)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.5, True)
    assert np.all(g["dq"][:3] == 0)
    assert np.all(np.isfinite(g["dq"])) and np.all(np.isfinite(g["dk"]))


def test_oracle_rejects_bad_arguments():
    q, k, v, do, cu_q, cu_k = _problem(1, [4], [4], 3, 2, 4)
    with pytest.raises(ValueError):
        O.backward(q, k, v, do, cu_q, cu_k, 0.5, False)


# ---- local (sliding-window) attention: query i sees keys
#      i + Lk - Lq - left .. i + Lk - Lq + right (negative = unbounded) ----

WINDOWS = [(3, 1), (0, 2), (4, -1), (-1, 2), (2, 0)]


@pytest.mark.parametrize("lq,lk", [(6, 9), (8, 8), (9, 6)])
@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("causal", [False, True])
def test_window_equals_explicit_minus_inf_mask(lq, lk, window, causal):
    left, right = window
    q, k, v, do, cu_q, cu_k = _problem(31, [lq], [lk], 2, 1, 4)
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    diag = i + lk - lq
    vis = np.ones((lq, lk), bool)
    if causal:
        vis &= j <= diag
    if right >= 0:
        vis &= j <= diag + right
    if left >= 0:
        vis &= j >= diag - left
    mask = np.where(vis, 0.0, -np.inf)
    oa, la = O.forward(q, k, v, cu_q, cu_k, 0.6, causal, window=window)
    ob, lb = O.forward(q, k, v, cu_q, cu_k, 0.6, False, mask=mask)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    for mode in ("contracted", "explicit"):
        a = O.backward(q, k, v, do, cu_q, cu_k, 0.6, causal, mode=mode, window=window)
        b = O.backward(q, k, v, do, cu_q, cu_k, 0.6, False, mask=mask, mode=mode)
        for key in ("dq", "dk", "dv"):
            assert np.array_equal(a[key], b[key]), (mode, key)


def test_window_zero_is_the_identity_attention():
    """window (0, 0) on a square problem: each query sees only its own key, so
    P = I: O = V, LSE_i = S_ii, dQ = dK = 0 and dV = dO summed over the
    query heads of the group."""
    q, k, v, do, cu_q, cu_k = _problem(32, [7], [7], 4, 2, 5)
    out, lse = O.forward(q, k, v, cu_q, cu_k, 0.7, False, window=(0, 0))
    G = 2
    for h in range(4):
        assert np.allclose(out[:, h], v[:, h // G], rtol=0, atol=1e-14)
        s_ii = 0.7 * np.einsum("id,id->i", q[:, h], k[:, h // G])
        assert np.allclose(lse[:, h], s_ii, rtol=0, atol=1e-13)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.7, False, window=(0, 0))
    assert np.abs(g["dq"]).max() < 1e-13 and np.abs(g["dk"]).max() < 1e-13
    for kv in range(2):
        assert np.allclose(g["dv"][:, kv], do[:, 2 * kv] + do[:, 2 * kv + 1], rtol=0,
                           atol=1e-13)


def test_window_right_zero_equals_causal():
    q, k, v, do, cu_q, cu_k = _problem(33, [5, 9], [8, 6], 2, 1, 4)
    a = O.backward(q, k, v, do, cu_q, cu_k, 0.5, True)
    b = O.backward(q, k, v, do, cu_q, cu_k, 0.5, False, window=(-1, 0))
    for key in ("dq", "dk", "dv", "lse"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("window,causal", [((2, 1), False), ((1, -1), True)])
def test_window_gradient_matches_central_differences(window, causal):
    q, k, v, do, cu_q, cu_k = _problem(34, [4, 6], [5, 6], 2, 1, 3)

    def loss():
        out, _ = O.forward(q, k, v, cu_q, cu_k, 0.8, causal, window=window)
        return float(np.sum(do * out))
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.8, causal, window=window)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = _central_diff(x, loss)
        assert np.allclose(g[name], fd, rtol=1e-6, atol=1e-7), name


# ---- soft-capped scores: every scaled score x becomes c * tanh(x / c) ----

SOFTCAP_FD_CASES = [
    # (lens_q, lens_k, H, Hk, D, causal, window, cap)
    ([5], [7], 2, 1, 3, False, (-1, -1), 0.9),
    ([4, 6], [5, 6], 2, 1, 3, True, (2, 0), 1.3),
    ([7], [5], 2, 2, 4, True, (-1, -1), 0.5),        # rows without keys
]


@pytest.mark.parametrize("case", SOFTCAP_FD_CASES)
@pytest.mark.parametrize("mode", ["contracted", "explicit"])
def test_softcap_gradient_matches_central_differences(case, mode):
    lq, lk, H, Hk, D, causal, window, cap = case
    q, k, v, do, cu_q, cu_k = _problem(41, lq, lk, H, Hk, D)
    q *= 2.0   # scaled scores of several units: the cap is far from linear

    def loss():
        out, _ = O.forward(q, k, v, cu_q, cu_k, 0.8, causal, window=window, softcap=cap)
        return float(np.sum(do * out))
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.8, causal, mode=mode, window=window,
                   softcap=cap)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = _central_diff(x, loss)
        err = np.abs(g[name] - fd)
        assert np.all(err <= 1e-7 * np.maximum(1.0, np.abs(g[name]))), (name, err.max())


def test_huge_softcap_is_no_cap():
    """c tanh(x / c) = x - x^3 / (3 c^2) + ...: at c = 1e7 the cap moves the
    scores by less than 1e-13."""
    q, k, v, do, cu_q, cu_k = _problem(42, [6, 9], [8, 7], 4, 2, 5)
    a = O.backward(q, k, v, do, cu_q, cu_k, 0.6, True)
    b = O.backward(q, k, v, do, cu_q, cu_k, 0.6, True, softcap=1e7)
    for key in ("dq", "dk", "dv", "lse"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-10, atol=1e-12, err_msg=key)


def test_tiny_softcap_gives_uniform_attention_and_no_score_gradient():
    """c = 1e-12: |capped score| <= c, so each row attends uniformly to the
    keys it sees (O = their mean V, LSE = ln n); every |x / c| is past 1e3,
    where tanh is 1 in fp64, so the cap's derivative and with it dQ and dK are
    exactly 0; dV_j = sum over the rows i that see j of dO_i / n_i."""
    lq, lk = 6, 9
    q, k, v, do, cu_q, cu_k = _problem(43, [lq], [lk], 2, 1, 4)
    cap = 1e-12
    out, lse = O.forward(q, k, v, cu_q, cu_k, 0.5, True, softcap=cap)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.5, True, softcap=cap)
    off = lk - lq
    dv = np.zeros_like(v)
    for i in range(lq):
        n = i + off + 1                      # bottom-right causal: keys 0 .. i + off
        for h in range(2):
            np.testing.assert_allclose(out[i, h], v[:n, 0].mean(axis=0), rtol=1e-12, atol=1e-12)
            assert abs(lse[i, h] - np.log(n)) <= 2 * cap
            dv[:n, 0] += do[i, h] / n
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    np.testing.assert_allclose(g["dv"], dv, rtol=1e-12, atol=1e-12)


def test_capped_scores_are_bounded_by_the_cap():
    """|c tanh(x / c)| < c: LSE_i lies within c of ln(number of visible keys)."""
    q, k, v, do, cu_q, cu_k = _problem(44, [10], [10], 2, 1, 8)
    q *= 5.0
    cap = 0.25
    _, lse = O.forward(q, k, v, cu_q, cu_k, 1.0, True, softcap=cap)
    n = np.arange(1, 11)[:, None]
    assert np.all(np.abs(lse - np.log(n)) <= cap)


# ---- dropout: keep bits Z from Philox4x32-10, O = (P * Z / (1 - p)) V ----

def test_philox_known_answer_vectors():
    gd = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for vec in gd["vectors"]:
        ctr = [int(x, 16) for x in vec["ctr"]]
        key = [int(x, 16) for x in vec["key"]]
        assert O.philox4x32_10(ctr, key) == [int(x, 16) for x in vec["out"]]


def test_dropout_mask_layout_and_threshold():
    """Element (b, h, i, j): word j % 4 of Philox at counter
    (j // 4, i, b*H + h, offset mod 2^32), key (seed lo, seed hi ^ offset hi);
    kept iff the word is >= floor(p * 2^32)."""
    p, seed, offset = 0.37, 0x0123456789ABCDEF, (5 << 32) + 77
    b, h, H, Lq, Lk = 3, 2, 5, 7, 11
    m = O.dropout_mask(p, seed, offset, b, h, H, Lq, Lk)
    thr = int(np.floor(p * 2**32))
    key = [seed & 0xFFFFFFFF, (seed >> 32) ^ (offset >> 32)]
    for i in range(Lq):
        for j in range(Lk):
            w = O.philox4x32_10([j // 4, i, b * H + h, offset & 0xFFFFFFFF], key)[j % 4]
            assert m[i, j] == (w >= thr)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_dropout_keeps_one_minus_p(p):
    """Kept fraction within 6 binomial standard deviations of 1 - p over 256K
    elements, and no visible dependence between neighbouring heads."""
    a = O.dropout_mask(p, 1234, 0, 0, 0, 2, 256, 1024).astype(np.float64)
    b = O.dropout_mask(p, 1234, 0, 0, 1, 2, 256, 1024).astype(np.float64)
    n = a.size
    sd = np.sqrt(p * (1 - p) / n)
    assert abs(a.mean() - (1 - p)) <= 6 * sd
    corr = np.corrcoef(a.ravel(), b.ravel())[0, 1]
    assert abs(corr) <= 6 / np.sqrt(n)
    assert np.all(O.dropout_mask(0.0, 1234, 0, 0, 0, 2, 8, 8) == 1)


def test_dropout_zero_is_no_dropout():
    q, k, v, do, cu_q, cu_k = _problem(51, [6, 9], [8, 7], 4, 2, 5)
    a = O.backward(q, k, v, do, cu_q, cu_k, 0.6, True)
    b = O.backward(q, k, v, do, cu_q, cu_k, 0.6, True, dropout=(0.0, 99, 7))
    for key in ("dq", "dk", "dv", "lse"):
        assert np.array_equal(a[key], b[key]), key


DROP_FD_CASES = [
    # (lens_q, lens_k, H, Hk, D, causal, window, softcap, p)
    ([5], [7], 2, 1, 3, False, (-1, -1), 0.0, 0.3),
    ([4, 6], [5, 6], 2, 1, 3, True, (2, 0), 0.0, 0.5),
    ([7], [5], 2, 2, 4, True, (-1, -1), 1.1, 0.2),        # rows without keys, softcap
]


@pytest.mark.parametrize("case", DROP_FD_CASES)
@pytest.mark.parametrize("mode", ["contracted", "explicit"])
def test_dropout_gradient_matches_central_differences(case, mode):
    """With the seed fixed the keep bits are constants, so the gradient of
    sum(dO * O) is that of a smooth function: central differences of the
    oracle's own dropout forward."""
    lq, lk, H, Hk, D, causal, window, cap, p = case
    q, k, v, do, cu_q, cu_k = _problem(52, lq, lk, H, Hk, D)
    drop = (p, 0xDEADBEEF12345, 3)

    def loss():
        out, _ = O.forward(q, k, v, cu_q, cu_k, 0.8, causal, window=window, softcap=cap,
                           dropout=drop)
        return float(np.sum(do * out))
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.8, causal, mode=mode, window=window,
                   softcap=cap, dropout=drop)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = _central_diff(x, loss)
        err = np.abs(g[name] - fd)
        assert np.all(err <= 1e-7 * np.maximum(1.0, np.abs(g[name]))), (name, err.max())


def test_dropout_output_is_unbiased():
    """E[Z / (1 - p)] = 1: averaged over 4000 offsets, O with dropout matches O
    without within 6 standard errors of the per-element sample mean."""
    q, k, v, do, cu_q, cu_k = _problem(53, [4], [6], 1, 1, 3)
    ref, lse_ref = O.forward(q, k, v, cu_q, cu_k, 0.9, False)
    outs = []
    for off in range(4000):
        o, lse = O.forward(q, k, v, cu_q, cu_k, 0.9, False, dropout=(0.4, 77, off))
        assert np.array_equal(lse, lse_ref)      # the LSE ignores dropout
        outs.append(o)
    outs = np.array(outs)
    se = outs.std(axis=0) / np.sqrt(len(outs))
    assert np.all(np.abs(outs.mean(axis=0) - ref) <= 6 * se + 1e-12)


def test_dropout_unit_with_base_replays_the_whole_call():
    """One (sequence, KV-head group) evaluated alone with drop_base = (its
    sequence, its first head, all heads) gives exactly the whole call's
    forward and gradients there (the keep bits name the element's place in
    the whole call); without the base it draws other bits and differs."""
    lens_q, lens_k, H, Hk, D = [9, 12, 7], [11, 12, 10], 6, 2, 5
    q, k, v, do, cu_q, cu_k = _problem(54, lens_q, lens_k, H, Hk, D)
    drop = (0.4, 0x5EED, 9)
    whole = O.backward(q, k, v, do, cu_q, cu_k, 0.7, True, dropout=drop)
    o_whole, lse_whole = O.forward(q, k, v, cu_q, cu_k, 0.7, True, dropout=drop)
    G = H // Hk
    for s, g in [(1, 1), (2, 0)]:
        qs, ks = slice(cu_q[s], cu_q[s + 1]), slice(cu_k[s], cu_k[s + 1])
        heads = list(range(g * G, (g + 1) * G))
        args = (q[qs][:, heads], k[ks][:, [g]], v[ks][:, [g]])
        cu1q, cu1k = [0, lens_q[s]], [0, lens_k[s]]
        unit = O.backward(*args, do[qs][:, heads], cu1q, cu1k, 0.7, True, dropout=drop,
                          drop_base=(s, g * G, H))
        assert np.array_equal(unit["dq"], whole["dq"][qs][:, heads])
        o, lse = O.forward(*args, cu1q, cu1k, 0.7, True, dropout=drop, drop_base=(s, g * G, H))
        assert np.array_equal(o, o_whole[qs][:, heads])
        assert np.array_equal(lse, lse_whole[qs][:, heads])
        # dK, dV of the whole call sum the group's heads only
        assert np.array_equal(unit["dk"], whole["dk"][ks][:, [g]])
        assert np.array_equal(unit["dv"], whole["dv"][ks][:, [g]])
        other = O.backward(*args, do[qs][:, heads], cu1q, cu1k, 0.7, True, dropout=drop)
        assert np.abs(other["dv"] - unit["dv"]).max() > 0.1 * np.abs(unit["dv"]).max()
    with pytest.raises(RuntimeError):
        O.backward(q, k, v, do, cu_q, cu_k, 0.7, True, dropout=drop, drop_base=(0, 1, H))


SUM_CASES = [
    # (lens_q, lens_k, H, Hk, D, causal, window, dropout)
    ([6, 9], [8, 7], 4, 2, 5, True, (-1, -1), None),
    ([11], [6], 2, 1, 4, True, (-1, -1), None),            # rows without keys
    ([10], [12], 2, 2, 3, False, (3, 2), None),
    ([9, 7], [9, 10], 4, 1, 4, True, (-1, -1), (0.3, 77, 5)),
]


@pytest.mark.parametrize("case", SUM_CASES)
@pytest.mark.parametrize("mode", ["contracted", "explicit"])
def test_key_gradient_sums_to_zero_and_value_gradient_to_summed_dout(case, mode):
    """Each row of dS sums to zero (P's rows sum to one; under dropout the
    row term is sum_j P M dP, which cancels it too), so sum_j dK_j = 0 per
    sequence and KV head; without dropout sum_j dV_j is the sum of dO over
    the group's rows that see a key."""
    lq, lk, H, Hk, D, causal, window, drop = case
    q, k, v, do, cu_q, cu_k = _problem(55, lq, lk, H, Hk, D)
    g = O.backward(q, k, v, do, cu_q, cu_k, 0.7, causal, mode=mode, window=window,
                   dropout=drop)
    _, lse = O.forward(q, k, v, cu_q, cu_k, 0.7, causal, window=window)
    G = H // Hk
    for s in range(len(lq)):
        ks, qs = slice(cu_k[s], cu_k[s + 1]), slice(cu_q[s], cu_q[s + 1])
        for kh in range(Hk):
            dk = g["dk"][ks, kh]
            assert np.abs(dk.sum(0)).max() <= 1e-12 * max(1.0, np.abs(dk).sum(0).max())
            if drop is None:
                heads = range(kh * G, (kh + 1) * G)
                want = sum((do[qs, h] * np.isfinite(lse[qs, h])[:, None]).sum(0) for h in heads)
                dv = g["dv"][ks, kh]
                assert np.abs(dv.sum(0) - want).max() <= 1e-12 * max(1.0, np.abs(dv).sum(0).max())
