"""ctypes wrapper of the fp64 CPU attention oracle.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  The GPU product path never imports it.

Every array is numpy fp64 in the oracle's packed, tokens-major layout:
q, dout, out, dq: [total_q, H, D]; k, v, dk, dv: [total_k, Hk, D];
lse, dj: [total_q, H].  cu_q / cu_k are the int64 row offsets of each
sequence (a dense batch of B equal-length sequences is cu = [0, S, 2S, ...]).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        common = [ctypes.c_int, _i64p, _i64p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_double, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint64, _i64p,
                  _dp]
        lib.oracle_forward.argtypes = common + [_dp, _dp, _dp, _dp, _dp]
        lib.oracle_backward.argtypes = common + [_dp] * 4 + [_dp] * 3 + [_dp, _dp]
        lib.oracle_backward_explicit.argtypes = common + [_dp] * 4 + [_dp] * 3 + [_dp, _dp]
        lib.oracle_rowdot.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      _dp, _dp, _dp]
        for f in (lib.oracle_forward, lib.oracle_backward,
                  lib.oracle_backward_explicit, lib.oracle_rowdot):
            f.restype = ctypes.c_int
        u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_dropout_mask.argtypes = [ctypes.c_double, ctypes.c_uint64, ctypes.c_uint64,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_uint8)]
        lib.oracle_dropout_mask.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _LIB = lib
    return _LIB


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _cu(cu):
    return np.ascontiguousarray(cu, dtype=np.int64)


def _shapes(q, k, cu_q, cu_k):
    if q.ndim != 3 or k.ndim != 3:
        raise ValueError("q and k must be [total, heads, dim]")
    total_q, H, D = q.shape
    total_k, Hk, Dk = k.shape
    if Dk != D or H % Hk:
        raise ValueError("bad head dims / head counts")
    if cu_q[-1] != total_q or cu_k[-1] != total_k or len(cu_q) != len(cu_k):
        raise ValueError("cu_seqlens do not match the packed rows")
    return len(cu_q) - 1, H, Hk, D


def num_threads() -> int:
    return int(_lib().oracle_num_threads())


def _drop(dropout, drop_base=None):
    """dropout = None or (p, seed, offset), drop_base = None or (b0, h0, hc)
    -> the four C arguments (a pointer from ndarray.ctypes.data_as holds a
    reference to its array)."""
    base = None
    if drop_base is not None:
        base = np.ascontiguousarray(np.array(drop_base, dtype=np.int64))
        if base.shape != (3,):
            raise ValueError("drop_base is (b0, h0, hc)")
    bp = None if base is None else base.ctypes.data_as(_i64p)
    if dropout is None:
        return 0.0, 0, 0, bp
    p, seed, offset = dropout
    return float(p), int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), bp


def forward(q, k, v, cu_q, cu_k, scale, causal, mask=None, window=(-1, -1), softcap=0.0,
            dropout=None, drop_base=None):
    """Returns (out [total_q,H,D], lse [total_q,H]) in fp64.  window =
    (left, right): query i sees keys i + Lk - Lq - left .. i + Lk - Lq + right
    (a negative size leaves that side unbounded).  softcap c > 0: every
    scaled score x becomes c * tanh(x / c) (LSE of the capped scores).
    dropout = (p, seed, offset): O uses P * Z / (1 - p) with the keep bits Z
    of dropout_mask (the LSE is that of the undropped scores).  drop_base =
    (b0, h0, hc): these sequences and heads replay the bits of sequences
    b0.. and heads h0.. of an hc-head call."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu_q, cu_k = _cu(cu_q), _cu(cu_k)
    nseq, H, Hk, D = _shapes(q, k, cu_q, cu_k)
    mask = None if mask is None else _f64(mask)
    out = np.empty(q.shape, np.float64)
    lse = np.empty(q.shape[:2], np.float64)
    rc = _lib().oracle_forward(nseq, cu_q.ctypes.data_as(_i64p), cu_k.ctypes.data_as(_i64p),
                               H, Hk, D, float(scale), int(bool(causal)), int(window[0]),
                               int(window[1]), float(softcap), *_drop(dropout, drop_base),
                               _ptr(mask), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse))
    if rc:
        raise RuntimeError("oracle_forward failed (%d)" % rc)
    return out, lse


def backward(q, k, v, dout, cu_q, cu_k, scale, causal, mask=None,
             mode="contracted", want_ds=False, window=(-1, -1), softcap=0.0, dropout=None,
             drop_base=None):
    """Exact attention gradient in fp64.

    mode="contracted": any size; mode="explicit": materialised softmax
    Jacobian, small inputs only (want_ds=True returns dS [H, Lq, Lk] for a
    single sequence).  drop_base as in forward().  Returns a dict with dq, dk, dv, dj (sum_k P_ik dP_ik)
    and, in contracted mode, lse; in explicit mode with want_ds, ds.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu_q, cu_k = _cu(cu_q), _cu(cu_k)
    nseq, H, Hk, D = _shapes(q, k, cu_q, cu_k)
    if dout.shape != q.shape or v.shape != k.shape:
        raise ValueError("dout/v shape mismatch")
    mask = None if mask is None else _f64(mask)
    dq = np.empty(q.shape, np.float64)
    dk = np.empty(k.shape, np.float64)
    dv = np.empty(k.shape, np.float64)
    dj = np.empty(q.shape[:2], np.float64)
    res = {"dq": dq, "dk": dk, "dv": dv, "dj": dj}
    lib = _lib()
    common = (nseq, cu_q.ctypes.data_as(_i64p), cu_k.ctypes.data_as(_i64p), H, Hk, D,
              float(scale), int(bool(causal)), int(window[0]), int(window[1]), float(softcap),
              *_drop(dropout, drop_base), _ptr(mask),
              _ptr(q), _ptr(k), _ptr(v),
              _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv))
    if mode == "contracted":
        lse = np.empty(q.shape[:2], np.float64)
        rc = lib.oracle_backward(*common, _ptr(dj), _ptr(lse))
        res["lse"] = lse
    elif mode == "explicit":
        ds = None
        if want_ds:
            if nseq != 1:
                raise ValueError("want_ds needs a single sequence")
            ds = np.empty((H, int(cu_q[1]), int(cu_k[1])), np.float64)
            res["ds"] = ds
        rc = lib.oracle_backward_explicit(*common, _ptr(ds), _ptr(dj))
    else:
        raise ValueError(mode)
    if rc:
        raise RuntimeError("oracle backward failed (%d)" % rc)
    return res


def rowdot(dout, out):
    """sum_d dout * out per (row, head), fp64, with `out` exactly as given."""
    dout, out = _f64(dout), _f64(out)
    if dout.shape != out.shape or dout.ndim != 3:
        raise ValueError("shape mismatch")
    T, H, D = dout.shape
    res = np.empty((T, H), np.float64)
    rc = _lib().oracle_rowdot(T, H, D, _ptr(dout), _ptr(out), _ptr(res))
    if rc:
        raise RuntimeError("oracle_rowdot failed")
    return res


def philox4x32_10(ctr, key):
    """Philox4x32-10 of a 4-word counter and a 2-word key -> 4 uint32 words."""
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    kk = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (ctypes.c_uint32 * 4)()
    _lib().oracle_philox4x32_10(c, kk, out)
    return [int(x) for x in out]


def dropout_mask(p, seed, offset, b, h, H, Lq, Lk):
    """Keep bits (uint8 0/1, [Lq, Lk]) of sequence b, query head h of H."""
    m = np.empty((Lq, Lk), np.uint8)
    rc = _lib().oracle_dropout_mask(float(p), int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                                    int(b), int(h), int(H), int(Lq), int(Lk),
                                    m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    if rc:
        raise RuntimeError("oracle_dropout_mask failed")
    return m
