"""Python binding of the MI355X attention C ABI (include/fa_bwd.h for the
backward, include/fa_fwd.h for the forward).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step runs in the library's gfx950 kernels.
There is no CPU fallback -- if the built library is missing this module
raises instead of computing anything.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_bwd.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
FA_DTYPE_BF16, FA_DTYPE_F16 = 0, 1
_DTYPES = {torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_F16}
_STATUS = {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED",
           3: "FA_ERR_WORKSPACE", 4: "FA_ERR_HIP"}


class FaBwdArgs(ctypes.Structure):
    """Mirror of fa_bwd_args."""
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("num_heads_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
        ("dout", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("do_stride", ctypes.c_int64 * 3), ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
        ("dq_stride", ctypes.c_int64 * 3), ("dk_stride", ctypes.c_int64 * 3),
        ("dv_stride", ctypes.c_int64 * 3),
        ("lse_stride", ctypes.c_int64 * 2),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("local_window", ctypes.c_int32),
        ("window_size_left", ctypes.c_int32),
        ("window_size_right", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("dropout_p", ctypes.c_float),
        ("philox_seed", ctypes.c_uint64),
        ("philox_offset", ctypes.c_uint64),
        ("deterministic", ctypes.c_int32),
        ("dq_accumulate", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("dropout_keep_max_bytes", ctypes.c_size_t),
        ("dropout_keep", ctypes.c_void_p),
        ("dropout_keep_bytes", ctypes.c_size_t),
    ]


class FaBwdWsLayout(ctypes.Structure):
    """Mirror of fa_bwd_ws_layout."""
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("head_dim_pad", ctypes.c_int32),
        ("q_tile", ctypes.c_int32),
        ("k_tile", ctypes.c_int32),
        ("off_lse2", ctypes.c_size_t), ("off_rowdot", ctypes.c_size_t),
        ("off_dq_acc", ctypes.c_size_t), ("off_turns", ctypes.c_size_t),
        ("off_flags", ctypes.c_size_t), ("off_keep", ctypes.c_size_t),
        ("keep_words", ctypes.c_int32),
        ("total_bytes", ctypes.c_size_t),
    ]


class FaFwdArgs(ctypes.Structure):
    """Mirror of fa_fwd_args."""
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("num_heads_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("lse_stride", ctypes.c_int64 * 2),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("local_window", ctypes.c_int32),
        ("window_size_left", ctypes.c_int32),
        ("window_size_right", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("dropout_p", ctypes.c_float),
        ("philox_seed", ctypes.c_uint64),
        ("philox_offset", ctypes.c_uint64),
        ("dropout_keep_out", ctypes.c_void_p),
        ("dropout_keep_out_bytes", ctypes.c_size_t),
    ]


EXPORTED = ("fa_bwd", "fa_bwd_preprocess", "fa_bwd_main", "fa_bwd_dq", "fa_bwd_dq_convert",
            "fa_bwd_debug_rowsum", "fa_bwd_noalloc", "fa_bwd_validate", "fa_bwd_workspace_size",
            "fa_bwd_workspace_layout", "fa_bwd_last_error", "fa_bwd_abi_version", "fa_fwd",
            "fa_fwd_validate", "fa_fwd_keep_bytes", "fa_probe_mfma_rate")

_LIB = None


def load_library(path: str = LIB_PATH):
    """Load the built library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            "libfa_bwd.so is not built (run python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(FaBwdArgs)
    for name in ("fa_bwd", "fa_bwd_preprocess", "fa_bwd_main", "fa_bwd_dq", "fa_bwd_dq_convert",
                 "fa_bwd_noalloc"):
        f = getattr(lib, name)
        f.argtypes = [P, ctypes.c_void_p]
        f.restype = ctypes.c_int
    lib.fa_bwd_debug_rowsum.argtypes = [P, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_bwd_debug_rowsum.restype = ctypes.c_int
    lib.fa_bwd_validate.argtypes = [P]
    lib.fa_bwd_validate.restype = ctypes.c_int
    lib.fa_bwd_workspace_size.argtypes = [P]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_layout.argtypes = [P, ctypes.POINTER(FaBwdWsLayout)]
    lib.fa_bwd_workspace_layout.restype = ctypes.c_int
    lib.fa_bwd_last_error.argtypes = []
    lib.fa_bwd_last_error.restype = ctypes.c_char_p
    lib.fa_bwd_abi_version.argtypes = []
    lib.fa_bwd_abi_version.restype = ctypes.c_int32
    PF = ctypes.POINTER(FaFwdArgs)
    lib.fa_fwd.argtypes = [PF, ctypes.c_void_p]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd_validate.argtypes = [PF]
    lib.fa_fwd_validate.restype = ctypes.c_int
    lib.fa_fwd_keep_bytes.argtypes = [PF]
    lib.fa_fwd_keep_bytes.restype = ctypes.c_size_t
    lib.fa_probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_mfma_rate.restype = ctypes.c_int
    _LIB = lib
    return lib


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_STATUS.get(status, status), msg))
        self.status = status


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _strides3(t: torch.Tensor, varlen: bool):
    s = t.stride()
    if varlen:   # (total, H, D)
        return (0, s[0], s[1])
    return (s[0], s[1], s[2])


@dataclass
class Problem:
    """Shapes of one backward call (derived from the tensors)."""
    batch: int
    seqlen_q: int
    seqlen_k: int
    heads: int
    heads_k: int
    head_dim: int
    varlen: bool
    total_q: int = 0
    total_k: int = 0


def _set_window(a, window):
    """window = None (no local window) or (left, right), negative = unbounded."""
    if window is None:
        a.local_window, a.window_size_left, a.window_size_right = 0, -1, -1
    else:
        a.local_window = 1
        a.window_size_left, a.window_size_right = int(window[0]), int(window[1])


def _set_dropout(a, dropout):
    """dropout = None or (p, seed, offset): the forward's rng state."""
    if dropout is None:
        a.dropout_p, a.philox_seed, a.philox_offset = 0.0, 0, 0
    else:
        p, seed, offset = dropout
        a.dropout_p = float(p)
        a.philox_seed, a.philox_offset = int(seed) & (2**64 - 1), int(offset) & (2**64 - 1)


def make_args(dout, q, k, v, out, lse, dq, dk, dv, softmax_scale, causal,
              cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
              max_seqlen_k=None, deterministic=False, workspace=None,
              dq_accumulate=False, window=None, softcap=0.0, dropout=None,
              dropout_keep_max_bytes=0, dropout_keep=None) -> FaBwdArgs:
    """Fill fa_bwd_args from tensors.  Dense tensors are (B, S, H, D); packed
    ones (total, H, D) with int32 device cu_seqlens and host max lengths.
    dq_accumulate=False: dQ by the separate query-tile pass (default);
    True: dQ partials accumulated in fp32 by the key-tile pass (atomic, or
    ordered when deterministic) and converted afterwards.
    dropout_keep_max_bytes: bound on the dropout keep-bit region of the
    workspace (0: the library's default).
    dropout_keep: the keep words a forward call wrote (a device tensor, see
    make_fwd_args), read instead of drawing the bits."""
    varlen = cu_seqlens_q is not None or cu_seqlens_k is not None
    a = FaBwdArgs()
    a.dtype = _DTYPES.get(q.dtype, 99)
    if varlen:
        if cu_seqlens_q is None or cu_seqlens_k is None:
            raise ValueError("cu_seqlens_q and cu_seqlens_k go together")
        a.batch = cu_seqlens_q.numel() - 1
        a.seqlen_q, a.seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
        a.num_heads, a.head_dim = q.shape[1], q.shape[2]
        a.num_heads_k = k.shape[1]
        a.total_q, a.total_k = q.shape[0], k.shape[0]
        a.cu_seqlens_q, a.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    else:
        a.batch, a.seqlen_q, a.num_heads, a.head_dim = q.shape
        a.seqlen_k, a.num_heads_k = k.shape[1], k.shape[2]
    for t in (dout, q, k, v, out, dq, dk, dv):
        if t.stride(-1) != 1:
            raise ValueError("the head_dim stride must be 1")
    a.dout, a.q, a.k, a.v, a.out = (_ptr(x) for x in (dout, q, k, v, out))
    a.lse = _ptr(lse)
    a.dq, a.dk, a.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    for name, t in (("do_stride", dout), ("q_stride", q), ("k_stride", k), ("v_stride", v),
                    ("o_stride", out), ("dq_stride", dq), ("dk_stride", dk),
                    ("dv_stride", dv)):
        getattr(a, name)[:] = _strides3(t, varlen)
    a.lse_stride[:] = (lse.stride(0), lse.stride(1))
    a.softmax_scale = float(softmax_scale)
    a.causal = int(bool(causal))
    _set_window(a, window)
    a.softcap = float(softcap)
    _set_dropout(a, dropout)
    a.deterministic = int(bool(deterministic))
    a.dq_accumulate = int(bool(dq_accumulate))
    a.dropout_keep_max_bytes = int(dropout_keep_max_bytes)
    if dropout_keep is not None:
        a.dropout_keep = dropout_keep.data_ptr()
        a.dropout_keep_bytes = dropout_keep.numel() * dropout_keep.element_size()
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def _check(status: int):
    if status != FA_OK:
        raise FaError(status, load_library().fa_bwd_last_error().decode())


def workspace_size(args: FaBwdArgs) -> int:
    n = load_library().fa_bwd_workspace_size(ctypes.byref(args))
    if n == 0:
        _check(load_library().fa_bwd_validate(ctypes.byref(args)) or FA_ERR_INVALID_ARG)
    return n


def workspace_layout(args: FaBwdArgs) -> FaBwdWsLayout:
    out = FaBwdWsLayout()
    _check(load_library().fa_bwd_workspace_layout(ctypes.byref(args), ctypes.byref(out)))
    return out


def validate(args: FaBwdArgs) -> int:
    return load_library().fa_bwd_validate(ctypes.byref(args))


def alloc_workspace(args: FaBwdArgs, device) -> torch.Tensor:
    """Caller-side workspace (torch allocation; the library never allocates).
    torch's caching allocator returns 256-byte aligned blocks."""
    n = workspace_size(args)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    args.workspace = ws.data_ptr()
    args.workspace_bytes = n
    return ws


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def run(args: FaBwdArgs, step: str = "all", stream=None):
    """Enqueue one of 'all', 'preprocess', 'main', 'dq', 'dq_convert', or
    'noalloc' (the whole backward on the library's scratch array; the
    args' workspace is ignored)."""
    lib = load_library()
    f = {"all": lib.fa_bwd, "preprocess": lib.fa_bwd_preprocess, "main": lib.fa_bwd_main,
         "dq": lib.fa_bwd_dq, "dq_convert": lib.fa_bwd_dq_convert,
         "noalloc": lib.fa_bwd_noalloc}[step]
    _check(f(ctypes.byref(args), _stream(stream)))


def debug_rowsum(args: FaBwdArgs, d_out: torch.Tensor, stream=None):
    """Enqueue fa_bwd_debug_rowsum: the preprocess step, also writing
    D = rowsum(dO * O) into d_out, an fp32 tensor with the lse tensor's
    shape and strides."""
    if d_out.dtype != torch.float32:
        raise ValueError("d_out must be float32")
    _check(load_library().fa_bwd_debug_rowsum(ctypes.byref(args), d_out.data_ptr(),
                                              _stream(stream)))


def ordered_wait_gave_up(args: FaBwdArgs, workspace: torch.Tensor) -> bool:
    """True if an ordered (deterministic accumulate-mode) wait of the last
    call on this workspace gave up -- its dq is then not bit-reproducible.
    Reads flags[0] of the workspace (synchronizes with the device)."""
    off = workspace_layout(args).off_flags
    return int(workspace[off:off + 4].view(torch.int32).item()) != 0


def fa_bwd(dout, q, k, v, out, lse, dq, dk, dv, softmax_scale, causal,
           cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
           deterministic=False, workspace=None, stream=None, dq_accumulate=False,
           window=None, softcap=0.0, dropout=None, dropout_keep=None):
    """dQ, dK, dV of attention, written into dq, dk, dv (same layouts as q, k, v).

    lse is the forward's natural-log log-sum-exp, (B, H, Sq) fp32 (packed:
    (num_seqs, H, max_seqlen_q)).  Returns the workspace tensor used (it
    holds the fp32 dQ accumulator and the row sums afterwards).
    With dq_accumulate and deterministic both set, the call waits for the
    device and raises if an ordered wait gave up (dq would then not be
    bit-reproducible).  dropout_keep: the forward's keep words (fa_fwd with
    keep=True), read instead of drawing the bits."""
    args = make_args(dout, q, k, v, out, lse, dq, dk, dv, softmax_scale, causal,
                     cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                     deterministic, workspace, dq_accumulate, window, softcap, dropout,
                     dropout_keep=dropout_keep)
    if workspace is None:
        workspace = alloc_workspace(args, q.device)
    run(args, "all", stream)
    if deterministic and dq_accumulate and ordered_wait_gave_up(args, workspace):
        raise FaError(FA_ERR_HIP, "an ordered dQ wait gave up: dq is not bit-reproducible")
    return workspace


def make_fwd_args(q, k, v, out, lse, softmax_scale, causal, cu_seqlens_q=None,
                  cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
                  window=None, softcap=0.0, dropout=None, keep_out=None) -> FaFwdArgs:
    """Fill fa_fwd_args from tensors (layouts as in make_args).  keep_out: a
    device tensor of at least keep_bytes() bytes that receives the dropout
    keep words for the backward's dropout_keep."""
    varlen = cu_seqlens_q is not None or cu_seqlens_k is not None
    a = FaFwdArgs()
    a.dtype = _DTYPES.get(q.dtype, 99)
    if varlen:
        if cu_seqlens_q is None or cu_seqlens_k is None:
            raise ValueError("cu_seqlens_q and cu_seqlens_k go together")
        a.batch = cu_seqlens_q.numel() - 1
        a.seqlen_q, a.seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
        a.num_heads, a.head_dim = q.shape[1], q.shape[2]
        a.num_heads_k = k.shape[1]
        a.total_q, a.total_k = q.shape[0], k.shape[0]
        a.cu_seqlens_q, a.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    else:
        a.batch, a.seqlen_q, a.num_heads, a.head_dim = q.shape
        a.seqlen_k, a.num_heads_k = k.shape[1], k.shape[2]
    for t in (q, k, v, out):
        if t.stride(-1) != 1:
            raise ValueError("the head_dim stride must be 1")
    a.q, a.k, a.v, a.out = (_ptr(x) for x in (q, k, v, out))
    a.lse = _ptr(lse)
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        getattr(a, name)[:] = _strides3(t, varlen)
    a.lse_stride[:] = (lse.stride(0), lse.stride(1))
    a.softmax_scale = float(softmax_scale)
    a.causal = int(bool(causal))
    _set_window(a, window)
    a.softcap = float(softcap)
    _set_dropout(a, dropout)
    if keep_out is not None:
        a.dropout_keep_out = keep_out.data_ptr()
        a.dropout_keep_out_bytes = keep_out.numel() * keep_out.element_size()
    return a


def keep_bytes(args: FaFwdArgs) -> int:
    """Bytes of the dropout keep words of a forward call (0 without dropout)."""
    return int(load_library().fa_fwd_keep_bytes(ctypes.byref(args)))


def validate_fwd(args: FaFwdArgs) -> int:
    return load_library().fa_fwd_validate(ctypes.byref(args))


def run_fwd(args: FaFwdArgs, stream=None):
    """Enqueue the forward."""
    _check(load_library().fa_fwd(ctypes.byref(args), _stream(stream)))


def fa_fwd(q, k, v, out, lse, softmax_scale, causal, cu_seqlens_q=None, cu_seqlens_k=None,
           max_seqlen_q=None, max_seqlen_k=None, stream=None, window=None, softcap=0.0,
           dropout=None, keep=False):
    """O and the natural-log LSE of attention, written into out (layout of q)
    and lse ((B, H, Sq) fp32; packed: (num_seqs, H, max_seqlen_q)).  With
    dropout and keep=True, also the keep words for the backward's
    dropout_keep: returns them (a uint32 device tensor), else None."""
    args = make_fwd_args(q, k, v, out, lse, softmax_scale, causal, cu_seqlens_q, cu_seqlens_k,
                         max_seqlen_q, max_seqlen_k, window, softcap, dropout)
    words = None
    if keep and dropout is not None and float(dropout[0]) > 0.0:
        n = keep_bytes(args)
        if n == 0:
            _check(validate_fwd(args) or FA_ERR_INVALID_ARG)
        words = torch.empty((n + 3) // 4, dtype=torch.int32, device=q.device)
        args.dropout_keep_out = words.data_ptr()
        args.dropout_keep_out_bytes = words.numel() * 4
    run_fwd(args, stream)
    return words
