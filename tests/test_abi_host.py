"""Host-only checks of the C ABI: the built library loads, exports every
function include/*.h declares, and rejects bad arguments with the right
status before touching the GPU.  Fake (never dereferenced) aligned addresses
stand in for device pointers."""
import ctypes
import glob
import os
import re

import pytest

import attention_backward_fa2_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_bwd.h")
FWD_HEADER = os.path.join(ROOT, "include", "fa_fwd.h")


def _declared_functions():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(fa_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = fa.load_library()
    names = _declared_functions()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fa.EXPORTED)
    assert lib.fa_bwd_abi_version() == 10


@pytest.mark.parametrize("header,struct,mirror", [
    (HEADER, "fa_bwd_args", fa.FaBwdArgs),
    (FWD_HEADER, "fa_fwd_args", fa.FaFwdArgs),
])
def test_struct_mirror_matches_header_field_order(header, struct, mirror):
    text = open(header).read()
    body = text[text.index("typedef struct " + struct):text.index("} %s;" % struct)]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    decl = re.findall(r"(\*?\w+)(?:\[\d\])?\s*[,;]", body)
    names = [d.lstrip("*") for d in decl]
    assert names == [f[0] for f in mirror._fields_]


BASE = 0x7f0000000000


def _args(**over):
    a = fa.FaBwdArgs()
    a.dtype = fa.FA_DTYPE_BF16
    a.batch, a.seqlen_q, a.seqlen_k = 2, 256, 384
    a.num_heads, a.num_heads_k, a.head_dim = 8, 2, 128
    H, Hk, D, Sq, Sk = 8, 2, 128, 256, 384
    addr = BASE
    for name in ("dout", "q", "k", "v", "out", "lse", "dq", "dk", "dv"):
        setattr(a, name, addr)
        addr += 1 << 30
    for name in ("do_stride", "q_stride", "o_stride", "dq_stride"):
        getattr(a, name)[:] = (Sq * H * D, H * D, D)
    for name in ("k_stride", "v_stride", "dk_stride", "dv_stride"):
        getattr(a, name)[:] = (Sk * Hk * D, Hk * D, D)
    a.lse_stride[:] = (H * Sq, Sq)
    a.softmax_scale = D ** -0.5
    a.causal = 1
    for k, v in over.items():
        if isinstance(getattr(a, k), ctypes.Array):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


def _with_ws(a):
    n = fa.workspace_size(a)
    a.workspace = BASE + (40 << 30)
    a.workspace_bytes = n
    return a


def test_workspace_layout_formula():
    a = _args(dq_accumulate=1)
    lay = fa.workspace_layout(a)
    rows = 2 * 256
    assert lay.rows == rows and lay.head_dim_pad == 128
    assert lay.q_tile == 64 and lay.k_tile == 128

    def al(x):
        return (x + 255) // 256 * 256
    assert lay.off_lse2 == 0
    assert lay.off_rowdot == al(8 * rows * 4)
    assert lay.off_dq_acc == lay.off_rowdot + al(8 * rows * 4)
    assert lay.off_turns == lay.off_dq_acc + al(8 * rows * 128 * 4)
    assert lay.off_flags == lay.off_turns + al(2 * 8 * 4 * 4)
    assert lay.total_bytes == lay.off_flags + 256
    assert fa.workspace_size(a) == lay.total_bytes


@pytest.mark.parametrize("d,pad", [(8, 64), (64, 64), (72, 96), (96, 96), (104, 128),
                                   (128, 128), (136, 192), (192, 192), (200, 256), (256, 256)])
def test_head_dim_padding(d, pad):
    a = _args(head_dim=d, do_stride=(256 * 8 * d, 8 * d, d), q_stride=(256 * 8 * d, 8 * d, d),
              o_stride=(256 * 8 * d, 8 * d, d), dq_stride=(256 * 8 * d, 8 * d, d),
              k_stride=(384 * 2 * d, 2 * d, d), v_stride=(384 * 2 * d, 2 * d, d),
              dk_stride=(384 * 2 * d, 2 * d, d), dv_stride=(384 * 2 * d, 2 * d, d))
    assert fa.workspace_layout(a).head_dim_pad == pad


def test_separate_dq_mode_needs_no_accumulator():
    a = _args()
    lay = fa.workspace_layout(a)
    rows = 2 * 256

    def al(x):
        return (x + 255) // 256 * 256
    assert lay.off_dq_acc == lay.off_turns == lay.off_flags == 2 * al(8 * rows * 4)
    assert lay.total_bytes == lay.off_flags + 256


def test_dropout_keep_region_in_the_separate_dq_mode_only():
    """With dropout, the separate-dQ backward keeps one 32-key word per (key
    word, head, row): 2 * ceil(seqlen_k / 64) words, after the flags; the
    accumulate mode and calls without dropout have none."""
    def al(x):
        return (x + 255) // 256 * 256
    rows = 2 * 256
    lay = fa.workspace_layout(_args(dropout_p=0.1))
    assert lay.keep_words == 2 * ((384 + 63) // 64) == 12
    assert lay.off_keep == lay.off_flags + 256
    assert lay.total_bytes == lay.off_keep + al(12 * 8 * rows * 4)
    # the bound: at it the region exists, one byte below it does not
    need = 12 * 8 * rows * 4
    assert fa.workspace_layout(_args(dropout_p=0.1, dropout_keep_max_bytes=need)).keep_words == 12
    for over in ({"dropout_p": 0.1, "dq_accumulate": 1}, {"dropout_p": 0.0},
                 {"dropout_p": 0.1, "dropout_keep_max_bytes": need - 1}):
        lay = fa.workspace_layout(_args(**over))
        assert lay.keep_words == 0 and lay.total_bytes == lay.off_keep == lay.off_flags + 256


def test_forward_keep_words_need_no_keep_region():
    """Given the forward's keep words, the separate-dQ backward reads them:
    its workspace has no keep region.  The words are checked for alignment,
    size (2 * ceil(seqlen_k / 64) words per row of every head) and 31-bit
    addressability before anything touches the GPU; without dropout or in
    the accumulate mode they are ignored."""
    rows = 2 * 256
    need = 12 * 8 * rows * 4
    ok = _args(dropout_p=0.1, dropout_keep=BASE + (50 << 30), dropout_keep_bytes=need)
    lay = fa.workspace_layout(ok)
    assert lay.keep_words == 0 and lay.total_bytes == lay.off_keep == lay.off_flags + 256
    assert fa.validate(_with_ws(ok)) == fa.FA_OK
    for over, status in (({"dropout_keep_bytes": need - 1}, fa.FA_ERR_INVALID_ARG),
                         ({"dropout_keep": BASE + (50 << 30) + 2}, fa.FA_ERR_INVALID_ARG)):
        a = _args(dropout_p=0.1, dropout_keep=BASE + (50 << 30), dropout_keep_bytes=need)
        for k, v in over.items():
            setattr(a, k, v)
        assert fa.load_library().fa_bwd_workspace_size(ctypes.byref(a)) == 0
        assert fa.validate(a) == status
    # ignored without dropout and in the accumulate mode (a bad pointer passes)
    for over in ({"dropout_p": 0.0}, {"dropout_p": 0.1, "dq_accumulate": 1}):
        a = _args(dropout_keep=BASE + 2, dropout_keep_bytes=1, **over)
        assert fa.validate(_with_ws(a)) == fa.FA_OK
    # num_heads * rows at 2^29 and above: the 31-bit word offsets would overflow
    big = _args(batch=1 << 16, seqlen_q=1 << 10, seqlen_k=64, num_heads=8, dropout_p=0.1,
                dropout_keep=BASE, dropout_keep_bytes=1 << 40,
                do_stride=(1024 * 8 * 128, 8 * 128, 128), q_stride=(1024 * 8 * 128, 8 * 128, 128),
                o_stride=(1024 * 8 * 128, 8 * 128, 128), dq_stride=(1024 * 8 * 128, 8 * 128, 128),
                lse_stride=(8 * 1024, 1024))
    assert fa.load_library().fa_bwd_workspace_size(ctypes.byref(big)) == 0
    assert fa.validate(big) == fa.FA_ERR_UNSUPPORTED


def test_step_entry_points_check_the_dq_mode_before_launching():
    lib = fa.load_library()
    a = _with_ws(_args())
    assert lib.fa_bwd_dq_convert(ctypes.byref(a), None) == fa.FA_ERR_INVALID_ARG
    b = _with_ws(_args(dq_accumulate=1))
    assert lib.fa_bwd_dq(ctypes.byref(b), None) == fa.FA_ERR_INVALID_ARG
    c = _args(dq_accumulate=2)
    c.workspace, c.workspace_bytes = BASE + (40 << 30), 1 << 40
    assert lib.fa_bwd(ctypes.byref(c), None) == fa.FA_ERR_INVALID_ARG


def test_valid_args_pass_validation():
    assert fa.validate(_with_ws(_args())) == fa.FA_OK
    assert fa.validate(_with_ws(_args(dtype=fa.FA_DTYPE_F16))) == fa.FA_OK
    # local windows: causal with a left size (right 0 or unbounded), and
    # two-sided windows without causal, huge sizes included
    for causal, left, right in [(1, 16, 0), (1, 3, -1), (0, -1, 8), (0, 5, 7), (0, 1 << 30, 2**31 - 1)]:
        a = _with_ws(_args(causal=causal, local_window=1, window_size_left=left,
                           window_size_right=right))
        assert fa.validate(a) == fa.FA_OK
    # without local_window the sizes are not read (a zero-filled struct has
    # no window, and causal with a positive right size is no error then)
    assert fa.validate(_with_ws(_args(causal=1, window_size_right=5))) == fa.FA_OK
    # soft cap: any finite positive value, 0 = off
    for cap in (0.0, 1e-30, 30.0, 1e30):
        assert fa.validate(_with_ws(_args(softcap=cap))) == fa.FA_OK
    # dropout: p in [0, 1), any seed and offset
    for pd in (0.0, 0.1, 0.999):
        a = _with_ws(_args(dropout_p=pd, philox_seed=2**64 - 1, philox_offset=2**63))
        assert fa.validate(a) == fa.FA_OK


@pytest.mark.parametrize("over,status", [
    ({"num_heads_k": 3}, fa.FA_ERR_INVALID_ARG),          # H % Hk != 0
    ({"q": 0}, fa.FA_ERR_INVALID_ARG),                    # null pointer
    ({"lse": 0}, fa.FA_ERR_INVALID_ARG),
    ({"dk": BASE + 8}, fa.FA_ERR_INVALID_ARG),            # misaligned
    ({"q_stride": (256 * 8 * 128, 8 * 128 + 4, 128)}, fa.FA_ERR_INVALID_ARG),
    ({"do_stride": (256 * 64, 64, 128 * 256)}, fa.FA_ERR_INVALID_ARG),   # rows overlap
    ({"k_stride": (1 << 30, 1 << 24, 128)}, fa.FA_ERR_UNSUPPORTED),      # 32-bit tile offsets
    ({"batch": -1}, fa.FA_ERR_INVALID_ARG),
    ({"head_dim": 0}, fa.FA_ERR_INVALID_ARG),
    ({"causal": 2}, fa.FA_ERR_INVALID_ARG),
    ({"causal": 1, "local_window": 1, "window_size_right": 4}, fa.FA_ERR_INVALID_ARG),
    ({"local_window": 2}, fa.FA_ERR_INVALID_ARG),
    ({"softcap": -1.0}, fa.FA_ERR_INVALID_ARG),
    ({"dropout_p": 1.0}, fa.FA_ERR_INVALID_ARG),
    ({"dropout_p": -0.1}, fa.FA_ERR_INVALID_ARG),
    ({"dropout_p": float("nan")}, fa.FA_ERR_INVALID_ARG),
    ({"softcap": float("nan")}, fa.FA_ERR_INVALID_ARG),
    ({"softcap": float("inf")}, fa.FA_ERR_INVALID_ARG),
    ({"seqlen_k": (1 << 29) + 1}, fa.FA_ERR_UNSUPPORTED),
    ({"softmax_scale": float("nan")}, fa.FA_ERR_INVALID_ARG),
    ({"cu_seqlens_q": BASE}, fa.FA_ERR_INVALID_ARG),      # only one cu_seqlens
    ({"dtype": 2}, fa.FA_ERR_UNSUPPORTED),
    ({"head_dim": 300}, fa.FA_ERR_UNSUPPORTED),
    ({"head_dim": 100}, fa.FA_ERR_UNSUPPORTED),           # not a multiple of 8
    ({"head_dim": 264}, fa.FA_ERR_UNSUPPORTED),           # > 256
    ({"head_dim": 192, "dq_accumulate": 1}, fa.FA_ERR_UNSUPPORTED),   # fused dQ: <= 128
])
def test_validation_errors(over, status):
    a = _args(**over)
    a.workspace = BASE + (40 << 30)
    a.workspace_bytes = 1 << 40
    assert fa.validate(a) == status
    assert fa.load_library().fa_bwd_last_error().decode() != ""
    assert fa.load_library().fa_bwd_workspace_size(ctypes.byref(a)) == 0


def test_workspace_errors():
    a = _args()
    assert fa.validate(a) == fa.FA_ERR_WORKSPACE            # none given
    _with_ws(a)
    a.workspace_bytes -= 1
    assert fa.validate(a) == fa.FA_ERR_WORKSPACE            # too small
    _with_ws(a)
    a.workspace += 64
    assert fa.validate(a) == fa.FA_ERR_WORKSPACE            # misaligned


def test_launch_entry_points_reject_before_touching_the_gpu():
    lib = fa.load_library()
    a = _args(num_heads_k=3)
    for name in ("fa_bwd", "fa_bwd_preprocess", "fa_bwd_main", "fa_bwd_dq", "fa_bwd_dq_convert"):
        assert getattr(lib, name)(ctypes.byref(a), None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd(None, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_debug_rowsum(ctypes.byref(a), BASE, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_debug_rowsum(None, BASE, None) == fa.FA_ERR_INVALID_ARG


def test_noalloc_rejects_before_touching_the_gpu():
    """fa_bwd_noalloc ignores the caller's workspace; a call whose workspace
    (without a dropout keep region) exceeds the library's scratch array, or
    with invalid arguments, is rejected on the host.  (No GPU here: any device
    call would fail with FA_ERR_HIP instead.)"""
    lib = fa.load_library()
    big = _args(batch=64, seqlen_q=4096, seqlen_k=4096, num_heads=32, num_heads_k=8,
                dq_accumulate=1)
    assert fa.workspace_size(big) > (64 << 20)
    assert lib.fa_bwd_noalloc(ctypes.byref(big), None) == fa.FA_ERR_WORKSPACE
    msg = lib.fa_bwd_last_error().decode()
    assert "fa_bwd_noalloc" in msg and str(64 << 20) in msg
    bad = _args(num_heads_k=3)
    assert lib.fa_bwd_noalloc(ctypes.byref(bad), None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_noalloc(None, None) == fa.FA_ERR_INVALID_ARG


def test_debug_rowsum_checks_its_output_before_touching_the_gpu():
    """fa_bwd_debug_rowsum: D_out must be given (when there are query rows)
    and 4-byte aligned; everything else is validated as for fa_bwd (a
    workspace is required)."""
    lib = fa.load_library()
    a = _args()
    _with_ws(a)
    assert lib.fa_bwd_debug_rowsum(ctypes.byref(a), None, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_debug_rowsum(ctypes.byref(a), BASE + 2, None) == fa.FA_ERR_INVALID_ARG
    b = _args()
    assert lib.fa_bwd_debug_rowsum(ctypes.byref(b), BASE, None) == fa.FA_ERR_WORKSPACE
    assert "workspace" in fa.load_library().fa_bwd_last_error().decode()


def test_varlen_layout_uses_total_rows():
    a = _args(cu_seqlens_q=BASE, cu_seqlens_k=BASE + 256, total_q=1000, total_k=1200,
              batch=5, seqlen_q=300, seqlen_k=400, dq_accumulate=1)
    lay = fa.workspace_layout(a)
    assert lay.rows == 1000
    assert lay.off_flags - lay.off_turns == ((5 * 8 * 5 * 4 + 255) // 256) * 256


def _fwd_args(**over):
    a = fa.FaFwdArgs()
    a.dtype = fa.FA_DTYPE_BF16
    a.batch, a.seqlen_q, a.seqlen_k = 2, 256, 384
    a.num_heads, a.num_heads_k, a.head_dim = 8, 2, 128
    H, Hk, D, Sq, Sk = 8, 2, 128, 256, 384
    addr = BASE
    for name in ("q", "k", "v", "out", "lse"):
        setattr(a, name, addr)
        addr += 1 << 30
    for name in ("q_stride", "o_stride"):
        getattr(a, name)[:] = (Sq * H * D, H * D, D)
    for name in ("k_stride", "v_stride"):
        getattr(a, name)[:] = (Sk * Hk * D, Hk * D, D)
    a.lse_stride[:] = (H * Sq, Sq)
    a.softmax_scale = D ** -0.5
    a.causal = 1
    for k, v in over.items():
        if isinstance(getattr(a, k), ctypes.Array):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


def test_forward_keep_bytes_and_checks():
    """fa_fwd_keep_bytes: 2 * ceil(seqlen_k / 64) words per row of every head
    (dense rows batch * seqlen_q, packed total_q), 0 without dropout or for
    invalid arguments; the output buffer is checked for alignment and size."""
    lib = fa.load_library()
    a = _fwd_args(dropout_p=0.2)
    need = 12 * 8 * (2 * 256) * 4
    assert fa.keep_bytes(a) == need
    assert fa.keep_bytes(_fwd_args()) == 0
    assert fa.keep_bytes(_fwd_args(dropout_p=0.2, num_heads_k=3)) == 0
    packed = _fwd_args(dropout_p=0.2, cu_seqlens_q=BASE, cu_seqlens_k=BASE + 256, total_q=1000,
                       total_k=1200, batch=5, seqlen_q=300, seqlen_k=700)
    assert fa.keep_bytes(packed) == 2 * 11 * 8 * 1000 * 4
    out = BASE + (50 << 30)
    assert fa.validate_fwd(_fwd_args(dropout_p=0.2, dropout_keep_out=out,
                                     dropout_keep_out_bytes=need)) == fa.FA_OK
    for ptr, n in ((out, need - 4), (out + 2, need)):
        b = _fwd_args(dropout_p=0.2, dropout_keep_out=ptr, dropout_keep_out_bytes=n)
        assert fa.validate_fwd(b) == fa.FA_ERR_INVALID_ARG
        assert lib.fa_fwd(ctypes.byref(b), None) == fa.FA_ERR_INVALID_ARG
        assert "dropout_keep_out" in lib.fa_bwd_last_error().decode()
    # ignored without dropout
    assert fa.validate_fwd(_fwd_args(dropout_keep_out=out + 2, dropout_keep_out_bytes=1)) == fa.FA_OK


def test_forward_valid_args_pass_validation():
    assert fa.validate_fwd(_fwd_args()) == fa.FA_OK
    assert fa.validate_fwd(_fwd_args(dtype=fa.FA_DTYPE_F16)) == fa.FA_OK
    assert fa.validate_fwd(_fwd_args(local_window=1, window_size_left=32,
                                     window_size_right=0)) == fa.FA_OK
    assert fa.validate_fwd(_fwd_args(causal=0, local_window=1, window_size_left=-1,
                                     window_size_right=9)) == fa.FA_OK
    assert fa.validate_fwd(_fwd_args(cu_seqlens_q=BASE, cu_seqlens_k=BASE + 256, total_q=1000,
                                     total_k=1200, batch=5, seqlen_q=300)) == fa.FA_OK


@pytest.mark.parametrize("over,status", [
    ({"num_heads_k": 3}, fa.FA_ERR_INVALID_ARG),
    ({"out": 0}, fa.FA_ERR_INVALID_ARG),
    ({"lse": 0}, fa.FA_ERR_INVALID_ARG),
    ({"k": 0}, fa.FA_ERR_INVALID_ARG),
    ({"v": BASE + 8}, fa.FA_ERR_INVALID_ARG),
    ({"lse": BASE + 2}, fa.FA_ERR_INVALID_ARG),
    ({"o_stride": (256 * 8 * 128, 8 * 128 + 4, 128)}, fa.FA_ERR_INVALID_ARG),
    ({"causal": 2}, fa.FA_ERR_INVALID_ARG),
    ({"local_window": 1, "window_size_right": 1}, fa.FA_ERR_INVALID_ARG),   # causal = 1
    ({"local_window": -1}, fa.FA_ERR_INVALID_ARG),
    ({"softcap": -0.5}, fa.FA_ERR_INVALID_ARG),
    ({"dropout_p": 1.5}, fa.FA_ERR_INVALID_ARG),
    ({"seqlen_q": (1 << 29) + 1}, fa.FA_ERR_UNSUPPORTED),
    ({"softmax_scale": float("inf")}, fa.FA_ERR_INVALID_ARG),
    ({"cu_seqlens_k": BASE}, fa.FA_ERR_INVALID_ARG),
    ({"dtype": 2}, fa.FA_ERR_UNSUPPORTED),
    ({"head_dim": 264}, fa.FA_ERR_UNSUPPORTED),
    ({"v_stride": (1 << 30, 1 << 24, 128)}, fa.FA_ERR_UNSUPPORTED),
])
def test_forward_validation_errors(over, status):
    lib = fa.load_library()
    a = _fwd_args(**over)
    assert fa.validate_fwd(a) == status
    assert lib.fa_bwd_last_error().decode() != ""
    assert lib.fa_fwd(ctypes.byref(a), None) == status     # rejected before any launch
    assert lib.fa_fwd(None, None) == fa.FA_ERR_INVALID_ARG


def test_missing_library_fails_loudly():
    """No CPU fallback: without the built library the binding raises (checked
    in a fresh interpreter, since a loaded library is cached)."""
    import subprocess
    import sys
    code = ("import attention_backward_fa2_amd as fa\n"
            "try:\n"
            "    fa.load_library('/nonexistent/libfa_bwd.so')\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0 and "raised: libfa_bwd.so is not built" in r.stdout, r.stdout + r.stderr
