"""The built library's gfx950 code has no uncovered inline-assembly hazard
(tests/code_hazards.py: vector-destination MFMA results and operands, and
LDS-DMA descriptors written by vector instructions).  CPU only: it
disassembles this library's own code objects."""
import os

import pytest

from tests import code_hazards as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "attention_backward_fa2_amd", "libfa_bwd.so")


def test_scanner_flags_each_hazard_kind():
    """Hand-written sequences with one hazard each (and their fixed forms)."""
    mfma = "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]"

    def check(seq):
        return H.check_kernel(seq, wrap=False)
    # a vector copy into the accumulator right before the MFMA
    assert [f[0] for f in check(["v_mov_b32_e32 v0, v40", mfma])] == ["mfma_operand"]
    assert check(["v_mov_b32_e32 v0, v40", "s_nop 1", mfma]) == []
    # reading the result too early, and after 12 states
    assert [f[0] for f in check([mfma, "s_nop 2", "v_add_f32_e32 v20, v3, v3"])] == \
        ["mfma_result"]
    assert check([mfma, "s_nop 11", "v_add_f32_e32 v20, v3, v3"]) == []
    # an accumulation chain is not a hazard
    assert check([mfma, mfma]) == []
    # a conditional branch falls through; after an unconditional one the
    # next instruction is reached by a jump only
    assert [f[0] for f in check([mfma, "s_cbranch_scc1 5", "v_add_f32_e32 v20, v3, v3"])] == \
        ["mfma_result"]
    assert check([mfma, "s_branch 5", "v_add_f32_e32 v20, v3, v3"]) == []
    # a descriptor restored by v_readlane right before an LDS-DMA load
    load = "buffer_load_dwordx4 v1, s[12:15], 0 offen lds"
    assert [f[0] for f in check(["v_readlane_b32 s13, v200, 3", load])] == ["vmem_sgpr"]
    assert check(["v_readlane_b32 s13, v200, 3", "s_nop 4", load]) == []


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_built_library_has_no_uncovered_hazards():
    if not os.path.exists(os.path.join(H.LLVM, "llvm-objdump")):
        pytest.skip("llvm-objdump not available")
    bad = H.scan(LIB)
    assert not bad, {k[:80]: v[:3] for k, v in bad.items()}
