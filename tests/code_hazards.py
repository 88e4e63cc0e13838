"""Scan the gfx950 code of the built library for the instruction hazards that
the compiler cannot cover because the instructions come from inline assembly.

The kernels issue some MFMAs (S and dP of the key-tile kernel, which keep
their results in ordinary registers next to accumulation-register operands)
and every LDS-DMA buffer load as asm statements; the compiler inserts wait
states for the instructions it generates, not for those.  The checks, on the
disassembly of every kernel (gfx950 rules, in wait states, an s_nop N
counting N + 1):

  mfma_result   an ordinary vector instruction reads or writes a register
                of a vector-destination MFMA result within 12 states after
                it (an MFMA that continues the accumulation is exempt);
  mfma_operand  an ordinary vector instruction writes an operand register
                of a vector-destination MFMA within 2 states before it;
  vmem_sgpr     a vector instruction (v_readlane, v_readfirstlane, a
                compare into scalar registers) writes a scalar register that
                an LDS-DMA buffer load reads as its descriptor within 5
                states after it.

Only this library's own build is disassembled (llvm-objdump of the code
objects in its .hip_fatbin section).
"""
import os
import re
import struct
import subprocess
import tempfile

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def code_objects(lib_path):
    """The gfx950 code objects embedded in the library, as bytes."""
    with tempfile.TemporaryDirectory() as td:
        fat = os.path.join(td, "fat.bin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                        ".hip_fatbin=" + fat, lib_path, os.path.join(td, "lib.copy")],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
    out = []
    pos = data.find(MAGIC)
    while pos >= 0:
        n = struct.unpack_from("<Q", data, pos + len(MAGIC))[0]
        q = pos + len(MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", data, q)
            triple = data[q + 24:q + 24 + tlen].decode()
            q += 24 + tlen
            if "gfx950" in triple and size:
                out.append(data[pos + off:pos + off + size])
        pos = data.find(MAGIC, pos + 1)
    return out


def disassemble(co_bytes):
    with tempfile.TemporaryDirectory() as td:
        p = os.path.join(td, "co.o")
        open(p, "wb").write(co_bytes)
        r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950",
                            "--no-show-raw-insn", "--no-leading-addr", p],
                           check=True, capture_output=True, text=True)
    return r.stdout


def kernels(disasm):
    """{kernel symbol: [instruction text, ...]}"""
    res, cur = {}, None
    for line in disasm.splitlines():
        m = re.match(r"^([0-9a-f]+ )?<(\S+)>:$", line.strip())
        if m:
            cur = m.group(2)
            res[cur] = []
            continue
        t = line.split(";")[0].split("//")[0].strip()
        if cur and t and not t.endswith(":"):
            res[cur].append(t)
    return res


def _regs(tok):
    m = re.match(r"-?([vas])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"-?([vas])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    if tok in ("vcc", "vcc_lo"):
        return {("s", "vcc")}
    return set()


def _ops(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    toks = [t.strip() for t in re.split(r",\s*(?![^\[]*\])", parts[1])]
    return parts[0], [t.split()[0] if t else t for t in toks]


def _states(line):
    op, a = _ops(line)
    if op == "s_nop":
        return int(a[0], 0) + 1
    return 1


def check_kernel(instrs, wrap=True):
    """Violations found in one kernel's instruction list (straight-line scan,
    with wrap: plus the first instructions again after the last, which
    approximates loop back edges).  An unconditional branch or the end of
    the program ends a straight line: the instruction after it is reached
    only by a jump, so nothing pending carries over (a conditional branch
    falls through and does carry)."""
    seq = instrs + instrs[:64] if wrap else list(instrs)
    found = []
    pend_res = []   # (index, result regs, states elapsed)
    pend_sw = []    # (index, scalar regs written by a vector instruction, states)
    for idx, line in enumerate(seq):
        op, a = _ops(line)
        w = _states(line)
        is_valu = op.startswith("v_") and not op.startswith("v_mfma")
        if is_valu and a:
            dst = _regs(a[0])
            src = set()
            for t in a[1:]:
                src |= _regs(t)
            for (j, res, el) in pend_res:
                if el < 12 and (dst | src) & res:
                    found.append(("mfma_result", el, line, seq[j]))
        if op.startswith("v_mfma") and a and a[0].startswith("v"):
            srcs = set()
            for t in a[1:]:
                srcs |= {r for r in _regs(t) if r[0] == "v"}
            back, k = 0, idx - 1
            while k >= 0 and back < 2:
                op2, a2 = _ops(seq[k])
                if op2.startswith("v_") and not op2.startswith("v_mfma") and a2 and \
                        _regs(a2[0]) & srcs:
                    found.append(("mfma_operand", back, seq[k], line))
                back += _states(seq[k])
                k -= 1
        if op.startswith("buffer_load") and "lds" in line:
            desc = set()
            for t in a:
                if t.startswith("s["):
                    desc |= _regs(t)
            for (j, sw, el) in pend_sw:
                if el < 5 and sw & desc:
                    found.append(("vmem_sgpr", el, seq[j], line))
        # age the pending lists by this instruction's states
        pend_res = [(j, r, el + w) for (j, r, el) in pend_res if el + w < 12]
        pend_sw = [(j, r, el + w) for (j, r, el) in pend_sw if el + w < 5]
        if op in ("s_branch", "s_endpgm", "s_setpc_b64"):
            pend_res, pend_sw = [], []
        if op.startswith("v_mfma") and a and a[0].startswith("v"):
            res = _regs(a[0])
            # an MFMA accumulating into these registers restarts the window
            pend_res = [(j, r, el) for (j, r, el) in pend_res if not (r & res)]
            pend_res.append((idx, res, 0))
        elif op.startswith("v_") and a and (op.startswith(("v_readlane", "v_readfirstlane"))
                                            or op.startswith("v_cmp")):
            sw = {r for r in _regs(a[0]) if r[0] == "s"}
            if sw:
                pend_sw.append((idx, sw, 0))
    # report each (kind, instruction pair) once
    uniq = []
    for f in found:
        if f not in uniq:
            uniq.append(f)
    return uniq


def scan(lib_path):
    """{kernel: [violations]} for every kernel of the library with any."""
    bad = {}
    for co in code_objects(lib_path):
        for name, instrs in kernels(disassemble(co)).items():
            if not instrs:
                continue
            v = check_kernel(instrs)
            if v:
                bad[name] = v
    return bad
