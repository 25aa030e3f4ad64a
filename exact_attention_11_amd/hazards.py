"""Build-time check of instruction hazards that the compiler cannot see.

Some kernels issue MFMAs and LDS copies (global_load_lds) as inline assembly.
The compiler's hazard recognizer does not know what these instructions are, so
this module checks the library's own gfx950 code object (disassembled with
llvm-objdump) along every control-flow path:

* result hazard: a non-MFMA vector, LDS or global instruction that reads or
  writes a VGPR an MFMA wrote must come at least RESULT_WAITS wait states after
  that MFMA (an MFMA that rewrites exactly the same registers as its
  accumulator, the in-place accumulation form, is exempt);
* operand hazard: an MFMA must come at least OPERAND_WAITS wait states after a
  vector ALU instruction that wrote any VGPR it reads;
* SGPR hazard (every kernel): a vector memory instruction that reads an SGPR
  (a scalar base address) must come at least SGPR_VMEM_WAITS wait states after
  a vector ALU instruction that wrote that SGPR (v_readfirstlane and the like).

Each instruction counts as one wait state and ``s_nop N`` as N + 1, which never
overstates the hardware's count.  RESULT_WAITS covers the longest (16-pass)
MFMA latency class, more than the 8-pass 32x32x16 products need.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile

RESULT_WAITS = 19
OPERAND_WAITS = 2
SGPR_VMEM_WAITS = 5
LLVM_BIN = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

_INSN = re.compile(r"^\s+(\S+)(.*?)\s*//\s*([0-9A-Fa-f]+):")
_TGT = re.compile(r"<([^>+]+)\+0x([0-9a-f]+)>")
_FUNC = re.compile(r"^([0-9a-f]+) <([^>]+)>:")
_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")
# Vector ALU instructions that write an SGPR: the first operand of these ...
_SGPR_DST_FIRST = ("v_readfirstlane", "v_readlane", "v_cmp_", "v_cmpx_")
# ... and the second (carry-out or flag) operand of these.
_SGPR_DST_SECOND = ("v_add_co_", "v_sub_co_", "v_subrev_co_", "v_addc_co_", "v_subb_co_", "v_subbrev_co_",
                    "v_div_scale_", "v_mad_u64_u32", "v_mad_i64_i32")
_VMEM = ("global_", "buffer_", "scratch_", "flat_")


def _regs(pattern, text: str) -> set:
    out = set()
    for m in pattern.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _vregs(text: str) -> set:
    return _regs(_VREG, text)


def _sgpr_writes(op: str, operands: str) -> set:
    args = [a.strip() for a in operands.split(",")]
    if op.startswith(_SGPR_DST_FIRST) and args:
        return _regs(_SREG, args[0])
    if op.startswith(_SGPR_DST_SECOND) and len(args) > 1:
        return _regs(_SREG, args[1])
    return set()


class Insn:
    __slots__ = ("addr", "op", "dst", "src", "text", "waits", "target", "sdst", "ssrc")

    def __init__(self, addr: int, op: str, operands: str, target):
        self.addr, self.op, self.text, self.target = addr, op, operands, target
        args = [a.strip() for a in operands.split(",")] if operands.strip() else []
        writes_first = op.startswith("v_") and not op.startswith("v_cmpx") and not op.startswith("v_cmp_")
        self.dst = _vregs(args[0]) if args and writes_first else set()
        self.src = set()
        for a in args[1:] if writes_first else args:
            self.src |= _vregs(a)
        self.waits = int(operands.split()[0], 0) + 1 if op == "s_nop" else 1
        # SGPRs a vector ALU instruction writes; SGPRs a vector memory instruction reads
        self.sdst = _sgpr_writes(op, operands) if op.startswith("v_") else set()
        self.ssrc = _regs(_SREG, operands) if op.startswith(_VMEM) else set()


def parse(dis: str) -> dict:
    """Function name -> list of instructions, from llvm-objdump -d output."""
    funcs, cur, base = {}, None, 0
    for line in dis.splitlines():
        m = _FUNC.match(line)
        if m:
            cur, base = m.group(2), int(m.group(1), 16)
            funcs[cur] = []
            continue
        m = _INSN.match(line)
        if not m or cur is None:
            continue
        target = None
        t = _TGT.search(line)
        if t and m.group(1).startswith(("s_cbranch", "s_branch")):
            target = base + int(t.group(2), 16)
        funcs[cur].append(Insn(int(m.group(3), 16), m.group(1), m.group(2), target))
    return funcs


def _successors(insns):
    index = {ins.addr: i for i, ins in enumerate(insns)}
    succ = []
    for i, ins in enumerate(insns):
        s = []
        if ins.op != "s_branch" and ins.op != "s_endpgm" and i + 1 < len(insns):
            s.append(i + 1)
        if ins.target is not None and ins.target in index:
            s.append(index[ins.target])
        succ.append(s)
    return succ


def _is_mfma(ins) -> bool:
    return ins.op.startswith("v_mfma")


def _accumulates_in_place(mfma, other) -> bool:
    if not _is_mfma(other) or other.op != mfma.op:
        return False
    args = [a.strip() for a in other.text.split(",")]
    return len(args) == 4 and _vregs(args[0]) == mfma.dst and _vregs(args[3]) == mfma.dst


def check_sgpr_function(insns) -> list:
    """SGPR hazards in one function: ("sgpr", writer address, memory instruction
    address, wait states between them)."""
    succ = _successors(insns)
    bad = []
    for i, ins in enumerate(insns):
        if not ins.sdst:
            continue
        seen = set()
        stack = [(j, 0) for j in succ[i]]
        while stack:
            j, w = stack.pop()
            if w >= SGPR_VMEM_WAITS or (j, w) in seen:
                continue
            seen.add((j, w))
            o = insns[j]
            if o.ssrc & ins.sdst:
                bad.append(("sgpr", ins.addr, o.addr, w))
                continue
            stack.extend((k, w + o.waits) for k in succ[j])
    return bad


def check_function(insns) -> list:
    """MFMA hazards in one function: (kind, mfma address, other address, wait states)."""
    succ = _successors(insns)
    pred = [[] for _ in insns]
    for i, s in enumerate(succ):
        for j in s:
            pred[j].append(i)
    bad = []
    for i, ins in enumerate(insns):
        if not _is_mfma(ins):
            continue
        # results: walk forward until RESULT_WAITS wait states have passed
        if ins.dst:
            seen = {}
            stack = [(j, 0) for j in succ[i]]
            while stack:
                j, w = stack.pop()
                if w >= RESULT_WAITS or seen.get(j, -1) >= RESULT_WAITS - w:
                    continue
                seen[j] = RESULT_WAITS - w
                o = insns[j]
                touched = (o.dst | o.src) & ins.dst
                if touched and o.op.startswith(("v_", "ds_", "global_", "buffer_", "flat_", "scratch_")):
                    if not _accumulates_in_place(ins, o):
                        bad.append(("result", ins.addr, o.addr, w))
                        continue
                if _is_mfma(o) and o.dst == ins.dst:
                    continue  # the accumulation chain continues; its own MFMA is checked separately
                stack.extend((k, w + o.waits) for k in succ[j])
        # operands: walk backward over OPERAND_WAITS wait states
        need = ins.src
        stack = [(j, 0) for j in pred[i]]
        seen = set()
        while stack:
            j, w = stack.pop()
            if w >= OPERAND_WAITS or (j, w) in seen:
                continue
            seen.add((j, w))
            o = insns[j]
            if o.op.startswith("v_") and not _is_mfma(o) and o.dst & need:
                bad.append(("operand", ins.addr, o.addr, w))
                continue
            stack.extend((k, w + o.waits) for k in pred[j])
    return bad


def disassemble(lib: str) -> str:
    """llvm-objdump -d of the gfx950 code object inside lib's offload bundle."""
    tools = {t: os.path.join(LLVM_BIN, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")}
    for t, p in tools.items():
        if not os.path.exists(p):
            found = shutil.which(t)
            if not found:
                raise RuntimeError(f"{t} not found")
            tools[t] = found
    with tempfile.TemporaryDirectory() as d:
        fat, co = os.path.join(d, "fatbin.bin"), os.path.join(d, "gfx950.co")
        subprocess.run([tools["llvm-objcopy"], f"--dump-section=.hip_fatbin={fat}", lib, os.path.join(d, "x")],
                       check=True, capture_output=True)
        subprocess.run([tools["clang-offload-bundler"], "--unbundle", "--type=o", f"--input={fat}",
                        f"--targets={TARGET}", f"--output={co}"], check=True, capture_output=True)
        res = subprocess.run([tools["llvm-objdump"], "-d", "--mcpu=gfx950", co], check=True, capture_output=True,
                             text=True)
        return res.stdout


def check_library(lib: str, pattern: str = "fa2_fwd_w64") -> list:
    """MFMA hazards in every kernel of lib whose name contains pattern (those
    that issue MFMAs as inline assembly) and SGPR hazards in every kernel."""
    funcs = parse(disassemble(lib))
    out = []
    names = [n for n in funcs if pattern in n]
    if not names:
        raise RuntimeError(f"no kernel matching {pattern!r} in {lib}")
    for n in names:
        out += [(n,) + b for b in check_function(funcs[n])]
    for n, insns in funcs.items():
        out += [(n,) + b for b in check_sgpr_function(insns)]
    return out
