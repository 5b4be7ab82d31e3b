"""Static check of the generated gfx950 code around hand-written MFMAs.

Some MFMAs in fa_kernels.hip are inline assembly, so that their accumulator
can live in VGPRs.  The compiler's hazard recognizer does not look inside
inline assembly: it inserts no wait states between such an MFMA and the
instructions around it.  The kernels provide those waits themselves (an
``s_nop`` drain that takes the accumulators as operands), but the register
allocator may still copy or spill an accumulator between the MFMA and the
drain, or write an MFMA operand right before it.  Either reads or writes a
register the matrix unit is still working on and gives wrong results
intermittently, with no fault.

``scan`` looks at the device assembly (``hipcc --cuda-device-only -S``) and
reports, for every inline-assembly MFMA:

* any compiler-emitted instruction that reads or writes the MFMA's
  destination registers, or a branch or label, before its result wait has
  passed: an XDL MFMA of N passes needs N + 4 wait states on gfx950 before a
  VALU or memory instruction may read or overwrite its result (the rule
  LLVM's hazard recognizer applies to the MFMAs it emits itself); the scan
  asks N + 5, one more, for the inline-asm forms here, 8-pass
  v_mfma_f32_32x32x16_bf16 (13), 4-pass v_mfma_f32_16x16x32_bf16 (9) and
  16-pass v_mfma_f32_32x32x64_f8f6f4 on FP8 operands (21), and
  ``result_wait`` (18) for any other;
* any compiler-emitted VALU instruction that writes one of the MFMA's source
  registers fewer than ``operand_wait`` wait states before it (2 are needed).

``scan_divergent_copies`` reports register copies placed right before the
end of a divergent region (see there).

Wait states are counted conservatively: one per instruction, ``N + 1`` for
``s_nop N``.  Other inline-assembly instructions count but are not reported
(the MFMA chains and the drain are written to respect the rules).

An inline-asm MFMA whose text carries the comment ``accumulate-only`` (the
ping-pong prefill's P V and row-sum MFMAs) promises that its accumulator is
read only by later MFMAs of the same chain (which the hardware orders) or
after an explicit drain.  For it a branch within the window is no finding:
the scan instead runs on through the branch in program order, so that an
access on the fall-through path is still reported.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

_RANGE = re.compile(r"^([va])\[(\d+):(\d+)\]$")
_SINGLE = re.compile(r"^([va])(\d+)$")


def _regs(tok: str) -> set:
    m = _RANGE.match(tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _SINGLE.match(tok)
    return {tok} if m else set()


def _operands(text: str) -> list:
    op = text.split()[0]
    out = []
    for part in text[len(op):].split(","):
        part = part.strip().split()
        out.append(_regs(part[0]) if part else set())
    return out


ACCUMULATE_ONLY = "accumulate-only"


def _instructions(asm: str, with_marks: bool = False):
    """(line number, text, inside inline asm, is control flow) per instruction;
    with_marks adds whether the line carried the accumulate-only marker."""
    out = []
    in_asm = False
    for no, line in enumerate(asm.splitlines(), 1):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        mark = ACCUMULATE_ONLY in t
        if re.match(r"^[\w.$]+:", t):
            out.append((no, t, in_asm, True, mark) if with_marks else (no, t, in_asm, True))
            continue
        t = t.split(";")[0].strip()
        if not t:
            continue
        op = t.split()[0]
        cf = op.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm"))
        out.append((no, t, in_asm, cf, mark) if with_marks else (no, t, in_asm, cf))
    return out


def _wait_states(text: str) -> int:
    parts = text.split()
    if parts[0] == "s_nop":
        return int(parts[1], 0) + 1
    return 1


# inline-asm MFMA opcode -> wait states before its result may be accessed
RESULT_WAIT = {"v_mfma_f32_32x32x16_bf16": 8 + 5, "v_mfma_f32_16x16x32_bf16": 4 + 5,
               "v_mfma_f32_32x32x64_f8f6f4": 16 + 5}


def scan(asm: str, result_wait: int = 18, operand_wait: int = 2) -> list:
    """Findings (one string each) for every inline-asm MFMA in ``asm``."""
    marked = _instructions(asm, with_marks=True)
    ins = [m[:4] for m in marked]
    findings = []
    for k, (no, text, in_asm, _) in enumerate(ins):
        if not (in_asm and text.startswith("v_mfma")):
            continue
        acc_only = marked[k][4]
        ops = _operands(text)
        dst, srcs = ops[0], set().union(*ops[1:]) if len(ops) > 1 else set()
        need = RESULT_WAIT.get(text.split()[0], result_wait)
        # after: nothing emitted by the compiler touches dst until the wait is over
        ws, j = 0, k + 1
        while j < len(ins) and ws < need:
            no2, t2, a2, cf = ins[j]
            if cf and acc_only:
                j += 1          # follow the fall-through path
                continue
            if cf:
                findings.append(f"line {no}: {text}: control flow {ws} wait states later "
                                f"(line {no2}: {t2})")
                break
            if not a2:
                hit = set().union(*_operands(t2)) & dst
                if hit:
                    findings.append(f"line {no}: {text}: its result is accessed {ws} wait "
                                    f"states later (line {no2}: {t2})")
                    break
            ws += _wait_states(t2)
            j += 1
        # before: no VALU write to an operand within operand_wait wait states
        ws, j = 0, k - 1
        while j >= 0 and ws < operand_wait:
            no2, t2, a2, cf = ins[j]
            if cf:
                break
            if not a2 and t2.startswith("v_"):
                hit = _operands(t2)[0] & srcs
                if hit:
                    findings.append(f"line {no}: {text}: operand written {ws} wait states "
                                    f"earlier (line {no2}: {t2})")
                    break
            ws += _wait_states(t2)
            j -= 1
    return findings


def scan_inline_dot(asm: str, result_wait: int = 3) -> list:
    """Findings for every inline-asm dot-product instruction (``v_dot*``).

    On CDNA3/CDNA4 a VALU dot instruction's result is not interlocked: a
    different VALU instruction (or a same-opcode dot reading it as an A/B
    operand) must wait 3 wait states before reading the VGPR a dot wrote;
    only the same dot opcode taking it as its accumulator may follow at
    once.  The compiler inserts those wait states for dots it emits itself,
    but not for one written as inline assembly, which it cannot see into.
    The kernels write no dot instruction today (this LLVM cannot select the
    gfx950 v_dot2c_f32_bf16 intrinsic, so one could only come as inline asm);
    this keeps one from coming back without its wait states.  A branch within
    the window is reported too.
    """
    ins = _instructions(asm)
    findings = []
    for k, (no, text, in_asm, _) in enumerate(ins):
        if not (in_asm and text.startswith("v_dot")):
            continue
        op = text.split()[0]
        dst = _operands(text)[0]
        ws, j = 0, k + 1
        while j < len(ins) and ws < result_wait:
            no2, t2, _, cf = ins[j]
            if cf:
                findings.append(f"line {no}: {text}: control flow {ws} wait states later "
                                f"(line {no2}: {t2})")
                break
            ops2 = _operands(t2)
            reads = set().union(*ops2[1:]) if len(ops2) > 1 else set()
            chained = t2.split()[0] == op and ops2[0] == dst and not (reads & dst)
            if not chained and (reads | (ops2[0] if ops2 else set())) & dst:
                findings.append(f"line {no}: {text}: its result is accessed {ws} wait "
                                f"states later (line {no2}: {t2})")
                break
            ws += _wait_states(t2)
            j += 1
    return findings


_COPIES = ("v_mov_b32", "v_mov_b64", "v_accvgpr_write_b32", "v_accvgpr_read_b32",
           "v_accvgpr_mov_b32")


def scan_divergent_copies(asm: str) -> list:
    """Register copies placed at the very end of a divergent region.

    A region opened by ``s_and_saveexec_b64 sX`` runs with some lanes off
    until ``s_or_b64 exec, exec, sX`` restores them.  A VGPR/AGPR copy right
    before that restore only reaches the active lanes; when the register
    allocator splits the live range of a value that every lane still needs
    (a loop-carried sum, say) and puts the copy there, the other lanes lose
    it.  This once produced wrong row sums in the lanes a causal-mask branch
    had skipped.  The kernels keep their masks as selects so that no such
    branch exists inside the key loop; any copy in this position is reported.
    """
    ins = _instructions(asm)
    findings = []
    for k, (no, text, _, _) in enumerate(ins):
        if not text.startswith("s_or_b64 exec, exec,"):
            continue
        j = k - 1
        while j >= 0:
            no2, t2, _, cf = ins[j]
            op = t2.split()[0]
            if cf and not op.startswith("s_"):
                j -= 1          # a label: keep looking back
                continue
            if cf or op.startswith("s_and_saveexec"):
                break           # a branch (no fall-through) or the region's start
            if op.startswith("s_"):
                j -= 1
                continue
            if re.sub(r"_e(32|64)$", "", op) in _COPIES:
                findings.append(f"line {no2}: {t2}: copy at the end of a divergent region "
                                f"(exec restored at line {no})")
                j -= 1
                continue
            break
    return findings


def device_asm(hipcc: str, flags: list, include: str, source: str) -> str:
    """The gfx950 assembly hipcc generates for ``source``."""
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "device.s")
        keep = [f for f in flags if f not in ("-shared", "-fPIC")]
        cmd = [hipcc, *keep, "--cuda-device-only", "-S", "-I", include, "-o", out, source]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc -S failed ({res.returncode}):\n{res.stderr[-4000:]}")
        with open(out) as f:
            return f.read()
