"""Wait states around the attention kernel's inline assembly.

The compiler inserts the wait states an MFMA needs after a VALU write of one
of its operands only for MFMAs it generates itself; the PV MFMAs of the
attention kernel are inline assembly (to keep O in the accumulation
registers), so nothing guards them but the kernel's own layout. This test
compiles the kernel to gfx950 assembly and checks, for every inline-assembly
MFMA, that no VALU instruction writes one of its operand registers (A, B or
the accumulator) fewer than MIN_WAIT wait states before it, and that nothing
but the next MFMA of the same accumulation touches its result registers fewer
than RESULT_WAIT wait states after it (each instruction issued in between is
one wait state, s_nop N is N + 1). The scan follows the instructions in the
order they are laid out, which is how straight-line code and the fall-through
of a branch issue; it does not cross an unconditional branch (what follows one
in the layout is reached only by jumps). The same scan checks the row loads
(inline-assembly buffer loads into LDS): no VALU instruction may write a scalar
register they read, M0 included, fewer than SGPR_WAIT wait states before them,
and a scalar write of M0 may not come right before them.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_kpool_amd", "csrc")
SRC = os.path.join(CSRC, "sparse_mla.hip")
# files whose kernels gather latent rows with inline-assembly loads into LDS
ROW_LOAD_SRCS = ["sparse_mla.hip", "sparse_mla_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
MIN_WAIT = 2       # VALU write of a VGPR/AGPR -> MFMA read of it (gfx950)
RESULT_WAIT = 18   # MFMA result -> read or write by another instruction (16-pass bound)
SGPR_WAIT = 5      # VALU write of an SGPR -> vector-memory read of it (gfx9)
M0_WAIT = 1        # write of M0 -> a load into LDS that takes its address from it

SREG = re.compile(r"\bs(?:\[(\d+):(\d+)\]|(\d+)\b)")
M0 = re.compile(r"\bm0\b")


def sregs(text):
    """Scalar registers named in an operand string: SGPR numbers, and "m0"."""
    out = set()
    for m in SREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    if M0.search(text):
        out.add("m0")
    return out

REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def regs(text):
    """The set of (kind, index) registers named in an operand string."""
    out = set()
    for m in REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, k) for k in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def valu_dest(line):
    """Registers a VALU instruction writes (its first operand), or an empty set."""
    parts = line.split(None, 1)
    op = parts[0]
    if not op.startswith("v_") or op.startswith("v_mfma") or op.startswith(("v_readfirstlane", "v_readlane", "v_cmp")):
        return set()
    if len(parts) < 2:
        return set()
    first = parts[1].split(",")[0]
    return regs(first)


def _assemble(src, extra):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = "/tmp/kp_hazard_check_" + os.path.basename(src) + ".s"
    subprocess.check_call([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *extra, "-x", "hip", src,
                           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-o", out],
                          stderr=subprocess.DEVNULL)
    return open(out).read().splitlines()


@pytest.fixture(scope="module")
def asm_lines():
    # the flags the library build uses for the attention forward
    return _assemble(SRC, ["-mllvm", "-amdgpu-mfma-vgpr-form"])


def instructions(asm_lines):
    """Instructions only (comments, labels, directives and asm markers
    dropped), each tagged with whether it sits inside an inline-assembly block."""
    instrs = []
    in_asm = False
    for raw in asm_lines:
        line = raw.strip()
        if line.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not line or line.startswith((";", ".")) or line.endswith(":"):
            continue
        instrs.append((line.split(";")[0].strip(), in_asm))
    return instrs


def unconditional(line):
    return line.startswith(("s_branch", "s_setpc", "s_endpgm"))


def wait_states(line):
    m = re.match(r"s_nop\s+(\d+)", line)
    return int(m.group(1)) + 1 if m else 1


def test_inline_mfma_operands_not_written_by_recent_valu(asm_lines):
    instrs = instructions(asm_lines)
    checked = 0
    bad = []
    for k, (line, in_asm) in enumerate(instrs):
        if not (in_asm and line.startswith("v_mfma")):
            continue
        checked += 1
        operands = regs(line.split(None, 1)[1])
        waits = 0
        j = k - 1
        while j >= 0 and waits < MIN_WAIT:
            prev = instrs[j][0]
            if unconditional(prev):
                break
            hit = valu_dest(prev) & operands
            if hit:
                bad.append(f"{prev!r} then {line!r} ({waits} wait states)")
                break
            waits += wait_states(prev)
            j -= 1
    assert checked > 0, "no inline-assembly MFMA found"
    assert not bad, "VALU write too close to an inline-assembly MFMA:\n" + "\n".join(bad[:10])


def test_inline_mfma_results_left_alone_until_done(asm_lines):
    instrs = instructions(asm_lines)
    checked = 0
    bad = []
    for k, (line, in_asm) in enumerate(instrs):
        if not (in_asm and line.startswith("v_mfma")):
            continue
        checked += 1
        ops = line.split(None, 1)[1].split(",")
        dest = regs(ops[0])
        waits = 0
        j = k + 1
        while j < len(instrs) and waits < RESULT_WAIT:
            nxt, nxt_asm = instrs[j]
            if unconditional(nxt):
                break
            parts = nxt.split(None, 1)
            touched = regs(parts[1]) if len(parts) > 1 else set()
            if touched & dest:
                chained = (nxt_asm and nxt.startswith("v_mfma")
                           and regs(parts[1].split(",")[0]) == dest
                           and regs(parts[1].split(",")[3]) == dest)
                if not chained:
                    bad.append(f"{line!r} then {nxt!r} ({waits} wait states)")
                break
            waits += wait_states(nxt)
            j += 1
    assert checked > 0, "no inline-assembly MFMA found"
    assert not bad, "inline-assembly MFMA result touched too soon:\n" + "\n".join(bad[:10])


@pytest.mark.parametrize("src", ROW_LOAD_SRCS)
def test_row_load_sgprs_settled(src):
    from sparse_attention_kpool_amd import build
    lines = _assemble(os.path.join(CSRC, src), build.EXTRA.get(src, []))
    instrs = instructions(lines)
    loads = 0
    bad = []
    for k, (line, in_asm) in enumerate(instrs):
        if not (in_asm and line.startswith("buffer_load") and line.endswith("lds")):
            continue
        loads += 1
        # the SGPRs the load names, and M0 (the LDS address it writes to)
        read = sregs(line.split(None, 1)[1]) | {"m0"}
        waits = 0
        j = k - 1
        while j >= 0 and waits < SGPR_WAIT:
            prev = instrs[j][0]
            if unconditional(prev):
                break
            parts = prev.split(None, 1)
            if parts[0].startswith("v_") and len(parts) > 1 and sregs(parts[1].split(",")[0]) & read:
                bad.append(f"{prev!r} then {line!r} ({waits} wait states)")
                break
            # M0 (the LDS address) written by a scalar move right before the load
            if waits < M0_WAIT and len(parts) > 1 and parts[1].split(",")[0].strip() == "m0":
                bad.append(f"{prev!r} then {line!r} ({waits} wait states)")
                break
            waits += wait_states(prev)
            j -= 1
    assert loads > 0, "no row load found"
    assert not bad, "VALU write of an SGPR too close to a row load:\n" + "\n".join(bad[:10])
