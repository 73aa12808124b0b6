"""Assumptions the GEMM kernels make about the code the compiler produces,
checked on the gfx950 assembly (host only).

1. Hazard bookkeeping of the inline-assembly MFMAs in gemm.hip's promotion
pipeline.

Those MFMAs are written as inline assembly, so the compiler does not insert
the wait states an MFMA result needs before a vector-ALU read (12 for this
instruction, what the compiler emits for its own MFMAs) nor those a vector-ALU
write of an operand needs before the MFMA reads it.  The kernel relies on
its instruction order instead; this test compiles the file and checks, for
every such MFMA in every instantiation, that
  * its destination registers are first read at least 12 wait states later
    (each instruction counts one, s_nop N counts N + 1), and
  * no vector-ALU instruction writes its A or B operand within the 3 wait
    states before it.

2. gemm_mx.hip's kernels count their direct global->LDS loads with partial
vmcnt waits, which holds because loads complete in order.  A register spill
would put scratch stores among them, and stores may complete out of order
with loads, so those kernels must use no scratch memory."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_fp8_linear_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(tok):
    m = re.match(r"[va]\[(\d+):(\d+)\]", tok)
    if m:
        return {(tok[0], r) for r in range(int(m.group(1)), int(m.group(2)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _instr(line):
    t = line.split(";")[0].strip()
    if not t or t.endswith(":") or t.startswith("."):
        return None, []
    op = t.split()[0]
    return op, [x.strip().split()[0] for x in t[len(op):].split(",") if x.strip()]


def _states(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    out = str(tmp_path_factory.mktemp("asm") / "gemm.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Wno-inline-asm", "-Wno-unused-function",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", "-o", out, os.path.join(CSRC, "gemm.hip")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    lines = open(out).read().splitlines()
    # the inline MFMAs sit between ;;#ASMSTART and ;;#ASMEND
    inline, inside = [], False
    for i, l in enumerate(lines):
        if ";;#ASMSTART" in l:
            inside = True
        elif ";;#ASMEND" in l:
            inside = False
        elif inside and l.strip().startswith("v_mfma"):
            inline.append(i)
    return lines, inline


def test_inline_mfmas_exist(asm):
    lines, inline = asm
    assert len(inline) >= 3 * 32, "the promotion pipeline's MFMAs were not found in the assembly"


def test_results_read_only_after_12_wait_states(asm):
    lines, inline = asm
    worst = None
    for i in inline:
        op, ops = _instr(lines[i])
        dst = _regs(ops[0])
        ws = 0
        for j in range(i + 1, min(i + 500, len(lines))):
            op2, ops2 = _instr(lines[j])
            if op2 is None:
                continue
            if op2.startswith(("s_cbranch", "s_branch", "s_endpgm", "s_setpc")):
                break
            srcs = set()
            stores = op2.startswith(("global_store", "ds_write", "buffer_store", "scratch_store", "flat_store"))
            for k, x in enumerate(ops2):
                if k == 0 and not stores:
                    continue
                srcs |= _regs(x)
            if srcs & dst:
                assert ws >= 12, f"line {i + 1}: MFMA result read after {ws} wait states at line {j + 1}: {lines[j]}"
                worst = ws if worst is None else min(worst, ws)
                break
            if ops2 and not stores and _regs(ops2[0]) & dst:
                break  # overwritten before any read
            ws += _states(op2, ops2)
    assert worst is not None


def test_operands_not_written_by_valu_just_before(asm):
    lines, inline = asm
    for i in inline:
        op, ops = _instr(lines[i])
        srcs = _regs(ops[1]) | _regs(ops[2])
        seen = 0
        for j in range(i - 1, max(0, i - 80), -1):
            op2, ops2 = _instr(lines[j])
            if op2 is None:
                continue
            if op2.startswith("v_") and not op2.startswith("v_mfma") and ops2:
                assert not (_regs(ops2[0]) & srcs), \
                    f"line {i + 1}: operand written by a VALU instruction {seen} wait states before: {lines[j]}"
            seen += _states(op2, ops2)
            if seen >= 3:
                break


def test_gemm_mx_kernels_use_no_scratch(tmp_path):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    out = str(tmp_path / "gemm_mx.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Wno-inline-asm", "-Wno-unused-function",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", "-o", out, os.path.join(CSRC, "gemm_mx.hip")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = open(out).read()
    kernels = re.findall(r"\.name:\s+(\S+)\n(?:.*\n)*?\s+\.private_segment_fixed_size:\s+(\d+)", text)
    assert any("gemm_mx" in k for k, _ in kernels)
    assert len(kernels) == text.count(".private_segment_fixed_size:")
    for name, priv in kernels:
        assert int(priv) == 0, f"{name} uses {priv} bytes of scratch"
    assert "scratch_store" not in text and "buffer_store_dword" not in text.replace("buffer_store_dwordx", "")
