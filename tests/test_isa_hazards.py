"""Static checks of the row-tile kernel's hand-written instructions.

The row-tile GEMV issues v_dot2c_f32_f16 with a DPP broadcast operand from
inline asm, so the compiler's hazard recognizer does not see them.  gfx950
needs (a) two wait states between a VALU write of a VGPR and a DPP read of
it, and (b) three wait states between a dot instruction's write of its
accumulator and any other instruction that reads or writes that register
(a chain of the same dot instruction accumulating into it is forwarded).
A missing (b) drops the last product of a block: exactly the failure this
test guards against.  Wait states are counted as the hardware does (an
s_nop n is n + 1 of them).  The kernel is compiled to gfx950 assembly here (no GPU
needed) and every such instruction is checked in straight-line code."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "bit_quantized_decode_pn3t_amd", "csrc", "pn_gemv_rows.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _split(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [t.strip() for t in re.split(r",\s*", parts[1])]


def _wait_states(line):
    if line.startswith("s_nop"):
        return int(line.split()[1], 0) + 1
    return 1


def find_hazards(asm):
    """Return descriptions of DPP-read and dot-write hazards in `asm`, and of
    any use of a hand-issued atomic's result register before a vmcnt wait
    (the compiler does not know the register is still being written)."""
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    ins = [l for l in lines if l and not l.startswith((".", "//")) and not l.endswith(":")]
    found = []
    for i, line in enumerate(ins):
        op, args = _split(line)
        if op.startswith("v_dot2c") and args:
            dst = _regs(args[0])
            ws = 0
            for nxt in ins[i + 1:i + 8]:
                op2, a2 = _split(nxt)
                if op2.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")) or ws >= 3:
                    break
                touched = set()
                for t in a2:
                    touched |= _regs(t.split()[0]) if t else set()
                if dst & touched:
                    srcs = _regs(a2[1]) | _regs(a2[2].split()[0]) if len(a2) > 2 else set()
                    if op2.startswith("v_dot2c") and _regs(a2[0]) == dst and not (dst & srcs):
                        break  # the next link of an accumulation chain
                    found.append("dot write -> use after %d wait states: %s -> %s" % (ws, line, nxt))
                    break
                ws += _wait_states(nxt)
        if op.startswith("global_atomic") and args and " sc0" in line:
            dst = _regs(args[0])
            for nxt in ins[i + 1:]:
                op2, a2 = _split(nxt)
                if op2.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")) or \
                        (op2 == "s_waitcnt" and "vmcnt" in nxt):
                    break
                touched = set()
                for j, t in enumerate(a2):
                    rs = _regs(t.split()[0]) if t else set()
                    # the compiler does 32-bit multiply-adds with
                    # v_mad_u64_u32 and leaves the addend's high half
                    # undefined: a read of it there is not a use
                    if j == 4 and op2.startswith("v_mad_u64_u32") and len(rs) == 2 and dst & rs == {max(rs)}:
                        continue
                    touched |= rs
                if dst & touched:
                    found.append("atomic result used before a wait: %s -> %s" % (line, nxt))
                    break
        if "_dpp" in op and len(args) > 1:
            src0 = _regs(args[1])
            ws = 0
            for back in range(1, 4):
                if i - back < 0 or ws >= 2:
                    break
                prev = ins[i - back]
                pop, pa = _split(prev)
                if pop.startswith("v_") and pa and not pop.startswith(("v_readfirstlane", "v_readlane", "v_cmp")) \
                        and (_regs(pa[0]) & src0):
                    found.append("VALU write -> DPP read after %d wait states: %s -> %s" % (ws, prev, line))
                    break
                ws += _wait_states(prev)
    return found


def test_checker_flags_a_planted_hazard():
    planted = """
    v_dot2c_f32_f16_dpp v10, v1, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
    v_fma_mix_f32 v20, v4, v10, v20
    v_mov_b32_e32 v7, 0
    v_dot2c_f32_f16_dpp v11, v7, v2 row_newbcast:1 row_mask:0xf bank_mask:0xf
    v_dot2c_f32_f16_dpp v12, v1, v2 row_newbcast:2 row_mask:0xf bank_mask:0xf
    v_dot2c_f32_f16_dpp v12, v1, v3 row_newbcast:4 row_mask:0xf bank_mask:0xf
    s_nop 2
    v_fma_mix_f32 v20, v4, v12, v20
    global_atomic_add v30, v[2:3], v31, off sc0
    v_mov_b32_e32 v32, v30
    s_waitcnt vmcnt(0)
    v_add_f32_e32 v40, v41, v42
    s_nop 1
    v_add_f32_dpp v43, v40, v43 row_shr:1 row_mask:0xf bank_mask:0xf
    v_add_f32_e32 v44, v41, v42
    s_nop 0
    v_add_f32_dpp v45, v44, v45 row_shr:1 row_mask:0xf bank_mask:0xf
    """
    got = find_hazards(planted)
    assert len(got) == 4, got
    assert "v_fma_mix_f32 v20, v4, v10" in got[0]
    assert "v_mov_b32_e32 v7" in got[1]
    assert "v_mov_b32_e32 v32, v30" in got[2]
    assert "v_add_f32_e32 v44" in got[3]  # s_nop 0 is one wait state; s_nop 1 before v43's read is enough


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_row_tile_kernel_has_no_hazards(tmp_path):
    out = tmp_path / "rows.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), "-o", str(out), SRC]
    subprocess.run(cmd, check=True, capture_output=True, cwd=os.path.dirname(SRC))
    asm = out.read_text()
    assert asm.count("v_dot2c_f32_f16_dpp") >= 1152  # both kernels, both types
    assert find_hazards(asm) == []


KERNEL_SOURCES = ["pn_gemv_rows.hip", "pn_kernels.hip", "pn_smallm.hip", "pn_prefill.hip", "pn_rotate.hip",
                  "pn_probe.hip"]


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_cache_maintenance(tmp_path, src):
    """No kernel writes back or invalidates L2 (buffer_wbl2 / buffer_inv).
    The compiler emits them for acquire or release atomics at agent scope.
    The row-tile kernel once counted its finished waves that way, and every
    finishing wave flushed its XCD's L2 under the waves still streaming.
    Every atomic here is relaxed: its ordering comes from explicit waits and
    the kernel boundary."""
    path = os.path.join(os.path.dirname(SRC), src)
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), "-o", str(out), path]
    subprocess.run(cmd, check=True, capture_output=True, cwd=os.path.dirname(SRC))
    asm = out.read_text()
    assert "s_endpgm" in asm
    bad = [l.strip() for l in asm.splitlines() if re.match(r"\s*buffer_(wbl2|inv)\b", l)]
    assert bad == [], bad
