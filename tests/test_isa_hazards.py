"""Static checks of the kernels' instruction streams on gfx950.

The row-tile GEMV issues v_dot2c_f32_f16 with a DPP broadcast operand from
inline asm, so the compiler's hazard recognizer does not see them.  gfx950
needs (a) two wait states between a VALU write of a VGPR and a DPP read of
it, and (b) three wait states between a dot instruction's write of its
accumulator and any other instruction that reads or writes that register
(a chain of the same dot instruction accumulating into it is forwarded).
A missing (b) drops the last product of a block: exactly the failure this
test guards against.  Wait states are counted as the hardware does (an
s_nop n is n + 1 of them).  The kernel is compiled to gfx950 assembly here (no GPU
needed) and every such instruction is checked in straight-line code.

MFMA accumulation chains: an MFMA that reads as its accumulator (SrcC) the
result of an MFMA of another shape (v_mfma_f32_16x16x32_f16 after
v_mfma_f32_16x16x16_f16, or the reverse) needs at least 5 wait states
between them on MI355X, while a chain of one shape is forwarded with none.
Measured: with the pair otherwise adjacent, 0 to 4 wait states gave wrong
values in about half of the 256 outputs of a 16 x 16 tile, 5 or more gave
the exact sums.  The compiler inserts none when the accumulator registers
match exactly, as for a chain of one shape; a dropped pn3t variant of
gemm_stream that ended a chain of two K = 32 steps with one K = 16 step got
wrong sums that way.  The shipped MFMA kernels start every block's chain
from a zero accumulator and keep one shape per chain; the check below walks
the control-flow graph of each compiled kernel backwards from every
accumulating MFMA and fails on a different-shape MFMA result reached within
5 wait states.

LDS reads issued from inline asm: the small-M DMA kernel reads each block's
activation operands from LDS one block ahead of their use, with inline
ds_read instructions the compiler does not know to be loads, each retired by
an s_waitcnt lgkmcnt tied to the registers it fills.  The compiler may
still copy or overwrite those registers before the wait if the asm output
is not the very register the consumer takes (a first form assembled a
128-bit operand from two 64-bit reads that way, and its pn3t products came
out as NaN).  The check tracks, over the control-flow graph, the LDS reads
possibly still outstanding (LDS operations complete in order, so an
lgkmcnt(N) retires every read with at least N younger LDS reads) and fails
on any instruction that touches their registers first."""
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


MFMA_SHAPE_WAIT = 5  # wait states a different-shape MFMA result needs before it is read as SrcC
BRANCHES = ("s_branch", "s_cbranch", "s_setpc", "s_endpgm")


def _regs2(tok):
    """Registers of an operand as (file, index) pairs: VGPRs and AGPRs."""
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _blocks(asm):
    """Basic blocks of every function in `asm`: lists of instructions, a
    label (or None) per block and the successor block indices."""
    blocks, labels = [[]], [None]
    for raw in asm.splitlines():
        line = raw.split(";")[0].strip()
        if not line or line.startswith((".", "//")) and not line.endswith(":"):
            continue
        if line.endswith(":"):
            blocks.append([])
            labels.append(line[:-1])
            continue
        blocks[-1].append(line)
        if line.startswith(BRANCHES):
            blocks.append([])
            labels.append(None)
    index = {l: i for i, l in enumerate(labels) if l}
    succ = []
    for i, b in enumerate(blocks):
        last = b[-1] if b else ""
        op, args = _split(last) if last else ("", [])
        out = []
        if op.startswith(("s_branch", "s_cbranch")) and args and args[0] in index:
            out.append(index[args[0]])
        if not op.startswith(("s_branch", "s_setpc", "s_endpgm")) and i + 1 < len(blocks):
            out.append(i + 1)
        succ.append(out)
    return blocks, labels, succ


def find_mfma_shape_hazards(asm, need=MFMA_SHAPE_WAIT):
    """Accumulating MFMAs that can read the result of an MFMA of another
    opcode fewer than `need` wait states after it, on some path."""
    blocks, labels, succ = _blocks(asm)
    pred = [[] for _ in blocks]
    for i, out in enumerate(succ):
        for j in out:
            pred[j].append(i)
    found = []
    for bi, b in enumerate(blocks):
        for ii, line in enumerate(b):
            op, args = _split(line)
            if not op.startswith("v_mfma") or len(args) < 4:
                continue
            srcc = _regs2(args[3].split()[0])
            if not srcc:
                continue  # a constant accumulator: a chain starts here
            # walk back over every path until `need` wait states have passed
            todo = [(bi, ii - 1, 0)]
            seen = set()
            while todo:
                cb, ci, ws = todo.pop()
                if (cb, ci, ws) in seen:
                    continue
                seen.add((cb, ci, ws))
                while ci >= 0 and ws < need:
                    prev = blocks[cb][ci]
                    pop, pa = _split(prev)
                    dst = _regs2(pa[0].split()[0]) if pa else set()
                    if dst & srcc:
                        if pop.startswith("v_mfma") and pop != op:
                            found.append("%s -> %s after %d wait states" % (prev, line, ws))
                        break  # the accumulator's producer on this path
                    ws += _wait_states(prev)
                    ci -= 1
                else:
                    if ws < need:
                        for p in pred[cb]:
                            todo.append((p, len(blocks[p]) - 1, ws))
    return found


def test_mfma_shape_checker_flags_a_planted_hazard():
    planted = """
_kernel:
    v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0
    v_mfma_f32_16x16x32_f16 v[0:3], v[12:15], v[16:19], v[0:3]
    v_mfma_f32_16x16x16_f16 v[0:3], v[20:21], v[22:23], v[0:3]
    s_nop 4
    v_mfma_f32_16x16x32_f16 v[24:27], v[4:7], v[8:11], v[0:3]
.LBB0_1:
    v_mfma_f32_16x16x16_f16 a[0:3], v[20:21], v[22:23], a[0:3]
    s_nop 7
    s_nop 7
    v_add_f32_e32 v30, v31, v32
    v_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]
    s_cbranch_scc1 .LBB0_1
    v_mfma_f32_16x16x32_f16 v[40:43], v[4:7], v[8:11], 0
    v_mov_b32_e32 v40, 0
    v_mfma_f32_16x16x16_f16 v[40:43], v[20:21], v[22:23], v[40:43]
    s_endpgm
"""
    got = find_mfma_shape_hazards(planted)
    # K=32 -> K=16 adjacent; the loop's K=32 -> its head's K=16 across the
    # back edge (one wait state: the branch); not the K=16 -> K=32 after 5
    # wait states, not the same-shape link, not after the v_mov rewrote v40
    assert len(got) == 2, got
    assert "v[0:3], v[12:15]" in got[0] and "v[20:21]" in got[0] and "after 0 wait states" in got[0]
    assert "a[0:3], v[4:7]" in got[1] and "a[0:3], v[20:21]" in got[1] and "after 1 wait states" in got[1]


SNIPPET = r"""
#include <hip/hip_runtime.h>
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
template <int NOPS>
__global__ void chain(const h8 *a8, const h4 *a4, f4 *out)
{
    const int l = threadIdx.x;
    const h8 x0 = a8[l], x1 = a8[l + 64];
    const h4 x2 = a4[l];
    __builtin_amdgcn_sched_barrier(0);
    f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(x0, x1, (f4){0, 0, 0, 0}, 0, 0, 0);
    if (NOPS) asm volatile("s_nop 4" : "+v"(d));
    d = __builtin_amdgcn_mfma_f32_16x16x16f16(x2, x2, d, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    out[l] = d;
}
template __global__ void chain<0>(const h8 *, const h4 *, f4 *);
template __global__ void chain<1>(const h8 *, const h4 *, f4 *);
"""


def _compile(tmp_path, src_path, name):
    out = tmp_path / (name + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), "-o", str(out), str(src_path)]
    subprocess.run(cmd, check=True, capture_output=True, cwd=os.path.dirname(SRC))
    return out.read_text()


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_compiler_leaves_mixed_chain_unguarded(tmp_path):
    """The case the check exists for: compiled with nothing in between, the
    K = 16 step follows the K = 32 step that writes its accumulator within a
    wait state or so (the compiler adds none for the accumulator); with an
    s_nop 4 between (the compiler adds one more after the asm) the pair is
    6 wait states apart and passes."""
    src = tmp_path / "chain.hip"
    src.write_text(SNIPPET)
    asm = _compile(tmp_path, src, "chain")
    got = find_mfma_shape_hazards(asm)
    assert len(got) == 1, got
    assert int(re.search(r"after (\d+) wait states", got[0]).group(1)) < MFMA_SHAPE_WAIT, got


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
@pytest.mark.parametrize("src,min_mfma", [("pn_smallm.hip", 16), ("pn_prefill.hip", 4)])
def test_mfma_kernels_keep_one_shape_per_chain(tmp_path, src, min_mfma):
    asm = _compile(tmp_path, os.path.join(os.path.dirname(SRC), src), src)
    assert len(re.findall(r"^\s*v_mfma", asm, re.M)) >= min_mfma
    assert find_mfma_shape_hazards(asm) == []


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


LDS_RETURNS = ("ds_read", "ds_bpermute", "ds_permute", "ds_swizzle")


def _lds_returns(op, line=""):
    return op.startswith(LDS_RETURNS) or (op.startswith("ds_") and "_rtn" in op)


def find_lds_use_before_wait(asm, cap=64):
    """Instructions that read or write a register an LDS read may still be
    filling, on some path (forward dataflow over the control-flow graph; the
    state maps each read to the fewest younger LDS reads issued after it on
    any path reaching the point)."""
    return _use_before_wait(asm, _lds_returns, _lds_returns, "lgkmcnt", cap)


def _vmem_returns(op, line):
    """Vector memory instructions that write a VGPR result: loads into
    registers and atomics that return (sc0), not stores or LDS DMA."""
    if op.startswith(("global_load", "buffer_load", "flat_load", "scratch_load")):
        return not line.rstrip().endswith(" lds") and " lds" not in line.split(";")[0].split(",")[-1]
    if op.startswith(("global_atomic", "buffer_atomic", "flat_atomic")):
        return " sc0" in line or " glc" in line
    return False


def _vmem_counts(op, line):
    return op.startswith(("global_", "buffer_", "flat_", "scratch_"))


def find_vmem_use_before_wait(asm, cap=64):
    """The same for vector memory results (a hand-issued atomic's result must
    not be touched before a vmcnt wait retires it); every vector memory
    instruction counts as younger, as the compiler counts them."""
    return _use_before_wait(asm, _vmem_returns, _vmem_counts, "vmcnt", cap)


def _use_before_wait(asm, returns, counts, counter, cap):
    blocks, labels, succ = _blocks(asm)
    entry = [None] * len(blocks)
    entry[0] = {}
    work = [0]
    found = set()
    # every function's first block is an entry too
    for bi, lab in enumerate(labels):
        if lab and not lab.startswith(".") and entry[bi] is None:
            entry[bi] = {}
            work.append(bi)

    def step(state, bi, record):
        st = dict(state)
        for ii, line in enumerate(blocks[bi]):
            op, args = _split(line)
            if op == "s_waitcnt":
                m = re.search(counter + r"\((\d+)\)", line)
                if m:
                    n = int(m.group(1))
                    st = {k: v for k, v in st.items() if v[0] < n}
                continue
            regs = set()
            for j, t in enumerate(args):
                rs = _regs2(t.split()[0]) if t else set()
                # the compiler does 32-bit multiply-adds with v_mad_u64_u32
                # and leaves the addend's high half undefined: not a use
                if j == 4 and op.startswith("v_mad_u64_u32") and len(rs) == 2:
                    rs = {min(rs)}
                regs |= rs
            # a younger read of the same kind into the same registers lands
            # after the older one (they return in order)
            ordered = returns(op, line)
            for key, (newer, dst) in st.items():
                if dst & regs and record and not ordered:
                    found.add("%s touches the registers of %s before its wait" % (line, key[2]))
            if counts(op, line):
                st = {k: (min(v[0] + 1, cap), v[1]) for k, v in st.items()}
            if returns(op, line) and args:
                st[(bi, ii, line)] = (0, _regs2(args[0].split()[0]))
        return st

    while work:
        bi = work.pop()
        out = step(entry[bi], bi, False)
        for sj in succ[bi]:
            cur = entry[sj]
            if cur is None:
                new = dict(out)
            else:
                new = dict(cur)
                for k, v in out.items():
                    new[k] = (min(v[0], new[k][0]), v[1]) if k in new else v
            if new != cur:
                entry[sj] = new
                work.append(sj)
    for bi in range(len(blocks)):
        if entry[bi] is not None:
            step(entry[bi], bi, True)
    return sorted(found)


def test_lds_wait_checker_flags_planted_uses():
    planted = """
_kernel:
    ds_read_b64 v[2:3], v10 offset:0
    ds_read_b64 v[4:5], v10 offset:8
    v_mov_b32_e32 v20, v2
    s_waitcnt lgkmcnt(1)
    v_mov_b32_e32 v21, v2
    v_mov_b32_e32 v22, v4
    s_waitcnt lgkmcnt(0)
    ds_read2_b64 v[30:33], v10 offset0:2 offset1:3
    s_cbranch_scc1 .LBB0_2
    v_add_f32_e32 v40, v41, v42
    s_waitcnt lgkmcnt(0)
.LBB0_2:
    v_mov_b32_e32 v31, 0
    s_waitcnt lgkmcnt(0)
    v_mov_b32_e32 v32, 0
    s_endpgm
"""
    got = find_lds_use_before_wait(planted)
    # v20 <- v2 before any wait; v22 <- v4 after lgkmcnt(1) (the younger read
    # may still be pending); v31 written at the join, where the branch taken
    # skipped the wait; not v21 <- v2 (retired by lgkmcnt(1)), not v32
    assert len(got) == 3, got
    assert any("v20, v2 " in g or g.startswith("v_mov_b32_e32 v20, v2") for g in got), got
    assert any(g.startswith("v_mov_b32_e32 v22, v4") for g in got), got
    assert any(g.startswith("v_mov_b32_e32 v31, 0") for g in got), got


COPY_SNIPPET = r"""
#include <hip/hip_runtime.h>
typedef unsigned int u2 __attribute__((ext_vector_type(2)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u2 rd(unsigned a)
{
    u2 r;
    asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
__global__ void copy_before_wait(u4 *out)
{
    extern __shared__ unsigned lds[];
    const unsigned a = (unsigned)(size_t)(__attribute__((address_space(3))) void *)(lds + 4 * threadIdx.x);
    const u2 r0 = rd(a), r1 = rd(a + 8);
    u4 x = {r0[1], r1[0], r0[0], r1[1]};
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x) :: "memory");
    out[threadIdx.x] = x;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_lds_wait_checker_catches_a_copy_before_the_wait(tmp_path):
    """Two asm reads whose results are rearranged into one operand before the
    tied wait: the compiler copies the registers before the data is in."""
    src = tmp_path / "copy.hip"
    src.write_text(COPY_SNIPPET)
    asm = _compile(tmp_path, src, "copy")
    assert find_lds_use_before_wait(asm) != []


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_small_m_kernels_wait_for_their_lds_reads(tmp_path):
    asm = _compile(tmp_path, os.path.join(os.path.dirname(SRC), "pn_smallm.hip"), "pn_smallm.hip")
    assert len(re.findall(r"^\s*ds_read2_b64", asm, re.M)) >= 16  # the read-ahead operands are there
    assert find_lds_use_before_wait(asm) == []


def test_vmem_wait_checker_flags_planted_uses():
    planted = """
_kernel:
    global_atomic_add v1, v[4:5], v3, off sc0
    buffer_load_dwordx4 v10, s[8:11], 0 offen lds
    v_add_u32_e32 v7, v1, v2
    s_waitcnt vmcnt(1)
    v_add_u32_e32 v8, v1, v2
    global_load_dword v20, v[4:5], off
    global_load_dword v22, v[4:5], off offset:4
    s_waitcnt vmcnt(1)
    v_mov_b32_e32 v21, v20
    global_store_dword v[4:5], v22, off
    global_load_dword v20, v[4:5], off offset:8
    s_endpgm
"""
    got = find_vmem_use_before_wait(planted)
    # v7 <- v1 before any wait; the store of v22 with its load possibly still
    # outstanding after vmcnt(1); not v8 <- v1 (the DMA load is younger than
    # the atomic), not v21 <- v20 (one younger load), not the second load
    # into v20 (loads return in order)
    assert len(got) == 2, got
    assert any(g.startswith("v_add_u32_e32 v7, v1") for g in got), got
    assert any(g.startswith("global_store_dword v[4:5], v22") for g in got), got


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_row_tile_grabs_are_waited_for(tmp_path):
    """The row-tile kernel's grabs are atomics issued from inline asm whose
    result is read a step later: no instruction may touch the result register
    before a vmcnt wait has retired the atomic, on any path."""
    asm = _compile(tmp_path, SRC, "rows")
    assert len(re.findall(r"^\s*global_atomic_add v\d+, v\[\d+:\d+\], v\d+, off sc0", asm, re.M)) >= 1
    assert find_vmem_use_before_wait(asm) == []


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_small_m_grabs_are_not_touched_early(tmp_path):
    """The small-M DMA kernel's group grab is read a group later, after at
    least one tile, whose every stage starts with an unconditional vmcnt(0)
    (the stage loop is a do-while).  The compiler wraps the tile in
    exec-masked regions, so the control-flow check above sees paths on which
    those regions are empty and the waits skipped, which no wave takes (every
    lane enters the tile); here the straight-line check asks that nothing
    touches the result register between the atomic and the first branch or
    wait, and the source keeps the read behind an asm statement tied to the
    register."""
    src = os.path.join(os.path.dirname(SRC), "pn_smallm.hip")
    asm = _compile(tmp_path, src, "smallm")
    assert len(re.findall(r"^\s*global_atomic_add v\d+, v\[\d+:\d+\], v\d+, off sc0", asm, re.M)) >= 2
    assert find_hazards(asm) == []
    text = open(src).read()
    assert 'asm volatile("" : "+v"(gr) :: "memory");  // read only here, after the stage waits' in text
    assert "} while (++s < nst);" in text
