"""Code generation checks on the built kernels (CPU only: reads the gfx950 code objects of
this build with the ROCm LLVM tools).

The kernels run at the register limit, and this compiler has been seen to place register
spill stores in the join block of a lane-dependent branch before the instruction that
restores the full execution mask.  Such a store saves only the lanes that took the branch;
the reload later hands the other lanes stale values, silently (a linear-verify kernel gave
wrong outputs that way).  The kernels avoid lane-dependent branches in their high-pressure
regions; this test checks every kernel for the pattern: a scratch store or load, or an
accumulator-register move, between the target of a branch taken when no lane is active and
the next write of the execution mask.
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJDIR = os.path.join(ROOT, "tree_verify_linear_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

pytestmark = pytest.mark.skipif(not os.path.isdir(OBJDIR) or not os.path.exists(f"{LLVM}/llvm-objdump"),
                                reason="needs the built objects and the ROCm LLVM tools")

_INST = re.compile(r"^\s+(\S.*?)\s*//\s*([0-9A-Fa-f]+):\s*[0-9A-F ]+(<(.+)\+0x([0-9a-f]+)>)?")
_FUNC = re.compile(r"^([0-9a-f]+) <(.+)>:$")
_NARROW = re.compile(r"s_(and|andn2|or|xor)_saveexec_b64|s_(and|andn2|mov|xor)_b64 exec")


def _disassemble(obj: str) -> str:
    with tempfile.TemporaryDirectory() as d:
        fb, co = os.path.join(d, "fatbin"), os.path.join(d, "code")
        subprocess.run([f"{LLVM}/llvm-objcopy", "-O", "binary", "--only-section=.hip_fatbin", obj, fb], check=True)
        if os.path.getsize(fb) == 0:
            return ""
        r = subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fb}",
                            f"--targets={TARGET}", f"--output={co}"], capture_output=True)
        if r.returncode != 0:
            return ""
        return subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--no-show-raw-insn", co], capture_output=True,
                              text=True, check=True).stdout


def _masked_spills(dis: str):
    insts, start, func = [], {}, None
    for line in dis.split("\n"):
        m = _FUNC.match(line)
        if m:
            func = m.group(2)
            continue
        m = _INST.match(line)
        if m and func:
            target = (m.group(4), int(m.group(5), 16)) if m.group(3) else None
            addr = int(m.group(2), 16)
            start.setdefault(func, addr)
            insts.append((addr, m.group(1).strip(), func, target))
    index = {a: i for i, (a, _, _, _) in enumerate(insts)}
    found = []
    for i, (_, text, func, target) in enumerate(insts):
        if not text.startswith("s_cbranch_execz") or not target:
            continue
        if not any(_NARROW.match(insts[k][1]) for k in range(max(0, i - 3), i)):
            continue                                   # not the entry of a lane-dependent region
        j = index.get(start[target[0]] + target[1])
        while j is not None and j < len(insts) and insts[j][2] == func:
            t = insts[j][1]
            if "exec" in t and not t.startswith("s_cbranch"):
                break
            if t.startswith(("s_cbranch", "s_branch", "s_endpgm")):
                break
            if t.startswith(("scratch_store", "scratch_load", "buffer_store", "v_accvgpr_write", "v_accvgpr_read")):
                found.append((func, t))
            j += 1
    return found


def _objects():
    if not os.path.isdir(OBJDIR):
        return []
    return sorted(os.path.join(OBJDIR, f) for f in os.listdir(OBJDIR) if f.endswith(".hip.o"))


def test_detector_finds_the_pattern():
    """The detector on a hand-written listing with the pattern, and without it."""
    head = "0000000000001000 <k>:\n"
    bad = head + "\n".join([
        "\ts_and_saveexec_b64 s[0:1], vcc // 000000001000: BE82206A",
        "\ts_cbranch_execz 2 // 000000001004: BF880002 <k+0xc>",
        "\tglobal_load_dword v1, v[2:3], off // 000000001008: DC508000",
        "\tscratch_store_dword off, v5, off offset:8 // 00000000100C: DC704008",
        "\ts_or_b64 exec, exec, s[0:1] // 000000001010: 87FE007E",
    ])
    good = bad.replace("\tscratch_store_dword off, v5, off offset:8 // 00000000100C: DC704008",
                       "\tv_add_f32_e32 v1, v1, v1 // 00000000100C: 02020301")
    assert len(_masked_spills(bad)) == 1
    assert _masked_spills(good) == []


@pytest.mark.parametrize("obj", _objects(), ids=os.path.basename)
def test_no_spill_under_a_narrowed_exec_mask(obj):
    dis = _disassemble(obj)
    found = _masked_spills(dis)
    assert not found, f"{os.path.basename(obj)}: {len(found)} spill accesses under a narrowed exec mask, " \
                      f"first in {found[0][0]}: {found[0][1]}"


def _functions(dis: str):
    funcs, cur = {}, None
    for line in dis.split("\n"):
        m = _FUNC.match(line)
        if m:
            cur = m.group(2)
            funcs[cur] = []
            continue
        m = _INST.match(line)
        if m and cur:
            funcs[cur].append(m.group(1).strip())
    return funcs


def test_plain_verify_waits_for_its_row_copies():
    """The plain bf16 verify waits for its global-to-LDS row copies by count: its first vector
    memory wait after the last copy leaves outstanding at most as many operations as it issued
    after the copies (the state tile's loads), so the copies themselves have landed."""
    obj = os.path.join(OBJDIR, "lin_tree.hip.o")
    if not os.path.exists(obj):
        pytest.skip("needs the built linear object")
    checked = 0
    for name, ins in _functions(_disassemble(obj)).items():
        if not re.search(r"lin_verify_kernelILi\d+ELi\d+ELb1ELb0ELb0E", name):
            continue
        first_mfma = next(i for i, x in enumerate(ins) if x.startswith("v_mfma"))
        copies = [i for i, x in enumerate(ins[:first_mfma]) if x.startswith("global_load_lds")]
        assert copies, name
        w = next(i for i in range(copies[-1], first_mfma) if re.match(r"s_waitcnt .*vmcnt\(\d+\)", ins[i]))
        allowed = int(re.search(r"vmcnt\((\d+)\)", ins[w]).group(1))
        after = sum(1 for x in ins[copies[-1] + 1:w] if re.match(r"(global|buffer)_load_(?!lds)", x))
        assert after >= allowed, f"{name}: waits for vmcnt({allowed}) with only {after} loads after the copies"
        checked += 1
    assert checked > 0


def test_attention_kernels_keep_everything_in_registers():
    """No attention kernel touches scratch memory.  Its PV accumulators are a register array
    indexed by row tile; a loop over row tiles that the compiler cannot unroll completely (an
    early exit on the run-time row-tile count, say) turns them into scratch memory, which
    keeps the results right and makes the kernel several times slower."""
    obj = os.path.join(OBJDIR, "attn_tree.hip.o")
    if not os.path.exists(obj):
        pytest.skip("needs the built attention object")
    checked = 0
    for name, ins in _functions(_disassemble(obj)).items():
        if "attn_kernel" not in name:
            continue
        bad = [x for x in ins if x.startswith(("scratch_", "buffer_load", "buffer_store"))]
        assert not bad, f"{name}: {len(bad)} scratch accesses, first {bad[0]}"
        checked += 1
    assert checked >= 8
