"""Static checks on the built gfx950 code object (CPU only).

The 16-bit kernels copy K and V tiles with the buffer unit's direct-to-LDS
loads. Two instruction orders around those copies gave nondeterministic
results during development, and the kernels are written to avoid both:

* an LDS write (``ds_write*``) by a wave while one of its own direct-to-LDS
  copies is in flight (issued, and not yet waited for with vmcnt(0));
* a scalar-memory load writing an SGPR that such an in-flight copy reads
  (its buffer resource or M0 source).

The code objects are taken from ``libfa_fwd.so`` (``codeobj.code_objects``)
and disassembled with the ROCm llvm-objdump; every
kernel is scanned in layout order, which is conservative across branches.
"""

import os
import re
import subprocess

import pytest

from tiled_exact_attention_fwd_amd.codeobj import LLVM, code_objects

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tiled_exact_attention_fwd_amd", "libfa_fwd.so")


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def scan(lines):
    """Returns the offending instructions of one kernel (layout order)."""
    live = set()           # SGPRs read by in-flight direct-to-LDS copies
    inflight = False
    bad = []
    m0_src = None
    for ins in lines:
        parts = ins.replace(",", " ").split()
        if not parts:
            continue
        op = parts[0]
        if op == "s_waitcnt" and re.search(r"vmcnt\(0\)", ins):
            live, inflight = set(), False
        elif op == "s_mov_b32" and len(parts) > 2 and parts[1] == "m0":
            m0_src = parts[2]
        elif op.startswith("buffer_load") and " lds" in f" {ins} ":
            inflight = True
            for t in parts[1:]:
                live |= _sgprs(t)
            if m0_src:
                live |= _sgprs(m0_src)
        elif op.startswith("ds_write") and inflight:
            bad.append(ins)
        elif (op.startswith("s_load") or op.startswith("s_buffer_load")) and len(parts) > 1:
            if _sgprs(parts[1]) & live:
                bad.append(ins)
    return bad


def test_scanner_flags_both_orders():
    """The scanner itself, on hand-written snippets of both bad orders."""
    dma = ["s_mov_b32 m0, s35", "buffer_load_dwordx4 v183, s[20:23], 0 offen lds"]
    assert scan(dma + ["ds_write_b128 v1, v[2:5]"]) == ["ds_write_b128 v1, v[2:5]"]
    assert scan(dma + ["s_load_dwordx2 s[22:23], s[0:1], 0x20"]) == ["s_load_dwordx2 s[22:23], s[0:1], 0x20"]
    assert scan(dma + ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_barrier", "ds_write_b128 v1, v[2:5]",
                       "s_load_dwordx2 s[22:23], s[0:1], 0x20"]) == []
    assert scan(["ds_write_b128 v1, v[2:5]"] + dma) == []


def test_no_lds_write_or_smem_overwrite_during_lds_copies(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libfa_fwd.so is not built")
    objdump = os.path.join(LLVM, "llvm-objdump")
    if not os.path.exists(objdump):
        pytest.skip("llvm-objdump not available")
    cos = code_objects(LIB)
    assert cos, "no gfx950 code object in the library"
    kernels = 0
    problems = {}
    for i, co in enumerate(cos):
        path = tmp_path / f"co{i}.elf"
        path.write_bytes(co)
        res = subprocess.run([objdump, "-d", "--mcpu=gfx950", "--no-show-raw-insn", str(path)],
                             capture_output=True, text=True, check=True)
        name, lines = None, []
        for raw in res.stdout.splitlines() + ["<end>:"]:
            m = re.match(r"^[0-9a-f]+ <(.+)>:$", raw) or (raw == "<end>:" and re.match(r"(.*)", "<end>"))
            if m:
                if name and "fwd_kernel" in name:
                    kernels += 1
                    bad = scan(lines)
                    if bad:
                        problems[name] = bad[:5]
                name, lines = m.group(1), []
                continue
            ins = raw.split("//")[0].strip()
            if ins:
                lines.append(ins)
    assert kernels >= 16, kernels
    assert not problems, problems


def test_no_scratch_memory():
    """Every kernel keeps its state in registers and LDS: no private
    (scratch) memory and no spilled registers -- except the 256 x 128 tile of
    the tile-size sweep, whose score and term registers do not fit beside the
    accumulators (the sweep table reports its spills)."""
    from tiled_exact_attention_fwd_amd.codeobj import kernel_resources
    res = kernel_resources(LIB)
    assert len(res) > 100
    sweep_256x128 = "ELi8ELi128E"   # Fwd16<..., WQ = 8 waves, BKT = 128 keys>
    bad = {n: r for n, r in res.items() if (r["scratch"] or r["vgpr_spill"]) and sweep_256x128 not in n}
    assert not bad, bad
