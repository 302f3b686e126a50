"""Static checks on the built gfx950 code object (CPU only).

The 16-bit kernels copy K and V tiles with the buffer unit's direct-to-LDS
loads. Two instruction orders around those copies gave nondeterministic
results during development, and the kernels are written to avoid both:

* an LDS write (``ds_write*``) by a wave while one of its own direct-to-LDS
  copies is in flight (issued, and not yet waited for with vmcnt(0));
* a scalar-memory load writing an SGPR that such an in-flight copy reads
  (its buffer resource or M0 source).

The code object is taken from ``libfa_fwd.so`` (the offload bundles in its
``.hip_fatbin`` section) and disassembled with the ROCm llvm-objdump; every
kernel is scanned in layout order, which is conservative across branches.
"""

import os
import re
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tiled_exact_attention_fwd_amd", "libfa_fwd.so")
LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _section(path, name):
    """Bytes of an ELF64 section, by name (minimal reader)."""
    data = open(path, "rb").read()
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    stroff = hdrs[shstrndx][4]
    for h in hdrs:
        end = data.index(b"\0", stroff + h[0])
        if data[stroff + h[0]:end].decode() == name:
            return data[h[4]:h[4] + h[5]]
    raise KeyError(name)


def _code_objects(fatbin):
    """gfx950 ELF code objects of every offload bundle in the section."""
    out = []
    pos = fatbin.find(MAGIC)
    while pos >= 0:
        n, = struct.unpack_from("<Q", fatbin, pos + len(MAGIC))
        q = pos + len(MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, q)
            triple = fatbin[q + 24:q + 24 + tlen].decode()
            q += 24 + tlen
            if "amdgcn" in triple and "gfx950" in triple:
                out.append(fatbin[pos + off:pos + off + size])
        pos = fatbin.find(MAGIC, pos + 1)
    return out


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
    cos = _code_objects(_section(LIB, ".hip_fatbin"))
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
