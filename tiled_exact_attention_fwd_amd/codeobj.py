"""Reading the gfx950 code objects built into libfa_fwd.so (host side only).

The library's device code sits in the offload bundles of its ``.hip_fatbin``
section.  These helpers extract the gfx950 ELF code objects and read each
kernel's resource metadata (registers, spills, LDS, scratch) from their notes
with the ROCm llvm-readelf; the static checks of the instruction stream and
the tile-size sweep use them.
"""

import os
import re
import struct
import subprocess
import tempfile

LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def section(path, name):
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


def code_objects(lib_path):
    """gfx950 ELF code objects of every offload bundle in the library."""
    fatbin = section(lib_path, ".hip_fatbin")
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


def kernel_resources(lib_path):
    """{mangled kernel name: {vgpr, agpr, vgpr_spill, lds, scratch}} from the
    code objects' metadata notes."""
    readelf = os.path.join(LLVM, "llvm-readelf")
    res = {}
    with tempfile.TemporaryDirectory() as d:
        for i, co in enumerate(code_objects(lib_path)):
            path = os.path.join(d, f"co{i}.elf")
            with open(path, "wb") as f:
                f.write(co)
            notes = subprocess.run([readelf, "--notes", path], capture_output=True, text=True,
                                   check=True).stdout
            for blk in notes.split("- .agpr_count:")[1:]:
                def num(key):
                    m = re.search(r"\." + key + r":\s+(\d+)", blk)
                    return int(m.group(1)) if m else 0
                name = re.search(r"\.name:\s+(\S+)", blk).group(1)
                res[name] = {"vgpr": num("vgpr_count"), "agpr": int(blk.split()[0]),
                             "vgpr_spill": num("vgpr_spill_count"),
                             "lds": num("group_segment_fixed_size"),
                             "scratch": num("private_segment_fixed_size")}
    return res
