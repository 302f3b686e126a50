"""Builds libfa_fwd.so in-tree with hipcc for gfx950.

    python -m tiled_exact_attention_fwd_amd.build

The library is plain C ABI (include/fa_fwd.h); the Python binding loads it
with ctypes.  Packed-fp32 VALU instructions are disabled: hipcc would
otherwise form them from ordinary float code.
"""

import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa_fwd.so")

ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
                "-Wall", "-Wno-unused-variable"]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def command(out=LIB, extra=()):
    flags = COMMON_FLAGS + DEVICE_FLAGS + list(extra)
    info = " ".join(COMMON_FLAGS + DEVICE_FLAGS)
    return ([hipcc()] + flags +
            [f"-I{INCLUDE}", f"-I{CSRC}", f'-DFA_BUILD_FLAGS="{info}"',
             os.path.join(CSRC, "fa_fwd.hip"), "-o", out])


def build(verbose=False):
    cmd = command()
    tmp = LIB + ".tmp"
    cmd[-1] = tmp
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
