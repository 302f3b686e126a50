"""Builds libfa_fwd.so in-tree with hipcc for gfx950.

    python -m tiled_exact_attention_fwd_amd.build [-v]

The library is plain C ABI (include/fa_fwd.h); the Python binding loads it
with ctypes.  The kernel instances live in separate translation units
(fa_fwd_inst16.hip once per element type, head dimension and mask;
fa_fwd_inst32.hip once per mask; fa_bwd_inst.hip, the backward, once per
element type and head dimension) that compile in parallel and are linked
with the host layers (fa_fwd.hip, fa_standard.hip, fa_bwd.hip).  Packed-fp32 VALU instructions are
disabled: hipcc would otherwise form them from ordinary float code.
"""

import concurrent.futures as cf
import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa_fwd.so")
OBJDIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-variable",
                "-Wno-pass-failed"]
INFO = " ".join(COMMON_FLAGS + DEVICE_FLAGS)

# (object name, source, defines)
UNITS = [("fa_fwd", "fa_fwd.hip", [f'-DFA_BUILD_FLAGS="{INFO}"']), ("fa_standard", "fa_standard.hip", []),
         ("fa_probe", "fa_probe.hip", [])]
for t in ("bf16", "f16"):
    for d in (64, 128):
        for c in (0, 1):
            UNITS.append((f"inst16_{t}_d{d}_c{c}", "fa_fwd_inst16.hip",
                          [f"-DFA_INST_T={t}", f"-DFA_INST_D={d}", f"-DFA_INST_C={c}"]))
for c in (0, 1):
    UNITS.append((f"inst32_c{c}", "fa_fwd_inst32.hip", [f"-DFA_INST_C={c}"]))
# backward kernels, one unit per element type and head dimension
UNITS.append(("fa_bwd", "fa_bwd.hip", []))
UNITS.append(("bwd_f32", "fa_bwd_inst32.hip", []))
for t in ("bf16", "f16"):
    for d in (64, 128):
        UNITS.append((f"bwd_{t}_d{d}", "fa_bwd_inst.hip", [f"-DFA_INST_T={t}", f"-DFA_INST_D={d}"]))
# tile-size sweep shapes (bf16, d = 128, no mask)
for tq in (64, 128, 256):
    for tk in (32, 64, 128):
        if (tq, tk) != (256, 64):
            UNITS.append((f"inst16t_q{tq}_k{tk}", "fa_fwd_inst16_tiles.hip", [f"-DFA_TQ={tq}", f"-DFA_TK={tk}"]))


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _clean(text):
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    return [ln for ln in text.splitlines() if noise not in ln]


def _compile(unit, verbose):
    name, src, defs = unit
    obj = os.path.join(OBJDIR, name + ".o")
    cmd = ([hipcc()] + COMMON_FLAGS + DEVICE_FLAGS + defs + [f"-I{INCLUDE}", f"-I{CSRC}", "-c",
           os.path.join(CSRC, src), "-o", obj])
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = _clean(res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} ({' '.join(defs)}):\n" + "\n".join(msgs))
    return obj, msgs


def build(verbose=False, jobs=None):
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(UNITS), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda u: _compile(u, verbose), UNITS))
    objs = [o for o, _ in results]
    if verbose:
        for _, msgs in results:
            if msgs:
                print("\n".join(msgs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + "\n".join(_clean(res.stdout + res.stderr)))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
