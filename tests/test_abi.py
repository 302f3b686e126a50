"""The C-ABI library without a GPU: it loads, exports every function that
include/*.h declares, and rejects bad arguments before any HIP call
(sizes must be positive, as the memory-model page's helpers require; null
pointers; bad flags; overlapping outputs; unsupported shapes)."""

import ctypes
import os
import re

import pytest

import tiled_exact_attention_fwd_amd as fa

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")

# fake, well separated device addresses: validation never dereferences them
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0   # counts devices without initialising one


# Calls whose arguments pass every check fail here only for lack of a GPU; with
# a device visible they would launch kernels on the fake addresses above, so
# they are made only where no device is visible.
NO_GPU = _no_gpu()


def declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_loads_and_exports_every_declared_symbol():
    lib = fa.lib()
    names = declared_functions()
    assert len(names) >= 9 and "fa_standard_fwd" in names
    for n in names:
        assert hasattr(lib, n), n
        assert n in fa.SIGNATURES, f"binding lacks {n}"
    # and the binding offers a function of the same name for each
    for n in names:
        assert callable(getattr(fa, n))


def test_build_info_and_strerror():
    assert "gfx950" in fa.fa_build_info()
    for st in (fa.FA_OK, fa.FA_ERR_INVALID, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP, 99):
        assert isinstance(fa.fa_strerror(st), str) and fa.fa_strerror(st)


def test_tile_shape():
    assert fa.fa_fwd_tile_shape(fa.FA_DTYPE_F32, 64, 0) == (fa.FA_OK, 64, 64)
    assert fa.fa_fwd_tile_shape(fa.FA_DTYPE_BF16, 128, 1) == (fa.FA_OK, 128, 64)
    assert fa.fa_fwd_tile_shape(fa.FA_DTYPE_F16, 64, 0) == (fa.FA_OK, 128, 64)
    assert fa.fa_fwd_tile_shape(fa.FA_DTYPE_BF16, 128, 0) == (fa.FA_OK, 256, 64)
    assert fa.fa_fwd_tile_shape(fa.FA_DTYPE_BF16, 96, 0)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_tile_shape(7, 64, 0)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_tile_shape(fa.FA_DTYPE_BF16, 64, 2)[0] == fa.FA_ERR_INVALID


def call(**over):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, N=100, d=64, scale=0.125, causal=0,
             stream=None, dtype=fa.FA_DTYPE_BF16)
    a.update(over)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                     a["d"], a["scale"], a["causal"], a["stream"], a["dtype"])


@pytest.mark.parametrize("field", ["B", "H", "N", "d"])
@pytest.mark.parametrize("value", [0, -1])
def test_nonpositive_sizes_are_invalid(field, value):
    assert call(**{field: value}) == fa.FA_ERR_INVALID


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_null_pointers_are_invalid(field):
    assert call(**{field: None}) == fa.FA_ERR_INVALID


def test_flags_and_scale():
    assert call(causal=2) == fa.FA_ERR_INVALID
    assert call(causal=-1) == fa.FA_ERR_INVALID
    for bad in (float("nan"), float("inf"), -float("inf")):
        assert call(scale=bad) == fa.FA_ERR_INVALID


def test_unsupported_shapes_and_types():
    assert call(d=32) == fa.FA_ERR_UNSUPPORTED
    assert call(d=256) == fa.FA_ERR_UNSUPPORTED
    assert call(dtype=5) == fa.FA_ERR_UNSUPPORTED
    # per-head extent beyond 2^31 bytes
    assert call(N=1 << 22, d=128) == fa.FA_ERR_UNSUPPORTED


def test_overlapping_outputs_are_invalid():
    nbytes = 2 * 3 * 100 * 64 * 2
    assert call(o=Q) == fa.FA_ERR_INVALID
    assert call(o=Q + nbytes - 2) == fa.FA_ERR_INVALID           # tail overlap
    assert call(lse=V + 16) == fa.FA_ERR_INVALID
    assert call(lse=O + 8) == fa.FA_ERR_INVALID                  # o and lse overlap
    # q, k, v may alias one another (read only): rejected only later, for lack of a GPU
    if NO_GPU:
        st = call(k=Q, v=Q)
        assert st in (fa.FA_ERR_HIP, fa.FA_ERR_UNSUPPORTED, fa.FA_OK)


def test_ex_argument_checks():
    def ex(**over):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=256, d=64, scale=0.125, causal=0,
                 stream=None, dtype=fa.FA_DTYPE_F32)
        a.update(over)
        return fa.fa_fwd_ex(**a)
    assert ex(out_dtype=2) == fa.FA_ERR_INVALID
    assert ex(tile_q=32, tile_k=64) == fa.FA_ERR_UNSUPPORTED
    assert ex(tile_q=-1) == fa.FA_ERR_INVALID
    assert fa.lib().fa_fwd_ex(None) == fa.FA_ERR_INVALID
    # the tile-size sweep shapes exist for bf16, d = 128, no mask, 16-bit output only
    sweep = dict(dtype=fa.FA_DTYPE_BF16, d=128)
    passes_checks = (fa.FA_ERR_HIP, fa.FA_ERR_UNSUPPORTED, fa.FA_OK)   # no GPU here
    for tq in (64, 128, 256):
        for tk in (32, 64, 128):
            if NO_GPU:
                assert ex(tile_q=tq, tile_k=tk, **sweep) in passes_checks
            if (tq, tk) != (128, 64):
                assert ex(tile_q=tq, tile_k=tk, causal=1, **sweep) == fa.FA_ERR_UNSUPPORTED
            elif NO_GPU:
                assert ex(tile_q=tq, tile_k=tk, causal=1, **sweep) in passes_checks
            if (tq, tk) != (256, 64):
                assert ex(tile_q=tq, tile_k=tk, out_dtype=1, **sweep) == fa.FA_ERR_UNSUPPORTED
            elif NO_GPU:
                assert ex(tile_q=tq, tile_k=tk, out_dtype=1, **sweep) in passes_checks
    assert ex(tile_q=128, tile_k=32, dtype=fa.FA_DTYPE_F16, d=128) == fa.FA_ERR_UNSUPPORTED
    assert ex(tile_q=128, tile_k=32, dtype=fa.FA_DTYPE_BF16, d=64) == fa.FA_ERR_UNSUPPORTED
    assert ex(tile_q=512, tile_k=64, **sweep) == fa.FA_ERR_UNSUPPORTED


def test_standard_argument_checks():
    S, P = 0x60000000, 0x70000000

    def std(**over):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, s=S, p=P, B=1, H=1, N=256, d=64, scale=0.125, causal=0,
                 stream=None, dtype=fa.FA_DTYPE_BF16)
        a.update(over)
        return fa.fa_standard_fwd(**a)
    assert std(B=0) == fa.FA_ERR_INVALID
    assert std(N=-1) == fa.FA_ERR_INVALID
    assert std(s=None) == fa.FA_ERR_INVALID
    assert std(p=P + 8) == fa.FA_ERR_INVALID              # not 16-byte aligned
    assert std(causal=2) == fa.FA_ERR_INVALID
    assert std(scale=float("nan")) == fa.FA_ERR_INVALID
    assert std(dtype=fa.FA_DTYPE_F32) == fa.FA_ERR_UNSUPPORTED
    assert std(d=96) == fa.FA_ERR_UNSUPPORTED
    assert std(N=1 << 23, d=128) == fa.FA_ERR_UNSUPPORTED
    assert std(N=1 << 22, d=128) == fa.FA_ERR_UNSUPPORTED


def test_per_dtype_entry_points_share_validation():
    for fn in (fa.fa_fwd_bf16, fa.fa_fwd_f16, fa.fa_fwd_f32):
        assert fn(Q, K, V, O, L, 0, 1, 1, 64, 1.0, 0, None) == fa.FA_ERR_INVALID
        assert fn(Q, K, V, O, L, 1, 1, 1, 48, 1.0, 0, None) == fa.FA_ERR_UNSUPPORTED


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(fa.FaLibraryMissing):
        fa.lib(str(tmp_path / "nope.so"))


def test_struct_layout_matches_header():
    # 5 pointers, 4 ints, float, int, pointer, 4 ints, pointer on LP64
    assert ctypes.sizeof(fa.FaArgs) == 5 * 8 + 4 * 4 + 4 + 4 + 8 + 4 * 4 + 8


def test_backward_argument_checks():
    DO, DQ, DK, DV, DL = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000

    def bwd(**over):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, delta=DL, B=2, H=3, N=100, d=64,
                 scale=0.125, causal=0, stream=None, dtype=fa.FA_DTYPE_BF16)
        a.update(over)
        return fa.fa_bwd(**a)
    nbytes = 2 * 3 * 100 * 64 * 2
    for field in ("B", "H", "N", "d"):
        assert bwd(**{field: 0}) == fa.FA_ERR_INVALID
        assert bwd(**{field: -3}) == fa.FA_ERR_INVALID
    for field in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta"):
        assert bwd(**{field: None}) == fa.FA_ERR_INVALID
    assert bwd(causal=2) == fa.FA_ERR_INVALID
    assert bwd(scale=float("inf")) == fa.FA_ERR_INVALID
    assert bwd(dq=Q + nbytes - 2) == fa.FA_ERR_INVALID            # output over an input
    assert bwd(dv=DK + 64) == fa.FA_ERR_INVALID                   # outputs overlap each other
    assert bwd(delta=L + 4) == fa.FA_ERR_INVALID                  # work array over the lse input
    if NO_GPU:
        assert bwd(dtype=fa.FA_DTYPE_F32) in (fa.FA_ERR_HIP, fa.FA_OK)        # fp32 is built
    assert bwd(dtype=fa.FA_DTYPE_F32, dq=Q + 2 * 3 * 100 * 64 * 4 - 4) == fa.FA_ERR_INVALID   # 4-byte elements
    assert bwd(dtype=9) == fa.FA_ERR_UNSUPPORTED
    assert bwd(d=96) == fa.FA_ERR_UNSUPPORTED
    assert bwd(N=1 << 23, d=128) == fa.FA_ERR_UNSUPPORTED
    assert bwd(N=1 << 22, d=128) == fa.FA_ERR_UNSUPPORTED      # N d 4 = 2^31: as for the forward
    # inputs may alias each other; with valid arguments the call only fails for lack of a GPU
    if NO_GPU:
        assert bwd(k=Q, v=Q) in (fa.FA_ERR_HIP, fa.FA_OK)
    for fn in (fa.fa_bwd_bf16, fa.fa_bwd_f16, fa.fa_bwd_f32):
        assert fn(Q, K, V, O, L, DO, DQ, DK, DV, DL, 0, 1, 1, 64, 1.0, 0, None) == fa.FA_ERR_INVALID
        assert fn(Q, K, V, O, L, DO, DQ, DK, DV, DL, 1, 1, 1, 48, 1.0, 0, None) == fa.FA_ERR_UNSUPPORTED


def test_backward_o32_argument_checks():
    """fa_bwd_o32: fa_bwd's checks, with o taken as fp32 (4-byte elements)
    whatever the element type of the rest."""
    DO, DQ, DK, DV, DL = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000

    def bwd(**over):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, delta=DL, B=2, H=3, N=100, d=64,
                 scale=0.125, causal=0, stream=None, dtype=fa.FA_DTYPE_BF16)
        a.update(over)
        return fa.fa_bwd_o32(**a)
    for field in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta"):
        assert bwd(**{field: None}) == fa.FA_ERR_INVALID
    assert bwd(B=0) == fa.FA_ERR_INVALID
    assert bwd(causal=2) == fa.FA_ERR_INVALID
    assert bwd(d=96) == fa.FA_ERR_UNSUPPORTED
    assert bwd(dtype=9) == fa.FA_ERR_UNSUPPORTED
    n16 = 2 * 3 * 100 * 64 * 2
    # an output just past a 16-bit O lies inside the fp32 one
    assert bwd(dq=O + n16) == fa.FA_ERR_INVALID
    assert bwd(dq=O + 2 * n16 - 4) == fa.FA_ERR_INVALID
    if NO_GPU:
        assert bwd(dq=O + 2 * n16) in (fa.FA_ERR_HIP, fa.FA_OK)
        assert fa.fa_bwd(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=O + n16, dk=DK, dv=DV, delta=DL, B=2, H=3,
                         N=100, d=64, scale=0.125, causal=0, stream=None,
                         dtype=fa.FA_DTYPE_BF16) in (fa.FA_ERR_HIP, fa.FA_OK)


def test_backward_noalloc_argument_checks():
    """fa_bwd_noalloc: fa_bwd's checks without the delta argument, and a
    problem beyond its fixed scratch array (one fp32 per query row) refused
    with FA_ERR_SCRATCH before any HIP call."""
    DO, DQ, DK, DV = 0x60000000, 0x70000000, 0x80000000, 0x90000000

    def bwd(**over):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, B=2, H=3, N=100, d=64,
                 scale=0.125, causal=0, stream=None, dtype=fa.FA_DTYPE_BF16)
        a.update(over)
        return fa.fa_bwd_noalloc(**a)
    assert fa.FA_ERR_SCRATCH == 4 and "scratch" in fa.fa_strerror(fa.FA_ERR_SCRATCH)
    for field in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv"):
        assert bwd(**{field: None}) == fa.FA_ERR_INVALID
    assert bwd(N=0) == fa.FA_ERR_INVALID
    assert bwd(dv=DK + 64) == fa.FA_ERR_INVALID
    assert bwd(d=96) == fa.FA_ERR_UNSUPPORTED
    rows = fa.BWD_NOALLOC_MAX_ROWS
    # one row more than the scratch holds, far apart fake buffers (1 GiB each)
    big = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40, lse=5 << 40, dout=6 << 40, dq=7 << 40, dk=8 << 40,
               dv=9 << 40, d=64)
    assert bwd(B=1, H=1, N=rows + 1, **big) == fa.FA_ERR_SCRATCH
    assert bwd(B=2, H=2, N=rows // 4 + 1, **big) == fa.FA_ERR_SCRATCH
    if NO_GPU:   # exactly the scratch size passes the checks; here it then fails for lack of a GPU
        assert bwd(B=1, H=1, N=rows, **big) == fa.FA_ERR_HIP


def test_split_count_argument_checks():
    for args in [(0, 1, 100, 64, 0), (1, -1, 100, 64, 0), (1, 1, 0, 64, 0), (1, 1, 100, 64, 2)]:
        assert fa.fa_fwd_split_count(*args, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_INVALID, args
    assert fa.fa_fwd_split_count(1, 1, 100, 96, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_split_count(1, 1, 100, 64, 0, 9)[0] == fa.FA_ERR_UNSUPPORTED
    assert fa.lib().fa_fwd_split_count(1, 1, 100, 64, 0, fa.FA_DTYPE_BF16, None) == fa.FA_ERR_INVALID
    if NO_GPU:   # valid arguments: the device query fails here
        assert fa.fa_fwd_split_count(1, 1, 100, 64, 0, fa.FA_DTYPE_BF16)[0] == fa.FA_ERR_HIP


def test_split_argument_checks():
    OP, LP = 0x60000000, 0x70000000

    def split(**over):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, o_part=OP, lse_part=LP, B=2, H=3, N=100, d=64, scale=0.125, causal=0,
                 splits=2, stream=None, dtype=fa.FA_DTYPE_BF16)
        a.update(over)
        return fa.fa_fwd_split(**a)
    assert split(B=0) == fa.FA_ERR_INVALID
    assert split(N=-5) == fa.FA_ERR_INVALID
    assert split(o_part=None) == fa.FA_ERR_INVALID
    assert split(lse_part=None) == fa.FA_ERR_INVALID
    assert split(splits=0) == fa.FA_ERR_INVALID
    assert split(o_part=Q + 64) == fa.FA_ERR_INVALID          # work array over an input
    assert split(lse_part=O + 16) == fa.FA_ERR_INVALID        # work array over the output
    assert split(lse_part=OP + 1024) == fa.FA_ERR_INVALID     # the two work arrays overlap
    assert split(scale=float("nan")) == fa.FA_ERR_INVALID
    if NO_GPU:
        assert split(dtype=fa.FA_DTYPE_F32) in (fa.FA_ERR_HIP, fa.FA_OK)  # fp32 is built
    assert split(dtype=fa.FA_DTYPE_F32, o_part=Q + 2 * 3 * 100 * 64 * 4 - 4) == fa.FA_ERR_INVALID
    assert split(d=80) == fa.FA_ERR_UNSUPPORTED
    assert split(causal=2) == fa.FA_ERR_INVALID
    if NO_GPU:   # valid: fails only for lack of a GPU
        assert split() in (fa.FA_ERR_HIP, fa.FA_ERR_UNSUPPORTED, fa.FA_OK)
        assert split(causal=1) in (fa.FA_ERR_HIP, fa.FA_ERR_UNSUPPORTED, fa.FA_OK)


def test_split_ranges_rule():
    # whole 64-key tiles, no empty range, never more ranges than asked for
    for N in (1, 63, 64, 65, 1000, 4096, 32768):
        for s in (1, 2, 3, 7, 64, 1000):
            r = fa.split_ranges(N, s)
            assert 1 <= len(r) <= s and r[0][0] == 0 and r[-1][1] == N
            assert all(a < b for a, b in r) and all(r[i][1] == r[i + 1][0] for i in range(len(r) - 1))
            assert all(a % 64 == 0 for a, _ in r)


def test_product_path_does_not_touch_the_oracle():
    """The binding, its build script and the input generators import nothing
    from oracle/ (only the tests, the smoke check and the bench's CPU
    baseline may); checked in a fresh interpreter and in the sources."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; import tiled_exact_attention_fwd_amd as fa, fa_workloads; "
            "import tiled_exact_attention_fwd_amd.build, tiled_exact_attention_fwd_amd.codeobj; fa.lib(); "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "assert not bad, bad")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    pkg = os.path.join(root, "tiled_exact_attention_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(import oracle|from oracle)", text, flags=re.M), f


def test_preallocated_outputs_are_checked():
    """attention() hands o and lse to the kernel as raw pointers: buffers of
    the wrong type, size, layout or device are refused before any launch."""
    import torch
    q = torch.empty((2, 3, 100, 64), dtype=torch.bfloat16)
    good_o, good_lse = torch.empty_like(q), torch.empty((2, 3, 100), dtype=torch.float32)
    fa.check_outputs(q, good_o, good_lse)
    fa.check_outputs(q, torch.empty(q.shape, dtype=torch.float32), good_lse, out_f32=True)
    bad_o = [torch.empty(q.shape, dtype=torch.float32),                 # fp32 without out_f32
             torch.empty((2, 3, 99, 64), dtype=torch.bfloat16),         # too small
             torch.empty((2, 3, 64, 100), dtype=torch.bfloat16).transpose(2, 3)]   # strided
    for o in bad_o:
        with pytest.raises(ValueError):
            fa.check_outputs(q, o, good_lse)
    with pytest.raises(ValueError):
        fa.check_outputs(q, good_o, good_lse, out_f32=True)             # bf16 o for an fp32 launch
    bad_lse = [torch.empty((2, 3, 100), dtype=torch.float16),
               torch.empty((2, 3, 50), dtype=torch.float32),
               torch.empty((2, 100, 3), dtype=torch.float32).transpose(1, 2)]
    for lse in bad_lse:
        with pytest.raises(ValueError):
            fa.check_outputs(q, good_o, lse)
    if torch.cuda.is_available():
        with pytest.raises(ValueError):
            fa.check_outputs(q.cuda(), good_o, good_lse)               # host buffers for a device launch


def test_launch_tile_argument_checks():
    """fa_fwd_launch_tile checks its arguments as fa_fwd_ex does, before any
    HIP call; with valid arguments it needs the device (its compute units
    decide between the persistent and the per-tile kernels)."""
    def lt(**over):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, N=100, d=64, scale=0.125, causal=0,
                 stream=None, dtype=fa.FA_DTYPE_BF16)
        a.update(over)
        return fa.fa_fwd_launch_tile(**a)
    assert lt(B=0)[0] == fa.FA_ERR_INVALID
    assert lt(q=None)[0] == fa.FA_ERR_INVALID
    assert lt(o=Q)[0] == fa.FA_ERR_INVALID
    assert lt(causal=3)[0] == fa.FA_ERR_INVALID
    assert lt(d=96)[0] == fa.FA_ERR_UNSUPPORTED
    assert lt(tile_q=32, tile_k=64)[0] == fa.FA_ERR_UNSUPPORTED
    a = fa.FaArgs(Q, K, V, O, L, 2, 3, 100, 64, 0.125, 0, None, fa.FA_DTYPE_BF16, 0, 0, 0, None)
    t = ctypes.c_int(0)
    assert fa.lib().fa_fwd_launch_tile(ctypes.byref(a), None, ctypes.byref(t)) == fa.FA_ERR_INVALID
    assert fa.lib().fa_fwd_launch_tile(None, ctypes.byref(t), ctypes.byref(t)) == fa.FA_ERR_INVALID
    if NO_GPU:
        assert lt()[0] == fa.FA_ERR_HIP
