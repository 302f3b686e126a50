"""GPU parity of the HIP forward pass against the float64 oracle.

Every launch goes through the C ABI (ctypes binding).  Inputs are the seeded
words of fa_workloads, uploaded as-is and decoded exactly for the oracle.
Gates are described in parity_util: G1 (fp32-output launch within the
tolerance), G2 (16-bit output within tolerance beyond its own half ulp), LSE
within 1e-3; tile counts bit-exact against oracle.block_counts at the shape
the library reports.
"""

import math

import numpy as np
import pytest
import torch

import fa_workloads as W
import oracle
import tiled_exact_attention_fwd_amd as fa
from parity_util import (TOL_O, TOL_LSE, assert_gates, gate_errors, out_to64,
                         sample_rows, to_dev)

pytestmark = pytest.mark.gpu

CODE = {"f32": fa.FA_DTYPE_F32, "f16": fa.FA_DTYPE_F16, "bf16": fa.FA_DTYPE_BF16}


def launch_tile(qd, kd, vd, o, lse, causal, scale):
    """The tile of the kernel the plain launch with these tensors runs."""
    B, H, N, d = qd.shape
    st, tq, tk = fa.fa_fwd_launch_tile(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                       B, H, N, d, float(scale), int(causal),
                                       torch.cuda.current_stream().cuda_stream, fa.dtype_code(qd.dtype))
    assert st == fa.FA_OK, fa.fa_strerror(st)
    return tq, tk


def expected_counts(qd, kd, vd, o, lse, causal, scale):
    """Block counts of P1 §2.2 (oracle.block_counts) at the tile the launch
    runs in, summed over its heads."""
    B, H, N, d = qd.shape
    tq, tk = launch_tile(qd, kd, vd, o, lse, causal, scale)
    c = oracle.block_counts(N, tq, tk, causal)
    return {k: v * B * H for k, v in c.items()}


def oracle_heads(words, dtype, scale, causal, heads, rows=None):
    """The float64 oracle on each listed head (threads: numpy and BLAS release
    the interpreter lock), in the order given."""
    from concurrent.futures import ThreadPoolExecutor

    def one(bh):
        b, h = bh
        vals = [W.decode64(w[b, h], dtype)[None, None] for w in words]
        return oracle.attention_ref(*vals, scale, causal, rows=rows)
    with ThreadPoolExecutor(16) as ex:
        return list(ex.map(one, heads))


def launch_all(qd, kd, vd, dtype, causal, scale):
    """Plain launch (output in the input type), fp32-output launch, and the
    instrumented launch; returns (o, lse, o32, lse32, counts)."""
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    if dtype == "f32":
        o32, lse32 = o, lse
    else:
        o32, lse32 = fa.attention(qd, kd, vd, causal=causal, scale=scale, out_f32=True)
    oc, lsec, cnt = fa.attention(qd, kd, vd, causal=causal, scale=scale, counters=True)
    torch.cuda.synchronize()
    # the instrumented kernel computes exactly what the plain one does
    assert torch.equal(oc.view(torch.int16) if dtype != "f32" else oc, o.view(torch.int16) if dtype != "f32" else o)
    assert torch.equal(lsec, lse)
    return o, lse, o32, lse32, cnt


def check_against_oracle(words, dtype, causal, scale, rows=None, heads=None, what=""):
    B, H, N, d = words[0].shape
    qd, kd, vd = (to_dev(w, dtype) for w in words)
    o, lse, o32, lse32, cnt = launch_all(qd, kd, vd, dtype, causal, scale)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    o_np, lse_np = out_to64(o), lse.cpu().numpy().astype(np.float64)
    o32_np = out_to64(o32)
    worst = {}
    sel = slice(None) if rows is None else rows
    for (b, h), (o_ref, lse_ref) in zip(heads, oracle_heads(words, dtype, scale, causal, heads, rows)):
        errs = gate_errors(o32_np[b, h, sel][None, None], None if dtype == "f32" else o_np[b, h, sel][None, None],
                           lse_np[b, h, sel][None, None], o_ref, lse_ref, dtype)
        assert_gates(errs, dtype, f"{what} head ({b},{h})")
        for k_, v_ in errs.items():
            worst[k_] = max(worst.get(k_, 0.0), v_)
    assert cnt == expected_counts(qd, kd, vd, o, lse, causal, scale), f"{what} counts {cnt}"
    return worst, (qd, kd, vd, o, lse, o32)


# ---------------------------------------------------------------------------
# Small shapes: several tiles, ragged tails, every instance; full oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 128, 200, 257])
def test_small_16bit(dtype, d, causal, N):
    words = W.make_words((2, 2, N, d), dtype, "normal", seed=N + d)
    worst, _ = check_against_oracle(words, dtype, causal, W.scale_for(d), what=f"N={N} d={d}")
    print(f"{dtype} d={d} causal={causal} N={N}: {worst}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 256, 300])
def test_small_f32(d, causal, N):
    words = W.make_words((1, 3, N, d), "f32", "normal", seed=N + d)
    worst, _ = check_against_oracle(words, "f32", causal, W.scale_for(d), what=f"N={N} d={d}")
    # fp32 matrix-core arithmetic: far inside the stated gate
    assert worst["g1"] < 1e-4 and worst["lse"] < 1e-4, worst
    print(f"f32 d={d} causal={causal} N={N}: {worst}")


def _random_shapes(seed, count):
    """Seeded shapes: N near tile boundaries (multiples of 64 and 128 plus or
    minus one) or anywhere up to 3000, both head dimensions, both masks."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        if rng.random() < 0.5:
            N = int(rng.integers(1, 24)) * int(rng.choice([64, 128])) + int(rng.choice([-1, 0, 1]))
        else:
            N = int(rng.integers(1, 3001))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 6)), max(N, 1), int(rng.choice([64, 128])),
                    str(rng.choice(["bf16", "f16"])), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,H,N,d,dtype,causal", _random_shapes(2024, 16))
def test_random_shapes(B, H, N, d, dtype, causal):
    """Seeded random shapes against the oracle on every head and row, with
    the tile counts of the launched kernel."""
    print(f"random shape {B}x{H}x{N}x{d} {dtype} causal={causal}", flush=True)
    words = W.make_words((B, H, N, d), dtype, "normal", N)
    worst, _ = check_against_oracle(words, dtype, causal, W.scale_for(d), what="random")
    print(worst)


def _random_persistent_shapes(seed, count):
    """Seeded d = 128 shapes with enough query tiles for the persistent
    kernels (more 256-row tiles, or causal pairs of them, than CUs)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        causal = i % 2 == 1
        if causal:   # an even number of 256-row tiles: the paired causal kernel
            wt = 2 * int(rng.integers(1, 6))
            N = 256 * wt - int(rng.integers(0, 256))
            heads = 512 // wt + int(rng.integers(1, 120))
        else:
            N = int(rng.integers(300, 2600))
            heads = int(rng.integers(96, 400))
        out.append((1, heads, N, str(rng.choice(["bf16", "f16"])), causal))
    return out


@pytest.mark.parametrize("B,H,N,dtype,causal", _random_persistent_shapes(2026, 6))
def test_random_persistent_shapes(B, H, N, dtype, causal):
    """Seeded shapes on the persistent kernels' path: three whole heads
    (first, middle, last) against the oracle, counts of the launched kernel."""
    print(f"random persistent shape {B}x{H}x{N}x128 {dtype} causal={causal}", flush=True)
    words = W.make_words((B, H, N, 128), dtype, "normal", N + H)
    heads = [(0, 0), (0, H // 2), (0, H - 1)]
    worst, _ = check_against_oracle(words, dtype, causal, W.scale_for(128), heads=heads, what="random persistent")
    print(worst)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_spiky_and_scales(dtype):
    """Running-max rescales (a few keys x8), a negative scale, a large scale
    that makes the softmax nearly one-hot."""
    words = W.make_words((1, 2, 300, 128), dtype, "spiky", seed=5)
    check_against_oracle(words, dtype, True, W.scale_for(128), what="spiky")
    words = W.make_words((1, 2, 190, 64), dtype, "normal", seed=6)
    check_against_oracle(words, dtype, False, -0.2, what="negative scale")
    check_against_oracle(words, dtype, True, 2.0, what="large scale")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d,scale,values,causal", [(128, 0.5, "normal", False), (64, 1.0, "normal", False),
                                                   (128, None, "spiky", False)])
def test_peaked_rows(dtype, d, scale, values, causal):
    """Softmax rows dominated by one or two keys that first appear after the
    row's reference was set (several tiles in): the dominant term has to be
    applied and summed consistently, or its 16-bit rounding shows in O at
    the 2^-8 level."""
    words = W.make_words((1, 2, 320, d), dtype, values, seed=d + 7)
    sc = W.scale_for(d) if scale is None else scale
    worst, _ = check_against_oracle(words, dtype, causal, sc, what=f"peaked d={d} scale={sc} {values}")
    print(f"{dtype} peaked d={d} scale={sc} {values}: {worst}")


# ---------------------------------------------------------------------------
# The named workloads at full size, launched as the benchmark launches them;
# sampled rows against the oracle, properties on every row
# ---------------------------------------------------------------------------

WORKLOAD_CASES = [("C1", False), ("C1", True), ("C2", False), ("C2b", False), ("C3", True),
                  ("C4", False), ("C4", True), ("C5", True)]


@pytest.mark.parametrize("name,causal", WORKLOAD_CASES)
def test_workload(name, causal):
    """Every head of the named workload, launched as the benchmark launches
    it.  Every row is compared with the oracle, except at the long-context
    shape (32 heads of 32768 rows), where the rows are 0, 1, N-2, N-1, both
    sides of every 64-row boundary (so of every query and key tile boundary
    of the kernels: 64, 128 and 256 rows) and 64 random ones -- exact per row,
    since the oracle computes each row over all its keys."""
    wl = W.WORKLOADS[name]
    print(f"workload {name} causal={causal} shape={wl.shape} dtype={wl.dtype}", flush=True)
    words = W.make_words(wl.shape, wl.dtype, wl.values, W.default_seed())
    rng = np.random.default_rng(123)
    B, H, N, d = wl.shape
    heads = [(b, h) for b in range(B) for h in range(H)]
    rows = None if N <= 4096 else sample_rows(N, 64, rng, n_random=64)
    worst, (qd, kd, vd, o, lse, o32) = check_against_oracle(
        words, wl.dtype, causal, W.scale_for(d), rows=rows, heads=heads, what=name)
    print(f"{name} causal={causal}: {worst}")
    # every row: the output is a convex combination of the visible value rows
    vf = vd.float()
    if causal:
        lo, hi = torch.cummin(vf, dim=2).values, torch.cummax(vf, dim=2).values
    else:
        lo, hi = vf.amin(dim=2, keepdim=True), vf.amax(dim=2, keepdim=True)
    tol = TOL_O[wl.dtype]
    assert bool((o32 >= lo - tol).all()) and bool((o32 <= hi + tol).all())
    assert bool(torch.isfinite(lse).all())


# ---------------------------------------------------------------------------
# Closed forms and degenerate cases, no oracle needed
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_closed_forms(dtype, d):
    B, H, N = 2, 2, 333
    words = W.make_words((B, H, N, d), dtype, "normal", seed=11)
    qd, kd, vd = (to_dev(w, dtype) for w in words)
    v64 = W.decode64(words[2], dtype)
    q64, k64 = W.decode64(words[0], dtype), W.decode64(words[1], dtype)
    tol = TOL_O[dtype]
    # scale 0: uniform weights over the visible keys
    for causal in (False, True):
        o32, lse = fa.attention(qd, kd, vd, causal=causal, scale=0.0, out_f32=(dtype != "f32"))
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        ref = (np.cumsum(v64, axis=2) if causal else np.sum(v64, axis=2, keepdims=True)) / cnt[:, None]
        assert np.max(np.abs(out_to64(o32) - ref)) <= tol
        assert np.max(np.abs(lse.cpu().numpy() - np.log(cnt))) <= TOL_LSE
    # causal row 0 sees only key 0: O_0 = V_0 exactly, LSE_0 = scale q0.k0
    s = W.scale_for(d)
    o, lse = fa.attention(qd, kd, vd, causal=True, scale=s)
    if dtype == "f32":
        # P_00 = 2^(s c - round(s c)) is 1 only to within an fp32 rounding
        assert torch.allclose(o[:, :, 0], vd[:, :, 0], rtol=4e-7, atol=0)
    else:
        # P_00 rounds to exactly 1 in 16 bits, so O_0 is V_0 bit for bit
        assert torch.equal(o[:, :, 0].float(), vd[:, :, 0].float())
    ref = s * np.einsum("bhd,bhd->bh", q64[:, :, 0], k64[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0].cpu().numpy() - ref)) <= TOL_LSE
    # identical key rows: uniform attention whatever the queries
    kk = kd[:, :, :1].expand(-1, -1, N, -1).contiguous()
    o32, lse = fa.attention(qd, kk, vd, causal=False, scale=s, out_f32=(dtype != "f32"))
    assert np.max(np.abs(out_to64(o32) - v64.mean(axis=2, keepdims=True))) <= tol
    dots = s * np.einsum("bhnd,bhd->bhn", q64, k64[:, :, 0])
    assert np.max(np.abs(lse.cpu().numpy() - (dots + math.log(N)))) <= TOL_LSE


def test_deterministic_and_entry_points_agree():
    """Repeated launches are bitwise identical (no LDS race shows up as
    run-to-run noise); the per-type entry points, the generic one and the
    extended one give the same bits."""
    words = W.make_words((4, 8, 1000, 64), "bf16", "normal", seed=3)
    qd, kd, vd = (to_dev(w, "bf16") for w in words)
    s = W.scale_for(64)
    o1, l1 = fa.attention(qd, kd, vd, causal=True, scale=s)
    for _ in range(2):
        o2, l2 = fa.attention(qd, kd, vd, causal=True, scale=s)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    # d = 128 under both masks (the two workgroup shapes), ragged N
    words = W.make_words((2, 8, 1500, 128), "bf16", "normal", seed=5)
    qd, kd, vd = (to_dev(w, "bf16") for w in words)
    for causal in (False, True):
        o1, l1 = fa.attention(qd, kd, vd, causal=causal, scale=W.scale_for(128))
        for _ in range(3):
            o2, l2 = fa.attention(qd, kd, vd, causal=causal, scale=W.scale_for(128))
            torch.cuda.synchronize()
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2), causal
    stream = torch.cuda.current_stream().cuda_stream
    for dtype, fn in (("bf16", fa.fa_fwd_bf16), ("f16", fa.fa_fwd_f16), ("f32", fa.fa_fwd_f32)):
        w = W.make_words((1, 2, 130, 128), dtype, "normal", seed=4)
        qd, kd, vd = (to_dev(x, dtype) for x in w)
        ref_o, ref_l = fa.attention(qd, kd, vd, causal=False, scale=0.1)
        o = torch.empty_like(ref_o)
        lse = torch.empty_like(ref_l)
        args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                1, 2, 130, 128, 0.1, 0, stream)
        assert fn(*args) == fa.FA_OK
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
        o.zero_()
        assert fa.fa_fwd(*args, CODE[dtype]) == fa.FA_OK
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o)


@pytest.mark.parametrize("B,H,N,d", [(5, 8, 4100, 64), (4, 16, 4096, 128), (1, 5, 700, 128)])
def test_causal_tile_order_covers_every_tile(B, H, N, d):
    """Causal launches issue query tiles longest first, in groups of heads
    per XCD: with 256 CUs, 40 heads of 33 query tiles form groups of 4 and 1
    head per XCD, 64 heads (the C3 shape) two groups of 4, and 5 heads (not
    a multiple of 8) take the order across all heads.  Every (head, query
    tile) is computed exactly once: the bits equal one launch per head, and
    the tile counts equal the oracle's."""
    words = W.make_words((B, H, N, d), "bf16", "normal", seed=11)
    qd, kd, vd = (to_dev(w, "bf16") for w in words)
    s = W.scale_for(d)
    o, lse = fa.attention(qd, kd, vd, causal=True, scale=s)
    _, _, cnt = fa.attention(qd, kd, vd, causal=True, scale=s, counters=True)
    torch.cuda.synchronize()
    assert cnt == expected_counts(qd, kd, vd, o, lse, True, s)
    for b in range(B):
        for h in range(H):
            q1, k1, v1 = (t[b:b + 1, h:h + 1].contiguous() for t in (qd, kd, vd))
            o1, l1 = fa.attention(q1, k1, v1, causal=True, scale=s)
            torch.cuda.synchronize()
            assert torch.equal(o[b, h].view(torch.int16), o1[0, 0].view(torch.int16)), (b, h)
            assert torch.equal(lse[b, h], l1[0, 0]), (b, h)


@pytest.mark.parametrize("dtype,B,H,N,d,scale,causal", [
    ("f16", 2, 72, 520, 128, -0.3, False),     # 432 query tiles: 2 or 1 per workgroup; last tile 8 rows
    ("bf16", 1, 300, 1000, 128, None, False),  # 1200 query tiles, 16 key tiles each
    ("bf16", 1, 300, 200, 128, None, False),   # 4 key tiles (every iteration a transition), 1 query tile per head
    ("bf16", 2, 130, 330, 128, 0.2, False),    # 6 key tiles (one plain iteration per tile), 2 query tiles per head
    # d = 64: the per-tile kernel, three 128-row workgroups per CU, many rounds of them
    ("bf16", 4, 80, 300, 64, None, False),     # 960 query tiles; ragged rows and keys
    ("f16", 3, 100, 330, 64, 0.2, False),      # 900 query tiles; positive non-default scale
    ("bf16", 2, 300, 1000, 64, None, True),    # causal: 8 query tiles per head (1 .. 16 key tiles)
    ("f16", 1, 600, 512, 64, -0.4, True),      # causal: 4 query tiles per head, negative scale
    ("bf16", 4, 50, 700, 64, None, True),      # causal: 6 query tiles, ragged last tile (rows and keys)
    # causal at d = 128: 256-row query tiles in pairs (the diagonal over the last 4 key tiles)
    ("bf16", 4, 32, 2000, 128, None, True),    # 8 tiles per head, ragged last tile (208 rows), 512 pairs
    ("f16", 2, 160, 1024, 128, -0.3, True),    # 4 tiles per head (4 .. 16 key tiles), negative scale
    ("bf16", 1, 260, 512, 128, None, True),    # one pair per head: tiles of 4 and 8 key tiles
])
def test_persistent_kernel(dtype, B, H, N, d, scale, causal):
    """Launches with more query tiles than the device has workgroup slots:
    at d = 128 the persistent kernel (without a mask; causal with an even
    number of 256-row query tiles), which pipelines across query tiles; at
    d = 64 many rounds of the per-tile kernel.  Every head matches the oracle,
    the instrumented instance gives the same bits and the tile counts (the
    counters launch in launch_all), and launches repeat bit for bit."""
    words = W.make_words((B, H, N, d), dtype, "normal", seed=21)
    s = W.scale_for(d) if scale is None else scale
    _, (qd, kd, vd, o, lse, _) = check_against_oracle(words, dtype, causal, s, what="persistent")
    for _ in range(2):
        o2, l2 = fa.attention(qd, kd, vd, causal=causal, scale=s)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


@pytest.mark.parametrize("shape,causal", [((2, 160, 1000, 128), False),  # persistent kernel
                                          ((2, 128, 1024, 128), True),   # causal persistent kernel (pairs)
                                          ((2, 300, 1000, 64), True),    # per-tile kernel, three per CU
                                          ((1, 8, 2048, 128), True)])    # per-tile kernel
def test_graph_replay(shape, causal):
    """A launch captured into a HIP graph replays to the bits of the eager
    launch, three times, with eager launches and fills in between."""
    words = W.make_words(shape, "bf16", "normal", seed=31)
    qd, kd, vd = (to_dev(w, "bf16") for w in words)
    s = W.scale_for(shape[3])
    o_ref, l_ref = fa.attention(qd, kd, vd, causal=causal, scale=s)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.attention(qd, kd, vd, causal=causal, scale=s, o=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.attention(qd, kd, vd, causal=causal, scale=s, o=o, lse=lse)
    for r in range(3):
        o.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref), r
        fa.attention(qd, kd, vd, causal=causal, scale=s)
        torch.cuda.synchronize()


SWEEP_TILES = [(64, 32), (64, 64), (64, 128), (128, 32), (128, 64), (128, 128), (256, 32), (256, 128)]


@pytest.mark.parametrize("tile", SWEEP_TILES)
def test_tile_sweep_shapes(tile):
    """Every tile-size sweep shape (bf16, d = 128, no mask) matches the oracle
    over several query and key tiles with ragged N, counts its tiles as the
    oracle's block counts at that shape, and its counting kernel computes the
    same bits as its plain one."""
    B, H, N, d = 1, 3, 300, 128
    words = W.make_words((B, H, N, d), "bf16", "normal", seed=41)
    qd, kd, vd = (to_dev(w, "bf16") for w in words)
    s = W.scale_for(d)
    o, lse = fa.attention(qd, kd, vd, scale=s, tile=tile)
    oc, lsec, cnt = fa.attention(qd, kd, vd, scale=s, tile=tile, counters=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), oc.view(torch.int16)) and torch.equal(lse, lsec)
    c = oracle.block_counts(N, tile[0], tile[1], False)
    assert cnt == {k_: v_ * B * H for k_, v_ in c.items()}, cnt
    o_np, lse_np = out_to64(o), lse.cpu().numpy().astype(np.float64)
    for h in range(H):
        vals = [W.decode64(w[0, h], "bf16")[None, None] for w in words]
        o_ref, lse_ref = oracle.attention_ref(*vals, s, False)
        errs = gate_errors(None, o_np[0, h][None, None], lse_np[0, h][None, None], o_ref, lse_ref, "bf16")
        assert_gates(errs, "bf16", f"tile {tile} head {h}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [200, 257])
def test_standard_baseline(dtype, d, causal, N):
    """The standard forward (S and P materialised in HBM, fa_standard_fwd):
    O passes the same gate against the oracle, and LSE the bound that S's
    16-bit rounding allows; S is scale Q K^T and each row of P the softmax
    of the stored S, within their 16-bit rounding; P is 0 above the diagonal
    under the causal mask."""
    B, H = 1, 2
    words = W.make_words((B, H, N, d), dtype, "normal", seed=51)
    qd, kd, vd = (to_dev(w, dtype) for w in words)
    sc = W.scale_for(d)
    o, lse, s_dev, p_dev = fa.standard_attention(qd, kd, vd, causal=causal, scale=sc)
    torch.cuda.synchronize()
    o_np, lse_np = out_to64(o), lse.cpu().numpy().astype(np.float64)
    s_np, p_np = out_to64(s_dev), out_to64(p_dev)
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    vis = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    for h in range(H):
        vals = [W.decode64(w[0, h], dtype) for w in words]
        o_ref, lse_ref = oracle.attention_ref(*(x[None, None] for x in vals), sc, causal)
        errs = gate_errors(None, o_np[0, h][None, None], lse_np[0, h][None, None], o_ref, lse_ref, dtype)
        assert errs["g2"] <= TOL_O[dtype], errs
        s_ref = float(np.float32(sc)) * (vals[0] @ vals[1].T)
        # LSE from the 16-bit S: d LSE / d S_j = P_j, so the error is at most
        # the largest rounding error of the row's visible S: half an ulp,
        # at most |S| 2^-(m+1) with m mantissa bits (bf16 7, fp16 10)
        bound = rel * np.abs(np.where(vis, s_ref, 0.0)).max(axis=1) + 1e-5
        assert np.all(np.abs(lse_np[0, h] - lse_ref.reshape(-1)) <= bound), "LSE"
        assert np.all(np.abs(s_np[0, h] - s_ref) <= rel * np.abs(s_ref) + 1e-3), "S"
        x = np.where(vis, s_np[0, h], -np.inf)
        p_ref = np.exp(x - x.max(axis=1, keepdims=True))
        p_ref /= p_ref.sum(axis=1, keepdims=True)
        assert np.all(np.abs(p_np[0, h] - p_ref) <= rel * p_ref + 1e-6), "P"
        assert np.all(p_np[0, h][~vis] == 0.0)


def test_guard_bands_untouched():
    """Ragged N: nothing is written outside o and lse."""
    B, H, N, d = 3, 5, 1000, 64
    words = W.make_words((B, H, N, d), "bf16", "normal", seed=9)
    qd, kd, vd = (to_dev(w, "bf16") for w in words)
    pad = 4096
    n_o, n_l = B * H * N * d, B * H * N
    obuf = torch.full((n_o + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((n_l + 2 * pad,), -3.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + n_o].view(B, H, N, d)
    lse = lbuf[pad:pad + n_l].view(B, H, N)
    for causal in (False, True):
        fa.attention(qd, kd, vd, causal=causal, o=o, lse=lse)
        torch.cuda.synchronize()
        assert bool((obuf[:pad] == 7.0).all()) and bool((obuf[pad + n_o:] == 7.0).all())
        assert bool((lbuf[:pad] == -3.0).all()) and bool((lbuf[pad + n_l:] == -3.0).all())
        assert bool(torch.isfinite(o.float()).all())


def test_maximum_size():
    """The largest head the library accepts at d = 128 (N d 4 < 2^31:
    N = 4194303, 1 GiB per tensor, a ragged last tile), causal bf16: sampled
    rows -- the first, the last, both sides of tile boundaries, random ones --
    against the oracle over all N keys."""
    import time
    N, d = (1 << 22) - 1, 128
    t0 = time.time()
    print(f"maximum size: B=1 H=1 N={N} d={d} bf16 causal", flush=True)
    words = W.make_words((1, 1, N, d), "bf16", "normal", seed=41)
    print(f"  inputs drawn ({time.time() - t0:.0f} s)", flush=True)
    qd, kd, vd = (to_dev(w, "bf16") for w in words)
    scale = W.scale_for(d)
    o, lse = fa.attention(qd, kd, vd, causal=True, scale=scale)
    torch.cuda.synchronize()
    print(f"  forward done ({time.time() - t0:.0f} s)", flush=True)
    # one more row would exceed the per-head limit
    bigger = fa.fa_fwd_bf16(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 1, N + 1,
                            d, scale, 1, torch.cuda.current_stream().cuda_stream)
    assert bigger == fa.FA_ERR_UNSUPPORTED
    rng = np.random.default_rng(9)
    rows = sample_rows(N, 128, rng, n_random=8, cap=24)
    vals = [W.decode64(w[0, 0], "bf16")[None, None] for w in words]
    o_ref, lse_ref = oracle.attention_ref(vals[0], vals[1], vals[2], scale, True, rows=rows)
    print(f"  oracle rows done ({time.time() - t0:.0f} s)", flush=True)
    o_np = out_to64(o[0, 0, rows])[None, None]
    lse_np = lse[0, 0, rows].cpu().numpy().astype(np.float64)[None, None]
    errs = gate_errors(None, o_np, lse_np, o_ref, lse_ref, "bf16")
    print(f"  {errs}", flush=True)
    assert_gates(errs, "bf16", "maximum size")
    assert bool(torch.isfinite(lse).all())
