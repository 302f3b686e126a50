"""GPU parity of the HIP backward pass (include/fa_bwd.h) against the float64
backward oracle (oracle.backward).

The device path is the composite the backward is built for: the HIP forward
writes O and LSE, the HIP backward rebuilds P from that LSE
("Flash Attention 原理", two pillars: recomputation) and returns dQ, dK, dV.
The oracle computes the exact gradients from Q, K, V and dO alone; nothing it
uses comes from the device.

Gate.  No tolerance is stated for gradients, and gradients have no fixed
scale, so the forward's output tolerances (1e-2 for bf16, 2e-3 for fp16 and
fp32, applied there to outputs of order one) are applied relative to the
largest reference entry of each gradient:
max(|g - g_ref| - half_ulp(g_ref)) <= tol * max|g_ref|, the half ulp being
the rounding of the 16-bit output itself.  A CPU emulation of the kernels'
arithmetic (P and dS rounded to the input type before their products, fp32
sums, O rounded to 16 bits) gives at most 6.1e-3 (bf16) and 9.0e-4 (fp16) on
the shapes below.
"""

import numpy as np
import pytest
import torch

import fa_workloads as W
import oracle
import tiled_exact_attention_fwd_amd as fa
from parity_util import half_ulp, out_to64, sample_rows, to_dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f16": 2e-3, "f32": 2e-3}


def inputs(shape, dtype, values, seed):
    words = W.make_words(shape, dtype, values, seed)
    dwords = W.encode(W.draw_dout(shape, seed), dtype)
    return words, dwords


def run_device(words, dwords, dtype, causal, scale):
    qd, kd, vd = (to_dev(w, dtype) for w in words)
    dod = to_dev(dwords, dtype)
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv, delta = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (qd, kd, vd, dod, o, lse), (dq, dk, dv, delta)


def grad_errors(dev, ref, dtype):
    out = {}
    for name, g, r in zip(("dq", "dk", "dv"), dev, ref):
        scale = float(np.max(np.abs(r))) or 1.0
        ex = float(np.max(np.abs(g - r) - half_ulp(r, dtype))) if r.size else 0.0
        out[name] = ex / scale
    return out


def check(words, dwords, dtype, causal, scale, heads=None, what=""):
    B, H, N, d = words[0].shape
    _, (dq, dk, dv, delta) = run_device(words, dwords, dtype, causal, scale)
    g = [out_to64(t) for t in (dq, dk, dv)]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    vals = [np.stack([W.decode64(w[b, h], dtype) for b, h in heads])[:, None] for w in (*words, dwords)]
    ref = oracle.attention_bwd_ref(*vals, scale, causal)
    dev = [np.stack([t[b, h] for b, h in heads])[:, None] for t in g]
    errs = grad_errors(dev, ref, dtype)
    for name, e in errs.items():
        assert e <= TOL[dtype], f"{what} {dtype} causal={causal} N={N} d={d}: {errs}"
    for t in g:
        assert np.all(np.isfinite(t))
    return errs, (dq, dk, dv, delta)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 200, 257])
def test_small(dtype, d, causal, N):
    print(f"backward small {dtype} d={d} causal={causal} N={N}", flush=True)
    words, dwords = inputs((1, 2, N, d), dtype, "normal", 3)
    errs, _ = check(words, dwords, dtype, causal, W.scale_for(d), what="small")
    print(errs)
    if dtype == "f32":
        # fp32 products throughout (no 16-bit P or dS): far inside the gate
        assert max(errs.values()) <= 1e-4, errs


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        if rng.random() < 0.5:
            N = int(rng.integers(1, 20)) * int(rng.choice([64, 128, 256])) + int(rng.choice([-1, 0, 1]))
        else:
            N = int(rng.integers(1, 2500))
        out.append((int(rng.integers(1, 3)), int(rng.integers(1, 5)), max(N, 1), int(rng.choice([64, 128])),
                    str(rng.choice(["bf16", "f16"])), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,H,N,d,dtype,causal", _random_shapes(2025, 10))
def test_random_shapes(B, H, N, d, dtype, causal):
    """Seeded random shapes (N near the 64-, 128- and 256-row block
    boundaries or anywhere up to 2500) against the gradient oracle."""
    print(f"backward random shape {B}x{H}x{N}x{d} {dtype} causal={causal}", flush=True)
    words, dwords = inputs((B, H, N, d), dtype, "normal", N)
    errs, _ = check(words, dwords, dtype, causal, W.scale_for(d), what="random")
    print(errs)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_spiky_causal(dtype):
    print(f"backward spiky {dtype}", flush=True)
    words, dwords = inputs((2, 2, 640, 128), dtype, "spiky", 5)
    errs, _ = check(words, dwords, dtype, True, W.scale_for(128), what="spiky")
    print(errs)


@pytest.mark.parametrize("name,causal", [("C2b", False), ("C3", True), ("C4", True), ("C4", False)])
def test_workload_shapes(name, causal):
    """The forward workloads' full shapes; the oracle checks a few whole
    heads, and every head must satisfy sum_k dK[k] = 0 (softmax ignores a
    shift shared by all keys)."""
    wl = W.WORKLOADS[name]
    print(f"backward workload {name} causal={causal} shape={wl.shape}", flush=True)
    words, dwords = inputs(wl.shape, wl.dtype, wl.values, W.default_seed())
    B, H, N, d = wl.shape
    allh = [(b, h) for b in range(B) for h in range(H)]
    heads = [allh[0], allh[len(allh) // 2], allh[-1]]
    errs, (dq, dk, dv, delta) = check(words, dwords, wl.dtype, causal, W.scale_for(d), heads=heads, what=name)
    print(name, causal, errs)
    colsum = dk.float().sum(dim=2).abs().max().item()
    dkmax = dk.float().abs().max().item()
    # the sum of N rounded terms: each carries the gate's relative error at most
    assert colsum <= TOL[wl.dtype] * dkmax * N ** 0.5, (colsum, dkmax)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_closed_forms_and_determinism(dtype):
    # N = 1: O = V whatever the scores, so dQ = dK = 0 and dV = dO.  On the
    # device P = exp(s - LSE) is 1 within fp32 rounding and rounds to exactly 1
    # for the dV product; dS = P (dP - D) is the difference of two fp32 dot
    # products of the same 64 terms summed in different orders, so dQ and dK
    # are zero up to that rounding.
    words, dwords = inputs((2, 3, 1, 64), dtype, "normal", 7)
    (qd, kd, vd, dod, _, _), (dq, dk, dv, _) = run_device(words, dwords, dtype, False, W.scale_for(64))
    bound = 64 * 2.0 ** -22 * float((dod.float().abs() * vd.float().abs()).sum(dim=3).max())
    bound *= float(max(qd.float().abs().max(), kd.float().abs().max()))
    assert float(dq.float().abs().max()) <= bound and float(dk.float().abs().max()) <= bound
    assert torch.equal(dv.view(torch.int16), dod.view(torch.int16))
    # repeated launches give the same bits
    words, dwords = inputs((2, 2, 300, 128), dtype, "normal", 8)
    for causal in (False, True):
        _, a = run_device(words, dwords, dtype, causal, W.scale_for(128))
        _, b = run_device(words, dwords, dtype, causal, W.scale_for(128))
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16),
                               y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16))


def test_entry_points_agree():
    words, dwords = inputs((1, 2, 130, 64), "bf16", "normal", 9)
    (qd, kd, vd, dod, o, lse), (dq, dk, dv, delta) = run_device(words, dwords, "bf16", True, 0.125)
    outs = [torch.empty_like(t) for t in (dq, dk, dv, delta)]
    st = fa.fa_bwd_bf16(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), dod.data_ptr(),
                        *[t.data_ptr() for t in outs], 1, 2, 130, 64, 0.125, 1,
                        torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    for x, y in zip(outs, (dq, dk, dv, delta)):
        assert torch.equal(x, y)
    # the work array holds rowsum(dO * O) of the forward's stored O
    ref = (dod.float() * o.float()).sum(dim=3)
    assert torch.allclose(delta, ref, atol=1e-4, rtol=1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_o32_equals_o16_bits(dtype, d, causal):
    """fa_bwd_o32 handed the 16-bit O widened to fp32 takes the same D, so
    it returns fa_bwd's bits."""
    print(f"backward o32 bits {dtype} d={d} causal={causal}", flush=True)
    words, dwords = inputs((2, 3, 700, d), dtype, "normal", 21)
    (qd, kd, vd, dod, o, lse), a = run_device(words, dwords, dtype, causal, W.scale_for(d))
    b = fa.attention_backward(qd, kd, vd, o.float(), lse, dod, causal=causal, scale=W.scale_for(d))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16),
                           y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_o32_accuracy(dtype):
    """D from the forward's fp32 O (fa_bwd_o32): within the gate on spiky
    causal heads, and no less accurate than D from the 16-bit O; D itself
    within fp32 rounding of the oracle's D from the exact O."""
    print(f"backward o32 accuracy {dtype}", flush=True)
    words, dwords = inputs((1, 4, 1536, 128), dtype, "spiky", 23)
    scale = W.scale_for(128)
    qd, kd, vd = (to_dev(w, dtype) for w in words)
    dod = to_dev(dwords, dtype)
    o16, lse = fa.attention(qd, kd, vd, causal=True, scale=scale)
    o32, lse32 = fa.attention(qd, kd, vd, causal=True, scale=scale, out_f32=True)
    r16 = fa.attention_backward(qd, kd, vd, o16, lse, dod, causal=True, scale=scale)
    r32 = fa.attention_backward(qd, kd, vd, o32, lse32, dod, causal=True, scale=scale)
    torch.cuda.synchronize()
    B, H, N, d = words[0].shape
    vals = [np.stack([W.decode64(w[0, h], dtype) for h in range(H)])[:, None] for w in (*words, dwords)]
    ref = oracle.attention_bwd_ref(*vals, scale, True)
    e = {}
    for tag, r in (("o16", r16), ("o32", r32)):
        dev = [out_to64(t)[0][:, None] for t in r[:3]]
        e[tag] = grad_errors(dev, ref, dtype)
    print(e)
    assert max(e["o32"].values()) <= TOL[dtype], e
    for name in ("dq", "dk", "dv"):
        assert e["o32"][name] <= e["o16"][name] * 1.05 + 1e-4, e
    # D = rowsum(dO * O) against the exact O (float64, the oracle's forward):
    # the fp32 O carries only the forward's rounding of each weight P to 16
    # bits (relative 2^-8 at most for bf16, so |dO_c| * 2^-8 * max_j |V_jc|
    # per column), not the 16-bit rounding of O itself
    o_ref, _ = oracle.attention_ref(vals[0], vals[1], vals[2], scale, True)
    d_ref = (vals[3] * o_ref).sum(axis=-1)[:, 0]
    d_dev = r32[3][0].double().cpu().numpy()
    vmax = np.abs(vals[2]).max(axis=2, keepdims=True)
    bound = 2.0 ** -8 * (np.abs(vals[3]) * vmax).sum(axis=-1)[:, 0] + 1e-30
    assert np.all(np.abs(d_dev - d_ref) <= bound), float(np.max(np.abs(d_dev - d_ref) / bound))


@pytest.mark.parametrize("causal", [False, True])
def test_graph_replay(causal):
    """The backward's two launches captured into a HIP graph replay to the
    bits of the eager call, three times, with eager work and fills between."""
    words, dwords = inputs((2, 4, 700, 128), "bf16", "normal", 12)
    (qd, kd, vd, dod, o, lse), ref = run_device(words, dwords, "bf16", causal, W.scale_for(128))
    outs = [torch.empty_like(t) for t in ref]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    B, H, N, d = qd.shape

    def call(handle):
        st = fa.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), dod.data_ptr(),
                       *[t.data_ptr() for t in outs], B, H, N, d, W.scale_for(128), int(causal), handle,
                       fa.FA_DTYPE_BF16)
        assert st == fa.FA_OK

    with torch.cuda.stream(stream):
        call(stream.cuda_stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream().cuda_stream)
    for r in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(outs, ref):
            assert torch.equal(x, y), r
        run_device(words, dwords, "bf16", causal, W.scale_for(128))


@pytest.mark.parametrize("B,H,N,d", [(4, 16, 4096, 128), (3, 8, 1000, 64), (1, 24, 2100, 128), (1, 5, 700, 64)])
def test_causal_order_writes_every_row(B, H, N, d):
    """Outputs filled with NaN beforehand are finite everywhere afterwards:
    the causal launch order (longest blocks first across an XCD's heads when
    the head count is a multiple of 8, across all heads otherwise) visits
    every block."""
    print(f"backward causal order B={B} H={H} N={N} d={d}", flush=True)
    words, dwords = inputs((B, H, N, d), "bf16", "normal", 13)
    qd, kd, vd = (to_dev(w, "bf16") for w in words)
    dod = to_dev(dwords, "bf16")
    o, lse = fa.attention(qd, kd, vd, causal=True, scale=W.scale_for(d))
    outs = [torch.full_like(qd, float("nan")) for _ in range(3)]
    delta = torch.full_like(lse, float("nan"))
    st = fa.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), dod.data_ptr(),
                   *[t.data_ptr() for t in outs], delta.data_ptr(), B, H, N, d, W.scale_for(d), 1,
                   torch.cuda.current_stream().cuda_stream, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    for t in outs + [delta]:
        assert bool(torch.isfinite(t).all())
    # and one head against the oracle
    h = (B - 1, H - 1)
    vals = [W.decode64(w[h], "bf16")[None, None] for w in (*words, dwords)]
    ref = oracle.attention_bwd_ref(*vals, W.scale_for(d), True)
    dev = [out_to64(t)[h][None, None] for t in outs]
    errs = grad_errors(dev, ref, "bf16")
    assert max(errs.values()) <= TOL["bf16"], errs


def test_long_context_sampled_rows():
    """The 32768-row causal workload (B=1, H=32, d=128, N(0, 0.5^2) inputs):
    dQ at every row and dK, dV at sampled key rows of one head against the
    row-chunked oracle, and sum_k dK = 0 on every head.  dQ is checked on
    every row so that the gate's scale is the gradient's largest entry: the
    largest dQ rows and the largest relative errors are both in the first
    rows, which see few keys (there D = rowsum(dO * O) from the 16-bit O
    dominates the error)."""
    wl = W.WORKLOADS["C5"]
    print(f"backward long context {wl.shape}", flush=True)
    words, dwords = inputs(wl.shape, wl.dtype, wl.values, W.default_seed())
    B, H, N, d = wl.shape
    scale = W.scale_for(d)
    (qd, kd, vd, dod, _, _), (dq, dk, dv, _) = run_device(words, dwords, wl.dtype, True, scale)
    # and the same with D from the forward's fp32 O (fa_bwd_o32)
    o32, lse32 = fa.attention(qd, kd, vd, causal=True, scale=scale, out_f32=True)
    dq32, dk32, dv32, _ = fa.attention_backward(qd, kd, vd, o32, lse32, dod, causal=True, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    qr = np.arange(N)
    kr = sample_rows(N, 256, rng, n_random=16, cap=24)
    b, h = 0, H - 1
    vals = [W.decode64(w[b, h], wl.dtype) for w in (*words, dwords)]
    ref = oracle.attention_bwd_sampled(*vals, scale, True, qr, kr, chunk=1024)
    dev = [out_to64(dq[b, h, qr]), out_to64(dk[b, h, kr]), out_to64(dv[b, h, kr])]
    errs = grad_errors(dev, ref, wl.dtype)
    dev32 = [out_to64(dq32[b, h, qr]), out_to64(dk32[b, h, kr]), out_to64(dv32[b, h, kr])]
    errs32 = grad_errors(dev32, ref, wl.dtype)
    print("long context", errs, "with the fp32 O", errs32)
    assert max(errs.values()) <= TOL[wl.dtype], errs
    assert max(errs32.values()) <= TOL[wl.dtype], errs32
    colsum = dk.float().sum(dim=2).abs().max().item()
    assert colsum <= TOL[wl.dtype] * dk.float().abs().max().item() * N ** 0.5


@pytest.mark.parametrize("causal", [False, True])
def test_zero_and_negative_scale(causal):
    """scale 0: P is uniform over the visible keys, so dQ = dK = 0 exactly
    (they carry the factor scale) and dV[k] is the mean-weighted sum of dO
    over the queries that see k (the oracle's closed form); a negative scale
    against the oracle."""
    words, dwords = inputs((1, 3, 150, 64), "bf16", "normal", 14)
    for scale in (0.0, -0.2):
        (_, _, _, _, _, _), (dq, dk, dv, _) = run_device(words, dwords, "bf16", causal, scale)
        vals = [W.decode64(w, "bf16") for w in (*words, dwords)]
        ref = oracle.attention_bwd_ref(*vals, scale, causal)
        dev = [out_to64(t) for t in (dq, dk, dv)]
        if scale == 0.0:
            assert not dq.any() and not dk.any()
            errs = grad_errors(dev[2:], ref[2:], "bf16")
        else:
            errs = grad_errors(dev, ref, "bf16")
        assert max(errs.values()) <= TOL["bf16"], (scale, errs)


def test_maximum_size():
    """The largest head the library accepts at d = 128 (N d 4 < 2^31,
    N = 4194303, ragged), causal bf16: every output finite, dQ at sampled
    rows against the oracle (each row alone), and one more row rejected."""
    import time
    N, d = (1 << 22) - 1, 128
    t0 = time.time()
    print(f"backward maximum size: B=1 H=1 N={N} d={d} bf16 causal", flush=True)
    words, dwords = inputs((1, 1, N, d), "bf16", "normal", 42)
    print(f"  inputs drawn ({time.time() - t0:.0f} s)", flush=True)
    (qd, kd, vd, dod, o, lse), (dq, dk, dv, delta) = run_device(words, dwords, "bf16", True, W.scale_for(d))
    print(f"  forward and backward done ({time.time() - t0:.0f} s)", flush=True)
    for t in (dq, dk, dv, delta):
        assert bool(torch.isfinite(t).all())
    st = fa.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), dod.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), 1, 1, N + 1, d,
                   W.scale_for(d), 1, torch.cuda.current_stream().cuda_stream, fa.FA_DTYPE_BF16)
    assert st == fa.FA_ERR_UNSUPPORTED
    rng = np.random.default_rng(10)
    # the first rows carry the largest dQ entries (the gate's scale), then
    # tile edges and random rows
    qr = np.unique(np.concatenate([np.arange(64), sample_rows(N, 256, rng, n_random=8, cap=24)]))
    vals = [W.decode64(w[0, 0], "bf16") for w in (*words, dwords)]
    ref, _, _ = oracle.attention_bwd_sampled(*vals, W.scale_for(d), True, qr, [], chunk=64)
    print(f"  oracle rows done ({time.time() - t0:.0f} s)", flush=True)
    errs = grad_errors([out_to64(dq[0, 0, qr])], [ref], "bf16")
    print(f"  {errs}", flush=True)
    assert errs["dq"] <= TOL["bf16"], errs


@pytest.mark.parametrize("causal", [False, True])
def test_f32_configuration(causal):
    """The fp32 configuration (B=1, H=1, N=256, d=64, N(0,1)) forward and
    backward against the oracle, and a ragged multi-head fp32 case."""
    for shape in ((1, 1, 256, 64), (2, 3, 300, 128)):
        words, dwords = inputs(shape, "f32", "normal", 15)
        errs, _ = check(words, dwords, "f32", causal, W.scale_for(shape[3]), what="f32")
        print("f32", shape, causal, errs)
        assert max(errs.values()) <= 1e-4, errs
