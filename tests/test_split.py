"""GPU parity of the split-KV forward (include/fa_fwd.h ``fa_fwd_split``)
against the float64 oracle.

Each key range's partial output and log-sum-exp are themselves exact
attention over that range's keys, so they are checked against
``oracle.attention_ref`` on the range (the fp32 partials within the fp32
gate G1); the merged 16-bit output and LSE are checked against the oracle
over all keys with the gates of the plain forward (G2, LSE 1e-3).  With one
range the merge multiplies by exp(0) = 1 and the result must equal the
plain forward's bits.
"""

import numpy as np
import pytest
import torch

import fa_workloads as W
import oracle
import tiled_exact_attention_fwd_amd as fa
from parity_util import TOL_O, TOL_LSE, gate_errors, assert_gates, out_to64, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def run(shape, dtype, splits, values="normal", seed=11, scale=None, causal=False):
    words = W.make_words(shape, dtype, values, seed)
    qd, kd, vd = (to_dev(w, dtype) for w in words)
    d = shape[3]
    scale = W.scale_for(d) if scale is None else scale
    o, lse, op, lp = fa.attention_split(qd, kd, vd, splits, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return words, (qd, kd, vd), (o, lse, op, lp), scale


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,splits", [(1, 3), (200, 2), (1000, 3), (1000, 7), (4100, 5)])
def test_split_matches_oracle(dtype, d, causal, N, splits):
    print(f"split {dtype} d={d} causal={causal} N={N} splits={splits}", flush=True)
    shape = (1, 2, N, d)
    words, _, (o, lse, op, lp), scale = run(shape, dtype, splits, causal=causal)
    rng = np.random.default_rng(N)
    rows = None if N <= 1000 else sample_rows(N, 64, rng)
    o_np, lse_np = out_to64(o), lse.cpu().numpy().astype(np.float64)
    op_np, lp_np = out_to64(op), lp.cpu().numpy().astype(np.float64)
    ranges = fa.split_ranges(N, splits)
    for h in range(2):
        vals = [W.decode64(w[0, h], dtype)[None, None] for w in words]
        sel = slice(None) if rows is None else rows
        o_ref, lse_ref = oracle.attention_ref(*vals, scale, causal, rows=rows)
        errs = gate_errors(None, o_np[0, h, sel][None, None], lse_np[0, h, sel][None, None], o_ref, lse_ref, dtype)
        assert_gates(errs, dtype, f"merged N={N} splits={splits} causal={causal} head {h}")
        if causal:
            # a range that starts after a row holds none of its keys: O = 0, LSE = -inf
            qrows = np.arange(N) if rows is None else rows
            for s, (k0, k1) in enumerate(ranges):
                blind = qrows[qrows < k0]
                assert np.all(np.isneginf(lp_np[s, 0, h, blind])) and np.all(op_np[s, 0, h, blind] == 0)
            continue
        # every range's partial is attention over that range's keys
        for s, (k0, k1) in enumerate(ranges):
            pr, plse = oracle.attention_ref(vals[0], vals[1][:, :, k0:k1], vals[2][:, :, k0:k1], scale, False, rows=rows)
            e1 = float(np.max(np.abs(op_np[s, 0, h, sel] - pr[0, 0])))
            el = float(np.max(np.abs(lp_np[s, 0, h, sel] - plse[0, 0])))
            assert e1 <= TOL_O[dtype] and el <= TOL_LSE, (s, k0, k1, e1, el)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_one_range_equals_plain_forward(dtype, d, causal):
    shape = (2, 3, 777, d)
    words, (qd, kd, vd), (o, lse, _, _), scale = run(shape, dtype, 1, causal=causal)
    o_ref, lse_ref = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    bits = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(o.view(bits), o_ref.view(bits))
    assert torch.equal(lse, lse_ref)


def test_long_few_heads_and_peaked():
    """One long sequence of two heads (the shape split-KV is for), spiky keys
    so that the ranges' maxima differ widely, a negative scale, and the
    causal mask."""
    shape = (1, 2, 32768, 128)
    for values, scale, causal in (("spiky", None, False), ("normal", -0.1, False), ("half", None, True)):
        print(f"split long {values} scale={scale} causal={causal}", flush=True)
        words, _, (o, lse, _, _), sc = run(shape, "bf16", 8, values=values, scale=scale, causal=causal)
        rng = np.random.default_rng(5)
        rows = sample_rows(32768, 256, rng, n_random=16)
        o_np, lse_np = out_to64(o), lse.cpu().numpy().astype(np.float64)
        for h in range(2):
            vals = [W.decode64(w[0, h], "bf16")[None, None] for w in words]
            o_ref, lse_ref = oracle.attention_ref(*vals, sc, causal, rows=rows)
            errs = gate_errors(None, o_np[0, h, rows][None, None], lse_np[0, h, rows][None, None], o_ref, lse_ref,
                               "bf16")
            assert_gates(errs, "bf16", f"long {values} head {h}")


def test_split_count_rule():
    """fa_fwd_split_count: ranges that bring the plain launch's (head, query
    tile) units up to one per CU without the mask, to two per CU under it;
    1 where the plain launch already fills the device."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    bf = fa.FA_DTYPE_BF16
    for (B, H, N, d, causal) in [(1, 1, 8192, 128, 0), (1, 1, 16384, 128, 0), (1, 2, 16384, 128, 0),
                                 (2, 8, 4096, 128, 0), (1, 1, 32768, 128, 1), (1, 1, 16384, 128, 1),
                                 (1, 2, 32768, 128, 1), (1, 32, 32768, 128, 1), (1, 1, 100, 64, 0), (16, 32, 1000, 64, 1)]:
        st, tq, _ = fa.fa_fwd_tile_shape(bf, d, causal)
        units = B * H * -(-N // tq)
        want = max(1, min((2 * cus if causal else cus) // units, -(-N // 64), 16))
        assert fa.fa_fwd_split_count(B, H, N, d, causal, bf) == (fa.FA_OK, want), (B, H, N, d, causal)
    if cus == 256:    # the counts the measurements behind the rule chose on MI355X
        assert fa.fa_fwd_split_count(1, 1, 8192, 128, 0, bf)[1] == 8
        assert fa.fa_fwd_split_count(1, 2, 16384, 128, 0, bf)[1] == 2
        assert fa.fa_fwd_split_count(1, 1, 32768, 128, 1, bf)[1] == 2
        assert fa.fa_fwd_split_count(1, 32, 32768, 128, 1, bf)[1] == 1
    # and attention_split without a count uses it
    words = W.make_words((1, 1, 8192, 128), "bf16", "normal", 5)
    qd, kd, vd = (to_dev(w, "bf16") for w in words)
    o, lse, op, lp = fa.attention_split(qd, kd, vd, causal=False)
    o1, lse1 = fa.attention(qd, kd, vd, causal=False)
    torch.cuda.synchronize()
    assert op.shape[0] == fa.fa_fwd_split_count(1, 1, 8192, 128, 0, bf)[1]
    assert float((o.float() - o1.float()).abs().max()) <= 2 ** -6
    assert float((lse - lse1).abs().max()) <= 1e-5


def test_graph_replay():
    """The split-KV call (partial and merge kernels) captured into a HIP graph
    replays to the bits of the eager call."""
    shape = (1, 2, 3000, 128)
    words, (qd, kd, vd), (o_ref, l_ref, _, _), scale = run(shape, "bf16", 4)
    B, H, N, d = shape
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    op = torch.empty((4, B, H, N, d), dtype=torch.float32, device=qd.device)
    lp = torch.empty((4, B, H, N), dtype=torch.float32, device=qd.device)

    def call(handle):
        st = fa.fa_fwd_split(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), op.data_ptr(),
                             lp.data_ptr(), B, H, N, d, scale, 0, 4, handle, fa.FA_DTYPE_BF16)
        assert st == fa.FA_OK

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream().cuda_stream)
    for r in range(3):
        o.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref), r
        run(shape, "bf16", 2)
