"""fa_bwd_noalloc (include/fa_bwd.h), the backward for callers that cannot
allocate: called through the C ABI, it must return what fa_bwd returns for
the same inputs -- the same kernels run, only the D work array lives in the
library's fixed scratch array -- on two calls in a row, the second with a
smaller problem (the scratch keeps the first call's contents).  Both results
are also held to the gradient gate against the float64 oracle."""

import numpy as np
import pytest
import torch

import fa_workloads as W
import oracle
import tiled_exact_attention_fwd_amd as fa
from parity_util import half_ulp, out_to64, to_dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f16": 2e-3, "f32": 2e-3}


def run_both(shape, dtype, causal, seed):
    words = W.make_words(shape, dtype, "normal", seed)
    dwords = W.encode(W.draw_dout(shape, seed), dtype)
    q, k, v = (to_dev(w, dtype) for w in words)
    do = to_dev(dwords, dtype)
    scale = W.scale_for(shape[3])
    o, lse = fa.attention(q, k, v, causal=causal, scale=scale)
    dq, dk, dv, _ = fa.attention_backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    nq, nk, nv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, H, N, d = shape
    stream = torch.cuda.current_stream().cuda_stream
    st = fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                           nq.data_ptr(), nk.data_ptr(), nv.data_ptr(), B, H, N, d, scale, int(causal), stream,
                           fa.dtype_code(q.dtype))
    assert st == fa.FA_OK, fa.fa_strerror(st)
    torch.cuda.synchronize()
    return words, dwords, scale, (dq, dk, dv), (nq, nk, nv)


def check_against_oracle(words, dwords, dtype, causal, scale, grads):
    B, H = words[0].shape[:2]
    vals = [np.stack([W.decode64(w[b, h], dtype) for b in range(B) for h in range(H)])[:, None]
            for w in (*words, dwords)]
    ref = oracle.attention_bwd_ref(*vals, scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        g64 = out_to64(g).reshape(r.shape)
        ex = float(np.max(np.abs(g64 - r) - half_ulp(r, dtype))) / (float(np.max(np.abs(r))) or 1.0)
        assert ex <= TOL[dtype], (name, ex)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_fa_bwd_on_two_calls(dtype, causal):
    # a larger problem first, then a smaller one over the same scratch
    for shape, seed in (((2, 3, 300, 64), 11), ((1, 2, 97, 128), 12)):
        print(f"noalloc backward {dtype} causal={causal} shape={shape}", flush=True)
        words, dwords, scale, ref, got = run_both(shape, dtype, causal, seed)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a.view(torch.int16) if dtype != "f32" else a.view(torch.int32),
                               b.view(torch.int16) if dtype != "f32" else b.view(torch.int32)), name
        check_against_oracle(words, dwords, dtype, causal, scale, got)


def test_noalloc_refuses_oversize_before_launch():
    q = torch.empty((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    rows = fa.BWD_NOALLOC_MAX_ROWS
    big = [1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40, 6 << 40, 7 << 40, 8 << 40, 9 << 40]
    st = fa.fa_bwd_noalloc(*big, 1, 1, rows + 1, 64, 0.125, 0, torch.cuda.current_stream().cuda_stream,
                           fa.FA_DTYPE_BF16)
    assert st == fa.FA_ERR_SCRATCH
    del q
