"""Pins for the float64 backward oracle (``oracle.backward``): central finite
differences of the forward definition, scalar brute force, torch autograd on
the CPU in float64, closed forms and invariants.  CPU only.

The gradients are not printed on the pages; they are fixed by the forward they
differentiate ("FlashAttention分块计算优化Transformer显存效率", §1.1 and §2.2),
and the recomputation they are built for is "Flash Attention 原理", two
pillars.  Finite differences of ``oracle.attention_ref`` pin the backward to
the forward without sharing its formulas.
"""

import numpy as np
import pytest

import oracle
from oracle import backward as obwd


def rand4(rng, B, H, N, d, n=4):
    return tuple(rng.standard_normal((B, H, N, d)) for _ in range(n))


def fd_grads(q, k, v, do, scale, causal, h=1e-6):
    """Central differences of L = sum(dO * O) with O from the forward oracle."""
    def loss(qq, kk, vv):
        o, _ = oracle.attention_ref(qq, kk, vv, scale, causal)
        return float(np.sum(do * o))
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [t.copy() for t in base]
            minus = [t.copy() for t in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("N,d,causal", [(1, 3, False), (3, 2, True), (5, 4, False), (6, 3, True)])
def test_matches_finite_differences_of_forward(N, d, causal):
    rng = np.random.default_rng(10 + N)
    q, k, v, do = rand4(rng, 1, 2, N, d)
    scale = 0.7
    ref = obwd.attention_bwd_ref(q, k, v, do, scale, causal)
    fd = fd_grads(q, k, v, do, scale, causal)
    for a, b in zip(ref, fd):
        np.testing.assert_allclose(a, b, atol=2e-8, rtol=0)


@pytest.mark.parametrize("N,d", [(1, 2), (4, 3), (7, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_scalar_brute_force(N, d, causal):
    rng = np.random.default_rng(20 + N)
    q, k, v, do = rand4(rng, 1, 2, N, d)
    scale = 0.9
    ref = obwd.attention_bwd_ref(q, k, v, do, scale, causal)
    brute = obwd.brute_bwd_ref(q, k, v, do, scale, causal)
    for a, b in zip(ref, brute):
        np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_float64(causal):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(3)
    q, k, v, do = rand4(rng, 2, 3, 37, 16)
    scale = 0.25
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    ref = obwd.attention_bwd_ref(q, k, v, do, scale, causal)
    for a, t in zip(ref, (tq, tk, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), atol=1e-12, rtol=0)


def test_closed_forms():
    rng = np.random.default_rng(4)
    # N = 1: softmax of one score is 1, so O = V: dQ = dK = 0, dV = dO
    q, k, v, do = rand4(rng, 2, 2, 1, 5)
    for causal in (False, True):
        dq, dk, dv = obwd.attention_bwd_ref(q, k, v, do, 0.3, causal)
        assert np.all(dq == 0) and np.all(dk == 0)
        np.testing.assert_allclose(dv, do, atol=0, rtol=0)
    # scale 0: uniform weights over the visible keys; dQ = dK = 0 and
    # dV[k] = sum over queries q that see k of dO[q] / (number of keys q sees)
    N = 9
    q, k, v, do = rand4(rng, 1, 1, N, 4)
    dq, dk, dv = obwd.attention_bwd_ref(q, k, v, do, 0.0, False)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[0, 0], np.repeat(do[0, 0].mean(axis=0, keepdims=True), N, 0), atol=1e-15)
    dq, dk, dv = obwd.attention_bwd_ref(q, k, v, do, 0.0, True)
    expect = np.array([sum(do[0, 0, i] / (i + 1) for i in range(j, N)) for j in range(N)])
    np.testing.assert_allclose(dv[0, 0], expect, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    """Shifting every key by one vector shifts each row's scores by a
    constant, which softmax ignores: sum_k dK[k] = 0.  The kernel's row
    identity sum_k P dP = sum_c dO O also holds on the definition."""
    rng = np.random.default_rng(5)
    q, k, v, do = rand4(rng, 2, 2, 23, 8)
    scale = 0.5
    dq, dk, dv = obwd.attention_bwd_ref(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # sum_q dV[q] = sum_q dO[q] (each row of P sums to one)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    o, _ = oracle.attention_ref(q, k, v, scale, causal)
    p = oracle.attention_probs(q, k, scale, causal)
    dp = do @ np.swapaxes(v, 2, 3)
    np.testing.assert_allclose(np.sum(p * dp, axis=3), np.sum(do * o, axis=3), atol=1e-12)


def test_selected_heads_equal_full():
    rng = np.random.default_rng(6)
    q, k, v, do = rand4(rng, 2, 3, 11, 4)
    full = obwd.attention_bwd_ref(q, k, v, do, 0.4, True)
    part = obwd.attention_bwd_ref(q, k, v, do, 0.4, True, heads=[(1, 2), (0, 1)])
    for f, p in zip(full, part):
        np.testing.assert_array_equal(p[0], f[1, 2])
        np.testing.assert_array_equal(p[1], f[0, 1])


def _variants():
    """Plausible slips in the gradient formulas, each a full replacement of the
    per-head function."""
    from oracle.attention import _scores, _softmax_rows, _visible

    def base(qh, kh, vh, doh, scale, causal):
        n = qh.shape[0]
        s = np.where(_visible(np.arange(n), kh.shape[0], causal), _scores(qh, kh, scale), -np.inf)
        p, _ = _softmax_rows(s)
        return p, doh @ vh.T

    def no_centering(qh, kh, vh, doh, scale, causal):
        p, dp = base(qh, kh, vh, doh, scale, causal)
        ds = p * dp
        return scale * ds @ kh, scale * ds.T @ qh, p.T @ doh

    def column_centering(qh, kh, vh, doh, scale, causal):
        p, dp = base(qh, kh, vh, doh, scale, causal)
        ds = p * (dp - np.sum(p * dp, axis=0, keepdims=True))
        return scale * ds @ kh, scale * ds.T @ qh, p.T @ doh

    def missing_scale(qh, kh, vh, doh, scale, causal):
        p, dp = base(qh, kh, vh, doh, scale, causal)
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        return ds @ kh, ds.T @ qh, p.T @ doh

    def untransposed_dv(qh, kh, vh, doh, scale, causal):
        p, dp = base(qh, kh, vh, doh, scale, causal)
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        return scale * ds @ kh, scale * ds.T @ qh, p @ doh

    def swapped_dk(qh, kh, vh, doh, scale, causal):
        p, dp = base(qh, kh, vh, doh, scale, causal)
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        return scale * ds @ kh, scale * ds @ qh, p.T @ doh

    return [no_centering, column_centering, missing_scale, untransposed_dv, swapped_dk]


@pytest.mark.parametrize("variant", _variants(), ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(monkeypatch, variant):
    rng = np.random.default_rng(7)
    q, k, v, do = rand4(rng, 1, 1, 4, 3)
    scale = 0.8
    fd = fd_grads(q, k, v, do, scale, True)
    monkeypatch.setattr(obwd, "_head_grads", variant)
    bad = obwd.attention_bwd_ref(q, k, v, do, scale, True)
    assert max(float(np.max(np.abs(a - b))) for a, b in zip(bad, fd)) > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_equal_full(causal):
    """The chunked, row-sampled form gives the full oracle's rows (chunks
    that do not divide N, rows at chunk edges, unordered and repeated rows)."""
    rng = np.random.default_rng(8)
    q, k, v, do = rand4(rng, 1, 1, 53, 6)
    full = obwd.attention_bwd_ref(q, k, v, do, 0.6, causal)
    qr = np.array([0, 9, 10, 52, 31, 9])
    kr = np.array([52, 0, 19, 20, 7])
    dq, dk, dv = obwd.attention_bwd_sampled(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.6, causal, qr, kr, chunk=10)
    np.testing.assert_allclose(dq, full[0][0, 0, qr], atol=1e-13, rtol=0)
    np.testing.assert_allclose(dk, full[1][0, 0, kr], atol=1e-13, rtol=0)
    np.testing.assert_allclose(dv, full[2][0, 0, kr], atol=1e-13, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_query_rows_only_equal_full(causal):
    rng = np.random.default_rng(9)
    q, k, v, do = rand4(rng, 1, 1, 41, 5)
    full = obwd.attention_bwd_ref(q, k, v, do, 0.7, causal)
    qr = np.array([40, 0, 17, 3])
    dq, dk, dv = obwd.attention_bwd_sampled(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.7, causal, qr, [], chunk=3)
    np.testing.assert_allclose(dq, full[0][0, 0, qr], atol=1e-13, rtol=0)
    assert dk.shape == (0, 5) and dv.shape == (0, 5)
