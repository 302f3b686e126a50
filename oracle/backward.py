"""Attention backward in float64 on the CPU: the gradients of the forward's
definition.  Test infrastructure only (see the package docstring); page tags
P1/P2/P3 are defined there.

The pages name recomputation as the method's second pillar (P3, "two
pillars", and its interview questions): the forward keeps only each row's
softmax statistics, and the backward rebuilds the probabilities tile by tile
from them instead of reading a stored N x N matrix.  The pages do not print
the gradient formulas; what the backward must produce is fixed by the forward
it differentiates (P1 §1.1, the standard computation O = softmax(scale Q K^T) V
with P1 §2.2's causal mask).  So this oracle is that derivative written out
with the plain chain rule, on materialised matrices, and it does NOT use the
row identity sum_k P dP = sum_c dO O that a fast kernel relies on: the
softmax Jacobian appears here in its textbook form.

For one head, with P = softmax(S) row by row and S = scale Q K^T (masked
entries -inf, so P = 0 there), and a loss whose gradient at O is dO:

    dV = P^T dO                      (O = P V, product rule)
    dP = dO V^T
    dS[q, k] = P[q, k] (dP[q, k] - sum_j P[q, j] dP[q, j])
                                     (softmax Jacobian, row q)
    dQ = scale dS K                  (S = scale Q K^T)
    dK = scale dS^T Q
"""

import numpy as np

from .attention import _as64, _scores, _softmax_rows, _visible


def _head_grads(qh, kh, vh, doh, scale, causal):
    n = qh.shape[0]
    s = _scores(qh, kh, scale)
    s = np.where(_visible(np.arange(n), kh.shape[0], causal), s, -np.inf)
    p, _ = _softmax_rows(s)
    dv = p.T @ doh
    dp = doh @ vh.T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    return dq, dk, dv


def attention_bwd_ref(q, k, v, dout, scale, causal, heads=None):
    """Gradients (dQ, dK, dV) of O = softmax(scale Q K^T [causal]) V at the
    output gradient ``dout``, in float64 with S, P, dP and dS materialised for
    whole heads.

    q, k, v, dout : array-like ``[B, H, N, d]`` (widened to float64).
    heads         : optional list of (b, h) pairs; when given only those heads
                    are computed and the outputs are ``[len(heads), N, d]``.

    Returns ``(dq, dk, dv)`` shaped like the inputs (or per selected head).
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, H = q.shape[:2]
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    out = [np.empty((len(sel),) + x.shape[2:]) for x in (q, k, v)]
    for i, (b, h) in enumerate(sel):
        g = _head_grads(q[b, h], k[b, h], v[b, h], dout[b, h], scale, causal)
        for o, x in zip(out, g):
            o[i] = x
    if heads is None:
        out = [o.reshape(x.shape) for o, x in zip(out, (q, k, v))]
    return tuple(out)


def brute_bwd_ref(q, k, v, dout, scale, causal):
    """Scalar pure-Python gradients for tiny inputs: the loss
    L = sum_{q,c} dO[q,c] O[q,c] differentiated entry by entry with the
    softmax Jacobian dP_k/dS_j = P_k (delta_kj - P_j), written as loops with
    ``math.exp``/``math.fsum``; an independent cross-check of
    ``attention_bwd_ref``."""
    import math
    qa = np.asarray(q, dtype=np.float64).tolist()
    ka = np.asarray(k, dtype=np.float64).tolist()
    va = np.asarray(v, dtype=np.float64).tolist()
    da = np.asarray(dout, dtype=np.float64).tolist()
    B, H, N, d = len(qa), len(qa[0]), len(qa[0][0]), len(qa[0][0][0])
    dq = np.zeros((B, H, N, d))
    dk = np.zeros((B, H, N, d))
    dv = np.zeros((B, H, N, d))
    for b in range(B):
        for h in range(H):
            Q, K, V, G = qa[b][h], ka[b][h], va[b][h], da[b][h]
            for i in range(N):
                keys = list(range(i + 1)) if causal else list(range(N))
                s = [scale * math.fsum(Q[i][c] * K[j][c] for c in range(d)) for j in keys]
                mx = max(s)
                w = [math.exp(t - mx) for t in s]
                den = math.fsum(w)
                p = [t / den for t in w]
                # dL/dP_j = dO_i . V_j ; dL/dV_j += P_j dO_i
                g = [math.fsum(G[i][c] * V[j][c] for c in range(d)) for j in keys]
                for a, j in enumerate(keys):
                    for c in range(d):
                        dv[b, h, j, c] += p[a] * G[i][c]
                # dL/dS_a = sum_j g_j P_j (delta_ja - P_a)
                for a, j in enumerate(keys):
                    dsa = math.fsum(g[t] * p[t] * ((1.0 if t == a else 0.0) - p[a])
                                    for t in range(len(keys)))
                    for c in range(d):
                        dq[b, h, i, c] += scale * dsa * K[j][c]
                        dk[b, h, j, c] += scale * dsa * Q[i][c]
    return dq, dk, dv


def attention_bwd_sampled(qh, kh, vh, doh, scale, causal, q_rows, k_rows, chunk=512):
    """The same gradients for ONE head, returned only at the query rows
    ``q_rows`` (dQ) and key rows ``k_rows`` (dK, dV), for heads too long to
    materialise N x N matrices whole.  Query rows are taken ``chunk`` at a
    time; every row's softmax, dP and Jacobian centring are over the complete
    row exactly as in ``attention_bwd_ref`` (nothing is blocked along keys),
    and the key-row gradients sum the rows' contributions.

    qh, kh, vh, doh : [N, d] arrays (widened to float64).
    Returns ``(dq [len(q_rows), d], dk [len(k_rows), d], dv [len(k_rows), d])``.
    With no key rows asked for, only the requested query rows are visited
    (a row's dQ needs only that row's P, dP and centring).
    """
    qh, kh, vh, doh = _as64(qh), _as64(kh), _as64(vh), _as64(doh)
    n, d = qh.shape
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    dq = np.zeros((len(q_rows), d))
    dk = np.zeros((len(k_rows), d))
    dv = np.zeros((len(k_rows), d))
    if len(k_rows) == 0:
        for i0 in range(0, len(q_rows), chunk):
            rows = q_rows[i0:i0 + chunk]
            s = np.where(_visible(rows, kh.shape[0], causal), _scores(qh[rows], kh, scale), -np.inf)
            p, _ = _softmax_rows(s)
            dp = doh[rows] @ vh.T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[i0:i0 + len(rows)] = scale * (ds @ kh)
        return dq, dk, dv
    for c0 in range(0, n, chunk):
        rows = np.arange(c0, min(c0 + chunk, n))
        s = np.where(_visible(rows, kh.shape[0], causal), _scores(qh[rows], kh, scale), -np.inf)
        p, _ = _softmax_rows(s)
        dp = doh[rows] @ vh.T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        dk += scale * (ds[:, k_rows].T @ qh[rows])
        dv += p[:, k_rows].T @ doh[rows]
        mine = np.nonzero((q_rows >= c0) & (q_rows < c0 + len(rows)))[0]
        if len(mine):
            dq[mine] = scale * (ds[q_rows[mine] - c0] @ kh)
    return dq, dk, dv
