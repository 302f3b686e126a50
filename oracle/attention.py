"""Attention forward in float64 on the CPU: the definition, the pages' tiled
algorithm, and a scalar brute force.  Test infrastructure only (see the
package docstring); page tags P1/P2/P3 are defined there.

Conventions shared by all three functions (the readings are listed with the
reasons in the design notes):

* Tensors are ``[B, H, N, d]``; each head is an N x d matrix whose rows are
  tokens (P1 §1.1, the row slices ``Q[i:i+B_q]``).
* ``scale`` multiplies Q.K^T; the pages use 1/sqrt(d) (P1 §1.1 and §3.2).
* Causal: key k is visible to query q iff k <= q, the diagonal included
  (P1 §2.2 -- lower-triangular mask, diagonal blocks computed).  With equal
  query and key lengths every row sees at least key 0.
* LSE_q = ln sum_k exp(S[q, k]) over the visible keys: the one number that
  carries the per-row maximum and normaliser kept for a recomputing backward
  pass (P3, "two pillars", recomputation).
"""

import math

import numpy as np


def _as64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Building blocks of the plain definition.  Kept as separate functions so the
# pin tests can swap one for a deliberately wrong version and show that a pin
# catches it.
# ---------------------------------------------------------------------------

def _scores(q_rows, k, scale):
    """S = scale * Q K^T for a block of query rows (P1 §1.1, step one of the
    standard computation; P1 §3.2 first line)."""
    return scale * (q_rows @ k.T)


def _visible(q_idx, n_keys, causal):
    """Boolean [len(q_idx), n_keys]: key k visible to query q (k <= q when
    causal, P1 §2.2)."""
    k_idx = np.arange(n_keys)
    if not causal:
        return np.ones((len(q_idx), n_keys), dtype=bool)
    return k_idx[None, :] <= np.asarray(q_idx)[:, None]


def _softmax_rows(s):
    """Row softmax of a score block whose masked entries are -inf, plus the
    per-row log-sum-exp.  softmax(x)_i = exp(x_i) / sum_j exp(x_j) (P1 §3.1);
    the maximum is subtracted first for range only, as in P3's worked example,
    which does not change the value."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    p = e / l
    lse = (m + np.log(l))[:, 0]
    return p, lse


def _head_rows(qh, kh, vh, scale, causal, rows):
    s = _scores(qh[rows], kh, scale)
    s = np.where(_visible(rows, kh.shape[0], causal), s, -np.inf)
    p, lse = _softmax_rows(s)
    return p @ vh, lse


def attention_ref(q, k, v, scale, causal, rows=None, chunk=512):
    """Exact attention O = softmax(scale * Q K^T [causal mask]) V and LSE.

    The plain definition (P1 §1.1, the standard three-step computation),
    evaluated in float64 with S and P materialised for whole rows.  P3's
    softmax section says the blocked method reaches this same result, so the
    definition itself is the oracle; no online logic is used here.

    q, k, v : array-like ``[B, H, N, d]`` (widened to float64).
    scale   : float multiplying Q K^T.
    causal  : bool.
    rows    : optional 1-D integer array of query rows; when given only those
              rows are computed (for sampled checks at large N), and the
              outputs have ``len(rows)`` in place of N.
    chunk   : rows per materialised block (memory only, no effect on value).

    Returns ``(o, lse)`` with shapes ``[B, H, R, d]`` and ``[B, H, R]``.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, _ = q.shape
    dv = v.shape[3]
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((B, H, len(sel), dv))
    lse = np.empty((B, H, len(sel)))
    for b in range(B):
        for h in range(H):
            for c0 in range(0, len(sel), chunk):
                r = sel[c0:c0 + chunk]
                o[b, h, c0:c0 + len(r)], lse[b, h, c0:c0 + len(r)] = \
                    _head_rows(q[b, h], k[b, h], v[b, h], scale, causal, r)
    return o, lse


def attention_probs(q, k, scale, causal):
    """The probability matrix P = softmax(scale * Q K^T [mask]) for every head,
    ``[B, H, N, N]`` in float64 (P1 §1.1 step two).  For small N only."""
    q, k = _as64(q), _as64(k)
    B, H, N, _ = q.shape
    out = np.empty((B, H, N, k.shape[2]))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], scale)
            s = np.where(_visible(rows, k.shape[2], causal), s, -np.inf)
            out[b, h], _ = _softmax_rows(s)
    return out


def tiled_ref(q, k, v, scale, causal, block_q, block_k):
    """The pages' block algorithm: loop over query blocks, stream key/value
    blocks, keep a running maximum, running sum and running output
    (P1 §1.1 loop skeleton; the per-block update is P1 §3.2's online softmax,
    which replaces the separately normalised per-block softmax that §1.1
    sketches, since summing separately normalised blocks is not exact).

    * State per query row starts at m = -inf, l = 0, O = 0 (the §3.2 sketch
      leaves the start state and the final division implicit; P3's merge
      example fixes them: the merged result equals the global softmax).
    * Causal: a key block whose first key lies after the block's last query
      is skipped without being touched (P1 §2.2); blocks that straddle the
      diagonal get the element mask.
    * Ragged N: the last blocks are simply shorter (P2 Q2 counts tiles with a
      ceiling).
    * After the last block: O = O_running / l and LSE = m + ln l.

    Returns ``(o, lse)`` like ``attention_ref``.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, _ = q.shape
    Nk, dv = k.shape[2], v.shape[3]
    o = np.empty((B, H, N, dv))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, h], k[b, h], v[b, h]
            for i0 in range(0, N, block_q):
                qi = np.arange(i0, min(i0 + block_q, N))
                Qi = Q[qi]
                m = np.full(len(qi), -np.inf)
                l = np.zeros(len(qi))
                acc = np.zeros((len(qi), dv))
                for j0 in range(0, Nk, block_k):
                    kj = np.arange(j0, min(j0 + block_k, Nk))
                    if causal and kj[0] > qi[-1]:
                        continue                      # block fully in the future
                    S = scale * (Qi @ K[kj].T)
                    if causal:
                        S = np.where(kj[None, :] <= qi[:, None], S, -np.inf)
                    m_new = np.maximum(m, S.max(axis=1))
                    # correction exp(m_old - m_new); a row that has seen no
                    # visible key yet keeps factor 1 instead of exp(-inf+inf)
                    corr = np.where(np.isneginf(m_new), 1.0, np.exp(m - m_new))
                    safe_m = np.where(np.isneginf(m_new), 0.0, m_new)
                    P = np.exp(S - safe_m[:, None])
                    l = l * corr + P.sum(axis=1)
                    acc = acc * corr[:, None] + P @ V[kj]
                    m = m_new
                o[b, h, qi] = acc / l[:, None]
                lse[b, h, qi] = m + np.log(l)
    return o, lse


def brute_ref(q, k, v, scale, causal):
    """Scalar pure-Python attention with ``math.exp`` and ``math.fsum``; no
    NumPy arithmetic.  For tiny inputs (N <= 16, d <= 8) as an independent
    cross-check of the definition.  Same formula as ``attention_ref``:
    O_q = sum_k exp(S_qk) V_k / sum_k exp(S_qk) over visible k."""
    qa = np.asarray(q, dtype=np.float64).tolist()
    ka = np.asarray(k, dtype=np.float64).tolist()
    va = np.asarray(v, dtype=np.float64).tolist()
    B, H = len(qa), len(qa[0])
    N, d = len(qa[0][0]), len(qa[0][0][0])
    dv = len(va[0][0][0])
    o = [[[[0.0] * dv for _ in range(N)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            Q, K, V = qa[b][h], ka[b][h], va[b][h]
            for i in range(N):
                keys = range(i + 1) if causal else range(len(K))
                s = {j: scale * math.fsum(Q[i][c] * K[j][c] for c in range(d))
                     for j in keys}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in keys}
                den = math.fsum(w.values())
                for c in range(dv):
                    o[b][h][i][c] = math.fsum(w[j] * V[j][c] for j in keys) / den
                lse[b][h][i] = mx + math.log(den)
    return np.array(o), np.array(lse)
