"""Pins for the float64 oracle: each test ties an oracle function to something
other than itself -- values the pages print (fixtures under tests/golden, each
with its citation), closed forms, invariants, a library routine, or brute
force -- so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.  CPU only.

Page tags: P1 = "FlashAttention分块计算优化Transformer显存效率"
(intelliparadigm.com); P2 = "14. FlashAttention Memory Model" (datawhalechina
llm-algo-leetcode); P3 = "Flash Attention 原理" (note.lovescie.com).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oatt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MiB = 1 << 20
KiB = 1 << 10


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def rand_qkv(rng, B, H, N, d, Nk=None):
    Nk = N if Nk is None else Nk
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, Nk, d)),
            rng.standard_normal((B, H, Nk, d)))


# ---------------------------------------------------------------------------
# P-1: the blocked-softmax worked example (P3, "Softmax 的分块计算")
# ---------------------------------------------------------------------------

def test_merge_worked_example_matches_page():
    g = golden("merge_example.json")
    r = oracle.blocked_softmax(g["x"], g["split"])
    assert r["local_max"] == g["local_max"]
    for nums, exps in zip(r["local_num"], g["local_numerator_exponents"]):
        assert nums == pytest.approx([math.exp(e) for e in exps], abs=0, rel=1e-15)
    # each local denominator is e^-1 + 1
    for s in r["local_sum"]:
        assert s == pytest.approx(math.exp(-1) + 1, rel=1e-15)
    assert r["global_max"] == g["global_max"]
    assert r["correction"][0] == pytest.approx(math.exp(g["first_block_correction_exponent"]), rel=1e-15)
    assert r["correction"][1] == 1.0
    # the merged result is the global softmax, written directly from its definition
    den = sum(math.exp(t) for t in g["x"])
    direct = [math.exp(t) / den for t in g["x"]]
    assert r["softmax"] == pytest.approx(direct, abs=4e-16)
    assert r["lse"] == pytest.approx(math.log(den), abs=1e-15)


def test_blocked_softmax_random_splits_match_scipy():
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(1)
    for n in (1, 2, 5, 17):
        x = rng.standard_normal(n) * 5
        for cut in range(1, n + 1):
            sizes = [cut] + ([n - cut] if n > cut else [])
            r = oracle.blocked_softmax(x, sizes)
            np.testing.assert_allclose(r["softmax"], softmax(x), atol=1e-15, rtol=1e-13)
            assert r["lse"] == pytest.approx(logsumexp(x), abs=1e-13)


def test_tiled_ref_reproduces_worked_example():
    """tiled_ref with one query row whose scores are [1,2,3,4] and key blocks
    of two: the running state after the two blocks must be the page's merge."""
    g = golden("merge_example.json")
    x = np.array(g["x"], dtype=np.float64)
    q = np.ones((1, 1, 1, 1))
    k = x.reshape(1, 1, 4, 1)                      # scale 1: S = [1,2,3,4]
    v = np.eye(4).reshape(1, 1, 4, 4)              # O row = the probabilities
    o, lse = oracle.tiled_ref(q, k, v, 1.0, False, 1, g["split"][0])
    den = sum(math.exp(t) for t in g["x"])
    np.testing.assert_allclose(o[0, 0, 0], np.exp(x) / den, atol=4e-16)
    assert lse[0, 0, 0] == pytest.approx(math.log(den), abs=1e-15)


# ---------------------------------------------------------------------------
# P-2: tiled == untiled == brute force on tiny inputs
# ---------------------------------------------------------------------------

def _adversarial(rng, N, d):
    """One key far dominant and late: forces several max rescales."""
    q, k, v = rand_qkv(rng, 1, 1, N, d)
    k[0, 0, -1] *= 30.0
    k[0, 0, N // 2] *= -20.0
    return q, k, v


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 13, 16])
@pytest.mark.parametrize("d", [1, 2, 4, 8])
def test_tiled_untiled_brute_agree(N, d):
    rng = np.random.default_rng(100 * N + d)
    cases = [rand_qkv(rng, 1, 2, N, d), _adversarial(rng, N, d)]
    scale = 1.0 / math.sqrt(d)
    for (q, k, v), causal in itertools.product(cases, (False, True)):
        ob, lb = oracle.brute_ref(q, k, v, scale, causal)
        oa, la = oracle.attention_ref(q, k, v, scale, causal)
        np.testing.assert_allclose(oa, ob, atol=1e-12, rtol=0)
        np.testing.assert_allclose(la, lb, atol=1e-12, rtol=0)
        for bq, bk in itertools.product(sorted({1, 2, 3, N}), repeat=2):
            ot, lt = oracle.tiled_ref(q, k, v, scale, causal, bq, bk)
            np.testing.assert_allclose(ot, ob, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lt, lb, atol=1e-12, rtol=0)


def test_tiled_matches_definition_mid_size_ragged():
    rng = np.random.default_rng(7)
    q, k, v = rand_qkv(rng, 2, 2, 77, 16)
    for causal in (False, True):
        oa, la = oracle.attention_ref(q, k, v, 0.25, causal)
        for bq, bk in ((64, 64), (16, 32), (32, 8), (128, 64)):
            ot, lt = oracle.tiled_ref(q, k, v, 0.25, causal, bq, bk)
            np.testing.assert_allclose(ot, oa, atol=1e-12)
            np.testing.assert_allclose(lt, la, atol=1e-12)


def test_rows_subset_equals_full():
    rng = np.random.default_rng(8)
    q, k, v = rand_qkv(rng, 1, 3, 300, 8)
    rows = np.array([0, 1, 63, 64, 127, 128, 255, 299])
    for causal in (False, True):
        of, lf = oracle.attention_ref(q, k, v, 0.3, causal)
        os_, ls = oracle.attention_ref(q, k, v, 0.3, causal, rows=rows, chunk=3)
        # same arithmetic, only the BLAS blocking of the row chunk differs
        np.testing.assert_allclose(os_, of[:, :, rows], atol=1e-14, rtol=0)
        np.testing.assert_allclose(ls, lf[:, :, rows], atol=1e-14, rtol=0)


# ---------------------------------------------------------------------------
# P-3 / P-4: invariants of the definition
# ---------------------------------------------------------------------------

def test_probability_rows_sum_to_one_and_mask_zero():
    rng = np.random.default_rng(2)
    q, k, _ = rand_qkv(rng, 2, 2, 40, 8)
    for causal in (False, True):
        p = oracle.attention_probs(q, k, 0.5, causal)
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-12, rtol=0)
        if causal:
            upper = np.triu(np.ones((40, 40), dtype=bool), 1)
            assert np.all(p[..., upper] == 0)
            assert np.all(np.diagonal(p, axis1=2, axis2=3) > 0)


def test_output_is_convex_combination_of_visible_values():
    rng = np.random.default_rng(3)
    q, k, v = rand_qkv(rng, 1, 2, 50, 6)
    k *= 3.0
    for causal in (False, True):
        o, _ = oracle.attention_ref(q, k, v, 1.0, causal)
        for b, h, i in itertools.product(range(1), range(2), range(50)):
            vis = v[b, h, : i + 1] if causal else v[b, h]
            assert np.all(o[b, h, i] >= vis.min(axis=0) - 1e-12)
            assert np.all(o[b, h, i] <= vis.max(axis=0) + 1e-12)


# ---------------------------------------------------------------------------
# P-10: closed forms
# ---------------------------------------------------------------------------

def test_closed_forms():
    rng = np.random.default_rng(4)
    q, k, v = rand_qkv(rng, 2, 2, 33, 5)
    s = 0.37
    # causal row 0 sees only key 0
    o, lse = oracle.attention_ref(q, k, v, s, True)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], s * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-14)
    # scale 0: uniform weights over the visible keys
    o, lse = oracle.attention_ref(q, k, v, 0.0, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, np.full(lse.shape, math.log(33)), atol=1e-14)
    o, lse = oracle.attention_ref(q, k, v, 0.0, True)
    cum = np.cumsum(v, axis=2) / np.arange(1, 34)[None, None, :, None]
    np.testing.assert_allclose(o, cum, atol=1e-14)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, 34)), lse.shape), atol=1e-14)
    # N = 1: output is V
    o, lse = oracle.attention_ref(q[:, :, :1], k[:, :, :1], v[:, :, :1], s, False)
    np.testing.assert_allclose(o, v[:, :, :1], atol=1e-15)
    # identical key rows: uniform attention
    kk = np.broadcast_to(k[:, :, :1], k.shape).copy()
    o, lse = oracle.attention_ref(q, kk, v, s, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    dots = s * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0])
    np.testing.assert_allclose(lse, dots + math.log(33), atol=1e-13)


def test_one_hot_attention_selects_value_row():
    """A query aligned with one key far above the rest copies that key's
    value row (the limit of a peaked softmax)."""
    d, N = 8, 12
    k = np.eye(N, d).reshape(1, 1, N, d) * 1.0
    k[0, 0, d:] = 0.0
    q = (80.0 * np.eye(N, d)[5]).reshape(1, 1, 1, d)
    q = np.broadcast_to(q, (1, 1, N, d)).copy()
    v = np.random.default_rng(5).standard_normal((1, 1, N, d))
    o, _ = oracle.attention_ref(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 5], (N, d)), atol=1e-30 + 1e-12)


# ---------------------------------------------------------------------------
# P-11: library routines
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_and_scipy_logsumexp(causal):
    import torch
    from scipy.special import logsumexp
    rng = np.random.default_rng(6)
    q, k, v = rand_qkv(rng, 2, 3, 67, 16)
    s = 1.0 / 4.0
    o, lse = oracle.attention_ref(q, k, v, s, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=s).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
    sc = s * np.einsum("bhqd,bhkd->bhqk", q, k)
    if causal:
        sc = np.where(np.tril(np.ones((67, 67), dtype=bool)), sc, -np.inf)
    np.testing.assert_allclose(lse, logsumexp(sc, axis=-1), atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# P-5 / P-9: block pattern and tile counts
# ---------------------------------------------------------------------------

def test_causal_figure_matches_page():
    g = golden("causal_figure_n8_b2.json")
    fig = oracle.causal_figure(g["N"], g["B"])
    assert fig == g["lines_as_printed"]
    flat = "".join(g["lines_as_printed"])
    assert flat.count(g["filled"]) == 20 and flat.count(g["empty"]) == 12
    c = oracle.block_counts(8, 2, 2, True)
    assert c == dict(computed=10, full=6, causal_masked=4, ragged=0, skipped=6)


def _counts_by_elements(N, bq, bk, causal):
    """Independent tile classification by enumerating every (query, key)
    element of every tile."""
    out = dict(computed=0, full=0, causal_masked=0, ragged=0, skipped=0)
    for q0 in range(0, N, bq):
        for k0 in range(0, N, bk):
            qs = range(q0, min(q0 + bq, N))
            ks = range(k0, min(k0 + bk, N))
            vis = [(not causal) or kk <= qq for qq in qs for kk in ks]
            if not any(vis):
                out["skipped"] += 1
                continue
            out["computed"] += 1
            if not all(vis):
                out["causal_masked"] += 1
            elif len(ks) < bk:
                out["ragged"] += 1
            else:
                out["full"] += 1
    return out


@pytest.mark.parametrize("N,bq,bk", [(8, 2, 2), (256, 64, 64), (100, 16, 32), (97, 32, 16),
                                      (130, 64, 128), (1000, 128, 64), (1000, 64, 64), (5, 8, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_block_counts_match_element_enumeration(N, bq, bk, causal):
    assert oracle.block_counts(N, bq, bk, causal) == _counts_by_elements(N, bq, bk, causal)


def test_block_counts_closed_forms():
    # equal square tiles, N a multiple of the tile: n(n+1)/2 computed, n on the diagonal
    for N, t in ((4096, 128), (256, 64), (32768, 128)):
        n = N // t
        assert oracle.block_counts(N, t, t, True) == dict(
            computed=n * (n + 1) // 2, full=n * (n - 1) // 2, causal_masked=n,
            ragged=0, skipped=n * (n - 1) // 2)
        assert oracle.block_counts(N, t, t, False) == dict(
            computed=n * n, full=n * n, causal_masked=0, ragged=0, skipped=0)
    # block_q = 2 block_k: query tile i computes key tiles 0..2i+1, two of them masked
    n = 4096 // 128
    c = oracle.block_counts(4096, 128, 64, True)
    assert c["computed"] == sum(2 * i + 2 for i in range(n))
    assert c["causal_masked"] == 2 * n
    # ragged non-causal at N=1000, 64x64: 16 query tiles x 1 short key tile
    c = oracle.block_counts(1000, 64, 64, False)
    assert c["computed"] == 256 and c["ragged"] == 16


def test_block_counts_reject_nonpositive():
    for bad in ((0, 64, 64), (64, 0, 64), (64, 64, -1)):
        with pytest.raises(ValueError):
            oracle.block_counts(*bad, True)


# ---------------------------------------------------------------------------
# P-6: the HBM traffic table (P1 §2.1) and P3's transfer count
# ---------------------------------------------------------------------------

def test_traffic_table_matches_page():
    g = golden("hbm_traffic_n4096.json")
    for mode, key in (("standard", "standard"), ("tiled", "flash")):
        t = oracle.traffic(g["N"], g["d"], g["block"], g["block"], g["elem_bytes"], False, mode)
        for op in "QKVSPO":
            assert t["reads"][op] == g[key][op]["read"] * MiB, (mode, op)
            assert t["writes"][op] == g[key][op]["write"] * MiB, (mode, op)
        assert t["read_total"] == g[key]["total_read"] * MiB
        assert t["write_total"] == g[key]["total_write"] * MiB
        assert t["lse_write"] == 4 * g["N"]


def test_transfer_count_six_to_two():
    g = golden("hbm_traffic_n4096.json")["transfers"]
    for mode, key in (("standard", "standard"), ("tiled", "flash")):
        t = oracle.traffic(4096, 128, 128, 128, 2, False, mode)
        # inputs are one read stream; S and P are one stream each
        reads = (t["reads"]["Q"] > 0) + (t["reads"]["S"] > 0) + (t["reads"]["P"] > 0)
        writes = sum(t["writes"][op] > 0 for op in "SPO")
        assert (reads, writes) == (g[key]["reads"], g[key]["writes"])


def test_traffic_causal_and_ragged_consistent_with_counts():
    t = oracle.traffic(4096, 128, 128, 128, 2, True, "tiled")
    c = oracle.block_counts(4096, 128, 128, True)
    assert t["reads"]["K"] == c["computed"] * 128 * 128 * 2 == int(16.5 * MiB)
    # ragged: every computed tile's real key rows are read once per query tile
    t = oracle.traffic(1000, 64, 128, 64, 2, False, "tiled")
    assert t["reads"]["K"] == 8 * 1000 * 64 * 2


# ---------------------------------------------------------------------------
# P-7 / P-8: on-chip budget (P1 §1.2) and P2's memory-model helpers
# ---------------------------------------------------------------------------

def test_sram_budget_table():
    g = golden("sram_budget_b128.json")
    b = oracle.sram_budget(g["block"], g["block"], g["d"], g["elem_bytes"])
    for row in ("Q_block", "K_block", "V_block", "S_block", "O_block"):
        assert b[row] == g["rows_kib"][row] * KiB
    assert b["stats"] == g["rows_kib"]["stats_approx"] * KiB
    assert b["total"] == g["total_approx_kib"] * KiB
    assert b["total"] <= g["sram_kib"] * KiB
    # the closed form printed on the total line does not add up to the rows
    assert oracle.sram_formula_as_printed(128, 128) == 96 * KiB != b["total"]


def test_p2_checks_and_cross_page_values():
    g = golden("p2_memory_model.json")
    # the page's three checks
    assert oracle.working_set_bytes(128, 128) > oracle.score_tile_bytes(128)
    with pytest.raises(ValueError):
        oracle.working_set_bytes(0, 128)
    assert oracle.materialization_ratio(4096, 64) > oracle.materialization_ratio(4096, 256)
    # positivity rule on every helper
    for f, args in ((oracle.score_bytes, (0,)), (oracle.score_bytes, (8, 1, -1)),
                    (oracle.tiles_1d, (8, 0)), (oracle.score_tile_bytes, (0,)),
                    (oracle.materialization_ratio, (0, 4))):
        with pytest.raises(ValueError):
            f(*args)
    # values the other page prints for the same quantities (P1 §1.2, §2.1)
    sram = golden("sram_budget_b128.json")
    traf = golden("hbm_traffic_n4096.json")
    assert oracle.score_tile_bytes(128) == sram["rows_kib"]["S_block"] * KiB
    assert oracle.working_set_bytes(128, 128) == 5 * 32 * KiB   # P1 rows without stats
    assert oracle.score_bytes(4096) == traf["standard"]["S"]["write"] * MiB
    assert oracle.tiles_1d(4096, 128) == 32                      # "32 reads" of K and V
    for tile in g["sweep_tiles"]:
        r = oracle.tile_tradeoff(g["sweep_seq_len"], tile, g["sweep_head_dim"])
        assert r["tile_count"] == oracle.tiles_1d(4096, tile) ** 2
        assert oracle.materialization_ratio(4096, tile) == r["tile_count"]
    assert oracle.tiles_1d(1000, 64) == 16 and oracle.tiles_1d(1000, 1000) == 1


# ---------------------------------------------------------------------------
# Planted mistakes: each deliberately wrong oracle part must fail a pin.
# ---------------------------------------------------------------------------

def _attention_pins_pass():
    """Run a reduced set of the attention pins; True if all hold."""
    from scipy.special import logsumexp
    import torch
    rng = np.random.default_rng(9)
    q, k, v = rand_qkv(rng, 1, 2, 21, 4)
    ok = True
    with np.errstate(all="ignore"):
        for causal in (False, True):
            o, lse = oracle.attention_ref(q, k, v, 0.5, causal)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                is_causal=causal, scale=0.5).numpy()
            ok &= np.allclose(o, ref, atol=1e-12, rtol=0)
            p = oracle.attention_probs(q, k, 0.5, causal)
            ok &= np.allclose(p.sum(-1), 1.0, atol=1e-12)
            sc = 0.5 * np.einsum("bhqd,bhkd->bhqk", q, k)
            if causal:
                sc = np.where(np.tril(np.ones((21, 21), dtype=bool)), sc, -np.inf)
            ok &= np.allclose(lse, logsumexp(sc, axis=-1), atol=1e-12)
        o, _ = oracle.attention_ref(q, k, v, 0.5, True)
        ok &= np.allclose(o[:, :, 0], v[:, :, 0], atol=1e-15)
    return bool(ok)


def test_planted_mistakes_are_caught(monkeypatch):
    assert _attention_pins_pass()
    good_scores, good_visible, good_soft = oatt._scores, oatt._visible, oatt._softmax_rows
    mutants = {
        "scale dropped": ("_scores", lambda qr, k, s: qr @ k.T),
        "operands swapped": ("_scores", lambda qr, k, s: s * (k[: len(qr)] @ qr.T)),
        "diagonal masked": ("_visible", lambda qi, n, c: np.arange(n)[None, :] < np.asarray(qi)[:, None]
                            if c else good_visible(qi, n, c)),
        "mask transposed": ("_visible", lambda qi, n, c: np.arange(n)[None, :] >= np.asarray(qi)[:, None]
                            if c else good_visible(qi, n, c)),
        "max not subtracted from lse": ("_softmax_rows",
                                        lambda s: (good_soft(s)[0], np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)))),
        "normalised over queries": ("_softmax_rows",
                                    lambda s: (np.exp(s) / np.exp(s).sum(0, keepdims=True), good_soft(s)[1])),
    }
    for name, (attr, fn) in mutants.items():
        monkeypatch.setattr(oatt, attr, fn)
        assert not _attention_pins_pass(), f"planted mistake not caught: {name}"
        monkeypatch.setattr(oatt, attr, {"_scores": good_scores, "_visible": good_visible,
                                         "_softmax_rows": good_soft}[attr])
    assert _attention_pins_pass()


def test_planted_mistakes_in_tiled_ref_are_caught(monkeypatch):
    """A tiled oracle that drops the running-output correction (the error the
    pages' loop skeleton would make if its per-block normalisation were taken
    literally) must disagree with brute force on an input that rescales."""
    rng = np.random.default_rng(10)
    q, k, v = _adversarial(rng, 9, 3)
    ob, _ = oracle.brute_ref(q, k, v, 0.7, False)
    real_exp = np.exp

    def no_correction(x, *a, **kw):
        r = real_exp(x, *a, **kw)
        # the correction factor is the only exp of a 1-D argument in tiled_ref
        return np.ones_like(r) if np.ndim(x) == 1 else r

    monkeypatch.setattr(oatt.np, "exp", no_correction)
    ot, _ = oracle.tiled_ref(q, k, v, 0.7, False, 3, 2)
    monkeypatch.setattr(oatt.np, "exp", real_exp)
    assert not np.allclose(ot, ob, atol=1e-6)
    ot, _ = oracle.tiled_ref(q, k, v, 0.7, False, 3, 2)
    np.testing.assert_allclose(ot, ob, atol=1e-12)
