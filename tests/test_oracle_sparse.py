"""Pins for the float64 sparse-attention oracle (CPU only).

Ties oracle.sparse to hand-derived fixtures, brute-force enumeration,
a library routine (torch scaled_dot_product_attention in float64 on the CPU,
for the all-blocks case), closed forms and invariants.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sparse as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_selection():
    g = json.load(open(os.path.join(GOLDEN, "select_tiny.json")))
    keys = np.array(g["keys"], dtype=np.float64)[:, None]
    kbar = S.pool_blocks(keys, g["block"])
    assert np.array_equal(kbar[:, 0], np.array(g["expected_kbar"], dtype=np.float64))
    length = keys.shape[0]
    for c in g["cases"]:
        scores = kbar[:, 0] * c["qbar"] / math.sqrt(g["d"])
        row = S.select_row(scores, c["i"], length, g["block"], c["topk"], c["n_init"], c["n_local"])
        assert row == c["expected"], c["why"]
    t = g["tie_case"]
    scores = np.array(t["keys_kbar"], dtype=np.float64) * t["qbar"]
    assert S.select_row(scores, t["i"], length, g["block"], t["topk"], t["n_init"], t["n_local"]) == t["expected"]


def test_golden_attention():
    g = json.load(open(os.path.join(GOLDEN, "attend_tiny.json")))
    q = np.array(g["q"])[None, None, :, None]
    k = np.array(g["k"])[None, None, :, None]
    v = np.array(g["v"])[None, None, :, None]
    idx = np.array([[[[0, -1]]]])  # one block of 3 tokens (block = 4 covers them all)
    o = S.sparse_attention_prefill(q, k, v, idx, block=4, scale=g["scale"])
    np.testing.assert_allclose(o[0, 0, :, 0], g["expected_o"], rtol=0, atol=g["tol"])


def test_pool_is_block_mean():
    rng = np.random.default_rng(0)
    x = rng.integers(-100, 100, (64 * 5 + 9, 3)).astype(np.float64) / 64.0
    p = S.pool_blocks(x, 64)
    assert p.shape == (6, 3)
    for j in range(5):
        # dyadic inputs: the mean is exact (sum * 2^-6)
        assert np.array_equal(p[j], x[64 * j:64 * (j + 1)].sum(axis=0) * 2.0 ** -6)
    np.testing.assert_allclose(p[5], x[320:].mean(axis=0), rtol=1e-15)


def test_forced_and_candidate_sets_enumerated():
    assert S.forced_blocks(0, 1, 2) == {0}
    assert S.forced_blocks(1, 1, 2) == {0, 1}
    assert S.forced_blocks(7, 1, 2) == {0, 6, 7}
    assert S.forced_blocks(7, 2, 3) == {0, 1, 5, 6, 7}
    assert S.candidate_blocks(7, 8 * 64, 64, 1, 2) == [1, 2, 3, 4, 5]
    assert S.candidate_blocks(2, 3 * 64, 64, 1, 2) == []
    # n_local = 0: the query's own block becomes a candidate unless it is partial
    assert S.candidate_blocks(3, 4 * 64, 64, 1, 0) == [1, 2, 3]
    assert S.candidate_blocks(3, 4 * 64 - 1, 64, 1, 0) == [1, 2]


def test_topk_against_brute_force_definition():
    # every pick >= every non-pick; among equal scores, every pick has a smaller index
    rng = np.random.default_rng(1)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        scores = rng.integers(0, 6, n).astype(np.float64)  # many exact ties
        cands = sorted(rng.choice(n, size=int(rng.integers(0, n + 1)), replace=False).tolist())
        k = int(rng.integers(0, 12))
        picks = S.top_k(scores, cands, k)
        assert len(picks) == min(k, len(cands))
        rest = [j for j in cands if j not in picks]
        for p in picks:
            for r in rest:
                assert scores[p] > scores[r] or (scores[p] == scores[r] and p < r)


def test_pooled_score_equals_mean_of_token_logits():
    # linearity: qbar.kbar/sqrt(d) = mean over group heads and block tokens of q_t^g.kbar/sqrt(d)
    rng = np.random.default_rng(2)
    b, hq, hkv, n, d, blk = 1, 4, 2, 5 * 16, 8, 16
    q = rng.standard_normal((b, hq, n, d))
    k = rng.standard_normal((b, hkv, n, d))
    _, scores, kbar = S.sparse_select_prefill(q, k, block=blk, topk=2)
    g = hq // hkv
    for h in range(hkv):
        for i in range(5):
            toks = q[0, h * g:(h + 1) * g, i * blk:(i + 1) * blk].reshape(-1, d)
            per_token = (toks @ kbar[0, h].T) / math.sqrt(d)
            np.testing.assert_allclose(scores[0, h, i], per_token.mean(axis=0), rtol=1e-12, atol=1e-14)


def test_planted_blocks_always_selected():
    rng = np.random.default_rng(3)
    b, hq, hkv, nblk, d, blk = 1, 2, 1, 30, 16, 8
    n = nblk * blk
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = 0.1 * rng.standard_normal((b, hq, n, d)) + u
    k = 0.1 * rng.standard_normal((b, hkv, n, d))
    planted = [3, 11, 20]
    for j in planted:
        k[0, 0, j * blk:(j + 1) * blk] += 5.0 * u
    idx, _, _ = S.sparse_select_prefill(q, k, block=blk, topk=3)
    for i in range(nblk):
        row = set(idx[0, 0, i].tolist())
        for j in planted:
            if 1 <= j <= i - 2:
                assert j in row


def test_topk_covering_all_candidates_and_zero():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, 10 * 8, 4))
    k = rng.standard_normal((1, 1, 10 * 8, 4))
    idx_all, _, _ = S.sparse_select_prefill(q, k, block=8, topk=100)
    for i in range(10):
        assert [j for j in idx_all[0, 0, i] if j >= 0] == list(range(i + 1))
    idx0, _, _ = S.sparse_select_prefill(q, k, block=8, topk=0)
    for i in range(10):
        assert [j for j in idx0[0, 0, i] if j >= 0] == sorted(S.forced_blocks(i, 1, 2))


@pytest.mark.parametrize("n", [96, 100])
def test_all_blocks_equals_dense_causal_and_sdpa(n):
    rng = np.random.default_rng(n)
    b, hq, hkv, d, blk = 2, 4, 2, 16, 16
    q, k, v = (rng.standard_normal((b, h, n, d)) for h in (hq, hkv, hkv))
    idx, _, _ = S.sparse_select_prefill(q, k, block=blk, topk=1000)
    o_sparse = S.sparse_attention_prefill(q, k, v, idx, block=blk)
    o_dense = S.dense_causal_attention(q, k, v)
    np.testing.assert_allclose(o_sparse, o_dense, rtol=1e-12, atol=1e-12)
    g = hq // hkv
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(np.repeat(k, g, axis=1))
    tv = torch.from_numpy(np.repeat(v, g, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy()
    np.testing.assert_allclose(o_sparse, ref, rtol=1e-10, atol=1e-10)


def test_closed_forms_constant_v_zero_q_first_token():
    rng = np.random.default_rng(5)
    b, h, n, d, blk = 1, 2, 48, 8, 16
    q = rng.standard_normal((b, h, n, d))
    k = rng.standard_normal((b, h, n, d))
    vrow = rng.standard_normal(d)
    v_const = np.tile(vrow, (b, h, n, 1))
    idx, _, _ = S.sparse_select_prefill(q, k, block=blk, topk=1)
    o = S.sparse_attention_prefill(q, k, v_const, idx, block=blk)
    np.testing.assert_allclose(o, np.broadcast_to(vrow, o.shape), rtol=1e-13, atol=1e-13)
    v = rng.standard_normal((b, h, n, d))
    o0 = S.sparse_attention_prefill(np.zeros_like(q), k, v, idx, block=blk)
    for hh in range(h):
        for t in range(n):
            i = t // blk
            toks = [s for j in idx[0, hh, i] if j >= 0 for s in range(j * blk, (j + 1) * blk) if s <= t]
            np.testing.assert_allclose(o0[0, hh, t], v[0, hh, toks].mean(axis=0), rtol=1e-12, atol=1e-12)
    o = S.sparse_attention_prefill(q, k, v, idx, block=blk)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], rtol=1e-13, atol=1e-13)


def test_pure_python_softmax_brute_force():
    rng = np.random.default_rng(6)
    n, d, blk = 12, 3, 4
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, n, d))
    v = rng.standard_normal((1, 1, n, d))
    idx = np.array([[[[0, -1], [0, 1], [1, 2]]]])
    o = S.sparse_attention_prefill(q, k, v, idx, block=blk, scale=0.7)
    for t in range(n):
        blocks = [j for j in idx[0, 0, t // blk] if j >= 0]
        toks = [s for j in blocks for s in range(j * blk, (j + 1) * blk) if s <= t]
        logits = [0.7 * sum(q[0, 0, t, a] * k[0, 0, s, a] for a in range(d)) for s in toks]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        z = sum(w)
        for a in range(d):
            ref = sum(w[r] * v[0, 0, s, a] for r, s in enumerate(toks)) / z
            assert abs(o[0, 0, t, a] - ref) < 1e-12


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(7)
    b, hq, hkv, n, d, blk = 1, 6, 2, 40, 8, 8
    q = rng.standard_normal((b, hq, n, d))
    k = rng.standard_normal((b, hkv, n, d))
    v = rng.standard_normal((b, hkv, n, d))
    idx, _, _ = S.sparse_select_prefill(q, k, block=blk, topk=2)
    o = S.sparse_attention_prefill(q, k, v, idx, block=blk)
    g = hq // hkv
    idx_rep = np.repeat(idx, g, axis=1)
    o_mha = S.sparse_attention_prefill(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), idx_rep, block=blk)
    np.testing.assert_allclose(o, o_mha, rtol=1e-13, atol=1e-13)


def test_decode_matches_prefill_last_position():
    # With length-1 a multiple of the block, the last query block holds one
    # token, so decode pooling equals prefill pooling and the selections agree;
    # the decode attention then equals the prefill row at length-1.
    rng = np.random.default_rng(8)
    b, hq, hkv, d, blk = 2, 4, 2, 8, 8
    length = 9 * blk + 1
    q = rng.standard_normal((b, hq, length, d))
    k = rng.standard_normal((b, hkv, length, d))
    v = rng.standard_normal((b, hkv, length, d))
    idx_p, _, kbar = S.sparse_select_prefill(q, k, block=blk, topk=3)
    o_p = S.sparse_attention_prefill(q, k, v, idx_p, block=blk)
    idx_d, _ = S.sparse_select_decode(q[:, :, -1], kbar, length, block=blk, topk=3)
    assert np.array_equal(idx_d, idx_p[:, :, -1])
    o_d = S.sparse_attention_decode(q[:, :, -1], k, v, idx_d, length, block=blk)
    np.testing.assert_allclose(o_d, o_p[:, :, -1], rtol=1e-12, atol=1e-12)


def test_rows_form_equals_full_form():
    rng = np.random.default_rng(9)
    b, hq, hkv, n, d, blk = 1, 4, 1, 70, 8, 16
    q = rng.standard_normal((b, hq, n, d))
    k = rng.standard_normal((b, hkv, n, d))
    v = rng.standard_normal((b, hkv, n, d))
    idx, _, _ = S.sparse_select_prefill(q, k, block=blk, topk=1)
    o = S.sparse_attention_prefill(q, k, v, idx, block=blk)
    rows = [(0, 0, 0), (0, 3, 69), (0, 2, 33)]
    r = S.sparse_attention_prefill_rows(q, k, v, idx, rows, block=blk)
    for i, (bb, hh, t) in enumerate(rows):
        np.testing.assert_allclose(r[i], o[bb, hh, t], rtol=1e-13, atol=1e-13)


def test_selection_rows_form_equals_full_form():
    """sparse_select_prefill_rows on chosen query blocks equals those rows of the
    full selection (indices, scores, pooled keys), including a ragged last block,
    several KV heads and planted ties."""
    rng = np.random.default_rng(11)
    b, hq, hkv, n, d, blk = 2, 6, 2, 16 * 13 + 5, 8, 16
    q = rng.integers(-2, 3, (b, hq, n, d)).astype(np.float64)
    k = rng.integers(-2, 3, (b, hkv, n, d)).astype(np.float64)
    idx, sc, kbar = S.sparse_select_prefill(q, k, block=blk, topk=3, n_init=1, n_local=2)
    blocks = [0, 1, 4, 7, 13]
    ri, rs, rk = S.sparse_select_prefill_rows(q, k, blocks, block=blk, topk=3, n_init=1, n_local=2)
    assert np.array_equal(ri, idx[:, :, blocks])
    np.testing.assert_allclose(rs, sc[:, :, blocks], rtol=1e-13, atol=1e-13)  # BLAS summation order
    np.testing.assert_array_equal(rk, kbar)
