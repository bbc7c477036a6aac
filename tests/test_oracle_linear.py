"""Pins for the float64 linear-attention oracle (CPU only).

Each test ties oracle.linear to something other than itself: exact rational
brute force, a hand-derived fixture, closed forms of geometric series,
special cases that reduce to a library routine (cumsum), or invariants
between independently written forms (quadratic / chunked / recurrent).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import linear as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_golden_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "linear_tiny.json")))
    q, k, v = (np.array(g[x]) for x in ("q", "k", "v"))
    o, s = L.linear_attention(q, k, v, g["lam"], np.array(g["state_in"]))
    assert np.array_equal(o, np.array(g["expected_o"]))
    assert np.array_equal(s, np.array(g["expected_state"]))
    dec = g["decode"]
    od, sd = L.linear_decode(np.array(dec["q"]), np.array(dec["k"]), np.array(dec["v"]), g["lam"], s)
    assert np.array_equal(od, np.array(dec["expected_o"]))
    assert np.array_equal(sd, np.array(dec["expected_state"]))


def test_exact_rational_brute_force():
    # Integer inputs and lam = 3/4: every quantity is a dyadic rational, so the
    # float64 oracle must agree with exact arithmetic to the last bit.
    rng = np.random.default_rng(7)
    n, dk, dv = 6, 3, 2
    q = rng.integers(-3, 4, (n, dk))
    k = rng.integers(-3, 4, (n, dk))
    v = rng.integers(-3, 4, (n, dv))
    s_in = rng.integers(-2, 3, (dk, dv))
    lam = Fraction(3, 4)
    o_ref = [[Fraction(0)] * dv for _ in range(n)]
    for t in range(n):
        for b in range(dv):
            acc = Fraction(0)
            for s in range(t + 1):
                dot = sum(int(q[t, a]) * int(k[s, a]) for a in range(dk))
                acc += lam ** (t - s) * dot * int(v[s, b])
            acc += lam ** (t + 1) * sum(int(q[t, a]) * int(s_in[a, b]) for a in range(dk))
            o_ref[t][b] = acc
    st_ref = [[lam ** n * int(s_in[a, b]) + sum(lam ** (n - 1 - s) * int(k[s, a]) * int(v[s, b])
                                                for s in range(n)) for b in range(dv)] for a in range(dk)]
    o, st = L.linear_attention(q, k, v, 0.75, s_in)
    assert np.array_equal(o, np.array([[float(x) for x in r] for r in o_ref]))
    assert np.array_equal(st, np.array([[float(x) for x in r] for r in st_ref]))


@pytest.mark.parametrize("lam", [0.9, 0.5, 1.0])
def test_closed_form_constant_keys_values(lam):
    # k_s = k, v_s = v for all s: o_t = (q_t.k) v * sum_{m=0..t} lam^m (geometric series).
    rng = np.random.default_rng(1)
    n, d = 50, 4
    q = _rand(rng, n, d)
    k1, v1 = _rand(rng, d), _rand(rng, d)
    k = np.tile(k1, (n, 1))
    v = np.tile(v1, (n, 1))
    o, st = L.linear_attention(q, k, v, lam)
    t = np.arange(n)
    geo = (t + 1.0) if lam == 1.0 else (1.0 - lam ** (t + 1)) / (1.0 - lam)
    expect = (q @ k1)[:, None] * geo[:, None] * v1[None, :]
    np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-12)
    geo_n = n if lam == 1.0 else (1.0 - lam ** n) / (1.0 - lam)
    np.testing.assert_allclose(st, geo_n * np.outer(k1, v1), rtol=1e-12, atol=1e-12)


def test_lambda_zero_is_diagonal_only():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 20, 8), _rand(rng, 20, 8), _rand(rng, 20, 5)
    s_in = _rand(rng, 8, 5)
    o, st = L.linear_attention(q, k, v, 0.0, s_in)
    np.testing.assert_allclose(o, np.sum(q * k, axis=1)[:, None] * v, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(st, np.outer(k[-1], v[-1]), rtol=1e-13, atol=1e-13)


def test_lambda_one_is_prefix_sum():
    # lam = 1: S_t = cumsum of outer products (library prefix sum), o_t = q_t S_t.
    rng = np.random.default_rng(3)
    n, dk, dv = 40, 6, 3
    q, k, v = _rand(rng, n, dk), _rand(rng, n, dk), _rand(rng, n, dv)
    prefix = np.cumsum(k[:, :, None] * v[:, None, :], axis=0)
    expect = np.einsum("ta,tab->tb", q, prefix)
    o, st = L.linear_attention(q, k, v, 1.0)
    np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, prefix[-1], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,chunk", [(200, 1), (200, 16), (200, 64), (256, 128), (200, 200), (130, 64), (97, 128)])
@pytest.mark.parametrize("with_state", [False, True])
def test_chunked_and_recurrent_equal_quadratic(n, chunk, with_state):
    rng = np.random.default_rng(n + chunk)
    d = 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    s_in = _rand(rng, d, d) if with_state else None
    for lam in (0.43, 0.97, 1.0):
        o_q, s_q = L.linear_attention(q, k, v, lam, s_in)
        o_c, s_c = L.linear_attention_chunked(q, k, v, lam, chunk, s_in)
        np.testing.assert_allclose(o_c, o_q, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(s_c, s_q, rtol=1e-10, atol=1e-10)
    o_r, s_r = L.linear_attention_recurrent(q, k, v, 0.97, s_in)
    o_q, s_q = L.linear_attention(q, k, v, 0.97, s_in)
    np.testing.assert_allclose(o_r, o_q, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(s_r, s_q, rtol=1e-10, atol=1e-10)


def test_state_carry_split_equals_whole():
    rng = np.random.default_rng(4)
    n1, n2, d = 70, 55, 8
    q, k, v = _rand(rng, n1 + n2, d), _rand(rng, n1 + n2, d), _rand(rng, n1 + n2, d)
    s0 = _rand(rng, d, d)
    lam = 0.9
    o_all, s_all = L.linear_attention(q, k, v, lam, s0)
    o1, s1 = L.linear_attention(q[:n1], k[:n1], v[:n1], lam, s0)
    o2, s2 = L.linear_attention(q[n1:], k[n1:], v[n1:], lam, s1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_all, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s2, s_all, rtol=1e-11, atol=1e-11)


def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(5)
    n, d = 33, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    s0 = _rand(rng, d, d)
    lam = 0.8
    o_all, s_all = L.linear_attention(q, k, v, lam, s0)
    _, s_prev = L.linear_attention(q[:-1], k[:-1], v[:-1], lam, s0)
    o_dec, s_dec = L.linear_decode(q[-1], k[-1], v[-1], lam, s_prev)
    np.testing.assert_allclose(o_dec, o_all[-1], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s_dec, s_all, rtol=1e-11, atol=1e-11)


def test_rows_and_batched_forms_agree():
    rng = np.random.default_rng(6)
    b, h, n, d = 2, 3, 45, 8
    q, k, v = _rand(rng, b, h, n, d), _rand(rng, b, h, n, d), _rand(rng, b, h, n, d)
    decay = np.array([0.5, 0.9, 1.0])
    s0 = _rand(rng, b, h, d, d)
    o, st = L.linear_prefill(q, k, v, decay, s0)
    oc, stc = L.linear_prefill(q, k, v, decay, s0, form="chunked", chunk=16)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(stc, st, rtol=1e-10, atol=1e-10)
    rows = [0, 7, 44]
    for bb in range(b):
        for hh in range(h):
            r = L.linear_attention_rows(q[bb, hh], k[bb, hh], v[bb, hh], decay[hh], rows, s0[bb, hh])
            np.testing.assert_allclose(r, o[bb, hh, rows], rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(L.final_state(k[bb, hh], v[bb, hh], decay[hh], s0[bb, hh]),
                                       st[bb, hh], rtol=1e-11, atol=1e-11)
