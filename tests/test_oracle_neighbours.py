"""Pins for oracle.neighbours: QK RMS normalisation, rotate-half RoPE and the
output gate (CPU only).

Each test ties the oracle to something other than itself: hand-derived
values, closed forms, invariants of rotations (norm preservation, the
relative-position property, composition of angles), an independent
complex-number formulation, and the split / decode identities of the
composed layer.
"""

import cmath
import math

import numpy as np
import pytest
import torch

from oracle import linear as L
from oracle import neighbours as NB


def test_rms_norm_hand_example():
    # x = [3, 4, 0, 0]: mean of squares 25/4, root 5/2; x / 2.5 = [1.2, 1.6, 0, 0].
    y = NB.rms_norm(np.array([3.0, 4.0, 0.0, 0.0]), np.array([1.0, 2.0, 3.0, 4.0]), eps=0.0)
    np.testing.assert_allclose(y, [1.2, 3.2, 0.0, 0.0], rtol=1e-15, atol=0)


def test_rms_norm_invariants():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 64))
    one = np.ones(64)
    y = NB.rms_norm(x, one, eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)          # unit RMS
    np.testing.assert_allclose(NB.rms_norm(7.5 * x, one, eps=0.0), y, rtol=1e-13)  # scale invariance
    g = rng.standard_normal(64)
    np.testing.assert_allclose(NB.rms_norm(x, g, eps=0.0), y * g, rtol=1e-13)      # weight per feature
    assert np.all(NB.rms_norm(np.zeros(8), np.ones(8)) == 0.0)                     # eps keeps zero finite
    # eps enters inside the root: mean square 1 -> 1/sqrt(1 + eps)
    np.testing.assert_allclose(NB.rms_norm(np.ones(4), np.ones(4), eps=0.25), 1.0 / math.sqrt(1.25), rtol=1e-15)


def test_rope_hand_examples():
    p = np.array([0.0, 0.7, 3.0])
    # d = 2: theta_0 = 1, so e_0 -> (cos p, sin p) and e_1 -> (-sin p, cos p)
    e0 = NB.rope(np.tile([1.0, 0.0], (3, 1)), p)
    e1 = NB.rope(np.tile([0.0, 1.0], (3, 1)), p)
    np.testing.assert_allclose(e0, np.stack([np.cos(p), np.sin(p)], 1), rtol=0, atol=1e-15)
    np.testing.assert_allclose(e1, np.stack([-np.sin(p), np.cos(p)], 1), rtol=0, atol=1e-15)
    # d = 4, base 100: theta = [1, 1/10]; feature 1 pairs with feature 3
    y = NB.rope(np.array([[0.0, 1.0, 0.0, 0.0]]), np.array([2.0]), base=100.0)
    np.testing.assert_allclose(y, [[0.0, math.cos(0.2), 0.0, math.sin(0.2)]], rtol=0, atol=1e-15)
    y = NB.rope(np.array([[0.0, 0.0, 0.0, 1.0]]), np.array([2.0]), base=100.0)
    np.testing.assert_allclose(y, [[0.0, -math.sin(0.2), 0.0, math.cos(0.2)]], rtol=0, atol=1e-15)


def test_rope_position_zero_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((6, 128))
    np.testing.assert_array_equal(NB.rope(x[:1], np.array([0.0])), x[:1])
    y = NB.rope(x, np.arange(6) * 1000.0 + 5.0)
    np.testing.assert_allclose(x[:, :64] ** 2 + x[:, 64:] ** 2, y[:, :64] ** 2 + y[:, 64:] ** 2, rtol=1e-12)


def test_rope_relative_position_and_composition():
    # <R(q, m), R(k, n)> depends on m - n only; R(R(x, a), b) = R(x, a + b).
    rng = np.random.default_rng(13)
    d = 64
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in [(5, 2), (1000, 997), (262143, 262140), (17, 40)]:
        lhs = NB.rope(q[None], np.array([float(m)])) @ NB.rope(k[None], np.array([float(n)]))[0]
        rhs = NB.rope(q[None], np.array([float(m - n)])) @ k
        np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-9)
    x = rng.standard_normal((1, d))
    a, b = np.array([123.0]), np.array([4567.0])
    np.testing.assert_allclose(NB.rope(NB.rope(x, a), b), NB.rope(x, a + b), rtol=1e-9, atol=1e-9)


def test_rope_matches_complex_rotation_loop():
    # Independent form: z_i = x_i + 1j * x_{i+d/2} multiplied by exp(1j * p * base**(-2i/d)).
    rng = np.random.default_rng(14)
    d, base = 16, 10000.0
    x = rng.standard_normal((3, d))
    pos = [0, 9, 31337]
    y = NB.rope(x, np.array(pos, dtype=np.float64), base)
    for r, p in enumerate(pos):
        for i in range(d // 2):
            z = complex(x[r, i], x[r, i + d // 2]) * cmath.exp(1j * p * base ** (-2.0 * i / d))
            assert abs(y[r, i] - z.real) < 1e-12 and abs(y[r, i + d // 2] - z.imag) < 1e-12


def test_output_gate():
    rng = np.random.default_rng(15)
    o, g = rng.standard_normal((4, 8)), rng.standard_normal((4, 8))
    np.testing.assert_allclose(NB.output_gate(o, np.zeros_like(g)), o / 2, rtol=1e-15)
    np.testing.assert_allclose(NB.output_gate(o, g) + NB.output_gate(o, -g), o, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(NB.output_gate(o, np.full_like(g, 40.0)), o, rtol=1e-15)
    np.testing.assert_allclose(NB.output_gate(o, np.full_like(g, math.log(3.0))), 0.75 * o, rtol=1e-15)


def _layer_inputs(seed, b=1, h=2, n=40, d=8):
    rng = np.random.default_rng(seed)
    q, k, v, g = (rng.standard_normal((b, h, n, d)) for _ in range(4))
    return q, k, v, g, rng.standard_normal(d) + 1.0, rng.standard_normal(d) + 1.0, np.array([0.9, 0.6][:h])


def test_fused_layer_with_nothing_enabled_is_the_plain_layer():
    q, k, v, _, _, _, dec = _layer_inputs(16)
    o, st = NB.linear_layer_fused(q, k, v, dec, rope_base=None)
    o2, st2 = L.linear_prefill(q, k, v, dec)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(st, st2)


def test_fused_layer_matches_token_loop():
    # Per-token loop with math.* and the recurrent form of the attention.
    q, k, v, g, gq, gk, dec = _layer_inputs(17, n=12, d=4)
    eps, base, pos0 = 1e-6, 500.0, 7
    o, _ = NB.linear_layer_fused(q, k, v, dec, None, gq, gk, eps, base, pos0, g)
    d = 4
    for h in range(2):
        s = np.zeros((d, d))
        for t in range(12):
            def prep(x, gam):
                r = 1.0 / math.sqrt(sum(xx * xx for xx in x) / d + eps)
                y = [x[i] * r * gam[i] for i in range(d)]
                out = [0.0] * d
                for i in range(d // 2):
                    a = (pos0 + t) * base ** (-2.0 * i / d)
                    out[i] = y[i] * math.cos(a) - y[i + d // 2] * math.sin(a)
                    out[i + d // 2] = y[i + d // 2] * math.cos(a) + y[i] * math.sin(a)
                return np.array(out)
            qh, kh = prep(q[0, h, t], gq), prep(k[0, h, t], gk)
            s = dec[h] * s + np.outer(kh, v[0, h, t])
            ot = qh @ s
            ot = ot / (1.0 + np.exp(-g[0, h, t]))
            np.testing.assert_allclose(o[0, h, t], ot, rtol=1e-11, atol=1e-12)


def test_fused_layer_split_rows_and_decode():
    q, k, v, g, gq, gk, dec = _layer_inputs(18, b=2, n=50)
    s0 = np.random.default_rng(19).standard_normal((2, 2, 8, 8))
    kw = dict(gamma_q=gq, gamma_k=gk, eps=1e-6, rope_base=10000.0)
    o, st = NB.linear_layer_fused(q, k, v, dec, s0, gate=g, **kw)
    n1 = 31
    o1, s1 = NB.linear_layer_fused(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], dec, s0, gate=g[:, :, :n1], **kw)
    o2, s2 = NB.linear_layer_fused(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], dec, s1, pos0=n1,
                                   gate=g[:, :, n1:], **kw)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s2, st, rtol=1e-11, atol=1e-12)
    rows = [0, 13, 49]
    r = NB.linear_layer_fused_rows(q[1, 1], k[1, 1], v[1, 1], dec[1], rows, s0[1, 1], gate=g[1, 1], **kw)
    np.testing.assert_allclose(r, o[1, 1, rows], rtol=1e-11, atol=1e-12)
    # decode of the last token at position 49 from the state after 49 tokens
    _, s49 = NB.linear_layer_fused(q[:, :, :49], k[:, :, :49], v[:, :, :49], dec, s0, **kw)
    od, sd = NB.linear_decode_fused(q[:, :, 49], k[:, :, 49], v[:, :, 49], s49, dec, pos=[49, 49],
                                    gate=g[:, :, 49], **kw)
    np.testing.assert_allclose(od, o[:, :, 49], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sd, st, rtol=1e-11, atol=1e-12)


def test_round_bf16_hand_values_and_library_cast():
    """Ties go to the even significand (bf16 spacing at 1 is 2^-7); values off
    the tie go to the nearer neighbour; the result equals torch's fp32 -> bf16
    cast (a library routine) on random fp32 values across many binades."""
    cases = [(1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6), (1 + 2 ** -8 + 2 ** -20, 1 + 2 ** -7),
             (-1.5, -1.5), (0.0, 0.0), (2 ** 40 * (1 + 3 * 2 ** -8), 2 ** 40 * (1 + 2 ** -6)),
             (-(2 ** -30) * (1 + 2 ** -8), -(2 ** -30))]
    for x, want in cases:
        assert NB.round_bf16(np.array([x]))[0] == want, x
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-40, 40, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(NB.round_bf16(x.astype(np.float64)), want)


def test_fused_layer_bf16_store_is_the_plain_layer_on_rounded_inputs():
    """store="bf16": the attention runs on the transformed q, k rounded to bf16,
    and nothing is rounded when no transform is enabled."""
    rng = np.random.default_rng(13)
    B, H, n, d = 1, 2, 40, 8
    q, k, v = (rng.standard_normal((B, H, n, d)) for _ in range(3))
    gq, gk = 1 + 0.1 * rng.standard_normal(d), 1 + 0.1 * rng.standard_normal(d)
    decay = [0.9, 1.0]
    o, st = NB.linear_layer_fused(q, k, v, decay, None, gq, gk, 1e-6, 100.0, 5, None, store="bf16")
    pos = np.arange(n) + 5.0
    qh = NB.round_bf16(NB.rope(NB.rms_norm(q, gq), pos, 100.0))
    kh = NB.round_bf16(NB.rope(NB.rms_norm(k, gk), pos, 100.0))
    ro, rs = L.linear_prefill(qh, kh, v, decay)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, rs, rtol=1e-12, atol=1e-12)
    o2, _ = NB.linear_layer_fused(q, k, v, decay, store="bf16", rope_base=None)
    np.testing.assert_array_equal(o2, L.linear_prefill(q, k, v, decay)[0])
    # decode and sampled rows take the same rounding
    od, _ = NB.linear_decode_fused(q[:, :, 7], k[:, :, 7], v[:, :, 7], np.zeros((B, H, d, d)), decay, gq, gk, 1e-6,
                                  100.0, [12], None, store="bf16")
    qd = NB.round_bf16(NB.rope(NB.rms_norm(q[:, :, 7:8], gq), np.array([12.0]), 100.0))[:, :, 0]
    kd = NB.round_bf16(NB.rope(NB.rms_norm(k[:, :, 7:8], gk), np.array([12.0]), 100.0))[:, :, 0]
    np.testing.assert_allclose(od, L.linear_decode_batched(qd, kd, v[:, :, 7], np.zeros((B, H, d, d)), decay)[0],
                               rtol=1e-12, atol=1e-12)
    rows = NB.linear_layer_fused_rows(q[0, 1], k[0, 1], v[0, 1], 1.0, [0, 17, 39], None, gq, gk, 1e-6, 100.0, 5,
                                     store="bf16")
    np.testing.assert_allclose(rows, o[0, 1, [0, 17, 39]], rtol=1e-12, atol=1e-12)
