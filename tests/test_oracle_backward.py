"""Pins for oracle.backward (CPU only): the gradients of the linear and sparse
attention definitions, tied to things other than their own formulas --
central finite differences of the forward oracle, an independent chunked
reverse recurrence, closed forms at decay 0 and for single-token rows, and
torch autograd of scaled_dot_product_attention in float64 (a library routine)
for the all-blocks case."""

import math

import numpy as np
import pytest
import torch

from oracle import backward as BW
from oracle import linear as L
from oracle import sparse as S


def fd_grad(f, x, h=1e-6):
    """Central finite differences of the scalar f at every element of x."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("lam", [0.0, 0.7, 1.0])
@pytest.mark.parametrize("with_state", [False, True])
def test_linear_gradients_match_finite_differences(lam, with_state):
    rng = np.random.default_rng(int(lam * 10) + 3 * with_state)
    n, d = 9, 3
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    do = rng.standard_normal((n, d))
    s_in = rng.standard_normal((d, d)) if with_state else None
    ds = rng.standard_normal((d, d)) if with_state else None

    def loss():
        o, s = L.linear_attention(q, k, v, lam, s_in)
        return float(np.sum(do * o) + (np.sum(ds * s) if ds is not None else 0.0))

    dq, dk, dv, dsi = BW.linear_attention_backward(q, k, v, do, lam, s_in, ds)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        np.testing.assert_allclose(g, fd_grad(loss, x), rtol=1e-7, atol=1e-7)
    if with_state:
        np.testing.assert_allclose(dsi, fd_grad(loss, s_in), rtol=1e-7, atol=1e-7)
    else:
        # the gradient a zero initial state would receive: d/dS_in at S_in = 0
        s_in = np.zeros((d, d))
        np.testing.assert_allclose(dsi, fd_grad(loss, s_in), rtol=1e-7, atol=1e-7)


@pytest.mark.parametrize("chunk", [1, 3, 4, 17])
@pytest.mark.parametrize("lam", [0.0, 0.43, 0.99, 1.0])
def test_linear_chunked_gradients_equal_quadratic(chunk, lam):
    rng = np.random.default_rng(chunk * 7 + int(lam * 100))
    n, d = 17, 4  # ragged tails for chunks 3 and 4
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    s_in, ds = rng.standard_normal((d, d)), rng.standard_normal((d, d))
    for si, dso in ((None, None), (s_in, None), (None, ds), (s_in, ds)):
        a = BW.linear_attention_backward(q, k, v, do, lam, si, dso)
        b = BW.linear_attention_backward_chunked(q, k, v, do, lam, chunk, si, dso)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=1e-10, atol=1e-10)


def test_linear_decay_zero_closed_form():
    """lam = 0: o_t = (q_t . k_t) v_t, so dq_t = (do_t . v_t) k_t, dk_t = (do_t . v_t) q_t,
    dv_t = (q_t . k_t) do_t; with dS the last token also gets dS v_t and k_t dS."""
    rng = np.random.default_rng(5)
    n, d = 6, 3
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    ds = rng.standard_normal((d, d))
    dq, dk, dv, dsi = BW.linear_attention_backward(q, k, v, do, 0.0, None, ds)
    c = np.sum(do * v, axis=1, keepdims=True)
    np.testing.assert_allclose(dq, c * k, rtol=1e-13, atol=1e-13)
    want_dk = c * q
    want_dk[-1] += ds @ v[-1]
    np.testing.assert_allclose(dk, want_dk, rtol=1e-13, atol=1e-13)
    want_dv = np.sum(q * k, axis=1, keepdims=True) * do
    want_dv[-1] += k[-1] @ ds
    np.testing.assert_allclose(dv, want_dv, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dsi, np.zeros((d, d)), atol=1e-15)


def test_linear_batched_driver_and_forms():
    rng = np.random.default_rng(8)
    B, H, n, d = 2, 3, 11, 4
    q, k, v, do = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    s_in, ds = rng.standard_normal((B, H, d, d)), rng.standard_normal((B, H, d, d))
    dec = [0.5, 1.0, 0.9]
    a = BW.linear_prefill_backward(q, k, v, do, dec, s_in, ds)
    b = BW.linear_prefill_backward(q, k, v, do, dec, s_in, ds, form="chunked", chunk=4)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-10, atol=1e-10)
    one = BW.linear_attention_backward(q[1, 2], k[1, 2], v[1, 2], do[1, 2], 0.9, s_in[1, 2], ds[1, 2])
    for x, y in zip(a, one):
        np.testing.assert_allclose(x[1, 2], y, rtol=1e-13, atol=1e-13)


def _sparse_case(seed, B=1, Hq=4, Hkv=2, n=21, d=3, block=4, topk=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, n, d))
    k = rng.standard_normal((B, Hkv, n, d))
    v = rng.standard_normal((B, Hkv, n, d))
    do = rng.standard_normal((B, Hq, n, d))
    idx, _, _ = S.sparse_select_prefill(q, k, block=block, topk=topk)
    return q, k, v, do, idx


def test_sparse_gradients_match_finite_differences():
    q, k, v, do, idx = _sparse_case(1)

    def loss():
        return float(np.sum(do * S.sparse_attention_prefill(q, k, v, idx, block=4)))

    dq, dk, dv = BW.sparse_attention_backward(q, k, v, idx, do, block=4)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        np.testing.assert_allclose(g, fd_grad(loss, x), rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("n", [16, 23])
def test_sparse_all_blocks_equals_sdpa_autograd(n):
    """With every block selected the gradients are those of dense causal
    attention: torch autograd through scaled_dot_product_attention in float64,
    with the KV heads repeated for the GQA group."""
    rng = np.random.default_rng(n)
    B, Hq, Hkv, d, blk = 1, 4, 2, 5, 4
    q = rng.standard_normal((B, Hq, n, d))
    k = rng.standard_normal((B, Hkv, n, d))
    v = rng.standard_normal((B, Hkv, n, d))
    do = rng.standard_normal((B, Hq, n, d))
    idx, _, _ = S.sparse_select_prefill(q, k, block=blk, topk=1000)
    dq, dk, dv = BW.sparse_attention_backward(q, k, v, idx, do, block=blk)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    g = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk.repeat_interleave(g, dim=1),
                                                         tv.repeat_interleave(g, dim=1), is_causal=True)
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-10)


def test_sparse_gqa_equals_mha_with_repeated_kv():
    q, k, v, do, idx = _sparse_case(4, Hq=6, Hkv=2, n=26, topk=2)
    g = 3
    dq, dk, dv = BW.sparse_attention_backward(q, k, v, idx, do, block=4)
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    idx_r = np.repeat(idx, g, axis=1)
    dq2, dk2, dv2 = BW.sparse_attention_backward(q, kr, vr, idx_r, do, block=4)
    np.testing.assert_allclose(dq, dq2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk, dk2.reshape(1, 2, g, 26, 3).sum(axis=2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv, dv2.reshape(1, 2, g, 26, 3).sum(axis=2), rtol=1e-12, atol=1e-12)


def test_sparse_first_token_closed_form():
    """Token 0 attends only to itself: p = 1, so its query gets no gradient, its
    value gets do_0 from that row, and its key gets nothing from that row."""
    q, k, v, do, idx = _sparse_case(6, Hq=2, Hkv=2, n=1)
    dq, dk, dv = BW.sparse_attention_backward(q, k, v, idx, do, block=4)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, do, rtol=1e-15)


def test_sparse_scale_enters_as_chain_rule():
    """Doubling the scale with q halved gives the same output; the gradients obey
    dq(q/2, 2s) = 2 dq(q, s) and equal dk, dv."""
    q, k, v, do, idx = _sparse_case(7)
    s = 1.0 / math.sqrt(3)
    a = BW.sparse_attention_backward(q, k, v, idx, do, block=4, scale=s)
    b = BW.sparse_attention_backward(q / 2, k, v, idx, do, block=4, scale=2 * s)
    np.testing.assert_allclose(b[0], 2 * a[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b[2], a[2], rtol=1e-12, atol=1e-12)


def test_sparse_dq_rows_equal_the_full_form():
    """The per-row dq (a row's gradient needs only its own keys) equals the rows
    of the batched gradient, GQA and ragged tail included."""
    q, k, v, do, idx = _sparse_case(9, B=2, Hq=6, Hkv=2, n=23, d=5, topk=2)
    dq, _, _ = BW.sparse_attention_backward(q, k, v, idx, do, block=4)
    rows = [(0, 0, 0), (1, 5, 22), (0, 3, 9), (1, 2, 17), (0, 4, 4)]
    got = BW.sparse_attention_backward_dq_rows(q, k, v, idx, do, rows, block=4)
    for r, (b, h, t) in enumerate(rows):
        np.testing.assert_allclose(got[r], dq[b, h, t], rtol=1e-12, atol=1e-13)


def test_sparse_kv_blocks_equal_the_full_form():
    """dk, dv of chosen key blocks, summed over the query blocks that selected
    them, equal the blocks of the batched gradient (GQA, the ragged last
    block, both batch rows)."""
    q, k, v, do, idx = _sparse_case(10, B=2, Hq=6, Hkv=2, n=27, d=5, topk=2)
    _, dk, dv = BW.sparse_attention_backward(q, k, v, idx, do, block=4)
    blocks = [(0, 0, 0), (1, 1, 3), (0, 1, 6), (1, 0, 5)]
    gk, gv = BW.sparse_attention_backward_kv_blocks(q, k, v, idx, do, blocks, block=4)
    for r, (b, kv, j) in enumerate(blocks):
        m = min(4, 27 - 4 * j)
        np.testing.assert_allclose(gk[r, :m], dk[b, kv, 4 * j:4 * j + m], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(gv[r, :m], dv[b, kv, 4 * j:4 * j + m], rtol=1e-11, atol=1e-12)

