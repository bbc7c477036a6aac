"""Degenerate sizes on the GPU: single tokens, sequences shorter than one
block or one chunk, a block plus one token, and a decode at the first
position.  Each case goes through the C ABI and is compared with the float64
oracle (indices exactly, outputs to the dtype's tolerance)."""

import math

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_amd as sala
from hybrid_sparse_linear_amd import inputs as I
from oracle import linear as OL
from oracle import sparse as OS
from parity import assert_close, host64

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def dev(x):
    return x.to("cuda")


@pytest.mark.parametrize("N,d,chunk,dt", [(1, 128, 128, I.BF16), (2, 64, 64, I.BF16), (17, 128, 64, I.BF16),
                                          (1, 64, 64, I.F32), (3, 128, 128, I.F32)])
def test_linear_prefill_shorter_than_a_chunk(N, d, chunk, dt):
    say("linear tiny", N, d, chunk, dt)
    B, H = 2, 3
    std = 1.0 / math.sqrt(d)
    x = I.linear_inputs(B, H, N, d, dt, 110, N, std)
    decay = torch.tensor([0.9, 1.0, 0.5])
    s0 = I.normal((B, H, d, d), 111, 1.0 / d, I.F32)
    o, st = sala.linear_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(decay), dev(s0), chunk=chunk)
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(decay), host64(s0))
    assert_close(o, ro, dt, "o")
    assert_close(st, rs, dt, "state")


def select_and_attend(B, Hq, Hkv, N, d, dt, topk):
    x = I.sparse_inputs(B, Hq, Hkv, N, d, dt, 112, N % 61, 1.0)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    idx, kp = sala.sparse_select(q, k, topk=topk)
    o = sala.sparse_prefill(q, k, v, idx)
    torch.cuda.synchronize()
    ridx, _, kbar = OS.sparse_select_prefill(host64(x["q"]), host64(x["k"]), 64, topk)
    assert np.array_equal(idx.cpu().numpy(), ridx), "indices"
    assert_close(kp, kbar, torch.float32, "k_pooled")
    ro = OS.sparse_attention_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), ridx, 64)
    assert_close(o, ro, dt, "o")
    return ridx


@pytest.mark.parametrize("N", [1, 5, 63, 64, 65, 64 * 3])
@pytest.mark.parametrize("dt,d", [(I.BF16, 128), (I.F32, 64)])
def test_sparse_prefill_within_the_first_blocks(N, dt, d):
    # no candidate block exists before block 3: every row is its forced
    # blocks only (block 0 and the local blocks), padded with -1
    say("sparse tiny", N, dt, d)
    ridx = select_and_attend(2, 4, 2, N, d, dt, topk=4)
    nqb = (N + 63) // 64
    for i in range(nqb):
        row = ridx[0, 0, i]
        assert list(row[row >= 0]) == list(range(i + 1))


@pytest.mark.parametrize("L", [1, 2, 64, 65, 64 * 3 + 1])
def test_sparse_decode_at_the_first_positions(L):
    say("decode tiny", L)
    B, Hq, Hkv, d, topk = 2, 8, 2, 128, 4
    kc = I.normal((B, Hkv, L, d), 113, 1.0, I.BF16)
    vc = I.normal((B, Hkv, L, d), 114, 1.0, I.BF16)
    q = I.normal((B, Hq, d), 115, 1.0, I.BF16)
    idx, kp = sala.sparse_select(dev(q[:, :, None]), dev(kc), topk=topk)
    o = sala.sparse_decode(dev(q), dev(kc), dev(vc), idx)
    torch.cuda.synchronize()
    kbar = np.stack([np.stack([OS.pool_blocks(host64(kc[b, h]), 64) for h in range(Hkv)]) for b in range(B)])
    assert_close(kp, kbar, torch.float32, "k_pooled")
    ridx, _ = OS.sparse_select_decode(host64(q), kbar, L, 64, topk)
    assert np.array_equal(idx[:, :, 0].cpu().numpy(), ridx), "indices"
    ro = OS.sparse_attention_decode(host64(q), host64(kc), host64(vc), ridx, L, 64)
    assert_close(o, ro, I.BF16, "o")


@pytest.mark.parametrize("dt,d", [(I.BF16, 128), (I.F32, 64)])
def test_linear_decode_from_an_empty_state(dt, d):
    # the first token of a sequence: S = k v^T, o = q . k v^T
    say("linear decode first token", dt, d)
    B, H = 2, 4
    x = I.linear_inputs(B, H, 1, d, dt, 116, 0, 1.0 / math.sqrt(d))
    state = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    o = sala.linear_decode(dev(x["q"][:, :, 0]), dev(x["k"][:, :, 0]), dev(x["v"][:, :, 0]), state, dev(torch.ones(H)))
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]))
    assert_close(o, ro[:, :, 0], dt, "o")
    assert_close(state, rs, dt, "state")
