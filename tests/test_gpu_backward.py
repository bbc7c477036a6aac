"""GPU parity of the backward calls through the C ABI against the float64
oracle's gradients (oracle.backward): the linear layer (dq, dk, dv, d state_in)
over several chunks and segments with ragged tails, both head dims and chunk
sizes, decays 0, 1 and in between, with and without a carried state and a
state gradient, and at the 32-head 32K shape; sparse attention at a fixed
selection (dq, dk, dv) on GQA shapes with ragged tails and the workloads'
group size."""

import math

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_amd as sala
from hybrid_sparse_linear_amd import inputs as I
from oracle import backward as BW
from oracle import sparse as OS
from parity import OnDevice, assert_close, host64

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def dev(x):
    return None if x is None else x.to("cuda")


LIN_BWD_CASES = [
    # B, H, N, d, chunk, dtype, with_state, with_dstate
    (2, 3, 1000, 128, 128, I.BF16, True, True),     # ragged tail (one segment: see test_linear_backward_segments)
    (1, 2, 777, 128, 64, I.BF16, True, False),      # chunk 64
    (1, 2, 600, 64, 128, I.BF16, False, True),      # d 64
    (1, 3, 333, 64, 64, I.BF16, False, False),
    (2, 2, 100, 128, 128, I.BF16, True, True),      # one segment, one partial chunk
    (2, 3, 1000, 128, 64, I.BF16, True, True),      # chunk 64, d 128: dK and dV in one pass, ragged tail
    (2, 2, 100, 128, 64, I.BF16, True, True),       # the same pass over one partial chunk
    (1, 4, 2048, 64, 64, I.F32, True, True),        # the tiny workload's linear shape
    (1, 2, 517, 128, 128, I.F32, False, True),
]


@pytest.mark.parametrize("case", LIN_BWD_CASES,
                         ids=lambda c: f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}C{c[4]}{str(c[5])[6:]}"
                                       f"{'S' if c[6] else ''}{'G' if c[7] else ''}")
def test_linear_prefill_backward(case):
    B, H, N, d, chunk, dt, with_state, with_dstate = case
    say("linear_prefill_backward", case)
    std = 1.0 / math.sqrt(d)
    x = I.linear_inputs(B, H, N, d, dt, 110, N % 97, std)
    do = I.normal((B, H, N, d), 111, std, dt)
    decay = torch.tensor(([0.0, 1.0, 0.9, 0.43] * 4)[:H], dtype=torch.float32)
    s0 = I.normal((B, H, d, d), 112, 1.0 / d) if with_state else None
    ds = I.normal((B, H, d, d), 113, 1.0 / d) if with_dstate else None
    dq, dk, dv, dsi = sala.linear_prefill_backward(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(do), dev(decay),
                                                   dev(s0), dev(ds), chunk=chunk)
    torch.cuda.synchronize()
    r = BW.linear_prefill_backward(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(do),
                                   decay.double().numpy(), None if s0 is None else host64(s0),
                                   None if ds is None else host64(ds))
    assert_close(dq, r[0], dt, "dq")
    assert_close(dk, r[1], dt, "dk")
    assert_close(dv, r[2], dt, "dv")
    assert_close(dsi, r[3], torch.float32 if dt == I.F32 else I.BF16, "dstate_in")


@pytest.mark.parametrize("C", [128, 64])
def test_linear_backward_segments(C):
    """Gradients over 8525 tokens (chunk 128: two segments of 34 chunks, each
    aggregated in parts of 32 + 2 chunks; chunk 64, where dK and dV come from
    one pass: four segments of 34 chunks) with lam 0.99 (part 0 weighted
    0.99^256 in the scan at chunk 128) and 0.9 (part 0 left out), an initial
    state and a state gradient: every element against the oracle's chunked
    backward."""
    B, H, N, d = 1, 2, 8525, 128
    say("linear_prefill_backward segments", B, H, N, d, C)
    std = 1.0 / math.sqrt(d)
    x = I.linear_inputs(B, H, N, d, I.BF16, 116, 5, std)
    do = I.normal((B, H, N, d), 117, std, I.BF16)
    decay = torch.tensor([0.99, 0.9], dtype=torch.float32)
    s0 = I.normal((B, H, d, d), 118, 1.0 / d)
    ds = I.normal((B, H, d, d), 119, 1.0 / d)
    dq, dk, dv, dsi = sala.linear_prefill_backward(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(do), dev(decay),
                                                   dev(s0), dev(ds), chunk=C)
    torch.cuda.synchronize()
    r = BW.linear_prefill_backward(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(do),
                                   decay.double().numpy(), host64(s0), host64(ds), form="chunked", chunk=C)
    assert_close(dq, r[0], I.BF16, "dq")
    assert_close(dk, r[1], I.BF16, "dk")
    assert_close(dv, r[2], I.BF16, "dv")
    assert_close(dsi, r[3], I.BF16, "dstate_in")


def test_linear_backward_full_size_heads():
    """The 32-head 32K linear workload (slope decays 0.43 .. 0.996): every row of
    three heads against the oracle's chunked backward (pinned equal to the
    definition)."""
    N = 32768
    say("linear_prefill_backward 32K")
    x = I.workload2_linear(0, "cuda", N=N)
    do = I.normal((1, 32, N, 128), 114, 1.0 / math.sqrt(128), I.BF16, "cuda")
    dec = x["decay"]
    dq, dk, dv, dsi = sala.linear_prefill_backward(x["q"], x["k"], x["v"], do, dec.cuda())
    torch.cuda.synchronize()
    for h in (0, 13, 31):
        r = BW.linear_attention_backward_chunked(host64(x["q"][0, h]), host64(x["k"][0, h]), host64(x["v"][0, h]),
                                                 host64(do[0, h]), float(dec[h]), 128)
        assert_close(dq[0, h], r[0], I.BF16, f"dq head {h}")
        assert_close(dk[0, h], r[1], I.BF16, f"dk head {h}")
        assert_close(dv[0, h], r[2], I.BF16, f"dv head {h}")
        assert_close(dsi[0, h], r[3], I.BF16, f"dstate_in head {h}")


@pytest.mark.parametrize("C", [128, 64])
def test_linear_backward_256K_heads(C):
    """The linear layer at the group's 262144 tokens (32 heads, 8 segments of
    32768 tokens per head aggregated in parts, the aggregate passes leaving out
    keys below 2^-126 and whole parts before them; at chunk 64 dK and dV come
    from one pass): every row of the fastest- and the slowest-decaying head
    against the oracle's chunked backward."""
    N = 262144
    say("linear_prefill_backward 256K chunk", C)
    x = I.workload2_linear(0, "cuda", N=N)
    do = I.normal((1, 32, N, 128), 115, 1.0 / math.sqrt(128), I.BF16, "cuda")
    dec = x["decay"]
    dq, dk, dv, dsi = sala.linear_prefill_backward(x["q"], x["k"], x["v"], do, dec.cuda(), chunk=C)
    torch.cuda.synchronize()
    for h in (0, 31):
        r = BW.linear_attention_backward_chunked(host64(x["q"][0, h]), host64(x["k"][0, h]), host64(x["v"][0, h]),
                                                 host64(do[0, h]), float(dec[h]), 128)
        assert_close(dq[0, h], r[0], I.BF16, f"dq head {h}")
        assert_close(dk[0, h], r[1], I.BF16, f"dk head {h}")
        assert_close(dv[0, h], r[2], I.BF16, f"dv head {h}")
        assert_close(dsi[0, h], r[3], I.BF16, f"dstate_in head {h}")


SP_BWD_CASES = [
    # B, Hq, Hkv, N, d, topk
    (2, 8, 2, 64 * 20 + 17, 128, 8),     # ragged tail, G = 4 (two head pairs)
    (1, 16, 1, 64 * 14 + 33, 128, 5),    # G = 16, the workloads' group size
    (1, 4, 1, 64 * 20 + 64, 64, 3),      # d 64
    (1, 12, 2, 64 * 9 + 5, 128, 100),    # every block selected (dense causal), G = 6
    (1, 6, 2, 64 * 3 + 1, 128, 1),       # a block plus one token; G = 3 (an idle half pair)
]


def _sparse_bwd_case(case, seed):
    B, Hq, Hkv, N, d, topk = case
    x = I.sparse_inputs(B, Hq, Hkv, N, d, I.BF16, seed, N % 71, 1.0, shift_frac=0.05)
    do = I.normal((B, Hq, N, d), seed + 1, 1.0, I.BF16)
    ridx, _, _ = OS.sparse_select_prefill(host64(x["q"]), host64(x["k"]), 64, topk)
    return x, do, ridx


@pytest.mark.parametrize("case", SP_BWD_CASES, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}k{c[5]}")
def test_sparse_prefill_backward(case):
    """dq against every rule; dk and dv, each row a sum over every query row and
    head that selected its key (up to N * G terms, row RMS up to ~5 here), against
    the relative rules: the absolute floor of 1 in the elementwise rule lies below
    that scale, and an exact computation that rounds only P to bf16 (as the MFMA
    operand) already exceeds it on the G = 16 case (CPU emulation: the same worst
    ratio, 1.023, as the kernel)."""
    say("sparse_prefill_backward", case)
    x, do, ridx = _sparse_bwd_case(case, 120)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    idx = dev(torch.from_numpy(ridx).to(torch.int32))
    dq, dk, dv = sala.sparse_prefill_backward(q, k, v, idx, dev(do))
    torch.cuda.synchronize()
    r = BW.sparse_attention_backward(host64(x["q"]), host64(x["k"]), host64(x["v"]), ridx, host64(do), 64)
    assert_close(dq, r[0], I.BF16, "dq")
    assert_close(dk, r[1], I.BF16, "dk", absolute_floor=False)
    assert_close(dv, r[2], I.BF16, "dv", absolute_floor=False)


@pytest.mark.parametrize("scale", [-0.06, 0.0, 0.2], ids=["negative", "zero", "positive"])
def test_sparse_backward_custom_scale(scale):
    """A scale other than 1/sqrt(d): above zero the dQ pass folds the scale into
    its exponent arguments; zero and below take the scaled form (masked scores
    stay -inf); both against the oracle's gradients at that scale."""
    case = (1, 8, 2, 64 * 6 + 21, 128, 3)
    say("sparse_prefill_backward scale", scale, case)
    x, do, ridx = _sparse_bwd_case(case, 123)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    idx = dev(torch.from_numpy(ridx).to(torch.int32))
    dq, dk, dv = sala.sparse_prefill_backward(q, k, v, idx, dev(do), scale=scale)
    torch.cuda.synchronize()
    r = BW.sparse_attention_backward(host64(x["q"]), host64(x["k"]), host64(x["v"]), ridx, host64(do), 64,
                                     scale=scale)
    assert_close(dq, r[0], I.BF16, "dq")
    assert_close(dk, r[1], I.BF16, "dk", absolute_floor=False)
    assert_close(dv, r[2], I.BF16, "dv", absolute_floor=False)


def test_sparse_backward_repeats_bit_for_bit():
    """Every sum of the backward runs in a fixed order: two calls give the same bits."""
    case = (1, 16, 2, 64 * 30 + 9, 128, 6)
    say("sparse_prefill_backward twice", case)
    x, do, ridx = _sparse_bwd_case(case, 121)
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(do)
    idx = dev(torch.from_numpy(ridx).to(torch.int32))
    a = sala.sparse_prefill_backward(q, k, v, idx, do)
    b = sala.sparse_prefill_backward(q, k, v, idx, do)
    torch.cuda.synchronize()
    for x1, x2 in zip(a, b):
        assert torch.equal(x1, x2)


def test_sparse_backward_workload_shape():
    """The sparse workload's head group and input recipe (16 query heads on one KV
    head, top-64 + 1 + 2, 5 % shifted key blocks) at N = 4480, so query blocks
    past the 66th select 67 blocks, against the oracle's gradients; the GPU's
    selection is fed in (the selection tests check it against the oracle's)."""
    N = 64 * 70
    say("sparse_prefill_backward workload shape", N)
    x = I.sparse_inputs(1, 16, 1, N, 128, I.BF16, 3, 0, 1.0, shift_frac=0.05)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    do = I.normal((1, 16, N, 128), 122, 1.0, I.BF16)
    idx, _ = sala.sparse_select(q, k)
    dq, dk, dv = sala.sparse_prefill_backward(q, k, v, idx, dev(do))
    torch.cuda.synchronize()
    r = BW.sparse_attention_backward(host64(x["q"]), host64(x["k"]), host64(x["v"]), idx.cpu().numpy(), host64(do),
                                     64)
    assert_close(dq, r[0], I.BF16, "dq")
    assert_close(dk, r[1], I.BF16, "dk", absolute_floor=False)
    assert_close(dv, r[2], I.BF16, "dv", absolute_floor=False)


def test_sparse_backward_full_size_samples():
    """The sparse workload at 131072 tokens (32 query heads on 2 KV heads,
    top-64 + 1 + 2 over the GPU's selection, 5 % shifted key blocks): dq on
    sampled rows against the oracle's per-row gradient, and dk, dv of sampled
    key blocks -- blocks that few query blocks selected, whose sums the oracle
    forms one by one over those query blocks and every head of the group."""
    N = 131072
    say("sparse_prefill_backward 128K samples")
    x = I.workload3_sparse(0, "cuda", N=N)
    q, k, v = x["q"], x["k"], x["v"]
    do = I.normal(q.shape, 131, 1.0, I.BF16, "cuda")
    idx, _ = sala.sparse_select(q, k)
    dq, dk, dv = sala.sparse_prefill_backward(q, k, v, idx, do)
    torch.cuda.synchronize()
    ih = idx.cpu().numpy()
    rng = np.random.default_rng(6)
    rows = [(0, int(h), int(t)) for h, t in zip(rng.integers(0, 32, 24), rng.integers(0, N, 24))]
    rows += [(0, 0, 0), (0, 31, N - 1), (0, 17, 64 * 66 + 5)]
    ref = BW.sparse_attention_backward_dq_rows(OnDevice(q), OnDevice(k), OnDevice(v), ih, OnDevice(do), rows, 64)
    got = np.stack([host64(dq[b, h, t]) for b, h, t in rows])
    assert_close(got, ref, I.BF16, "dq rows")
    # key blocks selected by 2 to 6 query blocks (their own and the next one at least)
    nqb = N // 64
    blocks = []
    for kv in range(2):
        counts = np.zeros(nqb, dtype=int)
        for i in range(nqb):
            sel = ih[0, kv, i]
            sel = sel[sel >= 0]
            counts[sel[sel <= i]] += 1
        short = [j for j in range(1, nqb) if 2 <= counts[j] <= 6]
        blocks += [(0, kv, int(j)) for j in rng.choice(short, 2, replace=False)]
    say("key blocks", blocks)
    rk, rv = BW.sparse_attention_backward_kv_blocks(OnDevice(q), OnDevice(k), OnDevice(v), ih, OnDevice(do), blocks, 64)
    gk = np.stack([host64(dk[b, kv, 64 * j:64 * j + 64]) for b, kv, j in blocks])
    gv = np.stack([host64(dv[b, kv, 64 * j:64 * j + 64]) for b, kv, j in blocks])
    assert_close(gk, rk, I.BF16, "dk blocks")
    assert_close(gv, rv, I.BF16, "dv blocks")


@pytest.mark.parametrize("N", [1, 5, 64, 65])
@pytest.mark.parametrize("dt", [I.BF16, I.F32], ids=["bf16", "f32"])
def test_linear_backward_short_sequences(N, dt):
    """A single token, a few tokens, one full chunk and a chunk plus one token,
    with a carried state and a state gradient."""
    B, H, d = 1, 2, 64
    say("linear_prefill_backward short", N, dt)
    std = 1.0 / math.sqrt(d)
    x = I.linear_inputs(B, H, N, d, dt, 116, 0, std)
    do = I.normal((B, H, N, d), 117, std, dt)
    decay = torch.tensor([0.5, 1.0], dtype=torch.float32)
    s0 = I.normal((B, H, d, d), 118, 1.0 / d)
    ds = I.normal((B, H, d, d), 119, 1.0 / d)
    dq, dk, dv, dsi = sala.linear_prefill_backward(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(do), dev(decay),
                                                   dev(s0), dev(ds), chunk=64)
    torch.cuda.synchronize()
    r = BW.linear_prefill_backward(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(do),
                                   decay.double().numpy(), host64(s0), host64(ds))
    for name, g, ref in (("dq", dq, r[0]), ("dk", dk, r[1]), ("dv", dv, r[2])):
        assert_close(g, ref, dt, name)
    assert_close(dsi, r[3], torch.float32 if dt == I.F32 else I.BF16, "dstate_in")


@pytest.mark.parametrize("N", [1, 7, 64, 65])
def test_sparse_backward_short_sequences(N):
    """The first token alone (its query gets no gradient, its value gets dO),
    a few tokens inside the first block, one block, a block plus one token."""
    case = (1, 4, 2, N, 128, 3)
    say("sparse_prefill_backward short", case)
    x, do, ridx = _sparse_bwd_case(case, 123)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    idx = dev(torch.from_numpy(ridx).to(torch.int32))
    dq, dk, dv = sala.sparse_prefill_backward(q, k, v, idx, dev(do))
    torch.cuda.synchronize()
    r = BW.sparse_attention_backward(host64(x["q"]), host64(x["k"]), host64(x["v"]), ridx, host64(do), 64)
    assert_close(dq, r[0], I.BF16, "dq")
    assert_close(dk, r[1], I.BF16, "dk", absolute_floor=False)
    assert_close(dv, r[2], I.BF16, "dv", absolute_floor=False)
