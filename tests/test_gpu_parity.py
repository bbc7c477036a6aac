"""GPU parity: every entry point through the C ABI against the float64 oracle,
at sizes the oracle finishes in seconds that span several tiles, chunks,
segments and a ragged tail, plus the degenerate cases of the method."""

import math

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_amd as sala
from hybrid_sparse_linear_amd import inputs as I
from oracle import linear as OL
from oracle import sparse as OS
from parity import assert_close, check_idx_row, host64, near_tie_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def dev(x):
    return None if x is None else x.to("cuda")


# ---------------------------------------------------------------- linear prefill

LIN_CASES = [
    # B, H, N, d, chunk, dtype, std, with_state.  bf16 cases use the workloads' input scale
    # (std 1/sqrt(d)): bf16 operand rounding errors scale with the summed terms, which at this
    # scale keeps the elementwise rule meaningful; the relative-norm check catches structure.
    (2, 3, 1000, 128, 128, I.BF16, 1.0 / math.sqrt(128), True),   # ragged tail (one segment: see LIN_SEG_CASES)
    (1, 2, 777, 128, 64, I.BF16, 1.0 / math.sqrt(128), True),     # chunk 64
    (1, 2, 600, 64, 128, I.BF16, 1.0 / 8.0, False),               # d 64
    (1, 3, 333, 64, 64, I.BF16, 1.0 / 8.0, True),
    (2, 2, 100, 128, 128, I.BF16, 1.0 / math.sqrt(128), True),    # one segment, one partial chunk
    (1, 4, 2048, 64, 64, I.F32, 1.0 / 8.0, False),               # tiny-group linear shape
    (1, 2, 517, 128, 128, I.F32, 0.5, True),
]


@pytest.mark.parametrize("case", LIN_CASES, ids=lambda c: f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}C{c[4]}{str(c[5])[6:]}")
def test_linear_prefill(case):
    B, H, N, d, chunk, dt, std, with_state = case
    say("linear_prefill", case)
    x = I.linear_inputs(B, H, N, d, dt, 90, N % 97, std)
    decay = torch.tensor(([0.0, 1.0, 0.9, 0.43] * 4)[:H], dtype=torch.float32)
    s0 = I.normal((B, H, d, d), 77, 1.0 / d) if with_state else None
    o, st = sala.linear_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(decay), dev(s0), chunk=chunk)
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), decay.double().numpy(),
                               None if s0 is None else host64(s0))
    assert_close(o, ro, dt, "o")
    assert_close(st, rs, torch.float32 if dt == I.F32 else I.BF16, "state")


# Sequences long enough for several segments (the bf16 plan keeps segments at
# least 32 chunks long) and for more than one aggregate part per segment (parts
# of at most 32 chunks, summed by the scan with weights lam^(segment end - part
# end)); the plans noted are the library's for these shapes.
LIN_SEG_CASES = [
    # B, H, N, d, chunk, decays
    # part 0's weight lam^(segment end - part end): 0.995^256 = 0.28 below; 0.95^64 = 0.04 and lam 1 next;
    # 0.999^256 = 0.77 last.  lam 0.9 and 0.3 leave part 0 out.
    (1, 2, 8525, 128, 128, (0.995, 0.9)),        # 2 segments of 34 chunks, parts of 32 + 2
    (1, 3, 10340, 128, 64, (1.0, 0.95, 0.3)),    # 5 segments of 33 chunks, parts of 32 + 1
    (2, 1, 4500, 64, 64, (0.999,)),              # d 64: 2 segments of 36 chunks, parts of 32 + 4
]


@pytest.mark.parametrize("case", LIN_SEG_CASES, ids=lambda c: f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}C{c[4]}")
def test_linear_prefill_segments_and_parts(case):
    B, H, N, d, C, decays = case
    say("linear_prefill segments and parts", case)
    x = I.linear_inputs(B, H, N, d, I.BF16, 96, N % 89, 1.0 / math.sqrt(d))
    decay = torch.tensor(decays, dtype=torch.float32)
    s0 = I.normal((B, H, d, d), 79, 1.0 / d)
    o, st = sala.linear_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(decay), dev(s0), chunk=C)
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), decay.double().numpy(), host64(s0),
                               form="chunked", chunk=C)
    assert_close(o, ro, I.BF16, "o")
    assert_close(st, rs, I.BF16, "state")


def test_linear_prefill_fast_decay_segments():
    """128 heads of 4133 tokens (chunk 64: two segments, the first in two
    aggregate parts) with decays from 0 to 1: the aggregate pass leaves out keys
    whose weight lam^n is below 2^-126 (and whole parts before them for lam <=
    0.43, none for lam >= 0.9), and every output row, head and final state must
    still match."""
    B, H, N, d, C = 4, 32, 4133, 128, 64
    say("linear_prefill fast decays", B, H, N, d, C)
    x = I.linear_inputs(B, H, N, d, I.BF16, 95, 3, 1.0 / math.sqrt(d))
    decay = torch.tensor(([0.0, 0.05, 0.2, 0.43, 0.6, 0.8, 0.85, 0.9, 0.95, 0.99, 0.999, 1.0] * 3)[:H],
                         dtype=torch.float32)
    s0 = I.normal((B, H, d, d), 78, 1.0 / d)
    o, st = sala.linear_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(decay), dev(s0), chunk=C)
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), decay.double().numpy(), host64(s0),
                               form="chunked", chunk=C)
    assert_close(o, ro, I.BF16, "o")
    assert_close(st, rs, I.BF16, "state")


def test_linear_prefill_large_inputs():
    """q, k, v ~ N(0, 0.25) -- four times the workloads' scale per factor -- over
    2085 tokens with lam = 1 (plain causal linear attention, outputs growing as
    sqrt(t)) and lam = 0.99, and a carried state: every row and every head held to
    the relative rules.  The absolute floor of 1 in the elementwise rule is
    below this output scale (row RMS up to ~60), where bf16 operand rounding alone
    gives absolute errors of ~0.3, so that one rule is not applied here."""
    B, H, N, d = 1, 2, 2085, 128
    say("linear_prefill large inputs", B, H, N, d)
    x = I.linear_inputs(B, H, N, d, I.BF16, 90, 7, 0.5)
    decay = torch.tensor([1.0, 0.99], dtype=torch.float32)
    s0 = I.normal((B, H, d, d), 76, 1.0)
    o, st = sala.linear_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(decay), dev(s0))
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), decay.double().numpy(), host64(s0))
    assert_close(o, ro, I.BF16, "o", absolute_floor=False)
    assert_close(st, rs, I.BF16, "state", absolute_floor=False)


def test_linear_prefill_state_alias_and_no_decay():
    say("linear_prefill alias")
    B, H, N, d = 1, 2, 700, 128
    x = I.linear_inputs(B, H, N, d, I.BF16, 91, 0, 1.0 / math.sqrt(d))
    s0 = I.normal((B, H, d, d), 78, 1.0 / d)
    sd = dev(s0.clone())
    o, st = sala.linear_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), None, sd, state_out=sd)
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), None, host64(s0))
    assert st.data_ptr() == sd.data_ptr()
    assert_close(o, ro, I.BF16, "o")
    assert_close(sd, rs, I.BF16, "state in place")


def test_linear_prefill_split_equals_whole_on_gpu():
    say("linear_prefill split")
    B, H, N1, N2, d = 1, 2, 640, 300, 128
    x = I.linear_inputs(B, H, N1 + N2, d, I.BF16, 92, 0, 1.0 / math.sqrt(d))
    decay = dev(torch.tensor([0.97, 0.999]))
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o1, s1 = sala.linear_prefill(q[:, :, :N1].contiguous(), k[:, :, :N1].contiguous(), v[:, :, :N1].contiguous(), decay)
    o2, s2 = sala.linear_prefill(q[:, :, N1:].contiguous(), k[:, :, N1:].contiguous(), v[:, :, N1:].contiguous(), decay,
                                 s1)
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), [0.97, 0.999])
    assert_close(torch.cat([o1, o2], dim=2), ro, I.BF16, "o split")
    assert_close(s2, rs, I.BF16, "state split")


# ---------------------------------------------------------------- linear decode

@pytest.mark.parametrize("dt,d", [(I.BF16, 128), (I.F32, 128), (I.BF16, 64), (I.F32, 64)])
def test_linear_decode(dt, d):
    say("linear_decode", dt, d)
    B, H = 3, 5
    x = I.linear_inputs(B, H, 1, d, dt, 93, d, 1.0 / math.sqrt(d))
    q, k, v = (x[n][:, :, 0].contiguous() for n in ("q", "k", "v"))
    s0 = I.normal((B, H, d, d), 79, 1.0 / d)
    decay = torch.tensor([0.0, 0.5, 0.9, 1.0, 0.99])
    sd = dev(s0.clone())
    o = sala.linear_decode(dev(q), dev(k), dev(v), sd, dev(decay))
    torch.cuda.synchronize()
    ro, rs = OL.linear_decode_batched(host64(q), host64(k), host64(v), host64(s0), decay.double().numpy())
    assert_close(o, ro, dt, "o")
    assert_close(sd, rs, torch.float32, "state")


def test_linear_decode_continues_prefill():
    say("linear decode after prefill")
    B, H, N, d = 1, 2, 513, 128
    x = I.linear_inputs(B, H, N + 1, d, I.BF16, 94, 0, 1.0 / math.sqrt(d))
    decay = dev(torch.tensor([0.95, 1.0]))
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    _, st = sala.linear_prefill(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(), v[:, :, :N].contiguous(), decay)
    o = sala.linear_decode(q[:, :, N].contiguous(), k[:, :, N].contiguous(), v[:, :, N].contiguous(), st, decay)
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), [0.95, 1.0])
    assert_close(o, ro[:, :, N], I.BF16, "decode row")
    assert_close(st, rs, I.BF16, "state")


# ---------------------------------------------------------------- sparse select

def oracle_select_check(idx_gpu, q, k, block, topk, n_init, n_local, what):
    ridx, scores, kbar = OS.sparse_select_prefill(host64(q), host64(k), block, topk, n_init, n_local)
    g = idx_gpu.cpu().numpy()
    B, Hkv, NQB, _ = ridx.shape
    N = q.shape[2]
    ties = 0
    for b in range(B):
        for h in range(Hkv):
            cand = [OS.candidate_blocks(i, N, block, n_init, n_local) for i in range(NQB)]
            nt = near_tie_rows(scores[b, h], cand, topk)
            for i in range(NQB):
                ok = check_idx_row(g[b, h, i], ridx[b, h, i], scores[b, h, i], cand[i],
                                   sorted(OS.forced_blocks(i, n_init, n_local)), topk, nt[i], f"{what} b{b} h{h} i{i}")
                ties += (not ok)
    return ridx, scores, kbar, ties


SEL_CASES = [
    # B, Hq, Hkv, N, d, dtype, topk, n_init, n_local, shift
    (2, 8, 2, 64 * 40 + 17, 128, I.BF16, 8, 1, 2, 0.05),
    (1, 4, 4, 2048, 64, I.F32, 4, 1, 2, 0.0),
    (1, 6, 2, 64 * 30, 128, I.BF16, 100, 1, 2, 0.0),     # k above every candidate count
    (1, 4, 1, 64 * 20 + 5, 64, I.BF16, 0, 1, 2, 0.0),     # k = 0: forced only
    (1, 4, 2, 64 * 25, 128, I.BF16, 5, 0, 0, 0.0),        # no forced blocks
    (1, 4, 2, 64 * 25 + 63, 128, I.F32, 3, 2, 3, 0.1),
    (1, 16, 1, 64 * 22 + 33, 128, I.BF16, 6, 1, 2, 0.05),  # G = 16, the workloads' group size
]


@pytest.mark.parametrize("case", SEL_CASES, ids=lambda c: f"Hq{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}k{c[6]}i{c[7]}l{c[8]}")
def test_sparse_select_prefill(case):
    B, Hq, Hkv, N, d, dt, topk, n_init, n_local, shift = case
    say("sparse_select", case)
    x = I.sparse_inputs(B, Hq, Hkv, N, d, dt, 95, N % 89, 1.0, shift_frac=shift)
    q, k = dev(x["q"]), dev(x["k"])
    idx, kp, sc = sala.sparse_select(q, k, topk=topk, n_init=n_init, n_local=n_local, return_scores=True)
    torch.cuda.synchronize()
    _, scores, kbar, _ = oracle_select_check(idx, x["q"], x["k"], 64, topk, n_init, n_local, "select")
    assert_close(kp, kbar, torch.float32, "k_pooled")
    # scores: compare every candidate entry
    g = host64(sc)
    nqb = scores.shape[2]
    for i in range(nqb):
        for j in OS.candidate_blocks(i, N, 64, n_init, n_local):
            assert abs(g[:, :, i, j] - scores[:, :, i, j]).max() <= 1e-5 * max(1.0, abs(scores[:, :, i, j]).max())


def test_sparse_select_without_scores_buffer_matches():
    say("sparse_select ws scores")
    x = I.sparse_inputs(1, 8, 2, 64 * 33, 128, I.BF16, 96, 0, 1.0, shift_frac=0.05)
    q, k = dev(x["q"]), dev(x["k"])
    a, _ = sala.sparse_select(q, k, topk=6)
    b, _, _ = sala.sparse_select(q, k, topk=6, return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    oracle_select_check(a, x["q"], x["k"], 64, 6, 1, 2, "select ws")


@pytest.mark.parametrize("L,dt,d,pooled_only", [(64 * 50 + 5, I.BF16, 128, False), (64 * 80, I.F32, 64, False),
                                                 (64 * 61 + 1, I.BF16, 128, True)])
def test_sparse_select_decode(L, dt, d, pooled_only):
    say("sparse_select decode", L, dt, d, pooled_only)
    B, Hq, Hkv, topk = 2, 8, 2, 8
    kc = I.normal((B, Hkv, L, d), 97, 1.0, dt)
    q = I.normal((B, Hq, 1, d), 98, 1.0, dt)
    kbar = np.stack([np.stack([OS.pool_blocks(host64(kc[b, h]), 64) for h in range(Hkv)]) for b in range(B)])
    if pooled_only:
        kp = dev(torch.from_numpy(kbar).float())
        idx, _ = sala.sparse_select(dev(q), None, k_pooled=kp, L=L, topk=topk)
    else:
        idx, kp = sala.sparse_select(dev(q), dev(kc), topk=topk)
    torch.cuda.synchronize()
    if not pooled_only:
        assert_close(kp, kbar, torch.float32, "k_pooled")
    kb_used = host64(kp)
    ridx, scores = OS.sparse_select_decode(host64(q[:, :, 0]), kb_used, L, 64, topk)
    i = (L - 1) // 64
    cands = OS.candidate_blocks(i, L, 64, 1, 2)
    g = idx.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            nt = near_tie_rows([scores[b, h]], [cands], topk)[0]
            check_idx_row(g[b, h, 0], ridx[b, h], scores[b, h], cands, sorted(OS.forced_blocks(i, 1, 2)), topk, nt,
                          f"decode b{b} h{h}")


@pytest.mark.parametrize("B,Hq,Hkv,L,d,topk", [(2, 8, 2, 64 * 300 + 7, 128, 100), (1, 2, 1, 64 * 32800 + 5, 64, 64)],
                         ids=["topk100", "NB32801"])
def test_sparse_select_decode_general_path(B, Hq, Hkv, L, d, topk):
    """Decode selection outside the two-level top-64 path: topk above 64, or
    more than 16384 pooled blocks (a cache past 1M tokens), where every score
    of the row is written and one workgroup ranks the row (past 16384
    candidates from global memory).  Exact against the oracle."""
    say("sparse_select decode, general path", B, Hq, Hkv, L, d, topk)
    NB = (L + 63) // 64
    kbar = I.normal((B, Hkv, NB, d), 133, 1.0, I.F32)
    q = I.normal((B, Hq, 1, d), 134, 1.0, I.BF16)
    idx, _ = sala.sparse_select(dev(q), None, k_pooled=dev(kbar), L=L, topk=topk)
    torch.cuda.synchronize()
    ridx, scores = OS.sparse_select_decode(host64(q[:, :, 0]), host64(kbar), L, 64, topk)
    i = (L - 1) // 64
    cands = OS.candidate_blocks(i, L, 64, 1, 2)
    g = idx.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            nt = near_tie_rows([scores[b, h]], [cands], topk)[0]
            check_idx_row(g[b, h, 0], ridx[b, h], scores[b, h], cands, sorted(OS.forced_blocks(i, 1, 2)), topk, nt,
                          f"decode b{b} h{h}")


@pytest.mark.parametrize("topk", [8, 100], ids=["top64_path", "general_path"])
def test_sparse_select_decode_group_of_64(topk):
    """Decode selection with 64 query heads per KV head (more than the 32 the
    top-64 path loads up front): the pooled query is the mean over all 64."""
    B, Hq, Hkv, d = 2, 128, 2, 128
    L = 64 * 300 + 7
    say("sparse_select decode G=64", topk)
    NB = (L + 63) // 64
    kbar = I.normal((B, Hkv, NB, d), 135, 1.0, I.F32)
    q = I.normal((B, Hq, 1, d), 136, 1.0, I.BF16)
    idx, _ = sala.sparse_select(dev(q), None, k_pooled=dev(kbar), L=L, topk=topk)
    torch.cuda.synchronize()
    ridx, scores = OS.sparse_select_decode(host64(q[:, :, 0]), host64(kbar), L, 64, topk)
    i = (L - 1) // 64
    cands = OS.candidate_blocks(i, L, 64, 1, 2)
    g = idx.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            nt = near_tie_rows([scores[b, h]], [cands], topk)[0]
            check_idx_row(g[b, h, 0], ridx[b, h], scores[b, h], cands, sorted(OS.forced_blocks(i, 1, 2)), topk, nt,
                          f"G64 b{b} h{h}")


def test_sparse_select_decode_many_chunks_reuses_workspace():
    """Decode selection over 1501 pooled blocks (several workgroups per row, a
    ragged last one), top-64: exact against the oracle, twice on one
    workspace with the same result."""
    say("sparse_select decode, 1501 blocks, workspace reuse")
    B, Hq, Hkv, d, topk = 2, 8, 2, 128, 64
    L = 64 * 1500 + 3
    NB = (L + 63) // 64
    kbar = I.normal((B, Hkv, NB, d), 131, 1.0, I.F32)
    q = I.normal((B, Hq, 1, d), 132, 1.0, I.BF16)
    nb = sala.workspace_bytes("sparse_select", dtype=1, B=B, Hq=Hq, Hkv=Hkv, d=d, Nq=1, L=L, block=64, topk=topk,
                              n_init=1, n_local=2)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    kp = dev(kbar)
    ridx, scores = OS.sparse_select_decode(host64(q[:, :, 0]), host64(kbar), L, 64, topk)
    i = (L - 1) // 64
    cands = OS.candidate_blocks(i, L, 64, 1, 2)
    first = None
    for call in range(2):
        idx, _ = sala.sparse_select(dev(q), None, k_pooled=kp, L=L, topk=topk, workspace=ws)
        torch.cuda.synchronize()
        g = idx.cpu().numpy()
        for b in range(B):
            for h in range(Hkv):
                nt = near_tie_rows([scores[b, h]], [cands], topk)[0]
                check_idx_row(g[b, h, 0], ridx[b, h], scores[b, h], cands, sorted(OS.forced_blocks(i, 1, 2)), topk,
                              nt, f"call {call} b{b} h{h}")
        if first is None:
            first = idx.clone()
        else:
            assert torch.equal(idx, first)


# ---------------------------------------------------------------- sparse prefill

ATT_CASES = [
    # B, Hq, Hkv, N, d, dtype, topk, std
    (2, 8, 2, 64 * 40 + 17, 128, I.BF16, 8, 1.0),
    (1, 12, 2, 64 * 24 + 30, 128, I.BF16, 4, 1.0),    # G = 6: a partly idle head group
    (1, 4, 1, 64 * 20 + 64, 64, I.BF16, 3, 1.0),
    (1, 4, 4, 2048, 64, I.F32, 4, 1.0 / 8.0),          # tiny-group sparse shape
    (1, 4, 2, 64 * 12 + 9, 128, I.F32, 2, 1.0),
    (1, 16, 1, 64 * 14 + 33, 128, I.BF16, 5, 1.0),    # G = 16: four full head groups per query block
]


@pytest.mark.parametrize("case", ATT_CASES, ids=lambda c: f"Hq{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}{str(c[5])[6:]}")
def test_sparse_prefill_with_oracle_idx(case):
    B, Hq, Hkv, N, d, dt, topk, std = case
    say("sparse_prefill", case)
    x = I.sparse_inputs(B, Hq, Hkv, N, d, dt, 99, N % 83, std, shift_frac=0.05)
    ridx, _, _ = OS.sparse_select_prefill(host64(x["q"]), host64(x["k"]), 64, topk)
    idx = dev(torch.from_numpy(ridx).to(torch.int32))
    o = sala.sparse_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), idx)
    torch.cuda.synchronize()
    ro = OS.sparse_attention_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), ridx, 64)
    assert_close(o, ro, dt, "o")


def test_sparse_prefill_all_blocks_is_dense_causal():
    say("sparse_prefill dense")
    B, Hq, Hkv, N, d = 1, 8, 2, 64 * 9 + 20, 128
    x = I.sparse_inputs(B, Hq, Hkv, N, d, I.BF16, 100, 0, 1.0)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    idx, _ = sala.sparse_select(q, k, topk=1000)
    o = sala.sparse_prefill(q, k, v, idx)
    torch.cuda.synchronize()
    ro = OS.dense_causal_attention(host64(x["q"]), host64(x["k"]), host64(x["v"]))
    assert_close(o, ro, I.BF16, "dense")


@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 8, 2, 64 * 10 + 17, 128), (2, 4, 1, 300, 64), (1, 12, 2, 64 * 6, 128)],
                         ids=["Hq8Hkv2N657d128", "B2Hq4Hkv1N300d64", "Hq12Hkv2N384d128"])
def test_dense_prefill(B, Hq, Hkv, N, d):
    """Dense causal attention (the full-attention comparison) against the
    oracle's textbook causal softmax; ragged tail, d 64 and 128, G = 4, 4, 6."""
    say("dense_prefill", B, Hq, Hkv, N, d)
    x = I.sparse_inputs(B, Hq, Hkv, N, d, I.BF16, 140, 0, 1.0)
    o = sala.dense_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]))
    torch.cuda.synchronize()
    ro = OS.dense_causal_attention(host64(x["q"]), host64(x["k"]), host64(x["v"]))
    assert_close(o, ro, I.BF16, "dense")


def test_dense_prefill_equals_sparse_with_every_block():
    """With every block 0..i selected, the sparse kernel visits the same blocks
    in the same order as the dense one: the outputs are bit-identical."""
    say("dense == sparse(all blocks)")
    B, Hq, Hkv, N, d = 1, 8, 2, 64 * 20 + 5, 128
    x = I.sparse_inputs(B, Hq, Hkv, N, d, I.BF16, 141, 0, 1.0)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    nqb = (N + 63) // 64
    row = torch.full((nqb, nqb), -1, dtype=torch.int32)
    for i in range(nqb):
        row[i, :i + 1] = torch.arange(i + 1, dtype=torch.int32)
    idx = dev(row.expand(B, Hkv, nqb, nqb).contiguous())
    o_sparse = sala.sparse_prefill(q, k, v, idx)
    o_dense = sala.dense_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o_sparse, o_dense)


def test_ceiling_microkernels():
    """The measured-ceiling microkernels run and the copy is exact."""
    say("ceilings")
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (1 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    sala.ceiling_copy(src, dst)
    out = torch.empty(64 * 512, dtype=torch.float32, device="cuda")
    sala.ceiling_mfma(64, 10, out)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_sparse_end_to_end_gpu_idx():
    say("sparse end to end")
    B, Hq, Hkv, N, d, topk = 1, 16, 2, 64 * 48 + 33, 128, 8
    x = I.sparse_inputs(B, Hq, Hkv, N, d, I.BF16, 101, 0, 1.0, shift_frac=0.05)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    idx, _ = sala.sparse_select(q, k, topk=topk)
    o = sala.sparse_prefill(q, k, v, idx)
    torch.cuda.synchronize()
    ridx, _, _, ties = oracle_select_check(idx, x["q"], x["k"], 64, topk, 1, 2, "e2e")
    # outputs with the GPU's own (validated) indices
    ro = OS.sparse_attention_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), idx.cpu().numpy(), 64)
    assert_close(o, ro, I.BF16, "o e2e")


# ---------------------------------------------------------------- sparse decode

@pytest.mark.parametrize("L,dt,d,G", [(64 * 50 + 5, I.BF16, 128, 4), (64 * 70, I.F32, 128, 16),
                                      (64 * 33 + 40, I.BF16, 64, 8), (100, I.BF16, 128, 2),
                                      (64 * 40 + 9, I.BF16, 128, 32)])  # G > 16: the vector-ALU split kernel
def test_sparse_decode(L, dt, d, G):
    say("sparse_decode", L, dt, d, G)
    B, Hkv, topk = 2, 2, 8
    Hq = G * Hkv
    kc = I.normal((B, Hkv, L, d), 102, 1.0, dt)
    vc = I.normal((B, Hkv, L, d), 103, 1.0, dt)
    q = I.normal((B, Hq, d), 104, 1.0, dt)
    kbar = np.stack([np.stack([OS.pool_blocks(host64(kc[b, h]), 64) for h in range(Hkv)]) for b in range(B)])
    ridx, _ = OS.sparse_select_decode(host64(q), kbar, L, 64, topk)
    idx = dev(torch.from_numpy(ridx).to(torch.int32))
    o = sala.sparse_decode(dev(q), dev(kc), dev(vc), idx)
    torch.cuda.synchronize()
    ro = OS.sparse_attention_decode(host64(q), host64(kc), host64(vc), ridx, L, 64)
    assert_close(o, ro, dt, "o")


def test_sparse_decode_equals_prefill_last_row():
    say("decode vs prefill")
    B, Hq, Hkv, d = 1, 8, 2, 128
    L = 64 * 30 + 1
    x = I.sparse_inputs(B, Hq, Hkv, L, d, I.BF16, 105, 0, 1.0)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    idx, kp = sala.sparse_select(q, k, topk=6)
    o = sala.sparse_prefill(q, k, v, idx)
    idx_d, _ = sala.sparse_select(q[:, :, -1:].contiguous(), None, k_pooled=kp, L=L, topk=6)
    od = sala.sparse_decode(q[:, :, -1].contiguous(), k, v, idx_d)
    torch.cuda.synchronize()
    assert torch.equal(idx_d[:, :, 0], idx[:, :, -1])
    assert_close(od, host64(o[:, :, -1]), I.BF16, "decode == prefill row")
