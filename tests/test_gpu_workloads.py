"""GPU parity at the benchmark workloads' full sizes, through the C ABI.

Where the oracle cannot evaluate every output in seconds, it checks a fixed
sample of outputs one by one (linear rows via the quadratic definition at
chosen positions, selection rows via pooled scores of chosen query blocks,
attention rows via the restricted softmax of chosen tokens), and the rest is
checked through properties that hold at any size (index structure).
Inputs are generated on the GPU by the seeded generator and copied to the
host only where the oracle reads them.
"""


import numpy as np
import pytest
import torch

import hybrid_sparse_linear_amd as sala
from hybrid_sparse_linear_amd import inputs as I
from oracle import linear as OL
from oracle import sparse as OS
from parity import OnDevice, assert_close, check_idx_row, host64, near_tie_rows, poisoned

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def idx_structure(idx, N, block, topk, n_init, n_local):
    """Every row: ascending, distinct, forced blocks present, candidate count, -1 padding."""
    g = idx.cpu().numpy()
    W = topk + n_init + n_local
    B, Hkv, NQB, _ = g.shape
    for i in range(NQB):
        sel = g[:, :, i]
        nc = len(OS.candidate_blocks(i, N, block, n_init, n_local))
        forced = sorted(OS.forced_blocks(i, n_init, n_local))
        n_exp = len(forced) + min(topk, nc)
        assert (sel[:, :, :n_exp] >= 0).all() and (sel[:, :, n_exp:] == -1).all(), f"row {i}: count"
        assert (np.diff(sel[:, :, :n_exp], axis=-1) > 0).all(), f"row {i}: not ascending"
        assert (sel[:, :, :n_exp] <= i).all(), f"row {i}: future block"
        for f in forced:
            assert (sel == f).any(axis=-1).all(), f"row {i}: forced block {f} missing"
    assert g.shape[-1] == W


def check_linear_rows(x, o, st, heads, rows, dt, state_heads=()):
    dec = x["decay"].double().numpy()
    for h in heads:
        q = host64(x["q"][0, h])
        k = host64(x["k"][0, h])
        v = host64(x["v"][0, h])
        ref = OL.linear_attention_rows(q, k, v, dec[h], rows)
        assert_close(o[0, h, rows], ref, dt, f"head {h} rows")
        if h in state_heads:
            assert_close(st[0, h], OL.final_state(k, v, dec[h]), dt, f"head {h} state")


def test_workload1_tiny_group_fp32():
    say("workload 1")
    outs = []
    for layer in range(3):
        x = I.workload1_linear(layer)
        o, st = sala.linear_prefill(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["decay"].cuda(), chunk=64)
        torch.cuda.synchronize()
        ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), x["decay"].double().numpy())
        assert_close(o, ro, I.F32, f"linear layer {layer}")
        assert_close(st, rs, I.F32, f"linear layer {layer} state")
    sp = I.workload1_sparse()
    q, k, v = sp["q"].cuda(), sp["k"].cuda(), sp["v"].cuda()
    idx, kp = sala.sparse_select(q, k, topk=4)
    o = sala.sparse_prefill(q, k, v, idx)
    torch.cuda.synchronize()
    ridx, scores, kbar = OS.sparse_select_prefill(host64(sp["q"]), host64(sp["k"]), 64, 4)
    g = idx.cpu().numpy()
    for h in range(4):
        cands = [OS.candidate_blocks(i, 2048, 64, 1, 2) for i in range(32)]
        nt = near_tie_rows(scores[0, h], cands, 4)
        for i in range(32):
            check_idx_row(g[0, h, i], ridx[0, h, i], scores[0, h, i], cands[i], sorted(OS.forced_blocks(i, 1, 2)), 4,
                          nt[i], f"h{h} i{i}")
    assert_close(kp, kbar, I.F32, "k_pooled")
    ro = OS.sparse_attention_prefill(host64(sp["q"]), host64(sp["k"]), host64(sp["v"]), g, 64)
    assert_close(o, ro, I.F32, "sparse layer")


def test_workload1_group_entry_point():
    """The group entry point (three linear layers, then selection and sparse
    attention on one stream) at the tiny fp32 workload, against the oracle."""
    say("workload 1 through layer_group_prefill")
    lin = [I.workload1_linear(layer) for layer in range(3)]
    sp = I.workload1_sparse()
    outs, o, idx = sala.layer_group_prefill([{n: x[n].cuda() for n in ("q", "k", "v", "decay")} for x in lin],
                                            {n: sp[n].cuda() for n in ("q", "k", "v")}, topk=4, chunk=64)
    torch.cuda.synchronize()
    for layer, (x, ol) in enumerate(zip(lin, outs)):
        ro, _ = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), x["decay"].double().numpy())
        assert_close(ol, ro, I.F32, f"group linear layer {layer}")
    ridx, scores, _ = OS.sparse_select_prefill(host64(sp["q"]), host64(sp["k"]), 64, 4)
    g = idx.cpu().numpy()
    for h in range(4):
        cands = [OS.candidate_blocks(i, 2048, 64, 1, 2) for i in range(32)]
        nt = near_tie_rows(scores[0, h], cands, 4)
        for i in range(32):
            check_idx_row(g[0, h, i], ridx[0, h, i], scores[0, h, i], cands[i], sorted(OS.forced_blocks(i, 1, 2)), 4,
                          nt[i], f"group h{h} i{i}")
    ro = OS.sparse_attention_prefill(host64(sp["q"]), host64(sp["k"]), host64(sp["v"]), g, 64)
    assert_close(o, ro, I.F32, "group sparse layer")


@pytest.mark.parametrize("N", [32768, 262144], ids=["workload2_32K", "workload4_linear_256K"])
def test_linear_prefill_full_size(N):
    say("linear full", N)
    workload = 2 if N == 32768 else 4
    x = I.workload2_linear(0, "cuda", N=N, workload=workload)
    x["decay"] = x["decay"]
    ws = torch.empty(max(1, sala.workspace_bytes("linear_prefill", dtype=1, B=1, H=32, N=N, d=128, chunk=128)),
                     dtype=torch.uint8, device="cuda")
    o, st = sala.linear_prefill(x["q"], x["k"], x["v"], x["decay"].cuda(), workspace=ws)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 127, 128, 129, 1000, N // 2 - 1, N // 2, N // 3, N - 129, N - 2, N - 1})
    heads = [0, 7, 31] if N > 32768 else [0, 5, 17, 31]
    check_linear_rows(x, o, st, heads, rows, I.BF16, state_heads=(0, 31))


def sparse_full_check(N, workload, n_rows=10, attn_rows_per_block=3):
    x = I.workload3_sparse(0 if workload == 3 else 3, "cuda", N=N, workload=workload)
    q, k, v = x["q"], x["k"], x["v"]
    Hq, Hkv, d = q.shape[1], k.shape[1], q.shape[3]
    nqb = N // 64
    ws_sel = poisoned((sala.workspace_bytes("sparse_select", dtype=1, B=1, Hq=Hq, Hkv=Hkv, d=d, Nq=N, L=N, block=64,
                                            topk=64, n_init=1, n_local=2) // 4,), torch.float32)
    idx = poisoned((1, Hkv, nqb, 67), torch.int32)
    kp = poisoned((1, Hkv, nqb, d), torch.float32)
    sala.sparse_select(q, k, k_pooled=kp, idx_out=idx, workspace=ws_sel)
    o = sala.sparse_prefill(q, k, v, idx)
    torch.cuda.synchronize()
    idx_structure(idx, N, 64, 64, 1, 2)
    g = idx.cpu().numpy()
    rng = np.random.default_rng(N)
    blocks = sorted({0, 1, 2, 65, 66, 67, nqb // 2, nqb - 1} | set(rng.integers(3, nqb, n_rows).tolist()))
    # the oracle's selection of the sampled query blocks, from the device tensors
    ridx, scores, kbar = OS.sparse_select_prefill_rows(OnDevice(q), OnDevice(k), blocks, 64, 64, 1, 2)
    ties = 0
    for h in range(Hkv):
        assert_close(kp[0, h], kbar[0, h], I.F32, f"k_pooled h{h}")
        for r, i in enumerate(blocks):
            cands = OS.candidate_blocks(i, N, 64, 1, 2)
            nt = near_tie_rows([scores[0, h, r]], [cands], 64)[0]
            ok = check_idx_row(g[0, h, i], ridx[0, h, r], scores[0, h, r], cands, sorted(OS.forced_blocks(i, 1, 2)),
                               64, nt, f"h{h} i{i}")
            ties += (not ok)
    # attention rows: the oracle's restricted softmax over the GPU's (validated) selection
    rows = [(0, hq, i * 64 + r) for i in blocks for hq in rng.choice(Hq, 2, replace=False).tolist()
            for r in rng.choice(64, attn_rows_per_block, replace=False).tolist()]
    ref = OS.sparse_attention_prefill_rows(OnDevice(q), OnDevice(k), OnDevice(v), g, rows, 64)
    got = np.stack([host64(o[b, hq, t]) for b, hq, t in rows])
    assert_close(got, ref, I.BF16, "attention rows")
    return ties


def test_workload3_sparse_full_size():
    say("workload 3")
    sparse_full_check(131072, 3)


def test_workload4_sparse_layer_256K():
    say("workload 4 sparse")
    sparse_full_check(262144, 4, n_rows=6, attn_rows_per_block=2)


def test_sparse_layer_1M_candidates_beyond_lds():
    """A 1M-token prefill: query blocks past 8194 have more candidate blocks
    (up to 16381) than the 8192 keys the selection holds in LDS, and rank them
    from the score rows in global memory; the sampled rows include the last
    block and, at random, others on both sides of that line."""
    say("sparse layer 1M")
    sparse_full_check(1048576, 4, n_rows=6, attn_rows_per_block=1)


def test_workload5_decode_1M():
    say("workload 5")
    lin, sp = I.workload5_decode("cuda")
    for layer, x in enumerate(lin):
        s0 = x["state"].clone()
        o = sala.linear_decode(x["q"], x["k"], x["v"], x["state"], x["decay"].cuda())
        torch.cuda.synchronize()
        ro, rs = OL.linear_decode_batched(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(s0),
                                          x["decay"].double().numpy())
        assert_close(o, ro, I.BF16, f"linear decode layer {layer}")
        assert_close(x["state"], rs, I.F32, f"linear decode state layer {layer}")
    L = sp["L"]
    q, kc, vc = sp["q"], sp["k_cache"], sp["v_cache"]
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    idx, kp = sala.sparse_select(q[:, :, None].contiguous(), kc)      # pooled cache built from the K cache
    idx2, _ = sala.sparse_select(q[:, :, None].contiguous(), None, k_pooled=kp, L=L)  # decode against the pooled cache
    o = sala.sparse_decode(q, kc, vc, idx2[:, :, 0].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    i = (L - 1) // 64
    cands = OS.candidate_blocks(i, L, 64, 1, 2)
    kbar = np.stack([np.stack([OS.pool_blocks(host64(kc[b, h]), 64) for h in range(Hkv)]) for b in range(B)])
    assert_close(kp, kbar, I.F32, "k_pooled")
    ridx, scores = OS.sparse_select_decode(host64(q), kbar, L, 64, 64, 1, 2)
    g = idx2[:, :, 0].cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            nt = near_tie_rows([scores[b, h]], [cands], 64)[0]
            check_idx_row(g[b, h], ridx[b, h], scores[b, h], cands, sorted(OS.forced_blocks(i, 1, 2)), 64, nt,
                          f"b{b} h{h}")
    # every head's output: the oracle's decode softmax over the GPU's (validated) selection
    ro = OS.sparse_attention_decode(host64(q), OnDevice(kc), OnDevice(vc), g, L, 64)
    assert_close(o, ro, I.BF16, "decode o")
