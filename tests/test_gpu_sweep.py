"""Seeded sweep of small random shapes through every forward entry point
against the float64 oracle: batch 1-2, KV heads 1-3, group sizes 1-16, head
dim 64 or 128, sequence lengths 1-900 (ragged against chunks, blocks and
segments), top-k 0-9 with 0-2 initial and 0-3 local blocks, per-head decays
anywhere in [0, 1], with and without a carried state, bf16 and fp32.  Each
seed is one case; the run stops at the first failing case (pytest -x), whose
id names the seed and shape."""

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

SEEDS = range(24)


def draw(seed):
    rng = np.random.default_rng(7000 + seed)
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    c = dict(B=int(rng.integers(1, 3)), Hkv=Hkv, Hq=Hkv * G, d=int(rng.choice([64, 128])),
             N=int(rng.integers(1, 901)), dt=[I.BF16, I.F32][int(rng.integers(0, 2))],
             topk=int(rng.integers(0, 10)), n_init=int(rng.integers(0, 3)), n_local=int(rng.integers(1, 4)),
             chunk=int(rng.choice([64, 128])), state=bool(rng.integers(0, 2)))
    c["decay"] = rng.uniform(0.0, 1.0, c["Hq"]).round(3).astype(np.float32)
    return c


def name(seed):
    c = draw(seed)
    return (f"s{seed}-B{c['B']}Hq{c['Hq']}Hkv{c['Hkv']}N{c['N']}d{c['d']}{str(c['dt'])[6:]}"
            f"k{c['topk']}i{c['n_init']}l{c['n_local']}C{c['chunk']}{'S' if c['state'] else ''}")


@pytest.mark.parametrize("seed", SEEDS, ids=name)
def test_random_shape(seed):
    c = draw(seed)
    print("[case]", name(seed), flush=True)
    B, Hq, Hkv, N, d, dt = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["dt"]
    std = 1.0 / math.sqrt(d)

    # linear prefill (the fp32 path has no chunking) and one decode step after it
    x = I.linear_inputs(B, Hq, N + 1, d, dt, 300 + seed, 0, std)
    decay = torch.from_numpy(c["decay"])
    s0 = I.normal((B, Hq, d, d), 310 + seed, 1.0 / d) if c["state"] else None
    q, k, v = (x[n][:, :, :N].contiguous() for n in ("q", "k", "v"))
    o, st = sala.linear_prefill(q.cuda(), k.cuda(), v.cuda(), decay.cuda(), None if s0 is None else s0.cuda(),
                                chunk=c["chunk"])
    od = sala.linear_decode(x["q"][:, :, N].contiguous().cuda(), x["k"][:, :, N].contiguous().cuda(),
                            x["v"][:, :, N].contiguous().cuda(), st, decay.cuda())
    torch.cuda.synchronize()
    ro, rs = OL.linear_prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), decay.double().numpy(),
                               None if s0 is None else host64(s0))
    assert_close(o, ro[:, :, :N], dt, "linear o")
    assert_close(od, ro[:, :, N], dt, "linear decode o")
    assert_close(st, rs, torch.float32 if dt == I.F32 else I.BF16, "linear state after decode")

    # block selection and sparse prefill over the GPU's (validated) selection
    sp = I.sparse_inputs(B, Hq, Hkv, N, d, dt, 320 + seed, 0, 1.0, shift_frac=0.1)
    kw = dict(topk=c["topk"], n_init=c["n_init"], n_local=c["n_local"])
    qd, kd, vd = sp["q"].cuda(), sp["k"].cuda(), sp["v"].cuda()
    idx, kp = sala.sparse_select(qd, kd, **kw)
    osp = sala.sparse_prefill(qd, kd, vd, idx)
    # decode of the last token against the pooled cache
    idx1, _ = sala.sparse_select(qd[:, :, N - 1:N].contiguous(), None, k_pooled=kp, L=N, **kw)
    o1 = sala.sparse_decode(qd[:, :, N - 1].contiguous(), kd, vd, idx1)
    torch.cuda.synchronize()
    qh, kh, vh = host64(sp["q"]), host64(sp["k"]), host64(sp["v"])
    ridx, scores, kbar = OS.sparse_select_prefill(qh, kh, 64, **kw)
    assert_close(kp, kbar, torch.float32, "k_pooled")
    g = idx.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            cands = [OS.candidate_blocks(i, N, 64, c["n_init"], c["n_local"]) for i in range(ridx.shape[2])]
            nt = near_tie_rows(scores[b, h], cands, c["topk"])
            for i in range(ridx.shape[2]):
                check_idx_row(g[b, h, i], ridx[b, h, i], scores[b, h, i], cands[i],
                              sorted(OS.forced_blocks(i, c["n_init"], c["n_local"])), c["topk"], nt[i],
                              f"b{b} h{h} i{i}")
    assert_close(osp, OS.sparse_attention_prefill(qh, kh, vh, g, 64), dt, "sparse o")
    gi = idx1[:, :, 0].cpu().numpy()
    rdi, dsc = OS.sparse_select_decode(qh[:, :, N - 1], kbar, N, 64, **kw)
    i = (N - 1) // 64
    dc = OS.candidate_blocks(i, N, 64, c["n_init"], c["n_local"])
    for b in range(B):
        for h in range(Hkv):
            nt = near_tie_rows([dsc[b, h]], [dc], c["topk"])[0]
            check_idx_row(gi[b, h], rdi[b, h], dsc[b, h], dc, sorted(OS.forced_blocks(i, c["n_init"], c["n_local"])),
                          c["topk"], nt, f"decode b{b} h{h}")
    assert_close(o1, OS.sparse_attention_decode(qh[:, :, N - 1], kh, vh, gi, N, 64), dt, "sparse decode o")
