"""GPU checks of the sparse layer in a generation loop over a fixed-capacity KV
cache: chunked prefill (sala_sparse_prefill_chunk) then one-token decode steps
(sala_sparse_decode_step) crossing block boundaries.  Each chunk and step must
equal the one-shot entry points run on the same prefix bit for bit (indices,
outputs, pooled keys), and the float64 oracle on its prefix (indices exactly
or by the near-tie rule, outputs within the bf16 tolerance)."""

import math

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_amd as sala
from hybrid_sparse_linear_amd import inputs as I
from oracle import sparse as OS
from parity import assert_close, check_idx_row, host64, near_tie_rows, poisoned

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def _oracle_prefix_checks(q, k, v, L, rows_q, topk, n_init, n_local, o_rows, idx_rows, qb0, what):
    """Oracle selection of every query block of the prefix, compared on blocks qb0 ..;
    outputs of the given query rows."""
    qh, kh, vh = host64(q[:, :, :L]), host64(k[:, :, :L]), host64(v[:, :, :L])
    ridx, scores, _ = OS.sparse_select_prefill(qh, kh, 64, topk, n_init, n_local)
    B, Hkv = k.shape[0], k.shape[1]
    for b in range(B):
        for h in range(Hkv):
            for i in range(qb0, ridx.shape[2]):
                cands = OS.candidate_blocks(i, L, 64, n_init, n_local)
                forced = sorted(OS.forced_blocks(i, n_init, n_local))
                nt = near_tie_rows([scores[b, h, i]], [cands], topk)[0]
                check_idx_row(idx_rows[b, h, i - qb0].tolist(), ridx[b, h, i].tolist(), scores[b, h, i], cands,
                              forced, topk, nt, f"{what} b{b} h{h} block {i}")
    gi = idx_rows.cpu().numpy()
    full = np.full((B, Hkv, (L + 63) // 64, gi.shape[-1]), -1, dtype=np.int64)
    full[:, :, qb0:] = gi
    full[:, :, :qb0] = ridx[:, :, :qb0]
    ref = OS.sparse_attention_prefill_rows(qh, kh, vh, full, rows_q)
    got = np.stack([host64(o_rows[b, hq, t - qb0 * 64]) for b, hq, t in rows_q])
    assert_close(got, ref, I.BF16, f"{what} attention rows")


def test_chunked_prefill_then_decode_steps():
    B, Hq, Hkv, d = 2, 8, 2, 128
    topk, n_init, n_local = 3, 1, 2
    T = 64 * 8 + 5
    cap = 64 * 9 + 11
    say("generation loop", B, Hq, Hkv, d, T, cap)
    x = I.sparse_inputs(B, Hq, Hkv, T, d, I.BF16, 98, 0, 1.0, "cpu", shift_frac=0.3)
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    kc = torch.zeros((B, Hkv, cap, d), dtype=I.BF16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = poisoned((B, Hkv, (cap + 63) // 64, d), torch.float32)  # every block is pooled before it is read
    kw = dict(topk=topk, n_init=n_init, n_local=n_local)
    ws = torch.empty(max(sala.workspace_bytes("sparse_prefill_chunk", dtype=1, B=B, Hq=Hq, Hkv=Hkv, capacity=cap, d=d,
                                              n=256, block=64, **kw),
                         sala.workspace_bytes("sparse_decode_step", dtype=1, B=B, Hq=Hq, Hkv=Hkv, capacity=cap, d=d,
                                              block=64, **kw)), dtype=torch.uint8, device="cuda")
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    for pos0, n in [(0, 192), (192, 256)]:
        L = pos0 + n
        say("chunk", pos0, n)
        o, idx = sala.sparse_prefill_chunk(sl(q, pos0, L), sl(k, pos0, L), sl(v, pos0, L), kc, vc, kp, pos0,
                                           workspace=ws, **kw)
        idx_f, kp_f = sala.sparse_select(sl(q, 0, L), sl(k, 0, L), **kw)
        o_f = sala.sparse_prefill(sl(q, 0, L), sl(k, 0, L), sl(v, 0, L), idx_f)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_f[:, :, pos0 // 64:]), "chunk indices differ from the one-shot selection"
        assert torch.equal(o, o_f[:, :, pos0:L]), "chunk outputs differ from the one-shot prefill"
        assert torch.equal(kp[:, :, :L // 64], kp_f[:, :, :L // 64])
        assert torch.equal(kc[:, :, :L], k[:, :, :L]) and torch.equal(vc[:, :, :L], v[:, :, :L])
        rows = [(0, 0, pos0), (1, 5, L - 1), (0, 7, pos0 + n // 2), (1, 2, pos0 + 63)]
        _oracle_prefix_checks(q, k, v, L, rows, topk, n_init, n_local, o, idx, pos0 // 64, f"chunk {pos0}")
    for t in range(448, T):
        L = t + 1
        o, idx = sala.sparse_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                                         kc, vc, kp, t, workspace=ws, **kw)
        idx_f, _ = sala.sparse_select(q[:, :, t:t + 1].contiguous(), sl(k, 0, L), **kw)
        o_f = sala.sparse_decode(q[:, :, t].contiguous(), sl(k, 0, L), sl(v, 0, L), idx_f[:, :, 0].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_f[:, :, 0]), f"step {t}: indices"
        assert torch.equal(o, o_f), f"step {t}: output"
        if t in (448, 449, 511, 512, T - 1):
            say("decode step vs oracle", t)
            kh = host64(k[:, :, :L])
            kbar = np.stack([np.stack([OS.pool_blocks(kh[b, h], 64) for h in range(Hkv)]) for b in range(B)])
            ridx, sc = OS.sparse_select_decode(host64(q[:, :, t]), kbar, L, 64, topk, n_init, n_local)
            i = t // 64
            cands = OS.candidate_blocks(i, L, 64, n_init, n_local)
            forced = sorted(OS.forced_blocks(i, n_init, n_local))
            for b in range(B):
                for h in range(Hkv):
                    nt = near_tie_rows([sc[b, h]], [cands], topk)[0]
                    check_idx_row(idx[b, h].tolist(), ridx[b, h].tolist(), sc[b, h], cands, forced, topk, nt,
                                  f"step {t} b{b} h{h}")
            ro = OS.sparse_attention_decode(host64(q[:, :, t]), host64(k[:, :, :L]), host64(v[:, :, :L]),
                                            idx.cpu().numpy(), L)
            assert_close(o, ro, I.BF16, f"step {t}")
    # pooled keys after the loop: a full pooling of the whole sequence, bit for bit
    _, kp_full = sala.sparse_select(q[:, :, T - 1:T].contiguous(), k, **kw)
    torch.cuda.synchronize()
    nb = (T + 63) // 64
    assert torch.equal(kp[:, :, :nb], kp_full)
    assert torch.equal(kc[:, :, :T], k) and torch.equal(vc[:, :, :T], v)


def test_decode_step_at_1M_equals_plain_decode():
    B, Hq, Hkv, d, cap = 4, 32, 2, 128, 1048576
    pos = cap - 1
    say("decode step 1M", B, Hq, Hkv, d, cap)
    lin, sp = I.workload5_decode("cuda")
    del lin
    kc, vc, q = sp["k_cache"], sp["v_cache"], sp["q"]
    k_new = I.normal((B, Hkv, d), 99, 1.0, I.BF16, "cuda")
    v_new = I.normal((B, Hkv, d), 100, 1.0, I.BF16, "cuda")
    _, kp = sala.sparse_select(q[:, :, None].contiguous(), kc)  # pooled keys of the cache (its last row replaced next)
    o, idx = sala.sparse_decode_step(q, k_new, v_new, kc, vc, kp, pos)
    idx_f, kp_f = sala.sparse_select(q[:, :, None].contiguous(), kc)  # the cache now holds the new token
    o_f = sala.sparse_decode(q, kc, vc, idx_f[:, :, 0].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(kc[:, :, pos], k_new) and torch.equal(vc[:, :, pos], v_new)
    assert torch.equal(kp, kp_f)
    assert torch.equal(idx, idx_f[:, :, 0])
    assert torch.equal(o, o_f)


def test_generation_loop_fp32():
    B, Hq, Hkv, d = 1, 4, 2, 64
    topk, n_init, n_local = 2, 1, 1
    T, cap = 64 * 4 + 3, 64 * 5
    say("generation loop fp32", B, Hq, Hkv, d, T, cap)
    x = I.sparse_inputs(B, Hq, Hkv, T, d, I.F32, 98, 1, 1.0 / 8.0, "cpu", shift_frac=0.3)
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((B, Hkv, (cap + 63) // 64, d), dtype=torch.float32, device="cuda")
    kw = dict(topk=topk, n_init=n_init, n_local=n_local)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    o, idx = sala.sparse_prefill_chunk(sl(q, 0, 192), sl(k, 0, 192), sl(v, 0, 192), kc, vc, kp, 0, **kw)
    idx_f, _ = sala.sparse_select(sl(q, 0, 192), sl(k, 0, 192), **kw)
    o_f = sala.sparse_prefill(sl(q, 0, 192), sl(k, 0, 192), sl(v, 0, 192), idx_f)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_f) and torch.equal(o, o_f)
    qh, kh, vh = host64(q[:, :, :192]), host64(k[:, :, :192]), host64(v[:, :, :192])
    # attention over the GPU's selection (its indices equal the one-shot call's, which the
    # selection tests pin to the oracle)
    assert_close(o, OS.sparse_attention_prefill(qh, kh, vh, idx.cpu().numpy()), I.F32, "fp32 chunk vs oracle")
    for t in range(192, T):
        L = t + 1
        o, idx = sala.sparse_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                                         kc, vc, kp, t, **kw)
        idx_f, _ = sala.sparse_select(q[:, :, t:t + 1].contiguous(), sl(k, 0, L), **kw)
        o_f = sala.sparse_decode(q[:, :, t].contiguous(), sl(k, 0, L), sl(v, 0, L), idx_f[:, :, 0].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_f[:, :, 0]) and torch.equal(o, o_f), f"fp32 step {t}"
    ro = OS.sparse_attention_decode(host64(q[:, :, T - 1]), host64(k), host64(v), idx.cpu().numpy(), T)
    assert_close(o, ro, I.F32, "fp32 last step vs oracle")
