"""GPU parity of the fused linear layer (QK RMS norm, rotate-half RoPE and the
output gate inside the linear-attention kernels) through the C ABI against
the float64 oracle (oracle.neighbours; bf16 layers with the transformed q and
k stored in bf16, as the kernels and an unfused producer keep them), on
ragged multi-chunk, multi-segment
shapes, with each neighbour alone and all together, at large positions, with
carried state, split prefills and decode steps, and at the 32-head 32K and
256K shapes on sampled rows."""

import math

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_amd as sala
from hybrid_sparse_linear_amd import inputs as I
from oracle import neighbours as NB
from parity import assert_close, host64

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def dev(x):
    return None if x is None else x.to("cuda")


DECAYS = [1.0, 0.9, 0.43, 0.99, 0.0, 0.97]

NB_CASES = [
    # B, H, N, d, chunk, pos0, norm_q, norm_k, rope, gate, with_state
    (1, 4, 293, 128, 128, 0, True, True, True, True, True),          # ragged tail
    (1, 2, 4500, 128, 64, 4096, True, True, True, True, True),       # 2 segments of 36 chunks, aggregate parts of 32 + 4
    (2, 2, 1000, 128, 128, 123456789, True, True, True, True, False),  # large positions
    (1, 3, 517, 128, 64, 77, True, False, True, False, True),         # chunk 64, k not normalised
    (1, 2, 600, 64, 128, 0, False, True, False, True, False),         # d 64, no RoPE
    (1, 2, 333, 64, 64, 4096, True, True, True, True, True),
    (1, 2, 130, 128, 128, 0, False, False, True, False, False),       # RoPE only, one segment
    (1, 2, 700, 128, 128, 0, False, False, False, True, True),        # gate only
    (1, 3, 1500, 128, 64, 0, False, False, False, True, True),        # gate only, chunk 64 (direct-load output pass)
    (1, 2, 900, 64, 128, 0, False, False, False, True, False),        # gate only, d 64 (direct-load output pass)
    (1, 2, 700, 64, 128, 55, True, True, True, True, True),          # d 64, chunk 128, all (direct-load, norm + RoPE in LDS)
]


def _case_inputs(B, H, N, d, seed):
    x = I.linear_inputs(B, H, N, d, I.BF16, 95, seed % 50, 1.0 / math.sqrt(d))
    nb = I.neighbour_inputs(B, H, N, d, 95, seed % 50)
    decay = torch.tensor((DECAYS * 2)[:H], dtype=torch.float32)
    return x, nb, decay


def _oracle(x, nb, decay, s0, norm_q, norm_k, rope, gate, pos0):
    return NB.linear_layer_fused(host64(x["q"]), host64(x["k"]), host64(x["v"]), decay.double().numpy(),
                                 None if s0 is None else host64(s0),
                                 host64(nb["gamma_q"]) if norm_q else None, host64(nb["gamma_k"]) if norm_k else None,
                                 1e-6, 10000.0 if rope else None, pos0, host64(nb["gate"]) if gate else None,
                                 store="bf16")


@pytest.mark.parametrize("case", NB_CASES, ids=lambda c: f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}C{c[4]}p{c[5]}"
                         f"{'Q' if c[6] else ''}{'K' if c[7] else ''}{'R' if c[8] else ''}{'G' if c[9] else ''}")
def test_fused_linear_prefill(case):
    B, H, N, d, chunk, pos0, norm_q, norm_k, rope, gate, with_state = case
    say("linear_prefill_fused", case)
    x, nb, decay = _case_inputs(B, H, N, d, N + pos0 % 1000)
    s0 = I.normal((B, H, d, d), 78, 1.0 / d) if with_state else None
    o, st = sala.linear_prefill_fused(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(decay), dev(s0),
                                      gamma_q=dev(nb["gamma_q"]) if norm_q else None,
                                      gamma_k=dev(nb["gamma_k"]) if norm_k else None, eps=1e-6,
                                      rope_base=10000.0 if rope else 0.0, pos0=pos0,
                                      gate=dev(nb["gate"]) if gate else None, chunk=chunk)
    torch.cuda.synchronize()
    ro, rs = _oracle(x, nb, decay, s0, norm_q, norm_k, rope, gate, pos0)
    assert_close(o, ro, I.BF16, "o")
    assert_close(st, rs, I.BF16, "state")


@pytest.mark.parametrize("N,d,chunk", [(1000, 128, 128), (333, 64, 64)])
def test_fused_with_nothing_enabled_is_bit_identical_to_plain(N, d, chunk):
    say("fused off == plain", N, d, chunk)
    x, _, decay = _case_inputs(1, 3, N, d, 5)
    s0 = I.normal((1, 3, d, d), 79, 1.0 / d)
    args = (dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(decay), dev(s0))
    o1, s1 = sala.linear_prefill(*args, chunk=chunk)
    o2, s2 = sala.linear_prefill_fused(*args, rope_base=0.0, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2)


def test_fused_split_prefill_and_decode_continue_the_sequence():
    B, H, N, d, n1 = 2, 4, 900, 128, 500
    say("fused split + decode", B, H, N, d, n1)
    x, nb, decay = _case_inputs(B, H, N + 1, d, 11)
    g = {k: dev(v) for k, v in nb.items()}
    q, k, v, gt = dev(x["q"]), dev(x["k"]), dev(x["v"]), g["gate"]
    kw = dict(gamma_q=g["gamma_q"], gamma_k=g["gamma_k"], eps=1e-6, rope_base=10000.0)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    o_all, s_all = sala.linear_prefill_fused(sl(q, 0, N), sl(k, 0, N), sl(v, 0, N), dev(decay), gate=sl(gt, 0, N), **kw)
    o1, s1 = sala.linear_prefill_fused(sl(q, 0, n1), sl(k, 0, n1), sl(v, 0, n1), dev(decay), gate=sl(gt, 0, n1), **kw)
    o2, s2 = sala.linear_prefill_fused(sl(q, n1, N), sl(k, n1, N), sl(v, n1, N), dev(decay), s1, pos0=n1,
                                       gate=sl(gt, n1, N), **kw)
    # decode of token N at position N from the state after N tokens
    state = s_all.clone()
    pos = torch.full((B,), N, dtype=torch.int64, device="cuda")
    od = sala.linear_decode_fused(q[:, :, N].contiguous(), k[:, :, N].contiguous(), v[:, :, N].contiguous(), state,
                                  dev(decay), pos=pos, gate=gt[:, :, N].contiguous(), **kw)
    torch.cuda.synchronize()
    ro, rs = NB.linear_layer_fused(host64(x["q"]), host64(x["k"]), host64(x["v"]), decay.double().numpy(), None,
                                   host64(nb["gamma_q"]), host64(nb["gamma_k"]), 1e-6, 10000.0, 0, host64(nb["gate"]),
                                   store="bf16")
    assert_close(o_all, ro[:, :, :N], I.BF16, "whole")
    assert_close(torch.cat([o1, o2], dim=2), ro[:, :, :N], I.BF16, "split")
    assert_close(s2, host64(s_all), I.BF16, "split state vs whole state")
    assert_close(od, ro[:, :, N], I.BF16, "decode row N")
    assert_close(state, rs, I.BF16, "decode state")


@pytest.mark.parametrize("dt", [I.BF16, I.F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [128, 64])
def test_fused_linear_decode(dt, d):
    B, H = 4, 6
    say("linear_decode_fused", dt, d)
    x = I.linear_inputs(B, H, 1, d, dt, 96, d, 1.0 / math.sqrt(d))
    nb = I.neighbour_inputs(B, H, 1, d, 96, d)
    gate = nb["gate"][:, :, 0].to(dt).contiguous()
    q, k, v = (x[t][:, :, 0].contiguous() for t in ("q", "k", "v"))
    s0 = I.normal((B, H, d, d), 80, 1.0 / d)
    decay = torch.tensor((DECAYS * 2)[:H], dtype=torch.float32)
    positions = [0, 7, 100003, 1048575]
    state = dev(s0)
    o = sala.linear_decode_fused(dev(q), dev(k), dev(v), state, dev(decay), gamma_q=dev(nb["gamma_q"]),
                                 gamma_k=dev(nb["gamma_k"]), eps=1e-6, rope_base=10000.0,
                                 pos=torch.tensor(positions, dtype=torch.int64, device="cuda"), gate=dev(gate))
    torch.cuda.synchronize()
    ro, rs = NB.linear_decode_fused(host64(q), host64(k), host64(v), host64(s0), decay.double().numpy(),
                                    host64(nb["gamma_q"]), host64(nb["gamma_k"]), 1e-6, 10000.0, positions,
                                    host64(gate), store="bf16" if dt == I.BF16 else None)
    assert_close(o, ro, dt, "o")
    assert_close(state, rs, dt, "state")


@pytest.mark.parametrize("N,chunk", [(32768, 128), (262144, 128), (32768, 64)], ids=["32K", "256K", "32K-c64"])
def test_fused_linear_full_size_rows(N, chunk):
    say("linear_prefill_fused full", N, chunk)
    x = I.workload2_linear(0, "cuda", N=N, workload=2 if N == 32768 else 4)
    nb = I.neighbour_inputs(1, 32, N, 128, 2 if N == 32768 else 4, 0, "cuda")
    ws = torch.empty(max(1, sala.workspace_bytes("linear_prefill", dtype=1, B=1, H=32, N=N, d=128, chunk=chunk)),
                     dtype=torch.uint8, device="cuda")
    o, st = sala.linear_prefill_fused(x["q"], x["k"], x["v"], x["decay"].cuda(), gamma_q=nb["gamma_q"],
                                      gamma_k=nb["gamma_k"], eps=1e-6, rope_base=10000.0, gate=nb["gate"],
                                      workspace=ws, chunk=chunk)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 127, 128, 1000, N // 2, N - 129, N - 1})
    dec = x["decay"].double().numpy()
    for h in ([0, 31] if N > 32768 else [0, 13, 31]):
        ref = NB.linear_layer_fused_rows(host64(x["q"][0, h]), host64(x["k"][0, h]), host64(x["v"][0, h]), dec[h],
                                         rows, None, host64(nb["gamma_q"]), host64(nb["gamma_k"]), 1e-6, 10000.0, 0,
                                         host64(nb["gate"][0, h]), store="bf16")
        assert_close(o[0, h, rows], ref, I.BF16, f"head {h} rows")


@pytest.mark.parametrize("dt", [I.BF16, I.F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("mode", ["norm+rope", "norm", "rope"])
def test_standalone_qk_norm_rope(dt, d, mode):
    B, H, N, pos0 = 2, 3, 333, 1000003
    say("qk_norm_rope", dt, d, mode)
    x = I.normal((B, H, N, d), 91, 1.0, dt)
    gamma = I.neighbour_inputs(1, 1, 1, d, 97, 0)["gamma_q"]
    norm, rope = "norm" in mode, "rope" in mode
    y = sala.qk_norm_rope(dev(x), gamma=dev(gamma) if norm else None, eps=1e-6,
                          rope_base=10000.0 if rope else 0.0, pos0=pos0)
    xi = dev(x)
    sala.qk_norm_rope(xi, gamma=dev(gamma) if norm else None, eps=1e-6, rope_base=10000.0 if rope else 0.0,
                      pos0=pos0, out=xi)  # in place
    torch.cuda.synchronize()
    ref = host64(x)
    if norm:
        ref = NB.rms_norm(ref, host64(gamma), 1e-6)
    if rope:
        ref = NB.rope(ref, np.arange(N, dtype=np.float64) + pos0)
    assert_close(y, ref, dt, "out")
    assert torch.equal(xi, y)


@pytest.mark.parametrize("dt", [I.BF16, I.F32], ids=["bf16", "f32"])
def test_standalone_output_gate(dt):
    say("output_gate", dt)
    o = I.normal((3, 5, 96), 92, 2.0, dt)
    g = I.normal((3, 5, 96), 93, 3.0, dt)
    r = sala.output_gate(dev(o), dev(g))
    torch.cuda.synchronize()
    assert_close(r, NB.output_gate(host64(o), host64(g)), dt, "gated")


def test_unfused_pipeline_matches_fused():
    B, H, N, d = 1, 4, 777, 128
    say("unfused vs fused", B, H, N, d)
    x, nb, decay = _case_inputs(B, H, N, d, 21)
    g = {k: dev(v) for k, v in nb.items()}
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    qh = sala.qk_norm_rope(q, gamma=g["gamma_q"], rope_base=10000.0, pos0=5)
    kh = sala.qk_norm_rope(k, gamma=g["gamma_k"], rope_base=10000.0, pos0=5)
    o, s = sala.linear_prefill(qh, kh, v, dev(decay))
    o = sala.output_gate(o, g["gate"])
    of, sf = sala.linear_prefill_fused(q, k, v, dev(decay), gamma_q=g["gamma_q"], gamma_k=g["gamma_k"],
                                       rope_base=10000.0, pos0=5, gate=g["gate"])
    torch.cuda.synchronize()
    ro, rs = _oracle(x, nb, decay, None, True, True, True, True, 5)
    assert_close(o, ro, I.BF16, "unfused")
    assert_close(of, ro, I.BF16, "fused")
    assert_close(s, rs, I.BF16, "unfused state")
