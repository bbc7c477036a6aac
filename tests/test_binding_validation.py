"""The Python binding checks every tensor's shape and dtype against the sizes
taken from its first argument before anything reaches the C ABI (which sees
only pointers).  These run on the CPU: a mismatch raises ValueError naming the
argument; a call whose tensors all match gets as far as the device check."""

import pytest
import torch

import hybrid_sparse_linear_amd as sala

BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_linear_prefill_checks():
    q = t(1, 2, 100, 128)
    raises("GPU", sala.linear_prefill, q, t(1, 2, 100, 128), t(1, 2, 100, 128))
    raises("k must have shape", sala.linear_prefill, q, t(1, 2, 99, 128), t(1, 2, 100, 128))
    raises("v must be", sala.linear_prefill, q, t(1, 2, 100, 128), t(1, 2, 100, 128, dtype=F32))
    raises("decay must have shape", sala.linear_prefill, q, q, q, t(3, dtype=F32))
    raises("decay must be", sala.linear_prefill, q, q, q, t(2))
    raises("state must have shape", sala.linear_prefill, q, q, q, None, t(1, 2, 128, 64, dtype=F32))
    raises("state_out must be", sala.linear_prefill, q, q, q, state_out=t(1, 2, 128, 128))
    raises("out must have shape", sala.linear_prefill, q, q, q, out=t(1, 2, 100, 64))
    raises("q must be a 4-d", sala.linear_prefill, t(2, 100, 128), q, q)


def test_linear_decode_checks():
    q = t(2, 4, 64)
    s = t(2, 4, 64, 64, dtype=F32)
    raises("GPU", sala.linear_decode, q, q, q, s)
    raises("state must have shape", sala.linear_decode, q, q, q, t(2, 4, 64, 128, dtype=F32))
    raises("state must be", sala.linear_decode, q, q, q, t(2, 4, 64, 64))
    raises("state must be given", sala.linear_decode, q, q, q, None)
    raises("k must have shape", sala.linear_decode, q, t(2, 3, 64), q, s)
    raises("decay must have shape", sala.linear_decode, q, q, q, s, t(2, dtype=F32))
    raises("out must be", sala.linear_decode, q, q, q, s, out=t(2, 4, 64, dtype=F32))
    raises("pos must have shape", sala.linear_decode_fused, q, q, q, s, pos=t(3, dtype=torch.int64))
    raises("gamma_q must have shape", sala.linear_decode_fused, q, q, q, s, gamma_q=t(128, dtype=F32))
    raises("gate must have shape", sala.linear_decode_fused, q, q, q, s, gate=t(2, 4, 65))


def test_fused_and_neighbour_checks():
    q = t(1, 2, 100, 128)
    raises("gate must be", sala.linear_prefill_fused, q, q, q, gate=t(1, 2, 100, 128, dtype=F32))
    raises("gamma_k must be", sala.linear_prefill_fused, q, q, q, gamma_k=t(128))
    raises("GPU", sala.linear_prefill_fused, q, q, q, gamma_q=t(128, dtype=F32))
    raises("gamma must have shape", sala.qk_norm_rope, q, gamma=t(64, dtype=F32))
    raises("out must have shape", sala.qk_norm_rope, q, out=t(1, 2, 100, 64))
    raises("gate must have shape", sala.output_gate, q, t(1, 2, 100, 64))
    raises("GPU", sala.output_gate, q, q)


def test_sparse_select_checks():
    q = t(1, 8, 640, 128)
    k = t(1, 2, 640, 128)
    raises("GPU", sala.sparse_select, q, k)
    raises("k must have shape", sala.sparse_select, q, t(2, 2, 640, 128))
    raises("k must be", sala.sparse_select, q, t(1, 2, 640, 128, dtype=F32))
    raises("k_pooled must have shape", sala.sparse_select, q, k, k_pooled=t(1, 2, 9, 128, dtype=F32))
    raises("k_pooled must be", sala.sparse_select, q, k, k_pooled=t(1, 2, 10, 128))
    raises("idx_out must have shape", sala.sparse_select, q, k, idx_out=t(1, 2, 10, 66, dtype=I32))
    raises("idx_out must be", sala.sparse_select, q, k, idx_out=t(1, 2, 10, 67, dtype=torch.int64))
    raises("all L", sala.sparse_select, t(1, 8, 639, 128), k)
    raises("L = 7 disagrees", sala.sparse_select, q, k, L=7)
    raises("k_pooled and L", sala.sparse_select, t(1, 8, 1, 128), None)
    qd = t(1, 8, 1, 128)
    raises("GPU", sala.sparse_select, qd, None, k_pooled=t(1, 2, 10, 128, dtype=F32), L=640)
    raises("k_pooled must have shape", sala.sparse_select, qd, None, k_pooled=t(1, 2, 11, 128, dtype=F32), L=640)
    raises("idx_out must have shape", sala.sparse_select, qd, k, idx_out=t(1, 2, 10, 67, dtype=I32))


def test_sparse_prefill_and_dense_checks():
    q = t(1, 8, 640, 128)
    k = t(1, 2, 640, 128)
    idx = t(1, 2, 10, 67, dtype=I32)
    raises("GPU", sala.sparse_prefill, q, k, k, idx)
    raises("v must have shape", sala.sparse_prefill, q, k, t(1, 2, 641, 128), idx)
    raises("k must be", sala.sparse_prefill, q, t(1, 2, 640, 128, dtype=F32), k, idx)
    raises("idx must have shape", sala.sparse_prefill, q, k, k, t(1, 2, 11, 67, dtype=I32))
    raises("idx must be an int32", sala.sparse_prefill, q, k, k, t(1, 2, 10, 67, dtype=torch.int64))
    raises("out must be", sala.sparse_prefill, q, k, k, idx, out=t(1, 8, 640, 128, dtype=F32))
    raises("GPU", sala.dense_prefill, q, k, k)
    raises("v must have shape", sala.dense_prefill, q, k, t(1, 2, 640, 64))


def test_sparse_decode_checks():
    q = t(2, 8, 128)
    kc = t(2, 2, 1000, 128)
    idx = t(2, 2, 67, dtype=I32)
    raises("GPU", sala.sparse_decode, q, kc, kc, idx)
    raises("v_cache must have shape", sala.sparse_decode, q, kc, t(2, 2, 999, 128), idx)
    raises("k_cache must be", sala.sparse_decode, q, t(2, 2, 1000, 128, dtype=F32), kc, idx)
    raises("idx must have shape", sala.sparse_decode, q, kc, kc, t(2, 1, 67, dtype=I32))
    raises("idx must have shape", sala.sparse_decode, q, kc, kc, t(2, 2, 2, 67, dtype=I32))
    raises("GPU", sala.sparse_decode, q, kc, kc, t(2, 2, 1, 67, dtype=I32))
    raises("L = 900 must equal", sala.sparse_decode, q, kc, kc, idx, L=900)
    raises("out must have shape", sala.sparse_decode, q, kc, kc, idx, out=t(2, 8, 64))


def test_generation_loop_checks():
    kc = t(1, 2, 640, 128)
    kp = t(1, 2, 10, 128, dtype=F32)
    q = t(1, 8, 128, 128)
    kn = t(1, 2, 128, 128)
    raises("GPU", sala.sparse_prefill_chunk, q, kn, kn, kc, kc, kp, 0)
    raises("k_pooled must have shape", sala.sparse_prefill_chunk, q, kn, kn, kc, kc, t(1, 2, 9, 128, dtype=F32), 0)
    raises("v_cache must be", sala.sparse_prefill_chunk, q, kn, kn, kc, t(1, 2, 640, 128, dtype=F32), kp, 0)
    raises("k_new must have shape", sala.sparse_prefill_chunk, q, t(1, 2, 127, 128), kn, kc, kc, kp, 0)
    raises("q must have the caches", sala.sparse_prefill_chunk, t(1, 8, 128, 128, dtype=F32), kn, kn, kc, kc, kp, 0)
    raises("idx_out must have shape", sala.sparse_prefill_chunk, q, kn, kn, kc, kc, kp, 0,
           idx_out=t(1, 2, 2, 66, dtype=I32))
    qd = t(1, 8, 128)
    kd = t(1, 2, 128)
    raises("GPU", sala.sparse_decode_step, qd, kd, kd, kc, kc, kp, 5)
    raises("v_new must have shape", sala.sparse_decode_step, qd, kd, t(1, 2, 64), kc, kc, kp, 5)
    raises("idx_out must be", sala.sparse_decode_step, qd, kd, kd, kc, kc, kp, 5, idx_out=t(1, 2, 67))
