"""The allocation-free decode step (sala_sparse_decode_step_noalloc, whose
workspace is the library's fixed per-GPU scratch array) against the decode
step with a caller-owned workspace, through the C ABI: two calls in a row on
the same GPU, the second with a smaller input (fewer batch rows and heads, a
shorter cache, a smaller top-k).  Same kernels, so every output -- indices,
attention output, the appended cache rows and the re-pooled block -- must be
bit-identical, and within the bf16 rule of the parity tests."""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_amd as sala
from hybrid_sparse_linear_amd import inputs as I
from parity import assert_close, poisoned

pytestmark = pytest.mark.gpu

CALLS = [
    # B, Hq, Hkv, d, capacity, pos, topk
    (4, 32, 2, 128, 64 * 2000 + 37, 64 * 2000 + 36, 64),   # the 1M workload's heads, a 128K cache
    (2, 8, 2, 128, 64 * 40 + 3, 64 * 31 + 9, 16),          # smaller: fewer rows, heads and blocks
]


def _inputs(B, Hq, Hkv, d, cap, seed):
    kc = I.normal((B, Hkv, cap, d), seed, 1.0, I.BF16, "cuda")
    vc = I.normal((B, Hkv, cap, d), seed + 1, 1.0, I.BF16, "cuda")
    q = I.normal((B, Hq, d), seed + 2, 1.0, I.BF16, "cuda")
    kn = I.normal((B, Hkv, d), seed + 3, 1.0, I.BF16, "cuda")
    vn = I.normal((B, Hkv, d), seed + 4, 1.0, I.BF16, "cuda")
    return q, kn, vn, kc, vc


def test_noalloc_decode_step_matches_the_workspace_call():
    for n, (B, Hq, Hkv, d, cap, pos, topk) in enumerate(CALLS):
        print("[case] noalloc decode step", n, (B, Hq, Hkv, d, cap, pos, topk), flush=True)
        q, kn, vn, kc, vc = _inputs(B, Hq, Hkv, d, cap, 500 + 10 * n)
        _, kp = sala.sparse_select(q[:, :, None].contiguous(), kc, topk=topk)  # pooled keys of the cache
        kc2, vc2, kp2 = kc.clone(), vc.clone(), kp.clone()
        o_ref, idx_ref = sala.sparse_decode_step(q, kn, vn, kc, vc, kp, pos, topk=topk)
        o = poisoned(q.shape, q.dtype)
        idx = poisoned((B, Hkv, topk + 3), torch.int32)
        sala.sparse_decode_step_noalloc(q, kn, vn, kc2, vc2, kp2, pos, idx, o, topk=topk)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref), f"call {n}: indices"
        assert torch.equal(o, o_ref), f"call {n}: output"
        assert torch.equal(kc2, kc) and torch.equal(vc2, vc), f"call {n}: caches"
        assert torch.equal(kp2, kp), f"call {n}: pooled keys"
        assert_close(o, o_ref.double().cpu().numpy(), I.BF16, f"call {n} output")
        assert (idx.cpu().numpy() >= -1).all()
