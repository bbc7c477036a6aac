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
from parity import assert_close, host64

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def dev(x):
    return None if x is None else x.to("cuda")


LIN_BWD_CASES = [
    # B, H, N, d, chunk, dtype, with_state, with_dstate
    (2, 3, 1000, 128, 128, I.BF16, True, True),     # 8 segments, ragged tail
    (1, 2, 777, 128, 64, I.BF16, True, False),      # chunk 64
    (1, 2, 600, 64, 128, I.BF16, False, True),      # d 64
    (1, 3, 333, 64, 64, I.BF16, False, False),
    (2, 2, 100, 128, 128, I.BF16, True, True),      # one segment, one partial chunk
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
