"""CPU checks of the acceptance rule in tests/parity.py: it must pass a
result carrying the error a correct bf16 kernel makes, and fail errors that
the looser whole-tensor rule let through -- a few percent confined to one
head or to one row, and a decay exponent off by one on one head.  The
mistakes are planted in float64 oracle output on the CPU."""

import math

import numpy as np
import pytest
import torch

from hybrid_sparse_linear_amd import inputs as I
from oracle import linear as OL
from oracle import sparse as OS
from parity import REL_NORM, TOL, parity_stats


def passes(g, r, dtype=torch.bfloat16):
    st = parity_stats(g, r, dtype)
    return max(st["elem_abs"], st["elem_slice"], st["row_norm"], st["slice_norm"]) <= 1.0


def old_rule_passes(g, r, dtype=torch.bfloat16):
    """The earlier rule: R16 elementwise plus one relative norm over the whole tensor."""
    err = np.abs(g - r)
    if (err > TOL[dtype] * np.maximum(1.0, np.abs(r))).any():
        return False
    return np.linalg.norm(g - r) / np.linalg.norm(r) <= REL_NORM[dtype]


def bf16_result(r, seed, rel=3e-3):
    """r with per-row relative noise of `rel` (the size of bf16 operand rounding in the
    kernels), rounded once to bf16 like a kernel's output."""
    rng = np.random.default_rng(seed)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    noisy = r + rel * rms * rng.standard_normal(r.shape)
    return torch.from_numpy(noisy).to(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module")
def linear_case():
    # the shapes and decays of the first bf16 linear parity case: B 2, H 3, N 1000, d 128
    B, H, N, d = 2, 3, 1000, 128
    x = I.linear_inputs(B, H, N, d, I.BF16, 90, N % 97, 1.0 / math.sqrt(d))
    decay = np.array([0.0, 1.0, 0.9])
    s0 = I.normal((B, H, d, d), 77, 1.0 / d)
    q, k, v = (x[n].double().numpy() for n in ("q", "k", "v"))
    ro, rs = OL.linear_prefill(q, k, v, decay, s0.double().numpy())
    return q, k, v, decay, s0.double().numpy(), ro, rs


def test_correct_bf16_error_passes(linear_case):
    *_, ro, rs = linear_case
    assert passes(bf16_result(ro, 1), ro)
    assert passes(bf16_result(rs, 2), rs)


@pytest.mark.parametrize("head", [0, 1, 2])
def test_five_percent_on_one_head_fails(linear_case, head):
    *_, ro, _ = linear_case
    g = bf16_result(ro, 3)
    g[1, head] *= 1.05
    assert not passes(g, ro)


def test_five_percent_on_one_row_fails(linear_case):
    *_, ro, _ = linear_case
    for b, h, t in [(0, 0, 17), (1, 1, 3), (1, 2, 999), (0, 1, 500)]:
        g = bf16_result(ro, 4)
        g[b, h, t] *= 1.05
        assert not passes(g, ro), (b, h, t)


def test_mutations_the_old_rule_missed(linear_case):
    q, k, v, decay, s0, ro, _ = linear_case
    # the decay-0 head scaled by 1.2
    g = bf16_result(ro, 5)
    g[:, 0] *= 1.2
    assert old_rule_passes(g, ro) and not passes(g, ro)
    # a decay exponent off by one on the 0.9 head: every weight lam^(t-s) becomes
    # lam^(t-s+1) (state term included), planted in the float64 definition
    bad = ro.copy()
    for b in range(2):
        o, _ = OL.linear_attention(q[b, 2], k[b, 2], v[b, 2], 0.9, s0[b, 2])
        bad[b, 2] = 0.9 * o
    assert not passes(bf16_result(bad, 6), ro)


def test_sparse_rows_and_sampled_rows():
    """Attention rows: one row of a prefill output, and one row of a sample of
    full-size rows (2-D), each carrying 5 % more than its value, fail."""
    x = I.sparse_inputs(1, 8, 2, 64 * 12 + 9, 128, I.BF16, 95, 1, 1.0, shift_frac=0.05)
    q, k, v = (x[n].double().numpy() for n in ("q", "k", "v"))
    idx, _, _ = OS.sparse_select_prefill(q, k, 64, 4)
    ro = OS.sparse_attention_prefill(q, k, v, idx, 64)
    assert passes(bf16_result(ro, 7), ro)
    g = bf16_result(ro, 7)
    g[0, 5, 700] *= 1.05            # a late row: attends to 7 blocks, small outputs
    assert not passes(g, ro)
    rows = ro[0, :, 640:650].reshape(-1, 128)
    assert passes(bf16_result(rows, 8), rows)
    g = bf16_result(rows, 8)
    g[13] *= 1.05
    assert not passes(g, rows)


def test_fp32_rule():
    rng = np.random.default_rng(9)
    r = rng.standard_normal((2, 3, 50, 64)) * 0.01
    g = r * (1 + 1e-7 * rng.standard_normal(r.shape))
    assert passes(g, r, torch.float32)
    g[1, 2, 7] *= 1 + 1e-4
    assert not passes(g, r, torch.float32)


def test_near_zero_row_judged_against_its_slice():
    """A row that is nearly zero by cancellation is held to FLOOR x the slice RMS,
    not to its own scale, so an fp32-accumulation-sized error there passes."""
    rng = np.random.default_rng(10)
    r = rng.standard_normal((1, 1, 100, 128))
    r[0, 0, 50] *= 1e-7
    g = r.copy()
    g[0, 0, 50] += 1e-7 * rng.standard_normal(128)
    g = torch.from_numpy(g).to(torch.bfloat16).double().numpy()
    assert passes(g, r)


def test_five_percent_on_one_element_fails(linear_case):
    """A single element 5 % off, where it is the largest of its row, fails."""
    *_, ro, _ = linear_case
    for b, h, t in [(0, 2, 400), (1, 1, 900)]:
        g = bf16_result(ro, 11)
        j = int(np.argmax(np.abs(ro[b, h, t])))
        g[b, h, t, j] = ro[b, h, t, j] * 1.05
        assert not passes(g, ro), (b, h, t)
