"""The seeded input generator: determinism, shapes, and the shifted-block recipe (CPU only)."""

import math

import torch

from hybrid_sparse_linear_amd import inputs as I


def test_deterministic_and_rounded_once():
    a = I.normal((4, 5), 11, 0.5, I.BF16)
    b = I.normal((4, 5), 11, 0.5, I.BF16)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    x = I.normal((4, 5), 11, 0.5, I.F32)
    assert torch.equal(x.to(I.BF16).view(torch.int16), a.view(torch.int16))


def test_slope_decay_values():
    lam = I.slope_decay(32)
    assert abs(float(lam[0]) - math.exp(-2 ** -0.25)) < 1e-7
    assert abs(float(lam[31]) - math.exp(-2 ** -8)) < 1e-7
    assert torch.all(lam[1:] > lam[:-1])


def test_shifted_blocks_recipe():
    x = I.sparse_inputs(1, 4, 2, 64 * 40 + 5, 16, I.F32, 9, 0, 1.0, shift_frac=0.05)
    assert x["shifted_blocks"].numel() == 2  # floor(0.05 * 40)
    base = I.sparse_inputs(1, 4, 2, 64 * 40 + 5, 16, I.F32, 9, 0, 1.0)
    diff = (x["k"] - base["k"]).reshape(1, 2, -1, 16)
    for j in range(40):
        blk = diff[:, :, j * 64:(j + 1) * 64]
        if j in x["shifted_blocks"].tolist():
            assert abs(float(blk.norm(dim=-1).mean()) - 2.0) < 1e-5
        else:
            assert float(blk.abs().max()) == 0.0
