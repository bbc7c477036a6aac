"""Comparison helpers for the GPU parity tests.

Acceptance rule for floating-point outputs (fixed per dtype):
  every element: |gpu - ref| <= tol * max(1, |ref|), tol = 1e-4 (fp32), 2e-2 (bf16)
Because the synthetic inputs make many outputs much smaller than 1, the
tests also require the relative Frobenius error ||gpu - ref|| / ||ref|| to stay
below REL_NORM[dtype] (1e-5 fp32, 1e-2 bf16): bf16 rounding of the MFMA
operands gives about 3e-3, while a dropped term, wrong decay exponent or
wrong index shows up as 1e-1 or more.

Block indices are compared bit-exactly, except rows whose float64 oracle
scores have a gap below NEAR_TIE = 1e-6 between the k-th and (k+1)-th
candidate: there several index sets are correct, and the GPU's picks are
accepted if no non-pick beats a pick by more than NEAR_TIE.
"""

import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
REL_NORM = {torch.float32: 1e-5, torch.bfloat16: 1e-2}
NEAR_TIE = 1e-6


def host64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(gpu, ref, dtype, what=""):
    g = host64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    tol = TOL[dtype]
    err = np.abs(g - r)
    bound = tol * np.maximum(1.0, np.abs(r))
    bad = err > bound
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    msg = (f"{what}: max abs err {err.max():.3e}, max rel err "
           f"{(err / np.maximum(np.abs(r), 1e-3)).max():.3e}, rel-norm {rel:.3e}, {int(bad.sum())} elements out of tol")
    assert not bad.any(), msg
    assert rel <= REL_NORM[dtype], msg
    return rel


def near_tie_rows(scores_rows, cand_lists, k):
    """For each row: True if the k-th / (k+1)-th oracle scores are within NEAR_TIE."""
    out = []
    for s, cands in zip(scores_rows, cand_lists):
        if k <= 0 or len(cands) <= k:
            out.append(False)
            continue
        v = np.sort(np.asarray([s[j] for j in cands]))[::-1]
        out.append(bool(v[k - 1] - v[k] < NEAR_TIE))
    return out


def check_idx_row(gpu_row, ref_row, scores, cands, forced, k, near_tie, what=""):
    """Exact match, or (on a near-tie row) a valid top-k within NEAR_TIE."""
    g = [int(x) for x in gpu_row]
    r = [int(x) for x in ref_row]
    if g == r:
        return True
    assert near_tie, f"{what}: index mismatch on a non-tie row\n gpu {g}\n ref {r}"
    sel = [x for x in g if x >= 0]
    assert sel == sorted(set(sel)), f"{what}: not ascending/distinct"
    assert set(forced) <= set(sel), f"{what}: forced block missing"
    picks = [x for x in sel if x not in forced]
    assert len(picks) == min(k, len(cands)) and set(picks) <= set(cands), f"{what}: wrong pick count/range"
    rest = [x for x in cands if x not in picks]
    if rest:
        assert min(scores[x] for x in picks) >= max(scores[x] for x in rest) - NEAR_TIE, f"{what}: picks not a top-k"
    assert len(g) == len(r) and all(x == -1 for x in g[len(sel):])
    return False
