"""Comparison helpers for the GPU parity tests.

Acceptance rule for floating-point outputs, tol = 1e-4 (fp32) or 2e-2 (bf16)
and REL_NORM = 1e-5 (fp32) or 1e-2 (bf16).  A "row" is one vector along the
last axis (one token's output, one state row, one pooled key); a "slice" is
every row of one (batch, head) for tensors of three or more dimensions, the
whole tensor otherwise.

  1. every element:  |g - r| <= tol * max(1, |r|)                (R16)
  2. every element:  |g - r| <= tol * max(|r|, rms(r_row), rms(r_slice))
  3. every row:      ||g - r|| / (sqrt(n) * s_row) <= REL_NORM
  4. every slice:    ||g - r|| / ||r|| <= REL_NORM
with s_row = max(rms(r_row), FLOOR * rms(r_slice)), FLOOR = 1/4 (bf16) or
1/16 (fp32).

Rule 1 alone is an absolute 0.02 wherever |r| < 1, which is most outputs at
the workloads' input scale (row RMS 0.01-0.3), so rules 2-4 hold every head
and every row to the dtype's relative bound: a 5 % error confined to one head
fails rule 4, and one confined to one row fails rule 3 in any row whose RMS is
above FLOOR/5 of its head's (1/20 for bf16).  The floor keeps a row whose true
value is nearly zero by cancellation (a decay-0 head's o_t = (q_t . k_t) v_t
with q_t . k_t near 0, measured down to 0.0014 of the head's RMS) from being
judged against its own vanishing scale: there the rounding of the summed
terms, not of the result, sets the error.  For bf16 that rounding is up to
2^-9 of each MFMA operand, on terms at about the head's RMS, so the floor times
REL_NORM must exceed 2^-9: 1/4 x 1e-2 > 2^-9 = 0.00195 (a CPU emulation that
rounds only P to bf16 exceeds the bound at FLOOR 1/16 on 2 of the 262144 rows
of a decay-0.43 head's dq at 256K, and reaches half of it at 1/4).  For fp32,
2^-24 is far below 1/16 x 1e-5.  bf16 operand rounding gives about 1e-3 to
6e-3 per row; a dropped term, a wrong decay exponent or a wrong index gives
1e-1 or more.

Block indices are compared bit-exactly, except rows whose float64 oracle
scores have a gap below NEAR_TIE = 1e-6 between the k-th and (k+1)-th
candidate: there several index sets are correct, and the GPU's picks are
accepted if no non-pick beats a pick by more than NEAR_TIE.

With SALA_PARITY_LOG set to a file path, every comparison appends one line
with its worst ratios (error over bound, 1 = at the bound) to that file.
"""

import os

import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
REL_NORM = {torch.float32: 1e-5, torch.bfloat16: 1e-2}
FLOOR = {torch.float32: 1.0 / 16.0, torch.bfloat16: 1.0 / 4.0}
NEAR_TIE = 1e-6


def host64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _rms(x, axis):
    return np.sqrt(np.mean(x * x, axis=axis))


def parity_stats(g, r, dtype):
    """Worst ratio to its bound of each rule (see the module docstring); <= 1 passes."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    tol, rn = TOL[dtype], REL_NORM[dtype]
    if r.ndim == 0:
        g, r = g.reshape(1), r.reshape(1)
    n = r.shape[-1]
    rows_r = r.reshape(-1, n)
    err = np.abs(g - r).reshape(-1, n)
    if r.ndim >= 3:
        lead = int(np.prod(r.shape[:-2]))
        slice_r = r.reshape(lead, -1)
        slice_e = (g - r).reshape(lead, -1)
        rows_per_slice = r.shape[-2]
    else:
        slice_r = r.reshape(1, -1)
        slice_e = (g - r).reshape(1, -1)
        rows_per_slice = rows_r.shape[0]
    slice_rms = _rms(slice_r, 1)
    s_row = np.maximum(_rms(rows_r, 1), FLOOR[dtype] * np.repeat(slice_rms, rows_per_slice))
    s_row = np.maximum(s_row, 1e-300)
    r1 = err / (tol * np.maximum(1.0, np.abs(rows_r)))
    slice_rms_row = np.maximum(np.repeat(slice_rms, rows_per_slice), 1e-300)
    r2 = err / (tol * np.maximum(np.abs(rows_r), np.maximum(_rms(rows_r, 1), slice_rms_row)[:, None]))
    r3 = np.sqrt(np.sum(err * err, axis=1)) / (np.sqrt(n) * s_row) / rn
    r4 = np.linalg.norm(slice_e, axis=1) / np.maximum(np.linalg.norm(slice_r, axis=1), 1e-300) / rn
    return {"elem_abs": float(r1.max()), "elem_slice": float(r2.max()), "row_norm": float(r3.max()),
            "slice_norm": float(r4.max()), "rows": int(rows_r.shape[0]),
            "bad_rows": int(((r1 > 1).any(axis=1) | (r2 > 1).any(axis=1) | (r3 > 1)).sum())}


def _log(what, dtype, st):
    path = os.environ.get("SALA_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(path, "a") as f:
        f.write(f"{test}\t{what}\t{str(dtype)[6:]}\t" + "\t".join(f"{k}={v:.3g}" if isinstance(v, float) else
                                                               f"{k}={v}" for k, v in st.items()) + "\n")


def assert_close(gpu, ref, dtype, what="", absolute_floor=True):
    """Rules 1-4 of the module docstring.  absolute_floor=False drops rule 1, for
    inputs far above the workloads' scale: there rule 1's floor of 1 is far below
    the output scale, and bf16 rounding of the MFMA operands alone exceeds it."""
    g = host64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output ({int((~np.isfinite(g)).sum())} elements)"
    st = parity_stats(g, r, dtype)
    if not absolute_floor:
        st["elem_abs_unchecked"] = st.pop("elem_abs")
    _log(what, dtype, st)
    err = np.abs(g - r)
    msg = (f"{what}: max abs err {err.max():.3e}; worst ratio to bound: elementwise (R16) "
           f"{st.get('elem_abs', st.get('elem_abs_unchecked')):.3f}{'' if absolute_floor else ' (not checked)'}, "
           f"elementwise vs row and slice scale {st['elem_slice']:.3f}, row norm {st['row_norm']:.3f}, "
           f"slice norm {st['slice_norm']:.3f}; {st['bad_rows']} of {st['rows']} rows out")
    assert max(st.get("elem_abs", 0.0), st["elem_slice"], st["row_norm"], st["slice_norm"]) <= 1.0, msg
    return st


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


class OnDevice:
    """A GPU tensor handed to an oracle function as a read-only array: indexing
    copies only the addressed elements to the host, widened to float64 (NumPy
    index arrays are moved to the tensor's device first).  Lets the oracle's
    own functions evaluate sampled rows of full-size inputs."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, key):
        key = key if isinstance(key, tuple) else (key,)
        key = tuple(torch.from_numpy(np.asarray(x)).to(self.t.device) if isinstance(x, np.ndarray) else x
                    for x in key)
        return host64(self.t[key])


def poisoned(shape, dtype, device="cuda"):
    """An output buffer filled with a value no kernel writes: NaN, or -123456789 for int32."""
    if dtype == torch.int32:
        return torch.full(tuple(shape), -123456789, dtype=dtype, device=device)
    return torch.full(tuple(shape), float("nan"), dtype=dtype, device=device)
