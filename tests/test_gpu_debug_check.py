"""The debug check of block-index rows (SALA_DEBUG_CHECK=1): rows that break
the contract of the gathering calls -- an entry beyond the blocks, a block
listed twice, a prefill row without its own query block -- are reported as an
error before any launch; valid rows pass, and with the variable unset nothing
is checked.  The kernels skip such entries either way (they never read
outside their buffers), so every call here is safe to run."""

import pytest
import torch

import hybrid_sparse_linear_amd as sala
from hybrid_sparse_linear_amd import inputs as I

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture
def check_on(monkeypatch):
    monkeypatch.setenv("SALA_DEBUG_CHECK", "1")


def _prefill_case():
    x = I.sparse_inputs(1, 4, 2, 64 * 9 + 5, 128, I.BF16, 11, 0, 1.0)
    q, k, v = x["q"].cuda(), x["k"].cuda(), x["v"].cuda()
    idx, _ = sala.sparse_select(q, k, topk=3)
    return q, k, v, idx


def test_valid_rows_pass(check_on):
    say("debug check: valid rows")
    q, k, v, idx = _prefill_case()
    sala.sparse_prefill(q, k, v, idx)
    do = torch.randn_like(q)
    sala.sparse_prefill_backward(q, k, v, idx, do)
    L = q.shape[2]
    i1, _ = sala.sparse_select(q[:, :, L - 1:L].contiguous(), k, topk=3)
    sala.sparse_decode(q[:, :, L - 1].contiguous(), k, v, i1)
    torch.cuda.synchronize()


@pytest.mark.parametrize("fault", ["beyond", "twice", "own"])
def test_bad_prefill_rows_are_reported(check_on, fault):
    say("debug check: prefill", fault)
    q, k, v, idx = _prefill_case()
    bad = idx.clone()
    nqb = idx.shape[2]
    if fault == "beyond":
        bad[0, 1, 5, 0] = nqb          # one past the last block
        want = "beyond"
    elif fault == "twice":
        bad[0, 0, 7, 1] = bad[0, 0, 7, 0]
        want = "twice"
    else:
        row = bad[0, 1, 4]
        row[row == 4] = -1             # the list now ends before block 4
        bad[0, 1, 4] = row
        want = "own query block"
    with pytest.raises(sala.SalaError, match=want):
        sala.sparse_prefill(q, k, v, bad)
    with pytest.raises(sala.SalaError, match=want):
        sala.sparse_prefill_backward(q, k, v, bad, torch.randn_like(q))
    torch.cuda.synchronize()


def test_bad_decode_rows_are_reported(check_on):
    say("debug check: decode")
    q, k, v, _ = _prefill_case()
    L = q.shape[2]
    i1, _ = sala.sparse_select(q[:, :, L - 1:L].contiguous(), k, topk=3)
    bad = i1.clone()
    bad[0, 0, 0, 2] = bad[0, 0, 0, 1]
    with pytest.raises(sala.SalaError, match="twice"):
        sala.sparse_decode(q[:, :, L - 1].contiguous(), k, v, bad)
    torch.cuda.synchronize()


def test_unset_means_unchecked(monkeypatch):
    say("debug check: off")
    monkeypatch.delenv("SALA_DEBUG_CHECK", raising=False)
    q, k, v, idx = _prefill_case()
    bad = idx.clone()
    bad[0, 0, 7, 1] = bad[0, 0, 7, 0]
    sala.sparse_prefill(q, k, v, bad)  # a block listed twice is attended twice; no error is raised
    torch.cuda.synchronize()
