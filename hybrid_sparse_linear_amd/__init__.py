"""libsala Python binding: the SALA hybrid attention layer group on MI355X.

Thin wrappers over the C ABI in ``include/sala.h``.  Each wrapper checks the
shape and dtype of every tensor it is given against the sizes taken from its
first argument (the C ABI sees only pointers, so a mismatched buffer would
otherwise become an out-of-bounds device access), then that every tensor is a
contiguous GPU tensor, allocates outputs and workspaces with torch when the
caller does not pass them, and calls the HIP library on torch's current
stream.  Every step of the computation runs in the HIP kernels; there is no
CPU or PyTorch fallback -- a missing ``libsala.so`` raises.

Entry points (same names as the C ABI, without the ``sala_`` prefix):
  linear_prefill   causal decayed linear attention over a sequence
  linear_prefill_backward  its gradients (dq, dk, dv, d state_in)
  linear_decode    one token of the same recurrence (state updated in place)
  sparse_select    pooled block scores and top-k block selection
  sparse_prefill   softmax attention over the selected blocks
  sparse_prefill_backward  its gradients (dq, dk, dv) at a fixed selection
  sparse_decode    one query token against the selected cached blocks
  dense_prefill    plain causal attention (the full-attention comparison)
  ceiling_mfma / ceiling_copy / ceiling_read   microkernels measuring this GPU's ceilings
  layer_group_prefill  three linear layers then one sparse layer, one stream

Debugging: with the environment variable SALA_DEBUG_POISON=1, every output,
index array and workspace the wrappers allocate is filled first (NaN for
float tensors, -123456789 for int32, 0xFF bytes for workspaces), so an
element a kernel fails to write shows up in a comparison.
"""

import ctypes
import math
import os

import torch

from ._lib import SALA_BF16, SALA_F32, SalaError, call, lib  # noqa: F401

__all__ = ["linear_prefill", "linear_prefill_backward", "linear_decode", "linear_prefill_fused", "linear_decode_fused", "qk_norm_rope",
           "output_gate", "sparse_prefill_chunk", "sparse_decode_step", "sparse_decode_step_noalloc", "sparse_select",
           "sparse_prefill", "sparse_prefill_backward", "sparse_decode",
           "dense_prefill", "layer_group_prefill", "workspace_bytes", "ceiling_mfma", "ceiling_copy", "ceiling_read", "SalaError"]

POISON_INT32 = -123456789


def _code(t):
    if t.dtype == torch.float32:
        return SALA_F32
    if t.dtype == torch.bfloat16:
        return SALA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return ctypes.c_void_p(0) if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _poisoning():
    return os.environ.get("SALA_DEBUG_POISON", "") == "1"


def _poison(t):
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    elif t.dtype == torch.int32:
        t.fill_(POISON_INT32)
    else:
        t.fill_(0xFF)
    return t


def _empty(shape, dtype, device):
    t = torch.empty(tuple(shape), dtype=dtype, device=device)
    return _poison(t) if _poisoning() else t


def _empty_like(x):
    return _empty(x.shape, x.dtype, x.device)


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libsala tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("libsala tensors must be contiguous")


def _want(t, name, shape, dtype):
    """t is None, or has exactly `shape` and `dtype`."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _dims(t, name, ndim):
    if not isinstance(t, torch.Tensor) or t.dim() != ndim:
        raise ValueError(f"{name} must be a {ndim}-d tensor")
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"{name} must be float32 or bfloat16, got {t.dtype}")
    return tuple(t.shape)


def _ws(nbytes, ws, like):
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return _empty((nbytes,), torch.uint8, like.device)


# operation codes of sala_workspace_bytes and the integer arguments it takes for each, in order
_WS_OPS = {
    "linear_prefill": (0, ("dtype", "B", "H", "N", "d", "chunk")),
    "sparse_select": (1, ("dtype", "B", "Hq", "Hkv", "d", "Nq", "L", "block", "topk", "n_init", "n_local")),
    "sparse_prefill": (2, ("dtype", "B", "Hq", "Hkv", "N", "d", "block", "n_sel")),
    "sparse_decode": (3, ("dtype", "B", "Hq", "Hkv", "L", "d", "block", "n_sel")),
    "sparse_prefill_chunk": (4, ("dtype", "B", "Hq", "Hkv", "capacity", "d", "n", "block", "topk", "n_init",
                                 "n_local")),
    "sparse_decode_step": (5, ("dtype", "B", "Hq", "Hkv", "capacity", "d", "block", "topk", "n_init", "n_local")),
    "sparse_prefill_backward": (6, ("dtype", "B", "Hq", "Hkv", "N", "d", "block", "n_sel")),
}


def workspace_bytes(op, **kw):
    """Workspace size in bytes of an entry point for the given arguments (sala_workspace_bytes)."""
    if op not in _WS_OPS:
        raise ValueError(f"unknown operation {op!r}")
    code, names = _WS_OPS[op]
    dims = (ctypes.c_int64 * len(names))(*[int(kw[n]) for n in names])
    nb = lib().sala_workspace_bytes(code, dims, len(names))
    if nb == ctypes.c_size_t(-1).value:
        raise SalaError("sala_workspace_bytes", -1, lib().sala_last_error().decode())
    return nb


def _check_linear(q, k, v, decay, state, out, state_out):
    B, H, N, d = _dims(q, "q", 4)
    _want(k, "k", q.shape, q.dtype)
    _want(v, "v", q.shape, q.dtype)
    _want(out, "out", q.shape, q.dtype)
    _want(decay, "decay", (H,), torch.float32)
    _want(state, "state", (B, H, d, d), torch.float32)
    _want(state_out, "state_out", (B, H, d, d), torch.float32)
    return B, H, N, d


def _check_gammas(d, gamma_q, gamma_k):
    _want(gamma_q, "gamma_q", (d,), torch.float32)
    _want(gamma_k, "gamma_k", (d,), torch.float32)


def linear_prefill(q, k, v, decay=None, state=None, *, chunk=None, out=None, state_out=None, workspace=None,
                   want_state=True):
    """o, S_out = causal linear attention of q, k, v [B, H, N, d] with per-head decay [H] (fp32).

    state: optional [B, H, d, d] fp32 carried state S[d_k][d_v].  Returns (o, S_out or None).
    """
    B, H, N, d = _check_linear(q, k, v, decay, state, out, state_out)
    _dev(q, k, v, decay, state, out, state_out, workspace)
    chunk = chunk or (64 if d == 64 else 128)
    dt = _code(q)
    o = _empty_like(q) if out is None else out
    so = state_out
    if so is None and want_state:
        so = _empty((B, H, d, d), torch.float32, q.device)
    nb = workspace_bytes("linear_prefill", dtype=dt, B=B, H=H, N=N, d=d, chunk=chunk)
    ws = _ws(nb, workspace, q)
    call("sala_linear_prefill", dt, B, H, N, d, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(decay), _ptr(state),
         _ptr(so), _ptr(ws), nb, _stream())
    return o, so


def linear_prefill_backward(q, k, v, dout, decay=None, state=None, dstate_out=None, *, chunk=None, dq=None, dk=None,
                            dv=None, want_dstate=True, workspace=None):
    """Gradients of linear_prefill(q, k, v, decay, state) for dL/do = dout [B, H, N, d] and
    dL/dS_out = dstate_out ([B, H, d, d] fp32 or None).  Returns (dq, dk, dv, dstate_in or None).
    chunk: the tile of the chunked form (64 or 128; the gradients do not depend on it beyond
    rounding); 64 by default, where dK and dV come from one pass at d = 128."""
    B, H, N, d = _check_linear(q, k, v, decay, state, None, None)
    _want(dout, "dout", q.shape, q.dtype)
    _want(dstate_out, "dstate_out", (B, H, d, d), torch.float32)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _want(t, name, q.shape, q.dtype)
    _dev(q, k, v, dout, decay, state, dstate_out, dq, dk, dv, workspace)
    chunk = chunk or 64
    dt = _code(q)
    dq = _empty_like(q) if dq is None else dq
    dk = _empty_like(q) if dk is None else dk
    dv = _empty_like(q) if dv is None else dv
    dsi = _empty((B, H, d, d), torch.float32, q.device) if want_dstate else None
    nb = workspace_bytes("linear_prefill", dtype=dt, B=B, H=H, N=N, d=d, chunk=chunk)
    ws = _ws(nb, workspace, q)
    call("sala_linear_prefill_backward", dt, B, H, N, d, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(decay),
         _ptr(state), _ptr(dstate_out), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsi), _ptr(ws), nb, _stream())
    return dq, dk, dv, dsi


def linear_decode(q, k, v, state, decay=None, *, out=None):
    """One decode token: state [B, H, d, d] fp32 is updated in place; returns o [B, H, d]."""
    B, H, d = _dims(q, "q", 3)
    _want(k, "k", q.shape, q.dtype)
    _want(v, "v", q.shape, q.dtype)
    _want(out, "out", q.shape, q.dtype)
    if state is None:
        raise ValueError("state must be given (it is updated in place)")
    _want(state, "state", (B, H, d, d), torch.float32)
    _want(decay, "decay", (H,), torch.float32)
    _dev(q, k, v, state, decay, out)
    o = _empty_like(q) if out is None else out
    call("sala_linear_decode", _code(q), B, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(decay), _ptr(state),
         _stream())
    return o


def linear_prefill_fused(q, k, v, decay=None, state=None, *, gamma_q=None, gamma_k=None, eps=1e-6,
                         rope_base=10000.0, pos0=0, gate=None, chunk=None, out=None, state_out=None,
                         workspace=None, want_state=True):
    """The linear layer with QK RMS norm, rotate-half RoPE (positions pos0 ..) and the
    output gate o * sigmoid(gate) applied inside its kernels (bf16).

    gamma_q, gamma_k: [d] fp32 or None; rope_base 0 / None = no RoPE; gate: like q or None.
    Returns (o, S_out or None) as linear_prefill.
    """
    B, H, N, d = _check_linear(q, k, v, decay, state, out, state_out)
    _want(gate, "gate", q.shape, q.dtype)
    _check_gammas(d, gamma_q, gamma_k)
    _dev(q, k, v, decay, state, out, state_out, gamma_q, gamma_k, gate, workspace)
    chunk = chunk or (64 if d == 64 else 128)
    dt = _code(q)
    o = _empty_like(q) if out is None else out
    so = state_out
    if so is None and want_state:
        so = _empty((B, H, d, d), torch.float32, q.device)
    nb = workspace_bytes("linear_prefill", dtype=dt, B=B, H=H, N=N, d=d, chunk=chunk)
    ws = _ws(nb, workspace, q)
    call("sala_linear_prefill_fused", dt, B, H, N, d, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(decay),
         _ptr(state), _ptr(so), _ptr(gamma_q), _ptr(gamma_k), float(eps), float(rope_base or 0.0), int(pos0),
         _ptr(gate), _ptr(ws), nb, _stream())
    return o, so


def linear_decode_fused(q, k, v, state, decay=None, *, gamma_q=None, gamma_k=None, eps=1e-6, rope_base=10000.0,
                        pos=None, gate=None, out=None):
    """One decode token with the neighbours fused (see linear_prefill_fused); pos: int64 [B]
    device tensor of positions (needed with RoPE).  state is updated in place; returns o."""
    B, H, d = _dims(q, "q", 3)
    _want(k, "k", q.shape, q.dtype)
    _want(v, "v", q.shape, q.dtype)
    _want(out, "out", q.shape, q.dtype)
    _want(gate, "gate", q.shape, q.dtype)
    if state is None:
        raise ValueError("state must be given (it is updated in place)")
    _want(state, "state", (B, H, d, d), torch.float32)
    _want(decay, "decay", (H,), torch.float32)
    _want(pos, "pos", (B,), torch.int64)
    _check_gammas(d, gamma_q, gamma_k)
    _dev(q, k, v, state, decay, out, gamma_q, gamma_k, pos, gate)
    o = _empty_like(q) if out is None else out
    call("sala_linear_decode_fused", _code(q), B, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(decay),
         _ptr(state), _ptr(gamma_q), _ptr(gamma_k), float(eps), float(rope_base or 0.0), _ptr(pos), _ptr(gate),
         _stream())
    return o


def qk_norm_rope(x, *, gamma=None, eps=1e-6, rope_base=0.0, pos0=0, out=None):
    """Standalone RMS norm (weight gamma [d] fp32 or None) then rotate-half RoPE at
    positions pos0 .. (rope_base 0 = none) of x [B, H, N, d]; out may be x."""
    B, H, N, d = _dims(x, "x", 4)
    _want(gamma, "gamma", (d,), torch.float32)
    _want(out, "out", x.shape, x.dtype)
    _dev(x, gamma, out)
    o = _empty_like(x) if out is None else out
    call("sala_qk_norm_rope", _code(x), B, H, N, d, _ptr(x), _ptr(o), _ptr(gamma), float(eps),
         float(rope_base or 0.0), int(pos0), _stream())
    return o


def output_gate(o, gate, *, out=None):
    """o * sigmoid(gate), elementwise (numel a multiple of 8); out may be o."""
    if not isinstance(o, torch.Tensor):
        raise ValueError("o must be a torch tensor")
    _want(gate, "gate", o.shape, o.dtype)
    _want(out, "out", o.shape, o.dtype)
    _dev(o, gate, out)
    r = _empty_like(o) if out is None else out
    call("sala_output_gate", _code(o), o.numel(), _ptr(o), _ptr(gate), _ptr(r), _stream())
    return r


def sparse_select(q, k=None, *, k_pooled=None, L=None, block=64, topk=64, n_init=1, n_local=2, idx_out=None,
                  return_scores=False, workspace=None):
    """Block selection.  q [B, Hq, Nq, d] with Nq == L (prefill) or Nq == 1 (decode).

    k [B, Hkv, L, d] (pooled into k_pooled), or k=None with k_pooled [B, Hkv, ceil(L/block), d] fp32 given.
    Returns (idx [B, Hkv, NQB, topk+n_init+n_local] int32, k_pooled[, scores]).
    """
    B, Hq, Nq, d = _dims(q, "q", 4)
    if k is not None:
        Bk, Hkv, L_k, dk = _dims(k, "k", 4)
        if L is not None and L != L_k:
            raise ValueError(f"L = {L} disagrees with k's {L_k} tokens")
        L = L_k
        _want(k, "k", (B, Hkv, L, d), q.dtype)
    else:
        if k_pooled is None or L is None:
            raise ValueError("without k, pass k_pooled and L")
        if k_pooled.dim() != 4:
            raise ValueError("k_pooled must be a 4-d tensor")
        Hkv = k_pooled.shape[1]
    if Nq != L and Nq != 1:
        raise ValueError(f"q must hold all L = {L} queries (prefill) or one (decode), got {Nq}")
    NB = (L + block - 1) // block
    NQB = 1 if (Nq == 1 and L != 1) else NB
    W = topk + n_init + n_local
    _want(k_pooled, "k_pooled", (B, Hkv, NB, d), torch.float32)
    _want(idx_out, "idx_out", (B, Hkv, NQB, W), torch.int32)
    _dev(q, k, k_pooled, idx_out, workspace)
    dt = _code(q)
    if k_pooled is None:
        k_pooled = _empty((B, Hkv, NB, d), torch.float32, q.device)
    idx = _empty((B, Hkv, NQB, W), torch.int32, q.device) if idx_out is None else idx_out
    scores = _empty((B, Hkv, NQB, NB), torch.float32, q.device) if return_scores else None
    # the size for scores == NULL covers every case (with a scores buffer the need is never larger)
    nb = workspace_bytes("sparse_select", dtype=dt, B=B, Hq=Hq, Hkv=Hkv, d=d, Nq=Nq, L=L, block=block, topk=topk,
                         n_init=n_init, n_local=n_local)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_select", dt, B, Hq, Hkv, d, Nq, L, block, topk, n_init, n_local, _ptr(q), _ptr(k),
         _ptr(k_pooled), _ptr(idx), _ptr(scores), _ptr(ws), nb, _stream())
    return (idx, k_pooled, scores) if return_scores else (idx, k_pooled)


def _check_idx(idx, shape_lead, allow_one_block=False):
    """idx: int32 of shape shape_lead + (n_sel,); with allow_one_block also
    shape_lead + (1, n_sel), the layout decode selection returns."""
    if not isinstance(idx, torch.Tensor) or idx.dtype != torch.int32:
        raise ValueError("idx must be an int32 tensor")
    lead = tuple(idx.shape[:-1])
    if allow_one_block and idx.dim() == len(shape_lead) + 2 and lead == tuple(shape_lead) + (1,):
        return idx.shape[-1]
    if lead != tuple(shape_lead) or idx.dim() != len(shape_lead) + 1:
        raise ValueError(f"idx must have shape {tuple(shape_lead)} + (n_sel,), got {tuple(idx.shape)}")
    return idx.shape[-1]


def sparse_prefill(q, k, v, idx, *, block=64, scale=None, out=None, workspace=None):
    """Softmax attention of q [B, Hq, N, d] over the blocks listed in idx [B, Hkv, NQB, n_sel]."""
    B, Hq, N, d = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[1]
    _want(k, "k", (B, Hkv, N, d), q.dtype)
    _want(v, "v", (B, Hkv, N, d), q.dtype)
    _want(out, "out", q.shape, q.dtype)
    n_sel = _check_idx(idx, (B, Hkv, (N + block - 1) // block))
    _dev(q, k, v, idx, out, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _code(q)
    o = _empty_like(q) if out is None else out
    nb = workspace_bytes("sparse_prefill", dtype=dt, B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, block=block, n_sel=n_sel)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_prefill", dt, B, Hq, Hkv, N, d, block, n_sel, ctypes.c_float(scale), _ptr(q), _ptr(k), _ptr(v),
         _ptr(idx), _ptr(o), _ptr(ws), nb, _stream())
    return o


def sparse_prefill_backward(q, k, v, idx, dout, *, block=64, scale=None, dq=None, dk=None, dv=None,
                            workspace=None):
    """Gradients (dq, dk, dv) of sparse_prefill(q, k, v, idx) for dL/do = dout, at the
    fixed selection idx (bf16)."""
    B, Hq, N, d = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[1]
    _want(k, "k", (B, Hkv, N, d), q.dtype)
    _want(v, "v", (B, Hkv, N, d), q.dtype)
    _want(dout, "dout", q.shape, q.dtype)
    _want(dq, "dq", q.shape, q.dtype)
    _want(dk, "dk", k.shape, k.dtype)
    _want(dv, "dv", k.shape, k.dtype)
    n_sel = _check_idx(idx, (B, Hkv, (N + block - 1) // block))
    _dev(q, k, v, idx, dout, dq, dk, dv, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _code(q)
    dq = _empty_like(q) if dq is None else dq
    dk = _empty_like(k) if dk is None else dk
    dv = _empty_like(k) if dv is None else dv
    nb = workspace_bytes("sparse_prefill_backward", dtype=dt, B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, block=block, n_sel=n_sel)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_prefill_backward", dt, B, Hq, Hkv, N, d, block, n_sel, ctypes.c_float(scale), _ptr(q), _ptr(k),
         _ptr(v), _ptr(idx), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), nb, _stream())
    return dq, dk, dv


def sparse_decode(q, k_cache, v_cache, idx, *, L=None, block=64, scale=None, out=None, workspace=None):
    """One query token per head, q [B, Hq, d], against the cached blocks listed in idx
    [B, Hkv, n_sel] (or [B, Hkv, 1, n_sel], as decode selection returns it)."""
    B, Hq, d = _dims(q, "q", 3)
    _, Hkv, Lk, _ = _dims(k_cache, "k_cache", 4)
    if L is not None and L != Lk:
        raise ValueError(f"L = {L} must equal the cache's {Lk} tokens (a cache of larger capacity: "
                         "sparse_decode_step)")
    L = Lk
    _want(k_cache, "k_cache", (B, Hkv, L, d), q.dtype)
    _want(v_cache, "v_cache", (B, Hkv, L, d), q.dtype)
    _want(out, "out", q.shape, q.dtype)
    n_sel = _check_idx(idx, (B, Hkv), allow_one_block=True)
    _dev(q, k_cache, v_cache, idx, out, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _code(q)
    o = _empty_like(q) if out is None else out
    nb = workspace_bytes("sparse_decode", dtype=dt, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, block=block, n_sel=n_sel)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_decode", dt, B, Hq, Hkv, L, d, block, n_sel, ctypes.c_float(scale), _ptr(q), _ptr(k_cache),
         _ptr(v_cache), _ptr(idx), _ptr(o), _ptr(ws), nb, _stream())
    return o


def _cache_dims(q, k_cache, v_cache, k_pooled, block):
    B, Hkv, cap, d = _dims(k_cache, "k_cache", 4)
    _want(v_cache, "v_cache", k_cache.shape, k_cache.dtype)
    if not isinstance(k_pooled, torch.Tensor):
        raise ValueError("k_pooled must be a torch tensor")
    _want(k_pooled, "k_pooled", (B, Hkv, (cap + block - 1) // block, d), torch.float32)
    if q.dtype != k_cache.dtype:
        raise ValueError("q must have the caches' dtype")
    return B, Hkv, cap, d


def sparse_prefill_chunk(q, k_new, v_new, k_cache, v_cache, k_pooled, pos0, *, block=64, topk=64, n_init=1,
                         n_local=2, scale=None, idx_out=None, out=None, workspace=None):
    """Tokens pos0 .. pos0+n-1 of a sequence whose earlier tokens sit in the caches:
    q [B, Hq, n, d], k_new, v_new [B, Hkv, n, d] are written into k_cache, v_cache
    [B, Hkv, capacity, d]; k_pooled [B, Hkv, ceil(capacity/64), d] fp32 is updated.
    Returns (o [B, Hq, n, d], idx [B, Hkv, ceil(n/64), n_sel])."""
    _, Hq, n, _ = _dims(q, "q", 4)
    B, Hkv, cap, d = _cache_dims(q, k_cache, v_cache, k_pooled, block)
    _want(q, "q", (B, Hq, n, d), k_cache.dtype)
    _want(k_new, "k_new", (B, Hkv, n, d), k_cache.dtype)
    _want(v_new, "v_new", (B, Hkv, n, d), k_cache.dtype)
    _want(out, "out", q.shape, q.dtype)
    n_sel = topk + n_init + n_local
    _want(idx_out, "idx_out", (B, Hkv, (n + block - 1) // block, n_sel), torch.int32)
    _dev(q, k_new, v_new, k_cache, v_cache, k_pooled, idx_out, out, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _code(q)
    o = _empty_like(q) if out is None else out
    idx = idx_out if idx_out is not None else _empty((B, Hkv, (n + block - 1) // block, n_sel), torch.int32,
                                                     q.device)
    nb = workspace_bytes("sparse_prefill_chunk", dtype=dt, B=B, Hq=Hq, Hkv=Hkv, capacity=cap, d=d, n=n, block=block,
                         topk=topk, n_init=n_init, n_local=n_local)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_prefill_chunk", dt, B, Hq, Hkv, cap, d, int(pos0), n, block, topk, n_init, n_local,
         ctypes.c_float(scale), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_pooled),
         _ptr(idx), _ptr(o), _ptr(ws), nb, _stream())
    return o, idx


def sparse_decode_step(q, k_new, v_new, k_cache, v_cache, k_pooled, pos, *, block=64, topk=64, n_init=1,
                       n_local=2, scale=None, idx_out=None, out=None, workspace=None):
    """One generated token at position pos: q [B, Hq, d], k_new, v_new [B, Hkv, d] are
    appended to the caches (see sparse_prefill_chunk).  Returns (o [B, Hq, d], idx [B, Hkv, n_sel])."""
    _, Hq, _ = _dims(q, "q", 3)
    B, Hkv, cap, d = _cache_dims(q, k_cache, v_cache, k_pooled, block)
    _want(q, "q", (B, Hq, d), k_cache.dtype)
    _want(k_new, "k_new", (B, Hkv, d), k_cache.dtype)
    _want(v_new, "v_new", (B, Hkv, d), k_cache.dtype)
    _want(out, "out", q.shape, q.dtype)
    n_sel = topk + n_init + n_local
    _want(idx_out, "idx_out", (B, Hkv, n_sel), torch.int32)
    _dev(q, k_new, v_new, k_cache, v_cache, k_pooled, idx_out, out, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _code(q)
    o = _empty_like(q) if out is None else out
    idx = idx_out if idx_out is not None else _empty((B, Hkv, n_sel), torch.int32, q.device)
    nb = workspace_bytes("sparse_decode_step", dtype=dt, B=B, Hq=Hq, Hkv=Hkv, capacity=cap, d=d, block=block,
                         topk=topk, n_init=n_init, n_local=n_local)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_decode_step", dt, B, Hq, Hkv, cap, d, int(pos), block, topk, n_init, n_local,
         ctypes.c_float(scale), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_pooled),
         _ptr(idx), _ptr(o), _ptr(ws), nb, _stream())
    return o, idx


def sparse_decode_step_noalloc(q, k_new, v_new, k_cache, v_cache, k_pooled, pos, idx_out, out, *, block=64, topk=64,
                               n_init=1, n_local=2, scale=None):
    """sparse_decode_step without a workspace and without allocating: the library's
    fixed per-GPU scratch array serves as the workspace, and the caller passes the
    outputs (idx_out [B, Hkv, n_sel] int32, out like q).  Calls that overlap on one
    GPU share that array and must not be made.  Returns (out, idx_out)."""
    _, Hq, _ = _dims(q, "q", 3)
    B, Hkv, cap, d = _cache_dims(q, k_cache, v_cache, k_pooled, block)
    _want(q, "q", (B, Hq, d), k_cache.dtype)
    _want(k_new, "k_new", (B, Hkv, d), k_cache.dtype)
    _want(v_new, "v_new", (B, Hkv, d), k_cache.dtype)
    if out is None or idx_out is None:
        raise ValueError("the allocation-free call needs out and idx_out")
    _want(out, "out", q.shape, q.dtype)
    _want(idx_out, "idx_out", (B, Hkv, topk + n_init + n_local), torch.int32)
    _dev(q, k_new, v_new, k_cache, v_cache, k_pooled, idx_out, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    call("sala_sparse_decode_step_noalloc", _code(q), B, Hq, Hkv, cap, d, int(pos), block, topk, n_init, n_local,
         ctypes.c_float(scale), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_pooled),
         _ptr(idx_out), _ptr(out), _stream())
    return out, idx_out


def dense_prefill(q, k, v, *, scale=None, out=None):
    """Causal softmax attention of q [B, Hq, N, d] over every earlier token of k, v [B, Hkv, N, d] (bf16)."""
    B, Hq, N, d = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[1]
    _want(k, "k", (B, Hkv, N, d), q.dtype)
    _want(v, "v", (B, Hkv, N, d), q.dtype)
    _want(out, "out", q.shape, q.dtype)
    _dev(q, k, v, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = _empty_like(q) if out is None else out
    call("sala_dense_prefill", _code(q), B, Hq, Hkv, N, d, ctypes.c_float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
         _stream())
    return o


def ceiling_mfma(workgroups, iters, out):
    """Launch the MFMA ceiling microkernel (flops = workgroups*8*iters*8*16384)."""
    _want(out, "out", (workgroups * 512,), torch.float32)
    _dev(out)
    call("sala_ceiling_mfma", workgroups, iters, _ptr(out), _stream())


def ceiling_copy(src, dst):
    """Launch the streaming-copy ceiling microkernel over src.nbytes bytes."""
    if not isinstance(src, torch.Tensor) or not isinstance(dst, torch.Tensor):
        raise ValueError("src and dst must be torch tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _dev(src, dst)
    call("sala_ceiling_copy", _ptr(src), _ptr(dst), nbytes, _stream())


def ceiling_read(src, out, nbytes=None):
    """Launch the read-only streaming microkernel over the first nbytes of src
    (default: all of it; 0: one workgroup that reads nothing).  out: fp32 with
    at least nbytes // 16384 + 1 elements."""
    total = src.numel() * src.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    if nbytes < 0 or nbytes > total or nbytes % 16:
        raise ValueError("nbytes must be a multiple of 16 within src")
    _want(out, "out", (out.numel(),), torch.float32)
    if out.numel() < nbytes // 16384 + 1:
        raise ValueError("out is too small")
    _dev(src, out)
    call("sala_ceiling_read", _ptr(src), nbytes, _ptr(out), _stream())


def layer_group_prefill(linear_layers, sparse_layer, *, block=64, topk=64, n_init=1, n_local=2, chunk=None,
                        workspaces=None, out=None, sparse_events=None):
    """The 3:1 group: each linear layer {q,k,v,decay}, then select + attend on the sparse layer {q,k,v}.

    Returns ([o_linear...], o_sparse, idx).  All launches go to torch's current stream.
    workspaces: optional {"linear": [uint8 tensor per layer] or one tensor, "select": ..., "sparse": ...}
    reused across calls.  out: optional preallocated {"linear": [o per layer], "sparse": o, "idx": idx,
    "k_pooled": k_pooled}.  sparse_events: optional (start, end) torch events recorded on the current
    stream around the sparse attention launch (its own duration, for measurement).
    """
    ws = workspaces or {}
    out = out or {}
    lws = ws.get("linear")
    outs = []
    for n, x in enumerate(linear_layers):
        w = lws[n] if isinstance(lws, (list, tuple)) else lws
        o = out["linear"][n] if "linear" in out else None
        outs.append(linear_prefill(x["q"], x["k"], x["v"], x.get("decay"), chunk=chunk, want_state=False,
                                   workspace=w, out=o)[0])
    sp = sparse_layer
    idx, _ = sparse_select(sp["q"], sp["k"], block=block, topk=topk, n_init=n_init, n_local=n_local,
                           workspace=ws.get("select"), idx_out=out.get("idx"), k_pooled=out.get("k_pooled"))
    if sparse_events is not None:
        sparse_events[0].record(torch.cuda.current_stream())
    o = sparse_prefill(sp["q"], sp["k"], sp["v"], idx, block=block, workspace=ws.get("sparse"), out=out.get("sparse"))
    if sparse_events is not None:
        sparse_events[1].record(torch.cuda.current_stream())
    return outs, o, idx
