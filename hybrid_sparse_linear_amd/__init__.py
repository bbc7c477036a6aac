"""libsala Python binding: the SALA hybrid attention layer group on MI355X.

Thin wrappers over the C ABI in ``include/sala.h``.  They check tensor
shapes, dtypes and devices, allocate outputs and workspaces with torch when
the caller does not pass them, and call the HIP library on torch's current
stream.  Every step of the computation runs in the HIP kernels; there is no
CPU or PyTorch fallback -- a missing ``libsala.so`` raises.

Entry points (same names as the C ABI, without the ``sala_`` prefix):
  linear_prefill   causal decayed linear attention over a sequence
  linear_decode    one token of the same recurrence (state updated in place)
  sparse_select    pooled block scores and top-k block selection
  sparse_prefill   softmax attention over the selected blocks
  sparse_decode    one query token against the selected cached blocks
  dense_prefill    plain causal attention (the full-attention comparison)
  ceiling_mfma / ceiling_copy   microkernels measuring this GPU's ceilings
  layer_group_prefill  three linear layers then one sparse layer, one stream
"""

import ctypes
import math

import torch

from ._lib import SALA_BF16, SALA_F32, SalaError, call, lib  # noqa: F401

__all__ = ["linear_prefill", "linear_decode", "linear_prefill_fused", "linear_decode_fused", "qk_norm_rope",
           "output_gate", "sparse_prefill_chunk", "sparse_decode_step", "sparse_select",
           "sparse_prefill", "sparse_decode",
           "dense_prefill", "layer_group_prefill", "workspace_bytes", "ceiling_mfma", "ceiling_copy", "SalaError"]


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


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libsala tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("libsala tensors must be contiguous")


def _ws(nbytes, ws, like):
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device)


def workspace_bytes(op, **kw):
    """Workspace size in bytes of an entry point for the given arguments."""
    L = lib()
    if op == "linear_prefill":
        return L.sala_linear_prefill_workspace(kw["dtype"], kw["B"], kw["H"], kw["N"], kw["d"], kw["chunk"])
    if op == "sparse_select":
        return L.sala_sparse_select_workspace(kw["dtype"], kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["Nq"], kw["L"],
                                              kw["block"], kw["topk"], kw["n_init"], kw["n_local"])
    if op == "sparse_prefill":
        return L.sala_sparse_prefill_workspace(kw["dtype"], kw["B"], kw["Hq"], kw["Hkv"], kw["N"], kw["d"],
                                               kw["block"], kw["n_sel"])
    if op == "sparse_decode":
        return L.sala_sparse_decode_workspace(kw["dtype"], kw["B"], kw["Hq"], kw["Hkv"], kw["L"], kw["d"],
                                              kw["block"], kw["n_sel"])
    if op == "sparse_prefill_chunk":
        return L.sala_sparse_prefill_chunk_workspace(kw["dtype"], kw["B"], kw["Hq"], kw["Hkv"], kw["capacity"],
                                                     kw["d"], kw["n"], kw["block"], kw["topk"], kw["n_init"],
                                                     kw["n_local"])
    if op == "sparse_decode_step":
        return L.sala_sparse_decode_step_workspace(kw["dtype"], kw["B"], kw["Hq"], kw["Hkv"], kw["capacity"],
                                                   kw["d"], kw["block"], kw["topk"], kw["n_init"], kw["n_local"])
    raise ValueError(op)


def linear_prefill(q, k, v, decay=None, state=None, *, chunk=None, out=None, state_out=None, workspace=None,
                   want_state=True):
    """o, S_out = causal linear attention of q, k, v [B, H, N, d] with per-head decay [H] (fp32).

    state: optional [B, H, d, d] fp32 carried state S[d_k][d_v].  Returns (o, S_out or None).
    """
    _dev(q, k, v, decay, state, out, state_out)
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    chunk = chunk or (64 if d == 64 else 128)
    dt = _code(q)
    o = torch.empty_like(q) if out is None else out
    so = state_out
    if so is None and want_state:
        so = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    nb = lib().sala_linear_prefill_workspace(dt, B, H, N, d, chunk)
    ws = _ws(nb, workspace, q)
    call("sala_linear_prefill", dt, B, H, N, d, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(decay), _ptr(state),
         _ptr(so), _ptr(ws), nb, _stream())
    return o, so


def linear_decode(q, k, v, state, decay=None, *, out=None):
    """One decode token: state [B, H, d, d] fp32 is updated in place; returns o [B, H, d]."""
    _dev(q, k, v, state, decay, out)
    B, H, d = q.shape
    o = torch.empty_like(q) if out is None else out
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
    _dev(q, k, v, decay, state, out, state_out, gamma_q, gamma_k, gate)
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if gate is not None and (gate.shape != q.shape or gate.dtype != q.dtype):
        raise ValueError("gate must match q in shape and dtype")
    for gname, gt in (("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        if gt is not None and (gt.shape != (d,) or gt.dtype != torch.float32):
            raise ValueError(f"{gname} must be a float32 [{d}] tensor")
    chunk = chunk or (64 if d == 64 else 128)
    dt = _code(q)
    o = torch.empty_like(q) if out is None else out
    so = state_out
    if so is None and want_state:
        so = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    nb = lib().sala_linear_prefill_workspace(dt, B, H, N, d, chunk)
    ws = _ws(nb, workspace, q)
    call("sala_linear_prefill_fused", dt, B, H, N, d, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(decay),
         _ptr(state), _ptr(so), _ptr(gamma_q), _ptr(gamma_k), float(eps), float(rope_base or 0.0), int(pos0),
         _ptr(gate), _ptr(ws), nb, _stream())
    return o, so


def linear_decode_fused(q, k, v, state, decay=None, *, gamma_q=None, gamma_k=None, eps=1e-6, rope_base=10000.0,
                        pos=None, gate=None, out=None):
    """One decode token with the neighbours fused (see linear_prefill_fused); pos: int64 [B]
    device tensor of positions (needed with RoPE).  state is updated in place; returns o."""
    _dev(q, k, v, state, decay, out, gamma_q, gamma_k, pos, gate)
    B, H, d = q.shape
    if pos is not None and (pos.dtype != torch.int64 or pos.shape != (B,)):
        raise ValueError("pos must be an int64 [B] tensor")
    o = torch.empty_like(q) if out is None else out
    call("sala_linear_decode_fused", _code(q), B, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(decay),
         _ptr(state), _ptr(gamma_q), _ptr(gamma_k), float(eps), float(rope_base or 0.0), _ptr(pos), _ptr(gate),
         _stream())
    return o


def qk_norm_rope(x, *, gamma=None, eps=1e-6, rope_base=0.0, pos0=0, out=None):
    """Standalone RMS norm (weight gamma [d] fp32 or None) then rotate-half RoPE at
    positions pos0 .. (rope_base 0 = none) of x [B, H, N, d]; out may be x."""
    _dev(x, gamma, out)
    B, H, N, d = x.shape
    if gamma is not None and (gamma.shape != (d,) or gamma.dtype != torch.float32):
        raise ValueError(f"gamma must be a float32 [{d}] tensor")
    o = torch.empty_like(x) if out is None else out
    call("sala_qk_norm_rope", _code(x), B, H, N, d, _ptr(x), _ptr(o), _ptr(gamma), float(eps),
         float(rope_base or 0.0), int(pos0), _stream())
    return o


def output_gate(o, gate, *, out=None):
    """o * sigmoid(gate), elementwise (numel a multiple of 8); out may be o."""
    _dev(o, gate, out)
    if gate.shape != o.shape or gate.dtype != o.dtype:
        raise ValueError("gate must match o in shape and dtype")
    r = torch.empty_like(o) if out is None else out
    call("sala_output_gate", _code(o), o.numel(), _ptr(o), _ptr(gate), _ptr(r), _stream())
    return r


def sparse_select(q, k=None, *, k_pooled=None, L=None, block=64, topk=64, n_init=1, n_local=2, idx_out=None,
                  return_scores=False, workspace=None):
    """Block selection.  q [B, Hq, Nq, d] with Nq == L (prefill) or Nq == 1 (decode).

    k [B, Hkv, L, d] (pooled into k_pooled), or k=None with k_pooled [B, Hkv, ceil(L/block), d] fp32 given.
    Returns (idx [B, Hkv, NQB, topk+n_init+n_local] int32, k_pooled[, scores]).
    """
    _dev(q, k, k_pooled, idx_out)
    B, Hq, Nq, d = q.shape
    if k is not None:
        Hkv, L = k.shape[1], k.shape[2]
    else:
        if k_pooled is None or L is None:
            raise ValueError("without k, pass k_pooled and L")
        Hkv = k_pooled.shape[1]
    NB = (L + block - 1) // block
    NQB = 1 if (Nq == 1 and L != 1) else NB
    W = topk + n_init + n_local
    dt = _code(q)
    if k_pooled is None:
        k_pooled = torch.empty((B, Hkv, NB, d), dtype=torch.float32, device=q.device)
    idx = torch.empty((B, Hkv, NQB, W), dtype=torch.int32, device=q.device) if idx_out is None else idx_out
    scores = torch.empty((B, Hkv, NQB, NB), dtype=torch.float32, device=q.device) if return_scores else None
    # the size for scores == NULL covers every case (with a scores buffer the need is never larger)
    nb = lib().sala_sparse_select_workspace(dt, B, Hq, Hkv, d, Nq, L, block, topk, n_init, n_local)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_select", dt, B, Hq, Hkv, d, Nq, L, block, topk, n_init, n_local, _ptr(q), _ptr(k),
         _ptr(k_pooled), _ptr(idx), _ptr(scores), _ptr(ws), nb, _stream())
    return (idx, k_pooled, scores) if return_scores else (idx, k_pooled)


def sparse_prefill(q, k, v, idx, *, block=64, scale=None, out=None, workspace=None):
    """Softmax attention of q [B, Hq, N, d] over the blocks listed in idx [B, Hkv, NQB, n_sel]."""
    _dev(q, k, v, idx, out)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    n_sel = idx.shape[-1]
    if idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _code(q)
    o = torch.empty_like(q) if out is None else out
    nb = lib().sala_sparse_prefill_workspace(dt, B, Hq, Hkv, N, d, block, n_sel)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_prefill", dt, B, Hq, Hkv, N, d, block, n_sel, ctypes.c_float(scale), _ptr(q), _ptr(k), _ptr(v),
         _ptr(idx), _ptr(o), _ptr(ws), nb, _stream())
    return o


def sparse_decode(q, k_cache, v_cache, idx, *, L=None, block=64, scale=None, out=None, workspace=None):
    """One query token per head, q [B, Hq, d], against the cached blocks listed in idx [B, Hkv, n_sel]."""
    _dev(q, k_cache, v_cache, idx, out)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    L = k_cache.shape[2] if L is None else L
    n_sel = idx.shape[-1]
    if idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _code(q)
    o = torch.empty_like(q) if out is None else out
    nb = lib().sala_sparse_decode_workspace(dt, B, Hq, Hkv, L, d, block, n_sel)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_decode", dt, B, Hq, Hkv, L, d, block, n_sel, ctypes.c_float(scale), _ptr(q), _ptr(k_cache),
         _ptr(v_cache), _ptr(idx), _ptr(o), _ptr(ws), nb, _stream())
    return o


def _cache_dims(k_cache, v_cache, k_pooled, block):
    B, Hkv, cap, d = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must share shape and dtype")
    if k_pooled.dtype != torch.float32 or tuple(k_pooled.shape) != (B, Hkv, (cap + block - 1) // block, d):
        raise ValueError("k_pooled must be float32 [B, Hkv, ceil(capacity / block), d]")
    return B, Hkv, cap, d


def sparse_prefill_chunk(q, k_new, v_new, k_cache, v_cache, k_pooled, pos0, *, block=64, topk=64, n_init=1,
                         n_local=2, scale=None, idx_out=None, out=None, workspace=None):
    """Tokens pos0 .. pos0+n-1 of a sequence whose earlier tokens sit in the caches:
    q [B, Hq, n, d], k_new, v_new [B, Hkv, n, d] are written into k_cache, v_cache
    [B, Hkv, capacity, d]; k_pooled [B, Hkv, ceil(capacity/64), d] fp32 is updated.
    Returns (o [B, Hq, n, d], idx [B, Hkv, ceil(n/64), n_sel])."""
    _dev(q, k_new, v_new, k_cache, v_cache, k_pooled, idx_out, out)
    B, Hkv, cap, d = _cache_dims(k_cache, v_cache, k_pooled, block)
    Hq, n = q.shape[1], q.shape[2]
    if k_new.shape != (B, Hkv, n, d) or v_new.shape != (B, Hkv, n, d):
        raise ValueError("k_new, v_new must be [B, Hkv, n, d]")
    n_sel = topk + n_init + n_local
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _code(q)
    o = torch.empty_like(q) if out is None else out
    idx = idx_out if idx_out is not None else torch.empty((B, Hkv, (n + block - 1) // block, n_sel),
                                                         dtype=torch.int32, device=q.device)
    nb = lib().sala_sparse_prefill_chunk_workspace(dt, B, Hq, Hkv, cap, d, n, block, topk, n_init, n_local)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_prefill_chunk", dt, B, Hq, Hkv, cap, d, int(pos0), n, block, topk, n_init, n_local,
         ctypes.c_float(scale), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_pooled),
         _ptr(idx), _ptr(o), _ptr(ws), nb, _stream())
    return o, idx


def sparse_decode_step(q, k_new, v_new, k_cache, v_cache, k_pooled, pos, *, block=64, topk=64, n_init=1,
                       n_local=2, scale=None, idx_out=None, out=None, workspace=None):
    """One generated token at position pos: q [B, Hq, d], k_new, v_new [B, Hkv, d] are
    appended to the caches (see sparse_prefill_chunk).  Returns (o [B, Hq, d], idx [B, Hkv, n_sel])."""
    _dev(q, k_new, v_new, k_cache, v_cache, k_pooled, idx_out, out)
    B, Hkv, cap, d = _cache_dims(k_cache, v_cache, k_pooled, block)
    Hq = q.shape[1]
    if k_new.shape != (B, Hkv, d) or v_new.shape != (B, Hkv, d):
        raise ValueError("k_new, v_new must be [B, Hkv, d]")
    n_sel = topk + n_init + n_local
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _code(q)
    o = torch.empty_like(q) if out is None else out
    idx = idx_out if idx_out is not None else torch.empty((B, Hkv, n_sel), dtype=torch.int32, device=q.device)
    nb = lib().sala_sparse_decode_step_workspace(dt, B, Hq, Hkv, cap, d, block, topk, n_init, n_local)
    ws = _ws(nb, workspace, q)
    call("sala_sparse_decode_step", dt, B, Hq, Hkv, cap, d, int(pos), block, topk, n_init, n_local,
         ctypes.c_float(scale), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_pooled),
         _ptr(idx), _ptr(o), _ptr(ws), nb, _stream())
    return o, idx


def dense_prefill(q, k, v, *, scale=None, out=None):
    """Causal softmax attention of q [B, Hq, N, d] over every earlier token of k, v [B, Hkv, N, d] (bf16)."""
    _dev(q, k, v, out)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    call("sala_dense_prefill", _code(q), B, Hq, Hkv, N, d, ctypes.c_float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
         _stream())
    return o


def ceiling_mfma(workgroups, iters, out):
    """Launch the MFMA ceiling microkernel (flops = workgroups*8*iters*8*16384)."""
    _dev(out)
    call("sala_ceiling_mfma", workgroups, iters, _ptr(out), _stream())


def ceiling_copy(src, dst):
    """Launch the streaming-copy ceiling microkernel over src.nbytes bytes."""
    _dev(src, dst)
    nbytes = src.numel() * src.element_size()
    call("sala_ceiling_copy", _ptr(src), _ptr(dst), nbytes, _stream())


def layer_group_prefill(linear_layers, sparse_layer, *, block=64, topk=64, n_init=1, n_local=2, chunk=None):
    """The 3:1 group: each linear layer {q,k,v,decay}, then select + attend on the sparse layer {q,k,v}.

    Returns ([o_linear...], o_sparse, idx).  All launches go to torch's current stream.
    """
    outs = [linear_prefill(x["q"], x["k"], x["v"], x.get("decay"), chunk=chunk, want_state=False)[0]
            for x in linear_layers]
    sp = sparse_layer
    idx, _ = sparse_select(sp["q"], sp["k"], block=block, topk=topk, n_init=n_init, n_local=n_local)
    o = sparse_prefill(sp["q"], sp["k"], sp["v"], idx, block=block)
    return outs, o, idx
