"""Gradients of the linear and sparse attention operations in float64 -- test
infrastructure only.

What the pages fix: the hybrid model is obtained by continual training of a
pretrained Transformer -- a low-cost training framework whose stages convert
softmax layers and then train the hybrid at growing context lengths
([P1] abstract; [P2] 技術概要 §2.3; [P3] §2 "Trainingsstrategie").  Training
needs the gradients of both attention operations; the pages give no
formula, so the gradients here are those of the forward definitions in
``oracle.linear`` and ``oracle.sparse`` (the plain chain rule, no
approximation), for a loss L whose gradients dL/do (and dL/dS_out) are given.

Linear attention, one head (lam = decay, D[t, s] = lam**(t - s) for s <= t):
    o = ((Q K^T) * D) V + diag(lam**(t+1)) Q S_in
    S_out = lam**N S_in + K^T diag(lam**(N-1-s)) V
  gives, with dO = dL/do and dS = dL/dS_out,
    dQ    = ((dO V^T) * D) K + diag(lam**(t+1)) dO S_in^T
    dK    = ((dO V^T) * D)^T Q + diag(lam**(N-1-s)) V dS^T
    dV    = ((Q K^T) * D)^T dO + diag(lam**(N-1-s)) K dS
    dS_in = Q^T diag(lam**(t+1)) dO + lam**N dS
  The chunked form walks the chunks backwards with the gradient of the state
  after chunk c, G_c (G_last = dS, G_{c-1} = lam**m G_c + Q_c^T diag(lam**(i+1))
  dO_c, dS_in = G_{-1}), next to the forward states S_{c-1}.

Sparse attention at a fixed selection (row t of query head h, its token set
A(t), p = softmax over A(t) of scale * q_t . k_s, o_t = sum_s p_s v_s):
    dv_s += p_s dO_t
    dp_s  = dO_t . v_s
    ds_s  = p_s (dp_s - dO_t . o_t)
    dq_t  = scale * sum_s ds_s k_s
    dk_s += scale * ds_s q_t
  summed over every row and every query head of the KV head's group.  The
  selection itself (a top-k of block scores) is piecewise constant in q and k
  and passes no gradient.

Functions:
  linear_attention_backward          quadratic (definition) form, one head
  linear_attention_backward_chunked  chunked reverse recurrence, one head
  linear_prefill_backward            batched [B, H, N, d] driver
  sparse_attention_backward          batched, rows of every query block
  sparse_attention_backward_dq_rows  dq of chosen (b, hq, t) rows only: a
                                     row's dq needs only that row's keys
  sparse_attention_backward_kv_blocks  dk, dv of chosen key blocks only: the
                                     rows of the query blocks that selected
                                     them, over the whole group
"""

import math

import numpy as np

from .linear import decay_mask
from .sparse import n_blocks


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def linear_attention_backward(q, k, v, do, lam=1.0, state_in=None, dstate_out=None):
    """Gradients (dq, dk, dv, dstate_in) of one head from the quadratic definition."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    lam = float(lam)
    n = q.shape[0]
    dm = decay_mask(lam, n)
    w_in = np.power(lam, np.arange(1, n + 1))          # lam**(t+1): weight of S_in in row t
    w_out = np.power(lam, n - 1 - np.arange(n))        # lam**(N-1-s): weight of key s in S_out
    dov = (do @ v.T) * dm                              # [t, s]
    dq = dov @ k
    dk = dov.T @ q
    dv = ((q @ k.T) * dm).T @ do
    ds_in = q.T @ (w_in[:, None] * do)
    if state_in is not None:
        dq = dq + w_in[:, None] * (do @ _f64(state_in).T)
    if dstate_out is not None:
        ds = _f64(dstate_out)
        dk = dk + w_out[:, None] * (v @ ds.T)
        dv = dv + w_out[:, None] * (k @ ds)
        ds_in = ds_in + (lam ** n) * ds
    return dq, dk, dv, ds_in


def linear_attention_backward_chunked(q, k, v, do, lam, chunk, state_in=None, dstate_out=None):
    """The same gradients by chunks: forward states S_{c-1} in a first sweep, then a
    backward sweep carrying the state gradient G_c (see the module docstring)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    lam = float(lam)
    n, dk_, dv_ = q.shape[0], k.shape[1], v.shape[1]
    starts = list(range(0, n, chunk))
    s = np.zeros((dk_, dv_)) if state_in is None else _f64(state_in).copy()
    s_before = []
    for c0 in starts:
        kc, vc = k[c0:c0 + chunk], v[c0:c0 + chunk]
        m = kc.shape[0]
        s_before.append(s)
        s = (lam ** m) * s + kc.T @ (np.power(lam, m - 1 - np.arange(m))[:, None] * vc)
    g = np.zeros((dk_, dv_)) if dstate_out is None else _f64(dstate_out).copy()
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for c, c0 in reversed(list(enumerate(starts))):
        qc, kc, vc, doc = q[c0:c0 + chunk], k[c0:c0 + chunk], v[c0:c0 + chunk], do[c0:c0 + chunk]
        m = qc.shape[0]
        dm = decay_mask(lam, m)
        w_in = np.power(lam, np.arange(1, m + 1))
        w_out = np.power(lam, m - 1 - np.arange(m))
        dov = (doc @ vc.T) * dm
        dq[c0:c0 + m] = dov @ kc + w_in[:, None] * (doc @ s_before[c].T)
        dk[c0:c0 + m] = dov.T @ qc + w_out[:, None] * (vc @ g.T)
        dv[c0:c0 + m] = ((qc @ kc.T) * dm).T @ doc + w_out[:, None] * (kc @ g)
        g = (lam ** m) * g + qc.T @ (w_in[:, None] * doc)
    return dq, dk, dv, g


def linear_prefill_backward(q, k, v, do, decay=None, state_in=None, dstate_out=None, form="quadratic",
                            chunk=None):
    """Batched [B, H, N, d] driver.  Returns (dq, dk, dv, dstate_in [B, H, d_k, d_v])."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b_, h_ = q.shape[:2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dsi = np.zeros((b_, h_, k.shape[-1], v.shape[-1]))
    for b in range(b_):
        for h in range(h_):
            lam = 1.0 if decay is None else float(decay[h])
            si = None if state_in is None else state_in[b, h]
            dso = None if dstate_out is None else dstate_out[b, h]
            if form == "quadratic":
                r = linear_attention_backward(q[b, h], k[b, h], v[b, h], do[b, h], lam, si, dso)
            elif form == "chunked":
                r = linear_attention_backward_chunked(q[b, h], k[b, h], v[b, h], do[b, h], lam, chunk, si, dso)
            else:
                raise ValueError(form)
            dq[b, h], dk[b, h], dv[b, h], dsi[b, h] = r
    return dq, dk, dv, dsi


def sparse_attention_backward(q, k, v, idx, do, block=64, scale=None):
    """Gradients (dq, dk, dv) of sparse_attention_prefill at the fixed selection idx.

    q, do [B, Hq, N, d]; k, v [B, Hkv, N, d]; idx [B, Hkv, NQB, W] (-1 padded).
    For token t of query block i and head h (KV head h // G), A(t) = tokens of
    the blocks listed in idx[b, h // G, i] that are <= t.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(b_):
        for h in range(hq):
            kv = h // g
            for i in range(n_blocks(n, block)):
                t0, t1 = i * block, min((i + 1) * block, n)
                toks = np.concatenate([np.arange(j * block, min((j + 1) * block, n))
                                       for j in idx[b, kv, i] if j >= 0])
                logits = scale * (q[b, h, t0:t1] @ k[b, kv, toks].T)
                logits = np.where(toks[None, :] <= np.arange(t0, t1)[:, None], logits, -np.inf)
                logits -= logits.max(axis=1, keepdims=True)
                p = np.exp(logits)
                p /= p.sum(axis=1, keepdims=True)                        # [rows, |toks|]
                o = p @ v[b, kv, toks]
                dp = do[b, h, t0:t1] @ v[b, kv, toks].T
                ds = p * (dp - np.sum(do[b, h, t0:t1] * o, axis=1, keepdims=True))
                dq[b, h, t0:t1] = scale * (ds @ k[b, kv, toks])
                np.add.at(dk[b, kv], toks, scale * (ds.T @ q[b, h, t0:t1]))
                np.add.at(dv[b, kv], toks, p.T @ do[b, h, t0:t1])
    return dq, dk, dv


def sparse_attention_backward_dq_rows(q, k, v, idx, do, rows, block=64, scale=None):
    """dq_t of sparse_attention_backward for selected (b, hq, t) triples only:
    p, dp = dO_t . v_s and ds = p (dp - sum_s p dp) over the row's own token set
    A(t), then dq_t = scale * sum_s ds_s k_s.  Returns [len(rows), d]."""
    hq, n, d = q.shape[1], q.shape[2], q.shape[-1]
    g = hq // k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = np.zeros((len(rows), d))
    for r, (b, h, t) in enumerate(rows):
        kv = h // g
        i = t // block
        toks = np.concatenate([np.arange(j * block, min((j + 1) * block, n))
                               for j in idx[b, kv, i] if j >= 0])
        toks = toks[toks <= t]
        kt = _f64(k[b, kv, toks])
        logits = scale * (kt @ _f64(q[b, h, t]))
        logits -= logits.max()
        p = np.exp(logits)
        p /= p.sum()
        dp = _f64(v[b, kv, toks]) @ _f64(do[b, h, t])
        ds = p * (dp - np.sum(p * dp))
        out[r] = scale * (ds @ kt)
    return out


def sparse_attention_backward_kv_blocks(q, k, v, idx, do, blocks, block=64, scale=None):
    """dk and dv of sparse_attention_backward for selected key blocks (b, kv, j)
    only: the sums over every query block i that lists j (j <= i), every row t
    of it with s <= t and every head of the group, each row's softmax taken over
    its own token set.  Returns (dk, dv), each [len(blocks), rows of block j, d]."""
    hq, n, d = q.shape[1], q.shape[2], q.shape[-1]
    g = hq // k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nb = n_blocks(n, block)
    dk = np.zeros((len(blocks), block, k.shape[-1]))
    dv = np.zeros((len(blocks), block, v.shape[-1]))
    for r, (b, kv, j) in enumerate(blocks):
        keys = np.arange(j * block, min((j + 1) * block, n))
        for i in range(j, nb):
            sel = [int(x) for x in idx[b, kv, i]]
            if -1 in sel:
                sel = sel[:sel.index(-1)]
            if j not in sel:
                continue
            t0, t1 = i * block, min((i + 1) * block, n)
            toks = np.concatenate([np.arange(x * block, min((x + 1) * block, n)) for x in sel])
            cols = np.searchsorted(toks, keys) if np.all(np.diff(toks) > 0) else None
            if cols is None:  # selection not ascending: find the key columns one by one
                cols = np.array([int(np.nonzero(toks == s_)[0][0]) for s_ in keys])
            kt, vt = _f64(k[b, kv, toks]), _f64(v[b, kv, toks])
            for h in range(kv * g, (kv + 1) * g):
                qi, doi = _f64(q[b, h, t0:t1]), _f64(do[b, h, t0:t1])
                logits = scale * (qi @ kt.T)
                logits = np.where(toks[None, :] <= np.arange(t0, t1)[:, None], logits, -np.inf)
                logits -= logits.max(axis=1, keepdims=True)
                p = np.exp(logits)
                p /= p.sum(axis=1, keepdims=True)
                dp = doi @ vt.T
                ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
                dk[r, :len(keys)] += scale * (ds[:, cols].T @ qi)
                dv[r, :len(keys)] += p[:, cols].T @ doi
    return dk, dv

