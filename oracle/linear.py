"""Lightning (causal linear) attention in float64 -- test infrastructure only.

What the pages fix:
  * Lightning Attention is the linear half of the hybrid, used in three of
    every four layers ([P1] abstract; [P2] 技術概要 §2.1; [P3] §2
    Architektur-Hybridisierung).
  * Its cost is O(N) in compute and memory ([P2] §1 and §2.1), reached
    through a recursive formulation ([P3] §2 Architektur-Hybridisierung).
  * Its structure stays close to softmax attention ([P2] §2.1).

Readings where the pages are silent (listed in the design notes):
  * No feature map, no normaliser and no 1/sqrt(d): softmax(Q K^T) V with
    the softmax dropped, i.e. (Q K^T masked) V.  Any positional encoding,
    QK normalisation or output gate ([P2] §2.2, [P3] §2) lives outside this
    operation: inputs are post-positional-encoding Q/K/V.
  * An optional per-head decay lam weights the pair (query t, key s) by
    lam**(t - s) for s <= t (weight 1 on the diagonal), zero for s > t.
    lam = 1 is plain causal linear attention.
  * The carried state is S = sum_s lam**(N-1-s) k_s v_s^T, shape [d_k, d_v],
    so that a query reads it as q @ S.

Forms implemented (all float64):
  linear_attention            -- the quadratic definition (reference form)
  linear_attention_rows       -- the same definition, evaluated for chosen rows
  linear_attention_chunked    -- intra-chunk masked product + inter-chunk state
  linear_attention_recurrent  -- S_t = lam S_{t-1} + k_t v_t^T ; o_t = q_t S_t
  linear_decode               -- one step of the recurrent form
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def decay_mask(lam, n):
    """D[t, s] = lam**(t - s) where s <= t, else 0 (causal decay mask)."""
    t = np.arange(n)
    diff = t[:, None] - t[None, :]
    return np.where(diff >= 0, np.power(float(lam), np.maximum(diff, 0)), 0.0)


def linear_attention(q, k, v, lam=1.0, state_in=None):
    """Quadratic definition for one head.

    q, k, v: [N, d]; state_in: [d_k, d_v] or None (= zero state).
    Returns (o [N, d_v], s_final [d_k, d_v]) with
      o[t]    = sum_{s<=t} lam**(t-s) (q_t . k_s) v_s + lam**(t+1) q_t @ S_in
      s_final = lam**N S_in + sum_s lam**(N-1-s) k_s v_s^T
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lam = float(lam)
    n = q.shape[0]
    o = ((q @ k.T) * decay_mask(lam, n)) @ v
    s_final = k.T @ (np.power(lam, (n - 1 - np.arange(n)))[:, None] * v)
    if state_in is not None:
        s_in = _f64(state_in)
        o = o + np.power(lam, np.arange(1, n + 1))[:, None] * (q @ s_in)
        s_final = s_final + (lam ** n) * s_in
    return o, s_final


def linear_attention_rows(q, k, v, lam, rows, state_in=None):
    """The quadratic definition evaluated only at the given query rows.

    Same formula as ``linear_attention``; each row t needs keys 0..t only,
    so long sequences can be checked on a sample of rows.
    Returns o_rows [len(rows), d_v].
    """
    lam = float(lam)
    out = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    for r, t in enumerate(rows):
        t = int(t)
        qt = _f64(q[t])
        ks = _f64(k[: t + 1])
        vs = _f64(v[: t + 1])
        w = (ks @ qt) * np.power(lam, t - np.arange(t + 1))
        out[r] = w @ vs
        if state_in is not None:
            out[r] += (lam ** (t + 1)) * (qt @ _f64(state_in))
    return out


def final_state(k, v, lam, state_in=None):
    """S_N = lam**N S_in + sum_s lam**(N-1-s) k_s v_s^T (definition of the carried state)."""
    k, v = _f64(k), _f64(v)
    lam = float(lam)
    n = k.shape[0]
    s = k.T @ (np.power(lam, (n - 1 - np.arange(n)))[:, None] * v)
    if state_in is not None:
        s = s + (lam ** n) * _f64(state_in)
    return s


def linear_attention_chunked(q, k, v, lam, chunk, state_in=None):
    """Chunked form for one head (tail chunk may be shorter).

    For each chunk c of length m:
      O_c = ((Q_c K_c^T) * D_m) V_c + diag(lam**(i+1)) Q_c S_{c-1}
      S_c = lam**m S_{c-1} + K_c^T diag(lam**(m-1-j)) V_c
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lam = float(lam)
    n, dv = q.shape[0], v.shape[1]
    s = np.zeros((k.shape[1], dv)) if state_in is None else _f64(state_in).copy()
    o = np.zeros((n, dv))
    for c0 in range(0, n, chunk):
        qc, kc, vc = q[c0:c0 + chunk], k[c0:c0 + chunk], v[c0:c0 + chunk]
        m = qc.shape[0]
        o[c0:c0 + m] = ((qc @ kc.T) * decay_mask(lam, m)) @ vc \
            + np.power(lam, np.arange(1, m + 1))[:, None] * (qc @ s)
        s = (lam ** m) * s + kc.T @ (np.power(lam, m - 1 - np.arange(m))[:, None] * vc)
    return o, s


def linear_attention_recurrent(q, k, v, lam, state_in=None):
    """Recurrent form: S_t = lam S_{t-1} + k_t v_t^T ; o_t = q_t S_t."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    lam = float(lam)
    n, dv = q.shape[0], v.shape[1]
    s = np.zeros((k.shape[1], dv)) if state_in is None else _f64(state_in).copy()
    o = np.zeros((n, dv))
    for t in range(n):
        s = lam * s + np.outer(k[t], v[t])
        o[t] = q[t] @ s
    return o, s


def linear_decode(q, k, v, lam, state):
    """One decode step for one head: S' = lam S + k v^T ; o = q S'.  Returns (o, S')."""
    s = float(lam) * _f64(state) + np.outer(_f64(k), _f64(v))
    return _f64(q) @ s, s


# ---------------------------------------------------------------- batched wrappers

def linear_prefill(q, k, v, decay=None, state_in=None, form="quadratic", chunk=None):
    """Batched [B, H, N, d] driver over the per-head forms above.

    decay: [H] (None = 1 for every head); state_in: [B, H, d_k, d_v] or None.
    Returns (o [B, H, N, d_v], state_out [B, H, d_k, d_v]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, h_, n, _ = q.shape
    dv = v.shape[-1]
    o = np.zeros((b_, h_, n, dv))
    st = np.zeros((b_, h_, k.shape[-1], dv))
    for b in range(b_):
        for h in range(h_):
            lam = 1.0 if decay is None else float(decay[h])
            s_in = None if state_in is None else state_in[b, h]
            if form == "quadratic":
                o[b, h], st[b, h] = linear_attention(q[b, h], k[b, h], v[b, h], lam, s_in)
            elif form == "chunked":
                o[b, h], st[b, h] = linear_attention_chunked(q[b, h], k[b, h], v[b, h], lam, chunk, s_in)
            elif form == "recurrent":
                o[b, h], st[b, h] = linear_attention_recurrent(q[b, h], k[b, h], v[b, h], lam, s_in)
            else:
                raise ValueError(form)
    return o, st


def linear_decode_batched(q, k, v, state, decay=None):
    """Batched decode step: q, k, v [B, H, d], state [B, H, d_k, d_v].  Returns (o, state')."""
    b_, h_, _ = q.shape
    o = np.zeros((b_, h_, v.shape[-1]))
    st = np.zeros(state.shape)
    for b in range(b_):
        for h in range(h_):
            lam = 1.0 if decay is None else float(decay[h])
            o[b, h], st[b, h] = linear_decode(q[b, h], k[b, h], v[b, h], lam, state[b, h])
    return o, st
