"""The linear layer's neighbours in float64 -- test infrastructure only.

What the pages fix:
  * HyPE: the linear-attention layers apply rotary position embedding (RoPE)
    to keep the relative order of tokens; the sparse layers apply none
    ([P2] 技術概要 §2.2; [P3] §2 Architektur-Hybridisierung, HyPE).
  * QK normalisation is added to stabilise activations, and an output gate
    follows every attention block against the attention sink
    ([P3] §2 Architektur-Hybridisierung, "Zusätzliche Verbesserungen").

Readings where the pages are silent (listed in the design notes):
  * QK normalisation is RMS normalisation over the head dimension with a
    learned per-feature weight gamma (one vector for queries, one for keys,
    shared by the heads of a layer) and eps = 1e-6 inside the root:
        x_hat = x / sqrt(mean(x**2) + eps) * gamma.
  * RoPE uses the rotate-half pairing: feature i is rotated with feature
    i + d/2 (i < d/2) by the angle p * theta_i, theta_i = base**(-2 i / d),
    base = 10000, p = the token's absolute position (0 for the first token of
    the sequence; a continued prefill or a decode step passes its offset).
  * Order inside a linear layer: normalise, then rotate, for q and for k;
    v is untouched.  The decayed linear attention then runs on the
    transformed q and k.
  * The output gate is elementwise: o * sigmoid(g), g being a gate
    pre-activation of the same shape as o, computed upstream from the
    layer input.
  * Where the transformed vectors are stored: with store="bf16" the
    normalised and rotated q and k are rounded once to bf16 (round to
    nearest even) before the attention, as an unfused producer writing
    them to memory at the inputs' precision would leave them; v and the
    attention itself stay in float64.  store=None keeps them exact.

Functions:
  round_bf16                           -- float64 -> nearest bf16 value (ties to even)
  rms_norm, rope, output_gate          -- the three neighbours
  linear_layer_fused                   -- norm + RoPE -> linear attention -> gate
  linear_decode_fused                  -- the same for one token per (b, h)
"""

import numpy as np

from . import linear as _lin


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, gamma, eps=1e-6):
    """x / sqrt(mean over the last axis of x**2 + eps) * gamma (gamma: [d])."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * _f64(gamma)


def rope_angles(positions, d, base=10000.0):
    """angle[p, i] = positions[p] * base**(-2 i / d) for i < d/2."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    return _f64(positions)[:, None] * theta[None, :]


def rope(x, positions, base=10000.0):
    """Rotate-half RoPE of x [..., n, d] at the given absolute positions [n].

    y_i       = x_i cos(a_i) - x_{i+d/2} sin(a_i)
    y_{i+d/2} = x_{i+d/2} cos(a_i) + x_i sin(a_i),   a_i = p * theta_i.
    """
    x = _f64(x)
    d = x.shape[-1]
    a = rope_angles(positions, d, base)
    c, s = np.cos(a), np.sin(a)
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def output_gate(o, g):
    """o * sigmoid(g), elementwise."""
    g = _f64(g)
    return _f64(o) / (1.0 + np.exp(-g))


def round_bf16(x):
    """The bf16 value nearest to each element (ties to the even significand).

    bf16 keeps the upper 16 bits of an IEEE fp32 pattern: the value is first
    taken to fp32 (nearest), then the low 16 bits are rounded off by adding
    0x7FFF plus the lowest kept bit and truncating.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _prologue(x, gamma, eps, base, positions, store=None):
    transformed = False
    if gamma is not None:
        x = rms_norm(x, gamma, eps)
        transformed = True
    if base is not None and base > 0:
        x = rope(x, positions, base)
        transformed = True
    if transformed and store == "bf16":
        x = round_bf16(x)
    return _f64(x)


def linear_layer_fused(q, k, v, decay=None, state_in=None, gamma_q=None, gamma_k=None, eps=1e-6,
                       rope_base=10000.0, pos0=0, gate=None, store=None):
    """One linear layer with its neighbours, batched [B, H, N, d].

    q_hat = RoPE(rms_norm(q)), k_hat = RoPE(rms_norm(k)) at positions
    pos0 .. pos0 + N - 1; (o, S) = decayed linear attention of (q_hat, k_hat, v);
    o <- o * sigmoid(gate).  A None gamma skips that normalisation, a None or
    non-positive rope_base skips RoPE, a None gate skips the gate; store="bf16"
    rounds the transformed q and k to bf16 (see the module docstring).
    Returns (o [B, H, N, d_v], state_out [B, H, d_k, d_v]).
    """
    n = np.shape(q)[2]
    pos = np.arange(n, dtype=np.float64) + float(pos0)
    qh = _prologue(q, gamma_q, eps, rope_base, pos, store)
    kh = _prologue(k, gamma_k, eps, rope_base, pos, store)
    o, st = _lin.linear_prefill(qh, kh, v, decay, state_in)
    if gate is not None:
        o = output_gate(o, gate)
    return o, st


def linear_layer_fused_rows(q, k, v, lam, rows, state_in=None, gamma_q=None, gamma_k=None, eps=1e-6,
                            rope_base=10000.0, pos0=0, gate=None, store=None):
    """linear_layer_fused for one head [N, d] at chosen query rows (long sequences)."""
    n = np.shape(q)[0]
    last = int(max(rows)) + 1
    pos = np.arange(last, dtype=np.float64) + float(pos0)
    kh = _prologue(k[:last], gamma_k, eps, rope_base, pos, store)
    qh = np.zeros((last, np.shape(q)[1]))
    rows_i = [int(r) for r in rows]
    qh[rows_i] = _prologue(_f64(q)[rows_i], gamma_q, eps, rope_base, pos[rows_i], store)
    o = _lin.linear_attention_rows(qh, kh, _f64(v)[:last], lam, rows_i, state_in)
    if gate is not None:
        o = output_gate(o, _f64(gate)[rows_i])
    assert last <= n
    return o


def linear_decode_fused(q, k, v, state, decay=None, gamma_q=None, gamma_k=None, eps=1e-6,
                        rope_base=10000.0, pos=None, gate=None, store=None):
    """One decode token per (b, h): q, k, v [B, H, d], state [B, H, d_k, d_v],
    pos [B] absolute positions.  Returns (o [B, H, d_v], state')."""
    b_, h_, _ = np.shape(q)
    qh = np.zeros(np.shape(q))
    kh = np.zeros(np.shape(k))
    for b in range(b_):
        p = np.array([float(pos[b])])
        qh[b] = _prologue(_f64(q)[b][:, None, :], gamma_q, eps, rope_base, p, store)[:, 0, :]
        kh[b] = _prologue(_f64(k)[b][:, None, :], gamma_k, eps, rope_base, p, store)[:, 0, :]
    o, st = _lin.linear_decode_batched(qh, kh, v, state, decay)
    if gate is not None:
        o = output_gate(o, gate)
    return o, st
