"""Block-sparse softmax attention (InfLLM-V2 style) in float64 -- test infrastructure only.

What the pages fix:
  * One layer in four is InfLLM-V2 sparse attention ([P1] abstract;
    [P2] 技術概要 §2.1; [P3] §2 Architektur-Hybridisierung).
  * It adds no parameters and can reach relevant tokens anywhere in the
    context, while the layer keeps its complete KV cache ([P2] §1 and §2.1;
    [P3] §1 Problemstellung and §2): sparse compute, dense storage.
  * Block selection of this family works from coarse block representations
    ([P4] abstract, which names InfLLM v2 as such a method).
  * Sparse layers apply no rotary encoding ([P2] §2.2; [P3] §2), so Q/K
    arrive as given.
  * The attention over the chosen tokens is exact softmax attention restricted
    to a block mask, the block-sparse variant of IO-aware exact attention
    ([P5] FlashAttention entry).

Readings where the pages are silent (listed in the design notes):
  * Block representation: the mean of the keys of a block (parameter-free).
  * Query representation: the mean over the block's query tokens and over the
    query heads sharing one KV head (one selection per KV head and query
    block, shared by the whole GQA group).
  * Score of key block j for query block i: qbar_i . kbar_j / sqrt(d).
  * Forced blocks: the first n_init blocks and the n_local blocks ending at
    the query's own block.  Candidates: the complete blocks strictly between
    them.  The top-k candidates by score are added (exact ties go to the
    smaller block index); with fewer candidates than k, all are taken.
  * The selected list is written ascending and padded with -1.
  * Decode: the cache holds L tokens including the current one; the query is
    at position L-1 and its query block is that single token (pooled over
    the group's heads).
"""

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def n_blocks(length, block):
    return (length + block - 1) // block


def pool_blocks(x, block):
    """Mean over the valid tokens of each block: x [L, d] -> [ceil(L/block), d]."""
    x = _f64(x)
    length = x.shape[0]
    out = np.zeros((n_blocks(length, block), x.shape[1]))
    for j in range(out.shape[0]):
        out[j] = x[j * block:(j + 1) * block].mean(axis=0)
    return out


def forced_blocks(i, n_init, n_local):
    """Initial blocks 0..n_init-1 and local blocks i-n_local+1..i, clipped to [0, i]."""
    f = set(range(0, min(n_init, i + 1)))
    f |= set(range(max(0, i - n_local + 1), i + 1))
    return f


def candidate_blocks(i, length, block, n_init, n_local):
    """Complete blocks j with n_init <= j <= i - n_local (never a forced block)."""
    return [j for j in range(n_init, i - n_local + 1) if (j + 1) * block <= length]


def top_k(scores, cands, k):
    """The min(k, len(cands)) candidates with the largest score; equal scores -> smaller index first."""
    cands = np.asarray(cands, dtype=np.int64)
    if k <= 0 or cands.size == 0:
        return []
    s = np.asarray([scores[j] for j in cands], dtype=np.float64)
    order = np.lexsort((cands, -s))  # primary: -score ascending; secondary: index ascending
    return sorted(int(j) for j in cands[order[:k]])


def select_row(scores, i, length, block, topk, n_init, n_local):
    """Selected block list for query block i: ascending, padded with -1 to topk+n_init+n_local."""
    width = topk + n_init + n_local
    sel = forced_blocks(i, n_init, n_local)
    sel |= set(top_k(scores, candidate_blocks(i, length, block, n_init, n_local), topk))
    row = sorted(sel)
    assert len(row) <= width
    return row + [-1] * (width - len(row))


def sparse_select_prefill(q, k, block=64, topk=64, n_init=1, n_local=2):
    """Prefill selection.  q [B, Hq, N, d], k [B, Hkv, N, d].

    Returns (idx [B, Hkv, NQB, W] int64, scores [B, Hkv, NQB, NB] float64,
    kbar [B, Hkv, NB, d]).  scores[i, j] = qbar_i . kbar_j / sqrt(d) for all j.
    """
    q, k = _f64(q), _f64(k)
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    nb = n_blocks(n, block)
    width = topk + n_init + n_local
    idx = np.full((b_, hkv, nb, width), -1, dtype=np.int64)
    scores = np.zeros((b_, hkv, nb, nb))
    kbar = np.zeros((b_, hkv, nb, d))
    for b in range(b_):
        for h in range(hkv):
            kbar[b, h] = pool_blocks(k[b, h], block)
            # qbar_i: mean over the G heads of the group and the tokens of block i
            qbar = np.zeros((nb, d))
            for i in range(nb):
                qbar[i] = q[b, h * g:(h + 1) * g, i * block:(i + 1) * block].reshape(-1, d).mean(axis=0)
            scores[b, h] = (qbar @ kbar[b, h].T) / math.sqrt(d)
            for i in range(nb):
                idx[b, h, i] = select_row(scores[b, h, i], i, n, block, topk, n_init, n_local)
    return idx, scores, kbar


def sparse_select_prefill_rows(q, k, blocks, block=64, topk=64, n_init=1, n_local=2):
    """The prefill selection of ``sparse_select_prefill`` for chosen query blocks only.

    q [B, Hq, N, d] and k [B, Hkv, N, d] may be any arrays indexable like NumPy
    arrays (only the rows read are converted); blocks: query block indices.
    Returns (idx [B, Hkv, len(blocks), W], scores [B, Hkv, len(blocks), NB],
    kbar [B, Hkv, NB, d]) with the same definitions.
    """
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    nb = n_blocks(n, block)
    width = topk + n_init + n_local
    idx = np.full((b_, hkv, len(blocks), width), -1, dtype=np.int64)
    scores = np.zeros((b_, hkv, len(blocks), nb))
    kbar = np.zeros((b_, hkv, nb, d))
    for b in range(b_):
        for h in range(hkv):
            kbar[b, h] = pool_blocks(k[b, h], block)
            for r, i in enumerate(blocks):
                qbar = _f64(q[b, h * g:(h + 1) * g, i * block:(i + 1) * block]).reshape(-1, d).mean(axis=0)
                scores[b, h, r] = (kbar[b, h] @ qbar) / math.sqrt(d)
                idx[b, h, r] = select_row(scores[b, h, r], i, n, block, topk, n_init, n_local)
    return idx, scores, kbar


def sparse_attention_prefill(q, k, v, idx, block=64, scale=None):
    """Softmax attention over the selected token sets.

    For token t in query block i and query head hq (KV head hq // G):
      A(t) = { s in the blocks listed in idx[b, hq // G, i] : s <= t, s < N }
      o_t  = sum_{s in A(t)} softmax_s(scale * q_t . k_s) v_s
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = np.zeros((b_, hq, n, v.shape[-1]))
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
                o[b, h, t0:t1] = (p / p.sum(axis=1, keepdims=True)) @ v[b, kv, toks]
    return o


def sparse_attention_prefill_rows(q, k, v, idx, rows, block=64, scale=None):
    """The same restricted softmax, for selected (b, hq, t) triples only.  Returns [len(rows), d_v]."""
    hq, d = q.shape[1], q.shape[-1]
    n = q.shape[2]
    g = hq // k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = np.zeros((len(rows), v.shape[-1]))
    for r, (b, h, t) in enumerate(rows):
        kv = h // g
        i = t // block
        toks = np.concatenate([np.arange(j * block, min((j + 1) * block, n))
                               for j in idx[b, kv, i] if j >= 0])
        toks = toks[toks <= t]
        logits = scale * (_f64(k[b, kv, toks]) @ _f64(q[b, h, t]))
        logits -= logits.max()
        p = np.exp(logits)
        out[r] = (p / p.sum()) @ _f64(v[b, kv, toks])
    return out


def dense_causal_attention(q, k, v, scale=None):
    """Textbook causal softmax attention, GQA: q [B, Hq, N, d], k/v [B, Hkv, N, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, hq, n, d = q.shape
    g = hq // k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = np.zeros((b_, hq, n, v.shape[-1]))
    causal = np.tril(np.ones((n, n), dtype=bool))
    for b in range(b_):
        for h in range(hq):
            s = scale * (q[b, h] @ k[b, h // g].T)
            s = np.where(causal, s, -np.inf)
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            o[b, h] = (p / p.sum(axis=1, keepdims=True)) @ v[b, h // g]
    return o


# ---------------------------------------------------------------- decode

def sparse_select_decode(q, kbar, length, block=64, topk=64, n_init=1, n_local=2):
    """Decode selection for the query at position length-1.

    q [B, Hq, d]; kbar [B, Hkv, NB, d] block means of the cache.
    qbar = mean over the G heads of the group; its query block is
    i = (length-1) // block.  Returns (idx [B, Hkv, W], scores [B, Hkv, NB]).
    """
    q, kbar = _f64(q), _f64(kbar)
    b_, hq, d = q.shape
    hkv = kbar.shape[1]
    g = hq // hkv
    i = (length - 1) // block
    width = topk + n_init + n_local
    idx = np.full((b_, hkv, width), -1, dtype=np.int64)
    scores = np.zeros((b_, hkv, kbar.shape[2]))
    for b in range(b_):
        for h in range(hkv):
            qbar = q[b, h * g:(h + 1) * g].mean(axis=0)
            scores[b, h] = (kbar[b, h] @ qbar) / math.sqrt(d)
            idx[b, h] = select_row(scores[b, h], i, length, block, topk, n_init, n_local)
    return idx, scores


def sparse_attention_decode(q, k_cache, v_cache, idx, length, block=64, scale=None):
    """Softmax over every cached token (< length) of the selected blocks.  q [B, Hq, d] -> [B, Hq, d_v]."""
    q = _f64(q)
    b_, hq, d = q.shape
    g = hq // k_cache.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = np.zeros((b_, hq, v_cache.shape[-1]))
    for b in range(b_):
        for h in range(hq):
            kv = h // g
            toks = np.concatenate([np.arange(j * block, min((j + 1) * block, length))
                                   for j in idx[b, kv] if j >= 0])
            logits = scale * (_f64(k_cache[b, kv, toks]) @ q[b, h])
            logits -= logits.max()
            p = np.exp(logits)
            o[b, h] = (p / p.sum()) @ _f64(v_cache[b, kv, toks])
    return o
