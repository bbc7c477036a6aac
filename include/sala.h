/*
 * sala.h -- C ABI of libsala, the MI355X (gfx950) hot path of the SALA hybrid
 * attention layer group: three Lightning (causal, decayed linear) attention
 * layers for every InfLLM-V2-style block-sparse softmax layer.
 *
 * Sources for the operations (the pages describing the method):
 *   "MiniCPM-SALA: Hybridizing Sparse and Linear Attention for Efficient
 *   Long-Context Modeling" -- abstract (fugumt.com summary of arXiv
 *   2602.11761); gist.science (ja) technical summary 技術概要 sections 1,
 *   2.1, 2.2; gist.science (de) technical summary section 2 "Methodik",
 *   subsection "Architektur-Hybridisierung".  Block selection from coarse
 *   block representations: "Punctuation-aware Hybrid Trainable Sparse
 *   Attention for Large Language Models", abstract.  Exact softmax attention
 *   restricted to a block mask: the FlashAttention entry in the related list
 *   of the fugumt.com page for arXiv 2607.21752.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, contiguous, row-major.  Q/K/V/O use the layout
 *     [B, heads, tokens, d] (head-major), so one (head, 64-token block) of K or
 *     V is one contiguous run.
 *   - Every pointer argument is a DEVICE pointer (memory from hipMalloc or
 *     torch on the current device) unless stated otherwise, 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued asynchronously on it; nothing synchronises.
 *   - The caller owns every buffer, including the workspace `ws`.  libsala
 *     never allocates or frees device memory and keeps no mutable global
 *     state, so calls on different streams do not interfere (they must not
 *     share output or workspace buffers while in flight).
 *   - Arguments are validated on the host before any HIP call; on error no
 *     device work is enqueued and a negative sala_status is returned.
 *     sala_last_error() then returns a thread-local message naming the
 *     offending argument.  No C++ exception crosses the ABI.
 *   - Kernel faults surface at the caller's next synchronisation, as usual.
 */
#ifndef SALA_H
#define SALA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SALA_F32 = 0,  /* fp32 inputs/outputs, fp32 arithmetic                      */
  SALA_BF16 = 1  /* bf16 inputs/outputs, bf16 MFMA with fp32 accumulation     */
} sala_dtype;

typedef enum {
  SALA_OK = 0,
  SALA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or shape     */
  SALA_ERR_UNSUPPORTED = -2, /* valid request outside what libsala covers      */
  SALA_ERR_WORKSPACE = -3,   /* ws too small (query the *_workspace call)      */
  SALA_ERR_HIP = -4          /* a HIP launch/runtime call failed               */
} sala_status;

/* ------------------------------------------------------------------------
 * sala_linear_prefill -- causal linear attention with per-head decay over a
 * whole sequence, continuing from an optional carried state.
 *
 * Definition (per batch row b and head h, lam = decay[h]):
 *   o_t   = sum_{s<=t} lam^(t-s) (q_t . k_s) v_s  +  lam^(t+1) q_t S_in
 *   S_out = lam^N S_in + sum_{s<N} lam^(N-1-s) k_s v_s^T
 * i.e. (Q K^T masked by the decayed causal mask) V, with no feature map, no
 * normaliser and no 1/sqrt(d).  The pages give Lightning attention's O(N)
 * cost through a recursive formulation (gist.science (de) section 2,
 * "Architektur-Hybridisierung") and its closeness to softmax attention
 * (gist.science (ja) section 2.1); the decay and the absence of a normaliser
 * are the plainest reading consistent with both.
 *
 *   dtype        SALA_BF16 (MFMA path) or SALA_F32.
 *   B, H, N, d   batch, heads, tokens (N >= 1), head dim (64 or 128).
 *   chunk        intra-chunk length of the bf16 path (64 or 128); any value in
 *                {64, 128} gives the same result up to rounding.  The fp32
 *                path works in tiles of 32 tokens whatever the chunk.
 *   q, k, v      [B, H, N, d] of dtype.
 *   o            [B, H, N, d] of dtype (output).
 *   decay        [H] fp32 in [0, 1], or NULL for lam = 1 on every head.
 *   state_in     [B, H, d, d] fp32, S[d_k][d_v], or NULL for a zero state.
 *   state_out    [B, H, d, d] fp32 or NULL; may alias state_in.
 *   ws, ws_bytes workspace of at least sala_linear_prefill_workspace(...)
 *                bytes (may be NULL when that is 0).
 * bf16: one head's rows N * d * 2 bytes must stay under 2 GiB (the kernels
 * address a head's rows with 32-bit offsets); larger N returns
 * SALA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
int sala_linear_prefill(int dtype, int B, int H, int N, int d, int chunk,
                        const void *q, const void *k, const void *v, void *o,
                        const float *decay, const float *state_in, float *state_out,
                        void *ws, size_t ws_bytes, void *stream);

size_t sala_linear_prefill_workspace(int dtype, int B, int H, int N, int d, int chunk);

/* ------------------------------------------------------------------------
 * sala_linear_prefill_backward -- gradients of sala_linear_prefill, for the
 * continual training by which the hybrid model is obtained from a pretrained
 * Transformer (MiniCPM-SALA abstract, "cost-effective continual training
 * framework"; gist.science (ja) 技術概要 section 2.3; gist.science (de)
 * section 2, "Trainingsstrategie").  For a loss L with dout = dL/do and
 * dstate_out = dL/dS_out (lam = decay[h], D[t,s] = lam^(t-s) for s <= t):
 *   dq       = ((dO V^T) * D) K + diag(lam^(t+1)) dO S_in^T
 *   dk       = ((dO V^T) * D)^T Q + diag(lam^(N-1-s)) V dS_out^T
 *   dv       = ((Q K^T) * D)^T dO + diag(lam^(N-1-s)) K dS_out
 *   dstate_in = Q^T diag(lam^(t+1)) dO + lam^N dS_out
 * the chain rule through the definition above (no approximation).
 *
 *   dtype, B, H, N, d, chunk, decay, state_in: as for sala_linear_prefill
 *                (the forward call's arguments).
 *   q, k, v      [B, H, N, d] of dtype: the forward call's inputs.
 *   dout         [B, H, N, d] of dtype: dL/do.
 *   dstate_out   [B, H, d, d] fp32 or NULL (L does not depend on S_out).
 *   dq, dk, dv   [B, H, N, d] of dtype (outputs); none may overlap q, k, v
 *                or dout.
 *   dstate_in    [B, H, d, d] fp32 or NULL (output, dL/dS_in).
 *   ws, ws_bytes at least sala_linear_prefill_workspace(...) bytes for the
 *                same arguments (three passes run in turn and share it).
 * Errors as sala_linear_prefill; an output equal to an input pointer:
 * SALA_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------ */
int sala_linear_prefill_backward(int dtype, int B, int H, int N, int d, int chunk,
                                 const void *q, const void *k, const void *v, const void *dout,
                                 const float *decay, const float *state_in, const float *dstate_out,
                                 void *dq, void *dk, void *dv, float *dstate_in,
                                 void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * sala_linear_decode -- one token of the same recurrence:
 *   S <- lam S + k v^T ;  o = q S        (state updated in place)
 *
 *   q, k, v   [B, H, d] of dtype (one token per (b, h)).
 *   o         [B, H, d] of dtype (output).
 *   decay     [H] fp32 or NULL (= 1).
 *   state     [B, H, d, d] fp32, read and overwritten.
 * ------------------------------------------------------------------------ */
int sala_linear_decode(int dtype, int B, int H, int d,
                       const void *q, const void *k, const void *v, void *o,
                       const float *decay, float *state, void *stream);

/* ------------------------------------------------------------------------
 * sala_linear_prefill_fused / sala_linear_decode_fused -- the linear layer
 * with its neighbours applied inside the kernels, so q, k and o make no
 * extra round trip through memory.  The pages add QK normalisation and an
 * output gate after every attention block, and give the linear layers
 * rotary position embedding (HyPE: none on the sparse layers)
 * (MiniCPM-SALA, gist.science (ja) 技術概要 section 2.2; gist.science (de)
 * section 2, "Architektur-Hybridisierung").  Forms used here:
 *   x_hat  = x / sqrt(mean_i x_i^2 + eps) * gamma          (q with gamma_q,
 *            k with gamma_k; NULL gamma: that vector is not normalised)
 *   RoPE   rotate-half: feature i < d/2 is turned with feature i + d/2 by
 *          p * rope_base^(-2i/d) at the token's absolute position p
 *          (rope_base 0: no RoPE); applied after the normalisation
 *   o      <- o * sigmoid(gate)  elementwise (gate NULL: no gate)
 * then the decayed linear attention of sala_linear_prefill / _decode runs on
 * the transformed q and k (v untouched).  The transformed q and k are
 * rounded to bf16 once, as an unfused producer would store them.
 *
 * prefill: as sala_linear_prefill, bf16 only (SALA_ERR_UNSUPPORTED for fp32);
 *   the tokens sit at positions pos0 .. pos0 + N - 1 (pos0 in [0, 2^40));
 *   gate [B, H, N, d] bf16 or NULL; gamma_q, gamma_k [d] fp32 or NULL;
 *   one head's rows N * d * 2 bytes must stay under 2 GiB.  Same workspace
 *   as sala_linear_prefill (sala_linear_prefill_workspace).
 * decode: as sala_linear_decode (bf16 or fp32); pos [B] int64 device array of
 *   the token positions (required when rope_base > 0); gate [B, H, d] of dtype
 *   or NULL.  The state is updated in place.
 * Errors: eps negative or not finite, rope_base neither 0 nor a finite base
 * > 1, misaligned optional pointers: SALA_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------ */
int sala_linear_prefill_fused(int dtype, int B, int H, int N, int d, int chunk,
                              const void *q, const void *k, const void *v, void *o,
                              const float *decay, const float *state_in, float *state_out,
                              const float *gamma_q, const float *gamma_k, float eps,
                              float rope_base, long long pos0, const void *gate,
                              void *ws, size_t ws_bytes, void *stream);

int sala_linear_decode_fused(int dtype, int B, int H, int d,
                             const void *q, const void *k, const void *v, void *o,
                             const float *decay, float *state,
                             const float *gamma_q, const float *gamma_k, float eps,
                             float rope_base, const long long *pos, const void *gate,
                             void *stream);

/* ------------------------------------------------------------------------
 * sala_qk_norm_rope -- the same neighbours as standalone streaming kernels,
 * for the sparse layers (QK normalisation without RoPE, per HyPE) and for an
 * unfused pipeline (MiniCPM-SALA, gist.science (ja) 技術概要 section 2.2;
 * gist.science (de) section 2, "Architektur-Hybridisierung").
 *   x, out  [B, H, N, d] of dtype (out may be x): per row, the RMS norm with
 *           weight gamma [d] fp32 (NULL: none), then rotate-half RoPE at
 *           position pos0 + t for token t (rope_base 0: none); same forms and
 *           errors as the fused calls.
 * sala_output_gate -- out = o * sigmoid(gate), elementwise over n elements of
 *   dtype (n a positive multiple of 8; out may be o).
 * ------------------------------------------------------------------------ */
int sala_qk_norm_rope(int dtype, int B, int H, int N, int d, const void *x, void *out,
                      const float *gamma, float eps, float rope_base, long long pos0,
                      void *stream);

int sala_output_gate(int dtype, size_t n, const void *o, const void *gate, void *out,
                     void *stream);

/* ------------------------------------------------------------------------
 * The sparse layer in a generation loop over a KV cache kept at a fixed
 * capacity: sparse layers keep the whole KV cache ("dense storage") and
 * reach all of it with sparse compute (MiniCPM-SALA, gist.science (ja)
 * 技術概要 section 1 and 2.1); the model decodes contexts of up to 1M tokens
 * on one GPU (same page, section 4.3).
 *
 * Layout shared by both calls:
 *   k_cache, v_cache  [B, Hkv, capacity, d] of dtype; row t holds token t.
 *   k_pooled          [B, Hkv, ceil(capacity / block), d] fp32; entry j holds
 *                     the mean of block j's tokens written so far.
 * Before a call that writes tokens from position p on, rows 0 .. p-1 hold the
 * earlier tokens and k_pooled holds their blocks (as earlier calls left them).
 * Selection and attention follow sala_sparse_select / sala_sparse_prefill /
 * sala_sparse_decode for the keys 0 .. (last written token).
 *
 * sala_sparse_prefill_chunk -- n tokens at positions pos0 .. pos0 + n - 1:
 *   q [B, Hq, n, d], k_new, v_new [B, Hkv, n, d] (the chunk's keys and
 *   values, written into the caches); the pooled keys of the blocks the chunk
 *   fills are recomputed; every query block of the chunk selects among all
 *   cached blocks; o [B, Hq, n, d]; idx [B, Hkv, ceil(n / block), n_sel].
 *   n > 1 needs pos0 % block == 0 (SALA_ERR_UNSUPPORTED otherwise); n == 1 is
 *   one decode step.  pos0 + n <= capacity.  A first chunk (pos0 = 0) is an
 *   ordinary prefill that also fills the caches.
 * sala_sparse_decode_step -- one token at position pos (0 <= pos < capacity):
 *   q [B, Hq, d], k_new, v_new [B, Hkv, d]; writes the token, recomputes the
 *   pooled key of block pos / block, selects for the query at pos (L = pos+1)
 *   and attends; o [B, Hq, d]; idx [B, Hkv, n_sel].
 * Workspaces: at least the *_workspace value for the same arguments (sized
 * for the whole capacity, so one buffer serves a whole generation loop).
 * Results equal sala_sparse_select + sala_sparse_prefill (or
 * sala_sparse_decode) run on the first pos0 + n (pos + 1) tokens bit for bit.
 * ------------------------------------------------------------------------ */
/* ------------------------------------------------------------------------
 * sala_sparse_decode_step_noalloc -- sala_sparse_decode_step for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without
 * ws / ws_bytes, the same kernels and bit-identical results.  The workspace
 * is a fixed device array of SALA_NOALLOC_SCRATCH_BYTES inside the library
 * (one per GPU, held from library load until the process ends); a call whose
 * workspace (sala_sparse_decode_step_workspace at capacity pos + 1) exceeds
 * it returns SALA_ERR_WORKSPACE and enqueues nothing.  The call allocates
 * nothing.  All calls on one GPU share that array: calls that may overlap on
 * one GPU (different streams, no ordering between them) race and must not be
 * made.  Failure to find the array's device address returns SALA_ERR_HIP.
 * ------------------------------------------------------------------------ */
#define SALA_NOALLOC_SCRATCH_BYTES (16u << 20)

int sala_sparse_decode_step_noalloc(int dtype, int B, int Hq, int Hkv, int capacity, int d, int pos, int block,
                                    int topk, int n_init, int n_local, float scale,
                                    const void *q, const void *k_new, const void *v_new,
                                    void *k_cache, void *v_cache, float *k_pooled, int32_t *idx, void *o,
                                    void *stream);

size_t sala_sparse_prefill_chunk_workspace(int dtype, int B, int Hq, int Hkv, int capacity, int d, int n,
                                           int block, int topk, int n_init, int n_local);
int sala_sparse_prefill_chunk(int dtype, int B, int Hq, int Hkv, int capacity, int d, int pos0, int n,
                              int block, int topk, int n_init, int n_local, float scale,
                              const void *q, const void *k_new, const void *v_new,
                              void *k_cache, void *v_cache, float *k_pooled, int32_t *idx, void *o,
                              void *ws, size_t ws_bytes, void *stream);

size_t sala_sparse_decode_step_workspace(int dtype, int B, int Hq, int Hkv, int capacity, int d, int block,
                                         int topk, int n_init, int n_local);
int sala_sparse_decode_step(int dtype, int B, int Hq, int Hkv, int capacity, int d, int pos, int block,
                            int topk, int n_init, int n_local, float scale,
                            const void *q, const void *k_new, const void *v_new,
                            void *k_cache, void *v_cache, float *k_pooled, int32_t *idx, void *o,
                            void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * sala_sparse_select -- block selection for the sparse layer.
 *
 * The sparse layers use InfLLM-V2, which adds no parameters and reaches the
 * whole context while keeping the full KV cache (gist.science (ja) sections
 * 1 and 2.1; gist.science (de) section 2); selection in this family scores
 * coarse block representations (PHSA abstract).  Reading used here:
 *   kbar_j = mean of the keys of block j (the valid ones, for a partial block)
 *   qbar_i = mean over the G = Hq/Hkv query heads of a KV head and over the
 *            query tokens of query block i (decode: the single query token)
 *   score  = qbar_i . kbar_j / sqrt(d), computed in fp32
 *   forced = blocks 0..n_init-1 and i-n_local+1..i (clipped to [0, i])
 *   cands  = complete blocks j with n_init <= j <= i-n_local
 *   chosen = forced U top-min(topk, |cands|) cands by score (exact fp32 ties
 *            go to the smaller j), written ascending, padded with -1.
 *
 *   Nq, L        queries sit at positions L-Nq .. L-1.  Supported: Nq == L
 *                (prefill: NQB = ceil(L/block) query blocks) and Nq == 1
 *                (decode: NQB = 1, query block i = (L-1)/block).
 *   block        64.   topk >= 0, n_init >= 0, n_local >= 0.
 *   q            [B, Hq, Nq, d] of dtype.
 *   k            [B, Hkv, L, d] of dtype, or NULL: then k_pooled must already
 *                hold the block means (decode against a pooled cache).
 *   k_pooled     [B, Hkv, ceil(L/block), d] fp32; written when k != NULL.
 *   idx          [B, Hkv, NQB, topk + n_init + n_local] int32 (output).
 *   scores       optional [B, Hkv, NQB, ceil(L/block)] fp32 (output, entry
 *                (i, j) meaningful only for candidates j of row i), or NULL.
 *   ws, ws_bytes at least sala_sparse_select_workspace(...) bytes.
 * ------------------------------------------------------------------------ */
int sala_sparse_select(int dtype, int B, int Hq, int Hkv, int d, int Nq, int L,
                       int block, int topk, int n_init, int n_local,
                       const void *q, const void *k, float *k_pooled, int32_t *idx,
                       float *scores, void *ws, size_t ws_bytes, void *stream);

size_t sala_sparse_select_workspace(int dtype, int B, int Hq, int Hkv, int d, int Nq, int L,
                                    int block, int topk, int n_init, int n_local);

/* ------------------------------------------------------------------------
 * sala_sparse_prefill -- softmax attention restricted to the selected blocks
 * (block-sparse exact attention, the FlashAttention related-list entry).
 *
 * For query head hq (KV head hq / G) and token t in query block i:
 *   A(t) = { s in the blocks listed in idx[b, hq/G, i] : s <= t }
 *   o_t  = sum_{s in A(t)} softmax_s(scale * q_t . k_s) v_s
 * idx rows list distinct blocks; the list ends at the first negative entry;
 * entries greater than i contribute nothing (they are skipped).  Every row
 * must contain its own block i (the forced local block does).  With the
 * environment variable SALA_DEBUG_CHECK=1, rows that break this (an entry
 * beyond the blocks, a block listed twice, a missing own block) are reported
 * as SALA_ERR_INVALID_ARG before the launch (the stream is synchronized; the
 * check is skipped during graph capture); the same holds for
 * sala_sparse_prefill_backward and sala_sparse_decode.
 *
 *   block        64.   n_sel = idx row length (topk + n_init + n_local).
 *   scale        usually 1/sqrt(d).
 *   q, o         [B, Hq, N, d];  k, v  [B, Hkv, N, d];  idx [B, Hkv, NQB, n_sel].
 *   ws, ws_bytes at least sala_sparse_prefill_workspace(...) bytes (0 in this
 *                version: ws may be NULL).
 * ------------------------------------------------------------------------ */
int sala_sparse_prefill(int dtype, int B, int Hq, int Hkv, int N, int d,
                        int block, int n_sel, float scale,
                        const void *q, const void *k, const void *v, const int32_t *idx,
                        void *o, void *ws, size_t ws_bytes, void *stream);

size_t sala_sparse_prefill_workspace(int dtype, int B, int Hq, int Hkv, int N, int d,
                                     int block, int n_sel);

/* ------------------------------------------------------------------------
 * sala_sparse_prefill_backward -- gradients of sala_sparse_prefill at a fixed
 * selection, for the continual training by which the hybrid is obtained
 * from a pretrained Transformer (MiniCPM-SALA abstract; gist.science (ja)
 * 技術概要 section 2.3; gist.science (de) section 2, "Trainingsstrategie").
 * With p the softmax of row t over A(t), o_t its output, dO = dL/do and
 * D_t = dO_t . o_t:
 *   ds_s = p_s (dO_t . v_s - D_t)
 *   dq_t = scale sum_{s in A(t)} ds_s k_s
 *   dk_s = scale sum over (t, hq) with s in A(t) of ds_s q_t  (all G heads)
 *   dv_s =       sum over (t, hq) with s in A(t) of p_s dO_t
 * The block selection is a top-k and passes no gradient.
 *
 *   dtype        SALA_BF16 (SALA_ERR_UNSUPPORTED otherwise).
 *   B, Hq, Hkv, N, d, block, n_sel, scale, q, k, v, idx: the forward call's.
 *   dout         [B, Hq, N, d]: dL/do.  D_t is formed from the recomputed fp32
 *                probabilities, so the forward's output is not needed.
 *   dq           [B, Hq, N, d]; dk, dv [B, Hkv, N, d] (outputs; every row is
 *                written, rows of never-selected blocks with 0).  None may
 *                overlap an input.
 *   ws, ws_bytes at least sala_sparse_prefill_backward_workspace(...) bytes
 *                (row statistics, the inverted selection and per-item fp32
 *                partial sums of dk, dv; about 0.27 * B * Hkv * N * d * 4
 *                bytes at the workloads' 67 selected blocks).
 * Every sum runs in a fixed order: results repeat bit for bit.
 * ------------------------------------------------------------------------ */
int sala_sparse_prefill_backward(int dtype, int B, int Hq, int Hkv, int N, int d,
                                 int block, int n_sel, float scale,
                                 const void *q, const void *k, const void *v, const int32_t *idx,
                                 const void *dout, void *dq, void *dk, void *dv,
                                 void *ws, size_t ws_bytes, void *stream);

size_t sala_sparse_prefill_backward_workspace(int dtype, int B, int Hq, int Hkv, int N, int d,
                                              int block, int n_sel);

/* ------------------------------------------------------------------------
 * sala_dense_prefill -- plain causal softmax attention over every earlier
 * token (exact attention, the FlashAttention related-list entry): the
 * full-attention layer the sparse layer replaces, for the layer-level
 * comparison with the hybrid group (MiniCPM-SALA abstract: speed against
 * full attention at 256K tokens).  The same kernel as sala_sparse_prefill
 * with every block 0..i of query block i selected.
 *
 *   o_t = sum_{s <= t} softmax_s(scale * q_t . k_s) v_s, GQA as above.
 *   dtype        SALA_BF16 only (SALA_ERR_UNSUPPORTED otherwise).
 *   q, o         [B, Hq, N, d];  k, v  [B, Hkv, N, d];  d in {64, 128}.
 * No workspace.
 * ------------------------------------------------------------------------ */
int sala_dense_prefill(int dtype, int B, int Hq, int Hkv, int N, int d, float scale,
                       const void *q, const void *k, const void *v, void *o, void *stream);

/* ------------------------------------------------------------------------
 * sala_sparse_decode -- one query token per (b, hq) at position L-1 attends
 * to every cached token (< L) of the blocks listed in idx[b, hq/G].
 *
 *   q            [B, Hq, d];  k_cache, v_cache [B, Hkv, L, d];
 *   idx          [B, Hkv, n_sel] int32 (distinct, ends at the first negative);
 *   o            [B, Hq, d] (output).
 *   ws, ws_bytes at least sala_sparse_decode_workspace(...) bytes.
 * ------------------------------------------------------------------------ */
int sala_sparse_decode(int dtype, int B, int Hq, int Hkv, int L, int d,
                       int block, int n_sel, float scale,
                       const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *idx, void *o, void *ws, size_t ws_bytes, void *stream);

size_t sala_sparse_decode_workspace(int dtype, int B, int Hq, int Hkv, int L, int d,
                                    int block, int n_sel);

/* ------------------------------------------------------------------------
 * Measured ceilings (not on the attention path; used by the benchmark to
 * report results against this GPU's practical peaks as well as the
 * published ones).
 *
 * sala_ceiling_mfma: `workgroups` x 512 threads each run `iters` rounds of
 *   8 independent bf16 MFMA 16x16x32 operations (16384 flops each per wave);
 *   out [workgroups * 512] fp32 is only written on an impossible checksum.
 *   Flops per launch: workgroups * 8 * iters * 8 * 16384.
 * sala_ceiling_copy: copies `bytes` (a multiple of 16, both pointers 16-byte
 *   aligned) from src to dst with 16-byte vector loads and stores.
 * sala_ceiling_read: reads `bytes` (a multiple of 16, src 16-byte aligned;
 *   src may be NULL when bytes is 0) with 16-byte vector loads, one
 *   contiguous 16 KiB run per workgroup of 256 threads; out [bytes / 16384 + 1]
 *   fp32 is only written on an impossible checksum.  With bytes = 0 a single
 *   workgroup runs and reads nothing (the cost of a launch that does no work).
 * ------------------------------------------------------------------------ */
int sala_ceiling_mfma(int workgroups, int iters, float *out, void *stream);
int sala_ceiling_copy(const void *src, void *dst, size_t bytes, void *stream);
int sala_ceiling_read(const void *src, size_t bytes, float *out, void *stream);

/* ------------------------------------------------------------------------
 * sala_workspace_bytes -- the workspace query of every entry point behind
 * one call: `op` names the operation and dims[0 .. ndims-1] are the integer
 * arguments of that operation's *_workspace query, in the order listed.
 *
 *   SALA_OP_LINEAR_PREFILL       dtype, B, H, N, d, chunk
 *   SALA_OP_SPARSE_SELECT        dtype, B, Hq, Hkv, d, Nq, L, block, topk, n_init, n_local
 *   SALA_OP_SPARSE_PREFILL       dtype, B, Hq, Hkv, N, d, block, n_sel
 *   SALA_OP_SPARSE_DECODE        dtype, B, Hq, Hkv, L, d, block, n_sel
 *   SALA_OP_SPARSE_PREFILL_CHUNK dtype, B, Hq, Hkv, capacity, d, n, block, topk, n_init, n_local
 *   SALA_OP_SPARSE_DECODE_STEP   dtype, B, Hq, Hkv, capacity, d, block, topk, n_init, n_local
 *   SALA_OP_SPARSE_PREFILL_BACKWARD dtype, B, Hq, Hkv, N, d, block, n_sel
 *   (sala_linear_prefill_backward uses SALA_OP_LINEAR_PREFILL's size)
 *
 * Returns the number of bytes (0: the call needs no workspace), or
 * (size_t)-1 when op is unknown, ndims does not match op, dims is NULL or a
 * dimension does not fit an int; sala_last_error() then says which.
 * ------------------------------------------------------------------------ */
typedef enum {
  SALA_OP_LINEAR_PREFILL = 0,
  SALA_OP_SPARSE_SELECT = 1,
  SALA_OP_SPARSE_PREFILL = 2,
  SALA_OP_SPARSE_DECODE = 3,
  SALA_OP_SPARSE_PREFILL_CHUNK = 4,
  SALA_OP_SPARSE_DECODE_STEP = 5,
  SALA_OP_SPARSE_PREFILL_BACKWARD = 6
} sala_op;

size_t sala_workspace_bytes(int op, const int64_t *dims, int ndims);

/* ------------------------------------------------------------------------ */
const char *sala_status_string(int status);  /* static string, never NULL      */
const char *sala_last_error(void);           /* thread-local detail, never NULL */
const char *sala_version(void);              /* build identification           */

#ifdef __cplusplus
}
#endif

#endif /* SALA_H */
