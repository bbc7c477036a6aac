// Internal interface between the C-ABI layer (sala_api.cpp) and the HIP
// kernel files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sala {

// The linear layer's neighbours, applied inside its kernels: RMS norm of q
// and k over the head dimension (weights gamma_q / gamma_k, nullptr = none),
// rotate-half RoPE at absolute positions (rope_base <= 0: none) and the output
// gate o * sigmoid(gate) (gate nullptr: none).
struct LinearNeighbours {
  const float *gamma_q, *gamma_k;
  float eps;
  float rope_base;
  long long pos0;          // prefill: position of token 0
  const long long *pos;    // decode: device array [B] of positions
  const void *gate;        // same layout and dtype as o
};

struct LinearPrefillArgs {
  int dtype, B, H, N, d, chunk;
  const void *q, *k, *v;
  void *o;
  const float *decay, *state_in;
  float *state_out;
  void *ws;
  const LinearNeighbours *nb;  // nullptr: the plain layer
  // the backward passes' switches (0 for the forward operation): tokens in
  // reverse order; initial state entering one decay step late; initial state
  // read transposed; final state written times lam
  int rev = 0, lag = 0, state_T = 0, scale_final = 0;
  // 1: the segment states a previous pass of the same plan left in ws are this
  // pass's states transposed (the dV pass after the dK pass); no aggregate or scan
  int reuse_states_T = 0;
};
size_t linear_prefill_workspace(int dtype, int B, int H, int N, int d, int chunk);
hipError_t launch_linear_prefill(const LinearPrefillArgs &a, hipStream_t st);

struct LinearBackwardArgs {
  int dtype, B, H, N, d, chunk;
  const void *q, *k, *v, *dout;
  const float *decay, *state_in, *dstate_out;
  void *dq, *dk, *dv;
  float *dstate_in;
  void *ws;
};
// Workspace: the same as the forward operation's (the passes run in turn).
hipError_t launch_linear_prefill_backward(const LinearBackwardArgs &a, hipStream_t st);

struct QkNormRopeArgs {
  int dtype, B, H, N, d;
  const void *x;
  void *out;
  const float *gamma;
  float eps, rope_base;
  long long pos0;
};
hipError_t launch_qk_norm_rope(const QkNormRopeArgs &a, hipStream_t st);
hipError_t launch_output_gate(int dtype, size_t n, const void *o, const void *g, void *out, hipStream_t st);

struct LinearDecodeArgs {
  int dtype, B, H, d;
  const void *q, *k, *v;
  void *o;
  const float *decay;
  float *state;
  const LinearNeighbours *nb;  // nullptr: the plain step
};
hipError_t launch_linear_decode(const LinearDecodeArgs &a, hipStream_t st);

struct SparseSelectArgs {
  int dtype, B, Hq, Hkv, d, Nq, L, block, topk, n_init, n_local;
  const void *q, *k;
  float *k_pooled;
  int32_t *idx;
  float *scores;  // user buffer or nullptr
  void *ws;
  int Lc;         // decode without k: k_pooled rows hold ceil(Lc / block) blocks (0: L)
};
// Decode step: token pos written into caches of Lc tokens per (b, KV head),
// and the pooled key of its block recomputed.
hipError_t launch_kv_append(int dtype, int BH, int Lc, int d, int block, int pos, const void *k_new,
                            const void *v_new, void *k_cache, void *v_cache, float *k_pooled, hipStream_t st);
// Continued prefill: rows pos0 .. pos0+n-1 of both caches written from [B*Hkv, n, d].
hipError_t launch_kv_write(int dtype, int BH, int Lc, int d, int pos0, int n, const void *k_new, const void *v_new,
                           void *k_cache, void *v_cache, hipStream_t st);
size_t sparse_select_workspace(int dtype, int B, int Hq, int Hkv, int d, int Nq, int L, int block, int topk,
                               int n_init, int n_local, bool want_scores);
hipError_t launch_sparse_select(const SparseSelectArgs &a, hipStream_t st);

struct SparsePrefillArgs {
  int dtype, B, Hq, Hkv, N, d, block, n_sel;
  float scale;
  const void *q, *k, *v;
  const int32_t *idx;
  void *o;
  void *ws;
  int L, Lc;  // continued prefill: N queries are the last of L keys held in rows of Lc tokens (0: N, L)
};
size_t sparse_prefill_workspace(int dtype, int B, int Hq, int Hkv, int N, int d, int block, int n_sel);
hipError_t launch_sparse_prefill(const SparsePrefillArgs &a, hipStream_t st);

struct SparseDecodeArgs {
  int dtype, B, Hq, Hkv, L, d, block, n_sel;
  float scale;
  const void *q, *k_cache, *v_cache;
  const int32_t *idx;
  void *o;
  void *ws;
  int Lc;  // cache rows hold Lc tokens (0: L)
};
size_t sparse_decode_workspace(int dtype, int B, int Hq, int Hkv, int L, int d, int block, int n_sel);
hipError_t launch_sparse_decode(const SparseDecodeArgs &a, hipStream_t st);

struct SparseBackwardArgs {
  int dtype, B, Hq, Hkv, N, d, block, n_sel;
  float scale;
  const void *q, *k, *v;
  const int32_t *idx;
  const void *dout;
  void *dq, *dk, *dv;
  void *ws;
};
size_t sparse_backward_workspace(int dtype, int B, int Hq, int Hkv, int N, int d, int block, int n_sel);
hipError_t launch_sparse_backward(const SparseBackwardArgs &a, hipStream_t st);

// Dense causal attention (every block up to the query's own): the sparse
// kernel with the block list replaced by 0..i.
hipError_t launch_dense_prefill(const SparsePrefillArgs &a, hipStream_t st);

// Device address of this device's fixed scratch array (allocation-free entry points).
hipError_t noalloc_scratch(void **out);

// Measured-ceiling microkernels (not on the attention path).
hipError_t launch_ceiling_mfma(int workgroups, int iters, float *out, hipStream_t st);
hipError_t launch_ceiling_copy(const void *src, void *dst, size_t bytes, hipStream_t st);
hipError_t launch_ceiling_read(const void *src, size_t bytes, float *out, hipStream_t st);

// Debug check of idx rows (see checks.hip): *result = ~0 when every row is
// valid, else (first bad row << 32 | entry << 2 | code).  Synchronizes st.
hipError_t debug_check_idx(const int32_t *idx, long long rows, int n_sel, int nqb, int nb, int own, hipStream_t st,
                           unsigned long long *result);

}  // namespace sala
