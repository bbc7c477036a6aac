// C ABI of libsala: argument validation and dispatch to the HIP launchers.
// Every check runs on the host before any HIP call; on failure nothing is
// enqueued and a negative status is returned with a thread-local message.

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/sala.h"
#include "sala_launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p, name)                                                      \
  do {                                                                            \
    if (!(p)) return fail(SALA_ERR_INVALID_ARG, "%s must not be NULL", name);     \
    if (!aligned16(p)) return fail(SALA_ERR_INVALID_ARG, "%s must be 16-byte aligned", name); \
  } while (0)

#define OPT_PTR(p, name)                                                          \
  do {                                                                            \
    if ((p) && !aligned16(p)) return fail(SALA_ERR_INVALID_ARG, "%s must be 16-byte aligned", name); \
  } while (0)

int check_dtype(int dtype) {
  if (dtype != SALA_F32 && dtype != SALA_BF16) return fail(SALA_ERR_INVALID_ARG, "dtype %d is not SALA_F32/SALA_BF16", dtype);
  return SALA_OK;
}

int check_d(int d) {
  if (d <= 0) return fail(SALA_ERR_INVALID_ARG, "d = %d must be positive", d);
  if (d != 64 && d != 128) return fail(SALA_ERR_UNSUPPORTED, "d = %d: libsala supports 64 and 128", d);
  return SALA_OK;
}

int check_ws(void *ws, size_t have, size_t need) {
  if (need == 0) return SALA_OK;
  if (!ws) return fail(SALA_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (!aligned16(ws)) return fail(SALA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  if (have < need) return fail(SALA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  return SALA_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(SALA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return SALA_OK;
}

// SALA_DEBUG_CHECK=1: the index rows given to the gathering calls are checked
// on the device against their contract before the launch (the stream is
// synchronized; skipped while it is captured into a graph).
int debug_idx(const int32_t *idx, long long rows, int n_sel, int nqb, int nb, int own, void *stream,
              const char *call) {
  const char *env = getenv("SALA_DEBUG_CHECK");
  if (!env || strcmp(env, "1") != 0) return SALA_OK;
  unsigned long long r = ~0ull;
  const hipError_t e = sala::debug_check_idx(idx, rows, n_sel, nqb, nb, own, static_cast<hipStream_t>(stream), &r);
  if (e != hipSuccess) return fail(SALA_ERR_HIP, "%s idx check: %s", call, hipGetErrorString(e));
  if (r == ~0ull) return SALA_OK;
  const long long row = (long long)(r >> 32);
  const int entry = (int)((r & 0xFFFFFFFFull) >> 2), code = (int)(r & 3ull);
  if (code == 1) return fail(SALA_ERR_INVALID_ARG, "%s: idx row %lld entry %d is beyond the %d blocks", call, row, entry, nb);
  if (code == 2) return fail(SALA_ERR_INVALID_ARG, "%s: idx row %lld entry %d lists a block twice", call, row, entry);
  return fail(SALA_ERR_INVALID_ARG, "%s: idx row %lld does not list its own query block %lld", call, row,
              row % (long long)nqb);
}

int check_sparse_common(int B, int Hq, int Hkv, int block, int topk_or_nsel, const char *what) {
  REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1, SALA_ERR_INVALID_ARG, "B, Hq, Hkv must be >= 1");
  REQUIRE(Hq % Hkv == 0, SALA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  REQUIRE(block >= 1, SALA_ERR_INVALID_ARG, "block must be >= 1");
  REQUIRE(block == 64, SALA_ERR_UNSUPPORTED, "block = %d: libsala supports 64", block);
  REQUIRE(topk_or_nsel >= 0, SALA_ERR_INVALID_ARG, "%s must be >= 0", what);
  return SALA_OK;
}

}  // namespace

extern "C" {

const char *sala_status_string(int status) {
  switch (status) {
    case SALA_OK: return "SALA_OK";
    case SALA_ERR_INVALID_ARG: return "SALA_ERR_INVALID_ARG";
    case SALA_ERR_UNSUPPORTED: return "SALA_ERR_UNSUPPORTED";
    case SALA_ERR_WORKSPACE: return "SALA_ERR_WORKSPACE";
    case SALA_ERR_HIP: return "SALA_ERR_HIP";
    default: return "SALA_ERR_UNKNOWN";
  }
}

const char *sala_last_error(void) { return g_err; }

const char *sala_version(void) { return "libsala 0.1 (gfx950)"; }

size_t sala_linear_prefill_workspace(int dtype, int B, int H, int N, int d, int chunk) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128) || (chunk != 64 && chunk != 128)) return 0;
  return sala::linear_prefill_workspace(dtype, B, H, N, d, chunk);
}

int sala_linear_prefill(int dtype, int B, int H, int N, int d, int chunk, const void *q, const void *k,
                        const void *v, void *o, const float *decay, const float *state_in, float *state_out,
                        void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  REQUIRE(B >= 1 && H >= 1 && N >= 1, SALA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if ((s = check_d(d))) return s;
  REQUIRE(chunk == 64 || chunk == 128, SALA_ERR_UNSUPPORTED, "chunk = %d: libsala supports 64 and 128", chunk);
  REQUIRE(dtype != SALA_BF16 || (long long)N * d * 2 < (1ll << 31), SALA_ERR_UNSUPPORTED,
          "one head's rows must stay under 2 GiB");
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(o, "o");
  OPT_PTR(decay, "decay");
  OPT_PTR(state_in, "state_in");
  OPT_PTR(state_out, "state_out");
  if ((s = check_ws(ws, ws_bytes, sala::linear_prefill_workspace(dtype, B, H, N, d, chunk)))) return s;
  sala::LinearPrefillArgs a{dtype, B, H, N, d, chunk, q, k, v, o, decay, state_in, state_out, ws};
  return hip_status(sala::launch_linear_prefill(a, static_cast<hipStream_t>(stream)), "sala_linear_prefill launch");
}

int sala_linear_prefill_backward(int dtype, int B, int H, int N, int d, int chunk, const void *q, const void *k,
                                 const void *v, const void *dout, const float *decay, const float *state_in,
                                 const float *dstate_out, void *dq, void *dk, void *dv, float *dstate_in, void *ws,
                                 size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  REQUIRE(B >= 1 && H >= 1 && N >= 1, SALA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if ((s = check_d(d))) return s;
  REQUIRE(chunk == 64 || chunk == 128, SALA_ERR_UNSUPPORTED, "chunk = %d: libsala supports 64 and 128", chunk);
  REQUIRE(dtype != SALA_BF16 || (long long)N * d * 2 < (1ll << 31), SALA_ERR_UNSUPPORTED,
          "one head's rows must stay under 2 GiB");
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(dout, "dout");
  REQUIRE_PTR(dq, "dq");
  REQUIRE_PTR(dk, "dk");
  REQUIRE_PTR(dv, "dv");
  OPT_PTR(decay, "decay");
  OPT_PTR(state_in, "state_in");
  OPT_PTR(dstate_out, "dstate_out");
  OPT_PTR(dstate_in, "dstate_in");
  const void *ins[] = {q, k, v, dout};
  const void *outs[] = {dq, dk, dv};
  for (const void *o : outs)
    for (const void *i : ins) REQUIRE(o != i, SALA_ERR_INVALID_ARG, "dq, dk, dv must not overlap q, k, v or dout");
  REQUIRE(dq != dk && dq != dv && dk != dv, SALA_ERR_INVALID_ARG, "dq, dk and dv must be distinct buffers");
  REQUIRE(!dstate_in || (dstate_in != state_in && dstate_in != dstate_out), SALA_ERR_INVALID_ARG,
          "dstate_in must not overlap state_in or dstate_out");
  if ((s = check_ws(ws, ws_bytes, sala::linear_prefill_workspace(dtype, B, H, N, d, chunk)))) return s;
  sala::LinearBackwardArgs a{dtype, B, H, N, d, chunk, q, k, v, dout, decay, state_in, dstate_out, dq, dk, dv,
                             dstate_in, ws};
  return hip_status(sala::launch_linear_prefill_backward(a, static_cast<hipStream_t>(stream)),
                    "sala_linear_prefill_backward launch");
}

int sala_linear_decode(int dtype, int B, int H, int d, const void *q, const void *k, const void *v, void *o,
                       const float *decay, float *state, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  REQUIRE(B >= 1 && H >= 1, SALA_ERR_INVALID_ARG, "B, H must be >= 1");
  if ((s = check_d(d))) return s;
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(o, "o");
  REQUIRE_PTR(state, "state");
  OPT_PTR(decay, "decay");
  sala::LinearDecodeArgs a{dtype, B, H, d, q, k, v, o, decay, state};
  return hip_status(sala::launch_linear_decode(a, static_cast<hipStream_t>(stream)), "sala_linear_decode launch");
}

namespace {
int check_neighbours(const float *gamma_q, const float *gamma_k, float eps, float rope_base, const void *gate) {
  OPT_PTR(gamma_q, "gamma_q");
  OPT_PTR(gamma_k, "gamma_k");
  OPT_PTR(gate, "gate");
  REQUIRE(eps >= 0.f && eps < 1e30f, SALA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  REQUIRE(rope_base == 0.f || (rope_base > 1.f && rope_base < 1e30f), SALA_ERR_INVALID_ARG,
          "rope_base must be 0 (no RoPE) or a finite base > 1");
  return SALA_OK;
}
}  // namespace

int sala_linear_prefill_fused(int dtype, int B, int H, int N, int d, int chunk, const void *q, const void *k,
                              const void *v, void *o, const float *decay, const float *state_in, float *state_out,
                              const float *gamma_q, const float *gamma_k, float eps, float rope_base, long long pos0,
                              const void *gate, void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  REQUIRE(dtype == SALA_BF16, SALA_ERR_UNSUPPORTED, "the fused linear prefill is bf16 only");
  REQUIRE(B >= 1 && H >= 1 && N >= 1, SALA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if ((s = check_d(d))) return s;
  REQUIRE(chunk == 64 || chunk == 128, SALA_ERR_UNSUPPORTED, "chunk = %d: libsala supports 64 and 128", chunk);
  REQUIRE((long long)N * d * 2 < (1ll << 31), SALA_ERR_UNSUPPORTED, "one head's rows must stay under 2 GiB");
  REQUIRE(pos0 >= 0 && pos0 < (1ll << 40), SALA_ERR_INVALID_ARG, "pos0 must be in [0, 2^40)");
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(o, "o");
  OPT_PTR(decay, "decay");
  OPT_PTR(state_in, "state_in");
  OPT_PTR(state_out, "state_out");
  if ((s = check_neighbours(gamma_q, gamma_k, eps, rope_base, gate))) return s;
  if ((s = check_ws(ws, ws_bytes, sala::linear_prefill_workspace(dtype, B, H, N, d, chunk)))) return s;
  sala::LinearNeighbours nb{gamma_q, gamma_k, eps, rope_base, pos0, nullptr, gate};
  sala::LinearPrefillArgs a{dtype, B, H, N, d, chunk, q, k, v, o, decay, state_in, state_out, ws, &nb};
  return hip_status(sala::launch_linear_prefill(a, static_cast<hipStream_t>(stream)),
                    "sala_linear_prefill_fused launch");
}

int sala_linear_decode_fused(int dtype, int B, int H, int d, const void *q, const void *k, const void *v, void *o,
                             const float *decay, float *state, const float *gamma_q, const float *gamma_k, float eps,
                             float rope_base, const long long *pos, const void *gate, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  REQUIRE(B >= 1 && H >= 1, SALA_ERR_INVALID_ARG, "B, H must be >= 1");
  if ((s = check_d(d))) return s;
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(o, "o");
  REQUIRE_PTR(state, "state");
  OPT_PTR(decay, "decay");
  if ((s = check_neighbours(gamma_q, gamma_k, eps, rope_base, gate))) return s;
  REQUIRE(rope_base == 0.f || pos, SALA_ERR_INVALID_ARG, "pos must not be NULL when rope_base > 0");
  OPT_PTR(pos, "pos");
  sala::LinearNeighbours nb{gamma_q, gamma_k, eps, rope_base, 0, pos, gate};
  sala::LinearDecodeArgs a{dtype, B, H, d, q, k, v, o, decay, state, &nb};
  return hip_status(sala::launch_linear_decode(a, static_cast<hipStream_t>(stream)), "sala_linear_decode_fused launch");
}

int sala_qk_norm_rope(int dtype, int B, int H, int N, int d, const void *x, void *out, const float *gamma, float eps,
                      float rope_base, long long pos0, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  REQUIRE(B >= 1 && H >= 1 && N >= 1, SALA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if ((s = check_d(d))) return s;
  REQUIRE(pos0 >= 0 && pos0 < (1ll << 40), SALA_ERR_INVALID_ARG, "pos0 must be in [0, 2^40)");
  REQUIRE_PTR(x, "x");
  REQUIRE_PTR(out, "out");
  if ((s = check_neighbours(gamma, nullptr, eps, rope_base, nullptr))) return s;
  sala::QkNormRopeArgs a{dtype, B, H, N, d, x, out, gamma, eps, rope_base, pos0};
  return hip_status(sala::launch_qk_norm_rope(a, static_cast<hipStream_t>(stream)), "sala_qk_norm_rope launch");
}

int sala_output_gate(int dtype, size_t n, const void *o, const void *gate, void *out, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  REQUIRE(n >= 1 && n % 8 == 0, SALA_ERR_INVALID_ARG, "n = %zu must be a positive multiple of 8", n);
  REQUIRE(n / 8 < (1ull << 38), SALA_ERR_INVALID_ARG, "n too large");
  REQUIRE_PTR(o, "o");
  REQUIRE_PTR(gate, "gate");
  REQUIRE_PTR(out, "out");
  return hip_status(sala::launch_output_gate(dtype, n, o, gate, out, static_cast<hipStream_t>(stream)),
                    "sala_output_gate launch");
}

size_t sala_sparse_select_workspace(int dtype, int B, int Hq, int Hkv, int d, int Nq, int L, int block, int topk,
                                    int n_init, int n_local) {
  if (B < 1 || Hkv < 1 || L < 1 || block < 1 || (Nq != 1 && Nq != L)) return 0;
  return sala::sparse_select_workspace(dtype, B, Hq, Hkv, d, Nq, L, block, topk, n_init, n_local, false);
}

int sala_sparse_select(int dtype, int B, int Hq, int Hkv, int d, int Nq, int L, int block, int topk, int n_init,
                       int n_local, const void *q, const void *k, float *k_pooled, int32_t *idx, float *scores,
                       void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_sparse_common(B, Hq, Hkv, block, topk, "topk"))) return s;
  if ((s = check_d(d))) return s;
  REQUIRE(L >= 1, SALA_ERR_INVALID_ARG, "L must be >= 1");
  REQUIRE(Nq == L || Nq == 1, SALA_ERR_UNSUPPORTED, "Nq = %d: supported are Nq == L (prefill) and Nq == 1 (decode)", Nq);
  REQUIRE(n_init >= 0 && n_local >= 0, SALA_ERR_INVALID_ARG, "n_init and n_local must be >= 0");
  REQUIRE(topk + n_init + n_local >= 1, SALA_ERR_INVALID_ARG, "topk + n_init + n_local must be >= 1");
  REQUIRE(topk + n_init + n_local <= 1024, SALA_ERR_UNSUPPORTED, "topk + n_init + n_local must be <= 1024");
  REQUIRE_PTR(q, "q");
  OPT_PTR(k, "k");
  REQUIRE_PTR(k_pooled, "k_pooled");
  REQUIRE_PTR(idx, "idx");
  OPT_PTR(scores, "scores");
  const size_t need = sala::sparse_select_workspace(dtype, B, Hq, Hkv, d, Nq, L, block, topk, n_init, n_local,
                                                    scores != nullptr);
  if ((s = check_ws(ws, ws_bytes, need))) return s;
  sala::SparseSelectArgs a{dtype, B, Hq, Hkv, d, Nq, L, block, topk, n_init, n_local, q, k, k_pooled, idx, scores, ws};
  return hip_status(sala::launch_sparse_select(a, static_cast<hipStream_t>(stream)), "sala_sparse_select launch");
}

size_t sala_sparse_prefill_workspace(int dtype, int B, int Hq, int Hkv, int N, int d, int block, int n_sel) {
  if (B < 1 || Hkv < 1 || N < 1 || block != 64 || (d != 64 && d != 128)) return 0;
  return sala::sparse_prefill_workspace(dtype, B, Hq, Hkv, N, d, block, n_sel);
}

int sala_sparse_prefill(int dtype, int B, int Hq, int Hkv, int N, int d, int block, int n_sel, float scale,
                        const void *q, const void *k, const void *v, const int32_t *idx, void *o, void *ws,
                        size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_sparse_common(B, Hq, Hkv, block, n_sel, "n_sel"))) return s;
  if ((s = check_d(d))) return s;
  REQUIRE(N >= 1, SALA_ERR_INVALID_ARG, "N must be >= 1");
  REQUIRE(n_sel >= 1 && n_sel <= 1024, SALA_ERR_UNSUPPORTED, "n_sel = %d must be in [1, 1024]", n_sel);
  REQUIRE(scale == scale, SALA_ERR_INVALID_ARG, "scale is NaN");
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(idx, "idx");
  REQUIRE_PTR(o, "o");
  if ((s = check_ws(ws, ws_bytes, sala::sparse_prefill_workspace(dtype, B, Hq, Hkv, N, d, block, n_sel)))) return s;
  const int nqb = (N + 63) / 64;
  if ((s = debug_idx(idx, (long long)B * Hkv * nqb, n_sel, nqb, nqb, 1, stream, "sala_sparse_prefill"))) return s;
  sala::SparsePrefillArgs a{dtype, B, Hq, Hkv, N, d, block, n_sel, scale, q, k, v, idx, o, ws};
  return hip_status(sala::launch_sparse_prefill(a, static_cast<hipStream_t>(stream)), "sala_sparse_prefill launch");
}

size_t sala_sparse_prefill_backward_workspace(int dtype, int B, int Hq, int Hkv, int N, int d, int block, int n_sel) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || block != 64 || (d != 64 && d != 128) || n_sel < 1 || n_sel > 1024)
    return 0;
  return sala::sparse_backward_workspace(dtype, B, Hq, Hkv, N, d, block, n_sel);
}

int sala_sparse_prefill_backward(int dtype, int B, int Hq, int Hkv, int N, int d, int block, int n_sel, float scale,
                                 const void *q, const void *k, const void *v, const int32_t *idx, const void *dout,
                                 void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  REQUIRE(dtype == SALA_BF16, SALA_ERR_UNSUPPORTED, "sala_sparse_prefill_backward supports SALA_BF16 only");
  if ((s = check_sparse_common(B, Hq, Hkv, block, n_sel, "n_sel"))) return s;
  if ((s = check_d(d))) return s;
  REQUIRE(N >= 1, SALA_ERR_INVALID_ARG, "N must be >= 1");
  REQUIRE(n_sel >= 1 && n_sel <= 1024, SALA_ERR_UNSUPPORTED, "n_sel = %d must be in [1, 1024]", n_sel);
  REQUIRE((long long)N * d * 2 < (1ll << 31), SALA_ERR_UNSUPPORTED, "one head's rows must stay under 2 GiB");
  REQUIRE(scale == scale, SALA_ERR_INVALID_ARG, "scale is NaN");
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(idx, "idx");
  REQUIRE_PTR(dout, "dout");
  REQUIRE_PTR(dq, "dq");
  REQUIRE_PTR(dk, "dk");
  REQUIRE_PTR(dv, "dv");
  const void *ins[] = {q, k, v, idx, dout};
  const void *outs[] = {dq, dk, dv};
  for (const void *x : outs)
    for (const void *y : ins) REQUIRE(x != y, SALA_ERR_INVALID_ARG, "dq, dk, dv must not overlap an input");
  REQUIRE(dq != dk && dq != dv && dk != dv, SALA_ERR_INVALID_ARG, "dq, dk and dv must be distinct buffers");
  if ((s = check_ws(ws, ws_bytes, sala::sparse_backward_workspace(dtype, B, Hq, Hkv, N, d, block, n_sel)))) return s;
  const int nqb = (N + 63) / 64;
  if ((s = debug_idx(idx, (long long)B * Hkv * nqb, n_sel, nqb, nqb, 1, stream, "sala_sparse_prefill_backward")))
    return s;
  sala::SparseBackwardArgs a{dtype, B, Hq, Hkv, N, d, block, n_sel, scale, q, k, v, idx, dout, dq, dk, dv, ws};
  return hip_status(sala::launch_sparse_backward(a, static_cast<hipStream_t>(stream)),
                    "sala_sparse_prefill_backward launch");
}

int sala_dense_prefill(int dtype, int B, int Hq, int Hkv, int N, int d, float scale, const void *q, const void *k,
                       const void *v, void *o, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  REQUIRE(dtype == SALA_BF16, SALA_ERR_UNSUPPORTED, "sala_dense_prefill supports SALA_BF16 only");
  if ((s = check_sparse_common(B, Hq, Hkv, 64, 1, "n_sel"))) return s;
  if ((s = check_d(d))) return s;
  REQUIRE(N >= 1, SALA_ERR_INVALID_ARG, "N must be >= 1");
  REQUIRE(scale == scale, SALA_ERR_INVALID_ARG, "scale is NaN");
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(o, "o");
  sala::SparsePrefillArgs a{dtype, B, Hq, Hkv, N, d, 64, 1, scale, q, k, v, nullptr, o, nullptr};
  return hip_status(sala::launch_dense_prefill(a, static_cast<hipStream_t>(stream)), "sala_dense_prefill launch");
}

int sala_ceiling_mfma(int workgroups, int iters, float *out, void *stream) {
  REQUIRE(workgroups >= 1 && iters >= 1, SALA_ERR_INVALID_ARG, "workgroups and iters must be >= 1");
  REQUIRE_PTR(out, "out");
  return hip_status(sala::launch_ceiling_mfma(workgroups, iters, out, static_cast<hipStream_t>(stream)),
                    "sala_ceiling_mfma launch");
}

int sala_ceiling_copy(const void *src, void *dst, size_t bytes, void *stream) {
  REQUIRE_PTR(src, "src");
  REQUIRE_PTR(dst, "dst");
  REQUIRE(bytes % 16 == 0, SALA_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  return hip_status(sala::launch_ceiling_copy(src, dst, bytes, static_cast<hipStream_t>(stream)),
                    "sala_ceiling_copy launch");
}

int sala_ceiling_read(const void *src, size_t bytes, float *out, void *stream) {
  REQUIRE(bytes % 16 == 0, SALA_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  REQUIRE(bytes == 0 || src != nullptr, SALA_ERR_INVALID_ARG, "src is NULL");
  REQUIRE(bytes / 16384 < (size_t)INT32_MAX, SALA_ERR_INVALID_ARG, "bytes too large");
  REQUIRE_PTR(out, "out");
  return hip_status(sala::launch_ceiling_read(src, bytes, out, static_cast<hipStream_t>(stream)),
                    "sala_ceiling_read launch");
}

size_t sala_sparse_decode_workspace(int dtype, int B, int Hq, int Hkv, int L, int d, int block, int n_sel) {
  if (B < 1 || Hkv < 1 || n_sel < 1 || (d != 64 && d != 128)) return 0;
  return sala::sparse_decode_workspace(dtype, B, Hq, Hkv, L, d, block, n_sel);
}

int sala_sparse_decode(int dtype, int B, int Hq, int Hkv, int L, int d, int block, int n_sel, float scale,
                       const void *q, const void *k_cache, const void *v_cache, const int32_t *idx, void *o, void *ws,
                       size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_sparse_common(B, Hq, Hkv, block, n_sel, "n_sel"))) return s;
  if ((s = check_d(d))) return s;
  REQUIRE(L >= 1, SALA_ERR_INVALID_ARG, "L must be >= 1");
  REQUIRE(n_sel >= 1 && n_sel <= 1024, SALA_ERR_UNSUPPORTED, "n_sel = %d must be in [1, 1024]", n_sel);
  REQUIRE(Hq / Hkv <= 32, SALA_ERR_UNSUPPORTED, "decode supports at most 32 query heads per KV head");
  REQUIRE(scale == scale, SALA_ERR_INVALID_ARG, "scale is NaN");
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k_cache, "k_cache");
  REQUIRE_PTR(v_cache, "v_cache");
  REQUIRE_PTR(idx, "idx");
  REQUIRE_PTR(o, "o");
  if ((s = check_ws(ws, ws_bytes, sala::sparse_decode_workspace(dtype, B, Hq, Hkv, L, d, block, n_sel)))) return s;
  if ((s = debug_idx(idx, (long long)B * Hkv, n_sel, 1, (L + 63) / 64, 0, stream, "sala_sparse_decode"))) return s;
  sala::SparseDecodeArgs a{dtype, B, Hq, Hkv, L, d, block, n_sel, scale, q, k_cache, v_cache, idx, o, ws};
  return hip_status(sala::launch_sparse_decode(a, static_cast<hipStream_t>(stream)), "sala_sparse_decode launch");
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t step_select_ws(int dtype, int B, int Hq, int Hkv, int d, int L, int block, int topk, int n_init, int n_local) {
  return align256(sala::sparse_select_workspace(dtype, B, Hq, Hkv, d, 1, L, block, topk, n_init, n_local, false));
}
}  // namespace

size_t sala_sparse_decode_step_workspace(int dtype, int B, int Hq, int Hkv, int capacity, int d, int block, int topk,
                                         int n_init, int n_local) {
  if (B < 1 || Hkv < 1 || Hq < 1 || capacity < 1 || block != 64 || (d != 64 && d != 128) || topk < 0 ||
      n_init < 0 || n_local < 0 || topk + n_init + n_local < 1)
    return 0;
  const int n_sel = topk + n_init + n_local;
  return step_select_ws(dtype, B, Hq, Hkv, d, capacity, block, topk, n_init, n_local) +
         sala::sparse_decode_workspace(dtype, B, Hq, Hkv, capacity, d, block, n_sel);
}

namespace {
// The decode step behind both entry points: with use_scratch, the workspace is
// this device's fixed scratch array (ws / ws_bytes ignored), looked up only
// after every argument has been validated.
int decode_step(int dtype, int B, int Hq, int Hkv, int capacity, int d, int pos, int block, int topk, int n_init,
                int n_local, float scale, const void *q, const void *k_new, const void *v_new, void *k_cache,
                void *v_cache, float *k_pooled, int32_t *idx, void *o, void *ws, size_t ws_bytes, bool use_scratch,
                void *stream) {
  int s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_sparse_common(B, Hq, Hkv, block, topk, "topk"))) return s;
  if ((s = check_d(d))) return s;
  REQUIRE(capacity >= 1, SALA_ERR_INVALID_ARG, "capacity must be >= 1");
  REQUIRE(pos >= 0 && pos < capacity, SALA_ERR_INVALID_ARG, "pos = %d must be in [0, capacity = %d)", pos, capacity);
  REQUIRE(n_init >= 0 && n_local >= 0, SALA_ERR_INVALID_ARG, "n_init and n_local must be >= 0");
  const int n_sel = topk + n_init + n_local;
  REQUIRE(n_sel >= 1, SALA_ERR_INVALID_ARG, "topk + n_init + n_local must be >= 1");
  REQUIRE(n_sel <= 1024, SALA_ERR_UNSUPPORTED, "topk + n_init + n_local must be <= 1024");
  REQUIRE(Hq / Hkv <= 32, SALA_ERR_UNSUPPORTED, "decode supports at most 32 query heads per KV head");
  REQUIRE(scale == scale, SALA_ERR_INVALID_ARG, "scale is NaN");
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k_new, "k_new");
  REQUIRE_PTR(v_new, "v_new");
  REQUIRE_PTR(k_cache, "k_cache");
  REQUIRE_PTR(v_cache, "v_cache");
  REQUIRE_PTR(k_pooled, "k_pooled");
  REQUIRE_PTR(idx, "idx");
  REQUIRE_PTR(o, "o");
  const int L = pos + 1;
  const size_t sel = step_select_ws(dtype, B, Hq, Hkv, d, L, block, topk, n_init, n_local);
  const size_t need = sel + sala::sparse_decode_workspace(dtype, B, Hq, Hkv, L, d, block, n_sel);
  if (use_scratch) {
    REQUIRE(need <= SALA_NOALLOC_SCRATCH_BYTES, SALA_ERR_WORKSPACE,
            "this step needs %zu bytes of workspace, more than the %u-byte scratch array of the allocation-free call",
            need, (unsigned)SALA_NOALLOC_SCRATCH_BYTES);
    if ((s = hip_status(sala::noalloc_scratch(&ws), "sala_sparse_decode_step_noalloc: scratch address"))) return s;
    ws_bytes = SALA_NOALLOC_SCRATCH_BYTES;
  }
  if ((s = check_ws(ws, ws_bytes, need))) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = sala::launch_kv_append(dtype, B * Hkv, capacity, d, block, pos, k_new, v_new, k_cache, v_cache,
                                        k_pooled, st);
  if (e != hipSuccess) return hip_status(e, "sala_sparse_decode_step append");
  sala::SparseSelectArgs sa{dtype, B, Hq, Hkv, d, 1, L, block, topk, n_init, n_local, q, nullptr, k_pooled, idx,
                            nullptr, ws, capacity};
  e = sala::launch_sparse_select(sa, st);
  if (e != hipSuccess) return hip_status(e, "sala_sparse_decode_step select");
  sala::SparseDecodeArgs da{dtype, B, Hq, Hkv, L, d, block, n_sel, scale, q, k_cache, v_cache, idx, o,
                            static_cast<char *>(ws) + sel, capacity};
  return hip_status(sala::launch_sparse_decode(da, st), "sala_sparse_decode_step attend");
}
}  // namespace

int sala_sparse_decode_step(int dtype, int B, int Hq, int Hkv, int capacity, int d, int pos, int block, int topk,
                            int n_init, int n_local, float scale, const void *q, const void *k_new, const void *v_new,
                            void *k_cache, void *v_cache, float *k_pooled, int32_t *idx, void *o, void *ws,
                            size_t ws_bytes, void *stream) {
  return decode_step(dtype, B, Hq, Hkv, capacity, d, pos, block, topk, n_init, n_local, scale, q, k_new, v_new,
                     k_cache, v_cache, k_pooled, idx, o, ws, ws_bytes, false, stream);
}

int sala_sparse_decode_step_noalloc(int dtype, int B, int Hq, int Hkv, int capacity, int d, int pos, int block,
                                    int topk, int n_init, int n_local, float scale, const void *q, const void *k_new,
                                    const void *v_new, void *k_cache, void *v_cache, float *k_pooled, int32_t *idx,
                                    void *o, void *stream) {
  return decode_step(dtype, B, Hq, Hkv, capacity, d, pos, block, topk, n_init, n_local, scale, q, k_new, v_new,
                     k_cache, v_cache, k_pooled, idx, o, nullptr, 0, true, stream);
}

size_t sala_sparse_prefill_chunk_workspace(int dtype, int B, int Hq, int Hkv, int capacity, int d, int n, int block,
                                           int topk, int n_init, int n_local) {
  if (n == 1) return sala_sparse_decode_step_workspace(dtype, B, Hq, Hkv, capacity, d, block, topk, n_init, n_local);
  if (B < 1 || Hkv < 1 || Hq < 1 || capacity < 1 || n < 1 || n > capacity || block != 64 || (d != 64 && d != 128))
    return 0;
  return sala::sparse_select_workspace(dtype, B, Hq, Hkv, d, n, capacity, block, topk, n_init, n_local, false);
}

int sala_sparse_prefill_chunk(int dtype, int B, int Hq, int Hkv, int capacity, int d, int pos0, int n, int block,
                              int topk, int n_init, int n_local, float scale, const void *q, const void *k_new,
                              const void *v_new, void *k_cache, void *v_cache, float *k_pooled, int32_t *idx, void *o,
                              void *ws, size_t ws_bytes, void *stream) {
  int s;
  REQUIRE(n >= 1, SALA_ERR_INVALID_ARG, "n must be >= 1");
  if (n == 1)
    return sala_sparse_decode_step(dtype, B, Hq, Hkv, capacity, d, pos0, block, topk, n_init, n_local, scale, q,
                                   k_new, v_new, k_cache, v_cache, k_pooled, idx, o, ws, ws_bytes, stream);
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_sparse_common(B, Hq, Hkv, block, topk, "topk"))) return s;
  if ((s = check_d(d))) return s;
  REQUIRE(capacity >= 1, SALA_ERR_INVALID_ARG, "capacity must be >= 1");
  REQUIRE(pos0 >= 0 && (long long)pos0 + n <= capacity, SALA_ERR_INVALID_ARG,
          "tokens pos0 .. pos0 + n - 1 (%d .. %lld) must lie in [0, capacity = %d)", pos0, (long long)pos0 + n - 1,
          capacity);
  REQUIRE(pos0 % block == 0, SALA_ERR_UNSUPPORTED, "a chunk of n > 1 tokens must start on a block boundary (pos0 = %d)",
          pos0);
  REQUIRE(n_init >= 0 && n_local >= 0, SALA_ERR_INVALID_ARG, "n_init and n_local must be >= 0");
  const int n_sel = topk + n_init + n_local;
  REQUIRE(n_sel >= 1, SALA_ERR_INVALID_ARG, "topk + n_init + n_local must be >= 1");
  REQUIRE(n_sel <= 1024, SALA_ERR_UNSUPPORTED, "topk + n_init + n_local must be <= 1024");
  REQUIRE(scale == scale, SALA_ERR_INVALID_ARG, "scale is NaN");
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k_new, "k_new");
  REQUIRE_PTR(v_new, "v_new");
  REQUIRE_PTR(k_cache, "k_cache");
  REQUIRE_PTR(v_cache, "v_cache");
  REQUIRE_PTR(k_pooled, "k_pooled");
  REQUIRE_PTR(idx, "idx");
  REQUIRE_PTR(o, "o");
  const int L = pos0 + n;
  const size_t need = sala::sparse_select_workspace(dtype, B, Hq, Hkv, d, n, L, block, topk, n_init, n_local, false);
  if ((s = check_ws(ws, ws_bytes, need))) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = sala::launch_kv_write(dtype, B * Hkv, capacity, d, pos0, n, k_new, v_new, k_cache, v_cache, st);
  if (e != hipSuccess) return hip_status(e, "sala_sparse_prefill_chunk write");
  sala::SparseSelectArgs sa{dtype, B, Hq, Hkv, d, n, L, block, topk, n_init, n_local, q, k_cache, k_pooled, idx,
                            nullptr, ws, capacity};
  e = sala::launch_sparse_select(sa, st);
  if (e != hipSuccess) return hip_status(e, "sala_sparse_prefill_chunk select");
  sala::SparsePrefillArgs pa{dtype, B, Hq, Hkv, n, d, block, n_sel, scale, q, k_cache, v_cache, idx, o, nullptr,
                             L, capacity};
  return hip_status(sala::launch_sparse_prefill(pa, st), "sala_sparse_prefill_chunk attend");
}

size_t sala_workspace_bytes(int op, const int64_t *dims, int ndims) {
  static const int nargs[] = {6, 11, 8, 8, 11, 10, 8};
  const size_t bad = (size_t)-1;
  if (op < SALA_OP_LINEAR_PREFILL || op > SALA_OP_SPARSE_PREFILL_BACKWARD) {
    fail(SALA_ERR_INVALID_ARG, "unknown operation %d", op);
    return bad;
  }
  if (!dims || ndims != nargs[op]) {
    fail(SALA_ERR_INVALID_ARG, "operation %d takes %d dimensions, got %d%s", op, nargs[op], ndims,
         dims ? "" : " (dims is NULL)");
    return bad;
  }
  int a[11];
  for (int i = 0; i < ndims; ++i) {
    if (dims[i] < -2147483648ll || dims[i] > 2147483647ll) {
      fail(SALA_ERR_INVALID_ARG, "dimension %d (%lld) does not fit an int", i, (long long)dims[i]);
      return bad;
    }
    a[i] = (int)dims[i];
  }
  g_err[0] = '\0';
  switch (op) {
    case SALA_OP_LINEAR_PREFILL: return sala_linear_prefill_workspace(a[0], a[1], a[2], a[3], a[4], a[5]);
    case SALA_OP_SPARSE_SELECT:
      return sala_sparse_select_workspace(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8], a[9], a[10]);
    case SALA_OP_SPARSE_PREFILL: return sala_sparse_prefill_workspace(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7]);
    case SALA_OP_SPARSE_DECODE: return sala_sparse_decode_workspace(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7]);
    case SALA_OP_SPARSE_PREFILL_CHUNK:
      return sala_sparse_prefill_chunk_workspace(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8], a[9], a[10]);
    case SALA_OP_SPARSE_DECODE_STEP:
      return sala_sparse_decode_step_workspace(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8], a[9]);
    default:
      return sala_sparse_prefill_backward_workspace(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7]);
  }
}

}  // extern "C"
