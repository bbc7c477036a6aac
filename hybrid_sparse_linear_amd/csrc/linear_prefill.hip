// Lightning (causal, decayed linear) attention prefill for gfx950.
//
// Operation (per batch row b, head h, lam = decay[h]):
//   o_t   = sum_{s<=t} lam^(t-s) (q_t . k_s) v_s + lam^(t+1) q_t S_in
//   S_out = lam^N S_in + sum_s lam^(N-1-s) k_s v_s^T           (S is [d_k][d_v])
// The pages give the linear layers an O(N) cost through a recursive
// formulation (MiniCPM-SALA, gist.science (de) section 2,
// "Architektur-Hybridisierung") and a structure close to softmax attention
// (gist.science (ja) 技術概要 section 2.1); no normaliser or feature map is
// applied.
//
// bf16 path: the sequence of each (b, h) is cut into segments of whole chunks
// so that B*H*segments workgroups fill the 256 CUs.
//   pass 1  lin_seg_aggregate: each segment except the last computes its own
//           decayed state contribution A_m = sum_{s in m} lam^(end-1-s) k_s v_s^T
//           (fp32, written to the workspace).
//   pass 2  lin_seg_scan: an element-wise scan over segments turns the A_m into
//           the state entering every segment, S_in(m) = lam^len S_in(m-1) + A_{m-1}.
//   pass 3  lin_seg_output: each segment walks its chunks.  Per chunk of C tokens:
//             O^T  = lam^(i+1) (S^T Q^T)  +  V^T (decay-masked K Q^T)
//             S    = lam^C S + (diag(lam^(C-1-j)) K)^T V
//           with bf16 MFMA 16x16x32 and fp32 accumulation; the fp32 master S
//           stays in registers, a bf16 copy of S^T in LDS feeds the Q S product.
//           The last segment writes S_out.
// fp32 path: lin_recurrent_f32 runs the recurrence S_t = lam S_{t-1} + k_t v_t^T,
// o_t = q_t S_t token by token with one thread per d_v column (small shapes).

#include "sala_common.hpp"
#include "sala_launch.hpp"

namespace sala {
namespace {

template <int C, int D>
struct LinCfg {
  static constexpr int NT = 512;                // 8 waves, two per SIMD
  static constexpr int NQT = C / 16;            // 16-query tiles per chunk (one per wave at C = 128)
  static constexpr int ND = D / 16;             // 16-wide feature tiles
  static constexpr int NDS = D / 32;            // 32-deep steps over features
  static constexpr int NKS = C / 32;            // 32-deep steps over chunk tokens
  static constexpr int NDV = ND * ND / 8;       // state tiles per wave (one d_k tile row or half of one)
  static constexpr int KCH = D / 8;             // 16-byte chunks per row of K_lds / St_lds
  static constexpr int TCH = C / 8;             // 16-byte chunks per row of Kt_lds / Vt_lds
  static constexpr int NB8 = (C / 8) * (D / 8); // 8x8 staging blocks per chunk (of K, and of V)
  static constexpr uint32_t K_OFF = 0;
  static constexpr uint32_t KT_OFF = K_OFF + C * D * 2;
  static constexpr uint32_t VT_OFF = KT_OFF + C * D * 2;
  static constexpr uint32_t ST_OFF = VT_OFF + C * D * 2;
  static constexpr uint32_t PW_OFF = ST_OFF + D * D * 2;
  static constexpr uint32_t LDS = PW_OFF + (C + 4) * 4;
  static_assert(2 * NB8 <= NT, "one 8x8 staging block per thread at most");
  // wave -> state tiles: d_k tile dkt(w), d_v tiles dv0(w) .. dv0(w)+NDV-1
  __device__ static int dkt(int w) { return ND == 8 ? w : (w >> 1); }
  __device__ static int dv0(int w) { return ND == 8 ? 0 : 2 * (w & 1); }
  // wave -> query tile (-1: none).  Waves w and w+4 share a SIMD; pairing
  // tiles w and 7-w balances the causal work per SIMD.
  __device__ static int qtile(int w) {
    if (NQT == 8) return w < 4 ? w : 11 - w;
    return w < NQT ? w : -1;
  }
};

// XOR swizzles of 16-byte chunks inside an LDS row (bank-conflict avoidance).
// swz_t: rows read 16 consecutive rows at one chunk, and written by 16 rows 8 apart.
template <int NCH>
__device__ __forceinline__ uint32_t swz_t(uint32_t row, uint32_t ch) {
  return ch ^ ((row ^ (row >> 3)) & (NCH - 1));
}
// swz_k: K rows are read in the key order of the 32-key pair permutation below.
template <int NCH>
__device__ __forceinline__ uint32_t swz_k(uint32_t row, uint32_t ch) {
  if constexpr (NCH == 16) return ch ^ ((row & 3) | ((row >> 1) & 12));
  else return ch ^ (((row >> 1) & 1) | ((row >> 2) & 6));
}
template <int NCH>
__device__ __forceinline__ uint32_t off_t(uint32_t row, uint32_t ch) { return (row * NCH + swz_t<NCH>(row, ch)) * 16u; }
template <int NCH>
__device__ __forceinline__ uint32_t off_k(uint32_t row, uint32_t ch) { return (row * NCH + swz_k<NCH>(row, ch)) * 16u; }

// Key permutation inside a 32-key pair of 16-key tiles: MFMA row r of tile t
// (t = 0, 1) holds key 8*(r/4) + 4*t + r%4, so that after K Q^T each lane's
// 4+4 accumulator rows of the two tiles are 8 consecutive keys -- exactly the
// k slots of the B operand of the following V^T P^T product.  Both tiles of a
// pair therefore hold keys from the whole 32-key range.
__device__ __forceinline__ int pair_key(int t, int r) { return ((r >> 2) << 3) + (t << 2) + (r & 3); }

// Transpose an 8x8 bf16 block: x[e] = row e (8 features, 4 dwords);
// y[f] = feature f across the 8 rows.
__device__ __forceinline__ void transpose8x8(const u32x4 (&x)[8], u32x4 (&y)[8]) {
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int p = f >> 1;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      uint32_t a = x[2 * qq][p], b = x[2 * qq + 1][p];
      y[f][qq] = (f & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

// Staging job of a thread: one 8x8 block of K (jobs 0 .. NB8-1) or of V
// (jobs NB8 .. 2*NB8-1) of the chunk starting at token c0; rows at or past
// t_end read as zero.
template <int C, int D>
__device__ __forceinline__ void load_block8(const uint16_t *kb, const uint16_t *vb, int tid, int c0, int t_end,
                                            u32x4 (&x)[8]) {
  using Cf = LinCfg<C, D>;
  if (tid >= 2 * Cf::NB8) return;
  const bool is_v = tid >= Cf::NB8;
  const int job = is_v ? tid - Cf::NB8 : tid;
  const int tg = job / (D / 8), fg = job % (D / 8);
  const uint16_t *src = is_v ? vb : kb;
  // unconditional loads of clamped rows, then zero the rows past t_end
  // (selects instead of a branch per load)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = c0 + 8 * tg + e;
    x[e] = gload16(src + (size_t)min(t, t_end - 1) * D + 8 * fg);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (c0 + 8 * tg + e >= t_end) x[e] = u32x4{0, 0, 0, 0};
  }
}

// Write a staged block: K -> K_lds (row-major, when WITH_K) and Kt_lds
// (transposed, row j scaled by lam^(m-1-j) in fp32 and rounded once);
// V -> Vt_lds (transposed).
template <int C, int D, bool WITH_K>
__device__ __forceinline__ void stage_block8(char *lds, int tid, int m, const float *pw, u32x4 (&x)[8]) {
  using Cf = LinCfg<C, D>;
  if (tid >= 2 * Cf::NB8) return;
  const bool is_v = tid >= Cf::NB8;
  const int job = is_v ? tid - Cf::NB8 : tid;
  const int tg = job / (D / 8), fg = job % (D / 8);
  u32x4 y[8];
  if (!is_v) {
    if constexpr (WITH_K) {
#pragma unroll
      for (int e = 0; e < 8; ++e) lds_store(lds + Cf::K_OFF, off_k<Cf::KCH>(8 * tg + e, fg), x[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 8 * tg + e;
      const float sc = (j < m) ? pw[m - 1 - j] : 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) x[e][p] = pack_bf16x2(bf16lo(x[e][p]) * sc, bf16hi(x[e][p]) * sc);
    }
    transpose8x8(x, y);
#pragma unroll
    for (int f = 0; f < 8; ++f) lds_store(lds + Cf::KT_OFF, off_t<Cf::TCH>(8 * fg + f, tg), y[f]);
  } else {
    transpose8x8(x, y);
#pragma unroll
    for (int f = 0; f < 8; ++f) lds_store(lds + Cf::VT_OFF, off_t<Cf::TCH>(8 * fg + f, tg), y[f]);
  }
}

// State update S = lam^m S + (Kt scaled)^T V for this wave's state tiles.
template <int C, int D>
__device__ __forceinline__ void state_update(const char *lds, int w, int lr, int lg, float lam_m,
                                             f32x4 (&Sacc)[LinCfg<C, D>::NDV]) {
  using Cf = LinCfg<C, D>;
#pragma unroll
  for (int a = 0; a < Cf::NDV; ++a) Sacc[a] *= lam_m;
#pragma unroll
  for (int ks = 0; ks < Cf::NKS; ++ks) {
    const u32x4 A = lds_load<u32x4>(lds + Cf::KT_OFF, off_t<Cf::TCH>(16 * Cf::dkt(w) + lr, 4 * ks + lg));
#pragma unroll
    for (int a = 0; a < Cf::NDV; ++a) {
      const u32x4 Bv = lds_load<u32x4>(lds + Cf::VT_OFF, off_t<Cf::TCH>(16 * (Cf::dv0(w) + a) + lr, 4 * ks + lg));
      Sacc[a] = mfma16x16x32(A, Bv, Sacc[a]);
    }
  }
}

// ---------------------------------------------------------------- pass 1
template <int C, int D>
__global__ __launch_bounds__(512) void lin_seg_aggregate(const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v,
                                                         const float *__restrict__ decay,
                                                         float *__restrict__ seg_state, int H, int N,
                                                         int seg_len, int nseg) {
  using Cf = LinCfg<C, D>;
  __shared__ __attribute__((aligned(16))) char lds[Cf::LDS];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int nagg = nseg - 1;
  const int bh = blockIdx.x / nagg, seg = blockIdx.x % nagg;
  const int h = bh % H;
  const int t_begin = seg * seg_len, t_end = min(N, t_begin + seg_len);
  const float lam = decay ? decay[h] : 1.f;
  float *pw = reinterpret_cast<float *>(lds + Cf::PW_OFF);
  for (int n = tid; n <= C; n += Cf::NT) pw[n] = (float)pow((double)lam, (double)n);
  const uint16_t *kb = k + (size_t)bh * N * D;
  const uint16_t *vb = v + (size_t)bh * N * D;

  f32x4 Sacc[Cf::NDV];
#pragma unroll
  for (int a = 0; a < Cf::NDV; ++a) Sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 x[8];
  load_block8<C, D>(kb, vb, tid, t_begin, t_end, x);
  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    const int m = min(C, t_end - c0);
    __syncthreads();
    stage_block8<C, D, false>(lds, tid, m, pw, x);
    __syncthreads();
    if (c0 + C < t_end) load_block8<C, D>(kb, vb, tid, c0 + C, t_end, x);
    state_update<C, D>(lds, w, lr, lg, pw[m], Sacc);
  }
  float *out = seg_state + ((size_t)bh * nseg + seg) * D * D;
#pragma unroll
  for (int a = 0; a < Cf::NDV; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[(size_t)(16 * Cf::dkt(w) + 4 * lg + i) * D + 16 * (Cf::dv0(w) + a) + lr] = Sacc[a][i];
}

// ---------------------------------------------------------------- pass 2
// seg_state[bh][m] holds A_m for m < nseg-1 on entry, S_in(m) for every m on exit.
__global__ __launch_bounds__(256) void lin_seg_scan(float *__restrict__ seg_state,
                                                    const float *__restrict__ state_in,
                                                    const float *__restrict__ decay, int H, int DD,
                                                    int N, int seg_len, int nseg) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= DD) return;
  const int h = bh % H;
  const double lam = decay ? (double)decay[h] : 1.0;
  const float lam_seg = (float)pow(lam, (double)seg_len);
  float s = state_in ? state_in[(size_t)bh * DD + e] : 0.f;
  float *base = seg_state + (size_t)bh * nseg * DD + e;
  for (int m = 0; m < nseg; ++m) {
    const float a = (m + 1 < nseg) ? base[(size_t)m * DD] : 0.f;
    base[(size_t)m * DD] = s;
    s = fmaf(lam_seg, s, a);
  }
}

// ---------------------------------------------------------------- pass 3
template <int C, int D>
__global__ __launch_bounds__(512) void lin_seg_output(const uint16_t *__restrict__ q,
                                                      const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v,
                                                      uint16_t *__restrict__ o,
                                                      const float *__restrict__ decay,
                                                      const float *__restrict__ seg_state,
                                                      size_t seg_stride, float *__restrict__ state_out,
                                                      int H, int N, int seg_len, int nseg) {
  using Cf = LinCfg<C, D>;
  __shared__ __attribute__((aligned(16))) char lds[Cf::LDS];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const int h = bh % H;
  const int t_begin = seg * seg_len, t_end = min(N, t_begin + seg_len);
  const float lam = decay ? decay[h] : 1.f;
  float *pw = reinterpret_cast<float *>(lds + Cf::PW_OFF);
  for (int n = tid; n <= C; n += Cf::NT) pw[n] = (float)pow((double)lam, (double)n);
  const size_t head_off = (size_t)bh * N * D;
  const uint16_t *qb = q + head_off, *kb = k + head_off, *vb = v + head_off;
  uint16_t *ob = o + head_off;
  const int qt = Cf::qtile(w);
  const int dkt = Cf::dkt(w), dv0 = Cf::dv0(w);

  f32x4 Sacc[Cf::NDV];
  const float *sin = seg_state ? seg_state + (size_t)bh * seg_stride * nseg + (size_t)seg * seg_stride : nullptr;
#pragma unroll
  for (int a = 0; a < Cf::NDV; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      Sacc[a][i] = sin ? sin[(size_t)(16 * dkt + 4 * lg + i) * D + 16 * (dv0 + a) + lr] : 0.f;

  u32x4 x[8];
  u32x4 qf[Cf::NDS];
  auto load_q = [&](int c0, u32x4 (&dst)[Cf::NDS]) {
    // rows past t_end load a clamped row; their outputs are never stored
    const int t = min(c0 + 16 * max(qt, 0) + lr, t_end - 1);
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s) dst[s] = gload16(qb + (size_t)t * D + 32 * s + 8 * lg);
  };
  load_block8<C, D>(kb, vb, tid, t_begin, t_end, x);
  load_q(t_begin, qf);

  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    const int m = min(C, t_end - c0);
    __syncthreads();
    stage_block8<C, D, true>(lds, tid, m, pw, x);
    // bf16 copy of S^T (rows d_v, columns d_k) for the Q S product
#pragma unroll
    for (int a = 0; a < Cf::NDV; ++a) {
      const int row = 16 * (dv0 + a) + lr;
      const uint32_t off = off_t<Cf::KCH>(row, 2 * dkt + (lg >> 1)) + (lg & 1) * 8;
      lds_store(lds + Cf::ST_OFF, off, u32x2{pack_bf16x2(Sacc[a][0], Sacc[a][1]), pack_bf16x2(Sacc[a][2], Sacc[a][3])});
    }
    __syncthreads();
    u32x4 qn[Cf::NDS];
    if (c0 + C < t_end) {
      load_block8<C, D>(kb, vb, tid, c0 + C, t_end, x);
      load_q(c0 + C, qn);
    }

    if (qt >= 0) {
      const int qq = 16 * qt + lr;  // this lane's query inside the chunk
      // (1) O^T = lam^(qq+1) * S^T Q^T
      f32x4 Oacc[Cf::ND];
#pragma unroll 2
      for (int dv = 0; dv < Cf::ND; ++dv) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < Cf::NDS; ++s)
          acc = mfma16x16x32(lds_load<u32x4>(lds + Cf::ST_OFF, off_t<Cf::KCH>(16 * dv + lr, 4 * s + lg)), qf[s], acc);
        Oacc[dv] = acc * pw[qq + 1];
      }
      // (2)+(3) P^T = decay-masked K Q^T over the causal key pairs; O^T += V^T P^T
      for (int p = 0; p <= (qt >> 1); ++p) {
        f32x4 P0 = {0.f, 0.f, 0.f, 0.f}, P1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < Cf::NDS; ++s) {
          const u32x4 A0 = lds_load<u32x4>(lds + Cf::K_OFF, off_k<Cf::KCH>(32 * p + pair_key(0, lr), 4 * s + lg));
          const u32x4 A1 = lds_load<u32x4>(lds + Cf::K_OFF, off_k<Cf::KCH>(32 * p + pair_key(1, lr), 4 * s + lg));
          P0 = mfma16x16x32(A0, qf[s], P0);
          P1 = mfma16x16x32(A1, qf[s], P1);
        }
        const int j0 = 32 * p + 8 * lg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ja = j0 + i, jb = j0 + 4 + i;
          P0[i] = (ja <= qq) ? P0[i] * pw[qq - ja] : 0.f;
          P1[i] = (jb <= qq) ? P1[i] * pw[qq - jb] : 0.f;
        }
        const u32x4 Bp = {pack_bf16x2(P0[0], P0[1]), pack_bf16x2(P0[2], P0[3]), pack_bf16x2(P1[0], P1[1]),
                          pack_bf16x2(P1[2], P1[3])};
#pragma unroll
        for (int dv = 0; dv < Cf::ND; ++dv)
          Oacc[dv] = mfma16x16x32(lds_load<u32x4>(lds + Cf::VT_OFF, off_t<Cf::TCH>(16 * dv + lr, 4 * p + lg)), Bp,
                                  Oacc[dv]);
      }
      // (4) write this lane's output row
      if (qq < m) {
        uint16_t *orow = ob + (size_t)(c0 + qq) * D;
#pragma unroll
        for (int dv = 0; dv < Cf::ND; ++dv)
          *reinterpret_cast<u32x2 *>(orow + 16 * dv + 4 * lg) =
              u32x2{pack_bf16x2(Oacc[dv][0], Oacc[dv][1]), pack_bf16x2(Oacc[dv][2], Oacc[dv][3])};
      }
    }

    // (5) S = lam^m S + (diag(lam^(m-1-j)) K)^T V
    state_update<C, D>(lds, w, lr, lg, pw[m], Sacc);

    if (c0 + C < t_end) {
#pragma unroll
      for (int s = 0; s < Cf::NDS; ++s) qf[s] = qn[s];
    }
  }

  if (state_out && seg == nseg - 1) {
    float *so = state_out + (size_t)bh * D * D;
#pragma unroll
    for (int a = 0; a < Cf::NDV; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(size_t)(16 * dkt + 4 * lg + i) * D + 16 * (dv0 + a) + lr] = Sacc[a][i];
  }
}

// ---------------------------------------------------------------- fp32 path
// One workgroup per (b, h); thread = one d_v column of the state.
template <int D>
__global__ __launch_bounds__(D) void lin_recurrent_f32(const float *__restrict__ q, const float *__restrict__ k,
                                                       const float *__restrict__ v, float *__restrict__ o,
                                                       const float *__restrict__ decay,
                                                       const float *__restrict__ state_in,
                                                       float *__restrict__ state_out, int H, int N) {
  constexpr int T = 32;  // tokens staged per step
  __shared__ float qs[T][D];
  __shared__ float ks[T][D];
  const int bh = blockIdx.x, h = bh % H, col = threadIdx.x;
  const float lam = decay ? decay[h] : 1.f;
  const size_t off = (size_t)bh * N * D;
  float S[D];
#pragma unroll
  for (int r = 0; r < D; ++r) S[r] = state_in ? state_in[(size_t)bh * D * D + (size_t)r * D + col] : 0.f;
  for (int t0 = 0; t0 < N; t0 += T) {
    const int nt = min(T, N - t0);
    __syncthreads();
    for (int i = col; i < nt * D; i += D) {
      qs[i / D][i % D] = q[off + (size_t)t0 * D + i];
      ks[i / D][i % D] = k[off + (size_t)t0 * D + i];
    }
    __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
      const float vv = v[off + (size_t)(t0 + tt) * D + col];
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < D; ++r) {
        S[r] = fmaf(lam, S[r], ks[tt][r] * vv);
        acc = fmaf(qs[tt][r], S[r], acc);
      }
      o[off + (size_t)(t0 + tt) * D + col] = acc;
    }
  }
  if (state_out) {
#pragma unroll
    for (int r = 0; r < D; ++r) state_out[(size_t)bh * D * D + (size_t)r * D + col] = S[r];
  }
}

// Segments: about 4 workgroups per CU over all (b, h), whole chunks each.
void seg_plan(int BH, int N, int C, int *seg_len, int *nseg) {
  const int target = 1024;
  const int nchunks = (N + C - 1) / C;
  int want = (target + BH - 1) / BH;
  if (want < 1) want = 1;
  if (want > nchunks) want = nchunks;
  const int cps = (nchunks + want - 1) / want;  // chunks per segment
  *seg_len = cps * C;
  *nseg = (N + *seg_len - 1) / *seg_len;
}

template <int C, int D>
hipError_t run_bf16(const LinearPrefillArgs &a, hipStream_t st) {
  const int BH = a.B * a.H;
  int seg_len, nseg;
  seg_plan(BH, a.N, C, &seg_len, &nseg);
  float *ws = static_cast<float *>(a.ws);
  const size_t DD = (size_t)D * D;
  const float *seg_state = a.state_in;  // nseg == 1: segment 0 starts from state_in
  if (nseg > 1) {
    hipLaunchKernelGGL((lin_seg_aggregate<C, D>), dim3(BH * (nseg - 1)), dim3(512), 0, st,
                       (const uint16_t *)a.k, (const uint16_t *)a.v, a.decay, ws, a.H, a.N, seg_len, nseg);
    hipLaunchKernelGGL(lin_seg_scan, dim3((unsigned)((DD + 255) / 256), BH), dim3(256), 0, st, ws,
                       a.state_in, a.decay, a.H, (int)DD, a.N, seg_len, nseg);
    seg_state = ws;
  }
  hipLaunchKernelGGL((lin_seg_output<C, D>), dim3(BH * nseg), dim3(512), 0, st, (const uint16_t *)a.q,
                     (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.o, a.decay, seg_state, DD,
                     a.state_out, a.H, a.N, seg_len, nseg);
  return hipGetLastError();
}

}  // namespace

size_t linear_prefill_workspace(int dtype, int B, int H, int N, int d, int chunk) {
  if (dtype != 1) return 0;
  int seg_len, nseg;
  seg_plan(B * H, N, chunk, &seg_len, &nseg);
  if (nseg <= 1) return 0;
  return (size_t)B * H * nseg * d * d * sizeof(float);
}

hipError_t launch_linear_prefill(const LinearPrefillArgs &a, hipStream_t st) {
  if (a.dtype == 0) {
    if (a.d == 64)
      hipLaunchKernelGGL(lin_recurrent_f32<64>, dim3(a.B * a.H), dim3(64), 0, st, (const float *)a.q,
                         (const float *)a.k, (const float *)a.v, (float *)a.o, a.decay, a.state_in, a.state_out,
                         a.H, a.N);
    else
      hipLaunchKernelGGL(lin_recurrent_f32<128>, dim3(a.B * a.H), dim3(128), 0, st, (const float *)a.q,
                         (const float *)a.k, (const float *)a.v, (float *)a.o, a.decay, a.state_in, a.state_out,
                         a.H, a.N);
    return hipGetLastError();
  }
  if (a.chunk == 128 && a.d == 128) return run_bf16<128, 128>(a, st);
  if (a.chunk == 64 && a.d == 128) return run_bf16<64, 128>(a, st);
  if (a.chunk == 128 && a.d == 64) return run_bf16<128, 64>(a, st);
  return run_bf16<64, 64>(a, st);
}

}  // namespace sala
