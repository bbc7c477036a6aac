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
  static constexpr int NT = 512;               // 8 waves, two per SIMD
  static constexpr int NCH = D / 8;            // 16-byte chunks per K / V / S^T row
  static constexpr int ROWB = D * 2;           // bytes per row
  static constexpr int ND = D / 16;            // 16-wide feature tiles
  static constexpr int NDS = D / 32;           // 32-deep steps over features
  static constexpr int NKS = C / 32;           // 32-deep steps over chunk tokens
  static constexpr int NQP = C / 32;           // pairs of 16-query tiles per chunk
  static constexpr int WPP = 8 / NQP;          // waves sharing one query pair (split over d_v)
  static constexpr int DVW = ND / WPP;         // output d_v tiles per wave
  static constexpr int SDV = ND * ND / 8;      // state tiles per wave (one d_k tile, SDV d_v tiles)
  static constexpr int RPP = NT / NCH;         // K/V rows staged per pass of the workgroup
  static constexpr int NSTG = C / RPP;         // staging passes (16-byte K and V pieces per thread)
  static constexpr uint32_t KN = 0;                    // K, natural [token][d_k], swizzled
  static constexpr uint32_t VN = KN + C * ROWB;        // V, natural [token][d_v], swizzled
  static constexpr uint32_t ST = VN + C * ROWB;        // bf16 S^T [d_v][d_k], swizzled
  static constexpr int PWZ = 32;                        // zero entries below n = 0
  static constexpr uint32_t PW = ST + D * ROWB;        // [PWZ zeros] lam^n, n = 0..C
  static constexpr uint32_t RW = PW + (PWZ + C + 4) * 4;  // lam^(m-1-j) for the chunk's rows, 0 past m
  static constexpr uint32_t LDS = RW + C * 4;
  static_assert(DVW >= 1 && NSTG >= 1 && SDV >= 1, "unsupported chunk / head size");
  // wave -> (query pair, d_v part).  Waves w and w+4 share a SIMD; they get
  // query pairs from opposite ends of the chunk so the causal work per SIMD
  // is even.
  __device__ static void qrole(int w, int &gq, int &part) {
    if (w < 4) {
      gq = w % NQP;
      part = w / NQP;
    } else {
      gq = NQP - 1 - (w - 4) % NQP;
      part = WPP / 2 + (w - 4) / NQP;
    }
  }
};

// K and V rows live in LDS in their natural layout with 16-byte chunks XOR-
// swizzled by row (fkv): conflict-free for the plain 16-byte reads of 16 rows
// of one key pair and for the transposed reads (lds_read_tr).
// S^T rows are read 16 consecutive rows at one chunk: row bits 0..2 go to
// chunk bits 1..3 (conflict-free by the same measurement as fkv).
__device__ __forceinline__ uint32_t fst(uint32_t row) { return (row & 7u) << 1; }

template <int C, int D>
__device__ __forceinline__ u32x4 tr_frag(const char *lds, uint32_t base_k0, uint32_t lane_tr, uint32_t xtr,
                                         int tile) {
  return sala::tr_frag(lds, base_k0, lane_tr, xtr, tile, LinCfg<C, D>::NCH, LinCfg<C, D>::ROWB);
}

// K and V rows c0 .. c0+C-1 -> registers (thread: NSTG 16-byte pieces of
// each).  Rows at or past t_end load a clamped row; store_kv zeroes them.
// Nothing here uses the loaded values, so the loads stay in flight until
// store_kv of the next chunk step.
template <int C, int D>
__device__ __forceinline__ void load_kv(const uint16_t *kb, const uint16_t *vb, int tid, int c0, int t_end,
                                        u32x4 (&xk)[LinCfg<C, D>::NSTG], u32x4 (&xv)[LinCfg<C, D>::NSTG]) {
  using Cf = LinCfg<C, D>;
  const int ch = tid % Cf::NCH;
#pragma unroll
  for (int u = 0; u < Cf::NSTG; ++u) {
    const int t = min(c0 + tid / Cf::NCH + Cf::RPP * u, t_end - 1);
    xk[u] = gload16(kb + (size_t)t * D + 8 * ch);
    xv[u] = gload16(vb + (size_t)t * D + 8 * ch);
  }
}
// Registers -> K_lds / V_lds (natural layout, fkv-swizzled); chunk rows at or
// past m are written as zero.
template <int C, int D>
__device__ __forceinline__ void store_kv(char *lds, int tid, int m, const u32x4 (&xk)[LinCfg<C, D>::NSTG],
                                         const u32x4 (&xv)[LinCfg<C, D>::NSTG]) {
  using Cf = LinCfg<C, D>;
  const uint32_t ch = tid % Cf::NCH;
  const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < Cf::NSTG; ++u) {
    const uint32_t row = tid / Cf::NCH + Cf::RPP * u;
    const uint32_t off = row * Cf::ROWB + ((ch ^ fkv(row)) & (Cf::NCH - 1)) * 16u;
    const bool live = (int)row < m;
    lds_store(lds + Cf::KN, off, live ? xk[u] : zero);
    lds_store(lds + Cf::VN, off, live ? xv[u] : zero);
  }
}

// State update for this wave's tiles (d_k tile sdk, d_v tiles sdv0 ..):
//   S = lam^m S + (diag(lam^(m-1-j)) K)^T V
// A = K^T fragments by transposed reads, scaled per token in fp32 and rounded
// once to bf16; B = V fragments by transposed reads.
template <int C, int D>
__device__ __forceinline__ void state_update(const char *lds, int sdk, int sdv0, int g, uint32_t lane_tr,
                                             uint32_t xtr, float lam_m, f32x4 (&Sacc)[LinCfg<C, D>::SDV]) {
  using Cf = LinCfg<C, D>;
#pragma unroll
  for (int a = 0; a < Cf::SDV; ++a) Sacc[a] *= lam_m;
#pragma unroll
  for (int ks = 0; ks < Cf::NKS; ++ks) {
    u32x4 A = tr_frag<C, D>(lds, Cf::KN + 32 * ks * Cf::ROWB, lane_tr, xtr, sdk);
    const f32x4 w0 = lds_load<f32x4>(lds + Cf::RW, (32 * ks + 8 * g) * 4);
    const f32x4 w1 = lds_load<f32x4>(lds + Cf::RW, (32 * ks + 8 * g + 4) * 4);
    A[0] = pack_bf16x2(bf16lo(A[0]) * w0[0], bf16hi(A[0]) * w0[1]);
    A[1] = pack_bf16x2(bf16lo(A[1]) * w0[2], bf16hi(A[1]) * w0[3]);
    A[2] = pack_bf16x2(bf16lo(A[2]) * w1[0], bf16hi(A[2]) * w1[1]);
    A[3] = pack_bf16x2(bf16lo(A[3]) * w1[2], bf16hi(A[3]) * w1[3]);
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a)
      Sacc[a] = mfma16x16x32(A, tr_frag<C, D>(lds, Cf::VN + 32 * ks * Cf::ROWB, lane_tr, xtr, sdv0 + a), Sacc[a]);
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
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int nagg = nseg - 1;
  const int bh = blockIdx.x / nagg, seg = blockIdx.x % nagg;
  const int h = bh % H;
  const int t_begin = seg * seg_len, t_end = min(N, t_begin + seg_len);
  const float lam = decay ? decay[h] : 1.f;
  float *pw = reinterpret_cast<float *>(lds + Cf::PW) + Cf::PWZ;  // pw[n] = lam^n, 0 for n < 0
  float *rw = reinterpret_cast<float *>(lds + Cf::RW);
  for (int n = tid - Cf::PWZ; n <= C; n += Cf::NT) pw[n] = n < 0 ? 0.f : (float)pow((double)lam, (double)n);
  const uint16_t *kb = k + (size_t)bh * N * D;
  const uint16_t *vb = v + (size_t)bh * N * D;
  const int sdk = (w * Cf::SDV) / Cf::ND, sdv0 = (w * Cf::SDV) % Cf::ND;
  const uint32_t lane_tr = tr_lane_off(l, Cf::ROWB), xtr = tr_lane_xor(l);

  f32x4 Sacc[Cf::SDV];
#pragma unroll
  for (int a = 0; a < Cf::SDV; ++a) Sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 xk[Cf::NSTG], xv[Cf::NSTG];
  load_kv<C, D>(kb, vb, tid, t_begin, t_end, xk, xv);
  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    const int m = min(C, t_end - c0);
    __syncthreads();
    store_kv<C, D>(lds, tid, m, xk, xv);
    if (tid < C) rw[tid] = (tid < m) ? pw[m - 1 - tid] : 0.f;
    __syncthreads();
    if (c0 + C < t_end) load_kv<C, D>(kb, vb, tid, c0 + C, t_end, xk, xv);
    state_update<C, D>(lds, sdk, sdv0, g, lane_tr, xtr, pw[m], Sacc);
  }
  float *out = seg_state + ((size_t)bh * nseg + seg) * D * D;
#pragma unroll
  for (int a = 0; a < Cf::SDV; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(size_t)(16 * sdk + 4 * g + i) * D + 16 * (sdv0 + a) + lr] = Sacc[a][i];
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
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const int h = bh % H;
  const int t_begin = seg * seg_len, t_end = min(N, t_begin + seg_len);
  const float lam = decay ? decay[h] : 1.f;
  float *pw = reinterpret_cast<float *>(lds + Cf::PW) + Cf::PWZ;  // pw[n] = lam^n, 0 for n < 0
  float *rw = reinterpret_cast<float *>(lds + Cf::RW);
  for (int n = tid - Cf::PWZ; n <= C; n += Cf::NT) pw[n] = n < 0 ? 0.f : (float)pow((double)lam, (double)n);
  const size_t head_off = (size_t)bh * N * D;
  const uint16_t *qb = q + head_off, *kb = k + head_off, *vb = v + head_off;
  uint16_t *ob = o + head_off;
  int gq, part;
  Cf::qrole(w, gq, part);
  const int dvb = part * Cf::DVW;  // first output d_v tile of this wave
  const int sdk = (w * Cf::SDV) / Cf::ND, sdv0 = (w * Cf::SDV) % Cf::ND;
  const uint32_t lane_tr = tr_lane_off(l, Cf::ROWB), xtr = tr_lane_xor(l);

  f32x4 Sacc[Cf::SDV];
  const float *sin = seg_state ? seg_state + (size_t)bh * seg_stride * nseg + (size_t)seg * seg_stride : nullptr;
#pragma unroll
  for (int a = 0; a < Cf::SDV; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      Sacc[a][i] = sin ? sin[(size_t)(16 * sdk + 4 * g + i) * D + 16 * (sdv0 + a) + lr] : 0.f;

  // Q fragments (B operands of Q^T): query tiles 2gq, 2gq+1 of the chunk;
  // rows past t_end load a clamped row whose outputs are never stored
  u32x4 qf[2][Cf::NDS];
  auto load_q = [&](int c0) {
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const int t = min(c0 + 32 * gq + 16 * tq + lr, t_end - 1);
#pragma unroll
      for (int s = 0; s < Cf::NDS; ++s) qf[tq][s] = gload16(qb + (size_t)t * D + 32 * s + 8 * g);
    }
  };
  u32x4 xk[Cf::NSTG], xv[Cf::NSTG];
  load_kv<C, D>(kb, vb, tid, t_begin, t_end, xk, xv);
  load_q(t_begin);

  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    const int m = min(C, t_end - c0);
    __syncthreads();
    store_kv<C, D>(lds, tid, m, xk, xv);
    // bf16 copy of S^T (rows d_v, columns d_k) for the Q S product
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a) {
      const uint32_t row = 16 * (sdv0 + a) + lr;
      const uint32_t off = row * Cf::ROWB + (((2 * sdk + (g >> 1)) ^ fst(row)) & (Cf::NCH - 1)) * 16u + (g & 1) * 8;
      lds_store(lds + Cf::ST, off, u32x2{pack_bf16x2(Sacc[a][0], Sacc[a][1]), pack_bf16x2(Sacc[a][2], Sacc[a][3])});
    }
    if (tid < C) rw[tid] = (tid < m) ? pw[m - 1 - tid] : 0.f;
    __syncthreads();
    if (c0 + C < t_end) load_kv<C, D>(kb, vb, tid, c0 + C, t_end, xk, xv);

    // (1) O^T = lam^(qq+1) * S^T Q^T for d_v tiles dvb .. and both query tiles
    f32x4 Oacc[Cf::DVW][2];
#pragma unroll
    for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
      const uint32_t row = 16 * (dvb + dvi) + lr;
#pragma unroll
      for (int s = 0; s < Cf::NDS; ++s) {
        const u32x4 A = lds_load<u32x4>(lds + Cf::ST, row * Cf::ROWB + (((4 * s + g) ^ fst(row)) & (Cf::NCH - 1)) * 16u);
        a0 = mfma16x16x32(A, qf[0][s], a0);
        a1 = mfma16x16x32(A, qf[1][s], a1);
      }
      Oacc[dvi][0] = a0;
      Oacc[dvi][1] = a1;
    }
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const float f = pw[32 * gq + 16 * tq + lr + 1];
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) Oacc[dvi][tq] *= f;
    }
    // (2)+(3) P^T = decay-masked K Q^T over the causal key pairs; O^T += V^T P^T
    for (int p = 0; p <= gq; ++p) {
      f32x4 P[2][2];
#pragma unroll
      for (int tq = 0; tq < 2; ++tq)
#pragma unroll
        for (int t = 0; t < 2; ++t) P[tq][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < Cf::NDS; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t row = 32 * p + pair_key(t, lr);
          const u32x4 A = lds_load<u32x4>(lds + Cf::KN, row * Cf::ROWB + (((4 * s + g) ^ fkv(row)) & (Cf::NCH - 1)) * 16u);
          P[0][t] = mfma16x16x32(A, qf[0][s], P[0][t]);
          P[1][t] = mfma16x16x32(A, qf[1][s], P[1][t]);
        }
      u32x4 Bp[2];
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const int qq = 32 * gq + 16 * tq + lr;
        // lam^(qq-j), zero for j > qq: the table's zero entries below n = 0
        // do the causal mask (qq - j >= -31 within the diagonal pair)
        const int nb = qq - 32 * p - 8 * g;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) P[tq][t][i] *= pw[nb - 4 * t - i];
        Bp[tq] = u32x4{pack_bf16x2(P[tq][0][0], P[tq][0][1]), pack_bf16x2(P[tq][0][2], P[tq][0][3]),
                       pack_bf16x2(P[tq][1][0], P[tq][1][1]), pack_bf16x2(P[tq][1][2], P[tq][1][3])};
      }
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        const u32x4 A = tr_frag<C, D>(lds, Cf::VN + 32 * p * Cf::ROWB, lane_tr, xtr, dvb + dvi);
        Oacc[dvi][0] = mfma16x16x32(A, Bp[0], Oacc[dvi][0]);
        Oacc[dvi][1] = mfma16x16x32(A, Bp[1], Oacc[dvi][1]);
      }
    }
    if (c0 + C < t_end) load_q(c0 + C);  // the Q fragments are free from here on
    // (4) this lane's output rows
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const int qq = 32 * gq + 16 * tq + lr;
      if (qq < m) {
        uint16_t *orow = ob + (size_t)(c0 + qq) * D;
#pragma unroll
        for (int dvi = 0; dvi < Cf::DVW; ++dvi)
          *reinterpret_cast<u32x2 *>(orow + 16 * (dvb + dvi) + 4 * g) =
              u32x2{pack_bf16x2(Oacc[dvi][tq][0], Oacc[dvi][tq][1]), pack_bf16x2(Oacc[dvi][tq][2], Oacc[dvi][tq][3])};
      }
    }
    // (5) S = lam^m S + (diag(lam^(m-1-j)) K)^T V
    state_update<C, D>(lds, sdk, sdv0, g, lane_tr, xtr, pw[m], Sacc);
  }

  if (state_out && seg == nseg - 1) {
    float *so = state_out + (size_t)bh * D * D;
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(size_t)(16 * sdk + 4 * g + i) * D + 16 * (sdv0 + a) + lr] = Sacc[a][i];
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
