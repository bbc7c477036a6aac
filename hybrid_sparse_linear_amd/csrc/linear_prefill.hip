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
  static constexpr int NQT = C / 16;           // 16-query tiles per chunk
  static constexpr int WPQ = 8 / NQT;          // waves sharing one query tile (split over d_v)
  static constexpr int DVW = ND / WPQ;         // output d_v tiles per wave
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
  // wave -> (query tile, d_v part).  Waves w and w+4 share a SIMD; they get
  // query tiles from opposite ends of the chunk, so the causal work (tile qt
  // meets key pairs 0 .. qt/2) is even per SIMD, and no two waves compute the
  // same decay-masked K Q^T tile.
  __device__ static void qrole(int w, int &qt, int &part) {
    if (w < 4) {
      qt = w;
      part = 0;
    } else {
      qt = NQT - 1 - (w - 4);
      part = WPQ - 1;
    }
  }
};

// K and V rows live in LDS in their natural layout with 16-byte chunks XOR-
// swizzled by row (fkv): conflict-free for the plain 16-byte reads of 16 rows
// of one key pair and for the transposed reads (lds_read_tr).  S^T rows are
// read 16 consecutive rows at one chunk and use fst.

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
// past m are written as zero (only the last chunk of a segment can be short,
// so full chunks take a branch without the per-dword selects).
template <int C, int D>
__device__ __forceinline__ void store_kv(char *lds, int tid, int m, const u32x4 (&xk)[LinCfg<C, D>::NSTG],
                                         const u32x4 (&xv)[LinCfg<C, D>::NSTG]) {
  using Cf = LinCfg<C, D>;
  const uint32_t ch = tid % Cf::NCH;
  const u32x4 zero = {0, 0, 0, 0};
  auto store = [&](bool whole) {
#pragma unroll
    for (int u = 0; u < Cf::NSTG; ++u) {
      const uint32_t row = tid / Cf::NCH + Cf::RPP * u;
      const uint32_t off = row * Cf::ROWB + ((ch ^ fkv(row)) & (Cf::NCH - 1)) * 16u;
      const bool live = whole || (int)row < m;
      lds_store(lds + Cf::KN, off, live ? xk[u] : zero);
      lds_store(lds + Cf::VN, off, live ? xv[u] : zero);
    }
  };
  if (m >= C) store(true);
  else store(false);
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

// ---------------------------------------------------------------- fused neighbours
// QK RMS normalisation and HyPE RoPE applied to q and k as they are staged,
// and the output gate applied to o as it is stored (MiniCPM-SALA, gist.science
// (ja) 技術概要 section 2.2 and gist.science (de) section 2,
// "Architektur-Hybridisierung": RoPE on the linear layers, QK normalisation,
// an output gate after every attention block).  Forms: x / sqrt(mean(x^2) +
// eps) * gamma over the head dimension; rotate-half RoPE, feature i turned
// with feature i + D/2 by p * base^(-2i/D) at the absolute position p;
// o * sigmoid(g).
struct NbK {
  const float *gq, *gk;   // RMS-norm weights [D] or nullptr
  float eps, rope_base;   // rope_base <= 0: no RoPE
  long long pos0;         // absolute position of token 0
  const uint16_t *gate;   // [B, H, N, D] bf16 gate pre-activation or nullptr
};

// Fused staging: a thread owns 16-byte piece hc (features 8hc .. 8hc+7) and
// piece hc + HC (features D/2 + 8hc ..) of rows tid/HC + RPF*u, so the
// rotate-half partners of its features are its own and a row's sum of
// squares is a sum over HC consecutive lanes.
template <int C, int D>
struct LinF {
  static constexpr int HC = D / 16;
  static constexpr int RPF = 512 / HC;
  static constexpr int NSF = (C + RPF - 1) / RPF;
  // tables after the plain layout: Q rows, gamma_q | gamma_k, theta_i / 2pi (fp64, fp32)
  static constexpr uint32_t QN = (LinCfg<C, D>::LDS + 15u) & ~15u;
  static constexpr uint32_t GAM = QN + C * LinCfg<C, D>::ROWB;
  static constexpr uint32_t TRV = GAM + 2 * D * 4;
  static constexpr uint32_t TRF = TRV + (D / 2) * 8;
  static constexpr uint32_t LDS = TRF + (D / 2) * 4;
};

// xr: buffer resource over one head's [N, D] rows
template <int C, int D>
__device__ __forceinline__ void load_rows_f(__amdgpu_buffer_rsrc_t xr, int tid, int c0, int t_end,
                                            u32x4 (&x)[LinF<C, D>::NSF][2]) {
  using F = LinF<C, D>;
  const uint32_t hc = tid % F::HC;
#pragma unroll
  for (int u = 0; u < F::NSF; ++u) {
    const uint32_t t = min(c0 + tid / F::HC + F::RPF * u, t_end - 1);
    x[u][0] = bload16(xr, (t * D + 8 * hc) * 2u);
    x[u][1] = bload16(xr, (t * D + D / 2 + 8 * hc) * 2u);
  }
}
// Rows -> LDS in the plain layout (fkv-swizzled 16-byte chunks); rows at or
// past m are written as zero (full chunks skip the per-dword selects).
template <int C, int D>
__device__ __forceinline__ void store_rows_f(char *dst, int tid, int m, const u32x4 (&x)[LinF<C, D>::NSF][2]) {
  using F = LinF<C, D>;
  using Cf = LinCfg<C, D>;
  const uint32_t hc = tid % F::HC;
  const u32x4 zero = {0, 0, 0, 0};
  auto store = [&](bool whole) {  // whole: a full chunk, no row past the end
#pragma unroll
    for (int u = 0; u < F::NSF; ++u) {
      const uint32_t row = tid / F::HC + F::RPF * u;
      if (F::RPF * F::NSF > C && row >= (uint32_t)C) continue;
      const bool live = whole || (int)row < m;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t ch = hc + F::HC * h;
        lds_store(dst, row * Cf::ROWB + ((ch ^ fkv(row)) & (Cf::NCH - 1)) * 16u, live ? x[u][h] : zero);
      }
    }
  };
  if (m >= C) store(true);
  else store(false);
}
// theta_i / 2pi for i < D/2 (fp64 and fp32) and the norm weights into LDS.
template <int C, int D>
__device__ __forceinline__ void nb_tables(char *lds, int tid, const NbK &nb) {
  using F = LinF<C, D>;
  float *gam = reinterpret_cast<float *>(lds + F::GAM);
  if (tid < D) gam[tid] = nb.gq ? nb.gq[tid] : 1.f;
  else if (tid < 2 * D) gam[tid] = nb.gk ? nb.gk[tid - D] : 1.f;
  if (tid < D / 2 && nb.rope_base > 0.f) {
    const double t = pow((double)nb.rope_base, -2.0 * tid / D) * 0.15915494309189535;  // / 2pi
    reinterpret_cast<double *>(lds + F::TRV)[tid] = t;
    reinterpret_cast<float *>(lds + F::TRF)[tid] = (float)t;
  }
}
// Fraction of a turn of p0 * theta_i / 2pi for this thread's features (fp64).
template <int C, int D>
__device__ __forceinline__ void rope_base_turns(const char *lds, int hc, long long p0, float (&b)[8]) {
  using F = LinF<C, D>;
  const double *trv = reinterpret_cast<const double *>(lds + F::TRV);
  const double p = (double)p0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double x = p * trv[8 * hc + e];
    b[e] = (float)(x - floor(x));
  }
}
// One row of q or k: lo = features 8hc .., hi = features D/2 + 8hc .., in place.
// cos / sin of the angles of this thread's features at chunk row `row`:
// turns = base turns of the chunk (fp64-reduced) + row * theta_i / 2pi.
template <int C, int D>
__device__ __forceinline__ void rope_cs(const char *lds, int hc, int row, const float (&b)[8], float (&c)[8],
                                        float (&sn)[8]) {
  const float *trf = reinterpret_cast<const float *>(lds + LinF<C, D>::TRF);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float turns = fmaf((float)row, trf[8 * hc + e], b[e]);
    c[e] = __builtin_amdgcn_cosf(turns);
    sn[e] = __builtin_amdgcn_sinf(turns);
  }
}
template <int C, int D>
__device__ __forceinline__ void nb_row(const char *lds, int hc, bool norm, int which, float eps, bool rope,
                                       const float (&c)[8], const float (&sn)[8], u32x4 &lo, u32x4 &hi) {
  using F = LinF<C, D>;
  if (!norm && !rope) return;  // rows pass through unchanged
  float a[8], z[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[2 * e] = bf16lo(lo[e]);
    a[2 * e + 1] = bf16hi(lo[e]);
    z[2 * e] = bf16lo(hi[e]);
    z[2 * e + 1] = bf16hi(hi[e]);
  }
  if (norm) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(z[e], z[e], fmaf(a[e], a[e], ss));
    ss = lane_group_sum<F::HC>(ss);
    const float r = rsqrtf(fmaf(ss, 1.f / D, eps));
    const char *gam = lds + F::GAM + which * D * 4;
    const f32x4 ga0 = lds_load<f32x4>(gam, 32u * hc), ga1 = lds_load<f32x4>(gam, 32u * hc + 16u);
    const f32x4 gz0 = lds_load<f32x4>(gam, (D / 2 + 8u * hc) * 4u), gz1 = lds_load<f32x4>(gam, (D / 2 + 8u * hc) * 4u + 16u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] *= r * ga0[e];
      a[e + 4] *= r * ga1[e];
      z[e] *= r * gz0[e];
      z[e + 4] *= r * gz1[e];
    }
  }
  if (rope) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ya = fmaf(-z[e], sn[e], a[e] * c[e]), yz = fmaf(a[e], sn[e], z[e] * c[e]);
      a[e] = ya;
      z[e] = yz;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = pack_bf16x2(a[2 * e], a[2 * e + 1]);
    hi[e] = pack_bf16x2(z[2 * e], z[2 * e + 1]);
  }
}

// ---------------------------------------------------------------- pass 1
// F: k is normalised and rotated as it is staged (the fused form).
template <int C, int D, bool F>
__global__ __launch_bounds__(512) void lin_seg_aggregate(const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v,
                                                         const float *__restrict__ decay,
                                                         float *__restrict__ seg_state, int H, int N,
                                                         int seg_len, int nseg, NbK nb) {
  using Cf = LinCfg<C, D>;
  using Fz = LinF<C, D>;
  __shared__ __attribute__((aligned(16))) char lds[F ? Fz::LDS : Cf::LDS];
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
  if constexpr (F) {
    nb_tables<C, D>(lds, tid, nb);
    const bool norm = nb.gk != nullptr, rope = nb.rope_base > 0.f;
    const int hc = tid % Fz::HC;
    const auto kr = buf_rsrc(kb, (uint32_t)N * D * 2u), vr = buf_rsrc(vb, (uint32_t)N * D * 2u);
    u32x4 xk[Fz::NSF][2], xv[Fz::NSF][2];
    load_rows_f<C, D>(kr, tid, t_begin, t_end, xk);
    load_rows_f<C, D>(vr, tid, t_begin, t_end, xv);
    for (int c0 = t_begin; c0 < t_end; c0 += C) {
      const int m = min(C, t_end - c0);
      __syncthreads();
      float bt[8], cs[8], sn[8];
      if (rope) rope_base_turns<C, D>(lds, hc, nb.pos0 + c0, bt);
#pragma unroll
      for (int u = 0; u < Fz::NSF; ++u) {
        const int row = tid / Fz::HC + Fz::RPF * u;
        if (rope) rope_cs<C, D>(lds, hc, row, bt, cs, sn);
        nb_row<C, D>(lds, hc, norm, 1, nb.eps, rope, cs, sn, xk[u][0], xk[u][1]);
        __builtin_amdgcn_sched_barrier(0);  // one row's temporaries live at a time
      }
      store_rows_f<C, D>(lds + Cf::KN, tid, m, xk);
      store_rows_f<C, D>(lds + Cf::VN, tid, m, xv);
      if (tid < C) rw[tid] = (tid < m) ? pw[m - 1 - tid] : 0.f;
      __syncthreads();
      if (c0 + C < t_end) {
        load_rows_f<C, D>(kr, tid, c0 + C, t_end, xk);
        load_rows_f<C, D>(vr, tid, c0 + C, t_end, xv);
      }
      state_update<C, D>(lds, sdk, sdv0, g, lane_tr, xtr, pw[m], Sacc);
    }
  } else {
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
// q, k and v of a chunk are staged through LDS in rows (a thread owns two
// 16-byte pieces of a row); q and k are normalised and rotated there when the
// neighbours ask for it, and the output is gated when a gate is given.  The
// output rows are stored after the state update so that gate loads are in
// flight during it.  (Loading q straight into MFMA fragments reads each row
// in 64-byte pieces; the row-wise staging is faster even with nothing to
// apply.)
template <int C, int D>
__global__ __launch_bounds__(512) void lin_seg_output(const uint16_t *__restrict__ q,
                                                      const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v,
                                                      uint16_t *__restrict__ o,
                                                      const float *__restrict__ decay,
                                                      const float *__restrict__ seg_state,
                                                      size_t seg_stride, float *__restrict__ state_out,
                                                      int H, int N, int seg_len, int nseg, NbK nb) {
  using Cf = LinCfg<C, D>;
  using Fz = LinF<C, D>;
  __shared__ __attribute__((aligned(16))) char lds[Fz::LDS];
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
  int qt, part;
  Cf::qrole(w, qt, part);
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

  // Q fragment s (B operand of Q^T, query tile qt): read from the staged Q
  // rows in LDS at each use
  const int qq = 16 * qt + lr;  // this lane's query row in the chunk
  auto qfrag = [&](int s) -> u32x4 {
    return lds_load<u32x4>(lds + Fz::QN, qq * Cf::ROWB + (((4 * s + g) ^ fkv(qq)) & (Cf::NCH - 1)) * 16u);
  };
  // this lane's output row, gated by gv when given
  auto store_out = [&](int c0, int m, const f32x4 (&Oacc)[Cf::DVW], const u32x2 (&gv)[Cf::DVW], bool gated) {
    if (qq < m) {
      uint16_t *orow = ob + (size_t)(c0 + qq) * D;
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        f32x4 x = Oacc[dvi];
        if (gated) {
          x[0] *= sigmoid_fast(bf16lo(gv[dvi][0]));
          x[1] *= sigmoid_fast(bf16hi(gv[dvi][0]));
          x[2] *= sigmoid_fast(bf16lo(gv[dvi][1]));
          x[3] *= sigmoid_fast(bf16hi(gv[dvi][1]));
        }
        *reinterpret_cast<u32x2 *>(orow + 16 * (dvb + dvi) + 4 * g) =
            u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      }
    }
  };

  // next chunk's 16-byte staging pieces (rows x halves)
  u32x4 xk[Fz::NSF][2], xv[Fz::NSF][2], xq[Fz::NSF][2];
  const int hc = tid % Fz::HC;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto qr = buf_rsrc(qb, head_bytes), kr = buf_rsrc(kb, head_bytes), vr = buf_rsrc(vb, head_bytes);
  const auto gr = buf_rsrc(nb.gate ? nb.gate + head_off : qb, head_bytes);
  nb_tables<C, D>(lds, tid, nb);
  const bool norm_q = nb.gq != nullptr, norm_k = nb.gk != nullptr, rope = nb.rope_base > 0.f;
  load_rows_f<C, D>(kr, tid, t_begin, t_end, xk);
  load_rows_f<C, D>(vr, tid, t_begin, t_end, xv);
  load_rows_f<C, D>(qr, tid, t_begin, t_end, xq);

  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    const int m = min(C, t_end - c0);
    __syncthreads();
    {
      float bt[8], cs[8], sn[8];
      if (rope) rope_base_turns<C, D>(lds, hc, nb.pos0 + c0, bt);
#pragma unroll
      for (int u = 0; u < Fz::NSF; ++u) {
        const int row = tid / Fz::HC + Fz::RPF * u;
        if (rope) rope_cs<C, D>(lds, hc, row, bt, cs, sn);
        nb_row<C, D>(lds, hc, norm_q, 0, nb.eps, rope, cs, sn, xq[u][0], xq[u][1]);
        nb_row<C, D>(lds, hc, norm_k, 1, nb.eps, rope, cs, sn, xk[u][0], xk[u][1]);
        __builtin_amdgcn_sched_barrier(0);  // one row's temporaries live at a time
      }
      store_rows_f<C, D>(lds + Fz::QN, tid, m, xq);
      store_rows_f<C, D>(lds + Cf::KN, tid, m, xk);
      store_rows_f<C, D>(lds + Cf::VN, tid, m, xv);
    }
    // bf16 copy of S^T (rows d_v, columns d_k) for the Q S product
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a) {
      const uint32_t row = 16 * (sdv0 + a) + lr;
      const uint32_t off = row * Cf::ROWB + (((2 * sdk + (g >> 1)) ^ fst(row)) & (Cf::NCH - 1)) * 16u + (g & 1) * 8;
      lds_store(lds + Cf::ST, off, u32x2{pack_bf16x2(Sacc[a][0], Sacc[a][1]), pack_bf16x2(Sacc[a][2], Sacc[a][3])});
    }
    if (tid < C) rw[tid] = (tid < m) ? pw[m - 1 - tid] : 0.f;
    __syncthreads();
    if (c0 + C < t_end) {
      load_rows_f<C, D>(kr, tid, c0 + C, t_end, xk);
      load_rows_f<C, D>(vr, tid, c0 + C, t_end, xv);
    }

    // (1) O^T = lam^(qq+1) * S^T Q^T for d_v tiles dvb .. of this wave's query tile
    f32x4 Oacc[Cf::DVW];
#pragma unroll
    for (int dvi = 0; dvi < Cf::DVW; ++dvi) Oacc[dvi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s) {
      const u32x4 q0 = qfrag(s);
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        const uint32_t row = 16 * (dvb + dvi) + lr;
        const u32x4 A = lds_load<u32x4>(lds + Cf::ST, row * Cf::ROWB + (((4 * s + g) ^ fst(row)) & (Cf::NCH - 1)) * 16u);
        Oacc[dvi] = mfma16x16x32(A, q0, Oacc[dvi]);
      }
    }
    {
      const float f = pw[qq + 1];
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) Oacc[dvi] *= f;
    }
    // (2)+(3) P^T = decay-masked K Q^T over the causal key pairs; O^T += V^T P^T
    // unrolled over the chunk's key pairs (the bound is the wave's uniform
    // query tile), so every LDS address below is a fixed register plus an
    // immediate offset rather than a per-pair add
#pragma unroll
    for (int p = 0; p < (Cf::NQT + 1) / 2; ++p) {
      if (p > qt / 2) break;
      f32x4 P[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < Cf::NDS; ++s) {
        const u32x4 q0 = qfrag(s);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t row = 32 * p + pair_key(t, lr);
          const u32x4 A = lds_load<u32x4>(lds + Cf::KN, row * Cf::ROWB + (((4 * s + g) ^ fkv(row)) & (Cf::NCH - 1)) * 16u);
          P[t] = mfma16x16x32(A, q0, P[t]);
        }
      }
      // lam^(qq-j), zero for j > qq: the table's zero entries below n = 0
      // do the causal mask (qq - j >= -31 within the diagonal pair)
      const int nb0 = qq - 32 * p - 8 * g;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) P[t][i] *= pw[nb0 - 4 * t - i];
      const u32x4 Bp = u32x4{pack_bf16x2(P[0][0], P[0][1]), pack_bf16x2(P[0][2], P[0][3]),
                             pack_bf16x2(P[1][0], P[1][1]), pack_bf16x2(P[1][2], P[1][3])};
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        const u32x4 A = tr_frag<C, D>(lds, Cf::VN + 32 * p * Cf::ROWB, lane_tr, xtr, dvb + dvi);
        Oacc[dvi] = mfma16x16x32(A, Bp, Oacc[dvi]);
      }
    }
    // gate values of this lane's outputs (a clamped row is never stored)
    u32x2 gv[Cf::DVW] = {};
    if (nb.gate) {
      const uint32_t t = min(c0 + qq, t_end - 1);
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) gv[dvi] = bload8(gr, (t * D + 16 * (dvb + dvi) + 4 * g) * 2u);
    }
    if (c0 + C < t_end) load_rows_f<C, D>(qr, tid, c0 + C, t_end, xq);
    // (5) S = lam^m S + (diag(lam^(m-1-j)) K)^T V, then (4) the (gated) output row
    state_update<C, D>(lds, sdk, sdv0, g, lane_tr, xtr, pw[m], Sacc);
    store_out(c0, m, Oacc, gv, nb.gate != nullptr);
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
  NbK nb{nullptr, nullptr, 0.f, 0.f, 0, nullptr};
  if (a.nb)
    nb = NbK{a.nb->gamma_q, a.nb->gamma_k, a.nb->eps, a.nb->rope_base, a.nb->pos0,
             static_cast<const uint16_t *>(a.nb->gate)};
  const bool k_transformed = nb.gk != nullptr || nb.rope_base > 0.f;
  const int BH = a.B * a.H;
  int seg_len, nseg;
  seg_plan(BH, a.N, C, &seg_len, &nseg);
  float *ws = static_cast<float *>(a.ws);
  const size_t DD = (size_t)D * D;
  const float *seg_state = a.state_in;  // nseg == 1: segment 0 starts from state_in
  if (nseg > 1) {
    if (k_transformed)
      hipLaunchKernelGGL((lin_seg_aggregate<C, D, true>), dim3(BH * (nseg - 1)), dim3(512), 0, st,
                         (const uint16_t *)a.k, (const uint16_t *)a.v, a.decay, ws, a.H, a.N, seg_len, nseg, nb);
    else
      hipLaunchKernelGGL((lin_seg_aggregate<C, D, false>), dim3(BH * (nseg - 1)), dim3(512), 0, st,
                         (const uint16_t *)a.k, (const uint16_t *)a.v, a.decay, ws, a.H, a.N, seg_len, nseg, nb);
    hipLaunchKernelGGL(lin_seg_scan, dim3((unsigned)((DD + 255) / 256), BH), dim3(256), 0, st, ws,
                       a.state_in, a.decay, a.H, (int)DD, a.N, seg_len, nseg);
    seg_state = ws;
  }
  hipLaunchKernelGGL((lin_seg_output<C, D>), dim3(BH * nseg), dim3(512), 0, st, (const uint16_t *)a.q,
                     (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.o, a.decay, seg_state, DD,
                     a.state_out, a.H, a.N, seg_len, nseg, nb);
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
