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
//           (fp32, written to the workspace), in parts of at most 32 chunks
//           spread over the CUs; parts whose keys cannot reach the segment's
//           end are left out.
//   pass 2  lin_seg_scan: an element-wise scan over segments sums each
//           segment's parts into A_m and turns the A_m into the state entering
//           every segment, S_in(m) = lam^len S_in(m-1) + A_{m-1}.
//   pass 3  lin_seg_output: each segment walks its chunks.  Per chunk of C tokens:
//             O^T  = lam^(i+1) (S^T Q^T)  +  V^T (decay-masked K Q^T)
//             S    = lam^C S + (diag(lam^(C-1-j)) K)^T V
//           with bf16 MFMA 16x16x32 and fp32 accumulation; the fp32 master S
//           stays in registers, a bf16 copy of S^T in LDS feeds the Q S product.
//           The last segment writes S_out.
//           Where two chunk buffers of k | v | q fit the LDS (chunk 64 at
//           d = 128, every chunk at d = 64), lin_seg_output_dma takes this
//           pass: the rows go from HBM straight into LDS (direct loads, the
//           next chunk in flight during the current one), and the fused
//           form's q/k norm and RoPE are applied to them there, in place.
// fp32 path: the same three passes on the VALU in fp32 over tiles of 32
// tokens (lin_f32_pass, lin_seg_scan).
//
// Backward (sala_linear_prefill_backward).  For dO = dL/do and dS = dL/dS_out,
//   dQ    = ((dO V^T) * D) K + diag(lam^(t+1)) dO S_in^T
//   dK    = ((dO V^T) * D)^T Q + diag(lam^(N-1-s)) V dS^T
//   dV    = ((Q K^T) * D)^T dO + diag(lam^(N-1-s)) K dS
//   dS_in = Q^T diag(lam^(t+1)) dO + lam^N dS
// (D the decayed causal mask).  The first is this same forward operation on
// (dO, V, K) with initial state S_in^T.  The other two are the forward
// operation on the time-reversed sequence -- (V, dO, Q) and (K, Q, dO) -- whose
// initial state dS^T / dS enters one decay step later (weight lam^r on
// reversed row r instead of lam^(r+1)); dS_in is lam times the final state of
// the (K, Q, dO) pass.  So every kernel below takes the switches of LinDir.
// The (K, Q, dO) pass's segment states, sums of Q dO^T, are the transposes of
// the (V, dO, Q) pass's sums of dO Q^T, so it reads those instead of running
// its own aggregate and scan.  Where four double-buffered tiles fit the LDS
// (chunk 64, d = 128), lin_seg_grad_kv computes dK and dV in one reversed
// pass from that one state.

#include "sala_common.hpp"
#include "sala_launch.hpp"

namespace sala {
namespace {

// Streaming accesses of the linear passes carry the non-temporal hint (cache
// policy bit nt): every row of q, k, v and o is touched once per pass, and a
// probe of this pass's access pattern without its arithmetic (a workgroup per
// CU, each streaming three inputs of one segment and writing one output)
// moved its bytes at 5.7 TB/s with the hint against 5.1 without.
constexpr int NT_HINT = 2;
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT_HINT));
}
__device__ __forceinline__ void bload16_lds_nt(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3))) *)lds, 16, off, 0, 0, NT_HINT);
}
__device__ __forceinline__ u32x4 gload16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void gstore16_nt(void *p, const u32x4 &v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
// 16-byte store at buffer offset off (dropped past the resource's end).
__device__ __forceinline__ void bstore16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, const u32x4 &v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                         off, 0, NT_HINT);
}

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

// Switches of the backward passes (all zero for the forward operation):
//   rev      tokens are read and written in reverse order (row N-1-t for t)
//   lag      the initial state enters one decay step later: weight lam^t on row
//            t (not lam^(t+1)) and lam^(t) in the states after it
//   state_T  the initial state is read transposed (S[j][i] for S[i][j])
//   scale    the final state is written multiplied by lam
struct LinDir {
  int rev, lag, state_T, scale;
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
template <int C, int D, bool REV>
__device__ __forceinline__ void load_kv(const uint16_t *kb, const uint16_t *vb, int tid, int c0, int t_end, int N,
                                        u32x4 (&xk)[LinCfg<C, D>::NSTG], u32x4 (&xv)[LinCfg<C, D>::NSTG]) {
  using Cf = LinCfg<C, D>;
  const int ch = tid % Cf::NCH;
#pragma unroll
  for (int u = 0; u < Cf::NSTG; ++u) {
    int t = min(c0 + tid / Cf::NCH + Cf::RPP * u, t_end - 1);
    if constexpr (REV) t = N - 1 - t;
    xk[u] = gload16_nt(kb + (size_t)t * D + 8 * ch);
    xv[u] = gload16_nt(vb + (size_t)t * D + 8 * ch);
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
// kn, vn: the K and V tiles; rw: lam^(m-1-j) for the chunk's rows.
template <int C, int D>
__device__ __forceinline__ void state_update(const char *kn, const char *vn, const char *rw, int sdk, int sdv0,
                                             int g, uint32_t lane_tr, uint32_t xtr, float lam_m,
                                             f32x4 (&Sacc)[LinCfg<C, D>::SDV]) {
  using Cf = LinCfg<C, D>;
#pragma unroll
  for (int a = 0; a < Cf::SDV; ++a) Sacc[a] *= lam_m;
#pragma unroll
  for (int ks = 0; ks < Cf::NKS; ++ks) {
    u32x4 A = tr_frag<C, D>(kn, 32 * ks * Cf::ROWB, lane_tr, xtr, sdk);
    const f32x4 w0 = lds_load<f32x4>(rw, (32 * ks + 8 * g) * 4);
    const f32x4 w1 = lds_load<f32x4>(rw, (32 * ks + 8 * g + 4) * 4);
    A[0] = pack_bf16x2(bf16lo(A[0]) * w0[0], bf16hi(A[0]) * w0[1]);
    A[1] = pack_bf16x2(bf16lo(A[1]) * w0[2], bf16hi(A[1]) * w0[3]);
    A[2] = pack_bf16x2(bf16lo(A[2]) * w1[0], bf16hi(A[2]) * w1[1]);
    A[3] = pack_bf16x2(bf16lo(A[3]) * w1[2], bf16hi(A[3]) * w1[3]);
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a)
      Sacc[a] = mfma16x16x32(A, tr_frag<C, D>(vn, 32 * ks * Cf::ROWB, lane_tr, xtr, sdv0 + a), Sacc[a]);
  }
}
template <int C, int D>
__device__ __forceinline__ void state_update(const char *lds, int sdk, int sdv0, int g, uint32_t lane_tr,
                                             uint32_t xtr, float lam_m, f32x4 (&Sacc)[LinCfg<C, D>::SDV]) {
  using Cf = LinCfg<C, D>;
  state_update<C, D>(lds + Cf::KN, lds + Cf::VN, lds + Cf::RW, sdk, sdv0, g, lane_tr, xtr, lam_m, Sacc);
}
// The same update on an NI x NJ block of tiles, d_k tiles sdk .. sdk+NI-1 and
// d_v tiles sdv .. sdv+NJ-1 (Sacc[NJ * i + j]): per 32 tokens a wave reads
// NI K^T and NJ V fragments, so a 2 x 4 block reads 6 where a 1 x 8 row of
// tiles reads 9.
template <int C, int D, int NI, int NJ>
__device__ __forceinline__ void state_update_blk(const char *kn, const char *vn, const char *rw, int sdk, int sdv,
                                                 int g, uint32_t lane_tr, uint32_t xtr, float lam_m,
                                                 f32x4 (&Sacc)[NI * NJ]) {
  using Cf = LinCfg<C, D>;
#pragma unroll
  for (int a = 0; a < NI * NJ; ++a) Sacc[a] *= lam_m;
#pragma unroll
  for (int ks = 0; ks < Cf::NKS; ++ks) {
    const f32x4 w0 = lds_load<f32x4>(rw, (32 * ks + 8 * g) * 4);
    const f32x4 w1 = lds_load<f32x4>(rw, (32 * ks + 8 * g + 4) * 4);
    u32x4 A[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      A[i] = tr_frag<C, D>(kn, 32 * ks * Cf::ROWB, lane_tr, xtr, sdk + i);
      A[i][0] = pack_bf16x2(bf16lo(A[i][0]) * w0[0], bf16hi(A[i][0]) * w0[1]);
      A[i][1] = pack_bf16x2(bf16lo(A[i][1]) * w0[2], bf16hi(A[i][1]) * w0[3]);
      A[i][2] = pack_bf16x2(bf16lo(A[i][2]) * w1[0], bf16hi(A[i][2]) * w1[1]);
      A[i][3] = pack_bf16x2(bf16lo(A[i][3]) * w1[2], bf16hi(A[i][3]) * w1[3]);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const u32x4 B = tr_frag<C, D>(vn, 32 * ks * Cf::ROWB, lane_tr, xtr, sdv + j);
#pragma unroll
      for (int i = 0; i < NI; ++i) Sacc[NJ * i + j] = mfma16x16x32(A[i], B, Sacc[NJ * i + j]);
    }
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
  // the tables (gamma_q | gamma_k, theta_i / 2pi in fp64 and fp32) as one
  // block of TAB bytes; the helpers below take a pointer to its start
  static constexpr uint32_t TAB = LDS - GAM, TRV_R = TRV - GAM, TRF_R = TRF - GAM;
};

// xr: buffer resource over one head's [N, D] rows (REV: row N-1-t holds token t)
template <int C, int D, bool REV = false>
__device__ __forceinline__ void load_rows_f(__amdgpu_buffer_rsrc_t xr, int tid, int c0, int t_end,
                                            u32x4 (&x)[LinF<C, D>::NSF][2], int N = 0) {
  using F = LinF<C, D>;
  const uint32_t hc = tid % F::HC;
#pragma unroll
  for (int u = 0; u < F::NSF; ++u) {
    uint32_t t = min(c0 + tid / F::HC + F::RPF * u, t_end - 1);
    if constexpr (REV) t = (uint32_t)(N - 1) - t;
    x[u][0] = bload16_nt(xr, (t * D + 8 * hc) * 2u);
    x[u][1] = bload16_nt(xr, (t * D + D / 2 + 8 * hc) * 2u);
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
__device__ __forceinline__ void nb_tables(char *tab, int tid, const NbK &nb) {
  using F = LinF<C, D>;
  float *gam = reinterpret_cast<float *>(tab);
  if (tid < D) gam[tid] = nb.gq ? nb.gq[tid] : 1.f;
  else if (tid < 2 * D) gam[tid] = nb.gk ? nb.gk[tid - D] : 1.f;
  if (tid < D / 2 && nb.rope_base > 0.f) {
    const double t = pow((double)nb.rope_base, -2.0 * tid / D) * 0.15915494309189535;  // / 2pi
    reinterpret_cast<double *>(tab + F::TRV_R)[tid] = t;
    reinterpret_cast<float *>(tab + F::TRF_R)[tid] = (float)t;
  }
}
// Fraction of a turn of p0 * theta_i / 2pi for this thread's features (fp64).
template <int C, int D>
__device__ __forceinline__ void rope_base_turns(const char *tab, int hc, long long p0, float (&b)[8]) {
  using F = LinF<C, D>;
  const double *trv = reinterpret_cast<const double *>(tab + F::TRV_R);
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
__device__ __forceinline__ void rope_cs(const char *tab, int hc, int row, const float (&b)[8], float (&c)[8],
                                        float (&sn)[8]) {
  const float *trf = reinterpret_cast<const float *>(tab + LinF<C, D>::TRF_R);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float turns = fmaf((float)row, trf[8 * hc + e], b[e]);
    c[e] = __builtin_amdgcn_cosf(turns);
    sn[e] = __builtin_amdgcn_sinf(turns);
  }
}
template <int C, int D>
__device__ __forceinline__ void nb_row(const char *tab, int hc, bool norm, int which, float eps, bool rope,
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
    const char *gam = tab + which * D * 4;
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
// A key s enters its segment's aggregate with weight lam^(t_end-1-s).  Keys
// whose weight is below 2^-126 (fp32's smallest normal number) are left out:
// their terms lie below fp32's range relative to the inputs, where the
// weights themselves flush to zero a few steps later.  For a fast-decaying
// head this skips all but the segment's last few chunks.  Returns the first
// chunk start to process (always a chunk boundary of the segment).
__device__ __forceinline__ int agg_first_row(float lam, int t_begin, int t_end, int C) {
  const float a = fabsf(lam);
  if (!(a < 1.f)) return t_begin;  // |lam| >= 1 (or NaN): every key counts
  const double keep = a == 0.f ? 1.0 : ceil(126.0 / -log2((double)a)) + 1.0;
  if (keep >= (double)(t_end - t_begin)) return t_begin;
  return t_begin + ((t_end - t_begin - (int)keep) / C) * C;
}

// F: k is normalised and rotated as it is staged (the fused form).
// Part p of segment seg (parts of part_len tokens, whole chunks):
// A_{seg,p} = sum over the part's keys of lam^(part end-1-s) k_s v_s^T, from the
// first key that reaches the segment's end (agg_first_row over the whole
// segment); a part wholly before it is left out (and skipped by the scan,
// which applies the same test).  Persistent, one workgroup per CU: each
// workgroup first lists the parts that are not left out (a prefix count per
// (b, h, segment), b and h from the last, whose slow decay keeps the most
// parts) and then takes every gridDim.x-th entry of that dense list, so the
// work spreads evenly whichever parts the decays leave out.
constexpr int AGG_MAX_PAIRS = 4096;  // (b, h, segment) pairs one list can hold
template <int C, int D, bool F, bool REV>
__global__ __launch_bounds__(512) void lin_seg_aggregate(const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v,
                                                         const float *__restrict__ decay,
                                                         float *__restrict__ seg_state, int H, int N, int BH,
                                                         int seg_len, int nseg, int part_len, int nparts, NbK nb) {
  using Cf = LinCfg<C, D>;
  using Fz = LinF<C, D>;
  __shared__ __attribute__((aligned(16))) char lds[F ? Fz::LDS : Cf::LDS];
  __shared__ int pre[AGG_MAX_PAIRS + 1];  // pre[j]: parts kept by the pairs before j
  __shared__ int wtot[8];
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int nsa = nseg - 1, npairs = BH * nsa;  // the host keeps npairs <= AGG_MAX_PAIRS
  // pair j = (bh, seg): bh = BH - 1 - j / nsa, seg = j % nsa
  auto first_part = [&](int j) {
    const int bh = BH - 1 - j / nsa, seg = j % nsa;
    const float lam = decay ? decay[bh % H] : 1.f;
    const int first = agg_first_row(lam, seg * seg_len, (seg + 1) * seg_len, C);
    return (first - seg * seg_len) / part_len;  // parts before it are left out
  };
  {
    int cnt[8], sum = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 8 * tid + e;
      cnt[e] = j < npairs ? nparts - first_part(j) : 0;
      sum += cnt[e];
    }
    int incl = sum;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (l >= o) incl += y;
    }
    if (l == 63) wtot[w] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int u = 0; u < w; ++u) run += wtot[u];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 8 * tid + e;
      if (j <= npairs) pre[j] = run;
      run += cnt[e];
    }
    __syncthreads();
  }
  const int total = pre[npairs];
  float *pw = reinterpret_cast<float *>(lds + Cf::PW) + Cf::PWZ;  // pw[n] = lam^n, 0 for n < 0
  float *rw = reinterpret_cast<float *>(lds + Cf::RW);
  const int sdk = (w * Cf::SDV) / Cf::ND, sdv0 = (w * Cf::SDV) % Cf::ND;
  const uint32_t lane_tr = tr_lane_off(l, Cf::ROWB), xtr = tr_lane_xor(l);
  if constexpr (F) nb_tables<C, D>(lds + Fz::GAM, tid, nb);
  int h_tab = -1;  // head whose lam^n is in pw
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int lo = 0, hi = npairs - 1;  // the pair j with pre[j] <= item < pre[j + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    const int j = __builtin_amdgcn_readfirstlane(lo);  // uniform: read from LDS, the same in every lane
    const int bh = BH - 1 - j / nsa, seg = j % nsa;
    const int part = __builtin_amdgcn_readfirstlane(nparts - (pre[j + 1] - pre[j]) + (item - pre[j]));
    const int h = bh % H;
    const float lam = decay ? decay[h] : 1.f;
    const int seg_end = (seg + 1) * seg_len;
    const int first = agg_first_row(lam, seg * seg_len, seg_end, C);
    const int p_begin = seg * seg_len + part * part_len, t_end = min(seg_end, p_begin + part_len);
    const int t_begin = max(p_begin, first);
    __syncthreads();  // the previous part's readers of the tables and tiles are done
    if (h != h_tab) {
      for (int n = tid - Cf::PWZ; n <= C; n += Cf::NT) pw[n] = n < 0 ? 0.f : (float)pow((double)lam, (double)n);
      h_tab = h;
    }
    const uint16_t *kb = k + (size_t)bh * N * D;
    const uint16_t *vb = v + (size_t)bh * N * D;
    f32x4 Sacc[Cf::SDV];
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a) Sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (F) {
      const bool norm = nb.gk != nullptr, rope = nb.rope_base > 0.f;
      const int hc = tid % Fz::HC;
      const auto kr = buf_rsrc(kb, (uint32_t)N * D * 2u), vr = buf_rsrc(vb, (uint32_t)N * D * 2u);
      u32x4 xk[Fz::NSF][2], xv[Fz::NSF][2];
      load_rows_f<C, D, REV>(kr, tid, t_begin, t_end, xk, N);
      load_rows_f<C, D, REV>(vr, tid, t_begin, t_end, xv, N);
      for (int c0 = t_begin; c0 < t_end; c0 += C) {
        const int m = min(C, t_end - c0);
        __syncthreads();
        float bt[8], cs[8], sn[8];
        if (rope) rope_base_turns<C, D>(lds + Fz::GAM, hc, nb.pos0 + c0, bt);
#pragma unroll
        for (int u = 0; u < Fz::NSF; ++u) {
          const int row = tid / Fz::HC + Fz::RPF * u;
          if (rope) rope_cs<C, D>(lds + Fz::GAM, hc, row, bt, cs, sn);
          nb_row<C, D>(lds + Fz::GAM, hc, norm, 1, nb.eps, rope, cs, sn, xk[u][0], xk[u][1]);
          __builtin_amdgcn_sched_barrier(0);  // one row's temporaries live at a time
        }
        store_rows_f<C, D>(lds + Cf::KN, tid, m, xk);
        store_rows_f<C, D>(lds + Cf::VN, tid, m, xv);
        if (tid < C) rw[tid] = (tid < m) ? pw[m - 1 - tid] : 0.f;
        __syncthreads();
        if (c0 + C < t_end) {
          load_rows_f<C, D, REV>(kr, tid, c0 + C, t_end, xk, N);
          load_rows_f<C, D, REV>(vr, tid, c0 + C, t_end, xv, N);
        }
        state_update<C, D>(lds, sdk, sdv0, g, lane_tr, xtr, pw[m], Sacc);
      }
    } else {
      u32x4 xk[Cf::NSTG], xv[Cf::NSTG];
      load_kv<C, D, REV>(kb, vb, tid, t_begin, t_end, N, xk, xv);
      for (int c0 = t_begin; c0 < t_end; c0 += C) {
        const int m = min(C, t_end - c0);
        __syncthreads();
        store_kv<C, D>(lds, tid, m, xk, xv);
        if (tid < C) rw[tid] = (tid < m) ? pw[m - 1 - tid] : 0.f;
        __syncthreads();
        if (c0 + C < t_end) load_kv<C, D, REV>(kb, vb, tid, c0 + C, t_end, N, xk, xv);
        state_update<C, D>(lds, sdk, sdv0, g, lane_tr, xtr, pw[m], Sacc);
      }
    }
    float *out = seg_state + (((size_t)bh * nseg + seg) * nparts + part) * D * D;
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[(size_t)(16 * sdk + 4 * g + i) * D + 16 * (sdv0 + a) + lr] = Sacc[a][i];
  }
}

// ---------------------------------------------------------------- pass 2
// seg_state[bh][m][p] holds A_{m,p} for m < nseg-1 on entry (parts the
// aggregate pass left out are not read), and seg_state[bh][m][0] holds
// S_in(m) for every m on exit.  A_m = sum_p lam^(end of m - end of p) A_{m,p}.
// dir.state_T: state_in is read transposed; dir.lag: the initial state's first
// transition decays by lam^(seg_len-1) (it enters one step late).
// C: the chunk the aggregate pass rounds its first key to (agg_first_row).
__global__ __launch_bounds__(256) void lin_seg_scan(float *__restrict__ seg_state,
                                                    const float *__restrict__ state_in,
                                                    const float *__restrict__ decay, int H, int D, int DD,
                                                    int N, int seg_len, int nseg, int part_len, int nparts, int C,
                                                    LinDir dir) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= DD) return;
  const int h = bh % H;
  const float lam_f = decay ? decay[h] : 1.f;
  const double lam = (double)lam_f;
  const float lam_seg = (float)pow(lam, (double)seg_len);
  const float lam_first = dir.lag ? (float)pow(lam, (double)(seg_len - 1)) : lam_seg;
  const int e_in = dir.state_T ? (e % D) * D + e / D : e;
  float s = state_in ? state_in[(size_t)bh * DD + e_in] : 0.f;
  float *base = seg_state + (size_t)bh * nseg * nparts * DD + e;
  // every aggregated segment is whole (it ends before the last one), so its
  // parts' weights are the same for every m: walking back from the segment
  // end, lam^0 for the last part (len_last tokens), then lam^len_last,
  // lam^(len_last + part_len), ...
  const int len_last = seg_len - (nparts - 1) * part_len;
  const double lam_last = pow(lam, (double)len_last), lam_part = pow(lam, (double)part_len);
  for (int m = 0; m < nseg; ++m) {
    float a = 0.f;
    if (m + 1 < nseg) {
      // parts before p_first were left out by the aggregate pass (its test)
      const int seg_end = (m + 1) * seg_len, first = agg_first_row(lam_f, m * seg_len, seg_end, C);
      const int p_first = (first - m * seg_len) / part_len;
      double wgt = 1.0;
      // eight parts' loads in flight at once, summed in the same order
      for (int p0 = nparts - 1; p0 >= p_first; p0 -= 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p0 - u >= p_first ? base[((size_t)m * nparts + p0 - u) * DD] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int p = p0 - u;
          if (p < p_first) break;
          a = fmaf((float)wgt, v[u], a);
          wgt *= (p == nparts - 1) ? lam_last : lam_part;
        }
      }
    }
    base[(size_t)m * nparts * DD] = s;
    s = fmaf(m == 0 ? lam_first : lam_seg, s, a);
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
// REV, dir: the backward passes' switches (LinDir); sin_T: seg_state is the
// caller's initial state, to be read transposed (one segment with dir.state_T).
template <int C, int D, bool REV>
__global__ __launch_bounds__(512) void lin_seg_output(const uint16_t *__restrict__ q,
                                                      const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v,
                                                      uint16_t *__restrict__ o,
                                                      const float *__restrict__ decay,
                                                      const float *__restrict__ seg_state,
                                                      size_t seg_stride, float *__restrict__ state_out,
                                                      int H, int N, int seg_len, int nseg, NbK nb, LinDir dir,
                                                      int sin_T) {
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
    for (int i = 0; i < 4; ++i) {
      const size_t r = 16 * sdk + 4 * g + i, c = 16 * (sdv0 + a) + lr;
      Sacc[a][i] = sin ? sin[sin_T ? c * D + r : r * D + c] : 0.f;
    }
  // the initial state enters one decay step late (backward passes): in this
  // segment's first chunk it is weighted lam^qq and decays by lam^(m-1)
  bool lag_chunk = dir.lag && seg == 0;

  // Q fragment s (B operand of Q^T, query tile qt): read from the staged Q
  // rows in LDS at each use
  const int qq = 16 * qt + lr;  // this lane's query row in the chunk
  auto qfrag = [&](int s) -> u32x4 {
    return lds_load<u32x4>(lds + Fz::QN, qq * Cf::ROWB + (((4 * s + g) ^ fkv(qq)) & (Cf::NCH - 1)) * 16u);
  };
  // this lane's output row, gated by gv when given; 16-byte stores of eight
  // consecutive d_v values (a row's four lanes cover 64 contiguous bytes per
  // store instead of 32 with one 8-byte store per d_v tile)
  auto store_out = [&](int c0, int m, const f32x4 (&Oacc)[Cf::DVW], const u32x2 (&gv)[Cf::DVW], bool gated) {
    if (qq < m) {
      uint16_t *orow = ob + (size_t)(REV ? N - 1 - (c0 + qq) : c0 + qq) * D;
      u32x2 ov[Cf::DVW];
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        f32x4 x = Oacc[dvi];
        if (gated) {
          x[0] *= sigmoid_fast(bf16lo(gv[dvi][0]));
          x[1] *= sigmoid_fast(bf16hi(gv[dvi][0]));
          x[2] *= sigmoid_fast(bf16lo(gv[dvi][1]));
          x[3] *= sigmoid_fast(bf16hi(gv[dvi][1]));
        }
        ov[dvi] = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      }
      // lanes l and l ^ 16 (g and g ^ 1) swap halves so that each holds eight
      // consecutive d_v values: g even tile dvi, g odd tile dvi + 1 (the two
      // lanes share qq, so both take this branch or neither does)
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; dvi += 2) {
        u32x2 a = ov[dvi], b = ov[dvi + 1];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const auto sw = __builtin_amdgcn_permlane16_swap(a[e], b[e], false, false);
          a[e] = sw[0];
          b[e] = sw[1];
        }
        const int tile = dvb + dvi + (g & 1);
        gstore16_nt(orow + 16 * tile + 8 * (g >> 1), u32x4{a[0], a[1], b[0], b[1]});
      }
    }
  };

  // next chunk's 16-byte staging pieces (rows x halves)
  u32x4 xk[Fz::NSF][2], xv[Fz::NSF][2], xq[Fz::NSF][2];
  const int hc = tid % Fz::HC;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto qr = buf_rsrc(qb, head_bytes), kr = buf_rsrc(kb, head_bytes), vr = buf_rsrc(vb, head_bytes);
  const auto gr = buf_rsrc(nb.gate ? nb.gate + head_off : qb, head_bytes);
  nb_tables<C, D>(lds + Fz::GAM, tid, nb);
  const bool norm_q = nb.gq != nullptr, norm_k = nb.gk != nullptr, rope = nb.rope_base > 0.f;
  load_rows_f<C, D, REV>(kr, tid, t_begin, t_end, xk, N);
  load_rows_f<C, D, REV>(vr, tid, t_begin, t_end, xv, N);
  load_rows_f<C, D, REV>(qr, tid, t_begin, t_end, xq, N);

  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    const int m = min(C, t_end - c0);
    __syncthreads();
    {
      float bt[8], cs[8], sn[8];
      if (rope) rope_base_turns<C, D>(lds + Fz::GAM, hc, nb.pos0 + c0, bt);
#pragma unroll
      for (int u = 0; u < Fz::NSF; ++u) {
        const int row = tid / Fz::HC + Fz::RPF * u;
        if (rope) rope_cs<C, D>(lds + Fz::GAM, hc, row, bt, cs, sn);
        nb_row<C, D>(lds + Fz::GAM, hc, norm_q, 0, nb.eps, rope, cs, sn, xq[u][0], xq[u][1]);
        nb_row<C, D>(lds + Fz::GAM, hc, norm_k, 1, nb.eps, rope, cs, sn, xk[u][0], xk[u][1]);
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
      load_rows_f<C, D, REV>(kr, tid, c0 + C, t_end, xk, N);
      load_rows_f<C, D, REV>(vr, tid, c0 + C, t_end, xv, N);
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
      const float f = pw[lag_chunk ? qq : qq + 1];
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
      uint32_t t = min(c0 + qq, t_end - 1);
      if constexpr (REV) t = (uint32_t)(N - 1) - t;
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) gv[dvi] = bload8(gr, (t * D + 16 * (dvb + dvi) + 4 * g) * 2u);
    }
    if (c0 + C < t_end) load_rows_f<C, D, REV>(qr, tid, c0 + C, t_end, xq, N);
    // (5) S = lam^m S + (diag(lam^(m-1-j)) K)^T V, then (4) the (gated) output row
    state_update<C, D>(lds, sdk, sdv0, g, lane_tr, xtr, pw[lag_chunk ? m - 1 : m], Sacc);
    store_out(c0, m, Oacc, gv, nb.gate != nullptr);
    lag_chunk = false;
  }

  if (state_out && seg == nseg - 1) {
    float *so = state_out + (size_t)bh * D * D;
    const float f = dir.scale ? lam : 1.f;
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(size_t)(16 * sdk + 4 * g + i) * D + 16 * (sdv0 + a) + lr] = Sacc[a][i] * f;
  }
}

// Pass 3 with direct loads (no q / k transform to apply): each chunk's k, v
// and q rows go from HBM straight into LDS (buffer loads with an LDS
// destination, 16 bytes per lane), into one of two buffers, so the next
// chunk's rows are in flight while this one is computed and no registers or
// LDS stores stage them.  The two buffers hold 3 C rows each (k | v | q), so
// this form runs with C = 64 at d = 128 (128 KB of LDS with the bf16 S^T).
// The arithmetic per chunk is that of lin_seg_output, except that each wave
// updates a 2 x 4 block of state tiles (d = 128).  Rows past a chunk's valid
// rows read as zero (the buffer resources cover the valid rows only).
template <int C, int D>
struct LinDma {
  using Cf = LinCfg<C, D>;
  static constexpr uint32_t TILE = C * Cf::ROWB;      // one [C][D] bf16 tile
  static constexpr int SLOTS = C * Cf::NCH / Cf::NT;  // 16-byte slots per thread and tile
  static constexpr int NST = Cf::DVW / 2;             // 16-byte output stores per thread and chunk
  static_assert(SLOTS >= 1 && C * Cf::NCH % Cf::NT == 0, "unsupported chunk / head size");
};
// the two chunk buffers, S^T and the decay tables fit the 160 KB of LDS
template <int C, int D>
constexpr bool dma_fits() {
  return 2 * 3 * C * D * 2 + D * D * 2 <= 156 * 1024;
}

// Workgroup barrier after this wave's LDS operations and all but its last VM
// vector memory operations are done.  __syncthreads would also wait for every
// direct load still in flight (its fence counts them as LDS writes); here the
// caller names what must have landed.  The signal fences keep the compiler
// from moving LDS accesses across.
template <int VM>
__device__ __forceinline__ void lds_barrier() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0070);  // vmcnt(VM) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// GATE: the output is gated (a compile-time switch: the gate loads' registers
// would otherwise be waited on before every reuse in the ungated form).
// NBT: q and k are normalised and rotated (NbK) once their rows have landed,
// in place in LDS, each thread taking the two 16-byte pieces of a row that
// hold rotate-half partners (as the staged form does in registers).
template <int C, int D, bool REV, bool GATE, bool NBT>
__global__ __launch_bounds__(512) void lin_seg_output_dma(const uint16_t *__restrict__ q,
                                                          const uint16_t *__restrict__ k,
                                                          const uint16_t *__restrict__ v,
                                                          uint16_t *__restrict__ o,
                                                          const float *__restrict__ decay,
                                                          const float *__restrict__ seg_state, size_t seg_stride,
                                                          float *__restrict__ state_out, int H, int N, int seg_len,
                                                          int nseg, NbK nb, LinDir dir, int sin_T) {
  using Cf = LinCfg<C, D>;
  using Dm = LinDma<C, D>;
  using Fz = LinF<C, D>;
  const uint16_t *gate = nb.gate;
  // two chunk buffers (k | v | q) and the S^T copy: separate arrays, so the
  // compiler sees that direct loads into one buffer do not touch the others
  __shared__ __attribute__((aligned(16))) char buf0[3 * Dm::TILE], buf1[3 * Dm::TILE];
  __shared__ __attribute__((aligned(16))) char stl[D * Cf::ROWB];
  __shared__ __attribute__((aligned(16))) float tab[Cf::PWZ + C + 4 + C];
  __shared__ __attribute__((aligned(16))) char nbt[NBT ? Fz::TAB : 16];  // norm weights, RoPE frequencies
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const int h = bh % H;
  const int t_begin = seg * seg_len, t_end = min(N, t_begin + seg_len);
  const float lam = decay ? decay[h] : 1.f;
  float *pw = tab + Cf::PWZ;          // pw[n] = lam^n, 0 for n < 0
  float *rw = tab + Cf::PWZ + C + 4;  // lam^(m-1-j) for the chunk's rows, 0 past m
  for (int n = tid - Cf::PWZ; n <= C; n += Cf::NT) pw[n] = n < 0 ? 0.f : (float)pow((double)lam, (double)n);
  if constexpr (NBT) nb_tables<C, D>(nbt, tid, nb);  // read after the first chunk barrier
  const size_t head_off = (size_t)bh * N * D;
  const uint16_t *qb = q + head_off, *kb = k + head_off, *vb = v + head_off;
  uint16_t *ob = o + head_off;
  int qt, part;
  Cf::qrole(w, qt, part);
  const int dvb = part * Cf::DVW;
  const int qq = 16 * qt + lr;  // this lane's query row in the chunk
  // state tiles: an NI x NJ block, d_k tiles sdk .. and d_v tiles sdv ..
  constexpr int NI = Cf::ND == 8 ? 2 : 1, NJ = Cf::SDV / NI, BI = Cf::ND / NI;
  const int sdk = NI * (w % BI), sdv = NJ * (w / BI);
  const uint32_t lane_tr = tr_lane_off(l, Cf::ROWB), xtr = tr_lane_xor(l);

  f32x4 Sacc[Cf::SDV];
  const float *sin = seg_state ? seg_state + (size_t)bh * seg_stride * nseg + (size_t)seg * seg_stride : nullptr;
#pragma unroll
  for (int a = 0; a < Cf::SDV; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t r = 16 * (sdk + a / NJ) + 4 * g + i, c = 16 * (sdv + a % NJ) + lr;
      Sacc[a][i] = sin ? sin[sin_T ? c * D + r : r * D + c] : 0.f;
    }
  bool lag_chunk = dir.lag && seg == 0;

  // Direct loads: the LDS slot of lane l in wave w for slot step u is
  // p = 512u + 64w + l of a tile (16 bytes each); it holds chunk row p / NCH at
  // swizzled position p % NCH, i.e. the logical 16-byte piece
  // (p % NCH) ^ f(row) of that row (the swizzles are involutions): f = fkv for
  // k and v, fst for q, whose fragments are 16 consecutive rows at one piece.
  uint32_t srow[Dm::SLOTS], spiece[Dm::SLOTS], spq[Dm::SLOTS];
#pragma unroll
  for (int u = 0; u < Dm::SLOTS; ++u) {
    const uint32_t p = Cf::NT * u + tid, row = p / Cf::NCH;
    srow[u] = row;
    spiece[u] = (((p % Cf::NCH) ^ fkv(row)) & (Cf::NCH - 1)) * 16u;
    spq[u] = (((p % Cf::NCH) ^ fst(row)) & (Cf::NCH - 1)) * 16u;
  }
  // Chunk rows c0 .. c0 + m - 1 (m = 0 past the segment: every load reads
  // zero).  REV: chunk row r is memory row N - 1 - (c0 + r); the resource
  // starts at memory row N - c0 - m, so rows r >= m fall past its end.
  auto chunk_rows = [&](int c0) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(max(0, min(C, t_end - c0)));  // uniform: the resources stay scalar
  };
  auto rows_rsrc = [&](const uint16_t *base, int c0, int m) __attribute__((always_inline)) {
    return buf_rsrc(base + (REV ? (size_t)(N - c0 - m) : (size_t)c0) * D, (uint32_t)m * Cf::ROWB);
  };
  // k, v and q rows of chunk c0 into buffer dst (k | v | q)
  auto load_chunk = [&](char *dst, int c0) __attribute__((always_inline)) {
    const int m = chunk_rows(c0);
    const auto kr = rows_rsrc(kb, c0, m), vr = rows_rsrc(vb, c0, m), qr = rows_rsrc(qb, c0, m);
#pragma unroll
    for (int u = 0; u < Dm::SLOTS; ++u) {
      const uint32_t r = REV ? (uint32_t)(m - 1) - srow[u] : srow[u];
      const uint32_t slot = (Cf::NT * u + 64 * w) * 16;
      bload16_lds_nt(kr, dst + slot, r * Cf::ROWB + spiece[u]);
      bload16_lds_nt(vr, dst + Dm::TILE + slot, r * Cf::ROWB + spiece[u]);
      bload16_lds_nt(qr, dst + 2 * Dm::TILE + slot, r * Cf::ROWB + spq[u]);
    }
  };
  const auto gr = buf_rsrc(GATE ? gate + head_off : qb, (uint32_t)N * D * 2u);

  // One chunk: cur holds its rows (landed by the barrier below); the rows of
  // chunk c0 + C go to nxt.
  auto step = [&](char *cur, char *nxt, int c0) __attribute__((always_inline)) {
    const int m = min(C, t_end - c0);
    // this wave's direct loads of the chunk have landed (only the previous
    // chunk's output stores, issued after them, may be outstanding); after
    // the barrier every wave's rows are in and the previous chunk is done
    // with nxt, S^T and rw
    lds_barrier<Dm::NST>();
    if constexpr (NBT) {
      // q and k rows of the chunk, normalised and rotated in place (rows past
      // the segment's end are zero and stay zero)
      const bool norm_q = nb.gq != nullptr, norm_k = nb.gk != nullptr, rope = nb.rope_base > 0.f;
      const int hc = tid % Fz::HC;
      float bt[8], cs[8], sn[8];
      if (rope) rope_base_turns<C, D>(nbt, hc, nb.pos0 + c0, bt);
#pragma unroll
      for (int u = 0; u < Fz::NSF; ++u) {
        const int row = tid / Fz::HC + Fz::RPF * u;
        if (Fz::RPF * Fz::NSF > C && row >= C) continue;
        if (rope) rope_cs<C, D>(nbt, hc, row, bt, cs, sn);
        char *qrow = cur + 2 * Dm::TILE + row * Cf::ROWB;
        char *krow = cur + row * Cf::ROWB;
        const uint32_t q0 = ((hc ^ fst(row)) & (Cf::NCH - 1)) * 16u, q1 = (((hc + Fz::HC) ^ fst(row)) & (Cf::NCH - 1)) * 16u;
        const uint32_t k0 = ((hc ^ fkv(row)) & (Cf::NCH - 1)) * 16u, k1 = (((hc + Fz::HC) ^ fkv(row)) & (Cf::NCH - 1)) * 16u;
        u32x4 ql = lds_load<u32x4>(qrow, q0), qh = lds_load<u32x4>(qrow, q1);
        u32x4 kl = lds_load<u32x4>(krow, k0), kh = lds_load<u32x4>(krow, k1);
        nb_row<C, D>(nbt, hc, norm_q, 0, nb.eps, rope, cs, sn, ql, qh);
        nb_row<C, D>(nbt, hc, norm_k, 1, nb.eps, rope, cs, sn, kl, kh);
        lds_store(qrow, q0, ql);
        lds_store(qrow, q1, qh);
        lds_store(krow, k0, kl);
        lds_store(krow, k1, kh);
      }
    }
    // gate values of this lane's outputs (a clamped row is never stored),
    // loaded before the next chunk's rows so that waiting for them waits for
    // nothing issued later
    u32x2 gv[Cf::DVW] = {};
    if constexpr (GATE) {
      uint32_t t = min(c0 + qq, t_end - 1);
      if constexpr (REV) t = (uint32_t)(N - 1) - t;
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) gv[dvi] = bload8(gr, (t * D + 16 * (dvb + dvi) + 4 * g) * 2u);
    }
    // bf16 S^T in 16-byte stores: of the tiles (sdk, j) and (sdk + 1, j), a
    // lane holds four d_k values of one d_v column in each; lanes 16 apart
    // swap halves so that each holds eight consecutive d_k values of one of
    // them (g even: tile sdk, g odd: tile sdk + 1).  S^T and rw are written
    // before the next chunk's loads are issued: a store that the compiler
    // cannot tell apart from a direct load in flight waits for that load, and
    // it loses that information when it pairs 8-byte stores.
    if constexpr (NI == 2) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const f32x4 &sa = Sacc[j], &sb = Sacc[NJ + j];
        uint32_t x[2] = {pack_bf16x2(sa[0], sa[1]), pack_bf16x2(sa[2], sa[3])};
        uint32_t y[2] = {pack_bf16x2(sb[0], sb[1]), pack_bf16x2(sb[2], sb[3])};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const auto sw = __builtin_amdgcn_permlane16_swap(x[e], y[e], false, false);
          x[e] = sw[0];
          y[e] = sw[1];
        }
        const uint32_t row = 16 * (sdv + j) + lr;
        const uint32_t ch = 2 * (sdk + (g & 1)) + (g >> 1);
        lds_store(stl, row * Cf::ROWB + ((ch ^ fst(row)) & (Cf::NCH - 1)) * 16u, u32x4{x[0], x[1], y[0], y[1]});
      }
    } else {  // one d_k tile per wave: 8-byte stores
#pragma unroll
      for (int a = 0; a < Cf::SDV; ++a) {
        const uint32_t row = 16 * (sdv + a % NJ) + lr;
        const uint32_t off =
            row * Cf::ROWB + (((2 * (sdk + a / NJ) + (g >> 1)) ^ fst(row)) & (Cf::NCH - 1)) * 16u + (g & 1) * 8;
        lds_store(stl, off, u32x2{pack_bf16x2(Sacc[a][0], Sacc[a][1]), pack_bf16x2(Sacc[a][2], Sacc[a][3])});
      }
    }
    if (tid < C) rw[tid] = (tid < m) ? pw[m - 1 - tid] : 0.f;
    load_chunk(nxt, c0 + C);  // past the segment: zeros
    lds_barrier<63>();  // S^T and rw written; the next chunk's loads stay in flight
    const char *kc = cur, *vc = cur + Dm::TILE, *qn = cur + 2 * Dm::TILE;
    u32x4 qf[Cf::NDS];
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s)
      qf[s] = lds_load<u32x4>(qn, qq * Cf::ROWB + (((4 * s + g) ^ fst(qq)) & (Cf::NCH - 1)) * 16u);
    // O^T = lam^(qq+1) S^T Q^T
    f32x4 Oacc[Cf::DVW];
#pragma unroll
    for (int dvi = 0; dvi < Cf::DVW; ++dvi) Oacc[dvi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s) {
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        const uint32_t row = 16 * (dvb + dvi) + lr;
        const u32x4 A = lds_load<u32x4>(stl, row * Cf::ROWB + (((4 * s + g) ^ fst(row)) & (Cf::NCH - 1)) * 16u);
        Oacc[dvi] = mfma16x16x32(A, qf[s], Oacc[dvi]);
      }
    }
    {
      const float f = pw[lag_chunk ? qq : qq + 1];
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) Oacc[dvi] *= f;
    }
    // P^T = decay-masked K Q^T over the causal key pairs; O^T += V^T P^T
#pragma unroll
    for (int p = 0; p < (Cf::NQT + 1) / 2; ++p) {
      if (p > qt / 2) break;
      f32x4 P[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < Cf::NDS; ++s) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t row = 32 * p + pair_key(t, lr);
          const u32x4 A = lds_load<u32x4>(kc, row * Cf::ROWB + (((4 * s + g) ^ fkv(row)) & (Cf::NCH - 1)) * 16u);
          P[t] = mfma16x16x32(A, qf[s], P[t]);
        }
      }
      const int nb0 = qq - 32 * p - 8 * g;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) P[t][i] *= pw[nb0 - 4 * t - i];
      const u32x4 Bp = u32x4{pack_bf16x2(P[0][0], P[0][1]), pack_bf16x2(P[0][2], P[0][3]),
                             pack_bf16x2(P[1][0], P[1][1]), pack_bf16x2(P[1][2], P[1][3])};
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        const u32x4 A = tr_frag<C, D>(vc, 32 * p * Cf::ROWB, lane_tr, xtr, dvb + dvi);
        Oacc[dvi] = mfma16x16x32(A, Bp, Oacc[dvi]);
      }
    }
    state_update_blk<C, D, NI, NJ>(kc, vc, reinterpret_cast<const char *>(rw), sdk, sdv, g, lane_tr, xtr,
                                   pw[lag_chunk ? m - 1 : m], Sacc);
    // output row qq: 16-byte stores of eight consecutive d_v values (lanes 16
    // apart swap halves), as in lin_seg_output.  Buffer stores over the
    // chunk's valid rows: rows past m are dropped by the range check, so
    // every wave issues the same NST stores in every chunk, which the vmcnt
    // of the barriers counts on.
    {
      const auto orr = rows_rsrc(ob, c0, chunk_rows(c0));
      const uint32_t orow = (REV ? (uint32_t)(m - 1 - qq) : (uint32_t)qq) * Cf::ROWB;
      u32x2 ov[Cf::DVW];
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        f32x4 x = Oacc[dvi];
        if constexpr (GATE) {
          x[0] *= sigmoid_fast(bf16lo(gv[dvi][0]));
          x[1] *= sigmoid_fast(bf16hi(gv[dvi][0]));
          x[2] *= sigmoid_fast(bf16lo(gv[dvi][1]));
          x[3] *= sigmoid_fast(bf16hi(gv[dvi][1]));
        }
        ov[dvi] = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      }
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; dvi += 2) {
        u32x2 a = ov[dvi], b = ov[dvi + 1];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const auto sw = __builtin_amdgcn_permlane16_swap(a[e], b[e], false, false);
          a[e] = sw[0];
          b[e] = sw[1];
        }
        const int tile = dvb + dvi + (g & 1);
        bstore16_nt(orr, orow + (16 * tile + 8 * (g >> 1)) * 2u, u32x4{a[0], a[1], b[0], b[1]});
      }
    }
    lag_chunk = false;
  };

  load_chunk(buf0, t_begin);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the entry state and the first chunk are in
  for (int c0 = t_begin; c0 < t_end; c0 += 2 * C) {
    step(buf0, buf1, c0);
    if (c0 + C >= t_end) break;
    step(buf1, buf0, c0 + C);
  }
  // the last step's loads of an empty successor write zeros into LDS: let
  // them land before the workgroup's LDS can be handed on
  __builtin_amdgcn_s_waitcnt(0x0F70);

  if (state_out && seg == nseg - 1) {
    float *so = state_out + (size_t)bh * D * D;
    const float f = dir.scale ? lam : 1.f;
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        so[(size_t)(16 * (sdk + a / NJ) + 4 * g + i) * D + 16 * (sdv + a % NJ) + lr] = Sacc[a][i] * f;
  }
}

// The dK and dV passes of the gradients in one reversed pass (direct loads).
// Both are decayed causal linear attention on the time-reversed sequence (see
// the header): dK with query v, key dO and value q, dV with query k, key q
// and value dO, and their states are transposes of each other,
//   S = sum_t (decay) dO_t q_t^T  for dK,   S^T  for dV,
// so one fp32 state S[d_v][d_k] serves both.  Per chunk of C reversed rows:
//   dK^T += lam^(r+1) S^T V^T + Q^T (decay-masked dO V^T)
//   dV^T += lam^(r+1) S   K^T + dO^T (decay-masked Q K^T)
//   S     = lam^C S + (diag(lam^(C-1-j)) dO)^T Q
// (r + 1 -> r and C -> C - 1 in the first chunk of the first segment: the
// initial state enters one step late).  The bf16 copy of S^T in LDS is read
// plainly for dK and transposed for dV.  k, v, q and dO rows go from HBM
// straight into LDS by direct loads, double-buffered (2 x 64 KB at C = 64,
// d = 128, with S^T the whole 160 KB), so the decay powers come from exp2 on
// the VALU rather than LDS tables:
//   lam^n = exp2(n * l2),  l2 = max(log2 lam, -16384)  (lam = 0: 0^0 = 1, 0^n = 0).
// seg_state / sin_T: the segments' entry states of the dK pass (its
// aggregate and scan); state_out receives dS_in = lam S_dV = lam S^T.
template <int C, int D>
constexpr bool gradkv_fits() {
  return 2 * 4 * C * D * 2 + D * D * 2 <= 160 * 1024 && LinCfg<C, D>::ND == 8;
}
template <int C, int D>
__global__ __launch_bounds__(512) void lin_seg_grad_kv(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                       const uint16_t *__restrict__ v,
                                                       const uint16_t *__restrict__ dout, uint16_t *__restrict__ dk,
                                                       uint16_t *__restrict__ dv, const float *__restrict__ decay,
                                                       const float *__restrict__ seg_state, size_t seg_stride,
                                                       float *__restrict__ state_out, int H, int N, int seg_len,
                                                       int nseg, int lag, int sin_T) {
  using Cf = LinCfg<C, D>;
  constexpr uint32_t TILE = C * Cf::ROWB;            // one [C][D] bf16 tile
  constexpr int SLOTS = C * Cf::NCH / Cf::NT;        // 16-byte slots per thread and tile
  constexpr int NST = Cf::DVW;                       // output stores per thread and chunk (dK and dV)
  static_assert(SLOTS >= 1 && C * Cf::NCH % Cf::NT == 0 && gradkv_fits<C, D>(), "unsupported chunk / head size");
  // tiles of a buffer: v (query of dK) | k (query of dV) | dO | q
  constexpr uint32_t TV = 0, TK = TILE, TO = 2 * TILE, TQ = 3 * TILE;
  __shared__ __attribute__((aligned(16))) char buf0[4 * TILE], buf1[4 * TILE];
  __shared__ __attribute__((aligned(16))) char stl[D * Cf::ROWB];  // bf16 S^T, fkv-swizzled
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const int h = bh % H;
  const int t_begin = seg * seg_len, t_end = min(N, t_begin + seg_len);
  const float lam = decay ? decay[h] : 1.f;
  const float l2 = fmaxf(log2f(lam), -16384.f);
  auto lpow = [&](int n) __attribute__((always_inline)) { return __builtin_amdgcn_exp2f((float)n * l2); };
  const size_t head_off = (size_t)bh * N * D;
  int qt, part;
  Cf::qrole(w, qt, part);
  const int dvb = part * Cf::DVW;
  const int qq = 16 * qt + lr;  // this lane's row in the chunk
  constexpr int NI = 2, NJ = Cf::SDV / 2;
  const int sdk = NI * (w % 4), sdv = NJ * (w / 4);  // state tiles: d_v (dO) tiles sdk.., d_k (q) tiles sdv..
  const uint32_t lane_tr = tr_lane_off(l, Cf::ROWB), xtr = tr_lane_xor(l);

  f32x4 Sacc[Cf::SDV];
  const float *sin = seg_state ? seg_state + (size_t)bh * seg_stride * nseg + (size_t)seg * seg_stride : nullptr;
#pragma unroll
  for (int a = 0; a < Cf::SDV; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t r = 16 * (sdk + a / NJ) + 4 * g + i, c = 16 * (sdv + a % NJ) + lr;
      Sacc[a][i] = sin ? sin[sin_T ? c * D + r : r * D + c] : 0.f;
    }
  bool lag_chunk = lag && seg == 0;

  // direct-load slots (as in lin_seg_output_dma): fst for the query tiles (16
  // consecutive rows at one piece), fkv for dO and q (read by key pairs and
  // transposed)
  uint32_t srow[SLOTS], spk[SLOTS], spq[SLOTS];
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const uint32_t p = Cf::NT * u + tid, row = p / Cf::NCH;
    srow[u] = row;
    spk[u] = (((p % Cf::NCH) ^ fkv(row)) & (Cf::NCH - 1)) * 16u;
    spq[u] = (((p % Cf::NCH) ^ fst(row)) & (Cf::NCH - 1)) * 16u;
  }
  // reversed rows: chunk row r is memory row N - 1 - (c0 + r); the resources
  // start at memory row N - c0 - m, so rows r >= m fall past their end
  auto chunk_rows = [&](int c0) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(max(0, min(C, t_end - c0)));
  };
  auto rows_rsrc = [&](const uint16_t *base, int c0, int m) __attribute__((always_inline)) {
    return buf_rsrc(base + head_off + (size_t)(N - c0 - m) * D, (uint32_t)m * Cf::ROWB);
  };
  auto load_chunk = [&](char *dst, int c0) __attribute__((always_inline)) {
    const int m = chunk_rows(c0);
    const auto vr = rows_rsrc(v, c0, m), kr = rows_rsrc(k, c0, m), orr = rows_rsrc(dout, c0, m),
               qr = rows_rsrc(q, c0, m);
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      const uint32_t rb = ((uint32_t)(m - 1) - srow[u]) * Cf::ROWB;
      const uint32_t slot = (Cf::NT * u + 64 * w) * 16;
      bload16_lds_nt(vr, dst + TV + slot, rb + spq[u]);
      bload16_lds_nt(kr, dst + TK + slot, rb + spq[u]);
      bload16_lds_nt(orr, dst + TO + slot, rb + spk[u]);
      bload16_lds_nt(qr, dst + TQ + slot, rb + spk[u]);
    }
  };
  // 16-byte stores of eight consecutive values of output row qq (lanes 16
  // apart swap halves); buffer stores over the chunk's valid rows, issued by
  // every lane in every chunk
  auto store_rows = [&](uint16_t *dst, int c0, int m, const f32x4 (&acc)[Cf::DVW]) __attribute__((always_inline)) {
    const auto orr = rows_rsrc(dst, c0, chunk_rows(c0));
    const uint32_t orow = (uint32_t)(m - 1 - qq) * Cf::ROWB;
    u32x2 ov[Cf::DVW];
#pragma unroll
    for (int dvi = 0; dvi < Cf::DVW; ++dvi)
      ov[dvi] = u32x2{pack_bf16x2(acc[dvi][0], acc[dvi][1]), pack_bf16x2(acc[dvi][2], acc[dvi][3])};
#pragma unroll
    for (int dvi = 0; dvi < Cf::DVW; dvi += 2) {
      u32x2 a = ov[dvi], b = ov[dvi + 1];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto sw = __builtin_amdgcn_permlane16_swap(a[e], b[e], false, false);
        a[e] = sw[0];
        b[e] = sw[1];
      }
      const int tile = dvb + dvi + (g & 1);
      bstore16_nt(orr, orow + (16 * tile + 8 * (g >> 1)) * 2u, u32x4{a[0], a[1], b[0], b[1]});
    }
  };

  auto step = [&](const char *cur, char *nxt, int c0) __attribute__((always_inline)) {
    const int m = min(C, t_end - c0);
    // this wave's direct loads of the chunk have landed (only the previous
    // chunk's output stores may be outstanding); the previous chunk is done
    // with nxt and S^T
    lds_barrier<NST>();
    // bf16 S^T (rows d_k, fkv-swizzled) in 16-byte stores: lanes 16 apart swap
    // halves of the tiles (sdk, j) and (sdk + 1, j), so each holds eight
    // consecutive d_v values of one of them; written before the next chunk's
    // loads are issued (see lin_seg_output_dma)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const f32x4 &sa = Sacc[j], &sb = Sacc[NJ + j];
      uint32_t x[2] = {pack_bf16x2(sa[0], sa[1]), pack_bf16x2(sa[2], sa[3])};
      uint32_t y[2] = {pack_bf16x2(sb[0], sb[1]), pack_bf16x2(sb[2], sb[3])};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto sw = __builtin_amdgcn_permlane16_swap(x[e], y[e], false, false);
        x[e] = sw[0];
        y[e] = sw[1];
      }
      const uint32_t row = 16 * (sdv + j) + lr;
      const uint32_t ch = 2 * (sdk + (g & 1)) + (g >> 1);
      lds_store(stl, row * Cf::ROWB + ((ch ^ fkv(row)) & (Cf::NCH - 1)) * 16u, u32x4{x[0], x[1], y[0], y[1]});
    }
    load_chunk(nxt, c0 + C);  // past the segment: zeros
    lds_barrier<63>();  // S^T written; the next chunk's loads stay in flight
    const char *tv = cur + TV, *tk = cur + TK, *to = cur + TO, *tq = cur + TQ;
    u32x4 fv[Cf::NDS], fk[Cf::NDS];  // query fragments of this lane's row: v (dK), k (dV)
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s) {
      const uint32_t off = qq * Cf::ROWB + (((4 * s + g) ^ fst(qq)) & (Cf::NCH - 1)) * 16u;
      fv[s] = lds_load<u32x4>(tv, off);
      fk[s] = lds_load<u32x4>(tk, off);
    }
    // dK^T = lam^(r+1) S^T V^T (S^T read plainly), dV^T = lam^(r+1) S K^T (S^T read transposed)
    f32x4 OK[Cf::DVW], OV[Cf::DVW];
#pragma unroll
    for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
      OK[dvi] = f32x4{0.f, 0.f, 0.f, 0.f};
      OV[dvi] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s) {
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        const uint32_t row = 16 * (dvb + dvi) + lr;
        const u32x4 A = lds_load<u32x4>(stl, row * Cf::ROWB + (((4 * s + g) ^ fkv(row)) & (Cf::NCH - 1)) * 16u);
        OK[dvi] = mfma16x16x32(A, fv[s], OK[dvi]);
        OV[dvi] = mfma16x16x32(tr_frag<C, D>(stl, 32 * s * Cf::ROWB, lane_tr, xtr, dvb + dvi), fk[s], OV[dvi]);
      }
    }
    {
      const float f = lpow(lag_chunk ? qq : qq + 1);
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        OK[dvi] *= f;
        OV[dvi] *= f;
      }
    }
    // decay-masked scores over the causal key pairs: P_K^T = dO V^T, P_V^T = Q K^T;
    // dK^T += Q^T P_K^T, dV^T += dO^T P_V^T
#pragma unroll
    for (int p = 0; p < (Cf::NQT + 1) / 2; ++p) {
      if (p > qt / 2) break;
      f32x4 PK[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 PV[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < Cf::NDS; ++s) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t row = 32 * p + pair_key(t, lr);
          const uint32_t off = row * Cf::ROWB + (((4 * s + g) ^ fkv(row)) & (Cf::NCH - 1)) * 16u;
          PK[t] = mfma16x16x32(lds_load<u32x4>(to, off), fv[s], PK[t]);
          PV[t] = mfma16x16x32(lds_load<u32x4>(tq, off), fk[s], PV[t]);
        }
      }
      // lam^(qq-j) for key j = 32p + 8g + 4t + i, zero for j > qq
      const int nb0 = qq - 32 * p - 8 * g;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = nb0 - 4 * t - i;
          const float f = n < 0 ? 0.f : lpow(n);
          PK[t][i] *= f;
          PV[t][i] *= f;
        }
      const u32x4 BK = u32x4{pack_bf16x2(PK[0][0], PK[0][1]), pack_bf16x2(PK[0][2], PK[0][3]),
                             pack_bf16x2(PK[1][0], PK[1][1]), pack_bf16x2(PK[1][2], PK[1][3])};
      const u32x4 BV = u32x4{pack_bf16x2(PV[0][0], PV[0][1]), pack_bf16x2(PV[0][2], PV[0][3]),
                             pack_bf16x2(PV[1][0], PV[1][1]), pack_bf16x2(PV[1][2], PV[1][3])};
#pragma unroll
      for (int dvi = 0; dvi < Cf::DVW; ++dvi) {
        OK[dvi] = mfma16x16x32(tr_frag<C, D>(tq, 32 * p * Cf::ROWB, lane_tr, xtr, dvb + dvi), BK, OK[dvi]);
        OV[dvi] = mfma16x16x32(tr_frag<C, D>(to, 32 * p * Cf::ROWB, lane_tr, xtr, dvb + dvi), BV, OV[dvi]);
      }
    }
    // S = lam^m S + (diag(lam^(m-1-j)) dO)^T Q on this wave's 2 x NJ tiles
    // (rows past m are zero, so their clamped weight does not matter)
    {
      const float f = lpow(lag_chunk ? m - 1 : m);
#pragma unroll
      for (int a = 0; a < Cf::SDV; ++a) Sacc[a] *= f;
#pragma unroll
      for (int ks = 0; ks < Cf::NKS; ++ks) {
        float wt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) wt[e] = lpow(max(m - 1 - (32 * ks + 8 * g + e), 0));
        u32x4 A[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          A[i] = tr_frag<C, D>(to, 32 * ks * Cf::ROWB, lane_tr, xtr, sdk + i);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            A[i][e] = pack_bf16x2(bf16lo(A[i][e]) * wt[2 * e], bf16hi(A[i][e]) * wt[2 * e + 1]);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const u32x4 B = tr_frag<C, D>(tq, 32 * ks * Cf::ROWB, lane_tr, xtr, sdv + j);
#pragma unroll
          for (int i = 0; i < NI; ++i) Sacc[NJ * i + j] = mfma16x16x32(A[i], B, Sacc[NJ * i + j]);
        }
      }
    }
    store_rows(dk, c0, m, OK);
    store_rows(dv, c0, m, OV);
    lag_chunk = false;
  };

  load_chunk(buf0, t_begin);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the entry state and the first chunk are in
  for (int c0 = t_begin; c0 < t_end; c0 += 2 * C) {
    step(buf0, buf1, c0);
    if (c0 + C >= t_end) break;
    step(buf1, buf0, c0 + C);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the empty successor's loads have landed

  if (state_out && seg == nseg - 1) {  // dS_in = lam S^T
    float *so = state_out + (size_t)bh * D * D;
#pragma unroll
    for (int a = 0; a < Cf::SDV; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        so[(size_t)(16 * (sdv + a % NJ) + lr) * D + 16 * (sdk + a / NJ) + 4 * g + i] = Sacc[a][i] * lam;
  }
}

// ---------------------------------------------------------------- fp32 path
// The bf16 path's segment plan in fp32 on the VALU, with tiles of FT tokens:
// lin_f32_pass<D, false> forms the aggregate of every segment but the last,
// lin_seg_scan turns them into the states entering the segments, and
// lin_f32_pass<D, true> walks each segment's tiles:
//   P = (Q K^T) * decay mask                                   [FT x FT]
//   O = P V + diag(w) Q S      w_i = lam^(i+1)  (lam^i while a late initial state is in its first tile)
//   S = f S + (diag(lam^(m-1-j)) K)^T V     f = lam^m  (lam^(m-1) there)
// S lives in LDS; each thread updates its own block of it.
constexpr int FT = 32;  // tokens per fp32 tile

template <int D>
struct F32Cfg {
  static constexpr int LD = D + 4;   // row stride (floats) of the staged tiles and of S
  static constexpr int SR = D / 16;  // S block of a thread: SR rows x SR columns (16 x 16 blocks)
  static constexpr int OR = 4;       // O block of a thread: OR rows (8 row groups) ...
  static constexpr int OC = D / 32;  // ... x OC columns (32 column groups)
};

template <int D, bool OUT>
__global__ __launch_bounds__(256) void lin_f32_pass(const float *__restrict__ q, const float *__restrict__ k,
                                                    const float *__restrict__ v, float *__restrict__ o,
                                                    const float *__restrict__ decay, float *__restrict__ seg_state,
                                                    const float *__restrict__ s_init, float *__restrict__ state_out,
                                                    int H, int N, int seg_len, int nseg, LinDir dir, int sin_T) {
  using Cf = F32Cfg<D>;
  constexpr int LD = Cf::LD, SR = Cf::SR, OR = Cf::OR, OC = Cf::OC;
  __shared__ __attribute__((aligned(16))) float Ks[FT][LD];
  __shared__ __attribute__((aligned(16))) float Vs[FT][LD];
  __shared__ __attribute__((aligned(16))) float Qs[OUT ? FT : 1][LD];
  __shared__ __attribute__((aligned(16))) float Ss[D][LD];
  __shared__ float Ps[OUT ? FT : 1][FT + 1];
  __shared__ float pw[FT + 1];  // lam^n, n = 0..FT
  const int tid = threadIdx.x;
  const int nblk = OUT ? nseg : nseg - 1;
  const int bh = blockIdx.x / nblk, seg = blockIdx.x % nblk;
  const int h = bh % H;
  const float lam = decay ? decay[h] : 1.f;
  const int t_begin = seg * seg_len, t_end = min(N, t_begin + seg_len);
  const size_t base = (size_t)bh * N * D;
  const size_t DD = (size_t)D * D;
  auto prow = [&](int t) -> size_t { return (size_t)(dir.rev ? N - 1 - t : t); };
  for (int n = tid; n <= FT; n += 256) pw[n] = (float)pow((double)lam, (double)n);
  // the state block of this thread: rows r0 .. r0+SR-1, columns c0 .. c0+SR-1
  const int r0 = SR * (tid >> 4), c0 = SR * (tid & 15);
  {
    const float *sin = nullptr;
    if (OUT) sin = nseg > 1 ? seg_state + ((size_t)bh * nseg + seg) * DD : (s_init ? s_init + (size_t)bh * DD : nullptr);
#pragma unroll
    for (int r = 0; r < SR; ++r)
#pragma unroll
      for (int c = 0; c < SR; ++c) {
        const int rr = r0 + r, cc = c0 + c;
        Ss[rr][cc] = sin ? sin[sin_T ? (size_t)cc * D + rr : (size_t)rr * D + cc] : 0.f;
      }
  }
  // O block of this thread: rows o0 .. o0+OR-1 of the tile, columns p0 .. p0+OC-1
  const int o0 = OR * (tid >> 5), p0 = OC * (tid & 31);
  for (int t0 = t_begin; t0 < t_end; t0 += FT) {
    const int m = min(FT, t_end - t0);
    __syncthreads();  // the previous tile's reads are done (and S is in LDS)
    for (int e = tid; e < FT * D / 4; e += 256) {
      const int i = e / (D / 4), c4 = 4 * (e % (D / 4));
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = kk, qq = kk;
      if (i < m) {
        const size_t g = base + prow(t0 + i) * D + c4;
        kk = *reinterpret_cast<const f32x4 *>(k + g);
        vv = *reinterpret_cast<const f32x4 *>(v + g);
        if (OUT) qq = *reinterpret_cast<const f32x4 *>(q + g);
      }
      *reinterpret_cast<f32x4 *>(&Ks[i][c4]) = kk;
      *reinterpret_cast<f32x4 *>(&Vs[i][c4]) = vv;
      if (OUT) *reinterpret_cast<f32x4 *>(&Qs[i][c4]) = qq;
    }
    __syncthreads();
    const bool late_first = dir.lag && t0 == 0;  // the initial state enters one step late
    if constexpr (OUT) {
      // P[i][j] = (q_i . k_j) lam^(i-j) for j <= i < m, else 0.  The dot
      // products (here and in Q S below) keep four partial sums, added as a
      // tree: sequential sums of 128 products left rows whose value cancels to
      // near zero off by more than fp32's relative bound (CPU emulation of
      // both orders against the float64 oracle).
      for (int e = tid; e < FT * FT; e += 256) {
        const int i = e / FT, j = e % FT;
        float acc = 0.f;
        if (j <= i && i < m) {
          float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
          for (int c = 0; c < D; c += 16) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&Qs[i][c + 4 * u]);
              const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&Ks[j][c + 4 * u]);
              part[u] = fmaf(a4[0], b4[0], fmaf(a4[1], b4[1], fmaf(a4[2], b4[2], fmaf(a4[3], b4[3], part[u]))));
            }
          }
          acc = ((part[0] + part[1]) + (part[2] + part[3])) * pw[i - j];
        }
        Ps[i][j] = acc;
      }
      __syncthreads();
      float acc[OR][OC], qs[4][OR][OC];
#pragma unroll
      for (int r = 0; r < OR; ++r)
#pragma unroll
        for (int c = 0; c < OC; ++c) {
          acc[r][c] = 0.f;
#pragma unroll
          for (int u = 0; u < 4; ++u) qs[u][r][c] = 0.f;
        }
      for (int j = 0; j < m; ++j) {
        float vv[OC], pp[OR];
#pragma unroll
        for (int c = 0; c < OC; ++c) vv[c] = Vs[j][p0 + c];
#pragma unroll
        for (int r = 0; r < OR; ++r) pp[r] = Ps[o0 + r][j];
#pragma unroll
        for (int r = 0; r < OR; ++r)
#pragma unroll
          for (int c = 0; c < OC; ++c) acc[r][c] = fmaf(pp[r], vv[c], acc[r][c]);
      }
#pragma unroll 2
      for (int r4 = 0; r4 < D; r4 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int rr = r4 + u;
          float ss[OC], qv[OR];
#pragma unroll
          for (int c = 0; c < OC; ++c) ss[c] = Ss[rr][p0 + c];
#pragma unroll
          for (int r = 0; r < OR; ++r) qv[r] = Qs[o0 + r][rr];
#pragma unroll
          for (int r = 0; r < OR; ++r)
#pragma unroll
            for (int c = 0; c < OC; ++c) qs[u][r][c] = fmaf(qv[r], ss[c], qs[u][r][c]);
        }
      }
#pragma unroll
      for (int r = 0; r < OR; ++r) {
        const int i = o0 + r;
        if (i >= m) continue;
        const float w = late_first ? pw[i] : pw[i + 1];
        float *orow = o + base + prow(t0 + i) * D + p0;
#pragma unroll
        for (int c = 0; c < OC; ++c)
          orow[c] = fmaf(w, (qs[0][r][c] + qs[1][r][c]) + (qs[2][r][c] + qs[3][r][c]), acc[r][c]);
      }
      __syncthreads();  // every read of S is done before it is updated
    }
    // S = f S + sum_j (lam^(m-1-j) k_j) v_j^T on this thread's block
    const float f = late_first ? pw[m - 1] : pw[m];
    float sb[SR][SR];
#pragma unroll
    for (int r = 0; r < SR; ++r)
#pragma unroll
      for (int c = 0; c < SR; ++c) sb[r][c] = f * Ss[r0 + r][c0 + c];
    for (int j = 0; j < m; ++j) {
      const float wj = pw[m - 1 - j];
      float kr[SR], vc[SR];
#pragma unroll
      for (int r = 0; r < SR; ++r) kr[r] = wj * Ks[j][r0 + r];
#pragma unroll
      for (int c = 0; c < SR; ++c) vc[c] = Vs[j][c0 + c];
#pragma unroll
      for (int r = 0; r < SR; ++r)
#pragma unroll
        for (int c = 0; c < SR; ++c) sb[r][c] = fmaf(kr[r], vc[c], sb[r][c]);
    }
#pragma unroll
    for (int r = 0; r < SR; ++r)
#pragma unroll
      for (int c = 0; c < SR; ++c) Ss[r0 + r][c0 + c] = sb[r][c];
  }
  // a segment's aggregate, or (last segment) the final state
  float *dst = nullptr;
  float fs = 1.f;
  if (!OUT) dst = seg_state + ((size_t)bh * nseg + seg) * DD;
  else if (seg == nseg - 1 && state_out) {
    dst = state_out + (size_t)bh * DD;
    fs = dir.scale ? lam : 1.f;
  }
  if (dst) {
#pragma unroll
    for (int r = 0; r < SR; ++r)
#pragma unroll
      for (int c = 0; c < SR; ++c) dst[(size_t)(r0 + r) * D + c0 + c] = Ss[r0 + r][c0 + c] * fs;
  }
}

// Segment plans.  The output pass runs one workgroup per (b, h, segment) in
// sequence over the segment's chunks, so its time is about
//   rounds * chunks per segment,  rounds = ceil(B*H*segments / 256 CUs);
// the bf16 plan takes, from enough segments to give every CU a workgroup, the
// number that minimises that, the fewest among equals, with no segment
// shorter than 32 chunks: each workgroup starts by reading its d x d entry
// state, and every segment boundary needs an aggregate of the keys that reach
// it (R28 keeps that short for fast-decaying heads and whole for slow ones),
// so fewer boundaries mean less aggregate work.  At 32 heads that is 8
// segments per head from 32K tokens up (one round).  The aggregates are
// computed over parts of at most 32 chunks, which the aggregate pass deals
// out evenly over the CUs.
// The fp32 path (VALU-bound, tiles of 32 tokens) keeps about 4 workgroups per
// CU and one part per segment.
struct SegPlan {
  int seg_len, nseg, part_len, nparts;
};
constexpr int NCU = 256;  // compute units of an MI355X
SegPlan seg_plan_bf16(int BH, int N, int C) {
  const int nchunks = (N + C - 1) / C;
  // at most AGG_MAX_PAIRS - 1 (b, h, segment) pairs with an aggregate
  const int max_seg = max(1, min(min(nchunks / 32, 1024), (AGG_MAX_PAIRS - 1) / BH + 1));
  const int min_seg = min(max_seg, max(1, NCU / BH));  // a workgroup for every CU where that is possible
  int best = 1;
  long long best_cost = -1;
  for (int ns = min_seg; ns <= max_seg; ++ns) {
    const long long rounds = ((long long)BH * ns + NCU - 1) / NCU;
    const long long cost = rounds * ((nchunks + ns - 1) / ns);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = ns;
    }
  }
  SegPlan p;
  const int cps = (nchunks + best - 1) / best;  // chunks per segment
  p.seg_len = cps * C;
  p.nseg = (N + p.seg_len - 1) / p.seg_len;
  const int ppc = max(min(cps, 32), (cps + 63) / 64);  // chunks per aggregate part (at most 64 parts)
  p.nparts = (cps + ppc - 1) / ppc;
  p.part_len = ppc * C;
  return p;
}
SegPlan seg_plan_f32(int BH, int N) {
  const int nchunks = (N + FT - 1) / FT;
  int want = (1024 + BH - 1) / BH;
  if (want > nchunks) want = nchunks;
  if (want < 1) want = 1;
  SegPlan p;
  const int cps = (nchunks + want - 1) / want;
  p.seg_len = cps * FT;
  p.nseg = (N + p.seg_len - 1) / p.seg_len;
  p.part_len = p.seg_len;
  p.nparts = 1;
  return p;
}

// The segments' entry states of the bf16 path: with one segment the caller's
// initial state; otherwise the aggregate pass and the scan (or, with
// reuse_states_T, the states a previous pass left in the workspace).
struct SegStates {
  SegPlan pl;
  const float *seg_state;
  size_t seg_stride;
  int sin_T;
};
NbK nb_args(const LinearPrefillArgs &a) {
  NbK nb{nullptr, nullptr, 0.f, 0.f, 0, nullptr};
  if (a.nb)
    nb = NbK{a.nb->gamma_q, a.nb->gamma_k, a.nb->eps, a.nb->rope_base, a.nb->pos0,
             static_cast<const uint16_t *>(a.nb->gate)};
  return nb;
}
template <int C, int D, bool REV>
SegStates seg_states_bf16(const LinearPrefillArgs &a, hipStream_t st) {
  const NbK nb = nb_args(a);
  const LinDir dir{a.rev, a.lag, a.state_T, a.scale_final};
  const bool k_transformed = nb.gk != nullptr || nb.rope_base > 0.f;
  const int BH = a.B * a.H;
  const SegPlan pl = seg_plan_bf16(BH, a.N, C);
  const int seg_len = pl.seg_len, nseg = pl.nseg;
  float *ws = static_cast<float *>(a.ws);
  const size_t DD = (size_t)D * D;
  const float *seg_state = a.state_in;  // nseg == 1: segment 0 starts from state_in
  size_t seg_stride = DD;
  int sin_T = a.state_T;
  if (nseg > 1 && a.reuse_states_T) {
    seg_state = ws;
    seg_stride = DD * pl.nparts;
    sin_T = 1;
  } else if (nseg > 1) {
    const dim3 agrid(min(BH * (nseg - 1) * pl.nparts, NCU));
    if (k_transformed)
      hipLaunchKernelGGL((lin_seg_aggregate<C, D, true, REV>), agrid, dim3(512), 0, st, (const uint16_t *)a.k,
                         (const uint16_t *)a.v, a.decay, ws, a.H, a.N, BH, seg_len, nseg, pl.part_len, pl.nparts,
                         nb);
    else
      hipLaunchKernelGGL((lin_seg_aggregate<C, D, false, REV>), agrid, dim3(512), 0, st, (const uint16_t *)a.k,
                         (const uint16_t *)a.v, a.decay, ws, a.H, a.N, BH, seg_len, nseg, pl.part_len, pl.nparts,
                         nb);
    hipLaunchKernelGGL(lin_seg_scan, dim3((unsigned)((DD + 255) / 256), BH), dim3(256), 0, st, ws,
                       a.state_in, a.decay, a.H, D, (int)DD, a.N, seg_len, nseg, pl.part_len, pl.nparts, C, dir);
    seg_state = ws;
    seg_stride = DD * pl.nparts;  // S_in(m) sits in part slot 0 of segment m
    sin_T = 0;  // the scan wrote the segment states in the plain layout
  }
  return SegStates{pl, seg_state, seg_stride, sin_T};
}

template <int C, int D, bool REV>
hipError_t run_bf16(const LinearPrefillArgs &a, hipStream_t st) {
  const NbK nb = nb_args(a);
  const LinDir dir{a.rev, a.lag, a.state_T, a.scale_final};
  const bool k_transformed = nb.gk != nullptr || nb.rope_base > 0.f;
  const int BH = a.B * a.H;
  const SegStates ss = seg_states_bf16<C, D, REV>(a, st);
  const int seg_len = ss.pl.seg_len, nseg = ss.pl.nseg;
  const float *seg_state = ss.seg_state;
  const size_t seg_stride = ss.seg_stride;
  const int sin_T = ss.sin_T;
  if constexpr (dma_fits<C, D>()) {
    const bool nbt = k_transformed || nb.gq != nullptr;  // q or k normalised or rotated
    auto kern = nb.gate ? (nbt ? lin_seg_output_dma<C, D, REV, true, true> : lin_seg_output_dma<C, D, REV, true, false>)
                        : (nbt ? lin_seg_output_dma<C, D, REV, false, true> : lin_seg_output_dma<C, D, REV, false, false>);
    hipLaunchKernelGGL(kern, dim3(BH * nseg), dim3(512), 0, st, (const uint16_t *)a.q, (const uint16_t *)a.k,
                       (const uint16_t *)a.v, (uint16_t *)a.o, a.decay, seg_state, seg_stride, a.state_out, a.H, a.N,
                       seg_len, nseg, nb, dir, sin_T);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((lin_seg_output<C, D, REV>), dim3(BH * nseg), dim3(512), 0, st, (const uint16_t *)a.q,
                     (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.o, a.decay, seg_state, seg_stride,
                     a.state_out, a.H, a.N, seg_len, nseg, nb, dir, sin_T);
  return hipGetLastError();
}

template <int C, int D>
hipError_t run_bf16(const LinearPrefillArgs &a, hipStream_t st) {
  return a.rev ? run_bf16<C, D, true>(a, st) : run_bf16<C, D, false>(a, st);
}

template <int D>
hipError_t run_f32(const LinearPrefillArgs &a, hipStream_t st) {
  const LinDir dir{a.rev, a.lag, a.state_T, a.scale_final};
  const int BH = a.B * a.H;
  const SegPlan pl = seg_plan_f32(BH, a.N);
  const int seg_len = pl.seg_len, nseg = pl.nseg;
  float *ws = static_cast<float *>(a.ws);
  const size_t DD = (size_t)D * D;
  const float *q = static_cast<const float *>(a.q), *k = static_cast<const float *>(a.k),
              *v = static_cast<const float *>(a.v);
  if (nseg > 1 && !a.reuse_states_T) {
    hipLaunchKernelGGL((lin_f32_pass<D, false>), dim3(BH * (nseg - 1)), dim3(256), 0, st, q, k, v, nullptr, a.decay,
                       ws, nullptr, nullptr, a.H, a.N, seg_len, nseg, dir, 0);
    hipLaunchKernelGGL(lin_seg_scan, dim3((unsigned)((DD + 255) / 256), BH), dim3(256), 0, st, ws, a.state_in,
                       a.decay, a.H, D, (int)DD, a.N, seg_len, nseg, pl.part_len, pl.nparts, FT, dir);
  }
  // one segment: the pass reads the caller's initial state itself (transposed if asked)
  hipLaunchKernelGGL((lin_f32_pass<D, true>), dim3(BH * nseg), dim3(256), 0, st, q, k, v, static_cast<float *>(a.o),
                     a.decay, ws, a.state_in, a.state_out, a.H, a.N, seg_len, nseg, dir,
                     nseg > 1 ? a.reuse_states_T : a.state_T);
  return hipGetLastError();
}

}  // namespace

size_t linear_prefill_workspace(int dtype, int B, int H, int N, int d, int chunk) {
  const SegPlan pl = dtype == 1 ? seg_plan_bf16(B * H, N, chunk) : seg_plan_f32(B * H, N);
  if (pl.nseg <= 1) return 0;
  return (size_t)B * H * pl.nseg * pl.nparts * d * d * sizeof(float);
}

hipError_t launch_linear_prefill(const LinearPrefillArgs &a, hipStream_t st) {
  if (a.dtype == 0) return a.d == 64 ? run_f32<64>(a, st) : run_f32<128>(a, st);
  if (a.chunk == 128 && a.d == 128) return run_bf16<128, 128>(a, st);
  if (a.chunk == 64 && a.d == 128) return run_bf16<64, 128>(a, st);
  if (a.chunk == 128 && a.d == 64) return run_bf16<128, 64>(a, st);
  return run_bf16<64, 64>(a, st);
}

// Gradients of the linear layer through three passes of the forward
// operation (see the header comment): dQ on (dO, V, K) from S_in^T; dK on the
// reversed (V, dO, Q) from a late dS^T; dV on the reversed (K, Q, dO) from a
// late dS, whose final state times lam is dS_in.  The passes run in order on
// `st` and share the workspace.
hipError_t launch_linear_prefill_backward(const LinearBackwardArgs &a, hipStream_t st) {
  LinearPrefillArgs pq{a.dtype, a.B, a.H, a.N, a.d, a.chunk, a.dout, a.v, a.k, a.dq, a.decay, a.state_in,
                       nullptr, a.ws, nullptr};
  pq.state_T = 1;
  hipError_t e = launch_linear_prefill(pq, st);
  if (e != hipSuccess) return e;
  LinearPrefillArgs pk{a.dtype, a.B, a.H, a.N, a.d, a.chunk, a.v, a.dout, a.q, a.dk, a.decay, a.dstate_out,
                       nullptr, a.ws, nullptr};
  pk.rev = 1;
  pk.lag = 1;
  pk.state_T = 1;
  if (a.dtype == 1 && a.chunk == 64 && a.d == 128) {
    // dK and dV in one reversed pass from the dK pass's segment states
    using Cf = LinCfg<64, 128>;
    const SegStates ss = seg_states_bf16<64, 128, true>(pk, st);
    hipLaunchKernelGGL((lin_seg_grad_kv<64, 128>), dim3(a.B * a.H * ss.pl.nseg), dim3(Cf::NT), 0, st,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (const uint16_t *)a.dout, (uint16_t *)a.dk, (uint16_t *)a.dv, a.decay, ss.seg_state,
                       ss.seg_stride, a.dstate_in, a.H, a.N, ss.pl.seg_len, ss.pl.nseg, 1, ss.sin_T);
    return hipGetLastError();
  }
  e = launch_linear_prefill(pk, st);
  if (e != hipSuccess) return e;
  LinearPrefillArgs pv{a.dtype, a.B, a.H, a.N, a.d, a.chunk, a.k, a.q, a.dout, a.dv, a.decay, a.dstate_out,
                       a.dstate_in, a.ws, nullptr};
  pv.rev = 1;
  pv.lag = 1;
  pv.scale_final = 1;
  // its states are sum Q dO^T, the transposes of the dK pass's sum dO Q^T (same
  // decays, same late start, initial dS against dS^T): read them transposed
  pv.reuse_states_T = 1;
  return launch_linear_prefill(pv, st);
}

}  // namespace sala
