// Sparse-layer decode for gfx950: one query token per (b, hq) at position L-1
// attends to every cached token (< L) of the blocks listed for its KV head.
// Same restricted softmax as the prefill (exact attention over a block mask:
// FlashAttention entry of the fugumt.com related list for arXiv 2607.21752);
// the KV cache is kept whole (MiniCPM-SALA, gist.science (ja) 技術概要 section 1).
//
// Split-K: a workgroup takes selected blocks of one (b, kv head) for all G
// query heads of that group (one gathered block feeds G heads) and writes
// (max, sum, unnormalised o) per head in log2 units; decode_combine merges the
// splits with the usual log-sum-exp rescaling.  bf16 with G <= 16 uses
// decode_attend_mfma (one wave per selected block, both products on MFMA);
// other cases use decode_partial (fp32 VALU, a few blocks per workgroup).

#include "sala_common.hpp"
#include "sala_launch.hpp"

namespace sala {
namespace {

constexpr int BLK = 64;
constexpr int MAXG = 32;

template <typename T>
__device__ __forceinline__ void load_row16(const T *p, float *f) {  // 16 bytes -> floats
  const u32x4 x = gload16(p);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { f[2 * e] = bf16lo(x[e]); f[2 * e + 1] = bf16hi(x[e]); }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(x[e]);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_partial(const T *__restrict__ q, const T *__restrict__ kc,
                                                      const T *__restrict__ vc, const int32_t *__restrict__ idx,
                                                      float *__restrict__ part, int Hq, int Hkv, int L, int Lc,
                                                      int n_sel, int nsplit, int bps, float scale_log2) {
  constexpr int KS = D + 4;                         // padded K row (floats)
  constexpr int EPL = sizeof(T) == 2 ? 8 : 4;       // elements per 16-byte load
  constexpr int CPR = D / EPL;                      // 16-byte loads per row
  constexpr int CPL = D / 64;                       // d_v columns per lane
  __shared__ __attribute__((aligned(16))) float ks[BLK * KS];
  __shared__ __attribute__((aligned(16))) float vs[BLK * D];
  __shared__ __attribute__((aligned(16))) float qs[MAXG * D];
  __shared__ float ps[MAXG][BLK];
  __shared__ int nvalid_sh;

  const int bkv = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
  const int b = bkv / Hkv, kvh = bkv % Hkv, G = Hq / Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int32_t *row = idx + (size_t)bkv * n_sel;
  if (tid < 64) {  // wave 0: the index of the first negative entry, 64 entries per load
    int n = n_sel;
    for (int e0 = 0; e0 < n_sel; e0 += 64) {
      const int e = e0 + tid;
      const uint64_t neg = __ballot(e < n_sel && row[e] < 0);
      if (neg != 0) {
        n = e0 + __builtin_ctzll(neg);
        break;
      }
    }
    if (tid == 0) nvalid_sh = n;
  }
  for (int x = tid; x < G * D; x += 256) {
    const int g = x / D, c = x % D;
    const size_t off = (size_t)(b * Hq + kvh * G + g) * D + c;
    float f;
    if constexpr (sizeof(T) == 2) f = bf16_to_f32(reinterpret_cast<const uint16_t *>(q)[off]);
    else f = q[off];
    qs[g * D + c] = f * scale_log2;
  }
  __syncthreads();
  const int e0 = sp * bps, e1 = min(nvalid_sh, e0 + bps);

  constexpr int HPW = MAXG / 4;  // heads per wave, upper bound
  float m_run[HPW], l_run[HPW], oacc[HPW][CPL];
#pragma unroll
  for (int a = 0; a < HPW; ++a) {
    m_run[a] = -INFINITY;
    l_run[a] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) oacc[a][c] = 0.f;
  }
  const T *kbase = kc + (size_t)bkv * Lc * D;  // cache rows hold Lc tokens
  const T *vbase = vc + (size_t)bkv * Lc * D;

  for (int e = e0; e < e1; ++e) {
    const int j = row[e];
    if ((size_t)j * BLK >= (size_t)L) continue;
    const int cnt = min(BLK, L - j * BLK);
    __syncthreads();
    for (int x = tid; x < BLK * CPR; x += 256) {
      const int r = x / CPR, c = (x % CPR) * EPL;
      float f[EPL], g2[EPL];
      if (r < cnt) {
        load_row16(kbase + ((size_t)j * BLK + r) * D + c, f);
        load_row16(vbase + ((size_t)j * BLK + r) * D + c, g2);
      } else {
#pragma unroll
        for (int u = 0; u < EPL; ++u) { f[u] = 0.f; g2[u] = 0.f; }
      }
#pragma unroll
      for (int u = 0; u < EPL; ++u) { ks[r * KS + c + u] = f[u]; vs[r * D + c + u] = g2[u]; }
    }
    __syncthreads();
    // logits for this wave's heads (h = w, w+4, ...), lane = key
#pragma unroll
    for (int a = 0; a < HPW; ++a) {
      const int h = w + 4 * a;
      if (h >= G) break;
      float s = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; c += 4) {
        const float4 kk = *reinterpret_cast<const float4 *>(&ks[lane * KS + c]);
        const float4 qq = *reinterpret_cast<const float4 *>(&qs[h * D + c]);
        s = fmaf(kk.x, qq.x, s);
        s = fmaf(kk.y, qq.y, s);
        s = fmaf(kk.z, qq.z, s);
        s = fmaf(kk.w, qq.w, s);
      }
      if (lane >= cnt) s = -INFINITY;
      const float bm = wave_max(s);
      const float mnew = fmaxf(m_run[a], bm);
      const float alpha = __builtin_amdgcn_exp2f(m_run[a] - mnew);
      const float p = __builtin_amdgcn_exp2f(s - mnew);
      l_run[a] = l_run[a] * alpha + wave_sum(p);
      m_run[a] = mnew;
      ps[h][lane] = p;
#pragma unroll
      for (int c = 0; c < CPL; ++c) oacc[a][c] *= alpha;
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < HPW; ++a) {
      const int h = w + 4 * a;
      if (h >= G) break;
      for (int kk = 0; kk < cnt; ++kk) {
        const float p = ps[h][kk];
#pragma unroll
        for (int c = 0; c < CPL; ++c) oacc[a][c] = fmaf(p, vs[kk * D + CPL * lane + c], oacc[a][c]);
      }
    }
  }
  // partials: [b*Hq + hq][split][D + 2] = (o..., m, l)
#pragma unroll
  for (int a = 0; a < HPW; ++a) {
    const int h = w + 4 * a;
    if (h >= G) break;
    float *dst = part + ((size_t)(b * Hq + kvh * G + h) * nsplit + sp) * (D + 2);
#pragma unroll
    for (int c = 0; c < CPL; ++c) dst[CPL * lane + c] = oacc[a][c];
    if (lane == 0) { dst[D] = m_run[a]; dst[D + 1] = l_run[a]; }
  }
}

// bf16, G <= 16: one wave per (b, kv head, entry e of the selected list).
// S^T = K Q^T for the block's 64 keys on MFMA (A = K rows in the 32-key pair
// order, loaded straight into registers; B = the group's <= 16 query heads),
// so each lane's accumulators are 8 consecutive keys of one head -- the B
// operand of O^T = V^T P^T.  Softmax over the 64 keys stays in registers
// (two cross-lane steps); V goes to LDS row-major by direct loads and its
// V^T fragments come from transposed LDS reads.  Writes (o unnormalised,
// max, sum) per head in log2 units for the combine.
template <int D>
__global__ __launch_bounds__(64) void decode_attend_mfma(const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ kc,
                                                         const uint16_t *__restrict__ vc,
                                                         const int32_t *__restrict__ idx, float *__restrict__ part,
                                                         int Hq, int Hkv, int L, int Lc, int n_sel, float scale_log2) {
  constexpr int NDS = D / 32, ND = D / 16, NCH = D / 8, ROWB = 2 * D;
  __shared__ __attribute__((aligned(16))) char vs[BLK * ROWB];
  const int bkv = blockIdx.x / n_sel, e = blockIdx.x % n_sel;
  const int b = bkv / Hkv, kvh = bkv % Hkv, G = Hq / Hkv;
  const int l = threadIdx.x, lr = l & 15, g = l >> 4;
  const int32_t *row = idx + (size_t)bkv * n_sel;
  // entries end at the first negative one: the wave checks 0..e, 64 at a time
  const int j = row[e];
  bool neg = false;
  for (int x0 = 0; x0 <= e; x0 += 64) {
    const int x = x0 + l;
    if (x <= e && row[x] < 0) neg = true;
  }
  const bool valid = !__any(neg) && (size_t)j * BLK < (size_t)L;
  float *dst = part + ((size_t)(b * Hq + kvh * G + lr) * n_sel + e) * (D + 2);
  if (!valid) {  // an empty split: the combine gives it zero weight
    if (lr < G) {
#pragma unroll
      for (int dvt = 0; dvt < ND; ++dvt)
        *reinterpret_cast<f32x4 *>(dst + 16 * dvt + 4 * g) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (g == 0) { dst[D] = -INFINITY; dst[D + 1] = 0.f; }
    }
    return;
  }
  const int cnt = min(BLK, L - j * BLK);
  const size_t base = (size_t)bkv * Lc + (size_t)j * BLK;  // cache rows hold Lc tokens
  // V rows -> LDS by direct loads: slot p = 64u + l holds row p / NCH, chunk
  // p % NCH after the fkv swizzle, so the lane fetches the logical chunk that
  // maps there (the XOR is an involution).  Rows past cnt repeat row cnt-1;
  // their weights are zero.
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int p = 64 * u + l, vrow = p / NCH, ch = (p % NCH) ^ (int)(fkv(vrow) & (NCH - 1));
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1))) *)(vc + (base + min(vrow, cnt - 1)) * D + 8 * ch),
        (void __attribute__((address_space(3))) *)(vs + 64 * u * 16), 16, 0, 0);
  }
  // K fragments (A operands) and the group's query fragments (B operands)
  u32x4 kf[2][2][NDS], qf[NDS];
  const uint16_t *qp = q + (size_t)(b * Hq + kvh * G + min(lr, G - 1)) * D;
#pragma unroll
  for (int s = 0; s < NDS; ++s) qf[s] = gload16(qp + 32 * s + 8 * g);
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t *kp = kc + (base + min(32 * pp + pair_key(t, lr), cnt - 1)) * D;
#pragma unroll
      for (int s = 0; s < NDS; ++s) kf[pp][t][s] = gload16(kp + 32 * s + 8 * g);
    }
  if (lr >= G) {
#pragma unroll
    for (int s = 0; s < NDS; ++s) qf[s] = u32x4{0, 0, 0, 0};
  }
  f32x4 S[2][2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NDS; ++s) acc = mfma16x16x32(kf[pp][t][s], qf[s], acc);
      S[pp][t] = acc;
    }
  // lane (head lr, group g) holds keys 32pp + 8g + 4t + i
  float mx = -INFINITY;
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = (32 * pp + 8 * g + 4 * t + i < cnt) ? S[pp][t][i] * scale_log2 : -INFINITY;
        S[pp][t][i] = x;
        mx = fmaxf(mx, x);
      }
  mx = row4_max(mx);
  float ls = 0.f;
  u32x4 Bp[2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    float p[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[t][i] = __builtin_amdgcn_exp2f(S[pp][t][i] - mx);
        ls += p[t][i];
      }
    Bp[pp] = u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]), pack_bf16x2(p[1][0], p[1][1]),
                   pack_bf16x2(p[1][2], p[1][3])};
  }
  ls = row4_sum(ls);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the V rows are in LDS
  const uint32_t lane_off = tr_lane_off(l, ROWB), lane_xor = tr_lane_xor(l);
  // every lane takes part in the MFMAs; only heads < G store
#pragma unroll
  for (int dvt = 0; dvt < ND; ++dvt) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
      o = mfma16x16x32(tr_frag(vs, 32 * pp * ROWB, lane_off, lane_xor, dvt, NCH, ROWB), Bp[pp], o);
    if (lr < G) *reinterpret_cast<f32x4 *>(dst + 16 * dvt + 4 * g) = o;
  }
  if (lr < G && g == 0) {
    dst[D] = mx;
    dst[D + 1] = ls;
  }
}

// Log-sum-exp merge of the splits of one (b, hq): thread (column c, part p)
// takes splits p, p + P, ... with all of its loads in flight at once (up to
// CU splits per thread, else in rounds), then the P parts merge through LDS.
template <typename T, int D>
__global__ __launch_bounds__(512) void decode_combine(const float *__restrict__ part, T *__restrict__ o, int nsplit) {
  constexpr int P = 512 / D, CU = 24;
  __shared__ float red_m[P][D], red_l[P][D], red_o[P][D];
  const int bh = blockIdx.x, c = threadIdx.x % D, p = threadIdx.x / D;
  const float *base = part + (size_t)bh * nsplit * (D + 2);
  float M = -INFINITY, lsum = 0.f, acc = 0.f;
  for (int s0 = p; s0 < nsplit; s0 += P * CU) {
    float mm[CU], ll[CU], oo[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int sp = min(s0 + P * u, nsplit - 1);
      const float *r = base + (size_t)sp * (D + 2);
      mm[u] = r[D];
      ll[u] = r[D + 1];
      oo[u] = r[c];
    }
    float mnew = M;
#pragma unroll
    for (int u = 0; u < CU; ++u)
      if (s0 + P * u < nsplit) mnew = fmaxf(mnew, mm[u]);
    if (mnew != -INFINITY) {
      const float a = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mnew);
      lsum *= a;
      acc *= a;
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const float wgt = (s0 + P * u < nsplit && mm[u] != -INFINITY) ? __builtin_amdgcn_exp2f(mm[u] - mnew) : 0.f;
        lsum = fmaf(ll[u], wgt, lsum);
        acc = fmaf(oo[u], wgt, acc);
      }
      M = mnew;
    }
  }
  red_m[p][c] = M;
  red_l[p][c] = lsum;
  red_o[p][c] = acc;
  __syncthreads();
  if (p != 0) return;
  float Mall = -INFINITY;
#pragma unroll
  for (int x = 0; x < P; ++x) Mall = fmaxf(Mall, red_m[x][c]);
  float L = 0.f, A = 0.f;
  if (Mall != -INFINITY) {
#pragma unroll
    for (int x = 0; x < P; ++x) {
      const float wgt = (red_m[x][c] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(red_m[x][c] - Mall);
      L = fmaf(red_l[x][c], wgt, L);
      A = fmaf(red_o[x][c], wgt, A);
    }
  }
  const float r = (L > 0.f) ? A / L : 0.f;
  if constexpr (sizeof(T) == 2) reinterpret_cast<uint16_t *>(o)[(size_t)bh * D + c] = f32_to_bf16(r);
  else o[(size_t)bh * D + c] = r;
}

void split_plan(int BHkv, int n_sel, int *nsplit, int *bps) {
  int want = (512 + BHkv - 1) / BHkv;
  if (want > n_sel) want = n_sel;
  if (want < 1) want = 1;
  *bps = (n_sel + want - 1) / want;
  *nsplit = (n_sel + *bps - 1) / *bps;
}

template <typename T, int D>
void run(const SparseDecodeArgs &a, hipStream_t st) {
  float *part = static_cast<float *>(a.ws);
  if (sizeof(T) == 2 && a.Hq / a.Hkv <= 16) {
    hipLaunchKernelGGL((decode_attend_mfma<D>), dim3(a.B * a.Hkv * a.n_sel), dim3(64), 0, st, (const uint16_t *)a.q,
                       (const uint16_t *)a.k_cache, (const uint16_t *)a.v_cache, a.idx, part, a.Hq, a.Hkv, a.L,
                       a.Lc ? a.Lc : a.L, a.n_sel, a.scale * 1.4426950408889634f);
    hipLaunchKernelGGL((decode_combine<T, D>), dim3(a.B * a.Hq), dim3(512), 0, st, part, (T *)a.o, a.n_sel);
    return;
  }
  int nsplit, bps;
  split_plan(a.B * a.Hkv, a.n_sel, &nsplit, &bps);
  hipLaunchKernelGGL((decode_partial<T, D>), dim3(a.B * a.Hkv * nsplit), dim3(256), 0, st, (const T *)a.q,
                     (const T *)a.k_cache, (const T *)a.v_cache, a.idx, part, a.Hq, a.Hkv, a.L, a.Lc ? a.Lc : a.L,
                     a.n_sel, nsplit, bps,
                     a.scale * 1.4426950408889634f);
  hipLaunchKernelGGL((decode_combine<T, D>), dim3(a.B * a.Hq), dim3(512), 0, st, part, (T *)a.o, nsplit);
}

}  // namespace

size_t sparse_decode_workspace(int dtype, int B, int Hq, int Hkv, int L, int d, int block, int n_sel) {
  (void)L; (void)block;
  int nsplit, bps;
  split_plan(B * Hkv, n_sel, &nsplit, &bps);
  if (dtype == 1 && Hq / Hkv <= 16) nsplit = n_sel;  // one split per selected block
  return (size_t)B * Hq * nsplit * (d + 2) * sizeof(float);
}

hipError_t launch_sparse_decode(const SparseDecodeArgs &a, hipStream_t st) {
  if (a.dtype == 1) {
    if (a.d == 128) run<uint16_t, 128>(a, st);
    else run<uint16_t, 64>(a, st);
  } else {
    if (a.d == 128) run<float, 128>(a, st);
    else run<float, 64>(a, st);
  }
  return hipGetLastError();
}

}  // namespace sala
