// Block-sparse softmax attention prefill for gfx950.
//
// For query head hq (KV head hq/G) and token t of query block i:
//   A(t) = { s in the blocks listed in idx[b, hq/G, i] : s <= t }
//   o_t  = softmax over A(t) of (scale * q_t . k_s), applied to v_s.
// The sparse layers keep the whole KV cache but compute over a subset of it
// (MiniCPM-SALA, gist.science (ja) 技術概要 section 1); the computation over
// the subset is exact softmax attention under a block mask, the block-sparse
// form of IO-aware exact attention (FlashAttention entry in the related list of
// the fugumt.com page for arXiv 2607.21752).  Only the published idea -- tiles
// staged on chip, an online softmax, no score matrix in HBM -- is used here.
//
// bf16 design (MI355X):
//   * One workgroup = 4 waves = 4 query heads of one GQA group x the 64 tokens
//     of one query block.  All heads of a group share the selected blocks, so
//     every gathered 64-key block (16 KiB of K + 16 KiB of V at d = 128) feeds
//     256 query rows from LDS.
//   * S^T = K Q^T on MFMA 16x16x32 (A = K rows from LDS, B = Q rows held in
//     registers), so each lane owns one query row and 16 keys per tile row:
//     row max/sum need only two cross-lane steps per block.
//   * O^T += V^T P^T with V pre-transposed per block in the workspace
//     (transpose_v_blocks), so the V^T operand is a 16-byte LDS read.
//   * K and V^T blocks are double buffered in LDS; the next block's global
//     loads are issued before the current block's MFMAs.
//   * Workgroups of one (b, kv head, query block) land on the same XCD so the
//     gathered blocks are shared in that XCD's L2.
// fp32 path: sparse_attn_f32, one thread per query token, fp32 FMA.

#include "sala_common.hpp"
#include "sala_launch.hpp"

namespace sala {
namespace {

constexpr int BLK = 64;  // tokens per KV / query block

template <int NCH>
__device__ __forceinline__ uint32_t swz_t(uint32_t row, uint32_t ch) {
  return ch ^ ((row ^ (row >> 3)) & (NCH - 1));
}
template <int NCH>
__device__ __forceinline__ uint32_t swz_k(uint32_t row, uint32_t ch) {
  if constexpr (NCH == 16) return ch ^ ((row & 3) | ((row >> 1) & 12));
  else return ch ^ (((row >> 1) & 1) | ((row >> 2) & 6));
}
__device__ __forceinline__ int pair_key(int t, int r) { return ((r >> 2) << 3) + (t << 2) + (r & 3); }

// V [bh][N][D] -> Vt [bh][NB][D][64] (keys contiguous), zero past N.
template <int D>
__global__ __launch_bounds__(256) void transpose_v_blocks(const uint16_t *__restrict__ v, uint16_t *__restrict__ vt,
                                                          int N, int NB) {
  const int bid = blockIdx.x;
  const int bh = bid / NB, j = bid % NB;
  const int tid = threadIdx.x;
  constexpr int FG = D / 8;
  if (tid >= 8 * FG) return;
  const int tg = tid / FG, fg = tid % FG;
  const uint16_t *src = v + ((size_t)bh * N + (size_t)j * BLK) * D;
  u32x4 x[8], y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = j * BLK + 8 * tg + e;
    x[e] = (t < N) ? gload16(src + (size_t)(8 * tg + e) * D + 8 * fg) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int p = f >> 1;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint32_t a = x[2 * qq][p], b = x[2 * qq + 1][p];
      y[f][qq] = (f & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
  uint16_t *dst = vt + ((size_t)bh * NB + j) * D * BLK;
#pragma unroll
  for (int f = 0; f < 8; ++f) gstore16(dst + (size_t)(8 * fg + f) * BLK + 8 * tg, y[f]);
}

template <int D>
struct SpCfg {
  static constexpr int NDS = D / 32;     // 32-deep feature steps
  static constexpr int ND = D / 16;      // 16-wide d_v tiles
  static constexpr int KCH = D / 8;      // chunks per K row
  static constexpr int TCH = BLK / 8;    // chunks per V^T row (8)
  static constexpr int KB = BLK * D * 2; // bytes of one K block (== V^T block)
  static constexpr int PER_T = KB / 16 / 256;  // 16-byte pieces per thread per block
};

template <int D>
__global__ __launch_bounds__(256) void sparse_attn_bf16(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                        const uint16_t *__restrict__ vt, const int32_t *__restrict__ idx,
                                                        uint16_t *__restrict__ o, int Hq, int Hkv, int N, int NQB,
                                                        int n_sel, int HG, int ntasks, float scale_log2) {
  using Cf = SpCfg<D>;
  __shared__ __attribute__((aligned(16))) char kbuf[2][Cf::KB];
  __shared__ __attribute__((aligned(16))) char vbuf[2][Cf::KB];
  __shared__ int sel[1024];
  __shared__ int nvalid_sh;

  // XCD-aware mapping: the HG workgroups of one task share blockIdx % 8.
  const int x = blockIdx.x;
  const int slot = x >> 3;
  const int task = (slot / HG) * 8 + (x & 7);
  const int hg = slot % HG;
  if (task >= ntasks) return;
  const int i = task % NQB;
  const int bkv = task / NQB;  // b * Hkv + kvh
  const int b = bkv / Hkv, kvh = bkv % Hkv;
  const int G = Hq / Hkv;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int hl = 4 * hg + w;
  const bool active = hl < G;
  const int hq = kvh * G + (active ? hl : 0);

  // selected-block list: entries in order until the first negative, skipping j > i
  if (tid == 0) {
    const int32_t *row = idx + ((size_t)bkv * NQB + i) * n_sel;
    int n = 0;
    for (int e = 0; e < n_sel; ++e) {
      const int j = row[e];
      if (j < 0) break;
      if (j <= i) sel[n++] = j;
    }
    nvalid_sh = n;
  }

  // Q fragments (B operand): lane holds Q[t = 64i + 16qt + lr][32s + 8lg .. +7]
  const uint16_t *qb = q + ((size_t)(b * Hq + hq) * N) * D;
  u32x4 qf[4][Cf::NDS];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int t = BLK * i + 16 * qt + lr;
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s)
      qf[qt][s] = (t < N) ? gload16(qb + (size_t)t * D + 32 * s + 8 * lg) : u32x4{0, 0, 0, 0};
  }

  f32x4 Oacc[4][Cf::ND];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt)
#pragma unroll
    for (int dv = 0; dv < Cf::ND; ++dv) Oacc[qt][dv] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) { mrow[qt] = -INFINITY; lrow[qt] = 0.f; }

  __syncthreads();
  const int nvalid = nvalid_sh;
  const uint16_t *kbase = k + ((size_t)bkv * N) * D;
  const int NB = (N + BLK - 1) / BLK;
  const uint16_t *vtbase = vt + ((size_t)bkv * NB) * D * BLK;

  u32x4 kreg[Cf::PER_T], vreg[Cf::PER_T];
  auto gather = [&](int j) {
    const uint16_t *ksrc = kbase + (size_t)j * BLK * D;
    const uint16_t *vsrc = vtbase + (size_t)j * D * BLK;
    const int rows_valid = min(BLK, N - j * BLK);
#pragma unroll
    for (int u = 0; u < Cf::PER_T; ++u) {
      const int c = tid + 256 * u;
      const int row = c / Cf::KCH;
      kreg[u] = (row < rows_valid) ? gload16(ksrc + (size_t)c * 8) : u32x4{0, 0, 0, 0};
      vreg[u] = gload16(vsrc + (size_t)c * 8);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < Cf::PER_T; ++u) {
      const int c = tid + 256 * u;
      const int krow = c / Cf::KCH, kch = c % Cf::KCH;
      lds_store(kbuf[buf], (krow * Cf::KCH + swz_k<Cf::KCH>(krow, kch)) * 16u, kreg[u]);
      const int vrow = c / Cf::TCH, vch = c % Cf::TCH;
      lds_store(vbuf[buf], (vrow * Cf::TCH + swz_t<Cf::TCH>(vrow, vch)) * 16u, vreg[u]);
    }
  };

  if (nvalid > 0) {
    gather(sel[0]);
    stage(0);
  }
  __syncthreads();

  for (int bi = 0; bi < nvalid; ++bi) {
    const int buf = bi & 1;
    const int j = sel[bi];
    if (bi + 1 < nvalid) gather(sel[bi + 1]);

    // S^T = K Q^T : tiles [kt][qt], lane holds keys 32p + 8lg + 4t + e for kt = 2p + t
    f32x4 Sacc[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) Sacc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int row = 32 * (kt >> 1) + pair_key(kt & 1, lr);
        const u32x4 A = lds_load<u32x4>(kbuf[buf], (row * Cf::KCH + swz_k<Cf::KCH>(row, 4 * s + lg)) * 16u);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) Sacc[kt][qt] = mfma16x16x32(A, qf[qt][s], Sacc[kt][qt]);
      }
    }

    // online softmax (log2 domain)
    const bool diag = (j == i);
    u32x4 Pf[4][2];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const int qq = 16 * qt + lr;  // query position inside the block
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1) + e;
          float xv = Sacc[kt][qt][e] * scale_log2;
          if (diag && key > qq) xv = -INFINITY;
          Sacc[kt][qt][e] = xv;
          mx = fmaxf(mx, xv);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[qt], mx);
      const float alpha = __builtin_amdgcn_exp2f(mrow[qt] - mnew);
      mrow[qt] = mnew;
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = __builtin_amdgcn_exp2f(Sacc[kt][qt][e] - mnew);
          Sacc[kt][qt][e] = pv;
          ps += pv;
        }
      lrow[qt] = lrow[qt] * alpha + ps;
#pragma unroll
      for (int dv = 0; dv < Cf::ND; ++dv) Oacc[qt][dv] *= alpha;
#pragma unroll
      for (int p = 0; p < 2; ++p)
        Pf[qt][p] = u32x4{pack_bf16x2(Sacc[2 * p][qt][0], Sacc[2 * p][qt][1]),
                          pack_bf16x2(Sacc[2 * p][qt][2], Sacc[2 * p][qt][3]),
                          pack_bf16x2(Sacc[2 * p + 1][qt][0], Sacc[2 * p + 1][qt][1]),
                          pack_bf16x2(Sacc[2 * p + 1][qt][2], Sacc[2 * p + 1][qt][3])};
    }

    // O^T += V^T P^T
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int dv = 0; dv < Cf::ND; ++dv) {
        const int row = 16 * dv + lr;
        const u32x4 A = lds_load<u32x4>(vbuf[buf], (row * Cf::TCH + swz_t<Cf::TCH>(row, 4 * p + lg)) * 16u);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) Oacc[qt][dv] = mfma16x16x32(A, Pf[qt][p], Oacc[qt][dv]);
      }

    if (bi + 1 < nvalid) stage(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
  uint16_t *ob = o + ((size_t)(b * Hq + hq) * N) * D;
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    float lt = lrow[qt];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
    const int t = BLK * i + 16 * qt + lr;
    if (t < N) {
#pragma unroll
      for (int dv = 0; dv < Cf::ND; ++dv)
        *reinterpret_cast<u32x2 *>(ob + (size_t)t * D + 16 * dv + 4 * lg) =
            u32x2{pack_bf16x2(Oacc[qt][dv][0] * inv, Oacc[qt][dv][1] * inv),
                  pack_bf16x2(Oacc[qt][dv][2] * inv, Oacc[qt][dv][3] * inv)};
    }
  }
}

// fp32: one workgroup = one (b, hq, query block); thread = one query token.
template <int D>
__global__ __launch_bounds__(64) void sparse_attn_f32(const float *__restrict__ q, const float *__restrict__ k,
                                                      const float *__restrict__ v, const int32_t *__restrict__ idx,
                                                      float *__restrict__ o, int Hq, int Hkv, int N, int NQB,
                                                      int n_sel, float scale) {
  __shared__ float qs[BLK][D + 1];
  __shared__ float ks[BLK][D];
  __shared__ float vs[BLK][D];
  const int bid = blockIdx.x;
  const int i = bid % NQB, bh = bid / NQB;  // bh = b * Hq + hq
  const int b = bh / Hq, hq = bh % Hq, G = Hq / Hkv, kvh = hq / G;
  const int tid = threadIdx.x;
  const int t = BLK * i + tid;
  const float *qb = q + (size_t)bh * N * D;
  const float *kb = k + (size_t)(b * Hkv + kvh) * N * D;
  const float *vb = v + (size_t)(b * Hkv + kvh) * N * D;
  for (int e = tid; e < BLK * D; e += 64) {
    const int r = e / D, c = e % D;
    qs[r][c] = (BLK * i + r < N) ? qb[(size_t)(BLK * i + r) * D + c] : 0.f;
  }
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const int32_t *row = idx + ((size_t)(b * Hkv + kvh) * NQB + i) * n_sel;
  for (int e = 0; e < n_sel; ++e) {
    const int j = row[e];
    if (j < 0) break;
    if (j > i) continue;
    __syncthreads();
    for (int x = tid; x < BLK * D; x += 64) {
      const int r = x / D, c = x % D;
      const bool ok = BLK * j + r < N;
      ks[r][c] = ok ? kb[(size_t)(BLK * j + r) * D + c] : 0.f;
      vs[r][c] = ok ? vb[(size_t)(BLK * j + r) * D + c] : 0.f;
    }
    __syncthreads();
    const int kmax = (j == i) ? tid : BLK - 1;  // causal inside the diagonal block
    for (int kk = 0; kk <= kmax; ++kk) {
      if (BLK * j + kk >= N) break;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) s = fmaf(qs[tid][c], ks[kk][c], s);
      s *= scale;
      const float mnew = fmaxf(m, s);
      const float alpha = expf(m - mnew);
      const float p = expf(s - mnew);
      lsum = lsum * alpha + p;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vs[kk][c], acc[c] * alpha);
      m = mnew;
    }
  }
  if (t < N) {
    const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
    float *orow = o + ((size_t)bh * N + t) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) orow[c] = acc[c] * inv;
  }
}

}  // namespace

size_t sparse_prefill_workspace(int dtype, int B, int Hq, int Hkv, int N, int d, int block, int n_sel) {
  (void)Hq; (void)n_sel;
  if (dtype != 1) return 0;
  const size_t NB = (size_t)(N + block - 1) / block;
  return (size_t)B * Hkv * NB * block * d * 2;  // V^T blocks
}

hipError_t launch_sparse_prefill(const SparsePrefillArgs &a, hipStream_t st) {
  const int NQB = (a.N + BLK - 1) / BLK;
  if (a.dtype == 0) {
    if (a.d == 64)
      hipLaunchKernelGGL(sparse_attn_f32<64>, dim3(a.B * a.Hq * NQB), dim3(64), 0, st, (const float *)a.q,
                         (const float *)a.k, (const float *)a.v, a.idx, (float *)a.o, a.Hq, a.Hkv, a.N, NQB,
                         a.n_sel, a.scale);
    else
      hipLaunchKernelGGL(sparse_attn_f32<128>, dim3(a.B * a.Hq * NQB), dim3(64), 0, st, (const float *)a.q,
                         (const float *)a.k, (const float *)a.v, a.idx, (float *)a.o, a.Hq, a.Hkv, a.N, NQB,
                         a.n_sel, a.scale);
    return hipGetLastError();
  }
  const int NB = NQB;
  uint16_t *vt = static_cast<uint16_t *>(a.ws);
  const int G = a.Hq / a.Hkv;
  const int HG = (G + 3) / 4;
  const int ntasks = a.B * a.Hkv * NQB;
  const int grid = ((ntasks + 7) / 8) * 8 * HG;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  if (a.d == 128) {
    hipLaunchKernelGGL(transpose_v_blocks<128>, dim3(a.B * a.Hkv * NB), dim3(256), 0, st, (const uint16_t *)a.v,
                       vt, a.N, NB);
    hipLaunchKernelGGL(sparse_attn_bf16<128>, dim3(grid), dim3(256), 0, st, (const uint16_t *)a.q,
                       (const uint16_t *)a.k, vt, a.idx, (uint16_t *)a.o, a.Hq, a.Hkv, a.N, NQB, a.n_sel, HG,
                       ntasks, scale_log2);
  } else {
    hipLaunchKernelGGL(transpose_v_blocks<64>, dim3(a.B * a.Hkv * NB), dim3(256), 0, st, (const uint16_t *)a.v, vt,
                       a.N, NB);
    hipLaunchKernelGGL(sparse_attn_bf16<64>, dim3(grid), dim3(256), 0, st, (const uint16_t *)a.q,
                       (const uint16_t *)a.k, vt, a.idx, (uint16_t *)a.o, a.Hq, a.Hkv, a.N, NQB, a.n_sel, HG,
                       ntasks, scale_log2);
  }
  return hipGetLastError();
}

}  // namespace sala
