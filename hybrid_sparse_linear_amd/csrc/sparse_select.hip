// Block selection for the InfLLM-V2-style sparse layer (gfx950).
//
// The sparse layers add no parameters and reach the whole context while the
// full KV cache is kept (MiniCPM-SALA, gist.science (ja) 技術概要 sections 1
// and 2.1; gist.science (de) section 2, "Architektur-Hybridisierung"); block
// selection of this family scores coarse block representations (PHSA
// abstract, fugumt.com, arXiv 2601.02819).  Reading implemented here:
//   kbar_j = mean of block j's keys;  qbar_i = mean over the GQA group's query
//   heads and the tokens of query block i;  score = qbar_i . kbar_j / sqrt(d);
//   chosen = forced {0..n_init-1} U {i-n_local+1..i}  U  top-k of the complete
//   blocks strictly between (ties -> smaller index), ascending, -1 padded.
//
// Kernels:
//   pool_rows       block means of K (fp32 out) and group/block means of Q
//   score_tiles     prefill scores: 64x64 fp32 tiles of Qbar Kbar^T, lower triangle only
//   score_decode    decode scores: one pooled query against every pooled key block
//   select_rows     per row: 4-pass radix select of the k-th largest fp32 key,
//                   index-ordered tie break, then the ascending write-out
//   score_decode_top64 + select_decode_final
//                   decode with top-k <= 64: exact local top-64 per 256 blocks
//                   (wave bitonic sort and merges), then a tree of top-64
//                   merges per row -- no contended histogram atomics

#include "sala_common.hpp"
#include "sala_launch.hpp"

namespace sala {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16
  static constexpr int PER16 = 8;
  __device__ static void unpack(const u32x4 &x, float *f) {
#pragma unroll
    for (int p = 0; p < 4; ++p) { f[2 * p] = bf16lo(x[p]); f[2 * p + 1] = bf16hi(x[p]); }
  }
};
template <>
struct Elem<float> {
  static constexpr int PER16 = 4;
  __device__ static void unpack(const u32x4 &x, float *f) {
#pragma unroll
    for (int p = 0; p < 4; ++p) f[p] = __uint_as_float(x[p]);
  }
};

// Mean of `nrows` rows of length d; row r lives at src(r).  256 threads.
// Writes the fp32 mean to dst[0..d).  NT: the rows are read with the
// non-temporal hint (query rows, read once here; key rows are left in the
// caches for the attention kernel's gathers).
template <typename T, bool NT, typename RowPtr>
__device__ void mean_rows(RowPtr src, int nrows, int d, float *dst, float *red /* 256*8 floats */) {
  constexpr int E = Elem<T>::PER16;
  const int cpr = d / E;  // 16-byte chunks per row
  const int slots = 256 / cpr;
  const int tid = threadIdx.x, c = tid % cpr, r0 = tid / cpr;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int r = r0; r < nrows; r += slots) {
    float f[E];
    const u32x4 *p = reinterpret_cast<const u32x4 *>(src(r) + c * E);
    Elem<T>::unpack(NT ? __builtin_nontemporal_load(p) : *p, f);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += f[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[r0 * d + c * E + e] = acc[e];
  __syncthreads();
  if (tid < d) {
    float s = 0.f;
    for (int r = 0; r < slots; ++r) s += red[r * d + tid];
    dst[tid] = s / (float)nrows;
  }
}

// grid.x = B*Hkv*NBp (key blocks kb0 .. kb0+NBp-1, when k != null) + B*Hkv*NQB
// (query blocks, prefill).  k rows hold Lc tokens (L valid); kbar rows hold
// NBs pooled blocks.
template <typename T>
__global__ __launch_bounds__(256) void pool_rows(const T *__restrict__ q, const T *__restrict__ k,
                                                 float *__restrict__ kbar, float *__restrict__ qbar, int Hq,
                                                 int Hkv, int Nq, int L, int Lc, int d, int block, int n_kblocks_total,
                                                 int NBp, int kb0, int NBs, int NQB) {
  __shared__ float red[256 * 8];
  const int bid = blockIdx.x;
  if (bid < n_kblocks_total) {
    const int bh = bid / NBp, j = kb0 + bid % NBp;
    const int cnt = min(block, L - j * block);
    const T *base = k + ((size_t)bh * Lc + (size_t)j * block) * d;
    mean_rows<T, false>([&](int r) { return base + (size_t)r * d; }, cnt, d, kbar + ((size_t)bh * NBs + j) * d,
                        red);
  } else {
    const int id = bid - n_kblocks_total;
    const int bh = id / NQB, i = id % NQB;  // bh = b*Hkv + h
    const int b = bh / Hkv, h = bh % Hkv, G = Hq / Hkv;
    const int cnt = min(block, Nq - i * block);
    const T *base = q + ((size_t)(b * Hq + h * G) * Nq + (size_t)i * block) * d;
    mean_rows<T, true>([&](int r) { return base + ((size_t)(r / cnt) * Nq + (r % cnt)) * d; }, G * cnt, d,
                       qbar + ((size_t)bh * NQB + i) * d, red);
  }
}

// Decode step: token pos of every (b, KV head) is written into the caches
// (rows of Lc tokens), and the pooled key of its block becomes the mean of the
// block's tokens 0 .. pos (the new one taken from k_new), summed in the same
// order as pool_rows, so it equals a full re-pool of the cache bit for bit.
template <typename T>
__global__ __launch_bounds__(256) void kv_append(const T *__restrict__ k_new, const T *__restrict__ v_new,
                                                 T *__restrict__ kc, T *__restrict__ vc, float *__restrict__ kbar,
                                                 int Lc, int NBs, int d, int block, int pos) {
  __shared__ float red[256 * 8];
  constexpr int E = Elem<T>::PER16;
  const int bh = blockIdx.x, tid = threadIdx.x, cpr = d / E;
  const T *kn = k_new + (size_t)bh * d;
  const T *vn = v_new + (size_t)bh * d;
  T *krow = kc + ((size_t)bh * Lc + pos) * d;
  T *vrow = vc + ((size_t)bh * Lc + pos) * d;
  if (tid < cpr) gstore16(krow + tid * E, gload16(kn + tid * E));
  else if (tid < 2 * cpr) gstore16(vrow + (tid - cpr) * E, gload16(vn + (tid - cpr) * E));
  const int j = pos / block, first = j * block, cnt = pos - first + 1;
  const T *base = kc + ((size_t)bh * Lc + first) * d;
  mean_rows<T, false>([&](int r) { return r == cnt - 1 ? kn : base + (size_t)r * d; }, cnt, d,
                      kbar + ((size_t)bh * NBs + j) * d, red);
}

// scores[bh][i][j] = (qbar_i . kbar_j) * inv_sqrt_d for the 64x64 tiles of
// query blocks i (local; global qb0 + i) against key blocks j that are not
// entirely after them.  nTk == 0: qb0 == 0 and a triangular grid of tiles
// J <= I; otherwise a rectangular grid of nTk key tiles per query tile whose
// tiles past the diagonal exit at once.  kbar rows hold NBs pooled blocks.
__global__ __launch_bounds__(256) void score_tiles(const float *__restrict__ qbar, const float *__restrict__ kbar,
                                                   float *__restrict__ scores, int NQB, int NB, int NBs, int qb0,
                                                   int nTk, int d, float inv_sqrt_d) {
  // rows padded to 132 floats: 16-byte aligned for the float4 reads below, and
  // 16 consecutive rows start 4 banks apart, so a wave's float4 reads of 16
  // rows cover the 64 banks once
  __shared__ __attribute__((aligned(16))) float qs[64][132];
  __shared__ __attribute__((aligned(16))) float ks[64][132];
  const int T = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  int I, J;
  if (nTk == 0) {
    I = (int)((sqrtf(8.f * (float)T + 1.f) - 1.f) * 0.5f);
    while ((I + 1) * (I + 2) / 2 <= T) ++I;
    while (I * (I + 1) / 2 > T) --I;
    J = T - I * (I + 1) / 2;
  } else {
    I = T / nTk;
    J = T % nTk;
    if (64 * J > qb0 + 64 * I + 63) return;  // every key block after every query block of the tile
  }
  const float *qb = qbar + ((size_t)bh * NQB + 64 * I) * d;
  const float *kb = kbar + ((size_t)bh * NBs + 64 * J) * d;
  const int d4 = d / 4;
  for (int e = tid; e < 64 * d4; e += 256) {
    const int r = e / d4, c = 4 * (e % d4);
    const float4 zero = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<float4 *>(&qs[r][c]) =
        (64 * I + r < NQB) ? *reinterpret_cast<const float4 *>(qb + (size_t)r * d + c) : zero;
    *reinterpret_cast<float4 *>(&ks[r][c]) =
        (64 * J + r < NB) ? *reinterpret_cast<const float4 *>(kb + (size_t)r * d + c) : zero;
  }
  __syncthreads();
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  // four features per LDS read; each accumulator still sums kk = 0, 1, 2, ... in order
  for (int kk = 0; kk < d; kk += 4) {
    float4 a[4], bb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = *reinterpret_cast<const float4 *>(&qs[ty + 16 * r][kk]);
#pragma unroll
    for (int c = 0; c < 4; ++c) bb[c] = *reinterpret_cast<const float4 *>(&ks[tx + 16 * c][kk]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[r][c] = fmaf(a[r].x, bb[c].x, acc[r][c]);
        acc[r][c] = fmaf(a[r].y, bb[c].y, acc[r][c]);
        acc[r][c] = fmaf(a[r].z, bb[c].z, acc[r][c]);
        acc[r][c] = fmaf(a[r].w, bb[c].w, acc[r][c]);
      }
  }
  float *out = scores + (size_t)bh * NQB * NB;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 64 * I + ty + 16 * r;
    if (i >= NQB) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 64 * J + tx + 16 * c;
      if (j < NB) out[(size_t)i * NB + j] = acc[r][c] * inv_sqrt_d;
    }
  }
}

// Decode: qbar = mean of the G query heads of KV head h; scores for 256 key
// blocks per workgroup.  8 lanes per key block, 128-byte coalesced reads.
template <typename T>
__global__ __launch_bounds__(256) void score_decode(const T *__restrict__ q, const float *__restrict__ kbar,
                                                    float *__restrict__ scores, int Hq, int Hkv, int NB, int NBs,
                                                    int d, float inv_sqrt_d) {
  __shared__ float qm[128];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv, G = Hq / Hkv, tid = threadIdx.x;
  if (tid < d) {
    float s = 0.f;
    for (int g = 0; g < G; ++g) {
      const size_t off = ((size_t)(b * Hq + h * G + g)) * d + tid;
      if constexpr (sizeof(T) == 2) s += bf16_to_f32(q[off]);
      else s += q[off];
    }
    qm[tid] = s / (float)G;
  }
  __syncthreads();
  const int grp = tid >> 3, l8 = tid & 7;
  const int nv = d / 32;  // float4 pieces per lane
  float qr[16];
  for (int vv = 0; vv < nv; ++vv)
#pragma unroll
    for (int e = 0; e < 4; ++e) qr[4 * vv + e] = qm[32 * vv + 4 * l8 + e];
  const float *kb = kbar + (size_t)bh * NBs * d;  // NBs: pooled blocks per row of kbar (capacity)
  for (int u = 0; u < 8; ++u) {
    const int j = blockIdx.x * 256 + grp + 32 * u;
    float acc = 0.f;
    if (j < NB) {
      for (int vv = 0; vv < nv; ++vv) {
        const float4 x = *reinterpret_cast<const float4 *>(kb + (size_t)j * d + 32 * vv + 4 * l8);
        acc = fmaf(x.x, qr[4 * vv], acc);
        acc = fmaf(x.y, qr[4 * vv + 1], acc);
        acc = fmaf(x.z, qr[4 * vv + 2], acc);
        acc = fmaf(x.w, qr[4 * vv + 3], acc);
      }
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 4, 64);
    if (l8 == 0 && j < NB) scores[(size_t)bh * NB + j] = acc * inv_sqrt_d;
  }
}

template <int NT>
__device__ int block_excl_scan(int v, int *tmp, int &total) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < NW; ++w) { const int t = tmp[w]; tmp[w] = run; run += t; }
    tmp[NW] = run;
  }
  __syncthreads();
  const int res = x - v + tmp[wid];
  total = tmp[NW];
  __syncthreads();
  return res;
}

// One workgroup per selection row.  rows_per_bh = NQB (prefill) or 1 (decode).
template <int NT, int MAXC>
__global__ __launch_bounds__(NT) void select_rows(const float *__restrict__ scores, int32_t *__restrict__ idx,
                                                  int rows_per_bh, int NB, int L, int block, int topk,
                                                  int n_init, int n_local, int fixed_i, int qb0) {
  __shared__ uint32_t keys[MAXC];
  __shared__ int hist[256];
  __shared__ int tmp[NT / 64 + 1];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_above;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;  // bh * rows_per_bh + r
  const int bh = row / rows_per_bh, r = row % rows_per_bh;
  const int i = (fixed_i >= 0) ? fixed_i : qb0 + r;  // global query block
  const int width = topk + n_init + n_local;
  const float *srow = scores + ((size_t)bh * rows_per_bh + r) * NB;
  int32_t *out = idx + (size_t)row * width;

  const int nfull = L / block;
  const int lo = n_init;
  const int hi = min(i - n_local, nfull - 1);
  const int ncand = max(0, hi - lo + 1);
  const int kk = min(topk, ncand);
  const bool in_lds = ncand <= MAXC;

  auto key_at = [&](int jj) -> uint32_t { return in_lds ? keys[jj] : float_key(srow[lo + jj]); };

  uint32_t thr = 0;  // the kk-th largest key
  int rem = 0;       // how many keys equal to thr are taken
  const bool take_all = (kk == ncand);
  if (!take_all && kk > 0) {
    if (in_lds)
      for (int jj = tid; jj < ncand; jj += NT) keys[jj] = float_key(srow[lo + jj]);
    uint32_t prefix = 0, pmask = 0;
    rem = kk;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int bb = tid; bb < 256; bb += NT) hist[bb] = 0;
      __syncthreads();
      for (int jj = tid; jj < ncand; jj += NT) {
        const uint32_t key = key_at(jj);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane owns bins 255-4*lane .. 252-4*lane (descending digit order)
        int c[4], s = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) { c[e] = hist[255 - 4 * tid - e]; s += c[e]; }
        int incl = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o, 64);
          if (tid >= o) incl += y;
        }
        int above = incl - s;  // keys with a larger digit (in lanes before this one)
        if (above < rem && rem <= incl) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (above < rem && rem <= above + c[e]) { sh_digit = 255u - 4u * tid - e; sh_above = above; }
            above += c[e];
          }
        }
      }
      __syncthreads();
      prefix |= sh_digit << shift;
      pmask |= 255u << shift;
      rem -= sh_above;
      __syncthreads();
    }
    thr = prefix;
  }

  // positions: [forced low][picks ascending][forced high][-1 ...]
  const int nlow = min(n_init, i + 1);
  const int hstart = max(n_init, i - n_local + 1);
  const int nhigh = max(0, i - hstart + 1);
  const int per = (ncand + NT - 1) / NT;
  const int j0 = tid * per, j1 = min(ncand, j0 + per);
  int total;
  if (take_all) {
    for (int jj = j0; jj < j1; ++jj) out[nlow + jj] = lo + jj;
  } else if (kk > 0) {
    int neq = 0;
    for (int jj = j0; jj < j1; ++jj) neq += (key_at(jj) == thr);
    const int eq_before = block_excl_scan<NT>(neq, tmp, total);
    int npk = 0, e = eq_before;
    for (int jj = j0; jj < j1; ++jj) {
      const uint32_t key = key_at(jj);
      if (key > thr) ++npk;
      else if (key == thr) { if (e < rem) ++npk; ++e; }
    }
    const int pk_before = block_excl_scan<NT>(npk, tmp, total);
    int pos = nlow + pk_before;
    e = eq_before;
    for (int jj = j0; jj < j1; ++jj) {
      const uint32_t key = key_at(jj);
      bool take = key > thr;
      if (key == thr) { take = e < rem; ++e; }
      if (take) out[pos++] = lo + jj;
    }
  }
  for (int t = tid; t < width; t += NT) {
    if (t < nlow) out[t] = t;
    else if (t >= nlow + kk && t < nlow + kk + nhigh) out[t] = hstart + (t - nlow - kk);
    else if (t >= nlow + kk + nhigh) out[t] = -1;
  }
}

// ---------------------------------------------------------------- decode selection, two exact levels
// Packed 64-bit candidate key: order-preserving score key in the high word,
// inverted block index in the low word, so a larger key is a better block
// and equal scores rank the smaller index first.  0 marks "not a candidate".
__device__ __forceinline__ uint64_t pack_key(float score, int j) {
  return ((uint64_t)float_key(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}
// Value of lane l ^ m.  m is a constant after unrolling, and every case is a
// VALU lane exchange: m <= 8 are DPP moves (xor 4 = row half-mirror then quad
// permutation [3,2,1,0]; xor 8 = row rotate by 8); m = 16 and 32 take the
// partner's row from v_permlane16_swap / v_permlane32_swap, which (with both
// operands v) return the lower and the upper row of each row pair.  The lane
// maps were checked on gfx950 with probes.
__device__ __forceinline__ uint32_t shfl_xor32(uint32_t v, int m) {
  const int x = (int)v;
  const int lane = __lane_id();
  switch (m) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
    case 4: {
      const int h = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_update_dpp(0, h, 0x1B, 0xF, 0xF, false);
    }
    case 8: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);
    case 16: {
      const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (lane & 16) ? p[0] : p[1];
    }
    default: {  // 32
      const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (lane & 32) ? p[0] : p[1];
    }
  }
}
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = shfl_xor32((uint32_t)v, m), hi = shfl_xor32((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
// Descending bitonic sort of one key per lane across a wave.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t o = shfl_xor64(x, j);
      const bool keep_max = ((lane & k) == 0) == ((lane & j) == 0);
      x = keep_max ? (x > o ? x : o) : (x < o ? x : o);
    }
  return x;
}
// a (this lane's element of a descending list) and b[] (another descending
// list of 64 in LDS): the top 64 of their union, descending.
__device__ __forceinline__ uint64_t wave_merge_top(uint64_t a, const uint64_t *b, int lane) {
  const uint64_t bb = b[63 - lane];
  uint64_t x = a > bb ? a : bb;
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) {
    const uint64_t o = shfl_xor64(x, j);
    x = ((lane & j) == 0) ? (x > o ? x : o) : (x < o ? x : o);
  }
  return x;
}

// Level 1: scores of 256 pooled blocks against the group-pooled query, and
// their exact local top-64 (descending packed keys) written to tops.
template <typename T, int d>
__global__ __launch_bounds__(256) void score_decode_top64(const T *__restrict__ q, const float *__restrict__ kbar,
                                                          float *__restrict__ scores, uint64_t *__restrict__ tops,
                                                          int Hq, int Hkv, int NB, int NBs, float inv_sqrt_d,
                                                          int lo, int hi) {
  __shared__ float qm[128];
  __shared__ float qpart[256];
  __shared__ float sc[256];
  __shared__ uint64_t lists[3][64];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv, G = Hq / Hkv, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int grp = tid >> 3, l8 = tid & 7;
  constexpr int nv = d / 32;  // float4 pieces per lane per pooled key
  const float *kb = kbar + (size_t)bh * NBs * d;  // NBs: pooled blocks per row of kbar (capacity)
  // block of local slot (u, grp): the u-th loads of all workgroups of a row
  // cover one contiguous run of 32 * gridDim.x blocks, so the HBM channels see
  // an even spread at every moment.  Any partition keeps the two levels exact.
  const int nchunk = gridDim.x, x = blockIdx.x;
  auto blk = [&](int u, int g) { return (u * nchunk + x) * 32 + g; };
  // all 8 x nv pooled-key loads of this lane go out first, the query loads
  // right behind them: one round trip for both
  float4 xs[8][nv];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int j = min(blk(u, grp), NB - 1);
#pragma unroll
    for (int vv = 0; vv < nv; ++vv) xs[u][vv] = *reinterpret_cast<const float4 *>(kb + (size_t)j * d + 32 * vv + 4 * l8);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the key loads ahead of the query loads
  constexpr int P = 256 / d;   // the G heads are split over P thread groups per dimension
  constexpr int QPT = 32 / P;  // heads per thread loaded up front (all of them for G <= 32)
  const int qc = tid % d, qp = tid / d;
  float qv[QPT];
  const T *qb = q + (size_t)(b * Hq + h * G) * d + qc;
  {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int g = min(qp + P * i, G - 1);
      if constexpr (sizeof(T) == 2) qv[i] = bf16_to_f32(qb[(size_t)g * d]);
      else qv[i] = qb[(size_t)g * d];
    }
  }
  {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < QPT; ++i) s += (qp + P * i < G) ? qv[i] : 0.f;
    // heads past the first 32 of a larger group, in the same order (i = QPT, ...)
    for (int g = qp + P * QPT; g < G; g += P) {
      if constexpr (sizeof(T) == 2) s += bf16_to_f32(qb[(size_t)g * d]);
      else s += qb[(size_t)g * d];
    }
    qpart[tid] = s;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  if (tid < d) {
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < 256 / d; ++p) s += qpart[p * d + tid];
    qm[tid] = s / (float)G;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  float qr[4 * nv];
#pragma unroll
  for (int vv = 0; vv < nv; ++vv)
#pragma unroll
    for (int e = 0; e < 4; ++e) qr[4 * vv + e] = qm[32 * vv + 4 * l8 + e];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float acc = 0.f;
#pragma unroll
    for (int vv = 0; vv < nv; ++vv) {
      acc = fmaf(xs[u][vv].x, qr[4 * vv], acc);
      acc = fmaf(xs[u][vv].y, qr[4 * vv + 1], acc);
      acc = fmaf(xs[u][vv].z, qr[4 * vv + 2], acc);
      acc = fmaf(xs[u][vv].w, qr[4 * vv + 3], acc);
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 4, 64);
    const int jl = grp + 32 * u, jg = blk(u, grp);
    if (l8 == 0) {
      sc[jl] = acc * inv_sqrt_d;
      if (scores && jg < NB) scores[(size_t)bh * NB + jg] = acc * inv_sqrt_d;
    }
  }
  __syncthreads();
  const int j = blk(tid >> 5, tid & 31);
  uint64_t key = (j >= lo && j <= hi) ? pack_key(sc[tid], j) : 0ull;
  key = wave_sort_desc(key, lane);
  if (w & 1) lists[w >> 1][lane] = key;  // waves 1 and 3 hand their lists over
  __syncthreads();
  if (w == 0 || w == 2) key = wave_merge_top(key, lists[w >> 1], lane);
  if (w == 2) lists[2][lane] = key;
  __syncthreads();
  if (w == 0) {
    key = wave_merge_top(key, lists[2], lane);
    tops[((size_t)bh * nchunk + x) * 64 + lane] = key;
  }
}

// Level 2 (one workgroup per row): the top 64 of a union is the top 64 of the
// union of the parts' top 64s, so the row's sorted local lists are merged
// pairwise (wave_merge_top) in a tree until one list is left; its first
// min(topk, candidates) keys are the picks.  Output: forced low blocks,
// picks ascending, forced high blocks, -1 padding.
__global__ __launch_bounds__(1024) void select_decode_final(const uint64_t *__restrict__ tops, int32_t *__restrict__ idx,
                                                            int nchunk, int topk, int n_init, int n_local, int i,
                                                            int ncand) {
  __shared__ uint64_t lists[2][64][64];
  __shared__ uint32_t pick_idx[64];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t *t = tops + (size_t)row * nchunk * 64;
  const int width = topk + n_init + n_local;
  int32_t *out = idx + (size_t)row * width;
  const int kk = min(topk, ncand);
  int n = 1;
  while (n < nchunk) n <<= 1;  // lists padded to a power of two with empty lists
  {  // every load in flight at once (n * 64 <= 4096 keys, four per thread)
    uint64_t tv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 1024 * u;
      tv[u] = ((e >> 6) < nchunk) ? t[e] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 1024 * u;
      if (e < n * 64) lists[0][e >> 6][e & 63] = tv[u];
    }
  }
  __syncthreads();
  int cur = 0;
  for (; n > 1; n >>= 1) {
    for (int m = w; m < n / 2; m += 16)
      lists[cur ^ 1][m][lane] = wave_merge_top(lists[cur][2 * m][lane], lists[cur][2 * m + 1], lane);
    __syncthreads();
    cur ^= 1;
  }
  if (tid < 64) pick_idx[tid] = 0xFFFFFFFFu - (uint32_t)(lists[cur][0][tid] & 0xFFFFFFFFull);
  __syncthreads();
  const int nlow = min(n_init, i + 1);
  const int hstart = max(n_init, i - n_local + 1);
  const int nhigh = max(0, i - hstart + 1);
  if (tid < kk) {
    const uint32_t me = pick_idx[tid];
    int pos = 0;
    for (int r = 0; r < kk; ++r) pos += pick_idx[r] < me;
    out[nlow + pos] = (int32_t)me;
  }
  for (int x = tid; x < width; x += 1024) {
    if (x < nlow) out[x] = x;
    else if (x >= nlow + kk && x < nlow + kk + nhigh) out[x] = hstart + (x - nlow - kk);
    else if (x >= nlow + kk + nhigh) out[x] = -1;
  }
}

}  // namespace

size_t sparse_select_workspace(int dtype, int B, int Hq, int Hkv, int d, int Nq, int L, int block, int topk,
                               int n_init, int n_local, bool want_scores) {
  (void)dtype; (void)Hq; (void)topk; (void)n_init; (void)n_local;
  const size_t NB = (size_t)(L + block - 1) / block;
  const size_t NQB = (Nq == 1) ? 1 : (size_t)(Nq + block - 1) / block;
  size_t bytes = 0;
  if (Nq != 1) bytes += (size_t)B * Hkv * NQB * d * sizeof(float);             // qbar
  if (Nq == 1 && topk <= 64 && (NB + 255) / 256 * 64 <= 4096) {
    bytes += (size_t)B * Hkv * ((NB + 255) / 256) * 64 * sizeof(uint64_t);    // local top-64 lists
  } else if (!want_scores) {
    bytes += (size_t)B * Hkv * NQB * NB * sizeof(float);                      // scores
  }
  return bytes;
}

// Rows pos0 .. pos0+n-1 of both caches (rows of Lc tokens) from k_new, v_new [BH, n, d].
template <typename T>
__global__ __launch_bounds__(256) void kv_write_rows(const T *__restrict__ k_new, const T *__restrict__ v_new,
                                                     T *__restrict__ kc, T *__restrict__ vc, int Lc, int n, int d,
                                                     int pos0, long long pieces) {
  constexpr int E = Elem<T>::PER16;
  const long long x = (long long)blockIdx.x * 256 + threadIdx.x;
  if (x >= pieces) return;
  const int cpr = d / E;
  const long long row = x / cpr;  // bh * n + r
  const int c = (int)(x % cpr), r = (int)(row % n);
  const long long bh = row / n;
  const size_t dst = ((size_t)bh * Lc + pos0 + r) * d + (size_t)c * E;
  const size_t src = (size_t)row * d + (size_t)c * E;
  gstore16(kc + dst, gload16(k_new + src));
  gstore16(vc + dst, gload16(v_new + src));
}

hipError_t launch_kv_write(int dtype, int BH, int Lc, int d, int pos0, int n, const void *k_new, const void *v_new,
                           void *k_cache, void *v_cache, hipStream_t st) {
  const long long pieces = (long long)BH * n * (d / (dtype == 1 ? 8 : 4));
  const dim3 grid((unsigned)((pieces + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(kv_write_rows<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, (uint16_t *)k_cache, (uint16_t *)v_cache, Lc, n, d, pos0, pieces);
  else
    hipLaunchKernelGGL(kv_write_rows<float>, grid, dim3(256), 0, st, (const float *)k_new, (const float *)v_new,
                       (float *)k_cache, (float *)v_cache, Lc, n, d, pos0, pieces);
  return hipGetLastError();
}

hipError_t launch_kv_append(int dtype, int BH, int Lc, int d, int block, int pos, const void *k_new,
                            const void *v_new, void *k_cache, void *v_cache, float *k_pooled, hipStream_t st) {
  const int NBs = (Lc + block - 1) / block;
  if (dtype == 1)
    hipLaunchKernelGGL(kv_append<uint16_t>, dim3(BH), dim3(256), 0, st, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, (uint16_t *)k_cache, (uint16_t *)v_cache, k_pooled, Lc, NBs, d, block,
                       pos);
  else
    hipLaunchKernelGGL(kv_append<float>, dim3(BH), dim3(256), 0, st, (const float *)k_new, (const float *)v_new,
                       (float *)k_cache, (float *)v_cache, k_pooled, Lc, NBs, d, block, pos);
  return hipGetLastError();
}

hipError_t launch_sparse_select(const SparseSelectArgs &a, hipStream_t st) {
  const int NB = (a.L + a.block - 1) / a.block;
  const int Lc = a.Lc ? a.Lc : a.L;                // k and k_pooled rows are laid out for Lc tokens
  const int NBs = (Lc + a.block - 1) / a.block;
  const bool decode = (a.Nq == 1);
  const int NQB = decode ? 1 : (a.Nq + a.block - 1) / a.block;
  const int qb0 = decode ? 0 : (a.L - a.Nq) / a.block;  // first query block of a continued prefill
  const int BH = a.B * a.Hkv;
  char *ws = static_cast<char *>(a.ws);
  float *qbar = nullptr;
  if (!decode) { qbar = reinterpret_cast<float *>(ws); ws += (size_t)BH * NQB * a.d * sizeof(float); }
  float *scores = a.scores ? a.scores : reinterpret_cast<float *>(ws);
  const float inv_sqrt_d = 1.0f / sqrtf((float)a.d);

  // key blocks to pool: all of them, or (continued prefill) those the query chunk fills
  const int kb0 = decode ? 0 : qb0;
  const int NBp = NB - kb0;
  const int nk = a.k ? BH * NBp : 0;
  const int nq = decode ? 0 : BH * NQB;
  if (nk + nq > 0) {
    if (a.dtype == 1)
      hipLaunchKernelGGL(pool_rows<uint16_t>, dim3(nk + nq), dim3(256), 0, st, (const uint16_t *)a.q,
                         (const uint16_t *)a.k, a.k_pooled, qbar, a.Hq, a.Hkv, a.Nq, a.L, Lc, a.d, a.block, nk, NBp,
                         kb0, NBs, NQB);
    else
      hipLaunchKernelGGL(pool_rows<float>, dim3(nk + nq), dim3(256), 0, st, (const float *)a.q,
                         (const float *)a.k, a.k_pooled, qbar, a.Hq, a.Hkv, a.Nq, a.L, Lc, a.d, a.block, nk, NBp,
                         kb0, NBs, NQB);
  }
  if (!decode) {
    const int nTq = (NQB + 63) / 64;
    if (qb0 == 0) {
      hipLaunchKernelGGL(score_tiles, dim3(nTq * (nTq + 1) / 2, BH), dim3(256), 0, st, qbar, a.k_pooled, scores,
                         NQB, NB, NBs, 0, 0, a.d, inv_sqrt_d);
    } else {
      const int nTk = (NB + 63) / 64;
      hipLaunchKernelGGL(score_tiles, dim3(nTq * nTk, BH), dim3(256), 0, st, qbar, a.k_pooled, scores, NQB, NB,
                         NBs, qb0, nTk, a.d, inv_sqrt_d);
    }
    // candidate keys held in LDS: 16 KiB up to 4096 blocks (more workgroups per CU), else 32 KiB
    if (NB <= 4096)
      hipLaunchKernelGGL((select_rows<256, 4096>), dim3(BH * NQB), dim3(256), 0, st, scores, a.idx, NQB, NB, a.L,
                         a.block, a.topk, a.n_init, a.n_local, -1, qb0);
    else
      hipLaunchKernelGGL((select_rows<256, 8192>), dim3(BH * NQB), dim3(256), 0, st, scores, a.idx, NQB, NB, a.L,
                         a.block, a.topk, a.n_init, a.n_local, -1, qb0);
  } else if (a.topk <= 64 && (NB + 255) / 256 * 64 <= 4096) {
    // two exact levels: local top-64 per 256 blocks, then threshold + rank per row
    const int nchunk = (NB + 255) / 256;
    uint64_t *tops = reinterpret_cast<uint64_t *>(ws);
    const int i = (a.L - 1) / a.block;
    const int lo = a.n_init, hi = min(i - a.n_local, a.L / a.block - 1);
    const int ncand = max(0, hi - lo + 1);
#define SALA_SCORE_TOP64(T, DD)                                                                                  \
  hipLaunchKernelGGL((score_decode_top64<T, DD>), dim3(nchunk, BH), dim3(256), 0, st, (const T *)a.q, a.k_pooled,   \
                     a.scores, tops, a.Hq, a.Hkv, NB, NBs, inv_sqrt_d, lo, hi)
    if (a.dtype == 1 && a.d == 128) SALA_SCORE_TOP64(uint16_t, 128);
    else if (a.dtype == 1) SALA_SCORE_TOP64(uint16_t, 64);
    else if (a.d == 128) SALA_SCORE_TOP64(float, 128);
    else SALA_SCORE_TOP64(float, 64);
#undef SALA_SCORE_TOP64
    hipLaunchKernelGGL(select_decode_final, dim3(BH), dim3(1024), 0, st, tops, a.idx, nchunk, a.topk, a.n_init,
                       a.n_local, i, ncand);
  } else {
    if (a.dtype == 1)
      hipLaunchKernelGGL(score_decode<uint16_t>, dim3((NB + 255) / 256, BH), dim3(256), 0, st,
                         (const uint16_t *)a.q, a.k_pooled, scores, a.Hq, a.Hkv, NB, NBs, a.d, inv_sqrt_d);
    else
      hipLaunchKernelGGL(score_decode<float>, dim3((NB + 255) / 256, BH), dim3(256), 0, st, (const float *)a.q,
                         a.k_pooled, scores, a.Hq, a.Hkv, NB, NBs, a.d, inv_sqrt_d);
    hipLaunchKernelGGL((select_rows<1024, 16384>), dim3(BH), dim3(1024), 0, st, scores, a.idx, 1, NB, a.L,
                       a.block, a.topk, a.n_init, a.n_local, (a.L - 1) / a.block, 0);
  }
  return hipGetLastError();
}

}  // namespace sala
