// Gradients of block-sparse softmax attention at a fixed selection (gfx950).
//
// For query head hq (KV head hq/G), token t of query block i, its token set
// A(t) = { s in the blocks listed in idx[b, hq/G, i] : s <= t }, the forward
// p = softmax_s(scale q_t . k_s) over A(t), o_t = sum_s p_s v_s.  Given
// dO = dL/do the chain rule gives, with D_t = dO_t . o_t = sum_s p_s dO_t . v_s,
//   ds_s = p_s (dO_t . v_s - D_t)
//   dq_t = scale sum_{s in A(t)} ds_s k_s
//   dk_s = scale sum_{(t, hq): s in A(t)} ds_s q_t     (over the group's heads)
//   dv_s = sum_{(t, hq): s in A(t)} p_s dO_t
// The hybrid model is trained from a pretrained Transformer by continual
// training (MiniCPM-SALA abstract; gist.science (ja) 技術概要 section 2.3;
// gist.science (de) section 2, "Trainingsstrategie"), which needs these
// gradients; the selection itself is a top-k and passes no gradient.
//
// Passes (bf16 inputs, bf16 MFMA 16x16x32 with fp32 accumulation):
//   sparse_bwd_dq    one workgroup = 8 waves = 4 query heads of a group x the
//                    64 rows of one query block (a wave: one head, two 16-row
//                    tiles, each K / V fragment read from LDS feeding both).  A first sweep over the selected blocks forms each
//                    row's log-sum-exp (log2 units) and D_t = sum_s p_s dP_s
//                    online from the fp32 scores, so that the row's dS sums to
//                    zero up to fp32 rounding (D_t from a bf16-rounded output
//                    would leave an error of that rounding on rows whose
//                    attention is peaked, where dq itself is small); a second
//                    forms S^T = K Q^T, dP^T = V dO^T, dS and dQ^T += K^T dS^T.
//                    It writes the log-sum-exp and D_t for the next pass.
//   bwd_mark / bwd_lists
//                    the inverse of the selection: a bitmap of (key block j,
//                    query block i) pairs, then per key block the list of the
//                    query blocks that selected it in increasing order, cut
//                    into work items of at most ITEM_QB query blocks.
//   sparse_bwd_dkv   one workgroup per work item (2 waves, two 16-key tiles of
//                    block j each, K and V rows held as MFMA operands): for
//                    every (query block, head) of the item, Q and dO rows are
//                    staged in LDS and S = Q K^T, dP = dO V^T, dV^T += dO^T P,
//                    dK^T += Q^T dS accumulate; the item's sums go to its own
//                    fp32 slot.
//   bwd_reduce       per key block: its items' slots summed in item order, then
//                    rounded once to bf16 (blocks no query block selected get 0).
// Every sum runs in a fixed order, so results are the same from run to run.

#include "sala_common.hpp"
#include "sala_launch.hpp"

namespace sala {
namespace {

constexpr int BB = 64;        // tokens per block
constexpr int ITEM_QB = 64;   // query blocks per work item of the dk/dv pass

template <int D>
struct BwCfg {
  static constexpr int NDS = D / 32;       // 32-deep feature steps
  static constexpr int ND = D / 16;        // 16-wide feature tiles
  static constexpr int NCH = D / 8;        // 16-byte chunks per row
  static constexpr int ROWB = D * 2;       // bytes per row
  static constexpr int TB = BB * D * 2;    // bytes of one 64-row tile
};

// Byte offset in LDS of 16-byte chunk ch of row r of a 64-row tile in the
// natural layout with the fkv row swizzle (conflict-free for plain reads of
// the 16 rows of a key pair and for transposed reads).
template <int D>
__device__ __forceinline__ uint32_t tile_off(uint32_t r, uint32_t ch) {
  return r * BwCfg<D>::ROWB + ((ch ^ fkv(r)) & (uint32_t)(BwCfg<D>::NCH - 1)) * 16u;
}

// Direct loads of a 64-row tile (rows from `base`, rows at or past `valid`
// read as zero) into LDS at `dst` in the tile_off layout, by NT threads.
template <int D, int NT>
__device__ __forceinline__ void load_tile(const uint16_t *base, int valid_rows, char *dst, int tid) {
  using Cf = BwCfg<D>;
  constexpr int PER = Cf::TB / 16 / NT;
  // the row count through readfirstlane: a clamp the compiler puts on the VALU
  // would make the resource look divergent (a waterfall loop around every load)
  const uint32_t rows = (uint32_t)__builtin_amdgcn_readfirstlane(min(max(valid_rows, 0), BB));
  const auto r = buf_rsrc(base, rows * D * 2u);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int p = NT * u + tid;  // LDS slot (16 bytes) of this lane
    const int row = p / Cf::NCH, ch = p % Cf::NCH;
    const uint32_t src = (uint32_t)(row * D + 8 * (ch ^ (int)(fkv(row) & (Cf::NCH - 1)))) * 2u;
    bload16_lds(r, dst + (NT * u + 64 * wv) * 16, src);
  }
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ------------------------------------------------------------------ dq pass
// FOLD (scale > 0): scores stay unscaled and scale * log2(e) is folded into the
// fma that subtracts each reference, and the factor `scale` of dS into the
// log-sum-exp (P scale = 2^(s - (lse - log2 scale))), two VALU operations
// fewer per score in the second sweep and one in the first.  A scale of zero
// or below keeps the scaled scores, whose masked entries are -inf.
template <int D, bool FOLD>
__global__ __launch_bounds__(512) void sparse_bwd_dq(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                     const uint16_t *__restrict__ v,
                                                     const uint16_t *__restrict__ dout,
                                                     const int32_t *__restrict__ idx, uint16_t *__restrict__ dq,
                                                     float *__restrict__ lse2_out, float *__restrict__ drow_out,
                                                     int Hq, int Hkv, int N, int NQB, int n_sel, int HG, int ntasks,
                                                     float scale) {
  using Cf = BwCfg<D>;
  __shared__ __attribute__((aligned(16))) char kb0[Cf::TB], kb1[Cf::TB];
  __shared__ __attribute__((aligned(16))) char vb0[Cf::TB], vb1[Cf::TB];
  __shared__ int sel[1024];
  __shared__ int nvalid_sh, diag_sh;

  // XCD-aware: the HG workgroups of one task share blockIdx % 8
  const int x = blockIdx.x;
  const int slot = x >> 3;
  const int task = (slot / HG) * 8 + (x & 7);
  const int hg = slot % HG;
  if (task >= ntasks) return;
  const int i = task % NQB;
  const int bkv = task / NQB;
  const int b = bkv / Hkv, kvh = bkv % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int hl = 4 * hg + (w & 3);
  const bool active = hl < G;
  const int hq = kvh * G + (active ? hl : 0);
  const int r0 = 32 * (w >> 2);               // this wave's first row in the query block: tiles r0, r0 + 16
  const float scale_log2 = scale * 1.4426950408889634f;

  // block list as in the forward: entries before the first negative one that
  // lie below the query block, in order, and the query's own block last
  if (tid < 64) {
    const int32_t *row = idx + ((size_t)bkv * NQB + i) * n_sel;
    int n = 0;
    bool has_diag = false;
    for (int e0 = 0; e0 < n_sel; e0 += 64) {
      const int e = e0 + tid;
      const int j = (e < n_sel) ? row[e] : -1;
      const uint64_t neg = __ballot(j < 0);
      const bool alive = neg == 0 || tid < __builtin_ctzll(neg);
      const bool keep = alive && j < i;
      const uint64_t kept = __ballot(keep);
      if (keep) sel[n + __builtin_popcountll(kept & ((1ull << tid) - 1))] = j;
      n += __builtin_popcountll(kept);
      has_diag = has_diag || __ballot(alive && j == i) != 0;
      if (neg != 0) break;
    }
    if (tid == 0) {
      if (has_diag) sel[n] = i;
      nvalid_sh = n + (has_diag ? 1 : 0);
      diag_sh = has_diag ? 1 : 0;
    }
  }

  // q and dO fragments (B operands): lane holds row BB*i + r0 + 16a + lr, features 32s + 8lg .. +7
  const size_t rowbase = ((size_t)(b * Hq + hq) * N) * D;
  u32x4 qf[2][Cf::NDS], df[2][Cf::NDS];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int t = BB * i + r0 + 16 * a + lr;
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s) {
      const bool ok = t < N;
      const size_t off = rowbase + (size_t)t * D + 32 * s + 8 * lg;
      qf[a][s] = ok ? gload16(q + off) : u32x4{0, 0, 0, 0};
      df[a][s] = ok ? gload16(dout + off) : u32x4{0, 0, 0, 0};
    }
  }

  __syncthreads();
  const int nvalid = nvalid_sh;
  const bool has_diag = diag_sh != 0;
  const uint16_t *kbase = k + (size_t)bkv * N * D;
  const uint16_t *vbase = v + (size_t)bkv * N * D;
  auto blk = [&](int e) { return __builtin_amdgcn_readfirstlane(sel[e]); };

  // per-lane LDS offsets: plain reads of K / V rows 32p + pair_key(tt, lr)
  // (tt = 0, 1 the two 16-key tiles of a 32-key pair), feature step s
  auto kv_off = [&](int p, int tt, int s) -> uint32_t {
    return tile_off<D>(32 * p + pair_key(tt, lr), 4 * s + lg);
  };
  const uint32_t tr_off = tr_lane_off(l, Cf::ROWB), tr_xor = tr_lane_xor(l);

  // S^T for keys 32p .. 32p+31 of one block: tile [tt][a] holds keys
  // 32p + 8lg + 4tt + e (e = 0..3) of row r0 + 16a + lr, unscaled with FOLD,
  // else in log2 units; masked keys (after the row in the diagonal block, or
  // at or past N) are -inf.  Each K fragment feeds both row tiles.
  auto scores = [&](const char *kbuf, int j, bool diag, int p, f32x4 (&S)[2][2]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int a = 0; a < 2; ++a) S[tt][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const u32x4 A = lds_load<u32x4>(kbuf, kv_off(p, tt, s));
#pragma unroll
        for (int a = 0; a < 2; ++a) S[tt][a] = mfma16x16x32(A, qf[a][s], S[tt][a]);
      }
    if (diag || (j + 1) * BB > N) {  // some key of the block is masked
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = 32 * p + 8 * lg + 4 * tt + e;
            const bool masked = (diag && key > r0 + 16 * a + lr) || (BB * j + key >= N);
            S[tt][a][e] = masked ? -INFINITY : (FOLD ? S[tt][a][e] : S[tt][a][e] * scale_log2);
          }
    } else if constexpr (!FOLD) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int a = 0; a < 2; ++a) S[tt][a] *= scale_log2;
    }
  };

  // dP^T = V dO^T for keys 32p .. 32p+31, tiles as in scores
  auto dprods = [&](const char *vbuf, int p, f32x4 (&dP)[2][2]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int a = 0; a < 2; ++a) dP[tt][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const u32x4 A = lds_load<u32x4>(vbuf, kv_off(p, tt, s));
#pragma unroll
        for (int a = 0; a < 2; ++a) dP[tt][a] = mfma16x16x32(A, df[a][s], dP[tt][a]);
      }
  };

  // The two sweeps walk the block list with K and V double buffered in LDS.
  auto sweep = [&](auto &&body) {
    if (nvalid <= 0) return;
    load_tile<D, 512>(kbase + (size_t)blk(0) * BB * D, N - blk(0) * BB, kb0, tid);
    load_tile<D, 512>(vbase + (size_t)blk(0) * BB * D, N - blk(0) * BB, vb0, tid);
    for (int e = 0; e < nvalid; ++e) {
      wait_vm0();
      __syncthreads();
      const bool odd = e & 1;
      const char *kcur = odd ? kb1 : kb0;
      const char *vcur = odd ? vb1 : vb0;
      if (e + 1 < nvalid) {
        const int jn = blk(e + 1);
        load_tile<D, 512>(kbase + (size_t)jn * BB * D, N - jn * BB, odd ? kb0 : kb1, tid);
        load_tile<D, 512>(vbase + (size_t)jn * BB * D, N - jn * BB, odd ? vb0 : vb1, tid);
      }
      body(kcur, vcur, blk(e), has_diag && e == nvalid - 1);
      __syncthreads();  // every wave is done with kcur / vcur before they are reloaded
    }
  };

  // sweep 1, online over the blocks, per row tile a: the reference m and this
  // lane's parts of lsum = sum 2^(s - m) and dsum = sum 2^(s - m) dP_s.  As in
  // the forward kernel, m moves (to the row max, rescaling the parts) only
  // when a score of the wave lies more than 8 above its row's m, so a term is
  // at most 2^8; the four lanes of a row are added once, after the sweep.
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f}, dsum[2] = {0.f, 0.f};
  sweep([&](const char *kcur, const char *vcur, int j, bool diag) {
    f32x4 S[2][2][2], dP[2][2][2];  // [p][tt][a]
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      scores(kcur, j, diag, p, S[p]);
      dprods(vcur, p, dP[p]);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      float mx = -INFINITY;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) mx = fmaxf(mx, S[p][tt][a][ee]);
      // FOLD: the scale is positive, so the max of the scaled scores is the scaled max
      if (FOLD) mx *= scale_log2;
      if (__any(mx > m[a] + 8.f)) {
        const float mn = fmaxf(m[a], row4_max(mx));
        const float alpha = mn == m[a] ? 1.f : __builtin_amdgcn_exp2f(m[a] - mn);
        lsum[a] *= alpha;
        dsum[a] *= alpha;
        m[a] = mn;
      }
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) {
            const float pe = __builtin_amdgcn_exp2f(FOLD ? fmaf(S[p][tt][a][ee], scale_log2, -m[a]) : S[p][tt][a][ee] - m[a]);
            lsum[a] += pe;
            dsum[a] = fmaf(pe, dP[p][tt][a][ee], dsum[a]);
          }
    }
  });
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    lsum[a] = row4_sum(lsum[a]);
    dsum[a] = row4_sum(dsum[a]);
  }
  // log2 of the row's sum of 2^s, and D_t; a row with no key (a list without
  // its own block) gets +inf, so its P is 0 (the forward gives it a zero output)
  float lse2[2], drow[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    lse2[a] = lsum[a] > 0.f ? m[a] + __builtin_amdgcn_logf(lsum[a]) : INFINITY;
    drow[a] = lsum[a] > 0.f ? dsum[a] / lsum[a] : 0.f;
  }

  // sweep 2, per 32-key half p: dQ^T += K^T dS^T with dS = P (dP - D) scale
  // (FOLD: P scale = 2^(s - (lse - log2 scale)) in one exponential)
  float lse2s[2];
  {
    const float l2s = FOLD ? log2f(scale) : 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a) lse2s[a] = lse2[a] - l2s;
  }
  f32x4 dQ[2][Cf::ND];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int dt = 0; dt < Cf::ND; ++dt) dQ[a][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  sweep([&](const char *kcur, const char *vcur, int j, bool diag) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      f32x4 S[2][2], dP[2][2];
      scores(kcur, j, diag, p, S);
      dprods(vcur, p, dP);
      u32x4 dS[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float ds[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) {
            if constexpr (FOLD) {
              const float prs = __builtin_amdgcn_exp2f(fmaf(S[tt][a][ee], scale_log2, -lse2s[a]));
              ds[tt][ee] = prs * (dP[tt][a][ee] - drow[a]);
            } else {
              const float pr = __builtin_amdgcn_exp2f(S[tt][a][ee] - lse2[a]);
              ds[tt][ee] = pr * (dP[tt][a][ee] - drow[a]) * scale;
            }
          }
        dS[a] = u32x4{pack_bf16x2(ds[0][0], ds[0][1]), pack_bf16x2(ds[0][2], ds[0][3]),
                      pack_bf16x2(ds[1][0], ds[1][1]), pack_bf16x2(ds[1][2], ds[1][3])};
      }
#pragma unroll
      for (int dt = 0; dt < Cf::ND; ++dt) {
        const u32x4 A = tr_frag(kcur, 32 * p * Cf::ROWB, tr_off, tr_xor, dt, Cf::NCH, Cf::ROWB);
#pragma unroll
        for (int a = 0; a < 2; ++a) dQ[a][dt] = mfma16x16x32(A, dS[a], dQ[a][dt]);
      }
    }
  });

  if (!active) return;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int t = BB * i + r0 + 16 * a + lr;
    if (t >= N) continue;
    uint16_t *dqrow = dq + rowbase + (size_t)t * D;
#pragma unroll
    for (int dt = 0; dt < Cf::ND; ++dt)
      *reinterpret_cast<u32x2 *>(dqrow + 16 * dt + 4 * lg) =
          u32x2{pack_bf16x2(dQ[a][dt][0], dQ[a][dt][1]), pack_bf16x2(dQ[a][dt][2], dQ[a][dt][3])};
    if (lg == 0) {
      const size_t r = (size_t)(b * Hq + hq) * N + t;
      lse2_out[r] = lse2[a];
      drow_out[r] = drow[a];
    }
  }
}

// ------------------------------------------------------------------ inverse index
// bitmap[bkv][j][w]: bit (i % 32) of word i / 32 set when query block i selects key block j
__global__ __launch_bounds__(256) void bwd_clear(uint32_t *__restrict__ p, size_t n) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) p[e] = 0u;
}

__global__ __launch_bounds__(256) void bwd_mark(const int32_t *__restrict__ idx, uint32_t *__restrict__ bitmap,
                                                int NQB, int NB, int n_sel, int WPR, long long rows) {
  const long long r = (long long)blockIdx.x * 256 + threadIdx.x;  // one thread per (bkv, i) row of idx
  if (r >= rows) return;
  const int i = (int)(r % NQB);
  const long long bkv = r / NQB;
  const int32_t *row = idx + r * n_sel;
  uint32_t *bm = bitmap + (size_t)bkv * NB * WPR;
  for (int e = 0; e < n_sel; ++e) {
    const int j = row[e];
    if (j < 0) break;
    if (j > i) continue;
    atomicOr(bm + (size_t)j * WPR + (i >> 5), 1u << (i & 31));
  }
}

// One workgroup per bkv: per key block j its count of selecting query blocks,
// the start of its list and of its work items (exclusive scans in j order), and
// the total number of items.  meta[bkv][j] = {list start, count, item start}.
__global__ __launch_bounds__(1024) void bwd_counts(const uint32_t *__restrict__ bitmap, int4 *__restrict__ meta,
                                                   int *__restrict__ nitems, int NB, int WPR) {
  __shared__ int part_l[1024], part_i[1024];
  const int bkv = blockIdx.x, tid = threadIdx.x;
  const uint32_t *bm = bitmap + (size_t)bkv * NB * WPR;
  const int per = (NB + 1023) / 1024;  // key blocks per thread, contiguous
  const int j0 = tid * per;
  int cl = 0, ci = 0;
  for (int j = j0; j < min(NB, j0 + per); ++j) {
    int c = 0;
    for (int w = 0; w < WPR; ++w) c += __popc(bm[(size_t)j * WPR + w]);
    cl += c;
    ci += (c + ITEM_QB - 1) / ITEM_QB;
  }
  part_l[tid] = cl;
  part_i[tid] = ci;
  __syncthreads();
  if (tid == 0) {
    int sl = 0, si = 0;
    for (int u = 0; u < 1024; ++u) {
      const int a = part_l[u], bb = part_i[u];
      part_l[u] = sl;
      part_i[u] = si;
      sl += a;
      si += bb;
    }
    nitems[bkv] = si;
  }
  __syncthreads();
  int sl = part_l[tid], si = part_i[tid];
  for (int j = j0; j < min(NB, j0 + per); ++j) {
    int c = 0;
    for (int w = 0; w < WPR; ++w) c += __popc(bm[(size_t)j * WPR + w]);
    meta[(size_t)bkv * NB + j] = int4{sl, c, si, 0};
    sl += c;
    si += (c + ITEM_QB - 1) / ITEM_QB;
  }
}

// One wave per (bkv, j): the query blocks of row j of the bitmap in increasing
// order into pairs[bkv][start ..], and the items of j into items[bkv][..] as
// {j, list start, length, 0}.
__global__ __launch_bounds__(64) void bwd_lists(const uint32_t *__restrict__ bitmap, const int4 *__restrict__ meta,
                                                int *__restrict__ pairs, int4 *__restrict__ items, int NB, int WPR,
                                                int pairs_per_bkv, int items_per_bkv) {
  const int x = blockIdx.x, lane = threadIdx.x;
  const int bkv = x / NB, j = x % NB;
  const uint32_t *row = bitmap + ((size_t)bkv * NB + j) * WPR;
  const int4 mt = meta[(size_t)bkv * NB + j];
  int *out = pairs + (size_t)bkv * pairs_per_bkv + mt.x;
  int base = 0;
  for (int w0 = 0; w0 < WPR; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t bits = (w < WPR) ? row[w] : 0u;
    const int c = __popc(bits);
    int incl = c;  // inclusive prefix over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int pos = base + incl - c;
    uint32_t bb = bits;
    while (bb) {
      const int bit = __builtin_ctz(bb);
      out[pos++] = 32 * w + bit;
      bb &= bb - 1;
    }
    base += __shfl(incl, 63, 64);
  }
  const int nit = (mt.y + ITEM_QB - 1) / ITEM_QB;
  for (int u = lane; u < nit; u += 64)
    items[(size_t)bkv * items_per_bkv + mt.z + u] = int4{j, mt.x + u * ITEM_QB, min(ITEM_QB, mt.y - u * ITEM_QB), 0};
}

// One workgroup per bkv: the order in which the dk/dv pass takes the items,
// sorted by the first query block of each item (a counting sort over buckets
// of 2^shift query blocks).  Each item still writes its own slot, so results
// do not depend on this order.
__global__ __launch_bounds__(1024) void bwd_order(const int *__restrict__ pairs, const int4 *__restrict__ items,
                                                  const int *__restrict__ nitems, int *__restrict__ order,
                                                  int pairs_per_bkv, int items_per_bkv, int shift) {
  constexpr int MAXB = 8192, PER = MAXB / 1024;
  __shared__ int hist[MAXB];
  __shared__ int wsum[16];
  const int bkv = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = nitems[bkv];
  const int4 *it = items + (size_t)bkv * items_per_bkv;
  const int *pl = pairs + (size_t)bkv * pairs_per_bkv;
  int *ord = order + (size_t)bkv * items_per_bkv;
  for (int u = tid; u < MAXB; u += 1024) hist[u] = 0;
  __syncthreads();
  for (int r = tid; r < n; r += 1024) atomicAdd(&hist[pl[it[r].y] >> shift], 1);
  __syncthreads();
  int loc[PER], sum = 0;  // exclusive scan: thread tid owns buckets PER*tid ..
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    loc[u] = sum;
    sum += hist[PER * tid + u];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
  for (int x = 0; x < w; ++x) before += wsum[x];
  const int base = before + incl - sum;
#pragma unroll
  for (int u = 0; u < PER; ++u) hist[PER * tid + u] = base + loc[u];
  __syncthreads();
  for (int r = tid; r < n; r += 1024) ord[atomicAdd(&hist[pl[it[r].y] >> shift], 1)] = r;
}

// ------------------------------------------------------------------ dk / dv pass
// Two waves, each holding two 16-key tiles of block j (keys 32w .. 32w + 31)
// as MFMA operands, so that every Q or dO fragment read from LDS (plain for S
// and dP, transposed for dK and dV) feeds two MFMAs: with one tile per wave
// the staged tiles were read twice as fast as the matrix cores consume them.
// Two workgroups share a CU (one wave per SIMD), each with its own staged
// tiles.
constexpr int DKV_KT = 2;                   // 16-key tiles per wave
constexpr int DKV_NW = BB / (16 * DKV_KT);  // waves per workgroup
constexpr int DKV_NT = 64 * DKV_NW;         // threads per workgroup

template <int D>
__global__ __launch_bounds__(DKV_NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void sparse_bwd_dkv(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ dout, const float *__restrict__ lse2, const float *__restrict__ drow,
    const int *__restrict__ pairs, const int4 *__restrict__ items, const int *__restrict__ nitems,
    const int *__restrict__ order, float *__restrict__ partial, int Hq, int Hkv, int N, int pairs_per_bkv,
    int items_per_bkv, float scale) {
  using Cf = BwCfg<D>;
  constexpr int KT = DKV_KT;
  __shared__ __attribute__((aligned(16))) char qb0[Cf::TB], qb1[Cf::TB];
  __shared__ __attribute__((aligned(16))) char ob0[Cf::TB], ob1[Cf::TB];
  __shared__ __attribute__((aligned(16))) float st0[2][256], st1[2][256];  // lse2, D of the 64 rows (+ pad)

  // Workgroup x runs on XCD x % 8.  Each XCD takes runs of 8 consecutive items
  // of the sorted order in turn, so the items resident on one XCD at a time
  // start at nearby query blocks and stage mostly the same Q and dO rows,
  // which its L2 then serves.
  const int ipb = (items_per_bkv + 63) & ~63;
  const int x = blockIdx.x;
  const int bkv = x / ipb, xr = x % ipb;
  const int y = xr >> 3;                       // position in this XCD's sequence
  const int rr = (y >> 3) * 64 + (xr & 7) * 8 + (y & 7);
  if (rr >= nitems[bkv]) return;
  const int r = order[(size_t)bkv * items_per_bkv + rr];  // the item this workgroup takes
  const int4 it = items[(size_t)bkv * items_per_bkv + r];
  const int j = it.x, start = it.y, len = it.z;
  const int b = bkv / Hkv, kvh = bkv % Hkv, G = Hq / Hkv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const float scale_log2 = scale * 1.4426950408889634f;
  int key[KT];  // this lane's key (column of S) in each of the wave's tiles
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) key[kt] = BB * j + 16 * (KT * w + kt) + lr;

  // K and V rows of this wave's keys as B operands
  u32x4 kf[KT][Cf::NDS], vf[KT][Cf::NDS];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const size_t off = ((size_t)bkv * N + key[kt]) * D;
#pragma unroll
    for (int s = 0; s < Cf::NDS; ++s) {
      kf[kt][s] = key[kt] < N ? gload16(k + off + 32 * s + 8 * lg) : u32x4{0, 0, 0, 0};
      vf[kt][s] = key[kt] < N ? gload16(v + off + 32 * s + 8 * lg) : u32x4{0, 0, 0, 0};
    }
  }
  f32x4 dK[KT][Cf::ND], dV[KT][Cf::ND];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int dt = 0; dt < Cf::ND; ++dt) dK[kt][dt] = dV[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int *plist = pairs + (size_t)bkv * pairs_per_bkv + start;
  const int steps = len * G;  // (query block, head) pairs, query block major
  // stage step n: Q and dO rows of query block plist[n / G], head kvh*G + n % G,
  // and their 64 log-sum-exps and D values
  auto stage = [&](int n, char *qd, char *od, float (*sd)[256]) {
    const int i = __builtin_amdgcn_readfirstlane(plist[n / G]);
    const int hq = kvh * G + n % G;
    const size_t rb = (size_t)(b * Hq + hq) * N + (size_t)i * BB;
    const int valid = N - i * BB;
    load_tile<D, DKV_NT>(q + rb * D, valid, qd, tid);
    load_tile<D, DKV_NT>(dout + rb * D, valid, od, tid);
    if (w == 0) {
      const uint32_t nb = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(BB, valid))) * 4u;  // uniform (see load_tile)
      bload16_lds(buf_rsrc(lse2 + rb, nb), sd[0], 16u * l);
      bload16_lds(buf_rsrc(drow + rb, nb), sd[1], 16u * l);
    }
  };
  const uint32_t tr_off = tr_lane_off(l, Cf::ROWB), tr_xor = tr_lane_xor(l);

  if (steps > 0) stage(0, qb0, ob0, st0);
  for (int n = 0; n < steps; ++n) {
    wait_vm0();
    __syncthreads();
    const bool odd = n & 1;
    const char *qc = odd ? qb1 : qb0;
    const char *oc = odd ? ob1 : ob0;
    const float(*sc)[256] = odd ? st1 : st0;
    if (n + 1 < steps) stage(n + 1, odd ? qb0 : qb1, odd ? ob0 : ob1, odd ? st0 : st1);
    const int i = plist[n / G];
    // a query block after the key block, both wholly before N: no pair is masked
    const bool interior = i > j && (i + 1) * BB <= N && (j + 1) * BB <= N;
#pragma unroll
    for (int p = 0; p < 2; ++p) {  // query rows 32p .. 32p + 31
      // S and dP tiles [kt][tt]: lane holds queries 32p + 8lg + 4tt + e of key key[kt]
      f32x4 S[KT][2], dP[KT][2];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) S[kt][tt] = dP[kt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < Cf::NDS; ++s)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const uint32_t off = tile_off<D>(32 * p + pair_key(tt, lr), 4 * s + lg);
          const u32x4 qa = lds_load<u32x4>(qc, off), oa = lds_load<u32x4>(oc, off);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            S[kt][tt] = mfma16x16x32(qa, kf[kt][s], S[kt][tt]);
            dP[kt][tt] = mfma16x16x32(oa, vf[kt][s], dP[kt][tt]);
          }
        }
      const f32x4 ls0 = lds_load<f32x4>(sc[0], (32 * p + 8 * lg) * 4), ls1 = lds_load<f32x4>(sc[0], (32 * p + 8 * lg + 4) * 4);
      const f32x4 dr0 = lds_load<f32x4>(sc[1], (32 * p + 8 * lg) * 4), dr1 = lds_load<f32x4>(sc[1], (32 * p + 8 * lg + 4) * 4);
      u32x4 Pf[KT], Sf[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        float pr[2][4], ds[2][4];
        if (interior) {  // every (query, key) pair of the step is live: no masks
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lsev = tt ? ls1[e] : ls0[e], drv = tt ? dr1[e] : dr0[e];
              pr[tt][e] = __builtin_amdgcn_exp2f(S[kt][tt][e] * scale_log2 - lsev);
              ds[tt][e] = pr[tt][e] * (dP[kt][tt][e] - drv) * scale;
            }
        } else {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int qrow = BB * i + 32 * p + 8 * lg + 4 * tt + e;  // the query's token
              const bool live = qrow < N && key[kt] < N && key[kt] <= qrow;
              const float lsev = tt ? ls1[e] : ls0[e], drv = tt ? dr1[e] : dr0[e];
              pr[tt][e] = live ? __builtin_amdgcn_exp2f(S[kt][tt][e] * scale_log2 - lsev) : 0.f;
              ds[tt][e] = pr[tt][e] * (dP[kt][tt][e] - drv) * scale;
            }
        }
        Pf[kt] = u32x4{pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                       pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3])};
        Sf[kt] = u32x4{pack_bf16x2(ds[0][0], ds[0][1]), pack_bf16x2(ds[0][2], ds[0][3]),
                       pack_bf16x2(ds[1][0], ds[1][1]), pack_bf16x2(ds[1][2], ds[1][3])};
      }
#pragma unroll
      for (int dt = 0; dt < Cf::ND; ++dt) {
        const u32x4 ot = tr_frag(oc, 32 * p * Cf::ROWB, tr_off, tr_xor, dt, Cf::NCH, Cf::ROWB);
        const u32x4 qt = tr_frag(qc, 32 * p * Cf::ROWB, tr_off, tr_xor, dt, Cf::NCH, Cf::ROWB);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          dV[kt][dt] = mfma16x16x32(ot, Pf[kt], dV[kt][dt]);
          dK[kt][dt] = mfma16x16x32(qt, Sf[kt], dK[kt][dt]);
        }
      }
    }
    __syncthreads();  // every wave is done with this step's buffers before they are reloaded
  }
  // this item's sums: partial[item][0 = dK, 1 = dV][key row][feature]
  float *pk = partial + ((size_t)bkv * items_per_bkv + r) * 2 * BB * D;
  float *pv = pk + BB * D;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int kr = 16 * (KT * w + kt) + lr;
#pragma unroll
    for (int dt = 0; dt < Cf::ND; ++dt) {
      *reinterpret_cast<f32x4 *>(pk + (size_t)kr * D + 16 * dt + 4 * lg) = dK[kt][dt];
      *reinterpret_cast<f32x4 *>(pv + (size_t)kr * D + 16 * dt + 4 * lg) = dV[kt][dt];
    }
  }
}

// One workgroup per (bkv, key block j): the sums of j's items in item order,
// rounded once to bf16 (0 where no query block selected j).
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce(const float *__restrict__ partial, const int4 *__restrict__ meta,
                                                  uint16_t *__restrict__ dk, uint16_t *__restrict__ dv, int N,
                                                  int NB, int items_per_bkv) {
  const int x = blockIdx.x;
  const int bkv = x / NB, j = x % NB;
  const int4 mt = meta[(size_t)bkv * NB + j];
  const int nit = (mt.y + ITEM_QB - 1) / ITEM_QB;
  const float *base = partial + ((size_t)bkv * items_per_bkv + mt.z) * 2 * BB * D;
  constexpr int PER = 2 * BB * D / 4 / 256;  // float4 pieces per thread (dK then dV)
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e4 = u * 256 + threadIdx.x;  // float4 index in [dK | dV]
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < nit; ++it) acc += *reinterpret_cast<const f32x4 *>(base + (size_t)it * 2 * BB * D + 4 * e4);
    const int which = (4 * e4) / (BB * D), rem = (4 * e4) % (BB * D);
    const int row = rem / D, col = rem % D;
    const int tok = BB * j + row;
    if (tok < N) {
      uint16_t *dst = (which ? dv : dk) + ((size_t)bkv * N + tok) * D + col;
      *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    }
  }
}

// Workspace layout (each part 256-byte aligned)
struct BwLayout {
  size_t lse, drow, bitmap, meta, nitems, pairs, items, order, partial, total;
  int NQB, WPR, pairs_per_bkv, items_per_bkv;
};
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
BwLayout bw_layout(int B, int Hq, int Hkv, int N, int d, int n_sel) {
  BwLayout L{};
  L.NQB = (N + BB - 1) / BB;
  L.WPR = (L.NQB + 31) / 32;
  L.pairs_per_bkv = L.NQB * n_sel;
  L.items_per_bkv = (L.pairs_per_bkv + ITEM_QB - 1) / ITEM_QB + L.NQB;
  const size_t BKV = (size_t)B * Hkv;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += al256(bytes); return o; };
  L.lse = take((size_t)B * Hq * N * 4);
  L.drow = take((size_t)B * Hq * N * 4);
  L.bitmap = take(BKV * L.NQB * L.WPR * 4);
  L.meta = take(BKV * L.NQB * 16);
  L.nitems = take(BKV * 4);
  L.pairs = take(BKV * L.pairs_per_bkv * 4);
  L.items = take(BKV * L.items_per_bkv * 16);
  L.order = take(BKV * L.items_per_bkv * 4);
  L.partial = take(BKV * L.items_per_bkv * 2 * BB * (size_t)d * 4);
  L.total = off;
  return L;
}

template <int D>
hipError_t run_bwd(const SparseBackwardArgs &a, hipStream_t st) {
  const BwLayout L = bw_layout(a.B, a.Hq, a.Hkv, a.N, a.d, a.n_sel);
  char *ws = static_cast<char *>(a.ws);
  float *lse = reinterpret_cast<float *>(ws + L.lse);
  float *drow = reinterpret_cast<float *>(ws + L.drow);
  uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + L.bitmap);
  int4 *meta = reinterpret_cast<int4 *>(ws + L.meta);
  int *nitems = reinterpret_cast<int *>(ws + L.nitems);
  int *pairs = reinterpret_cast<int *>(ws + L.pairs);
  int4 *items = reinterpret_cast<int4 *>(ws + L.items);
  int *order = reinterpret_cast<int *>(ws + L.order);
  float *partial = reinterpret_cast<float *>(ws + L.partial);
  const int NQB = L.NQB, BKV = a.B * a.Hkv, G = a.Hq / a.Hkv;
  const int HG = (G + 3) / 4;
  const int ntasks = BKV * NQB;
  const int grid_dq = ((ntasks + 7) / 8) * 8 * HG;
  hipLaunchKernelGGL((a.scale > 0.f ? sparse_bwd_dq<D, true> : sparse_bwd_dq<D, false>), dim3(grid_dq), dim3(512), 0, st,
                     (const uint16_t *)a.q,
                     (const uint16_t *)a.k, (const uint16_t *)a.v, (const uint16_t *)a.dout,
                     a.idx, (uint16_t *)a.dq, lse, drow, a.Hq, a.Hkv, a.N, NQB, a.n_sel, HG, ntasks, a.scale);
  const size_t nbits = (size_t)BKV * NQB * L.WPR;
  hipLaunchKernelGGL(bwd_clear, dim3((unsigned)((nbits + 255) / 256)), dim3(256), 0, st, bitmap, nbits);
  const long long rows = (long long)BKV * NQB;
  hipLaunchKernelGGL(bwd_mark, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, a.idx, bitmap, NQB, NQB,
                     a.n_sel, L.WPR, rows);
  hipLaunchKernelGGL(bwd_counts, dim3(BKV), dim3(1024), 0, st, bitmap, meta, nitems, NQB, L.WPR);
  hipLaunchKernelGGL(bwd_lists, dim3(BKV * NQB), dim3(64), 0, st, bitmap, meta, pairs, items, NQB, L.WPR,
                     L.pairs_per_bkv, L.items_per_bkv);
  int shift = 0;
  while (((NQB - 1) >> shift) >= 8192) ++shift;  // at most 8192 buckets of first query blocks
  hipLaunchKernelGGL(bwd_order, dim3(BKV), dim3(1024), 0, st, pairs, items, nitems, order, L.pairs_per_bkv,
                     L.items_per_bkv, shift);
  hipLaunchKernelGGL((sparse_bwd_dkv<D>), dim3(BKV * ((L.items_per_bkv + 63) & ~63)), dim3(DKV_NT), 0, st,
                     (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, (const uint16_t *)a.dout,
                     lse, drow, pairs, items, nitems, order, partial, a.Hq, a.Hkv, a.N, L.pairs_per_bkv,
                     L.items_per_bkv, a.scale);
  hipLaunchKernelGGL((bwd_reduce<D>), dim3(BKV * NQB), dim3(256), 0, st, partial, meta, (uint16_t *)a.dk,
                     (uint16_t *)a.dv, a.N, NQB, L.items_per_bkv);
  return hipGetLastError();
}

}  // namespace

size_t sparse_backward_workspace(int dtype, int B, int Hq, int Hkv, int N, int d, int block, int n_sel) {
  (void)dtype; (void)block;
  return bw_layout(B, Hq, Hkv, N, d, n_sel).total;
}

hipError_t launch_sparse_backward(const SparseBackwardArgs &a, hipStream_t st) {
  return a.d == 128 ? run_bwd<128>(a, st) : run_bwd<64>(a, st);
}

}  // namespace sala
