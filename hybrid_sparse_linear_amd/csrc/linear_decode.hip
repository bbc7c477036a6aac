// One decode token of Lightning (decayed linear) attention for gfx950:
//   S <- lam S + k v^T ;  o = q S          (S is [d_k][d_v] fp32, updated in place)
// The recurrent form the pages credit for the O(N) cost (MiniCPM-SALA,
// gist.science (de) section 2, "Architektur-Hybridisierung"), one step at a
// time.  The state read and write dominate: 2 * d * d * 4 bytes per (b, h).
//
// Layout: D/32 workgroups per (b, h), each owning 32 d_v columns of S.
// Thread = (column quad, row group): one 16-byte state read and write per
// row it owns; the partial q.S over its rows is summed across row groups in LDS.

#include "sala_common.hpp"
#include "sala_launch.hpp"

namespace sala {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T *p, size_t i) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
  else return p[i];
}
template <typename T>
__device__ __forceinline__ void st(T *p, size_t i, float f) {
  if constexpr (sizeof(T) == 2) reinterpret_cast<uint16_t *>(p)[i] = f32_to_bf16(f);
  else p[i] = f;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void lin_decode(const T *__restrict__ q, const T *__restrict__ k,
                                                  const T *__restrict__ v, T *__restrict__ o,
                                                  const float *__restrict__ decay, float *__restrict__ state, int H) {
  constexpr int CG = D / 32;      // column groups per (b, h)
  constexpr int RG = 32;          // row groups
  constexpr int RPT = D / RG;     // rows per thread
  __shared__ float part[RG][33];
  const int bh = blockIdx.x / CG, cg = blockIdx.x % CG;
  const int h = bh % H, tid = threadIdx.x;
  const int cq = tid & 7, rg = tid >> 3;  // column quad 0..7, row group 0..31
  const int c0 = 32 * cg + 4 * cq;
  float *S = state + (size_t)bh * D * D;
  // the state reads go out first; q, k, v (a few bytes, shared by many
  // threads) follow without a barrier, so everything is one round trip
  float4 s[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) s[r] = *reinterpret_cast<const float4 *>(S + (size_t)(rg + RG * r) * D + c0);
  float qr[RPT], kr[RPT], vv[4];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    qr[r] = ld(q, (size_t)bh * D + rg + RG * r);
    kr[r] = ld(k, (size_t)bh * D + rg + RG * r);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = ld(v, (size_t)bh * D + c0 + e);
  const float lam = decay ? decay[h] : 1.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    float4 x = s[r];
    x.x = fmaf(lam, x.x, kr[r] * vv[0]);
    x.y = fmaf(lam, x.y, kr[r] * vv[1]);
    x.z = fmaf(lam, x.z, kr[r] * vv[2]);
    x.w = fmaf(lam, x.w, kr[r] * vv[3]);
    *reinterpret_cast<float4 *>(S + (size_t)(rg + RG * r) * D + c0) = x;
    acc[0] = fmaf(qr[r], x.x, acc[0]);
    acc[1] = fmaf(qr[r], x.y, acc[1]);
    acc[2] = fmaf(qr[r], x.z, acc[2]);
    acc[3] = fmaf(qr[r], x.w, acc[3]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) part[rg][4 * cq + e] = acc[e];
  __syncthreads();
  if (tid < 32) {
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) t += part[r][tid];
    st(o, (size_t)bh * D + 32 * cg + tid, t);
  }
}

}  // namespace

hipError_t launch_linear_decode(const LinearDecodeArgs &a, hipStream_t st) {
  const int BH = a.B * a.H;
  const dim3 blk(256);
  if (a.dtype == 1) {
    if (a.d == 128)
      hipLaunchKernelGGL((lin_decode<uint16_t, 128>), dim3(BH * 4), blk, 0, st, (const uint16_t *)a.q,
                         (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.o, a.decay, a.state, a.H);
    else
      hipLaunchKernelGGL((lin_decode<uint16_t, 64>), dim3(BH * 2), blk, 0, st, (const uint16_t *)a.q,
                         (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.o, a.decay, a.state, a.H);
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL((lin_decode<float, 128>), dim3(BH * 4), blk, 0, st, (const float *)a.q, (const float *)a.k,
                         (const float *)a.v, (float *)a.o, a.decay, a.state, a.H);
    else
      hipLaunchKernelGGL((lin_decode<float, 64>), dim3(BH * 2), blk, 0, st, (const float *)a.q, (const float *)a.k,
                         (const float *)a.v, (float *)a.o, a.decay, a.state, a.H);
  }
  return hipGetLastError();
}

}  // namespace sala
