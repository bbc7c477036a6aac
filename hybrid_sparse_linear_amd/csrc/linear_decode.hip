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

// Kernel-side neighbour parameters (the fused step): RMS norm of q and k,
// rotate-half RoPE at pos[b], output gate o * sigmoid(gate).
struct NbD {
  const float *gq, *gk;
  float eps, rope_base;
  const long long *pos;
  const void *gate;
};

// F: the first D threads normalise and rotate q (threads < D/2, one rotate-half
// pair each) and k (threads D/2 .. D-1) into LDS while the state loads are in
// flight; the values are rounded to T as an unfused producer would store them.
template <typename T, int D, bool F>
__global__ __launch_bounds__(256) void lin_decode(const T *__restrict__ q, const T *__restrict__ k,
                                                  const T *__restrict__ v, T *__restrict__ o,
                                                  const float *__restrict__ decay, float *__restrict__ state, int H,
                                                  NbD nb) {
  constexpr int CG = D / 32;      // column groups per (b, h)
  constexpr int RG = 32;          // row groups
  constexpr int RPT = D / RG;     // rows per thread
  __shared__ float part[RG][33];
  __shared__ float qk[2][D];
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
  if constexpr (F) {
    if (tid < D) {
      // wave 0 (D = 128) or its first half (D = 64) handles q, the next k
      const int which = tid / (D / 2), i = tid % (D / 2);
      const T *x = (which ? k : q) + (size_t)bh * D;
      float a = ld(x, i), z = ld(x, i + D / 2);
      const float *gam = which ? nb.gk : nb.gq;
      if (gam) {
        float ss = fmaf(a, a, z * z);
#pragma unroll
        for (int o2 = D / 4; o2 >= 1; o2 >>= 1) ss += __shfl_xor(ss, o2, 64);  // over the D/2 lanes of this vector
        const float r = rsqrtf(fmaf(ss, 1.f / D, nb.eps));
        a *= r * gam[i];
        z *= r * gam[i + D / 2];
      }
      if (nb.rope_base > 0.f) {
        const double t = pow((double)nb.rope_base, -2.0 * i / D) * 0.15915494309189535;  // theta_i / 2pi
        const double x2 = (double)nb.pos[bh / H] * t;
        const float turns = (float)(x2 - floor(x2));
        const float c = __builtin_amdgcn_cosf(turns), sn = __builtin_amdgcn_sinf(turns);
        const float ya = fmaf(-z, sn, a * c), yz = fmaf(a, sn, z * c);
        a = ya;
        z = yz;
      }
      if constexpr (sizeof(T) == 2) {
        a = bf16_to_f32(f32_to_bf16(a));
        z = bf16_to_f32(f32_to_bf16(z));
      }
      qk[which][i] = a;
      qk[which][i + D / 2] = z;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      qr[r] = qk[0][rg + RG * r];
      kr[r] = qk[1][rg + RG * r];
    }
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      qr[r] = ld(q, (size_t)bh * D + rg + RG * r);
      kr[r] = ld(k, (size_t)bh * D + rg + RG * r);
    }
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
    const size_t oi = (size_t)bh * D + 32 * cg + tid;
    if constexpr (F) {
      if (nb.gate) t *= sigmoid_fast(ld(static_cast<const T *>(nb.gate), oi));
    }
    st(o, oi, t);
  }
}

template <typename T, int D>
void launch_t(const LinearDecodeArgs &a, hipStream_t st) {
  const int BH = a.B * a.H;
  NbD nb{nullptr, nullptr, 0.f, 0.f, nullptr, nullptr};
  if (a.nb) {
    nb = NbD{a.nb->gamma_q, a.nb->gamma_k, a.nb->eps, a.nb->rope_base, a.nb->pos, a.nb->gate};
    hipLaunchKernelGGL((lin_decode<T, D, true>), dim3(BH * (D / 32)), dim3(256), 0, st, (const T *)a.q,
                       (const T *)a.k, (const T *)a.v, (T *)a.o, a.decay, a.state, a.H, nb);
  } else {
    hipLaunchKernelGGL((lin_decode<T, D, false>), dim3(BH * (D / 32)), dim3(256), 0, st, (const T *)a.q,
                       (const T *)a.k, (const T *)a.v, (T *)a.o, a.decay, a.state, a.H, nb);
  }
}

}  // namespace

hipError_t launch_linear_decode(const LinearDecodeArgs &a, hipStream_t st) {
  if (a.dtype == 1) {
    if (a.d == 128) launch_t<uint16_t, 128>(a, st);
    else launch_t<uint16_t, 64>(a, st);
  } else {
    if (a.d == 128) launch_t<float, 128>(a, st);
    else launch_t<float, 64>(a, st);
  }
  return hipGetLastError();
}

}  // namespace sala
