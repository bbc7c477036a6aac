// The attention layers' neighbours as standalone streaming kernels for gfx950:
// QK RMS normalisation with optional rotate-half RoPE, and the output gate.
// The pages add QK normalisation and an output gate after every attention
// block, and RoPE on the linear layers only (MiniCPM-SALA, gist.science (ja)
// 技術概要 section 2.2; gist.science (de) section 2,
// "Architektur-Hybridisierung").  The linear layer can take all three inside
// its own kernels (sala_linear_prefill_fused); these kernels serve the sparse
// layers (normalisation and gate, no RoPE) and an unfused pipeline.
//
// qk_norm_rope: a thread owns 16-byte piece hc (features 8hc .. 8hc+7) and
// piece hc + D/16 (features D/2 + 8hc ..) of one row, so its rotate-half
// partners are its own and a row's sum of squares is a sum over D/16
// consecutive lanes.  The angle p * theta_i is reduced to a fraction of a turn
// in fp64, then sin / cos come from the hardware (which takes turns).
// Both kernels are HBM-bound: a row is read once and written once; out may
// be the input itself (each thread reads its pieces before writing them).

#include "sala_common.hpp"
#include "sala_launch.hpp"

namespace sala {
namespace {

template <typename T>
struct Vec;  // 8 consecutive elements of a row
template <>
struct Vec<uint16_t> {
  u32x4 w;
  __device__ void load(const uint16_t *p) { w = gload16(p); }
  __device__ void store(uint16_t *p) const { gstore16(p, w); }
  __device__ float get(int e) const { return (e & 1) ? bf16hi(w[e >> 1]) : bf16lo(w[e >> 1]); }
  __device__ void put(const float (&x)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
  }
};
template <>
struct Vec<float> {
  f32x4 a, b;
  __device__ void load(const float *p) {
    a = *reinterpret_cast<const f32x4 *>(p);
    b = *reinterpret_cast<const f32x4 *>(p + 4);
  }
  __device__ void store(float *p) const {
    *reinterpret_cast<f32x4 *>(p) = a;
    *reinterpret_cast<f32x4 *>(p + 4) = b;
  }
  __device__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
  __device__ void put(const float (&x)[8]) {
    a = f32x4{x[0], x[1], x[2], x[3]};
    b = f32x4{x[4], x[5], x[6], x[7]};
  }
};

// rows = B*H*N rows of D features; row r sits at position pos0 + r % N.
template <typename T, int D>
__global__ __launch_bounds__(256) void qk_norm_rope(const T *x, T *out, const float *__restrict__ gamma,
                                                    float eps, float rope_base, long long pos0, int N, long long rows) {
  constexpr int HC = D / 16;  // lanes per row
  __shared__ double trv[D / 2];
  const int tid = threadIdx.x;
  if (tid < D / 2 && rope_base > 0.f) trv[tid] = pow((double)rope_base, -2.0 * tid / D) * 0.15915494309189535;
  __syncthreads();
  const long long row = (long long)blockIdx.x * (256 / HC) + tid / HC;
  const int hc = tid % HC;
  // lanes of a row stay together (HC divides 64), so a row past the end is
  // skipped by all of its lanes at once
  if (row >= rows) return;
  const T *src = x + row * D;
  T *dst = out + row * D;
  Vec<T> lo, hi;
  lo.load(src + 8 * hc);
  hi.load(src + D / 2 + 8 * hc);
  float a[8], z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = lo.get(e);
    z[e] = hi.get(e);
  }
  if (gamma) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(z[e], z[e], fmaf(a[e], a[e], ss));
    ss = lane_group_sum<HC>(ss);
    const float r = rsqrtf(fmaf(ss, 1.f / D, eps));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] *= r * gamma[8 * hc + e];
      z[e] *= r * gamma[D / 2 + 8 * hc + e];
    }
  }
  if (rope_base > 0.f) {
    const double p = (double)(pos0 + row % N);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double t = p * trv[8 * hc + e];
      const float turns = (float)(t - floor(t));
      const float c = __builtin_amdgcn_cosf(turns), sn = __builtin_amdgcn_sinf(turns);
      const float ya = fmaf(-z[e], sn, a[e] * c), yz = fmaf(a[e], sn, z[e] * c);
      a[e] = ya;
      z[e] = yz;
    }
  }
  lo.put(a);
  hi.put(z);
  lo.store(dst + 8 * hc);
  hi.store(dst + D / 2 + 8 * hc);
}

// out[i] = o[i] * sigmoid(g[i]) over n elements, 8 per thread (n % 8 == 0).
template <typename T>
__global__ __launch_bounds__(256) void output_gate(const T *o, const T *__restrict__ g, T *out,
                                                   long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  Vec<T> ov, gv;
  ov.load(o + 8 * i);
  gv.load(g + 8 * i);
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = ov.get(e) * sigmoid_fast(gv.get(e));
  ov.put(r);
  ov.store(out + 8 * i);
}

template <typename T, int D>
void launch_norm_rope(const QkNormRopeArgs &a, hipStream_t st) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int RPB = 256 / (D / 16);
  hipLaunchKernelGGL((qk_norm_rope<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                     (const T *)a.x, (T *)a.out, a.gamma, a.eps, a.rope_base, a.pos0, a.N, rows);
}

}  // namespace

hipError_t launch_qk_norm_rope(const QkNormRopeArgs &a, hipStream_t st) {
  if (a.dtype == 1) {
    if (a.d == 128) launch_norm_rope<uint16_t, 128>(a, st);
    else launch_norm_rope<uint16_t, 64>(a, st);
  } else {
    if (a.d == 128) launch_norm_rope<float, 128>(a, st);
    else launch_norm_rope<float, 64>(a, st);
  }
  return hipGetLastError();
}

hipError_t launch_output_gate(int dtype, size_t n, const void *o, const void *g, void *out, hipStream_t st) {
  const long long n8 = (long long)(n / 8);
  const dim3 grid((unsigned)((n8 + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(output_gate<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)o, (const uint16_t *)g,
                       (uint16_t *)out, n8);
  else
    hipLaunchKernelGGL(output_gate<float>, grid, dim3(256), 0, st, (const float *)o, (const float *)g, (float *)out,
                       n8);
  return hipGetLastError();
}

}  // namespace sala
