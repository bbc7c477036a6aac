// Debug check of block-index rows, run by the C ABI before the gathering
// kernels when SALA_DEBUG_CHECK=1.  The kernels themselves never read outside
// their buffers whatever idx holds (entries past a row's first negative one,
// below zero, or beyond the query's block or the cached blocks are skipped);
// this check reports the rows that break the documented contract, which the
// kernels would otherwise process silently:
//   code 1  an entry before the first negative one is >= the number of blocks
//   code 2  a block listed twice before the first negative entry
//   code 3  (prefill rows) the query's own block is missing
// It synchronizes the stream and is skipped while the stream is being
// captured into a graph.

#include "sala_common.hpp"
#include "sala_launch.hpp"

namespace sala {
namespace {

// first bad (row << 32 | entry << 2 | code) of the last check on this GPU
__device__ unsigned long long idx_bad[1];

__global__ void idx_check_clear(unsigned long long *bad) { bad[0] = ~0ull; }

// one thread per row; own: the row's query block is row % nqb and must be listed
__global__ __launch_bounds__(256) void idx_check(const int32_t *__restrict__ idx, long long rows, int n_sel,
                                                 int nqb, int nb, int own, unsigned long long *bad) {
  const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int32_t *row = idx + r * n_sel;
  const int i = own ? (int)(r % nqb) : -1;
  int n = n_sel, code = 0, at = 0;
  bool has_own = false;
  for (int e = 0; e < n_sel; ++e) {
    const int j = row[e];
    if (j < 0) {
      n = e;
      break;
    }
    if (j >= nb) {
      code = 1;
      at = e;
      break;
    }
    has_own = has_own || j == i;
  }
  for (int e = 1; e < n && code == 0; ++e)
    for (int f = 0; f < e; ++f)
      if (row[f] == row[e]) {
        code = 2;
        at = e;
        break;
      }
  if (code == 0 && own && !has_own) code = 3;
  if (code) atomicMin(bad, ((unsigned long long)r << 32) | ((unsigned long long)at << 2) | (unsigned long long)code);
}

}  // namespace

hipError_t debug_check_idx(const int32_t *idx, long long rows, int n_sel, int nqb, int nb, int own, hipStream_t st,
                           unsigned long long *result) {
  *result = ~0ull;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return e;
  if (cs != hipStreamCaptureStatusNone) return hipSuccess;  // no synchronization inside a capture
  unsigned long long *bad = nullptr;
  e = hipGetSymbolAddress(reinterpret_cast<void **>(&bad), HIP_SYMBOL(idx_bad));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(idx_check_clear, dim3(1), dim3(1), 0, st, bad);
  if (rows > 0)
    hipLaunchKernelGGL(idx_check, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, idx, rows, n_sel, nqb, nb,
                       own, bad);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned long long host = ~0ull;
  e = hipMemcpyAsync(&host, bad, sizeof(host), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  *result = host;
  return hipSuccess;
}

}  // namespace sala
