// Scratch memory of the allocation-free decode step (sala_sparse_decode_step_noalloc).
//
// Some callers cannot allocate device memory at call time (code under HIP
// graph capture, tight serving loops).  For them the decode step's workspace
// -- the selection's local top-64 lists or score row and the attention's
// split-K partials, which the caller otherwise passes as `ws` -- lives in one
// file-scope device array of fixed size.  Each GPU the library runs on holds
// its own copy of the array from module load until the process ends.  Calls on
// one GPU share that copy, so calls that overlap on one GPU race; nothing in
// it has to start at zero (every kernel writes its part of the workspace
// before reading it).

#include <mutex>

#include "../../include/sala.h"
#include "sala_launch.hpp"

namespace sala {

static __device__ __align__(256) char scratch[SALA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};
}  // namespace

// Device address of the current device's copy of `scratch`, looked up once per
// device with that device current.  The host-side name of the array is only a
// stand-in for the symbol: every use on the host goes through this address.
hipError_t noalloc_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace sala
