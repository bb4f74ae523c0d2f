// Scratch memory for the layer entry point that allocates nothing
// (moe_layer_forward_noalloc): the workspace of the fused layer lives in a
// file-scope device array instead of a caller-provided buffer.
//
// Each GPU the library runs on holds its own copy of the array (a code-object
// global, zero when the code object is loaded) until the process ends.  Its
// device address is looked up once per device with hipGetSymbolAddress; host
// code uses only that address (in host code the array's name is a host-side
// stand-in, not device memory).
//
// The array carries the same state as a caller's workspace: a call counter, a
// status word and values tagged with the call number.  Every call gets a new
// number, so nothing has to be cleared between calls; the only state that must
// start at zero is the whole array before its first use, which the loader's
// zero-fill gives (and a fill kernel repeats on the first call of a device when
// the stream is not being captured).  All calls on one GPU share the array:
// calls that overlap on one GPU (different streams, no ordering) race.
#include <mutex>

#include "qmoe_internal.h"

namespace qmoe {

namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of scratch per device; null until set up

__global__ void k_fill_zero(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The device address of this device's scratch, set up on the first call.
hipError_t scratch_of_device(void** out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return e;
    if (cs == hipStreamCaptureStatusNone) {
      // stream-ordered before the first layer launch; under capture the loader's
      // zero-fill stands (a captured fill would run again at every replay)
      const int64_t n16 = (int64_t)(kNoAllocScratchBytes / 16);
      hipLaunchKernelGGL(k_fill_zero, dim3(256), dim3(256), 0, s, static_cast<uint4*>(ptr), n16);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_layer_noalloc(const qmoe_layer& L, const float* x, const float* residual,
                                float* out, int32_t* idx, float* w, hipStream_t s) {
  void* ws = nullptr;
  hipError_t e = scratch_of_device(&ws, s);
  if (e != hipSuccess) return e;
  return launch_layer(L, x, nullptr, 0.f, residual, out, idx, w, ws, s);
}

}  // namespace qmoe
