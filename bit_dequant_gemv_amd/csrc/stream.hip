// Streaming-read calibration: how fast one launch can read a given number of
// bytes from HBM on this machine.  The layer kernels read their weights once per
// call, so the bandwidth they can reach depends on the bytes one launch moves
// (launch and ramp-up latency weigh more on small launches); this kernel gives
// the attainable rate for the same bytes per launch, with nothing computed.
//
// Loads are 16 bytes, non-temporal (the cache policy of the weight streams), four
// independent loads in flight per lane, on a grid of two workgroups per CU (the
// shape that read fastest on MI355X: more requests in flight slow the stream
// down).  Each lane folds what it read into one word with xor; the word is
// stored only if it equals a key the caller passes, so the loads cannot be
// dropped and, in practice, nothing is written.
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kSB = 256;  // threads per workgroup
constexpr int kInFlight = 4;

__global__ __launch_bounds__(kSB) void k_stream_read(const uint4* __restrict__ p, int64_t n16,
                                                     uint32_t key, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kSB;
  int64_t i = (int64_t)blockIdx.x * kSB + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    uint4 v[kInFlight];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) v[j] = ld_stream16(p + i + j * stride);
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = ld_stream16(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == key) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t key, uint32_t* sink,
                              hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int64_t want = (n16 + (int64_t)kSB * kInFlight - 1) / ((int64_t)kSB * kInFlight);
  const int grid = (int)(want < 2 * cus ? want : 2 * cus);
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(kSB), 0, s, static_cast<const uint4*>(buf), n16,
                     key, sink);
  return hipGetLastError();
}

}  // namespace qmoe
