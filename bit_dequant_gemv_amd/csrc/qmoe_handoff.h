// Values handed from workgroup to workgroup inside one launch, as 64-bit tagged
// words: (call number << 32) | value bits, written with agent-scope atomic stores
// (write-through to the device coherence point) and read until they carry the
// current call's number, so that the buffers never need resetting.  The call
// number comes from a counter kept in the caller's workspace (word CTRL_EPOCH),
// which every workgroup reads at its start and one workgroup advances once it has
// seen a word from every other.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {
namespace {

constexpr uint32_t kSpinLimit = 1u << 18;
// u64 words per 128-byte line: a value written by several CUs into one shared line
// becomes visible ~0.6 us later than one whose line has a single writer, so words
// that many workgroups wait for (the fused layer's completion flags and logits)
// get a line per writer
constexpr int kLine = 16;
// buffers of values read by every workgroup rotate over calls (call number % 4),
// so that a line still cached from an earlier read of the same slot is rare
constexpr int kSlotsH = 4;

// control words at the start of the workspace
enum { CTRL_EPOCH = 0, CTRL_STATUS = 1, CTRL_ZERO = 8 };  // CTRL_ZERO is never written

__device__ __forceinline__ void tag_put(uint64_t* p, float v, uint32_t tag) {
  const uint64_t u = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
  __hip_atomic_store(p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t tag_get(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void flag_status(uint32_t* ctrl, uint32_t bit) {
  __hip_atomic_fetch_or(ctrl + CTRL_STATUS, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Read N tagged words src[j * stride] (j < N) into v (their values), every load
// issued before any is checked (one round trip); nothing is read when !valid (v is
// then zeros).  Ordinary (L2-cacheable) loads, so the 32 workgroups of an XCD
// share one fetch from memory.  A word still carrying an old tag comes from a
// stale cached line (the buffer slot was last used several calls ago) or from a
// store not yet visible: those words are re-read coherently, all of them per
// pass, until they carry the tag (bounded; on time-out ok is cleared).
template <int N>
__device__ __forceinline__ void read_tagged_strided(const uint64_t* src, int stride, bool valid, float (&v)[N],
                                                    uint32_t tag, bool& ok) {
  static_assert(N <= 32, "at most 32 words");
  uint64_t r[N];
#pragma unroll
  for (int j = 0; j < N; ++j) r[j] = valid ? src[(int64_t)j * stride] : ((uint64_t)tag << 32);
  uint32_t pending = 0;
  for (uint32_t spins = 0;; ++spins) {
#pragma unroll
    for (int j = 0; j < N; ++j)
      if ((uint32_t)(r[j] >> 32) != tag) pending |= 1u << j;
      else pending &= ~(1u << j);
    if (!pending) break;
    if (spins > kSpinLimit) {
      ok = false;
      break;
    }
    if (spins) __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < N; ++j)
      if ((pending >> j) & 1u) r[j] = tag_get(const_cast<uint64_t*>(src) + (int64_t)j * stride);
  }
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = __uint_as_float((uint32_t)r[j]);
}

}  // namespace
}  // namespace qmoe
