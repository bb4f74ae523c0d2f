// Device-side synthetic input generator (test and benchmark infrastructure).
//
// Implements the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror,
// Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11) and the value
// mappings of the host generator in synth/__init__.py, so that expert pools of
// any size can be generated directly in HBM and regenerated on the host for
// any expert that a check needs.  Word n of stream (seed, tid) is lane n % 4
// of Philox applied to counter (n/4 low, n/4 high, 0, 0) with key (seed, tid).
//
// Built with -ffp-contract=off: the uniform mapping must round its multiply and
// its add separately to match the host bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct U4 { uint32_t v[4]; };

__device__ __forceinline__ U4 philox(uint64_t block, uint32_t k0, uint32_t k1) {
  uint32_t c0 = (uint32_t)block, c1 = (uint32_t)(block >> 32), c2 = 0u, c3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  U4 o;
  o.v[0] = c0; o.v[1] = c1; o.v[2] = c2; o.v[3] = c3;
  return o;
}

__device__ __forceinline__ uint32_t word_at(uint64_t n, uint32_t seed, uint32_t tid) {
  U4 o = philox(n >> 2, seed, tid);
  return o.v[n & 3];
}

__device__ __forceinline__ float uniform_map(uint32_t w, float lo, float span) {
  const float u = (float)(w >> 8) * 5.9604644775390625e-08f;  // exact: < 2^24 times 2^-24
  return __fadd_rn(lo, __fmul_rn(u, span));
}

// Irwin-Hall sum of sixteen 16-bit halves of words 8i..8i+7, centred (exact
// integer), times c = sigma / (65536 * sqrt(16/12)) rounded to binary32.
__device__ __forceinline__ float normal_at(uint64_t i, uint32_t seed, uint32_t tid, float c) {
  const U4 a = philox(2 * i, seed, tid);
  const U4 b = philox(2 * i + 1, seed, tid);
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s += (int32_t)(a.v[j] & 0xFFFFu) + (int32_t)(a.v[j] >> 16);
    s += (int32_t)(b.v[j] & 0xFFFFu) + (int32_t)(b.v[j] >> 16);
  }
  return __fmul_rn((float)(s - 524280), c);
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__global__ void k_fill_words(uint32_t* __restrict__ dst, uint64_t n_words, uint32_t seed,
                             uint32_t tid) {
  const uint64_t blk = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one Philox block
  const uint64_t w0 = blk * 4;
  if (w0 >= n_words) return;
  const U4 o = philox(blk, seed, tid);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (w0 + j < n_words) dst[w0 + j] = o.v[j];
}

__global__ void k_fill_tail_bytes(uint8_t* __restrict__ dst, uint64_t start, uint64_t n_bytes,
                                  uint32_t seed, uint32_t tid) {
  // bytes [start, n_bytes) of the stream, start a multiple of 4, fewer than 4 bytes
  const uint64_t n = start + threadIdx.x;
  if (n >= n_bytes) return;
  const uint32_t w = word_at(n >> 2, seed, tid);
  dst[n] = (uint8_t)(w >> (8 * (n & 3)));
}

__global__ void k_fill_uniform_f32(float* __restrict__ dst, uint64_t n, uint32_t seed,
                                   uint32_t tid, float lo, float span) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  dst[i] = uniform_map(word_at(i, seed, tid), lo, span);
}

__global__ void k_fill_normal_f32(float* __restrict__ dst, uint64_t n, uint32_t seed,
                                  uint32_t tid, float c) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  dst[i] = normal_at(i, seed, tid, c);
}

__global__ void k_fill_normal_bf16(uint16_t* __restrict__ dst, uint64_t n, uint32_t seed,
                                   uint32_t tid, float c) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  dst[i] = (uint16_t)bf16_rne_bits(normal_at(i, seed, tid, c));
}

__device__ __forceinline__ uint32_t tensor_id(uint32_t kind, uint32_t expert, uint32_t layer) {
  return kind | (expert << 8) | (layer << 20);
}

// One launch per tensor of the expert block, grid.y = expert.
__global__ void k_pool_codes(uint8_t* __restrict__ base, int64_t stride, int expert0, int layer,
                             uint32_t seed, uint32_t kind, uint64_t offset, uint64_t n_words) {
  const uint64_t blk = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t w0 = blk * 4;
  if (w0 >= n_words) return;
  const int e = blockIdx.y;
  const U4 o = philox(blk, seed, tensor_id(kind, (uint32_t)(expert0 + e), (uint32_t)layer));
  uint32_t* dst = reinterpret_cast<uint32_t*>(base + (int64_t)e * stride + offset);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (w0 + j < n_words) dst[w0 + j] = o.v[j];
}

__global__ void k_pool_sb(uint8_t* __restrict__ base, int64_t stride, int expert0, int layer,
                          uint32_t seed, uint32_t scale_kind, uint32_t bias_kind, uint64_t offset,
                          uint64_t n, float s_lo, float s_span, float b_c) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int e = blockIdx.y;
  const uint32_t ex = (uint32_t)(expert0 + e);
  const float s = uniform_map(word_at(i, seed, tensor_id(scale_kind, ex, (uint32_t)layer)), s_lo,
                              s_span);
  const float b = normal_at(i, seed, tensor_id(bias_kind, ex, (uint32_t)layer), b_c);
  uint32_t* dst = reinterpret_cast<uint32_t*>(base + (int64_t)e * stride + offset);
  dst[i] = bf16_rne_bits(s) | (bf16_rne_bits(b) << 16);
}

inline int grid_for(uint64_t n, int bs) { return (int)((n + bs - 1) / bs); }

}  // namespace

extern "C" {

// All functions: device pointers, asynchronous on `stream` (hipStream_t, NULL =
// default stream); return 0, or -1 for bad arguments, -5 for a launch error.

int synth_fill_bytes(void* dst, uint64_t n_bytes, uint32_t seed, uint32_t tid, void* stream) {
  if (!dst || ((uintptr_t)dst & 3)) return -1;
  if (n_bytes == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t n_full = n_bytes / 4;
  if (n_full) {
    const uint64_t blocks = (n_full + 3) / 4;
    hipLaunchKernelGGL(k_fill_words, dim3(grid_for(blocks, 256)), dim3(256), 0, s,
                       (uint32_t*)dst, n_full, seed, tid);
  }
  if (n_bytes & 3)
    hipLaunchKernelGGL(k_fill_tail_bytes, dim3(1), dim3(4), 0, s, (uint8_t*)dst, n_full * 4,
                       n_bytes, seed, tid);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int synth_fill_uniform_f32(float* dst, uint64_t n, uint32_t seed, uint32_t tid, float lo,
                           float span, void* stream) {
  if (!dst) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_fill_uniform_f32, dim3(grid_for(n, 256)), dim3(256), 0,
                     (hipStream_t)stream, dst, n, seed, tid, lo, span);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int synth_fill_normal_f32(float* dst, uint64_t n, uint32_t seed, uint32_t tid, float c,
                          void* stream) {
  if (!dst) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_fill_normal_f32, dim3(grid_for(n, 256)), dim3(256), 0,
                     (hipStream_t)stream, dst, n, seed, tid, c);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int synth_fill_normal_bf16(uint16_t* dst, uint64_t n, uint32_t seed, uint32_t tid, float c,
                           void* stream) {
  if (!dst) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_fill_normal_bf16, dim3(grid_for(n, 256)), dim3(256), 0,
                     (hipStream_t)stream, dst, n, seed, tid, c);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Fill n_experts canonical expert blocks: expert j at base + j*stride, using the
// streams of expert id expert0 + j of `layer`.
int synth_fill_expert_pool(void* base, int64_t stride, int n_experts, int expert0, int layer,
                           uint32_t seed, int hidden, int inter, int bits, float s_lo,
                           float s_span, float b_c, void* stream) {
  if (!base || n_experts < 0 || n_experts > 65535 || expert0 < 0 || expert0 + n_experts > 4096 ||
      layer < 0 || layer >= 4096 || (bits != 2 && bits != 4) || hidden <= 0 || inter <= 0 ||
      hidden % 64 || inter % 64 || ((uintptr_t)base & 3))
    return -1;
  const uint64_t gu_codes = (uint64_t)inter * hidden * bits / 8;
  const uint64_t dn_codes = (uint64_t)hidden * inter * bits / 8;
  const uint64_t gu_sb = (uint64_t)inter * (hidden / 64);  // words
  const uint64_t dn_sb = (uint64_t)hidden * (inter / 64);
  const uint64_t total = 2 * gu_codes + dn_codes + 4 * (2 * gu_sb + dn_sb);
  if (stride < (int64_t)total || (stride & 3)) return -1;
  if (n_experts == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t code_off[3] = {0, gu_codes, 2 * gu_codes};
  const uint64_t code_len[3] = {gu_codes, gu_codes, dn_codes};
  const uint64_t sb0 = 2 * gu_codes + dn_codes;
  const uint64_t sb_off[3] = {sb0, sb0 + 4 * gu_sb, sb0 + 8 * gu_sb};
  const uint64_t sb_len[3] = {gu_sb, gu_sb, dn_sb};
  for (int m = 0; m < 3; ++m) {
    const uint64_t nw = code_len[m] / 4;
    const uint64_t blocks = (nw + 3) / 4;
    hipLaunchKernelGGL(k_pool_codes, dim3(grid_for(blocks, 256), n_experts), dim3(256), 0, s,
                       (uint8_t*)base, stride, expert0, layer, seed, (uint32_t)m, code_off[m], nw);
    hipLaunchKernelGGL(k_pool_sb, dim3(grid_for(sb_len[m], 256), n_experts), dim3(256), 0, s,
                       (uint8_t*)base, stride, expert0, layer, seed, (uint32_t)(3 + m),
                       (uint32_t)(6 + m), sb_off[m], sb_len[m], s_lo, s_span, b_c);
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
