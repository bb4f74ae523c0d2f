// Device building blocks of libqmoe (gfx950, wave64).
//
// Quantized row dot product.  The page "flash-moe 소개" (discuss.pytorch.kr),
// section "FMA 최적화 역양자화 커널", rewrites (nibble*scale + bias)*x as
// fma(nibble, scale*x, bias*x) so that the inner loop is one FMA per weight.
// Here the same identity is taken one step further, per group of 64 inputs:
//
//     sum_k (q_k s + b) x_k  =  s * sum_k q_k x_k  +  b * sum_k x_k
//
// sum_k x_k of a lane's inputs is fixed for a whole matrix, so the inner loop is
// one code conversion and one FMA per weight, and scale and bias cost two FMAs
// per 32 (4-bit) or 64 (2-bit) weights.
//
// Work split: a "lane group" of LG lanes (a power of two <= 64) owns one row at
// a time; lane gl of the group owns the 16-byte chunks gl, gl+LG, ... (CPL of
// them) of every row, so its slice of x is loop-invariant and lives in VGPRs,
// pre-scaled so that a code can be converted straight from its byte position:
//   4-bit: a chunk holds 32 codes.  w & 0x0F0F0F0F leaves the even codes as
//          bytes, w & 0xF0F0F0F0 leaves 16 * (odd codes) as bytes; each byte
//          becomes a float in one v_cvt_f32_ubyteN, and the odd x are stored
//          divided by 16 (exact).
//   2-bit: a chunk holds 64 codes = one group; masks 0x03.., 0x0C.., 0x30..,
//          0xC0.. leave 4^m * code; the matching x are stored divided by 4^m.
// The per-row partial sums of a group are combined with xor shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

constexpr int kGroup = 64;

template <int BITS>
struct QTraits;
template <>
struct QTraits<4> {
  static constexpr int EPC = 32;  // codes per 16-byte chunk
  static constexpr int CPG = 2;   // chunks per group of 64
};
template <>
struct QTraits<2> {
  static constexpr int EPC = 64;
  static constexpr int CPG = 1;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// byte j of v as a float (the backend selects v_cvt_f32_ubyteJ)
__device__ __forceinline__ float ubyte_f(uint32_t v, int j) {
  return (float)((v >> (8 * j)) & 0xFFu);
}

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }
__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// sum over aligned groups of LG lanes (LG a power of two <= 64)
template <int LG>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = LG >> 1; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// dot of one 16-byte chunk of codes with the matching pre-scaled x
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4 c, const float* xr);

template <>
__device__ __forceinline__ float chunk_dot<4>(const uint4 c, const float* xr) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = w[i] & 0x0F0F0F0Fu;
    const uint32_t hi = w[i] & 0xF0F0F0F0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a0 = fmaf(ubyte_f(lo, j), xr[8 * i + 2 * j], a0);
      a1 = fmaf(ubyte_f(hi, j), xr[8 * i + 2 * j + 1], a1);
    }
  }
  return a0 + a1;
}

template <>
__device__ __forceinline__ float chunk_dot<2>(const uint4 c, const float* xr) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t v = w[i] & (0x03030303u << (2 * m));
#pragma unroll
      for (int j = 0; j < 4; ++j) a[m] = fmaf(ubyte_f(v, j), xr[16 * i + 4 * j + m], a[m]);
    }
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// scale applied to x element e of a chunk so the raw byte position can be used
template <int BITS>
__device__ __forceinline__ float xscale(int e) {
  if (BITS == 4) return (e & 1) ? 0.0625f : 1.0f;
  const int m = e & 3;
  return m == 0 ? 1.0f : (m == 1 ? 0.25f : (m == 2 ? 0.0625f : 0.015625f));
}

// A lane's slice of x for one matrix and the dot products of its rows.
template <int BITS, int LG, int CPL>
struct RowDot {
  static constexpr int EPC = QTraits<BITS>::EPC;
  float xr[CPL][EPC];
  float xs[CPL];

  // x: the input vector (global or LDS), C: 16-byte chunks per row, gl: lane in group
  __device__ __forceinline__ void load_x(const float* x, int C, int gl) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = gl + i * LG;
      float s = 0.f;
      if (c < C) {
        const float4* p = reinterpret_cast<const float4*>(x + c * EPC);
#pragma unroll
        for (int v = 0; v < EPC / 4; ++v) {
          const float4 f = p[v];
          xr[i][4 * v + 0] = f.x * xscale<BITS>(4 * v + 0);
          xr[i][4 * v + 1] = f.y * xscale<BITS>(4 * v + 1);
          xr[i][4 * v + 2] = f.z * xscale<BITS>(4 * v + 2);
          xr[i][4 * v + 3] = f.w * xscale<BITS>(4 * v + 3);
          s += (f.x + f.y) + (f.z + f.w);
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) xr[i][e] = 0.f;
      }
      xs[i] = s;
    }
  }

  // Issue the loads of R rows: codes row pointers and sb row pointers; rows with
  // ok[r] == false (and chunks >= C) read nothing and contribute zero.
  template <int R>
  __device__ __forceinline__ void fetch(const uint8_t* const* crow, const uint32_t* const* srow,
                                        const bool* ok, int C, int gl, uint4 (&q)[R][CPL],
                                        uint32_t (&s)[R][CPL]) const {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = gl + i * LG;
        if (ok[r] && c < C) {
          q[r][i] = *reinterpret_cast<const uint4*>(crow[r] + 16 * c);
          s[r][i] = srow[r][c / QTraits<BITS>::CPG];
        } else {
          q[r][i] = make_uint4(0u, 0u, 0u, 0u);
          s[r][i] = 0u;
        }
      }
    }
  }

  // Lane partial sums of R fetched rows (before the group reduction).
  template <int R>
  __device__ __forceinline__ void dots(const uint4 (&q)[R][CPL], const uint32_t (&s)[R][CPL],
                                       float (&out)[R]) const {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const float d = chunk_dot<BITS>(q[r][i], xr[i]);
        acc = fmaf(bf16_lo(s[r][i]), d, acc);
        acc = fmaf(bf16_hi(s[r][i]), xs[i], acc);
      }
      out[r] = acc;
    }
  }
};

}  // namespace qmoe
