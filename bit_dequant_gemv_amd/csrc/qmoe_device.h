// Device building blocks of libqmoe (gfx950, wave64).
//
// Quantized row dot product.  The page "flash-moe 소개" (discuss.pytorch.kr),
// section "FMA 최적화 역양자화 커널", rewrites (nibble*scale + bias)*x as
// fma(nibble, scale*x, bias*x) so that the dequantisation costs no extra
// instruction per weight.  Here the same identity is applied per group of 64
// inputs,
//
//     sum_k (q_k s + b) x_k  =  s * sum_k q_k x_k  +  b * sum_k x_k ,
//
// so scale and bias cost two FMAs per 32 (4-bit) or 64 (2-bit) weights, and the
// inner sum sum_k q_k x_k is computed with integer dot instructions instead of
// per-weight float conversions:
//
//   * Each 16-byte chunk of a row (32 four-bit or 64 two-bit codes) meets a
//     chunk of x that a lane keeps for the whole matrix.  That x chunk is put in
//     24-bit block fixed point: E is chosen so that |x_k| < 2^E for the chunk,
//     X_k = rint(x_k * 2^(22-E)) (|X_k| <= 2^22) and U_k = X_k + 2^23 lies in
//     [0, 2^24).  U_k is split into six 4-bit digits ("planes").
//   * v_dot8_u32_u4 multiplies eight packed 4-bit codes by eight 4-bit digits and
//     accumulates in 32 bits, exactly.  Six planes give sum_k q_k U_k; one more dot
//     with 0x11111111 gives sum_k q_k, which removes the 2^23 offset.  Nothing is
//     rounded until the per-chunk integer totals are converted to float.
//   * 4-bit codes are used as they sit in memory.  2-bit codes are spread to
//     nibbles with two masks ((w & 0x33333333) << 2 and w & 0xCCCCCCCC), which
//     multiplies every code by 4; the chunk scale carries the 1/4.
// Cost: 7 dot instructions per 8 four-bit codes plus ~14 instructions per chunk,
// about 1.3 VALU instructions per weight, against 2.25 for one float conversion
// and one FMA per weight.  Accuracy: the x chunk keeps 23 significant bits
// relative to its largest element; the integer sums are exact.
//
// Work split: a "lane group" of LG lanes (a power of two <= 64) owns one row at a
// time; lane gl of the group owns the 16-byte chunks gl, gl+LG, ... (CPL of them)
// of every row, so its x planes are loop-invariant and live in VGPRs.  Partial
// row sums of a group are combined with xor shuffles.
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
  static constexpr int EPW = 8;   // codes per 32-bit word
  static constexpr int PW = 24;   // plane words per chunk: 4 code words x 6 digits
  static constexpr float FACTOR = 1.0f;
};
template <>
struct QTraits<2> {
  static constexpr int EPC = 64;
  static constexpr int CPG = 1;
  static constexpr int EPW = 16;
  static constexpr int PW = 48;   // 4 code words x 2 nibble halves x 6 digits
  static constexpr float FACTOR = 0.25f;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// (the hardware reciprocal, within 1 ulp, instead of a full division)
__device__ __forceinline__ float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__device__ __forceinline__ uint32_t udot8(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_udot8(a, b, c, false);
}

// Cross-lane moves without LDS round trips: DPP within 16-lane rows and
// readlane across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each row

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Largest / smallest u32 over the wave (wave-uniform result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return min(a, b);
}

// Order-preserving u32 key of a float's bits (larger key = larger value; -0 is
// mapped to +0 first, so the two zeros tie).  Key 0 means "no expert": no finite
// value maps to it.
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  b = b == 0x80000000u ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Wave-wide arg-max of (key, index) pairs: m = the largest key (0 when every lane
// holds 0, i.e. nothing), wi = the smallest index among the lanes holding m
// (0xFFFFFFFF if none).  Both results are wave-uniform.
__device__ __forceinline__ void wave_argmax(uint32_t k, uint32_t i, uint32_t& m, uint32_t& wi) {
  m = wave_max_u32(k);
  const uint64_t b = __builtin_amdgcn_ballot_w64(k == m && m != 0u);
  if (b == 0)
    wi = 0xFFFFFFFFu;
  else if ((b & (b - 1)) == 0)  // one lane: the common case
    wi = (uint32_t)__builtin_amdgcn_readlane((int)i, __builtin_ctzll(b));
  else  // equal keys: the lower index
    wi = wave_min_u32(k == m ? i : 0xFFFFFFFFu);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over aligned groups of LG lanes (LG a power of two <= 64).  The result is
// valid in the group's first lane (and, for LG <= 16, in every lane of the group).
template <int LG>
__device__ __forceinline__ float group_sum(float v) {
  if (LG >= 2) v += dpp_f<kDppXor1>(v);
  if (LG >= 4) v += dpp_f<kDppXor2>(v);
  if (LG >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (LG >= 16) v += dpp_f<kDppMirror>(v);
  if (LG == 32) {
    const float a = readlane_f(v, 0) + readlane_f(v, 16);
    const float b = readlane_f(v, 32) + readlane_f(v, 48);
    v = (threadIdx.x & 32) ? b : a;
  } else if (LG == 64) {
    v = (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
  }
  return v;
}

// The same sum, valid in the group's last lane (and, for LG <= 16, in every lane
// of the group).  For LG = 32 and 64 the gfx9 DPP row broadcasts carry the row
// sums on (lane 15 of a row into the next row; lane 31 into rows 2 and 3), so no
// value leaves the vector unit.
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
template <int LG>
__device__ __forceinline__ float group_sum_last(float v) {
  if (LG >= 2) v += dpp_f<kDppXor1>(v);
  if (LG >= 4) v += dpp_f<kDppXor2>(v);
  if (LG >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (LG >= 16) v += dpp_f<kDppMirror>(v);
  if (LG >= 32)  // rows 1 and 3 += the last lane of rows 0 and 2
    v += __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast15, 0xA, 0xF, false));
  if (LG >= 64)  // row 3 += lane 31
    v += __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast31, 0x8, 0xF, false));
  return v;
}
template <int LG>
__device__ __forceinline__ bool group_last(int lane) {
  return (lane & (LG - 1)) == LG - 1;
}

// Fixed-point parameters of a chunk with largest magnitude m: f = 2^(22-E) and
// scale = 2^(E-22) where 2^E > m.  A zero (or negligibly small, < 2^-105) chunk
// gets f = scale = 0; a chunk holding Inf/NaN gets scale = NaN.
__device__ __forceinline__ void chunk_exp(float m, float& f, float& scale) {
  const uint32_t e = (__float_as_uint(m) >> 23) & 0xFFu;  // biased exponent of m >= 0
  if (e == 255u) {
    f = 0.f;
    scale = __builtin_nanf("");
  } else if (e <= 21u) {
    f = 0.f;
    scale = 0.f;
  } else {
    f = __uint_as_float((275u - e) << 23);
    scale = __uint_as_float((e - 21u) << 23);
  }
}

// rint(x*f) + 2^23 in two instructions: |x*f| < 2^22 and x*f is exact (f is a power
// of two), so fma(x, f, 1.5*2^23) lands in [2^23, 2^24), where the spacing of
// floats is 1: the single rounding of the fma is round-to-nearest-even of x*f, and
// the float's bits are 0x4B000000 + 2^22 + rint(x*f).  (A chunk with Inf/NaN has
// f = 0 and a NaN scale: its words are don't-cares.)
__device__ __forceinline__ uint32_t to_u24(float x, float f) {
  return __float_as_uint(fmaf(x, f, 12582912.0f)) - 0x4AC00000u;
}

// Nibble transpose of eight 24-bit values: out[d] holds digit d (bits 4d..4d+3) of
// e[j] in nibble j, d = 0..5.  Byte permutes gather byte b of the even and of the
// odd elements (one byte per element), then masks split each gathered byte into
// its low digit (2b) and high digit (2b+1), already in element order.
__device__ __forceinline__ void nibble_planes8(const uint32_t (&e)[8], uint32_t* out) {
  constexpr uint32_t M = 0x0F0F0F0Fu;
  uint32_t E[3], O[3];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const uint32_t a = e[par], b = e[2 + par], c = e[4 + par], d = e[6 + par];
    const uint32_t x01 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a.B0 b.B0 a.B1 b.B1
    const uint32_t y01 = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c.B0 d.B0 c.B1 d.B1
    const uint32_t x2 = __builtin_amdgcn_perm(b, a, 0x0C0C0602u);   // a.B2 b.B2 0 0
    const uint32_t y2 = __builtin_amdgcn_perm(d, c, 0x0C0C0602u);   // c.B2 d.B2 0 0
    uint32_t* g = par ? O : E;
    g[0] = __builtin_amdgcn_perm(y01, x01, 0x05040100u);  // byte 0 of a, b, c, d
    g[1] = __builtin_amdgcn_perm(y01, x01, 0x07060302u);  // byte 1
    g[2] = __builtin_amdgcn_perm(y2, x2, 0x05040100u);    // byte 2
  }
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    out[2 * b] = (E[b] & M) | ((O[b] & M) << 4);
    out[2 * b + 1] = ((E[b] >> 4) & M) | (O[b] & ~M);
  }
}

// Planes of one 32-bit code word worth of x values (v: EPW values, f from chunk_exp).
// 4-bit: out[d], d = 0..5, nibble j = digit d of element j.
// 2-bit: out[h*6 + d]: half h = 0 pairs with (w & 0x33333333) << 2 (elements
// 4b+0, 4b+2 of the word in nibbles 2b, 2b+1), h = 1 with w & 0xCCCCCCCC
// (elements 4b+1, 4b+3).
template <int BITS>
__device__ __forceinline__ void prep_word(const float* v, float f, uint32_t* out) {
  constexpr int EPW = QTraits<BITS>::EPW;
  uint32_t u[EPW];
#pragma unroll
  for (int j = 0; j < EPW; ++j) u[j] = to_u24(v[j], f);
  if (BITS == 4) {
    const uint32_t e[8] = {u[0], u[1], u[2], u[3], u[4], u[5], u[6], u[7]};
    nibble_planes8(e, out);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // nibble k of half h holds element 2k + h of the word
      uint32_t e[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = u[(2 * k + h) % EPW];
      nibble_planes8(e, out + 6 * h);
    }
  }
}

// Integer total of one chunk: sum_k q_k X_k (times 4 for 2-bit codes) as a float.
__device__ __forceinline__ float combine_planes(const uint32_t (&a)[6], uint32_t qs) {
  // Horner form: four shift-adds (each plane sum is < 2^13, so low < 2^30)
  uint32_t low = (a[4] << 4) + a[3];
  low = (low << 4) + a[2];
  low = (low << 4) + a[1];
  low = (low << 4) + a[0];
  const int top = (int)a[5] + (int)qs * -8;
  return fmaf((float)top, 1048576.0f, (float)(int)low);
}

template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4 c, const uint32_t* P);

template <>
__device__ __forceinline__ float chunk_dot<4>(const uint4 c, const uint32_t* P) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t a[6] = {0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t qs = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int d = 0; d < 6; ++d) a[d] = udot8(w[i], P[6 * i + d], a[d]);
    qs = udot8(w[i], 0x11111111u, qs);
  }
  return combine_planes(a, qs);
}

template <>
__device__ __forceinline__ float chunk_dot<2>(const uint4 c, const uint32_t* P) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t a[6] = {0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t qs = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w0 = (w[i] & 0x33333333u) << 2;
    const uint32_t w1 = w[i] & 0xCCCCCCCCu;
#pragma unroll
    for (int d = 0; d < 6; ++d) {
      a[d] = udot8(w0, P[12 * i + d], a[d]);
      a[d] = udot8(w1, P[12 * i + 6 + d], a[d]);
    }
    qs = udot8(w0, 0x11111111u, qs);
    qs = udot8(w1, 0x11111111u, qs);
  }
  return combine_planes(a, qs);
}

// The planes of word w (EPW values v, zeros when !valid) of an input vector, the
// chunk scale and the chunk sum: lanes w..w+3 of one DPP quad hold the 4 words of
// a chunk, and all four must call this together.
template <int BITS, int STRIDE = QTraits<BITS>::PW>
__device__ __forceinline__ void prep_x_word(const float (&v)[QTraits<BITS>::EPW], bool valid, int w,
                                            uint32_t* planes, float* scl, float* xsum) {
  constexpr int EPW = QTraits<BITS>::EPW;
  constexpr int NPW = BITS == 4 ? 6 : 12;  // plane words per code word
  float m = 0.f, s = 0.f;
#pragma unroll
  for (int j = 0; j < EPW; j += 4) {
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j]), fabsf(v[j + 1])), fmaxf(fabsf(v[j + 2]), fabsf(v[j + 3]))));
    s += (v[j] + v[j + 1]) + (v[j + 2] + v[j + 3]);
  }
  // a chunk is 4 consecutive words = 4 consecutive lanes (one DPP quad)
  m = fmaxf(m, dpp_f<kDppXor1>(m));
  m = fmaxf(m, dpp_f<kDppXor2>(m));
  s += dpp_f<kDppXor1>(s);
  s += dpp_f<kDppXor2>(s);
  float f, scale;
  chunk_exp(m, f, scale);
  if (valid) {
    uint32_t p[NPW];
    prep_word<BITS>(v, f, p);
    const int c = w >> 2, i = w & 3;
#pragma unroll
    for (int k = 0; k < NPW; ++k) planes[c * STRIDE + i * NPW + k] = p[k];
    if (i == 0) {
      scl[c] = scale * QTraits<BITS>::FACTOR;
      xsum[c] = s;
    }
  }
}

// Workgroup-cooperative preparation of the x planes of a whole input vector into
// shared memory: planes[c*PW ...], scl[c] (chunk scale, 2-bit 1/4 included) and
// xsum[c] (plain sum of the chunk's x) for chunks c < n/EPC.  Every thread of the
// workgroup must call it (shuffles inside); nthreads a multiple of 64.
template <int BITS, int STRIDE = QTraits<BITS>::PW>
__device__ __forceinline__ void prep_x_coop(const float* x, int n, uint32_t* planes, float* scl,
                                            float* xsum, int tid, int nthreads) {
  constexpr int EPW = QTraits<BITS>::EPW;
  const int words = n / EPW;
  for (int w0 = 0; w0 < words; w0 += nthreads) {
    const int w = w0 + tid;
    const bool valid = w < words;
    float v[EPW];
#pragma unroll
    for (int j = 0; j < EPW; j += 4) {
      float4 f4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (valid) f4 = *reinterpret_cast<const float4*>(x + (int64_t)w * EPW + j);
      v[j] = f4.x;
      v[j + 1] = f4.y;
      v[j + 2] = f4.z;
      v[j + 3] = f4.w;
    }
    prep_x_word<BITS, STRIDE>(v, valid, w, planes, scl, xsum);
  }
}

// Float form of the chunk dot (one v_cvt_f32_ubyteN and one FMA per code), used
// where an input vector meets too few rows to repay building its planes.  The
// odd (4-bit) or 4^m-position (2-bit) x values are stored pre-divided by 16 or
// 4^m (exact), so each code is converted straight from its byte position.
__device__ __forceinline__ float ubyte_f(uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xFFu); }

// Hide a masked word from the optimiser, which would otherwise fold the mask
// into each byte extraction and lose the single-instruction conversion.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

template <int BITS>
__device__ __forceinline__ float xscale_f(int e) {
  if (BITS == 4) return (e & 1) ? 0.0625f : 1.0f;
  const int m = e & 3;
  return m == 0 ? 1.0f : (m == 1 ? 0.25f : (m == 2 ? 0.0625f : 0.015625f));
}

template <int BITS>
__device__ __forceinline__ float chunk_dot_f(const uint4 c, const float* xr);

template <>
__device__ __forceinline__ float chunk_dot_f<4>(const uint4 c, const float* xr) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float a[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = opaque(w[i] & 0x0F0F0F0Fu);
    const uint32_t hi = opaque(w[i] & 0xF0F0F0F0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[(j & 1) * 2] = fmaf(ubyte_f(lo, j), xr[8 * i + 2 * j], a[(j & 1) * 2]);
      a[(j & 1) * 2 + 1] = fmaf(ubyte_f(hi, j), xr[8 * i + 2 * j + 1], a[(j & 1) * 2 + 1]);
    }
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

template <>
__device__ __forceinline__ float chunk_dot_f<2>(const uint4 c, const float* xr) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t v = opaque(w[i] & (0x03030303u << (2 * m)));
#pragma unroll
      for (int j = 0; j < 4; ++j) a[m] = fmaf(ubyte_f(v, j), xr[16 * i + 4 * j + m], a[m]);
    }
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// A lane's single chunk of x in float form (CPL = 1) and its row dots.
template <int BITS, int LG>
struct RowDotF {
  static constexpr int EPC = QTraits<BITS>::EPC;
  float xr[EPC];
  float xs;

  __device__ __forceinline__ void load_x(const float* x, int C, int gl) {
    xs = 0.f;
    if (gl < C) {
      const float4* p = reinterpret_cast<const float4*>(x + gl * EPC);
#pragma unroll
      for (int v = 0; v < EPC / 4; ++v) {
        const float4 f = p[v];
        xr[4 * v + 0] = f.x * xscale_f<BITS>(4 * v + 0);
        xr[4 * v + 1] = f.y * xscale_f<BITS>(4 * v + 1);
        xr[4 * v + 2] = f.z * xscale_f<BITS>(4 * v + 2);
        xr[4 * v + 3] = f.w * xscale_f<BITS>(4 * v + 3);
        xs += (f.x + f.y) + (f.z + f.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) xr[e] = 0.f;
    }
  }

  // lane partial of one row: s = scale|bias word of the lane's group (0 = no row)
  __device__ __forceinline__ float dot(const uint4 q, uint32_t s) const {
    return fmaf(bf16_lo(s), chunk_dot_f<BITS>(q, xr), bf16_hi(s) * xs);
  }
};

// Streaming loads of weights: non-temporal (the nt cache policy), so a stream that
// is read once does not displace reused lines from the caches.  On gfx950 this
// also raises the sustained read rate of a long weight stream (measured: 4.8 ->
// 6.2 TB/s for a 288 MB 4-bit matrix).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream4(const uint32_t* p) {
  return __builtin_nontemporal_load(p);
}

// A lane's slice of x (as fixed-point planes) for one matrix, and the row dots.
template <int BITS, int LG, int CPL>
struct RowDot {
  static constexpr int EPC = QTraits<BITS>::EPC;
  static constexpr int PW = QTraits<BITS>::PW;
  uint32_t P[CPL][PW];
  float sc[CPL];
  float xs[CPL];

  // x: the input vector (global or LDS); prepares the lane's own chunks
  __device__ __forceinline__ void load_x(const float* x, int C, int gl) {
    constexpr int EPW = QTraits<BITS>::EPW;
    constexpr int NPW = BITS == 4 ? 6 : 12;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = gl + i * LG;
      if (c < C) {
        const float* xc = x + c * EPC;
        float m = 0.f, s = 0.f;
#pragma unroll
        for (int j = 0; j < EPC; j += 4) {
          const float4 f4 = *reinterpret_cast<const float4*>(xc + j);
          m = fmaxf(m, fmaxf(fmaxf(fabsf(f4.x), fabsf(f4.y)), fmaxf(fabsf(f4.z), fabsf(f4.w))));
          s += (f4.x + f4.y) + (f4.z + f4.w);
        }
        float f, scale;
        chunk_exp(m, f, scale);
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          float v[EPW];
#pragma unroll
          for (int j = 0; j < EPW; j += 4) {
            const float4 f4 = *reinterpret_cast<const float4*>(xc + wd * EPW + j);
            v[j] = f4.x;
            v[j + 1] = f4.y;
            v[j + 2] = f4.z;
            v[j + 3] = f4.w;
          }
          prep_word<BITS>(v, f, &P[i][wd * NPW]);
        }
        sc[i] = scale * QTraits<BITS>::FACTOR;
        xs[i] = s;
      } else {
#pragma unroll
        for (int k = 0; k < PW; ++k) P[i][k] = 0u;
        sc[i] = 0.f;
        xs[i] = 0.f;
      }
    }
  }

  // planes prepared by prep_x_coop (shared or global memory)
  template <int STRIDE = PW>
  __device__ __forceinline__ void load_prepped(const uint32_t* planes, const float* scl,
                                               const float* xsum, int C, int gl) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = gl + i * LG;
      if (c < C) {
        const uint4* p = reinterpret_cast<const uint4*>(planes + c * STRIDE);
#pragma unroll
        for (int k = 0; k < PW / 4; ++k) {
          const uint4 v = p[k];
          P[i][4 * k] = v.x;
          P[i][4 * k + 1] = v.y;
          P[i][4 * k + 2] = v.z;
          P[i][4 * k + 3] = v.w;
        }
        sc[i] = scl[c];
        xs[i] = xsum[c];
      } else {
#pragma unroll
        for (int k = 0; k < PW; ++k) P[i][k] = 0u;
        sc[i] = 0.f;
        xs[i] = 0.f;
      }
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
        if (ok[r] && c < C) {  // unsigned lane offsets: a scalar row base plus a 32-bit offset
          q[r][i] = ld_stream16(crow[r] + 16u * (uint32_t)c);
          s[r][i] = ld_stream4(srow[r] + (uint32_t)c / QTraits<BITS>::CPG);
        } else {
          q[r][i] = make_uint4(0u, 0u, 0u, 0u);
          s[r][i] = 0u;
        }
      }
    }
  }

  // The same loads without per-row conditions: every row pointer is valid and
  // every chunk gl + i*LG is < C (the caller guarantees both).  A straight run
  // of loads lets each row's dots wait only for that row's data.
  template <int R>
  __device__ __forceinline__ void fetch_always(const uint8_t* const* crow,
                                               const uint32_t* const* srow, int gl,
                                               uint4 (&q)[R][CPL], uint32_t (&s)[R][CPL]) const {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint32_t c = (uint32_t)(gl + i * LG);
        q[r][i] = ld_stream16(crow[r] + 16u * c);
        s[r][i] = ld_stream4(srow[r] + c / QTraits<BITS>::CPG);
      }
    }
  }

  // Loads with no conditions at all: a chunk past the row (gl + i*LG >= C) reads the
  // row's last chunk instead, which adds nothing since the x planes of such a chunk
  // are zero (load_x / load_prepped); every row pointer must be valid.
  template <int R>
  __device__ __forceinline__ void fetch_clamped(const uint8_t* const* crow,
                                                const uint32_t* const* srow, int C, int gl,
                                                uint4 (&q)[R][CPL], uint32_t (&s)[R][CPL]) const {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint32_t c = (uint32_t)min(gl + i * LG, C - 1);
        q[r][i] = ld_stream16(crow[r] + 16u * c);
        s[r][i] = ld_stream4(srow[r] + c / QTraits<BITS>::CPG);
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
        const float d = chunk_dot<BITS>(q[r][i], P[i]);
        acc = fmaf(bf16_lo(s[r][i]) * sc[i], d, acc);
        acc = fmaf(bf16_hi(s[r][i]), xs[i], acc);
      }
      out[r] = acc;
    }
  }
};

}  // namespace qmoe
