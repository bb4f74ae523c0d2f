// Stand-alone kernels of libqmoe: quantized GEMV, expert FFN with SwiGLU,
// router GEMV + top-K, combine, RMSNorm.  (The fused single-launch layer lives in
// layer.hip.)  Sources: "flash-moe 소개" (discuss.pytorch.kr), sections
// "FMA 최적화 역양자화 커널" and "손으로 작성한 Metal 컴퓨트 셰이더".
#include <math.h>

#include <algorithm>

#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kBlock = 256;  // 4 waves

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// rows per lane-group pass, by loads per lane: keep about four 16-byte loads in flight
template <int CPL>
struct RowsPerPass {
  static constexpr int R = CPL >= 4 ? 1 : (CPL == 2 ? 2 : 4);
};

// x planes of the whole input prepared once per workgroup in dynamic LDS, then
// each lane takes its chunks' planes.  LDS: C*PW words of planes, C scales, C sums.
template <int BITS, int LG, int CPL>
__device__ __forceinline__ void load_x_shared(RowDot<BITS, LG, CPL>& rd, const float* x, int n, int C,
                                              int gl) {
  extern __shared__ uint32_t smem[];
  uint32_t* planes = smem;
  float* scl = reinterpret_cast<float*>(smem + C * QTraits<BITS>::PW);
  float* xsum = scl + C;
  prep_x_coop<BITS>(x, n, planes, scl, xsum, threadIdx.x, blockDim.x);
  __syncthreads();
  rd.load_prepped(planes, scl, xsum, C, gl);
}

template <int BITS>
inline size_t prep_lds_bytes(int n) {
  const int C = n / QTraits<BITS>::EPC;
  return (size_t)C * (QTraits<BITS>::PW + 2) * 4;
}

// The input vector of an expert FFN kernel, with the weight rows' loads issued in
// between (fetch): the n inputs are loaded into registers first, unconditionally
// (kXW words of 8 per thread, a thread past the end reading the last word again),
// then the rows; then the inputs are staged in dynamic LDS after the planes and
// the planes are built there while the rows are still on their way, and each lane
// takes its chunks' planes.  Vector memory completes in issue order, and a
// straight run of loads lets each use wait for its own data only.
constexpr int kXW = 4;  // words per thread: n <= 8 * kXW * kBlock = 8192 inputs
template <int BITS, int LG, int CPL, typename Fetch>
__device__ __forceinline__ void x_planes_around(RowDot<BITS, LG, CPL>& rd, const float* x, int n,
                                                int C, int gl, Fetch fetch) {
  extern __shared__ uint32_t smem[];
  const int words = n / 8;
  float4 xr[2 * kXW];
#pragma unroll
  for (int k = 0; k < kXW; ++k) {
    const int w = min((int)threadIdx.x + k * kBlock, words - 1);
    xr[2 * k] = reinterpret_cast<const float4*>(x + 8 * w)[0];
    xr[2 * k + 1] = reinterpret_cast<const float4*>(x + 8 * w)[1];
  }
  fetch();  // (a scheduling barrier here would push xr to scratch memory)
  uint32_t* planes = smem;
  float* scl = reinterpret_cast<float*>(smem + C * QTraits<BITS>::PW);
  float* xsum = scl + C;
  float* xs = xsum + C;  // staged inputs
#pragma unroll
  for (int k = 0; k < kXW; ++k) {  // a clamped thread writes the last word again, unchanged
    const int w = min((int)threadIdx.x + k * kBlock, words - 1);
    reinterpret_cast<float4*>(xs + 8 * w)[0] = xr[2 * k];
    reinterpret_cast<float4*>(xs + 8 * w)[1] = xr[2 * k + 1];
  }
  __syncthreads();
  prep_x_coop<BITS>(xs, n, planes, scl, xsum, threadIdx.x, blockDim.x);
  __syncthreads();
  rd.load_prepped(planes, scl, xsum, C, gl);
}

template <int BITS>
inline size_t ffn_lds_bytes(int n) {
  return prep_lds_bytes<BITS>(n) + (size_t)n * 4;
}

// ---------------------------------------------------------------------------
// y = W x
// A persistent grid (a few workgroups per CU) walks the rows; each wave keeps the
// next R rows' loads in flight while it reduces the current ones.
// ---------------------------------------------------------------------------
template <int BITS, int LG, int CPL, int R>
__global__ __launch_bounds__(kBlock) void k_qgemv(const uint8_t* __restrict__ codes,
                                                  const uint32_t* __restrict__ sb,
                                                  const float* __restrict__ x,
                                                  float* __restrict__ y, int rows, int cols) {
  constexpr int RPW = 64 / LG;
  const int C = cols * BITS / 128;
  const int G = cols / kGroup;
  const int64_t rowbytes = (int64_t)cols * BITS / 8;
  const int lane = threadIdx.x & 63;
  const int gl = lane % LG, sub = lane / LG;
  RowDot<BITS, LG, CPL> rd;
  load_x_shared<BITS, LG, CPL>(rd, x, cols, C, gl);
  const int64_t step = (int64_t)gridDim.x * (kBlock / 64) * RPW * R;
  // Unconditional loads (a row past the end reads the last row, which every such
  // wave shares in cache), so that the dots of one pass wait only for that pass's
  // rows and the next pass's loads stay in flight meanwhile.
  auto fetch_rows = [&](int64_t base, uint4 (&q)[R][CPL], uint32_t (&s)[R][CPL]) {
    const uint8_t* crow[R];
    const uint32_t* srow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = min(base + r * RPW + sub, (int64_t)rows - 1);
      crow[r] = codes + row * rowbytes;
      srow[r] = sb + row * G;
    }
    rd.template fetch_clamped<R>(crow, srow, C, gl, q, s);
  };
  int64_t base = ((int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6)) * RPW * R;
  uint4 q[R][CPL];
  uint32_t s[R][CPL];
  if (base < rows) fetch_rows(base, q, s);
  for (; base < rows; base += step) {
    uint4 qn[R][CPL];
    uint32_t sn[R][CPL];
    fetch_rows(base + step, qn, sn);
    float p[R];
    rd.template dots<R>(q, s, p);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = group_sum<LG>(p[r]);
      if (gl == 0 && base + r * RPW + sub < rows) y[base + r * RPW + sub] = v;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        q[r][i] = qn[r][i];
        s[r][i] = sn[r][i];
      }
  }
}

// workgroups per CU for the persistent stand-alone GEMV (measured best: 4)
constexpr int kQgemvBlocksPerCU = 4;

template <int BITS, int LG, int CPL>
hipError_t run_qgemv(const uint8_t* codes, const uint32_t* sb, const float* x, float* y, int rows,
                     int cols, hipStream_t s) {
  constexpr int R = RowsPerPass<CPL>::R;
  const int64_t waves = (rows + (64 / LG) * R - 1) / ((64 / LG) * R);
  const int cus = device_cus();
  const int64_t cap = (int64_t)kQgemvBlocksPerCU * (cus > 0 ? cus : 256);
  const int blocks = (int)std::min<int64_t>(ceil_div(waves, 4), cap);
  hipLaunchKernelGGL((k_qgemv<BITS, LG, CPL, R>), dim3(blocks), dim3(kBlock),
                     prep_lds_bytes<BITS>(cols), s, codes, sb, x, y, rows, cols);
  return hipGetLastError();
}

template <int BITS>
hipError_t dispatch_qgemv(const uint8_t* codes, const uint32_t* sb, const float* x, float* y,
                          int rows, int cols, hipStream_t s) {
  const int C = cols * BITS / 128;
  if (C <= 1) return run_qgemv<BITS, 1, 1>(codes, sb, x, y, rows, cols, s);
  if (C <= 2) return run_qgemv<BITS, 2, 1>(codes, sb, x, y, rows, cols, s);
  if (C <= 4) return run_qgemv<BITS, 4, 1>(codes, sb, x, y, rows, cols, s);
  if (C <= 8) return run_qgemv<BITS, 8, 1>(codes, sb, x, y, rows, cols, s);
  if (C <= 16) return run_qgemv<BITS, 16, 1>(codes, sb, x, y, rows, cols, s);
  if (C <= 32) return run_qgemv<BITS, 32, 1>(codes, sb, x, y, rows, cols, s);
  if (C <= 64) return run_qgemv<BITS, 64, 1>(codes, sb, x, y, rows, cols, s);
  if (C <= 128) return run_qgemv<BITS, 64, 2>(codes, sb, x, y, rows, cols, s);
  return run_qgemv<BITS, 64, 4>(codes, sb, x, y, rows, cols, s);
}

// ---------------------------------------------------------------------------
// Expert FFN: h = silu(G x) * (U x), then y = D h, experts chosen on the device
// ---------------------------------------------------------------------------
struct PoolArgs {
  const uint8_t* base;
  int64_t stride;
  int E, H, I;
  int64_t off_g, off_u, off_d, off_gsb, off_usb, off_dsb;
};

inline PoolArgs pool_args(const qmoe_expert_pool& p) {
  const qmoe_expert_offsets o = expert_offsets(p.hidden, p.inter, p.bits);
  PoolArgs a;
  a.base = static_cast<const uint8_t*>(p.base);
  a.stride = p.stride;
  a.E = p.num_experts;
  a.H = p.hidden;
  a.I = p.inter;
  a.off_g = o.gate_codes;
  a.off_u = o.up_codes;
  a.off_d = o.down_codes;
  a.off_gsb = o.gate_sb;
  a.off_usb = o.up_sb;
  a.off_dsb = o.down_sb;
  return a;
}

// grid.y = expert slot; x of slot i at x + i*x_stride; h[i][I] written
template <int BITS, int LG, int CPL, int R>
__global__ __launch_bounds__(kBlock) void k_ffn_gateup(PoolArgs P, const int32_t* __restrict__ idx,
                                                       const float* x,  // not restrict: see x_planes_around
                                                       int64_t x_stride, float* __restrict__ h) {
  constexpr int RPW = 64 / LG;
  const int slot = blockIdx.y;
  const int e = idx[slot];
  const bool eok = (unsigned)e < (unsigned)P.E;
  const int C = P.H * BITS / 128;
  const int G = P.H / kGroup;
  const int64_t rowbytes = (int64_t)P.H * BITS / 8;
  const uint8_t* blk = P.base + (eok ? (int64_t)e * P.stride : 0);
  const uint8_t* gc = blk + P.off_g;
  const uint8_t* uc = blk + P.off_u;
  const uint32_t* gs = reinterpret_cast<const uint32_t*>(blk + P.off_gsb);
  const uint32_t* us = reinterpret_cast<const uint32_t*>(blk + P.off_usb);
  const int lane = threadIdx.x & 63;
  const int gl = lane % LG, sub = lane / LG;
  RowDot<BITS, LG, CPL> rd;
  // a pass's rows, unconditionally (a row past the end reads the last one)
  auto fetch = [&](int base, uint4 (&q)[2 * R][CPL], uint32_t (&s)[2 * R][CPL]) {
    const uint8_t* crow[2 * R];
    const uint32_t* srow[2 * R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = min(base + r * RPW + sub, P.I - 1);
      crow[2 * r] = gc + j * rowbytes;
      crow[2 * r + 1] = uc + j * rowbytes;
      srow[2 * r] = gs + (int64_t)j * G;
      srow[2 * r + 1] = us + (int64_t)j * G;
    }
    rd.template fetch_clamped<2 * R>(crow, srow, C, gl, q, s);
  };
  const int nw = gridDim.x * (kBlock / 64);
  int base = (blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6)) * RPW * R;
  uint4 q[2 * R][CPL];
  uint32_t s[2 * R][CPL];
  // the first pass's rows go out between the loads and the planes of x
  x_planes_around<BITS, LG, CPL>(rd, x + slot * x_stride, P.H, C, gl, [&] { fetch(base, q, s); });
  for (bool first = true; base < P.I; base += nw * RPW * R, first = false) {
    if (!first) fetch(base, q, s);
    float p[2 * R];
    rd.template dots<2 * R>(q, s, p);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float a = group_sum<LG>(p[2 * r]);
      const float u = group_sum<LG>(p[2 * r + 1]);
      const int j = base + r * RPW + sub;
      if (gl == 0 && j < P.I) h[(int64_t)slot * P.I + j] = eok ? silu_f(a) * u : __builtin_nanf("");
    }
  }
}

// grid.y = expert slot; input h[slot], output y[slot][H]
template <int BITS, int LG, int CPL, int R>
__global__ __launch_bounds__(kBlock) void k_ffn_down(PoolArgs P, const int32_t* __restrict__ idx,
                                                     const float* h,  // not restrict: see x_planes_around
                                                     float* __restrict__ y) {
  constexpr int RPW = 64 / LG;
  const int slot = blockIdx.y;
  const int e = idx[slot];
  const bool eok = (unsigned)e < (unsigned)P.E;
  const int C = P.I * BITS / 128;
  const int G = P.I / kGroup;
  const int64_t rowbytes = (int64_t)P.I * BITS / 8;
  const uint8_t* blk = P.base + (eok ? (int64_t)e * P.stride : 0);
  const uint8_t* dc = blk + P.off_d;
  const uint32_t* ds = reinterpret_cast<const uint32_t*>(blk + P.off_dsb);
  const int lane = threadIdx.x & 63;
  const int gl = lane % LG, sub = lane / LG;
  RowDot<BITS, LG, CPL> rd;
  auto fetch = [&](int base, uint4 (&q)[R][CPL], uint32_t (&s)[R][CPL]) {
    const uint8_t* crow[R];
    const uint32_t* srow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = min(base + r * RPW + sub, P.H - 1);
      crow[r] = dc + n * rowbytes;
      srow[r] = ds + (int64_t)n * G;
    }
    rd.template fetch_clamped<R>(crow, srow, C, gl, q, s);
  };
  const int nw = gridDim.x * (kBlock / 64);
  int base = (blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6)) * RPW * R;
  uint4 q[R][CPL];
  uint32_t s[R][CPL];
  // the first pass's rows go out between the loads and the planes of h
  x_planes_around<BITS, LG, CPL>(rd, h + (int64_t)slot * P.I, P.I, C, gl, [&] { fetch(base, q, s); });
  for (bool first = true; base < P.H; base += nw * RPW * R, first = false) {
    if (!first) fetch(base, q, s);
    float p[R];
    rd.template dots<R>(q, s, p);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = group_sum<LG>(p[r]);
      const int n = base + r * RPW + sub;
      if (gl == 0 && n < P.H) y[(int64_t)slot * P.H + n] = eok ? v : __builtin_nanf("");
    }
  }
}

template <int BITS, int LG, int CPL>
hipError_t run_gateup(const PoolArgs& P, const int32_t* idx, int n, const float* x,
                      int64_t x_stride, float* h, hipStream_t s) {
  constexpr int R = RowsPerPass<CPL>::R > 1 ? RowsPerPass<CPL>::R / 2 : 1;
  const int waves = ceil_div(P.I, (64 / LG) * R);
  hipLaunchKernelGGL((k_ffn_gateup<BITS, LG, CPL, R>), dim3(ceil_div(waves, 4), n), dim3(kBlock),
                     ffn_lds_bytes<BITS>(P.H), s, P, idx, x, x_stride, h);
  return hipGetLastError();
}

template <int BITS, int LG, int CPL>
hipError_t run_down(const PoolArgs& P, const int32_t* idx, int n, const float* h, float* y,
                    hipStream_t s) {
  // half the rows per pass of the stand-alone GEMV: twice the workgroups, every
  // CU busy for one expert (measured: 8.59 -> 8.22 us per expert FFN call)
  constexpr int R = RowsPerPass<CPL>::R > 1 ? RowsPerPass<CPL>::R / 2 : 1;
  const int waves = ceil_div(P.H, (64 / LG) * R);
  hipLaunchKernelGGL((k_ffn_down<BITS, LG, CPL, R>), dim3(ceil_div(waves, 4), n), dim3(kBlock),
                     ffn_lds_bytes<BITS>(P.I), s, P, idx, h, y);
  return hipGetLastError();
}

template <int BITS>
hipError_t dispatch_gateup(const PoolArgs& P, const int32_t* idx, int n, const float* x,
                           int64_t xs, float* h, hipStream_t s) {
  const int C = P.H * BITS / 128;
  if (C <= 1) return run_gateup<BITS, 1, 1>(P, idx, n, x, xs, h, s);
  if (C <= 2) return run_gateup<BITS, 2, 1>(P, idx, n, x, xs, h, s);
  if (C <= 4) return run_gateup<BITS, 4, 1>(P, idx, n, x, xs, h, s);
  if (C <= 8) return run_gateup<BITS, 8, 1>(P, idx, n, x, xs, h, s);
  if (C <= 16) return run_gateup<BITS, 16, 1>(P, idx, n, x, xs, h, s);
  if (C <= 32) return run_gateup<BITS, 32, 1>(P, idx, n, x, xs, h, s);
  if (C <= 64) return run_gateup<BITS, 64, 1>(P, idx, n, x, xs, h, s);
  if (C <= 128) return run_gateup<BITS, 64, 2>(P, idx, n, x, xs, h, s);
  return run_gateup<BITS, 64, 4>(P, idx, n, x, xs, h, s);
}

template <int BITS>
hipError_t dispatch_down(const PoolArgs& P, const int32_t* idx, int n, const float* h, float* y,
                         hipStream_t s) {
  const int C = P.I * BITS / 128;
  if (C <= 1) return run_down<BITS, 1, 1>(P, idx, n, h, y, s);
  if (C <= 2) return run_down<BITS, 2, 1>(P, idx, n, h, y, s);
  if (C <= 4) return run_down<BITS, 4, 1>(P, idx, n, h, y, s);
  if (C <= 8) return run_down<BITS, 8, 1>(P, idx, n, h, y, s);
  if (C <= 16) return run_down<BITS, 16, 1>(P, idx, n, h, y, s);
  if (C <= 32) return run_down<BITS, 32, 1>(P, idx, n, h, y, s);
  if (C <= 64) return run_down<BITS, 64, 1>(P, idx, n, h, y, s);
  if (C <= 128) return run_down<BITS, 64, 2>(P, idx, n, h, y, s);
  return run_down<BITS, 64, 4>(P, idx, n, h, y, s);
}

// ---------------------------------------------------------------------------
// Router GEMV (bf16 [E][H] times fp32 x) and top-K with renormalised softmax
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_chunk_dot(const uint4 c, const float* xr) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0 = fmaf(bf16_lo(w[i]), xr[2 * i], a0);
    a1 = fmaf(bf16_hi(w[i]), xr[2 * i + 1], a1);
  }
  return a0 + a1;
}

// grid (row blocks, T); each lane group owns one router row at a time
template <int LG, int CPL>
__global__ __launch_bounds__(kBlock) void k_router(const uint16_t* __restrict__ router,
                                                   const float* __restrict__ x,
                                                   float* __restrict__ logits, int E, int H) {
  constexpr int RPW = 64 / LG;
  const int t = blockIdx.y;
  const int C = H / 8;
  const int lane = threadIdx.x & 63;
  const int gl = lane % LG, sub = lane / LG;
  float xr[CPL][8];
  const float* xt = x + (int64_t)t * H;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = gl + i * LG;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < C) f = reinterpret_cast<const float4*>(xt + 8 * c)[v];
      xr[i][4 * v + 0] = f.x;
      xr[i][4 * v + 1] = f.y;
      xr[i][4 * v + 2] = f.z;
      xr[i][4 * v + 3] = f.w;
    }
  }
  const int nw = gridDim.x * (kBlock / 64);
  for (int base = (blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6)) * RPW; base < E;
       base += nw * RPW) {
    const int e = base + sub;
    uint4 q[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = gl + i * LG;
      q[i] = (e < E && c < C)
                 ? reinterpret_cast<const uint4*>(router + (int64_t)e * H)[c]
                 : make_uint4(0u, 0u, 0u, 0u);
    }
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc += bf16_chunk_dot(q[i], xr[i]);
    acc = group_sum<LG>(acc);
    if (gl == 0 && e < E) logits[(int64_t)t * E + e] = acc;
  }
}

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return bi < 0 || av > bv || (av == bv && ai < bi);
}

// one block per token: K rounds of a block-wide arg-max (ties to the lower index)
__global__ __launch_bounds__(kBlock) void k_topk(const float* __restrict__ logits, int E, int K,
                                                 int32_t* __restrict__ idx, float* __restrict__ w) {
  constexpr int PER = kMaxExperts / kBlock;
  const int t = blockIdx.x;
  const float* l = logits + (int64_t)t * E;
  float v[PER];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = threadIdx.x + kBlock * j;
    v[j] = e < E ? l[e] : 0.f;
  }
  __shared__ float sv[kBlock / 64];
  __shared__ int si[kBlock / 64];
  __shared__ float selv[kMaxTopK];
  __shared__ int seli[kMaxTopK];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int k = 0; k < K; ++k) {
    float bv = 0.f;
    int bi = -1;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = threadIdx.x + kBlock * j;
      if (e < E && !((taken >> j) & 1u) && better(v[j], e, bv, bi)) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (oi >= 0 && better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      sv[wv] = bv;
      si[wv] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float b = sv[0];
      int i = si[0];
      for (int q = 1; q < kBlock / 64; ++q)
        if (si[q] >= 0 && better(sv[q], si[q], b, i)) {
          b = sv[q];
          i = si[q];
        }
      selv[k] = b;
      seli[k] = i;
    }
    __syncthreads();
    const int won = seli[k];
    if (won >= 0 && (won % kBlock) == (int)threadIdx.x) taken |= 1u << (won / kBlock);
  }
  if (threadIdx.x == 0) {
    const float m = selv[0];
    float ex[kMaxTopK];
    float sum = 0.f;
    for (int k = 0; k < K; ++k) {
      ex[k] = expf(selv[k] - m);
      sum += ex[k];
    }
    const float inv = 1.0f / sum;
    for (int k = 0; k < K; ++k) {
      idx[(int64_t)t * K + k] = seli[k];
      w[(int64_t)t * K + k] = ex[k] * inv;
    }
  }
}

// Router GEMV for a batch of tokens: the router rows are read once per 16 tokens
// instead of once per token.  grid (ceil(E/8), ceil(T/16)), 256*G threads: the
// block owns 8 experts x 16 tokens and its G groups of 4 waves split H into G
// slices.  In a group, half-wave hw owns a 4-expert x 4-token tile and its 32
// lanes split the slice, lane l taking k = 128 i + 4 l .. +3, so that one load
// instruction covers 512 contiguous bytes.  The 32 lane sums of an output are
// added across the half-wave, then the G slice sums in group order (in LDS).
// Needs (H / G) % 128 == 0.  With BITS > 0 the workgroups of the first 16 columns
// also write the fixed-point planes of one token of their tile each (planes of
// token t at xplanes + t*pw: C*PW plane words, C scales, C sums), which the
// batched layer takes next.
constexpr int kRtE = 8, kRtT = 16;
template <int G, int BITS>
__global__ __launch_bounds__(kBlock * G) void k_router_tiled(const uint16_t* __restrict__ router,
                                                             const float* __restrict__ x,
                                                             float* __restrict__ logits, int T,
                                                             int E, int H, uint32_t* xplanes,
                                                             int pw) {
  __shared__ float red[G][kRtE * kRtT];
  const int grp = threadIdx.x / kBlock, tid = threadIdx.x % kBlock;
  const int lane = tid & 63, hw = tid >> 5, l = lane & 31;
  const int le = (hw & 1) * 4, lt = (hw >> 1) * 4;  // the tile's first local expert / token
  const int e0 = blockIdx.x * kRtE + le, t0 = blockIdx.y * kRtT + lt;
  const int hs = H / G;
  const uint16_t* rp[4];
  const float* xp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // rows past the end repeat the last one; never stored
    rp[j] = router + (int64_t)min(e0 + j, E - 1) * H + grp * hs + 4 * l;
    xp[j] = x + (int64_t)min(t0 + j, T - 1) * H + grp * hs + 4 * l;
  }
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
#pragma unroll 2
  for (int k = 0; k < hs; k += 128) {
    float4 xv[4];
    uint2 rv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[j] = *reinterpret_cast<const float4*>(xp[j] + k);
      rv[j] = *reinterpret_cast<const uint2*>(rp[j] + k);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float r0 = bf16_lo(rv[a].x), r1 = bf16_hi(rv[a].x);
      const float r2 = bf16_lo(rv[a].y), r3 = bf16_hi(rv[a].y);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[a][b] = fmaf(r0, xv[b].x, acc[a][b]);
        acc[a][b] = fmaf(r1, xv[b].y, acc[a][b]);
        acc[a][b] = fmaf(r2, xv[b].z, acc[a][b]);
        acc[a][b] = fmaf(r3, xv[b].w, acc[a][b]);
      }
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float v = group_sum_last<32>(acc[a][b]);
      if (l == 31) red[grp][(le + a) * kRtT + lt + b] = v;
    }
  __syncthreads();
  if ((int)threadIdx.x < kRtE * kRtT) {
    const int e = blockIdx.x * kRtE + (int)threadIdx.x / kRtT;
    const int t = blockIdx.y * kRtT + (int)threadIdx.x % kRtT;
    float v = red[0][threadIdx.x];
#pragma unroll
    for (int g = 1; g < G; ++g) v += red[g][threadIdx.x];
    if (e < E && t < T) logits[(int64_t)t * E + e] = v;
  }
  if constexpr (BITS > 0) {
    const int t = blockIdx.y * kRtT + (int)blockIdx.x;
    if ((int)blockIdx.x < kRtT && t < T) {  // uniform per workgroup
      uint32_t* planes = xplanes + (int64_t)t * pw;
      const int C = H / QTraits<BITS>::EPC;
      float* scl = reinterpret_cast<float*>(planes + C * QTraits<BITS>::PW);
      prep_x_coop<BITS>(x + (int64_t)t * H, H, planes, scl, scl + C, threadIdx.x, blockDim.x);
    }
  }
}

// Top-K with renormalised softmax, one wave per token (4 tokens per workgroup):
// K rounds of a wave-wide arg-max over order-preserving keys (larger logit, then
// lower index; -0 counts as +0).  Lane l holds experts l + 64 j, j < PER.
template <int PER>
__global__ __launch_bounds__(kBlock) void k_topk_wave(const float* __restrict__ logits, int T,
                                                      int E, int K, int32_t* __restrict__ idx,
                                                      float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kBlock / 64) + (int)(threadIdx.x >> 6);
  if (t >= T) return;
  const float* lt = logits + (int64_t)t * E;
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? order_key(__float_as_uint(lt[e])) : 0u;
  }
  uint32_t bk = 0, bi = 0xFFFFFFFFu;
  auto best = [&]() {
    bk = 0;
    bi = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (key[j] > bk) {  // strictly larger: the lower index wins a tie
        bk = key[j];
        bi = lane + 64 * j;
      }
  };
  best();
  uint32_t pk[kMaxTopK], pi[kMaxTopK];
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    pk[r] = 0;
    pi[r] = 0xFFFFFFFFu;
    if (r < K) {
      wave_argmax(bk, bi, pk[r], pi[r]);
      if (pk[r] != 0 && bi == pi[r]) {
#pragma unroll
        for (int j = 0; j < PER; ++j)
          if (lane + 64 * j == (int)pi[r]) key[j] = 0;
        best();
      }
    }
  }
  // softmax over the picks (uniform values); lane r writes pick r
  const float m = key_value(pk[0]);
  float ex[kMaxTopK], sum = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    ex[r] = r < K ? expf(key_value(pk[r]) - m) : 0.f;
    sum += ex[r];
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r)
    if (r < K && lane == r) {
      idx[(int64_t)t * K + r] = (int32_t)pi[r];
      w[(int64_t)t * K + r] = ex[r] * inv;
    }
}

template <int LG, int CPL>
hipError_t run_router(const uint16_t* router, const float* x, float* logits, int T, int E, int H,
                      hipStream_t s) {
  const int waves = ceil_div(E, 64 / LG);
  hipLaunchKernelGGL((k_router<LG, CPL>), dim3(ceil_div(waves, 4), T), dim3(kBlock), 0, s, router,
                     x, logits, E, H);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine and RMSNorm
// ---------------------------------------------------------------------------
// block-wide sum (all threads get the result)
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = group_sum<64>(v);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}

__global__ __launch_bounds__(kBlock) void k_combine(const float* __restrict__ yr,
                                                    const float* __restrict__ w,
                                                    const float* __restrict__ ys,
                                                    const uint16_t* __restrict__ g,
                                                    const float* __restrict__ x,
                                                    const float* residual, float* out, int H,
                                                    int K) {
  __shared__ float red[kBlock / 64];
  float d = 0.f;
  for (int h = threadIdx.x; h < H; h += kBlock) d += __uint_as_float((uint32_t)g[h] << 16) * x[h];
  const float gamma = sigmoid_f(block_sum(d, red));
  const int n = blockIdx.x * kBlock + threadIdx.x;
  if (n >= H) return;
  float acc = residual[n];
  for (int k = 0; k < K; ++k) acc = fmaf(w[k], yr[(int64_t)k * H + n], acc);
  out[n] = fmaf(gamma, ys[n], acc);
}

__global__ __launch_bounds__(1024) void k_rmsnorm(const float* v, const float* __restrict__ w,
                                                  float eps, int n, float* out) {
  __shared__ float red[16];
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s = fmaf(v[i], v[i], s);
  const float tot = block_sum(s, red);
  const float r = 1.0f / sqrtf(tot / (float)n + eps);
  __syncthreads();  // every read of v is done before out (which may alias v) is written
  for (int i = threadIdx.x; i < n; i += blockDim.x) out[i] = v[i] * r * w[i];
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_qgemv(int bits, const uint8_t* codes, const uint32_t* sb, const float* x,
                        float* y, int rows, int cols, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  return bits == 4 ? dispatch_qgemv<4>(codes, sb, x, y, rows, cols, s)
                   : dispatch_qgemv<2>(codes, sb, x, y, rows, cols, s);
}

hipError_t launch_ffn(const qmoe_expert_pool& pool, const int32_t* idx, int n, const float* x,
                      int64_t x_stride, float* y, float* h_ws, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const PoolArgs P = pool_args(pool);
  hipError_t err = pool.bits == 4 ? dispatch_gateup<4>(P, idx, n, x, x_stride, h_ws, s)
                                  : dispatch_gateup<2>(P, idx, n, x, x_stride, h_ws, s);
  if (err != hipSuccess) return err;
  return pool.bits == 4 ? dispatch_down<4>(P, idx, n, h_ws, y, s)
                        : dispatch_down<2>(P, idx, n, h_ws, y, s);
}

hipError_t launch_router_topk(const uint16_t* router, const float* x, int T, int H, int E, int K,
                              float* logits, int32_t* idx, float* w, hipStream_t s, int prep_bits,
                              uint32_t* xplanes, int pw, bool* prepped) {
  if (prepped) *prepped = false;
  if (T == 0) return hipSuccess;
  const int C = H / 8;
  hipError_t err;
  if (T >= 8 && H % 128 == 0) {
    // the planes need a workgroup per token in the first 16 columns: E >= 8*15+1
    const bool prep = prep_bits && xplanes && H % 512 == 0 && E > kRtE * (kRtT - 1);
    dim3 grid(ceil_div(E, kRtE), ceil_div(T, kRtT));
    if (prep && prep_bits == 4)
      hipLaunchKernelGGL((k_router_tiled<4, 4>), grid, dim3(4 * kBlock), 0, s, router, x, logits, T, E,
                         H, xplanes, pw);
    else if (prep)
      hipLaunchKernelGGL((k_router_tiled<4, 2>), grid, dim3(4 * kBlock), 0, s, router, x, logits, T, E,
                         H, xplanes, pw);
    else if (H % 512 == 0)
      hipLaunchKernelGGL((k_router_tiled<4, 0>), grid, dim3(4 * kBlock), 0, s, router, x, logits, T, E,
                         H, nullptr, 0);
    else
      hipLaunchKernelGGL((k_router_tiled<1, 0>), grid, dim3(kBlock), 0, s, router, x, logits, T, E, H,
                         nullptr, 0);
    err = hipGetLastError();
    if (prepped) *prepped = prep && err == hipSuccess;
  } else if (C <= 8) err = run_router<8, 1>(router, x, logits, T, E, H, s);
  else if (C <= 16) err = run_router<16, 1>(router, x, logits, T, E, H, s);
  else if (C <= 32) err = run_router<32, 1>(router, x, logits, T, E, H, s);
  else if (C <= 64) err = run_router<64, 1>(router, x, logits, T, E, H, s);
  else if (C <= 128) err = run_router<64, 2>(router, x, logits, T, E, H, s);
  else if (C <= 256) err = run_router<64, 4>(router, x, logits, T, E, H, s);
  else if (C <= 512) err = run_router<64, 8>(router, x, logits, T, E, H, s);
  else err = run_router<64, 16>(router, x, logits, T, E, H, s);
  if (err != hipSuccess) return err;
  const dim3 tg(ceil_div(T, kBlock / 64));
  if (E <= 512) hipLaunchKernelGGL(k_topk_wave<8>, tg, dim3(kBlock), 0, s, logits, T, E, K, idx, w);
  else if (E <= 1024) hipLaunchKernelGGL(k_topk_wave<16>, tg, dim3(kBlock), 0, s, logits, T, E, K, idx, w);
  else hipLaunchKernelGGL(k_topk, dim3(T), dim3(kBlock), 0, s, logits, E, K, idx, w);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_routed, const float* w, const float* y_shared,
                          const uint16_t* g, const float* x, const float* residual, float* out,
                          int H, int K, hipStream_t s) {
  if (H == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3(ceil_div(H, kBlock)), dim3(kBlock), 0, s, y_routed, w,
                     y_shared, g, x, residual, out, H, K);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* v, const float* w, float eps, int n, float* out,
                          hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm, dim3(1), dim3(1024), 0, s, v, w, eps, n, out);
  return hipGetLastError();
}

}  // namespace qmoe
