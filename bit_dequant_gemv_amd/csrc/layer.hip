// One MoE layer at batch 1 in a single kernel launch.
//
// The page "flash-moe 소개" (discuss.pytorch.kr), section "레이어당 파이프라인 상세
// 구조", runs this path as: router GEMV inside a second command buffer, a device
// to host copy, softmax + top-K on the CPU, then a third command buffer with the
// expert forward, combine and norm.  Here it is one launch with no host round
// trip: every workgroup (all co-resident) computes the routing itself from the
// logits, and the experts are addressed by index in the resident pool.
//
// Data flow inside the launch (NB workgroups of 8 waves; "rank" numbers waves so
// that consecutive ranks sit in different workgroups):
//   A  ranks 0..E      : router rows (rank E = shared-expert gate vector g)
//      next I/RPWH ranks: shared-expert gate/up rows + SwiGLU -> hs[I]
//   B  each workgroup   : top-K of the E logits (redundantly, ties to the lower
//                         index), gamma = sigmoid(g.x)
//      all ranks       : routed gate/up rows + SwiGLU -> hr[K][I]
//   C  workgroup b owns output rows [b*RB, b*RB+RB): down rows of the shared and
//      the K routed experts, then out = residual + sum_k w_k y_k + gamma y_s.
// Values that cross workgroups (logits, hs, hr) are stored as 64-bit words
// (epoch << 32 | value bits) with agent-scope atomic stores; consumers poll the
// words until they carry this call's epoch, so no grid barrier is needed and the
// words never need resetting.  The epoch lives in the workspace: every wave
// reads it at start and workgroup 0 advances it once it has consumed the
// outputs of every wave (the grid is sized so that every wave owns at least one
// phase-A or phase-B row, and a wave can only tag an output after reading the
// epoch).  The down-projection codes of phase C are fetched into
// registers before their input exists, so their HBM latency overlaps phase B.
// Every wait is bounded; on time-out a status bit is set and the call's output
// is undefined (it never hangs).
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kLB = 512;         // threads per workgroup
constexpr int kLW = kLB / 64;    // waves per workgroup
constexpr int kFusedMaxI = 1024;
constexpr int kFusedMaxK = 4;
constexpr int kFusedMaxE = 2048;
constexpr int kMaxRoutedItems = 4;  // phase-C routed down items per wave
constexpr uint32_t kSpinLimit = 1u << 18;

// control words at the start of the workspace
enum { CTRL_EPOCH = 0, CTRL_STATUS = 1, CTRL_ZERO = 8 };  // CTRL_ZERO is never written

struct LayerArgs {
  const uint8_t* rbase;  // routed pool
  int64_t rstride;
  const uint8_t* sblk;   // shared expert block
  int64_t off_g, off_u, off_d, off_gsb, off_usb, off_dsb;
  const uint16_t* router;
  const uint16_t* g;
  const float* x;
  const float* residual;
  float* out;
  int32_t* idx_out;
  float* w_out;
  uint32_t* ctrl;
  uint64_t* logits;  // [E+1]
  uint64_t* hs;      // [I]
  uint64_t* hr;      // [K][I]
  int E, K, H, I, RB;
};

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

// Copy n tagged values into LDS (every thread takes i = tid + j*kLB), waiting
// until each carries `tag`.  Returns false on time-out.
template <int PER>
__device__ bool poll_to_lds(uint64_t* src, int n, uint32_t tag, float* dst) {
  uint32_t pending = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if ((int)threadIdx.x + j * kLB < n) pending |= 1u << j;
  for (uint32_t spins = 0; pending; ++spins) {
    uint64_t v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = (pending >> j) & 1u ? tag_get(src + threadIdx.x + j * kLB) : 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (((pending >> j) & 1u) && (uint32_t)(v[j] >> 32) == tag) {
        dst[threadIdx.x + j * kLB] = __uint_as_float((uint32_t)v[j]);
        pending &= ~(1u << j);
      }
    }
    if (!pending) break;
    if (spins > kSpinLimit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return bi < 0 || av > bv || (av == bv && ai < bi);
}

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

template <int BITS, int LGH, int CPLH, int LGI, int CPLR>
__global__ __launch_bounds__(kLB, 2) void k_layer(LayerArgs A) {
  constexpr int RPWH = 64 / LGH;  // gate/up rows per wave pass
  constexpr int RPWI = 64 / LGI;  // down rows per wave pass
  constexpr int PER_L = (kFusedMaxE + 1 + kLB - 1) / kLB;
  const int NB = gridDim.x, wg = blockIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rank = wv * NB + wg;
  const int W = NB * kLW;
  const int E = A.E, K = A.K, H = A.H, I = A.I;

  __shared__ float s_hs[kFusedMaxI];
  __shared__ float s_hr[kFusedMaxK * kFusedMaxI];
  __shared__ float s_y[kFusedMaxK + 1][2 * kLW * 8];
  __shared__ int s_idx[kFusedMaxK];
  __shared__ float s_w[kFusedMaxK];
  __shared__ float s_gamma;
  __shared__ float s_rv[kLW];
  __shared__ int s_ri[kLW];

  const uint32_t tag = __hip_atomic_load(A.ctrl + CTRL_EPOCH, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) + 1u;
  bool ok_all = true;

  const int Ch = H * BITS / 128, Gh = H / kGroup;
  const int64_t rbh = (int64_t)H * BITS / 8;
  const int Ci = I * BITS / 128, Gi = I / kGroup;
  const int64_t rbi = (int64_t)I * BITS / 8;

  // output rows owned by this workgroup
  const int row0 = wg * A.RB;
  const int nrows = max(0, min(A.RB, H - row0));
  const int ditems = (nrows + RPWI - 1) / RPWI;
  const float resid = (int)threadIdx.x < nrows ? A.residual[row0 + threadIdx.x] : 0.f;

  // ---- prefetch: this wave's shared-expert down rows (known before anything runs)
  const int gli = lane % LGI, subi = lane / LGI;
  RowDot<BITS, LGI, 1> dI;
  uint4 q_sd[1][1];
  uint32_t s_sd[1][1];
  {
    const int nl = wv * RPWI + subi;
    const bool ok = wv < ditems && nl < nrows;
    const uint8_t* cr = A.sblk + A.off_d + (int64_t)(row0 + nl) * rbi;
    const uint32_t* sr = reinterpret_cast<const uint32_t*>(A.sblk + A.off_dsb) + (int64_t)(row0 + nl) * Gi;
    dI.template fetch<1>(&cr, &sr, &ok, Ci, gli, q_sd, s_sd);
  }

  // ---- phase A: router rows, shared gate/up rows (the host sizes the grid so that
  // every phase-A row has its own wave: E + 1 + I/RPWH <= waves)
  const int glh = lane % LGH, subh = lane / LGH;
  const int n_sp = I / RPWH;
  if (rank <= E) {
    const uint16_t* row = rank < E ? A.router + (int64_t)rank * H : A.g;
    float acc = 0.f;
#pragma unroll
    for (int h0 = 0; h0 < CPLR; h0 += 4) {  // four 16-byte chunks in flight per step
      uint4 q[4];
      float xr[4][8];
#pragma unroll
      for (int i = 0; i < 4 && h0 + i < CPLR; ++i) {
        const int c = lane + 64 * (h0 + i);
        q[i] = reinterpret_cast<const uint4*>(row)[c];
        const float4 f0 = reinterpret_cast<const float4*>(A.x + 8 * c)[0];
        const float4 f1 = reinterpret_cast<const float4*>(A.x + 8 * c)[1];
        xr[i][0] = f0.x; xr[i][1] = f0.y; xr[i][2] = f0.z; xr[i][3] = f0.w;
        xr[i][4] = f1.x; xr[i][5] = f1.y; xr[i][6] = f1.z; xr[i][7] = f1.w;
      }
#pragma unroll
      for (int i = 0; i < 4 && h0 + i < CPLR; ++i) acc += bf16_chunk_dot(q[i], xr[i]);
    }
    acc = group_sum<64>(acc);
    if (lane == 0) tag_put(A.logits + rank, acc, tag);
  } else if (rank < E + 1 + n_sp) {
    RowDot<BITS, LGH, CPLH> dA;
    dA.load_x(A.x, Ch, glh);
    const int j = (rank - E - 1) * RPWH + subh;
    const uint8_t* cr[2] = {A.sblk + A.off_g + (int64_t)j * rbh, A.sblk + A.off_u + (int64_t)j * rbh};
    const uint32_t* sr[2] = {reinterpret_cast<const uint32_t*>(A.sblk + A.off_gsb) + (int64_t)j * Gh,
                             reinterpret_cast<const uint32_t*>(A.sblk + A.off_usb) + (int64_t)j * Gh};
    const bool ok[2] = {true, true};
    uint4 q[2][CPLH];
    uint32_t s[2][CPLH];
    dA.template fetch<2>(cr, sr, ok, Ch, glh, q, s);
    float p[2];
    dA.template dots<2>(q, s, p);
    const float a = group_sum<LGH>(p[0]);
    const float u = group_sum<LGH>(p[1]);
    if (glh == 0) tag_put(A.hs + j, silu_f(a) * u, tag);
  }

  // ---- shared h -> LDS, shared down rows (prefetched codes)
  ok_all &= poll_to_lds<(kFusedMaxI + kLB - 1) / kLB>(A.hs, I, tag, s_hs);
  __syncthreads();
  if (wv < ditems) {
    dI.load_x(s_hs, Ci, gli);
    float p[1];
    dI.template dots<1>(q_sd, s_sd, p);
    const float v = group_sum<LGI>(p[0]);
    const int nl = wv * RPWI + subi;
    if (gli == 0 && nl < nrows) s_y[K][nl] = v;
  }

  // ---- phase B: top-K from the logits (every workgroup), ties to the lower index
  {
    float lv[PER_L];
    {
      uint32_t pending = 0;
#pragma unroll
      for (int j = 0; j < PER_L; ++j)
        if ((int)threadIdx.x + j * kLB <= E) pending |= 1u << j;
      for (uint32_t spins = 0; pending; ++spins) {
        uint64_t v[PER_L];
#pragma unroll
        for (int j = 0; j < PER_L; ++j)
          v[j] = (pending >> j) & 1u ? tag_get(A.logits + threadIdx.x + j * kLB) : 0;
#pragma unroll
        for (int j = 0; j < PER_L; ++j)
          if (((pending >> j) & 1u) && (uint32_t)(v[j] >> 32) == tag) {
            lv[j] = __uint_as_float((uint32_t)v[j]);
            pending &= ~(1u << j);
          }
        if (!pending) break;
        if (spins > kSpinLimit) {
          ok_all = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if ((int)threadIdx.x == E % kLB) s_gamma = sigmoid_f(lv[E / kLB]);
    uint32_t taken = 0;
    for (int k = 0; k < K; ++k) {
      float bv = 0.f;
      int bi = -1;
#pragma unroll
      for (int j = 0; j < PER_L; ++j) {
        const int e = threadIdx.x + j * kLB;
        if (e < E && !((taken >> j) & 1u) && better(lv[j], e, bv, bi)) {
          bv = lv[j];
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
        s_rv[wv] = bv;
        s_ri[wv] = bi;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        float b = s_rv[0];
        int i = s_ri[0];
        for (int q = 1; q < kLW; ++q)
          if (s_ri[q] >= 0 && better(s_rv[q], s_ri[q], b, i)) {
            b = s_rv[q];
            i = s_ri[q];
          }
        s_idx[k] = i;
        s_w[k] = b;  // logit for now
      }
      __syncthreads();
      const int won = s_idx[k];
      if (won >= 0 && won % kLB == (int)threadIdx.x) taken |= 1u << (won / kLB);
    }
    if (threadIdx.x == 0) {
      const float m = s_w[0];
      float ex[kFusedMaxK];
      float sum = 0.f;
      for (int k = 0; k < K; ++k) {
        ex[k] = expf(s_w[k] - m);
        sum += ex[k];
      }
      const float inv = 1.0f / sum;
      for (int k = 0; k < K; ++k) s_w[k] = ex[k] * inv;
      if (wg == 0) {
        for (int k = 0; k < K; ++k) {
          A.idx_out[k] = s_idx[k];
          A.w_out[k] = s_w[k];
        }
      }
    }
    __syncthreads();
  }

  // ---- prefetch: this wave's routed down rows for phase C
  uint4 q_rd[kMaxRoutedItems][1];
  uint32_t s_rd[kMaxRoutedItems][1];
#pragma unroll
  for (int m = 0; m < kMaxRoutedItems; ++m) {
    const int t = wv * kMaxRoutedItems + m;
    const int k = ditems > 0 ? t / ditems : 0, d = ditems > 0 ? t % ditems : 0;
    const int e = t < K * ditems ? s_idx[k] : -1;
    const int nl = d * RPWI + subi;
    const bool ok = (unsigned)e < (unsigned)E && nl < nrows;
    const uint8_t* blk = A.rbase + (ok ? (int64_t)e * A.rstride : 0);
    const uint8_t* cr = blk + A.off_d + (int64_t)(row0 + nl) * rbi;
    const uint32_t* sr = reinterpret_cast<const uint32_t*>(blk + A.off_dsb) + (int64_t)(row0 + nl) * Gi;
    uint4 qq[1][1];
    uint32_t ss[1][1];
    dI.template fetch<1>(&cr, &sr, &ok, Ci, gli, qq, ss);
    q_rd[m][0] = qq[0][0];
    s_rd[m][0] = ss[0][0];
  }

  // ---- phase B: routed gate/up rows + SwiGLU
  RowDot<BITS, LGH, CPLH> dH;
  dH.load_x(A.x, Ch, glh);
  const int n_rp = K * n_sp;
  // two row pairs per step so that four rows of codes are in flight per wave
  for (int it = rank; it < n_rp; it += 2 * W) {
    const uint8_t* cr[4];
    const uint32_t* sr[4];
    bool ok[4];
    int kk[2], jj[2];
    bool eok[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int item = it + v * W;
      const bool valid = item < n_rp;
      kk[v] = valid ? item / n_sp : 0;
      jj[v] = valid ? (item % n_sp) * RPWH + subh : 0;
      const int e = valid ? s_idx[kk[v]] : -1;
      eok[v] = (unsigned)e < (unsigned)E;
      const uint8_t* blk = A.rbase + (eok[v] ? (int64_t)e * A.rstride : 0);
      cr[2 * v] = blk + A.off_g + (int64_t)jj[v] * rbh;
      cr[2 * v + 1] = blk + A.off_u + (int64_t)jj[v] * rbh;
      sr[2 * v] = reinterpret_cast<const uint32_t*>(blk + A.off_gsb) + (int64_t)jj[v] * Gh;
      sr[2 * v + 1] = reinterpret_cast<const uint32_t*>(blk + A.off_usb) + (int64_t)jj[v] * Gh;
      ok[2 * v] = ok[2 * v + 1] = eok[v];
    }
    uint4 q[4][CPLH];
    uint32_t s[4][CPLH];
    dH.template fetch<4>(cr, sr, ok, Ch, glh, q, s);
    float p[4];
    dH.template dots<4>(q, s, p);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const float a = group_sum<LGH>(p[2 * v]);
      const float u = group_sum<LGH>(p[2 * v + 1]);
      if (glh == 0 && it + v * W < n_rp)
        tag_put(A.hr + (int64_t)kk[v] * I + jj[v], eok[v] ? silu_f(a) * u : __builtin_nanf(""), tag);
    }
  }

  // ---- phase C: routed h -> LDS, down rows, combine
  ok_all &= poll_to_lds<(kFusedMaxK * kFusedMaxI + kLB - 1) / kLB>(A.hr, K * I, tag, s_hr);
  __syncthreads();
  // Workgroup 0 has now seen outputs of every wave of the grid (logits, hs, hr),
  // so every wave has read the epoch: advance it for the next call.
  if (wg == 0 && threadIdx.x == 0)
    __hip_atomic_store(A.ctrl + CTRL_EPOCH, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int prev_k = -1;
#pragma unroll
  for (int m = 0; m < kMaxRoutedItems; ++m) {
    const int t = wv * kMaxRoutedItems + m;
    if (t < K * ditems) {
      const int k = t / ditems, d = t % ditems;
      if (k != prev_k) {
        dI.load_x(s_hr + k * I, Ci, gli);
        prev_k = k;
      }
      uint4 qq[1][1] = {{q_rd[m][0]}};
      uint32_t ss[1][1] = {{s_rd[m][0]}};
      float p[1];
      dI.template dots<1>(qq, ss, p);
      const float v = group_sum<LGI>(p[0]);
      const int nl = d * RPWI + subi;
      const int e = s_idx[k];
      if (gli == 0 && nl < nrows) s_y[k][nl] = (unsigned)e < (unsigned)E ? v : __builtin_nanf("");
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < nrows) {
    float acc = resid;
    for (int k = 0; k < K; ++k) acc = fmaf(s_w[k], s_y[k][threadIdx.x], acc);
    A.out[row0 + threadIdx.x] = fmaf(s_gamma, s_y[K][threadIdx.x], acc);
  }
  if (!ok_all) flag_status(A.ctrl, 1u);
}

struct FusedCfg {
  int nb = 0, rb = 0;
};

inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

struct WsLayout {
  int64_t ctrl, logits, hs, hr, total;
};

WsLayout fused_ws(int E, int K, int I) {
  WsLayout w;
  w.ctrl = 0;
  w.logits = 256;
  w.hs = w.logits + align256((int64_t)(E + 1) * 8);
  w.hr = w.hs + align256((int64_t)I * 8);
  w.total = w.hr + align256((int64_t)K * I * 8);
  return w;
}

// unfused fallback: logits[E] | y_routed[K][H] | y_shared[H] | h[K][I] (ctrl block stays zero)
struct UnfusedWs {
  int64_t logits, yr, ys, h, total;
};

UnfusedWs unfused_ws(int E, int K, int H, int I) {
  UnfusedWs u;
  u.logits = 256;
  u.yr = u.logits + align256((int64_t)E * 4);
  u.ys = u.yr + align256((int64_t)K * H * 4);
  u.h = u.ys + align256((int64_t)H * 4);
  u.total = u.h + align256((int64_t)K * I * 4);
  return u;
}

using KernelFn = void (*)(LayerArgs);

template <int BITS, int H, int I>
KernelFn pick() {
  constexpr int CH = H * BITS / 128;
  constexpr int LGH = CH >= 64 ? 64 : CH;
  constexpr int CPLH = CH >= 64 ? CH / 64 : 1;
  constexpr int CI = I * BITS / 128;
  constexpr int LGI = CI >= 64 ? 64 : CI;
  static_assert(CI <= 64, "down rows must fit one chunk per lane");
  return k_layer<BITS, LGH, CPLH, LGI, H / 512>;
}

template <int BITS, int H>
KernelFn pick_i(int I) {
  if (I == 256) return pick<BITS, H, 256>();
  if (I == 512) return pick<BITS, H, 512>();
  if (I == 1024) return pick<BITS, H, 1024>();
  return nullptr;
}

template <int BITS>
KernelFn pick_h(int H, int I) {
  if (H == 1024) return pick_i<BITS, 1024>(I);
  if (H == 2048) return pick_i<BITS, 2048>(I);
  if (H == 4096) return pick_i<BITS, 4096>(I);
  return nullptr;
}

// grid geometry for the fused kernel, or nb == 0 when the shape needs the fallback
FusedCfg fused_config(const qmoe_layer& L, KernelFn fn) {
  FusedCfg c;
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  if (!fn || K > kFusedMaxK || E > kFusedMaxE || I > kFusedMaxI) return c;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return c;
  static int cus[64] = {0};  // per-device CU count; concurrent first calls store equal values
  if (dev < 0 || dev >= 64) return c;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return c;
    cus[dev] = n;
  }
  int blocks_per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks_per_cu, reinterpret_cast<const void*>(fn),
                                                   kLB, 0) != hipSuccess ||
      blocks_per_cu < 1)
    return c;
  int nb = cus[dev] * (blocks_per_cu < 2 ? blocks_per_cu : 2);
  // every wave must own at least one phase-A or phase-B row (epoch hand-over)
  const int bits = L.routed.bits;
  const int ch = H * bits / 128;
  const int rpwh = 64 / (ch >= 64 ? 64 : ch);
  const int n_sp = I / rpwh;
  const int n_items = (E + 1 + n_sp) > K * n_sp ? (E + 1 + n_sp) : K * n_sp;
  if (nb * kLW > n_items) nb = n_items / kLW;
  if (nb < 1 || nb * kLW < E + 1 + n_sp) return c;  // one phase-A row per wave
  const int ci = I * bits / 128;
  const int rpwi = 64 / (ci >= 64 ? 64 : ci);
  int rb = (H + nb - 1) / nb;
  rb = (rb + rpwi - 1) / rpwi * rpwi;
  const int ditems = rb / rpwi;
  if (ditems > kLW || K * ditems > kLW * kMaxRoutedItems || rb > 2 * kLW * 8) return c;
  c.nb = nb;
  c.rb = rb;
  return c;
}

KernelFn fused_kernel(const qmoe_layer& L) {
  const int H = L.routed.hidden, I = L.routed.inter;
  return L.routed.bits == 4 ? pick_h<4>(H, I) : pick_h<2>(H, I);
}

}  // namespace

size_t layer_workspace_bytes(const qmoe_layer& L) {
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  const WsLayout f = fused_ws(E, K, I);
  const UnfusedWs u = unfused_ws(E, K, H, I);
  return (size_t)(f.total > u.total ? f.total : u.total);
}

hipError_t launch_layer(const qmoe_layer& L, const float* x, const float* residual, float* out,
                        int32_t* idx, float* w, void* ws, hipStream_t s) {
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  KernelFn fn = fused_kernel(L);
  const FusedCfg cfg = fused_config(L, fn);
  if (cfg.nb > 0) {
    const WsLayout wl = fused_ws(E, K, I);
    const qmoe_expert_offsets o = expert_offsets(H, I, L.routed.bits);
    LayerArgs A;
    A.rbase = static_cast<const uint8_t*>(L.routed.base);
    A.rstride = L.routed.stride;
    A.sblk = static_cast<const uint8_t*>(L.shared.base);
    A.off_g = o.gate_codes;
    A.off_u = o.up_codes;
    A.off_d = o.down_codes;
    A.off_gsb = o.gate_sb;
    A.off_usb = o.up_sb;
    A.off_dsb = o.down_sb;
    A.router = L.router;
    A.g = L.shared_gate;
    A.x = x;
    A.residual = residual;
    A.out = out;
    A.idx_out = idx;
    A.w_out = w;
    A.ctrl = reinterpret_cast<uint32_t*>(wsb + wl.ctrl);
    A.logits = reinterpret_cast<uint64_t*>(wsb + wl.logits);
    A.hs = reinterpret_cast<uint64_t*>(wsb + wl.hs);
    A.hr = reinterpret_cast<uint64_t*>(wsb + wl.hr);
    A.E = E;
    A.K = K;
    A.H = H;
    A.I = I;
    A.RB = cfg.rb;
    hipLaunchKernelGGL(fn, dim3(cfg.nb), dim3(kLB), 0, s, A);
    return hipGetLastError();
  }
  // fallback: the unfused chain of stand-alone kernels
  const UnfusedWs u = unfused_ws(E, K, H, I);
  float* logits = reinterpret_cast<float*>(wsb + u.logits);
  float* yr = reinterpret_cast<float*>(wsb + u.yr);
  float* ys = reinterpret_cast<float*>(wsb + u.ys);
  float* h = reinterpret_cast<float*>(wsb + u.h);
  const int32_t* zero_idx = reinterpret_cast<const int32_t*>(wsb) + CTRL_ZERO;  // stays zero
  hipError_t err = launch_router_topk(L.router, x, 1, H, E, K, logits, idx, w, s);
  if (err == hipSuccess) err = launch_ffn(L.routed, idx, K, x, 0, yr, h, s);
  if (err == hipSuccess) err = launch_ffn(L.shared, zero_idx, 1, x, 0, ys, h, s);
  if (err == hipSuccess) err = launch_combine(yr, w, ys, L.shared_gate, x, residual, out, H, K, s);
  return err;
}

}  // namespace qmoe
