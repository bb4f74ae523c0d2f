// GatedDeltaNet recurrence, one decode step for every head.
//
// The page "flash-moe 소개" (discuss.pytorch.kr), section "Accelerate BLAS를 이용한
// 선형 어텐션 가속", updates a 128x128 state per head (64 heads) in each linear-attention layer with a
// scale, a matrix-vector product and a rank-1 update; section "Qwen3.5-397B-A17B
// 모델 아키텍처" puts 45 such layers among the 60.  Per head, with the state S as
// [dk][dv] (S^T k is the value recalled for the key k):
//   S <- alpha S;  u = S^T k;  S <- S + k (beta (v - u))^T;  o = S^T q.
// Written per column j of S (the values at index j, a vector over the keys c):
//   a = c . k,  b = c . q,  d = beta (v_j - alpha a),
//   c <- alpha c + d k,  o_j = alpha b + d (k . q),
// so every column is independent: one pass over the state, each column read and
// written once.  The state is kept with those columns contiguous ([heads][dv][dk]),
// DK/4 lanes per column with a float4 each; the three dots are reductions over the
// column's lanes.  The pass is HBM bound: 2 * heads * dv * dk * 4 bytes per step.
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

// threads per workgroup: 1024 (fewer, larger workgroups) measured 3.27 us per step
// against 3.53 us at 256; two or four columns per lane group were slower (4.0, 4.7)
constexpr int kGB = 1024;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DK>
__global__ __launch_bounds__(kGB) void k_gdn(float* S, const float* q, const float* k, const float* v,
                                           const float* alpha, const float* beta, float* o,
                                           int64_t nrows, int dv) {
  constexpr int LG = DK / 4;    // lanes per column
  constexpr int CPW = 64 / LG;  // columns per wave
  const int lane = threadIdx.x & 63;
  const int gl = lane % LG;
  const int64_t col = ((int64_t)blockIdx.x * (kGB / 64) + (threadIdx.x >> 6)) * CPW + lane / LG;
  const bool live = col < nrows;
  const int64_t c = live ? col : nrows - 1;  // past the end: the last column, not stored
  const int h = (int)(c / dv), j = (int)(c - (int64_t)h * dv);
  f32x4_t* sp = reinterpret_cast<f32x4_t*>(S + c * DK) + gl;
  const f32x4_t s4 = __builtin_nontemporal_load(sp);
  const float4 k4 = reinterpret_cast<const float4*>(k + (int64_t)h * DK)[gl];
  const float4 q4 = reinterpret_cast<const float4*>(q + (int64_t)h * DK)[gl];
  const float vj = v[c];
  const float al = alpha[h], be = beta[h];
  float a = s4.x * k4.x, b = s4.x * q4.x, kq = k4.x * q4.x;
  a = fmaf(s4.y, k4.y, a);
  b = fmaf(s4.y, q4.y, b);
  kq = fmaf(k4.y, q4.y, kq);
  a = fmaf(s4.z, k4.z, a);
  b = fmaf(s4.z, q4.z, b);
  kq = fmaf(k4.z, q4.z, kq);
  a = fmaf(s4.w, k4.w, a);
  b = fmaf(s4.w, q4.w, b);
  kq = fmaf(k4.w, q4.w, kq);
  a = group_sum<LG>(a);
  b = group_sum<LG>(b);
  kq = group_sum<LG>(kq);
  const float d = be * (vj - al * a);
  f32x4_t n4;
  n4.x = fmaf(d, k4.x, al * s4.x);
  n4.y = fmaf(d, k4.y, al * s4.y);
  n4.z = fmaf(d, k4.z, al * s4.z);
  n4.w = fmaf(d, k4.w, al * s4.w);
  if (live) {
    __builtin_nontemporal_store(n4, sp);
    if (gl == 0) o[c] = fmaf(d, kq, al * b);
  }
}

template <int DK>
hipError_t launch_dk(float* S, const float* q, const float* k, const float* v, const float* alpha,
                     const float* beta, float* o, int heads, int dv, hipStream_t s) {
  constexpr int CPB = (kGB / 64) * (64 / (DK / 4));  // columns per workgroup
  const int64_t nrows = (int64_t)heads * dv;
  const int64_t nb = (nrows + CPB - 1) / CPB;
  hipLaunchKernelGGL(k_gdn<DK>, dim3((unsigned)nb), dim3(kGB), 0, s, S, q, k, v, alpha, beta, o, nrows,
                     dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_step(float* S, const float* q, const float* k, const float* v, const float* alpha,
                           const float* beta, float* o, int heads, int dk, int dv, hipStream_t s) {
  if (heads == 0) return hipSuccess;
  if (dk == 64) return launch_dk<64>(S, q, k, v, alpha, beta, o, heads, dv, s);
  if (dk == 128) return launch_dk<128>(S, q, k, v, alpha, beta, o, heads, dv, s);
  return launch_dk<256>(S, q, k, v, alpha, beta, o, heads, dv, s);
}

}  // namespace qmoe
