// Batched decode through one MoE layer: T tokens, each routed to its own top-K.
//
// Row t of the result equals the batch-1 layer on token t.  To read each active
// expert's weights once per batch, the (token, k) pairs are grouped by expert:
// a histogram over the routed expert ids, an exclusive scan into per-expert
// offsets, and a stable scatter of the pair ids (pair p = t*K + k, in ascending
// p within an expert).  The shared expert is one more group holding every token
// (pair ids T*K + t).  Then, for each group, the expert's gate/up rows are
// applied to each of its tokens (a row block stays in cache across the group's
// tokens), the down rows likewise, and a per-token combine adds the weighted
// routed outputs, the sigmoid-gated shared output and the residual.
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kBB = 256;  // threads per workgroup

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

struct BatchWs {
  int64_t logits, grp, h, y, total;
  // grp block: n_groups | group_expert[E+1] | group_off[E+2] | pair_list[T*K+T]
};

BatchWs batch_ws(int E, int K, int H, int I, int T) {
  BatchWs b;
  const int64_t P = (int64_t)T * K + T;
  b.logits = 256;
  b.grp = b.logits + align256((int64_t)T * E * 4);
  b.h = b.grp + align256(4 * (1 + (E + 1) + (E + 2) + P));
  b.y = b.h + align256(P * I * 4);
  b.total = b.y + align256(P * H * 4);
  return b;
}

struct GroupTables {
  int* n_groups;
  int* group_expert;  // expert id, or -1 for the shared expert
  int* group_off;     // [n_groups + 1] offsets into pair_list
  int* pair_list;
};

GroupTables group_tables(uint8_t* ws, const BatchWs& b, int E) {
  GroupTables g;
  int* base = reinterpret_cast<int*>(ws + b.grp);
  g.n_groups = base;
  g.group_expert = base + 1;
  g.group_off = base + 1 + (E + 1);
  g.pair_list = base + 1 + (E + 1) + (E + 2);
  return g;
}

// one workgroup: histogram -> scan -> stable scatter (deterministic)
__global__ __launch_bounds__(1024) void k_group(const int32_t* __restrict__ idx, int T, int K,
                                                int E, GroupTables G) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts];
  __shared__ int wsum[16];
  const int P = T * K;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int e = idx[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan of cnt (pairs) and of (cnt > 0) (group slots), E <= 4096, 1024 threads x 4
  const int per = (E + blockDim.x - 1) / blockDim.x;
  int lp = 0, lg = 0;
  for (int j = 0; j < per; ++j) {
    const int e = threadIdx.x * per + j;
    if (e < E) {
      lp += cnt[e];
      lg += cnt[e] > 0;
    }
  }
  // scan (lp, lg) packed: lp < 2^16 (P <= 2048), lg < 2^13
  int v = (lp << 16) | lg;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = v;
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m, 64);
    if (lane >= m) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
      const int t = wsum[i];
      wsum[i] = acc;
      acc += t;
    }
  }
  __syncthreads();
  int excl = incl - v + wsum[wv];
  int ep = excl >> 16, eg = excl & 0xFFFF;
  for (int j = 0; j < per; ++j) {
    const int e = threadIdx.x * per + j;
    if (e < E) {
      off[e] = ep;
      if (cnt[e] > 0) {
        G.group_expert[eg] = e;
        G.group_off[eg] = ep;
        ++eg;
      }
      ep += cnt[e];
    }
  }
  __syncthreads();
  // last thread owning the totals writes the shared group
  if (threadIdx.x == blockDim.x - 1) {
    const int ng = eg;  // total routed groups (inclusive end of the last thread)
    G.group_expert[ng] = -1;
    G.group_off[ng] = ep;
    G.group_off[ng + 1] = ep + T;
    G.n_groups[0] = ng + 1;
  }
  // stable scatter: rank of pair p among earlier pairs of the same expert
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int e = idx[p];
    if ((unsigned)e >= (unsigned)E) continue;
    int r = 0;
    for (int q = 0; q < p; ++q) r += idx[q] == e;
    G.pair_list[off[e] + r] = p;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < T; t += blockDim.x) {
    // the shared group's pairs follow every routed pair
    int routed = 0;
    for (int e = 0; e < E; ++e) routed += cnt[e];
    G.pair_list[routed + t] = P + t;
  }
}

struct PoolArgsB {
  const uint8_t* rbase;
  int64_t rstride;
  const uint8_t* sblk;
  int E, H, I, T, K;
  int64_t off_g, off_u, off_d, off_gsb, off_usb, off_dsb;
};

__device__ __forceinline__ int token_of(int p, int T, int K) { return p < T * K ? p / K : p - T * K; }

// grid (row blocks, group slots); rows of one block are applied to every token of the group
template <int BITS, int LG, int CPL>
__global__ __launch_bounds__(kBB) void k_bgateup(PoolArgsB P, GroupTables G,
                                                 const float* __restrict__ x,
                                                 float* __restrict__ h, int rows_per_block) {
  constexpr int RPW = 64 / LG;
  const int gi = blockIdx.y;
  if (gi >= G.n_groups[0]) return;
  const int e = G.group_expert[gi];
  const bool eok = e == -1 || (unsigned)e < (unsigned)P.E;
  const uint8_t* blk = e == -1 ? P.sblk : P.rbase + (eok ? (int64_t)e * P.rstride : 0);
  const int C = P.H * BITS / 128, G_ = P.H / kGroup;
  const int64_t rb = (int64_t)P.H * BITS / 8;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gl = lane % LG, sub = lane / LG;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(P.I, r0 + rows_per_block);
  const int p0 = G.group_off[gi], p1 = G.group_off[gi + 1];
  RowDot<BITS, LG, CPL> rd;
  extern __shared__ uint32_t smem[];
  uint32_t* planes = smem;
  float* scl = reinterpret_cast<float*>(smem + C * QTraits<BITS>::PW);
  float* xsum = scl + C;
  for (int pi = p0; pi < p1; ++pi) {
    const int p = G.pair_list[pi];
    const int t = token_of(p, P.T, P.K);
    __syncthreads();  // the previous token's planes are no longer read
    prep_x_coop<BITS>(x + (int64_t)t * P.H, P.H, planes, scl, xsum, threadIdx.x, blockDim.x);
    __syncthreads();
    rd.load_prepped(planes, scl, xsum, C, gl);
    for (int j0 = r0 + wv * RPW; j0 < r1; j0 += (kBB / 64) * RPW) {
      const int j = j0 + sub;
      const bool ok = eok && j < r1;
      const uint8_t* cr[2] = {blk + P.off_g + (int64_t)j * rb, blk + P.off_u + (int64_t)j * rb};
      const uint32_t* sr[2] = {reinterpret_cast<const uint32_t*>(blk + P.off_gsb) + (int64_t)j * G_,
                               reinterpret_cast<const uint32_t*>(blk + P.off_usb) + (int64_t)j * G_};
      const bool okk[2] = {ok, ok};
      uint4 q[2][CPL];
      uint32_t s[2][CPL];
      rd.template fetch<2>(cr, sr, okk, C, gl, q, s);
      float pp[2];
      rd.template dots<2>(q, s, pp);
      const float a = group_sum<LG>(pp[0]);
      const float u = group_sum<LG>(pp[1]);
      if (gl == 0 && j < r1) h[(int64_t)p * P.I + j] = eok ? silu_f(a) * u : __builtin_nanf("");
    }
  }
}

template <int BITS, int LG, int CPL>
__global__ __launch_bounds__(kBB) void k_bdown(PoolArgsB P, GroupTables G,
                                               const float* __restrict__ h,
                                               float* __restrict__ y, int rows_per_block) {
  constexpr int RPW = 64 / LG;
  const int gi = blockIdx.y;
  if (gi >= G.n_groups[0]) return;
  const int e = G.group_expert[gi];
  const bool eok = e == -1 || (unsigned)e < (unsigned)P.E;
  const uint8_t* blk = e == -1 ? P.sblk : P.rbase + (eok ? (int64_t)e * P.rstride : 0);
  const int C = P.I * BITS / 128, G_ = P.I / kGroup;
  const int64_t rb = (int64_t)P.I * BITS / 8;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gl = lane % LG, sub = lane / LG;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(P.H, r0 + rows_per_block);
  const int p0 = G.group_off[gi], p1 = G.group_off[gi + 1];
  RowDot<BITS, LG, CPL> rd;
  extern __shared__ uint32_t smem[];
  uint32_t* planes = smem;
  float* scl = reinterpret_cast<float*>(smem + C * QTraits<BITS>::PW);
  float* xsum = scl + C;
  for (int pi = p0; pi < p1; ++pi) {
    const int p = G.pair_list[pi];
    __syncthreads();
    prep_x_coop<BITS>(h + (int64_t)p * P.I, P.I, planes, scl, xsum, threadIdx.x, blockDim.x);
    __syncthreads();
    rd.load_prepped(planes, scl, xsum, C, gl);
    for (int n0 = r0 + wv * RPW; n0 < r1; n0 += (kBB / 64) * RPW) {
      const int n = n0 + sub;
      const bool ok = eok && n < r1;
      const uint8_t* cr = blk + P.off_d + (int64_t)n * rb;
      const uint32_t* sr = reinterpret_cast<const uint32_t*>(blk + P.off_dsb) + (int64_t)n * G_;
      uint4 q[1][CPL];
      uint32_t s[1][CPL];
      rd.template fetch<1>(&cr, &sr, &ok, C, gl, q, s);
      float pp[1];
      rd.template dots<1>(q, s, pp);
      const float v = group_sum<LG>(pp[0]);
      if (gl == 0 && n < r1) y[(int64_t)p * P.H + n] = eok ? v : __builtin_nanf("");
    }
  }
}

// one workgroup per token: gamma_t = sigmoid(g . x_t), then the combine
__global__ __launch_bounds__(kBB) void k_bcombine(const float* __restrict__ y,
                                                  const float* __restrict__ w,
                                                  const uint16_t* __restrict__ g,
                                                  const float* __restrict__ x,
                                                  const float* residual, float* out, int T, int K,
                                                  int H) {
  __shared__ float red[kBB / 64];
  const int t = blockIdx.x;
  const float* xt = x + (int64_t)t * H;
  float d = 0.f;
  for (int i = threadIdx.x; i < H; i += kBB) d += __uint_as_float((uint32_t)g[i] << 16) * xt[i];
  d = group_sum<64>(d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = d;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < kBB / 64; ++i) tot += red[i];
  const float gamma = sigmoid_f(tot);
  const float* ys = y + ((int64_t)T * K + t) * H;
  for (int n = threadIdx.x; n < H; n += kBB) {
    float acc = residual[(int64_t)t * H + n];
    for (int k = 0; k < K; ++k) acc = fmaf(w[t * K + k], y[((int64_t)t * K + k) * H + n], acc);
    out[(int64_t)t * H + n] = fmaf(gamma, ys[n], acc);
  }
}

template <int BITS, int LG, int CPL>
void run_bgateup(const PoolArgsB& P, const GroupTables& G, int ngroups_max, const float* x,
                 float* h, hipStream_t s) {
  constexpr int RPW = 64 / LG;
  const int rpb = (kBB / 64) * RPW * 4;
  const size_t lds = (size_t)(P.H / QTraits<BITS>::EPC) * (QTraits<BITS>::PW + 2) * 4;
  hipLaunchKernelGGL((k_bgateup<BITS, LG, CPL>), dim3(ceil_div(P.I, rpb), ngroups_max), dim3(kBB),
                     lds, s, P, G, x, h, rpb);
}

template <int BITS, int LG, int CPL>
void run_bdown(const PoolArgsB& P, const GroupTables& G, int ngroups_max, const float* h, float* y,
               hipStream_t s) {
  constexpr int RPW = 64 / LG;
  const int rpb = (kBB / 64) * RPW * 4;
  const size_t lds = (size_t)(P.I / QTraits<BITS>::EPC) * (QTraits<BITS>::PW + 2) * 4;
  hipLaunchKernelGGL((k_bdown<BITS, LG, CPL>), dim3(ceil_div(P.H, rpb), ngroups_max), dim3(kBB), lds,
                     s, P, G, h, y, rpb);
}

template <int BITS>
void dispatch_bgateup(const PoolArgsB& P, const GroupTables& G, int ng, const float* x, float* h,
                      hipStream_t s) {
  const int C = P.H * BITS / 128;
  if (C <= 1) return run_bgateup<BITS, 1, 1>(P, G, ng, x, h, s);
  if (C <= 2) return run_bgateup<BITS, 2, 1>(P, G, ng, x, h, s);
  if (C <= 4) return run_bgateup<BITS, 4, 1>(P, G, ng, x, h, s);
  if (C <= 8) return run_bgateup<BITS, 8, 1>(P, G, ng, x, h, s);
  if (C <= 16) return run_bgateup<BITS, 16, 1>(P, G, ng, x, h, s);
  if (C <= 32) return run_bgateup<BITS, 32, 1>(P, G, ng, x, h, s);
  if (C <= 64) return run_bgateup<BITS, 64, 1>(P, G, ng, x, h, s);
  if (C <= 128) return run_bgateup<BITS, 64, 2>(P, G, ng, x, h, s);
  return run_bgateup<BITS, 64, 4>(P, G, ng, x, h, s);
}

template <int BITS>
void dispatch_bdown(const PoolArgsB& P, const GroupTables& G, int ng, const float* h, float* y,
                    hipStream_t s) {
  const int C = P.I * BITS / 128;
  if (C <= 1) return run_bdown<BITS, 1, 1>(P, G, ng, h, y, s);
  if (C <= 2) return run_bdown<BITS, 2, 1>(P, G, ng, h, y, s);
  if (C <= 4) return run_bdown<BITS, 4, 1>(P, G, ng, h, y, s);
  if (C <= 8) return run_bdown<BITS, 8, 1>(P, G, ng, h, y, s);
  if (C <= 16) return run_bdown<BITS, 16, 1>(P, G, ng, h, y, s);
  if (C <= 32) return run_bdown<BITS, 32, 1>(P, G, ng, h, y, s);
  if (C <= 64) return run_bdown<BITS, 64, 1>(P, G, ng, h, y, s);
  if (C <= 128) return run_bdown<BITS, 64, 2>(P, G, ng, h, y, s);
  return run_bdown<BITS, 64, 4>(P, G, ng, h, y, s);
}

}  // namespace

size_t batched_workspace_bytes(const qmoe_layer& L, int T) {
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  return (size_t)batch_ws(E, K, H, I, T).total;
}

hipError_t launch_layer_batched(const qmoe_layer& L, const float* x, const float* residual,
                                float* out, int T, int32_t* idx, float* w, void* ws,
                                hipStream_t s) {
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const BatchWs b = batch_ws(E, K, H, I, T);
  float* logits = reinterpret_cast<float*>(wsb + b.logits);
  float* h = reinterpret_cast<float*>(wsb + b.h);
  float* y = reinterpret_cast<float*>(wsb + b.y);
  const GroupTables G = group_tables(wsb, b, E);
  hipError_t err = launch_router_topk(L.router, x, T, H, E, K, logits, idx, w, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, s, idx, T, K, E, G);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const qmoe_expert_offsets o = expert_offsets(H, I, L.routed.bits);
  PoolArgsB P;
  P.rbase = static_cast<const uint8_t*>(L.routed.base);
  P.rstride = L.routed.stride;
  P.sblk = static_cast<const uint8_t*>(L.shared.base);
  P.E = E;
  P.H = H;
  P.I = I;
  P.T = T;
  P.K = K;
  P.off_g = o.gate_codes;
  P.off_u = o.up_codes;
  P.off_d = o.down_codes;
  P.off_gsb = o.gate_sb;
  P.off_usb = o.up_sb;
  P.off_dsb = o.down_sb;
  const int ng_max = (T * K < E ? T * K : E) + 1;
  if (L.routed.bits == 4) {
    dispatch_bgateup<4>(P, G, ng_max, x, h, s);
    dispatch_bdown<4>(P, G, ng_max, h, y, s);
  } else {
    dispatch_bgateup<2>(P, G, ng_max, x, h, s);
    dispatch_bdown<2>(P, G, ng_max, h, y, s);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_bcombine, dim3(T), dim3(kBB), 0, s, y, w, L.shared_gate, x, residual, out, T,
                     K, H);
  return hipGetLastError();
}

}  // namespace qmoe
