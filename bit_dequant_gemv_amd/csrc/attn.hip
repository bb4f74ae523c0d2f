// Full-attention decode: one token of grouped-query attention over a key/value
// cache, with rotary position embedding.
//
// The page "flash-moe 소개" (discuss.pytorch.kr), section "손으로 작성한 Metal 컴퓨트
// 셰이더", lists GPU attention (Q@K^T, softmax, scores@V) and RoPE among the
// hand-written kernels; section "Qwen3.5-397B-A17B 모델 아키텍처" puts 15 full-
// attention layers among the 60.  Per token:
//   q, k <- rope(q, pos), rope(k, pos)   (rotate-half on the first rot_dim dims)
//   K[g][pos], V[g][pos] <- k[g], v[g]
//   o[h] = sum_{t <= pos} softmax_t(q[h] . K[g][t] / sqrt(D)) V[g][t],  g = h / (Hq/Hkv)
// Two launches: k_attn_part (rotations and cache rows; a workgroup per KV head and
// key range, one wave per query head of the group, so each key and value row is
// read from HBM once for the whole group; online softmax over tiles of 32 keys
// staged in LDS) and k_attn_combine (the ranges' partial results merged).
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

// keys per LDS tile (16-key tiles, three workgroups per CU, measured slower: 26.8 against
// 26.0 us at context 8192)
constexpr int kTK = 32;
constexpr int kPF = 2;  // float4 of K and of V per thread and tile held in registers
constexpr int kSPL = 64 / kTK;  // lanes per key in the score phase, each summing D / kSPL dims
constexpr int kMaxSplit = 2048;  // splits per head: at most ceil(256 / Hkv) <= 256, or T / kTK

// a partial result record: acc[D], m, l, padding to a multiple of 16 bytes
template <int D>
constexpr int rec() {
  return D + 4;
}

// Partial attention of the G query heads of KV head g over keys [t0, t1): the
// running max m, the sum of weights l and the weighted sum of values acc[D], in
// part[h][split][D + 4] = {acc..., m, l, -, -}.  One wave per query head (measured
// faster than a wave serving four heads, 25.9 against 33.0 us at context 8192, and
// than waves reading rows straight from memory for all 16 heads, 31.6 us).
// RoPE and the cache append are done here too: every workgroup takes the rotation
// angles of position pos (rot_dim / 2 of them, the same for every head) and rotates
// its group's q rows into LDS; the workgroup whose range holds pos rotates the new
// k, writes k and v to row pos of the caches and puts them into its tile directly
// (no other workgroup reads that row in this call).
// The query side: q rows of q_stride floats (D, or 2D when the query projection
// interleaves each head's D query values with its D gate values: the query is the
// first half of the row); qnw / knw: RMS-normalisation weights [D] of q and k, or
// null; gate: the rows' second halves copied out ([Hq][D]), or null.
struct AttnQ {
  int q_stride;
  const float* qnw;
  const float* knw;
  float eps;
  float* gate;
};

template <int D>
__global__ __launch_bounds__(1024) void k_attn_part(const float* q, const float* knew,
                                                    const float* vnew, float* kc, float* vc,
                                                    float* part, int G, int64_t Tmax, int pos,
                                                    float theta, int rot_dim, int chunk, int nsplit,
                                                    AttnQ Q) {
  constexpr int KS = D + 4;  // padded K row in LDS: lanes reading different rows spread over banks
  __shared__ __align__(16) float s_k[kTK * KS];
  __shared__ __align__(16) float s_v[kTK * D];
  __shared__ __align__(16) float s_q[16 * D];
  __shared__ float s_cs[2][D / 2];                // cos, sin of the rotation pairs
  __shared__ __align__(16) float s_kn[D], s_vn[D];  // the token's rotated k and its v
  __shared__ float s_qr[16], s_kr;                 // RMS scales of the q heads and of k
  const int g = blockIdx.x, split = blockIdx.y;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = g * G + wv;
  const int nthr = G * 64;
  const int T = pos + 1;
  const int t0 = split * chunk, t1 = min(T, t0 + chunk);
  const bool owns_pos = t0 <= pos && pos < t1;
  float* kg = kc + (int64_t)g * Tmax * D;
  float* vg = vc + (int64_t)g * Tmax * D;
  // Tile loads go to registers first, kPF float4 of K and of V per thread: the
  // range's first tile is requested before the rotation angles and the q rows are
  // prepared, and each later tile as soon as the one before is in LDS, so HBM
  // latency overlaps that work and the previous tile's scores.  The loads are
  // unconditional (row and index clamped into the range: a key past the range or
  // the row at pos, still stale here, is replaced or ignored when the tile is
  // stored).  One buffer: the 1024-thread workgroup caps a thread at 128 VGPRs,
  // and a second buffer spilled across the double-precision angle computation.
  constexpr int TQ = kTK * D / 4;  // float4 of K (and of V) per tile
  auto issue = [&](int tb, float4 (&rk)[kPF], float4 (&rv)[kPF]) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      const int i = min((int)threadIdx.x + u * nthr, TQ - 1);
      const int t = min(tb + i / (D / 4), t1 - 1), c4 = i % (D / 4);
      rk[u] = reinterpret_cast<const float4*>(kg + (int64_t)t * D)[c4];
      rv[u] = reinterpret_cast<const float4*>(vg + (int64_t)t * D)[c4];
    }
  };
  float4 rk[kPF], rv[kPF];
  issue(t0, rk, rv);
  const int half = rot_dim / 2;
  for (int i = threadIdx.x; i < half; i += nthr) {
    // in double: pos * theta^(-2i/rot_dim) reaches 1e4 rad and more
    const double ang = (double)pos * pow((double)theta, -2.0 * i / rot_dim);
    double sn, cs;
    sincos(ang, &sn, &cs);
    s_cs[0][i] = (float)cs;
    s_cs[1][i] = (float)sn;
  }
  // RMS normalisation scales, 1 / sqrt(mean(x^2) + eps): wave wv for query head
  // h = g*G + wv, wave 0 of the workgroup that owns pos for the new key
  auto rms_scale = [&](const float* x) -> float {
    float ss = 0.f;
#pragma unroll
    for (int d = lane; d < D; d += 64) ss = fmaf(x[d], x[d], ss);
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) ss += __shfl_xor(ss, o2);
    return 1.0f / sqrtf(ss / (float)D + Q.eps);
  };
  if (Q.qnw) {
    const float r = rms_scale(q + (int64_t)h * Q.q_stride);
    if (lane == 0) s_qr[wv] = r;
  }
  if (Q.knw && owns_pos && wv == 0) {
    const float r = rms_scale(knew + (int64_t)g * D);
    if (lane == 0) s_kr = r;
  }
  if (Q.gate && split == 0)  // the gate halves of the group's query rows, copied out
    for (int i = threadIdx.x; i < G * D; i += nthr)
      Q.gate[(int64_t)(g * G + i / D) * D + i % D] = q[(int64_t)(g * G + i / D) * Q.q_stride + D + i % D];
  __syncthreads();
  // x_d of a row, scaled by r * w_d (normalised) when w is given, then rotated:
  // pair (d, d + half) for d < half, (d - half, d) below rot_dim
  auto rot = [&](const float* x, int d, float r, const float* w) -> float {
    auto val = [&](int e) { return w ? x[e] * r * w[e] : x[e]; };
    if (d < half) return val(d) * s_cs[0][d] - val(d + half) * s_cs[1][d];
    if (d < rot_dim) return val(d) * s_cs[0][d - half] + val(d - half) * s_cs[1][d - half];
    return val(d);
  };
  for (int i = threadIdx.x; i < G * D; i += nthr)
    s_q[i] = rot(q + (int64_t)(g * G + i / D) * Q.q_stride, i % D, Q.qnw ? s_qr[i / D] : 1.f, Q.qnw);
  if (owns_pos) {
    for (int d = threadIdx.x; d < D; d += nthr) {
      const float kr = rot(knew + (int64_t)g * D, d, Q.knw ? s_kr : 1.f, Q.knw),
                  vr = vnew[(int64_t)g * D + d];
      s_kn[d] = kr;
      s_vn[d] = vr;
      kg[(int64_t)pos * D + d] = kr;
      vg[(int64_t)pos * D + d] = vr;
    }
  }
  const float scale = 1.0f / sqrtf((float)D);
  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int kt = lane % kTK, kh = lane / kTK;  // score phase: key kt, part kh of the dims
  for (int tb = t0; tb < t1; tb += kTK) {
    const int nk = min(kTK, t1 - tb);
    __syncthreads();  // the previous tile is consumed (and s_q, s_kn, s_vn are written)
    // the tile from its registers into LDS (slots past the registers' reach, when
    // the workgroup has fewer than TQ / kPF threads, are loaded here directly)
    auto put = [&](int i, float4 kv, float4 vv) {
      const int t = i / (D / 4), c4 = i % (D / 4);
      if (tb + t == pos) {  // this token: from LDS (its cache row is written above)
        kv = reinterpret_cast<const float4*>(s_kn)[c4];
        vv = reinterpret_cast<const float4*>(s_vn)[c4];
      }
      *reinterpret_cast<float4*>(s_k + t * KS + 4 * c4) = kv;
      reinterpret_cast<float4*>(s_v)[i] = vv;
    };
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      const int i = (int)threadIdx.x + u * nthr;
      if (i < TQ) put(i, rk[u], rv[u]);
    }
    for (int i = (int)threadIdx.x + kPF * nthr; i < TQ; i += nthr) {
      const int t = min(tb + i / (D / 4), t1 - 1), c4 = i % (D / 4);
      put(i, reinterpret_cast<const float4*>(kg + (int64_t)t * D)[c4],
          reinterpret_cast<const float4*>(vg + (int64_t)t * D)[c4]);
    }
    __syncthreads();
    if (tb + kTK < t1) issue(tb + kTK, rk, rv);  // the next tile, into the freed registers
    // scores: lane (kt, kh) sums part kh of q_h . K_kt
    float sp = 0.f;
    const float* kr = s_k + kt * KS + kh * (D / kSPL);
    const float* qh = s_q + wv * D + kh * (D / kSPL);
#pragma unroll 8
    for (int c = 0; c < D / kSPL; c += 4) {
      const float4 a = *reinterpret_cast<const float4*>(kr + c);
      const float4 b = *reinterpret_cast<const float4*>(qh + c);
      sp = fmaf(a.x, b.x, sp);
      sp = fmaf(a.y, b.y, sp);
      sp = fmaf(a.z, b.z, sp);
      sp = fmaf(a.w, b.w, sp);
    }
#pragma unroll
    for (int o = 32; o >= kTK; o >>= 1) sp += __shfl_xor(sp, o);
    const float sc = kt < nk ? sp * scale : -INFINITY;
    float tmax = sc;
#pragma unroll
    for (int o = kTK / 2; o >= 1; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
    const float mn = fmaxf(m, tmax);
    const float corr = __expf(m - mn);  // m = -inf on the first tile: 0
    const float p = kt < nk ? __expf(sc - mn) : 0.f;
    float ps = p;
#pragma unroll
    for (int o = kTK / 2; o >= 1; o >>= 1) ps += __shfl_xor(ps, o);
    l = fmaf(l, corr, ps);
    m = mn;
    acc.x *= corr;
    acc.y *= corr;
    acc.z *= corr;
    acc.w *= corr;
    // values: lane owns dims 4*lane .. 4*lane+3 (a lane past D/4 repeats lane 0's
    // dims and stores nothing); the weight of key t comes from lane t
    const int vl = lane < D / 4 ? lane : 0;
    for (int t = 0; t < nk; ++t) {
      const float pt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), t));
      const float4 vv = reinterpret_cast<const float4*>(s_v + t * D)[vl];
      acc.x = fmaf(pt, vv.x, acc.x);
      acc.y = fmaf(pt, vv.y, acc.y);
      acc.z = fmaf(pt, vv.z, acc.z);
      acc.w = fmaf(pt, vv.w, acc.w);
    }
  }
  float* out = part + ((int64_t)h * nsplit + split) * rec<D>();
  if (lane < D / 4) reinterpret_cast<float4*>(out)[lane] = acc;
  if (lane == 0) {
    out[D] = m;
    out[D + 1] = l;
  }
}

// The partial results of head h merged: weights w_s = exp(m_s - M) of the splits,
// o = sum_s w_s acc_s / sum_s w_s l_s.  1024 threads: 1024/D groups of D threads,
// group j summing the splits s = j (mod 1024/D) with its loads issued 16 at a time.
template <int D>
__global__ __launch_bounds__(1024) void k_attn_combine(const float* part, float* o, int nsplit) {
  constexpr int NG = 1024 / D;
  __shared__ float s_w[kMaxSplit];
  __shared__ float s_red[16];
  __shared__ float s_acc[1024];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* ph = part + (int64_t)h * nsplit * rec<D>();
  float mx = -INFINITY;
  for (int s = tid; s < nsplit; s += 1024) mx = fmaxf(mx, ph[(int64_t)s * rec<D>() + D]);
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
  if (lane == 0) s_red[wv] = mx;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) M = fmaxf(M, s_red[w]);
  __syncthreads();  // s_red is reused
  float ls = 0.f;
  for (int s = tid; s < nsplit; s += 1024) {
    const float* ps = ph + (int64_t)s * rec<D>();
    const float w = __expf(ps[D] - M);
    s_w[s] = w;
    ls = fmaf(w, ps[D + 1], ls);
  }
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) ls += __shfl_xor(ls, o2);
  if (lane == 0) s_red[wv] = ls;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) L += s_red[w];
  const int d = tid % D, j = tid / D;
  float a = 0.f;
  for (int s0 = j; s0 < nsplit; s0 += 16 * NG) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int s = min(s0 + u * NG, nsplit - 1);  // past the end: a valid record, weight 0
      v[u] = ph[(int64_t)s * rec<D>() + d];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int s = s0 + u * NG;
      a = fmaf(s < nsplit ? s_w[s] : 0.f, v[u], a);
    }
  }
  s_acc[tid] = a;
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) t += s_acc[g * D + tid];
    o[(int64_t)h * D + tid] = t / L;
  }
}

// keys per split: about one workgroup per CU (a workgroup fills a CU's LDS), whole
// tiles
// (128 ranges measured 35.7 us)
constexpr int kWantSplits = 256;  // 512 measured slower (30.2 us)
int attn_chunk(int Hkv, int T) {
  const int64_t want = kWantSplits;
  int64_t c = ((int64_t)T * Hkv + want - 1) / want;
  c = (c + kTK - 1) / kTK * kTK;
  return (int)(c < kTK ? kTK : c);
}

template <int D>
hipError_t launch_d(const float* q, const float* k, const float* v, float* kc, float* vc, int Hq,
                    int Hkv, int64_t Tmax, int pos, float theta, int rot_dim, float* o, float* ws,
                    const AttnQ& Q, hipStream_t s) {
  const int T = pos + 1, G = Hq / Hkv;
  const int chunk = attn_chunk(Hkv, T);
  const int nsplit = (T + chunk - 1) / chunk;
  float* part = ws;
  hipLaunchKernelGGL(k_attn_part<D>, dim3(Hkv, nsplit), dim3(G * 64), 0, s, q, k, v, kc, vc, part, G,
                     Tmax, pos, theta, rot_dim, chunk, nsplit, Q);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_attn_combine<D>, dim3(Hq), dim3(1024), 0, s, part, o, nsplit);
  return hipGetLastError();
}

}  // namespace

// splits of any T <= Tmax: at most ceil(T / kTK) (chunks hold whole tiles) and at most
// ceil(256 / Hkv) (chunks hold at least T * Hkv / 256 keys)
size_t attn_workspace_bytes(int Hq, int Hkv, int D, int Tmax) {
  const int64_t a = ((int64_t)Tmax + kTK - 1) / kTK, b = (kWantSplits + Hkv - 1) / Hkv;
  const int64_t nsplit = a < b ? a : b;
  return (size_t)((int64_t)Hq * nsplit * (D + 4)) * 4;
}

hipError_t launch_attn_decode(const float* q, const float* k, const float* v, float* kc, float* vc,
                              int Hq, int Hkv, int D, int Tmax, int pos, float theta, int rot_dim,
                              float* o, void* ws, hipStream_t s, bool q_gate_rows,
                              const float* q_norm_w, const float* k_norm_w, float eps, float* gate) {
  float* w = static_cast<float*>(ws);
  AttnQ Q;
  Q.q_stride = q_gate_rows ? 2 * D : D;
  Q.qnw = q_norm_w;
  Q.knw = k_norm_w;
  Q.eps = eps;
  Q.gate = q_gate_rows ? gate : nullptr;
  if (D == 64) return launch_d<64>(q, k, v, kc, vc, Hq, Hkv, Tmax, pos, theta, rot_dim, o, w, Q, s);
  if (D == 128) return launch_d<128>(q, k, v, kc, vc, Hq, Hkv, Tmax, pos, theta, rot_dim, o, w, Q, s);
  return launch_d<256>(q, k, v, kc, vc, Hq, Hkv, Tmax, pos, theta, rot_dim, o, w, Q, s);
}

}  // namespace qmoe
