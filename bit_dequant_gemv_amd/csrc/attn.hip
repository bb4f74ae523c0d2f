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
// Two launches: k_attn_mma (rotations and cache rows, then the scores and the
// weighted values of a key range on the matrix cores; a workgroup per KV head and
// key range, so each key and value row is read from HBM once for the whole query
// group) and k_attn_combine (the ranges' partial results merged).
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kMaxSplit = 2048;  // ranges per head: at most ceil(256 / Hkv) <= 256

// a partial result record: acc[D], m, l, padding to a multiple of 16 bytes
template <int D>
constexpr int rec() {
  return D + 4;
}

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

// Partial attention of the G <= 16 query heads of KV head g over keys [t0, t1): the
// running max m, the sum of weights l and the weighted sum of values acc[D], in
// part[h][split][D + 4] = {acc..., m, l, -, -}, on the matrix cores.  The heads are
// the 16 columns of v_mfma_f32_16x16x4_f32 tiles (heads past G are zero), so
// every key and value row is read once per workgroup, from HBM straight into the
// operand registers, with no LDS staging:
//   scores  S^T[key][head] = sum_d K[key][d] q[head][d]: A = 16 keys x 4 dims, B =
//           4 dims x 16 heads; lane group lg = l/16 walks its quarter of the dims
//           (a contiguous slice of the key row), one dim per step;
//   values  O^T[dim][head] += sum_key V[key][dim] P[head][key]: at step j lane group
//           lg takes key 4*lg + j, whose weight is register j of the lane's score
//           tile (D[row 4*lg + v][col l%16]), so the weights never move; a lane's
//           float4 of V at dims 4*(l%16) + 64c .. +3 feeds four tiles, tile (c, comp)
//           holding dims 64c + 4*row + comp.
// A workgroup has 4 waves; wave w takes the range's 16-key subtiles w, w + 4, ...
// with its own online softmax (max and sum per head), and the 4 waves merge through
// LDS into the record.  Each wave requests its keys, then q is normalised and rotated,
// then the wave requests its values.
constexpr int kMmaKeys = 64;  // keys per workgroup pass: 4 waves x 16

template <int D>
__global__ __launch_bounds__(256) void k_attn_mma(const float* q, const float* knew,
                                                  const float* vnew, float* kc, float* vc,
                                                  float* part, int G, int64_t Tmax, int pos,
                                                  float theta, int rot_dim, int chunk, int nsplit,
                                                  AttnQ Q) {
  constexpr int DQ = D / 4;   // dims per lane group in the score phase
  constexpr int NC = D / 64;  // 64-dim blocks of the value phase
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  // normalised q rows (rows >= G zero), then rotated; after the key loop the same
  // memory holds two waves' value sums [dim][head] for the merge
  __shared__ __align__(16) float s_qq[2 * 16 * D];
  float* s_qn = s_qq;
  float* s_q = s_qq + 16 * D;
  float* s_o = s_qq;
  __shared__ float s_cs[2][D / 2];
  __shared__ __align__(16) float s_kn[D], s_vn[D];
  __shared__ float s_ml[4][2][16];                // per wave: running max, weight sum per head
  const int g = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int r = lane & 15, lg = lane >> 4;
  const int T = pos + 1;
  const int t0 = split * chunk, t1 = min(T, t0 + chunk);
  const bool owns_pos = t0 <= pos && pos < t1;
  float* kg = kc + (int64_t)g * Tmax * D;
  float* vg = vc + (int64_t)g * Tmax * D;
  const int half = rot_dim / 2;

  // ---- loads, in order of need.  q: the 16 lanes tid = 16*qh + ql of head qh hold its
  // float4 at dims 64u + 4*ql (u < D/64): coalesced here, and without LDS bank
  // conflicts below (heads past G read head 0, unused)
  const int qh = tid >> 4, ql = tid & 15;
  float4 qv[D / 64], qw[D / 64];
  {
    const float* qrow = q + (int64_t)(g * G + (qh < G ? qh : 0)) * Q.q_stride;
    const float* wrow = Q.qnw ? Q.qnw : q;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) {
      qv[u] = reinterpret_cast<const float4*>(qrow + 64 * u)[ql];
      qw[u] = reinterpret_cast<const float4*>(wrow + 64 * u)[ql];
    }
  }
  // the new key and value (every workgroup reads them; the owner of pos uses them):
  // thread tid < D/4 holds dims 4*tid .. +3
  float4 kn4 = make_float4(0.f, 0.f, 0.f, 0.f), vn4 = kn4, kw4 = kn4;
  if (tid < D / 4) {
    kn4 = reinterpret_cast<const float4*>(knew + (int64_t)g * D)[tid];
    vn4 = reinterpret_cast<const float4*>(vnew + (int64_t)g * D)[tid];
    kw4 = reinterpret_cast<const float4*>(Q.knw ? Q.knw : knew)[tid];
  }
  // a subtile's loads: K rows in the score operand layout (lane: key r, dims
  // DQ*lg .. +DQ-1, a contiguous slice) and V rows in the value operand layout (lane:
  // keys 4*lg + j, dims 4r + 64c ..); keys past the range read its last row
  float kr[DQ];
  float4 vr[4][NC];
  auto load_k = [&](int kb) {
    const int key = min(kb + r, t1 - 1);
    const float4* kp = reinterpret_cast<const float4*>(kg + (int64_t)key * D + DQ * lg);
#pragma unroll
    for (int u = 0; u < DQ / 4; ++u) {
      const float4 f = kp[u];
      kr[4 * u] = f.x, kr[4 * u + 1] = f.y, kr[4 * u + 2] = f.z, kr[4 * u + 3] = f.w;
    }
  };
  auto load_v = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vk = min(kb + 4 * lg + j, t1 - 1);
      const float4* vp = reinterpret_cast<const float4*>(vg + (int64_t)vk * D) + r;
#pragma unroll
      for (int c = 0; c < NC; ++c) vr[j][c] = vp[16 * c];
    }
  };
  auto load_sub = [&](int kb) { load_k(kb); load_v(kb); };
  const int kb0 = t0 + 16 * wv;
  // the keys go out before the prologue, the values after it: the prologue's work is
  // not queued behind all 32 loads (a wave stalls at a load the memory pipeline has no
  // room for), and the scores, which need the keys first, start sooner
  load_k(min(kb0, t1 - 1));  // a wave with no subtile loads the last row, unused
  // ---- rotation angles.  pos * theta^(-2i/rot_dim) reaches 1e4 rad and more, so the
  // angle is formed and reduced modulo 2 pi in double (2 pi in two parts: exact for
  // these magnitudes); the cosine and sine of the reduced angle are taken in float
  static_assert(D / 2 <= 256, "one thread per rotation pair");
  if (tid < half) {
    const double f = exp(-2.0 * tid / rot_dim * log((double)theta));
    const double ang = (double)pos * f;
    const double k = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
    const double red = fma(-k, 2.4492935982947064e-16, fma(-k, 6.283185307179586, ang));
    float sn, cs;
    sincosf((float)red, &sn, &cs);
    s_cs[0][tid] = cs;
    s_cs[1][tid] = sn;
  }
  // ---- q normalisation: 1 / sqrt(mean(x^2) + eps) over the head's D dims (its 16
  // lanes add their sums); the result goes to s_qn and, for the dims past rot_dim
  // (the pair pass below overwrites the others), to s_q
  {
    float rq = 1.f;
    if (Q.qnw) {
      float ss = 0.f;
#pragma unroll
      for (int u = 0; u < D / 64; ++u)
        ss = fmaf(qv[u].x, qv[u].x, fmaf(qv[u].y, qv[u].y, fmaf(qv[u].z, qv[u].z, fmaf(qv[u].w, qv[u].w, ss))));
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) ss += __shfl_xor(ss, o2);
      rq = 1.0f / sqrtf(ss / (float)D + Q.eps);
    }
#pragma unroll
    for (int u = 0; u < D / 64; ++u) {
      float4 x = qv[u];
      if (Q.qnw) x = make_float4(x.x * rq * qw[u].x, x.y * rq * qw[u].y, x.z * rq * qw[u].z, x.w * rq * qw[u].w);
      if (qh >= G) x = make_float4(0.f, 0.f, 0.f, 0.f);
      reinterpret_cast<float4*>(s_qn + qh * D + 64 * u)[ql] = x;
      reinterpret_cast<float4*>(s_q + qh * D + 64 * u)[ql] = x;
    }
  }
  // the new key's normalisation (threads below D/4 hold it: one wave, or part of one)
  float kn[4] = {kn4.x, kn4.y, kn4.z, kn4.w};
  if (Q.knw && owns_pos && wv == 0) {
    float ss = fmaf(kn4.x, kn4.x, fmaf(kn4.y, kn4.y, fmaf(kn4.z, kn4.z, kn4.w * kn4.w)));
    if (tid >= D / 4) ss = 0.f;
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) ss += __shfl_xor(ss, o2);
    const float rk = 1.0f / sqrtf(ss / (float)D + Q.eps);
    kn[0] *= rk * kw4.x, kn[1] *= rk * kw4.y, kn[2] *= rk * kw4.z, kn[3] *= rk * kw4.w;
  }
  if (owns_pos && tid < D / 4) {
    reinterpret_cast<float4*>(s_kn)[tid] = make_float4(kn[0], kn[1], kn[2], kn[3]);  // rotated below
    reinterpret_cast<float4*>(s_vn)[tid] = vn4;
  }
  __syncthreads();
  // ---- rotations by pairs: (x_i, x_{i+half}) -> (x_i c - x_{i+half} s, x_{i+half} c +
  // x_i s) for i < half, consecutive pairs on consecutive lanes; the new key's pairs
  // (its row is one more item list) after the 16 q rows
  float kpair[2][2];  // the key pair of this thread, if any (half <= 128 < 256: at most one)
  for (int it = tid; it < 17 * half; it += 256) {
    const int hh = it / half, i = it % half;
    const float* src = hh < 16 ? s_qn + hh * D : s_kn;
    const float x1 = src[i], x2 = src[i + half], c = s_cs[0][i], sn = s_cs[1][i];
    const float y1 = fmaf(x1, c, -x2 * sn), y2 = fmaf(x2, c, x1 * sn);
    if (hh < 16) {
      s_q[hh * D + i] = y1;
      s_q[hh * D + i + half] = y2;
    } else {
      kpair[(it - tid) / 256 & 1][0] = y1;
      kpair[(it - tid) / 256 & 1][1] = y2;
    }
  }
  __syncthreads();  // s_kn is read above and rewritten below
  if (owns_pos) {
    for (int it = tid; it < 17 * half; it += 256)
      if (it >= 16 * half) {
        const int i = it - 16 * half;
        s_kn[i] = kpair[(it - tid) / 256 & 1][0];
        s_kn[i + half] = kpair[(it - tid) / 256 & 1][1];
      }
  }
  __syncthreads();
  if (owns_pos && tid < D / 4) {  // the rotated key and the value into row pos of the caches
    reinterpret_cast<float4*>(kg + (int64_t)pos * D)[tid] = reinterpret_cast<const float4*>(s_kn)[tid];
    reinterpret_cast<float4*>(vg + (int64_t)pos * D)[tid] = vn4;
  }
  load_v(min(kb0, t1 - 1));
  const float scale = 1.0f / sqrtf((float)D);
  float m = -INFINITY, l = 0.f;  // of head r (every lane group holds the same)
  f32x4 o[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int cp = 0; cp < 4; ++cp) o[c][cp] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb = kb0; kb < t1; kb += 4 * 16) {
    if (kb != kb0) load_sub(kb);
    // the row at pos (also where a key past the range was clamped to it) was read
    // before this call wrote it: the new key and value instead
    if (owns_pos && min(kb + r, t1 - 1) == pos) {
#pragma unroll
      for (int s2 = 0; s2 < DQ; ++s2) kr[s2] = s_kn[DQ * lg + s2];
    }
    if (owns_pos) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (min(kb + 4 * lg + j, t1 - 1) == pos) {
#pragma unroll
          for (int c = 0; c < NC; ++c) vr[j][c] = reinterpret_cast<const float4*>(s_vn)[r + 16 * c];
        }
    }
    // scores of the subtile's 16 keys for the 16 heads (q from LDS, 16 dims at a time)
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h4 = 0; h4 < DQ / 16; ++h4) {
      float qa[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 e = reinterpret_cast<const float4*>(s_q + r * D + DQ * lg + 16 * h4)[u];
        qa[4 * u] = e.x, qa[4 * u + 1] = e.y, qa[4 * u + 2] = e.z, qa[4 * u + 3] = e.w;
      }
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) st = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[16 * h4 + s2], qa[s2], st, 0, 0, 0);
    }
    // lane: keys kb + 4*lg + v of head r
    const int nk = min(16, t1 - kb);
    float sv[4], tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = 4 * lg + v < nk ? st[v] * scale : -INFINITY;
      tmax = fmaxf(tmax, sv[v]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(m, tmax);
    const float corr = __expf(m - mn);  // m = -inf on the first subtile: 0
    float p[4], ps = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] = 4 * lg + v < nk ? __expf(sv[v] - mn) : 0.f;
      ps += p[v];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = fmaf(l, corr, ps);
    m = mn;
    // values: the tiles' columns are heads, so the rescale is the lane's own corr
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int cp = 0; cp < 4; ++cp) o[c][cp] *= corr;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        o[c][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[j][c].x, p[j], o[c][0], 0, 0, 0);
        o[c][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[j][c].y, p[j], o[c][1], 0, 0, 0);
        o[c][2] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[j][c].z, p[j], o[c][2], 0, 0, 0);
        o[c][3] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[j][c].w, p[j], o[c][3], 0, 0, 0);
      }
  }
  // ---- the 4 waves' states merged: M = max m_w, O = sum_w e^(m_w - M) O_w, L likewise,
  // in two rounds through the q buffers (free once every wave is past its loop): waves
  // 2, 3 hand their weighted sums to waves 0, 1, then wave 1 to wave 0.
  // Tile (c, cp) register v of lane l: dim 64c + 4*(4*lg + v) + cp, head r.
  if (lg == 0) {
    s_ml[wv][0][r] = m;
    s_ml[wv][1][r] = l;
  }
  __syncthreads();
  float M = s_ml[0][0][r];
#pragma unroll
  for (int w = 1; w < 4; ++w) M = fmaxf(M, s_ml[w][0][r]);
  const float fw = m == -INFINITY ? 0.f : __expf(m - M);  // this wave's weight (no keys: 0)
  auto put_o = [&](int slot) {  // the wave's sums, already weighted
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int cp = 0; cp < 4; ++cp)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          s_o[slot * D * 16 + (64 * c + 4 * (4 * lg + v) + cp) * 16 + r] = o[c][cp][v];
  };
  auto add_o = [&](int slot) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int cp = 0; cp < 4; ++cp)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[c][cp][v] += s_o[slot * D * 16 + (64 * c + 4 * (4 * lg + v) + cp) * 16 + r];
  };
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int cp = 0; cp < 4; ++cp) o[c][cp] *= fw;
  if (wv >= 2) put_o(wv - 2);
  __syncthreads();
  if (wv < 2) add_o(wv);
  __syncthreads();
  if (wv == 1) put_o(0);
  __syncthreads();
  if (wv == 0) {
    add_o(0);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_ml[w][0][r];
      L = fmaf(mw == -INFINITY ? 0.f : __expf(mw - M), s_ml[w][1][r], L);
    }
    if (r < G) {
      float* out = part + ((int64_t)(g * G + r) * nsplit + split) * rec<D>();
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int cp = 0; cp < 4; ++cp)
#pragma unroll
          for (int v = 0; v < 4; ++v) out[64 * c + 4 * (4 * lg + v) + cp] = o[c][cp][v];
      if (lg == 0) {
        out[D] = M;
        out[D + 1] = L;
      }
    }
  }
  if (Q.gate && split == 0)  // the gate halves of the group's query rows, copied out
    for (int i = tid; i < G * D; i += 256)
      Q.gate[(int64_t)(g * G + i / D) * D + i % D] = q[(int64_t)(g * G + i / D) * Q.q_stride + D + i % D];
}

// The partial results of head h merged: weights w_s = exp(m_s - M) of the splits,
// o = sum_s w_s acc_s / sum_s w_s l_s.  A workgroup per head and slice of DB dims
// (blockIdx.y), 1024 threads: 1024/DB groups of DB threads, group j summing the
// splits s = j (mod 1024/DB) with its loads issued UB at a time.  Every slice's
// workgroup computes the head's weights itself.  (Measured at 32 heads, D 256 and
// 128 ranges per head: one workgroup per head took 18.0 us per token, 64-dim
// slices 17.2, and 8 instead of 16 loads at a time, none of them past the last
// range, 17.0.)
template <int D, int DB, int UB>
__global__ __launch_bounds__(1024) void k_attn_combine(const float* part, float* o, int nsplit) {
  constexpr int NG = 1024 / DB;
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
  const int d = (int)blockIdx.y * DB + tid % DB, j = tid / DB;
  float a = 0.f;
  for (int s0 = j; s0 < nsplit; s0 += UB * NG) {
    float v[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int s = min(s0 + u * NG, nsplit - 1);  // past the end: a valid record, weight 0
      v[u] = ph[(int64_t)s * rec<D>() + d];
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int s = s0 + u * NG;
      a = fmaf(s < nsplit ? s_w[s] : 0.f, v[u], a);
    }
  }
  s_acc[tid] = a;
  __syncthreads();
  if (tid < DB) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) t += s_acc[g * DB + tid];
    o[(int64_t)h * D + (int)blockIdx.y * DB + tid] = t / L;
  }
}

// key ranges: about one workgroup per CU, in whole passes of the 4 waves
constexpr int kWantSplits = 256;
int attn_chunk(int Hkv, int T, int unit) {
  const int64_t want = kWantSplits;
  int64_t c = ((int64_t)T * Hkv + want - 1) / want;
  c = (c + unit - 1) / unit * unit;
  return (int)(c < unit ? unit : c);
}

template <int D>
hipError_t launch_d(const float* q, const float* k, const float* v, float* kc, float* vc, int Hq,
                    int Hkv, int64_t Tmax, int pos, float theta, int rot_dim, float* o, float* ws,
                    const AttnQ& Q, hipStream_t s) {
  const int T = pos + 1, G = Hq / Hkv;
  float* part = ws;
  const int chunk = attn_chunk(Hkv, T, kMmaKeys);
  const int nsplit = (T + chunk - 1) / chunk;
  hipLaunchKernelGGL(k_attn_mma<D>, dim3(Hkv, nsplit), dim3(256), 0, s, q, k, v, kc, vc, part, G, Tmax,
                     pos, theta, rot_dim, chunk, nsplit, Q);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  constexpr int DB = D < 64 ? D : 64;
  hipLaunchKernelGGL((k_attn_combine<D, DB, 8>), dim3(Hq, D / DB), dim3(1024), 0, s, part, o, nsplit);
  return hipGetLastError();
}

}  // namespace

// ranges of any T <= Tmax: at most ceil(T / kMmaKeys) (ranges hold whole passes) and
// at most ceil(256 / Hkv) (ranges hold at least T * Hkv / 256 keys)
size_t attn_workspace_bytes(int Hq, int Hkv, int D, int Tmax) {
  const int64_t a = ((int64_t)Tmax + kMmaKeys - 1) / kMmaKeys, b = (kWantSplits + Hkv - 1) / Hkv;
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
