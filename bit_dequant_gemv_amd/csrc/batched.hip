// Batched decode through one MoE layer: T tokens, each routed to its own top-K.
//
// Row t of the result is the batch-1 layer on token t (up to the order of fp32 sums).  To read each active
// expert's weights once per batch, the (token, k) pairs are grouped by expert:
// a histogram over the routed expert ids, an exclusive scan into per-expert
// offsets, and a stable scatter of the pair ids (pair p = t*K + k, in ascending
// p within an expert).  The shared expert takes every token (pair ids T*K + t).
// Each expert's pairs are cut into chunks of at most kChunk, so a popular expert
// (the shared one always) is spread over many workgroups.  The fixed-point x
// planes of every token are built once; a workgroup then loads its block of an
// expert's gate/up rows into registers and applies them to each token of its
// chunk.  The shared expert's gate/up chunks (32 tokens each) run on the matrix
// cores instead, as fp32 GEMM tiles of dequantised weights by the tokens' x.  The
// SwiGLU outputs h get planes of their own, the down rows go the same way as the
// routed gate/up rows, and a per-token combine adds the weighted routed outputs,
// the sigmoid-gated shared output and the residual.
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kBB = 256;  // threads per workgroup

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

// most pairs per group chunk.  The shared expert serves every token, and each of its
// chunks reads its rows again: 32 measured best on the 64-token batch (320 us,
// against 324 at 8, 322 at 16 and 332 at 64)
constexpr int kChunk = 32;

template <int BITS>
constexpr int plane_words(int n) {  // per vector: planes, then C scales, then C sums
  return (n / QTraits<BITS>::EPC) * (QTraits<BITS>::PW + 2);
}

struct BatchWs {
  int64_t logits, grp, xp, h, hp, y, total;
  // grp block: n_groups | group_expert[GM] | group_off[GM+1] | pair_list[T*K+T]
};

// group chunks in all, at most: a routed expert's chunks hold >= 1 pair each
// (<= T*K of them), the shared expert's ceil(T / kChunk)
inline int max_groups(int T, int K) { return T * K + (T + kChunk - 1) / kChunk; }

BatchWs batch_ws(int E, int K, int H, int I, int T, int bits) {
  BatchWs b;
  const int64_t P = (int64_t)T * K + T;
  const int GM = max_groups(T, K);
  const int pvx = bits == 4 ? plane_words<4>(H) : plane_words<2>(H);
  const int pvh = bits == 4 ? plane_words<4>(I) : plane_words<2>(I);
  b.logits = 256;
  b.grp = b.logits + align256((int64_t)T * E * 4);
  b.xp = b.grp + align256(4 * (1 + GM + (GM + 1) + P));
  b.h = b.xp + align256((int64_t)T * pvx * 4);
  b.hp = b.h + align256(P * I * 4);
  b.y = b.hp + align256(P * pvh * 4);
  b.total = b.y + align256(P * H * 4);
  return b;
}

struct GroupTables {
  int* n_groups;
  int* group_expert;  // expert id, or -1 for the shared expert
  int* group_off;     // [n_groups + 1] offsets into pair_list
  int* pair_list;
};

GroupTables group_tables(uint8_t* ws, const BatchWs& b, int T, int K) {
  GroupTables g;
  const int GM = max_groups(T, K);
  int* base = reinterpret_cast<int*>(ws + b.grp);
  g.n_groups = base;
  g.group_expert = base + 1;
  g.group_off = base + 1 + GM;
  g.pair_list = base + 1 + GM + (GM + 1);
  return g;
}

// one workgroup: histogram -> scan -> stable scatter (deterministic); groups are
// chunks of at most kChunk pairs of one expert, in expert order, the shared
// expert's chunks last
__global__ __launch_bounds__(1024) void k_group(const int32_t* __restrict__ idx, int T, int K,
                                                int E, GroupTables G) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts];
  __shared__ __align__(16) int sidx[kMaxBatch * kMaxTopK + 16];  // + padding of -1
  __shared__ int wsum[16];
  const int P = T * K;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  for (int p = threadIdx.x; p < P + 16; p += blockDim.x) sidx[p] = p < P ? idx[p] : -1;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int e = sidx[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan of cnt (pairs) and of the chunk counts, E <= 4096, 1024 threads x 4
  const int per = (E + blockDim.x - 1) / blockDim.x;
  int lp = 0, lg = 0;
  for (int j = 0; j < per; ++j) {
    const int e = threadIdx.x * per + j;
    if (e < E) {
      lp += cnt[e];
      lg += (cnt[e] + kChunk - 1) / kChunk;
    }
  }
  // scan (lp, lg) packed: both < 2^16 (P <= 2048 pairs, at most P chunks)
  const int v = (lp << 16) | lg;
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
  const int excl = incl - v + wsum[wv];
  int ep = excl >> 16, eg = excl & 0xFFFF;
  for (int j = 0; j < per; ++j) {
    const int e = threadIdx.x * per + j;
    if (e < E) {
      off[e] = ep;
      for (int c = 0; c < cnt[e]; c += kChunk) {
        G.group_expert[eg] = e;
        G.group_off[eg] = ep + c;
        ++eg;
      }
      ep += cnt[e];
    }
  }
  // the last thread holds the totals: the shared expert's chunks follow
  __shared__ int routed;  // routed pairs in all
  if (threadIdx.x == blockDim.x - 1) {
    routed = ep;
    int g = eg;
    for (int c = 0; c < T; c += kChunk) {
      G.group_expert[g] = -1;
      G.group_off[g] = ep + c;
      ++g;
    }
    G.group_off[g] = ep + T;
    G.n_groups[0] = g;
  }
  __syncthreads();
  // stable scatter: rank of pair p among earlier pairs of the same expert (the
  // list is read 16 entries at a time; entries at or past p do not count)
  const int4* s4 = reinterpret_cast<const int4*>(sidx);
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int e = sidx[p];
    if ((unsigned)e >= (unsigned)E) continue;
    int r = 0;
    for (int q0 = 0; q0 < p; q0 += 16) {
      int4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = s4[q0 / 4 + u];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + 4 * u;
        r += (q < p && v[u].x == e) + (q + 1 < p && v[u].y == e) + (q + 2 < p && v[u].z == e) +
             (q + 3 < p && v[u].w == e);
      }
    }
    G.pair_list[off[e] + r] = p;
  }
  // the shared expert's pairs follow every routed pair
  for (int t = threadIdx.x; t < T; t += blockDim.x) G.pair_list[routed + t] = P + t;
}

// fixed-point planes of n-element vectors, one workgroup per vector:
// out + v*pw words (pw = plane_words(n))
template <int BITS>
__global__ __launch_bounds__(kBB) void k_bprep(const float* __restrict__ src, int n, int pw,
                                               uint32_t* __restrict__ out) {
  const int v = blockIdx.x;
  const int C = n / QTraits<BITS>::EPC;
  uint32_t* planes = out + (int64_t)v * pw;
  float* scl = reinterpret_cast<float*>(planes + C * QTraits<BITS>::PW);
  prep_x_coop<BITS>(src + (int64_t)v * n, n, planes, scl, scl + C, threadIdx.x, blockDim.x);
}

struct PoolArgsB {
  const uint8_t* rbase;
  int64_t rstride;
  const uint8_t* sblk;
  int E, H, I, T, K;
  int64_t off_g, off_u, off_d, off_gsb, off_usb, off_dsb;
};

__device__ __forceinline__ int token_of(int p, int T, int K) { return p < T * K ? p / K : p - T * K; }

// ---------------------------------------------------------------------------
// The shared expert's gate/up chunks on the matrix cores.
//
// A chunk of the shared expert holds up to kChunk tokens, so each of its weight
// rows meets 32 input columns: a small GEMM, (rows x K) by (K x tokens), where the
// routed experts' chunks (one or two tokens) stay row dots on the vector ALUs.  The
// routed chunks keep the row dots because a 16-column tile would be 1/16 used and
// the per-group scale then costs as many ALU operations as the dots it replaces.
// The weights are dequantised in fp32, w = fma(code, scale, bias) (one rounding of
// the exact code*scale + bias), and are the A operand of v_mfma_f32_16x16x4_f32;
// the tokens' fp32 inputs are the B operand.  The products are the fp32 products
// of a plain float GEMV; only the order of the fp32 sums differs.
//
// Operands of the 16x16x4 fp32 MFMA: lane l gives A[l%16][l/16] and B[l/16][l%16]
// and gets D[4*(l/16) + v][l%16] in result register v.  The four k slots of a step
// are the four lane groups g = l/16; group g walks chunk 4*kb + g of the row (its
// 16-byte code load), one code per step, so a step covers code n of four chunks at
// once and a lane's B value is its column's input at that same position.
// The waves split the chunks (wave w takes chunks 4*kb + g with kb = w mod 4) and
// add their 16x32 partial tiles through LDS; wave 0 writes the results.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kMfmaCols = 16;  // columns (tokens) per MFMA tile
static_assert(kChunk == 2 * kMfmaCols, "a shared chunk is two column tiles");
static_assert(kBB == 256, "four waves share the chunks of a row");

template <int NM>
constexpr int mfma_red_floats() {  // LDS for the cross-wave sum: waves 1..3, NM x 2 tiles x 4 x 64
  return 3 * NM * 2 * 4 * 64;
}

// NM = 2: gate and up rows, SwiGLU into dst; NM = 1: down rows into dst.
// codes[m] / sb[m]: the matrix's code rows (K*BITS/8 bytes each) and scale|bias
// words (K/64 each).  Output rows [row0, row_end).  Column c < p1 - p0 of the chunk
// is pair pair_list[p0 + c]; its input row is src + in_row * src_ld with in_row its
// token (src_token) or the pair itself, its output row dst + pair * dst_ld.
template <int BITS, int NM>
__device__ __forceinline__ void shared_chunk_mfma(const uint8_t* const (&codes)[NM],
                                                  const uint32_t* const (&sb)[NM], int K,
                                                  int row0, int row_end, const float* src,
                                                  int64_t src_ld, bool src_token, float* dst,
                                                  int64_t dst_ld, const int* pair_list, int p0,
                                                  int p1, int T, int Kt, float* red) {
  constexpr int EPC = QTraits<BITS>::EPC, EPW = QTraits<BITS>::EPW, CPG = QTraits<BITS>::CPG;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  constexpr int PIECES = EPC / 8;  // eight codes (two float4 of input) per piece
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int C = K / EPC, GW = K / kGroup;
  const int64_t rb = (int64_t)K * BITS / 8;
  const float* xs[2];
  int pc[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int c = p0 + tt * kMfmaCols + r;
    pc[tt] = c < p1 ? pair_list[c] : -1;
    xs[tt] = pc[tt] < 0 ? nullptr : src + (int64_t)(src_token ? token_of(pc[tt], T, Kt) : pc[tt]) * src_ld;
  }
  const int n_kb = (C + 3) / 4;  // chunk blocks of the row, four chunks each
  for (int rt0 = row0; rt0 < row_end; rt0 += 16) {
    const int row = rt0 + r;
    const bool rok = row < row_end;
    f32x4_t acc[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[m][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kb = wv; kb < n_kb; kb += 4) {
      const int ch = 4 * kb + g;
      const bool cok = ch < C;
      uint4 q[NM];
      float sc[NM], bi[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (cok && rok) {
          q[m] = ld_stream16(codes[m] + row * rb + 16 * ch);
          const uint32_t s = ld_stream4(sb[m] + (int64_t)row * GW + ch / CPG);
          sc[m] = bf16_lo(s);
          bi[m] = bf16_hi(s);
        } else {  // no row or no chunk: zero weights
          q[m] = make_uint4(0u, 0u, 0u, 0u);
          sc[m] = bi[m] = 0.f;
        }
      }
      // a piece: eight codes and two float4 of each column's input.  The loop stays
      // rolled and loads one piece at a time, so this path needs few registers: it
      // shares the kernel (and its register count) with the routed experts' row dots,
      // whose waves hide its load latency
#pragma unroll 1
      for (int pi = 0; pi < PIECES; ++pi) {
        float b[2][8];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          if (xs[tt] && cok) {
            const float4* xp = reinterpret_cast<const float4*>(xs[tt] + ch * EPC + 8 * pi);
            const float4 u = xp[0], v = xp[1];
            b[tt][0] = u.x, b[tt][1] = u.y, b[tt][2] = u.z, b[tt][3] = u.w;
            b[tt][4] = v.x, b[tt][5] = v.y, b[tt][6] = v.z, b[tt][7] = v.w;
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) b[tt][j] = 0.f;
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            // code j of the piece: the low 8*BITS bits of the current word
            const float a = fmaf((float)((q[m].x >> (BITS * j)) & MASK), sc[m], bi[m]);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
              acc[m][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b[tt][j], acc[m][tt], 0, 0, 0);
          }
        }
        // eight codes consumed: the next word moves in (4-bit), or the word's upper half (2-bit)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if (BITS == 4 || (pi & 1)) q[m] = make_uint4(q[m].y, q[m].z, q[m].w, 0u);
          else q[m].x >>= 16;
        }
      }
    }
    // the four waves' partial tiles: 1..3 through LDS into wave 0
    if (wv > 0) {
      float* o = red + (wv - 1) * (NM * 2 * 4 * 64);
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v) o[((m * 2 + tt) * 4 + v) * 64 + lane] = acc[m][tt][v];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const float* o = red + w * (NM * 2 * 4 * 64);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[m][tt][v] += o[((m * 2 + tt) * 4 + v) * 64 + lane];
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        if (pc[tt] < 0) continue;
        float* d = dst + (int64_t)pc[tt] * dst_ld;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int orow = rt0 + 4 * g + v;
          if (orow < row_end) {
            if constexpr (NM == 2) d[orow] = silu_f(acc[0][tt][v]) * acc[1][tt][v];
            else d[orow] = acc[0][tt][v];
          }
        }
      }
    }
    __syncthreads();
  }
}


// grid (row blocks, group chunks): a wave loads NR gate/up row pairs once and
// applies them to every token of its chunk, taking each token's prepared planes.
template <int BITS, int LG, int CPL, int NR>
__global__ __launch_bounds__(kBB) void k_bgateup(PoolArgsB P, GroupTables G,
                                                 const uint32_t* __restrict__ xp,
                                                 const float* __restrict__ xf,
                                                 float* __restrict__ h, int rows_per_block) {
  constexpr int RPW = 64 / LG;
  __shared__ float red[mfma_red_floats<2>()];
  // groups in reverse: the shared expert's chunks (the most tokens each) start first
  const int ng = G.n_groups[0];
  if ((int)blockIdx.y >= ng) return;
  const int gi = ng - 1 - (int)blockIdx.y;
  const int e = G.group_expert[gi];
  if (e == -1) {  // a shared-expert chunk (uniform per workgroup): matrix cores, fp32 x
    const uint8_t* const cm[2] = {P.sblk + P.off_g, P.sblk + P.off_u};
    const uint32_t* const sm[2] = {reinterpret_cast<const uint32_t*>(P.sblk + P.off_gsb),
                                   reinterpret_cast<const uint32_t*>(P.sblk + P.off_usb)};
    const int row0 = (int)blockIdx.x * rows_per_block;
    shared_chunk_mfma<BITS, 2>(cm, sm, P.H, row0, min(P.I, row0 + rows_per_block), xf, P.H, true, h,
                               P.I, G.pair_list, G.group_off[gi], G.group_off[gi + 1], P.T, P.K, red);
    return;
  }
  const bool eok = e == -1 || (unsigned)e < (unsigned)P.E;
  const uint8_t* blk = e == -1 ? P.sblk : P.rbase + (eok ? (int64_t)e * P.rstride : 0);
  const int C = P.H * BITS / 128, G_ = P.H / kGroup;
  const int pw = C * (QTraits<BITS>::PW + 2);
  const int64_t rb = (int64_t)P.H * BITS / 8;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gl = lane % LG, sub = lane / LG;
  const int r1 = min(P.I, (int)(blockIdx.x + 1) * rows_per_block);
  const int p0 = G.group_off[gi], p1 = G.group_off[gi + 1];
  int jr[NR];
  bool ok[2 * NR];
  const uint8_t* cr[2 * NR];
  const uint32_t* sr[2 * NR];
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    jr[n] = blockIdx.x * rows_per_block + (wv * NR + n) * RPW + sub;
    ok[2 * n] = ok[2 * n + 1] = eok && jr[n] < r1;
    const int j = ok[2 * n] ? jr[n] : 0;
    cr[2 * n] = blk + P.off_g + (int64_t)j * rb;
    cr[2 * n + 1] = blk + P.off_u + (int64_t)j * rb;
    sr[2 * n] = reinterpret_cast<const uint32_t*>(blk + P.off_gsb) + (int64_t)j * G_;
    sr[2 * n + 1] = reinterpret_cast<const uint32_t*>(blk + P.off_usb) + (int64_t)j * G_;
  }
  RowDot<BITS, LG, CPL> rd;
  uint4 q[2 * NR][CPL];
  uint32_t s[2 * NR][CPL];
  rd.template fetch<2 * NR>(cr, sr, ok, C, gl, q, s);
  // the first token's planes go out right behind the rows, before anything waits
  // for them, so that both arrive in one round trip
  auto planes_of = [&](int pi) {
    const int t = token_of(G.pair_list[pi], P.T, P.K);
    const uint32_t* planes = xp + (int64_t)t * pw;
    const float* scl = reinterpret_cast<const float*>(planes + C * QTraits<BITS>::PW);
    rd.load_prepped(planes, scl, scl + C, C, gl);
  };
  if (p0 < p1) planes_of(p0);
  __builtin_amdgcn_sched_barrier(0);
  for (int pi = p0; pi < p1; ++pi) {
    const int p = G.pair_list[pi];
    if (pi != p0) planes_of(pi);
    float pp[2 * NR];
    rd.template dots<2 * NR>(q, s, pp);
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      const float a = group_sum<LG>(pp[2 * n]);
      const float u = group_sum<LG>(pp[2 * n + 1]);
      if (gl == 0 && jr[n] < r1) h[(int64_t)p * P.I + jr[n]] = eok ? silu_f(a) * u : __builtin_nanf("");
    }
  }
}

// (the shared expert's down rows stay row dots: measured on the 64-token batch, the
// matrix-core branch here made the batch slower, 316.9 against 312.3 us, since its
// chunk of 64 rows x 1024 is short and waits on its inputs' load latency)
template <int BITS, int LG, int CPL, int NR>
__global__ __launch_bounds__(kBB) void k_bdown(PoolArgsB P, GroupTables G,
                                               const uint32_t* __restrict__ hp,
                                               float* __restrict__ y, int rows_per_block) {
  constexpr int RPW = 64 / LG;
  // groups in reverse: the shared expert's chunks (the most tokens each) start first
  const int ng = G.n_groups[0];
  if ((int)blockIdx.y >= ng) return;
  const int gi = ng - 1 - (int)blockIdx.y;
  const int e = G.group_expert[gi];
  const bool eok = e == -1 || (unsigned)e < (unsigned)P.E;
  const uint8_t* blk = e == -1 ? P.sblk : P.rbase + (eok ? (int64_t)e * P.rstride : 0);
  const int C = P.I * BITS / 128, G_ = P.I / kGroup;
  const int pw = C * (QTraits<BITS>::PW + 2);
  const int64_t rb = (int64_t)P.I * BITS / 8;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gl = lane % LG, sub = lane / LG;
  const int r1 = min(P.H, (int)(blockIdx.x + 1) * rows_per_block);
  const int p0 = G.group_off[gi], p1 = G.group_off[gi + 1];
  int nr[NR];
  bool ok[NR];
  const uint8_t* cr[NR];
  const uint32_t* sr[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    nr[i] = blockIdx.x * rows_per_block + (wv * NR + i) * RPW + sub;
    ok[i] = eok && nr[i] < r1;
    const int n = ok[i] ? nr[i] : 0;
    cr[i] = blk + P.off_d + (int64_t)n * rb;
    sr[i] = reinterpret_cast<const uint32_t*>(blk + P.off_dsb) + (int64_t)n * G_;
  }
  RowDot<BITS, LG, CPL> rd;
  uint4 q[NR][CPL];
  uint32_t s[NR][CPL];
  rd.template fetch<NR>(cr, sr, ok, C, gl, q, s);
  // the first pair's planes go out right behind the rows (as in k_bgateup)
  auto planes_of = [&](int pi) {
    const uint32_t* planes = hp + (int64_t)G.pair_list[pi] * pw;
    const float* scl = reinterpret_cast<const float*>(planes + C * QTraits<BITS>::PW);
    rd.load_prepped(planes, scl, scl + C, C, gl);
  };
  if (p0 < p1) planes_of(p0);
  __builtin_amdgcn_sched_barrier(0);
  for (int pi = p0; pi < p1; ++pi) {
    const int p = G.pair_list[pi];
    if (pi != p0) planes_of(pi);
    float pp[NR];
    rd.template dots<NR>(q, s, pp);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float v = group_sum<LG>(pp[i]);
      if (gl == 0 && nr[i] < r1) y[(int64_t)p * P.H + nr[i]] = eok ? v : __builtin_nanf("");
    }
  }
}

// grid (T, column slices of kCombineCols): gamma_t = sigmoid(g . x_t) (each slice
// computes it again), then the combine of the slice's columns, four per thread
// (H % 4 == 0)
constexpr int kCombineCols = 1024;
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
  for (int i = 4 * threadIdx.x; i < H; i += 4 * kBB) {
    const float4 xv = *reinterpret_cast<const float4*>(xt + i);
    const uint2 gv = *reinterpret_cast<const uint2*>(g + i);
    d = fmaf(bf16_lo(gv.x), xv.x, d);
    d = fmaf(bf16_hi(gv.x), xv.y, d);
    d = fmaf(bf16_lo(gv.y), xv.z, d);
    d = fmaf(bf16_hi(gv.y), xv.w, d);
  }
  d = group_sum<64>(d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = d;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < kBB / 64; ++i) tot += red[i];
  const float gamma = sigmoid_f(tot);
  const int n = blockIdx.y * kCombineCols + 4 * threadIdx.x;
  if (n >= H) return;
  float4 acc = *reinterpret_cast<const float4*>(residual + (int64_t)t * H + n);
  for (int k = 0; k < K; ++k) {
    const float wk = w[t * K + k];
    const float4 v = *reinterpret_cast<const float4*>(y + ((int64_t)t * K + k) * H + n);
    acc.x = fmaf(wk, v.x, acc.x);
    acc.y = fmaf(wk, v.y, acc.y);
    acc.z = fmaf(wk, v.z, acc.z);
    acc.w = fmaf(wk, v.w, acc.w);
  }
  const float4 v = *reinterpret_cast<const float4*>(y + ((int64_t)T * K + t) * H + n);
  acc.x = fmaf(gamma, v.x, acc.x);
  acc.y = fmaf(gamma, v.y, acc.y);
  acc.z = fmaf(gamma, v.z, acc.z);
  acc.w = fmaf(gamma, v.w, acc.w);
  *reinterpret_cast<float4*>(out + (int64_t)t * H + n) = acc;
}
static_assert(kCombineCols == 4 * kBB, "one float4 of columns per thread");

template <int BITS, int LG, int CPL>
void run_bgateup(const PoolArgsB& P, const GroupTables& G, int gm, const uint32_t* xp,
                 const float* xf, float* h, hipStream_t s) {
  constexpr int RPW = 64 / LG;
  // four gate/up row pairs per wave (measured on the 64-token batch: 324 us against
  // 328 with two pairs, 389 with eight, 402 with one)
  constexpr int NR = 4;
  const int rpb = (kBB / 64) * NR * RPW;
  hipLaunchKernelGGL((k_bgateup<BITS, LG, CPL, NR>), dim3(ceil_div(P.I, rpb), gm), dim3(kBB), 0, s,
                     P, G, xp, xf, h, rpb);
}

template <int BITS, int LG, int CPL>
void run_bdown(const PoolArgsB& P, const GroupTables& G, int gm, const uint32_t* hp, float* y,
               hipStream_t s) {
  constexpr int RPW = 64 / LG;
  constexpr int NR = CPL >= 4 ? 4 : 8;
  const int rpb = (kBB / 64) * NR * RPW;
  hipLaunchKernelGGL((k_bdown<BITS, LG, CPL, NR>), dim3(ceil_div(P.H, rpb), gm), dim3(kBB), 0, s, P,
                     G, hp, y, rpb);
}

template <int BITS>
void dispatch_bgateup(const PoolArgsB& P, const GroupTables& G, int gm, const uint32_t* xp,
                      const float* xf, float* h, hipStream_t s) {
  const int C = P.H * BITS / 128;
  if (C <= 1) return run_bgateup<BITS, 1, 1>(P, G, gm, xp, xf, h, s);
  if (C <= 2) return run_bgateup<BITS, 2, 1>(P, G, gm, xp, xf, h, s);
  if (C <= 4) return run_bgateup<BITS, 4, 1>(P, G, gm, xp, xf, h, s);
  if (C <= 8) return run_bgateup<BITS, 8, 1>(P, G, gm, xp, xf, h, s);
  if (C <= 16) return run_bgateup<BITS, 16, 1>(P, G, gm, xp, xf, h, s);
  if (C <= 32) return run_bgateup<BITS, 32, 1>(P, G, gm, xp, xf, h, s);
  if (C <= 64) return run_bgateup<BITS, 64, 1>(P, G, gm, xp, xf, h, s);
  if (C <= 128) return run_bgateup<BITS, 64, 2>(P, G, gm, xp, xf, h, s);
  return run_bgateup<BITS, 64, 4>(P, G, gm, xp, xf, h, s);
}

template <int BITS>
void dispatch_bdown(const PoolArgsB& P, const GroupTables& G, int gm, const uint32_t* hp, float* y,
                    hipStream_t s) {
  const int C = P.I * BITS / 128;
  if (C <= 1) return run_bdown<BITS, 1, 1>(P, G, gm, hp, y, s);
  if (C <= 2) return run_bdown<BITS, 2, 1>(P, G, gm, hp, y, s);
  if (C <= 4) return run_bdown<BITS, 4, 1>(P, G, gm, hp, y, s);
  if (C <= 8) return run_bdown<BITS, 8, 1>(P, G, gm, hp, y, s);
  if (C <= 16) return run_bdown<BITS, 16, 1>(P, G, gm, hp, y, s);
  if (C <= 32) return run_bdown<BITS, 32, 1>(P, G, gm, hp, y, s);
  if (C <= 64) return run_bdown<BITS, 64, 1>(P, G, gm, hp, y, s);
  if (C <= 128) return run_bdown<BITS, 64, 2>(P, G, gm, hp, y, s);
  return run_bdown<BITS, 64, 4>(P, G, gm, hp, y, s);
}

template <int BITS>
void run_prep(const float* src, int count, int n, uint32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_bprep<BITS>, dim3(count), dim3(kBB), 0, s, src, n, plane_words<BITS>(n), out);
}

}  // namespace

size_t batched_workspace_bytes(const qmoe_layer& L, int T) {
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  return (size_t)batch_ws(E, K, H, I, T, L.routed.bits).total;
}

hipError_t launch_layer_batched(const qmoe_layer& L, const float* x, const float* residual,
                                float* out, int T, int32_t* idx, float* w, void* ws,
                                hipStream_t s) {
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  const int bits = L.routed.bits;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const BatchWs b = batch_ws(E, K, H, I, T, bits);
  float* logits = reinterpret_cast<float*>(wsb + b.logits);
  uint32_t* xp = reinterpret_cast<uint32_t*>(wsb + b.xp);
  float* h = reinterpret_cast<float*>(wsb + b.h);
  uint32_t* hp = reinterpret_cast<uint32_t*>(wsb + b.hp);
  float* y = reinterpret_cast<float*>(wsb + b.y);
  const GroupTables G = group_tables(wsb, b, T, K);
  bool prepped = false;  // the router can build the x planes on the way
  hipError_t err = launch_router_topk(L.router, x, T, H, E, K, logits, idx, w, s, bits, xp,
                                      bits == 4 ? plane_words<4>(H) : plane_words<2>(H), &prepped);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, s, idx, T, K, E, G);
  if (!prepped) {
    if (bits == 4) run_prep<4>(x, T, H, xp, s);
    else run_prep<2>(x, T, H, xp, s);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const qmoe_expert_offsets o = expert_offsets(H, I, bits);
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
  const int gm = max_groups(T, K);
  const int npairs = T * K + T;
  if (bits == 4) {
    dispatch_bgateup<4>(P, G, gm, xp, x, h, s);
    run_prep<4>(h, npairs, I, hp, s);
    dispatch_bdown<4>(P, G, gm, hp, y, s);
  } else {
    dispatch_bgateup<2>(P, G, gm, xp, x, h, s);
    run_prep<2>(h, npairs, I, hp, s);
    dispatch_bdown<2>(P, G, gm, hp, y, s);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_bcombine, dim3(T, ceil_div(H, kCombineCols)), dim3(kBB), 0, s, y, w,
                     L.shared_gate, x, residual, out, T, K, H);
  return hipGetLastError();
}

}  // namespace qmoe
