// One MoE layer at batch 1 in a single kernel launch.
//
// The page "flash-moe 소개" (discuss.pytorch.kr), section "레이어당 파이프라인 상세
// 구조", runs this path as: router GEMV inside a second command buffer, a device
// to host copy, softmax + top-K on the CPU, then a third command buffer with the
// expert forward, combine and norm.  Here it is one launch with no host round
// trip: every workgroup (all co-resident, one per CU) computes the routing itself
// from the logits, and the experts are addressed by index in the resident pool.
//
// NB = H/16 workgroups of 8 waves; workgroup b owns output rows [16b, 16b+16).
// "rank" = wave * NB + workgroup numbers the waves so that consecutive ranks sit
// in different workgroups.  Schedule of a workgroup:
//   1. issue loads: x (staged in LDS; RMS-normalised here when the layer is given
//      a norm weight), the shared-gate vector and its router rows (4 waves per
//      row);
//   2. router dots -> logits (tagged stores); then issue the loads of the wave's
//      shared down rows (into registers);
//   3. x as fixed-point planes in LDS (once per workgroup);
//   4. shared gate/up + SwiGLU -> hs: its row pairs (one per rank below I/RPWH)
//      are loaded once the logits are in (step 5), its dots run once the routed
//      rows of step 6 are on their way;
//   5. top-K: every thread polls its logits; from the 8 wave maxima a lower bound
//      L of the K-th largest logit; the keys >= L go to an LDS list; one wave
//      ranks them (larger value, then lower index) and passes the picks on;
//      renormalised softmax of the K selected logits;
//   6. issue loads: two routed gate/up row pairs per wave, then (into registers)
//      the wave's routed down rows of this workgroup's output rows;
//   7. routed gate/up dots + SwiGLU -> hr (tagged); one tagged flag;
//   8. hs read straight into its planes (no LDS copy of the values); the shared
//      down rows; the dot of gamma = sigmoid(g . x);
//   9. hr read into its planes the same way; the routed down rows; out = residual +
//      sum_k w_k y_k + gamma y_shared.
// Values that cross workgroups (logits, hs, hr) are 64-bit words (epoch << 32 |
// value bits) written with agent-scope atomic stores (write-through to the
// device coherence point), so they never need resetting.  The logits are polled
// word by word.  The h values are read by every workgroup, once its own dots are
// done, with ordinary cacheable loads (one fetch per XCD's L2); a word with an
// old epoch (a stale cached line, or a store not yet visible) is re-read
// coherently until it carries the current one, and the h buffers rotate over 4
// slots so that stale lines are rare.  (Waiting first for a tagged completion
// flag of every workgroup, which each still writes, measured slower; one shared
// counter instead is far slower still: device-scope atomics on one word
// serialise at ~25 ns each.)  The epoch lives in the workspace: every wave of
// every workgroup reads it before the workgroup's first barrier, every h word is
// tagged after that barrier, and workgroup 0 advances the epoch once it has read
// every h word.  Every wait is bounded; on time-out a status bit is set and the
// output is undefined (it never hangs).
#include <type_traits>

#include "qmoe_device.h"
#include "qmoe_handoff.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

// Phase timestamps (a build with QMOE_PHASE_PROBE defined only): thread 0 of every
// workgroup records the real-time counter (100 MHz) at the phase boundaries of
// the single-layer kernel and stores them at the end, per call number modulo 64,
// so the recording adds no memory traffic while the layer runs.  The product
// build compiles none of it.
#ifdef QMOE_PHASE_PROBE
constexpr int kProbeCalls = 64, kProbeWgs = 512, kProbePhases = 16;
__device__ uint32_t g_phase[kProbeCalls * kProbeWgs * kProbePhases];
#define QMOE_PT_DECL uint32_t pt_[kProbePhases] = {0}
#define QMOE_PT(k)                                                        \
  do {                                                                    \
    if (!STACK && threadIdx.x == 0) pt_[k] = (uint32_t)__builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define QMOE_PT_STORE()                                                                   \
  do {                                                                                    \
    if (!STACK && threadIdx.x == 0 && blockIdx.x < kProbeWgs) {                          \
      for (int k_ = 0; k_ < kProbePhases; ++k_)                                           \
        g_phase[((s_tag % kProbeCalls) * kProbeWgs + blockIdx.x) * kProbePhases + k_] = pt_[k_]; \
    }                                                                                     \
  } while (0)
#else
#define QMOE_PT_DECL
#define QMOE_PT(k)
#define QMOE_PT_STORE()
#endif

constexpr int kLB = 512;         // threads per workgroup
constexpr int kLW = kLB / 64;    // waves per workgroup
constexpr int kRB = 16;          // output rows per workgroup
constexpr int kFusedMaxK = 4;
constexpr int kFusedMaxE = 2048;
static_assert(kFusedMaxE % 64 == 0, "the ranking wave reads the candidate list 64 at a time");
struct LayerArgs {
  const uint8_t* rbase;  // routed pool
  int64_t rstride;
  const uint8_t* sblk;   // shared expert block
  int64_t off_g, off_u, off_d, off_gsb, off_usb, off_dsb;
  const uint16_t* router;
  const uint16_t* g;
  const float* x;         // the layer input, or (norm_w set) the stream h it is normalised from
  const float* norm_w;    // RMSNorm weight [H], or null
  float eps;
  const float* residual;
  float* out;
  int32_t* idx_out;
  float* w_out;
  uint32_t* ctrl;
  uint64_t* logits;  // [E/2][kLine]: logit e is word e % 2 of line e / 2
  uint64_t* flags;   // [NB][kLine]: workgroup b has issued all its h stores
  uint64_t* hs;      // [kSlotsH][I], word-transposed (see hpos in k_layer)
  uint64_t* hr;      // [kSlotsH][kFusedMaxK * I], word-transposed
  int E, K;
};

// A decoder stack in one launch: the workgroups stay resident from layer to layer.
// Per layer, the weights that differ; the shapes, K and the block offsets are the
// same for every layer.
struct StackLayer {
  const uint8_t* rbase;
  const uint8_t* sblk;
  const uint16_t* router;
  const uint16_t* g;
  const float* norm_w;
  int64_t rstride;
};
constexpr int kStackMax = 32;  // layers per launch (the table travels as kernel arguments)
static_assert(kRB == kLine, "a workgroup's output rows fill one line of the stack's hand-over buffer");

struct StackArgs {
  LayerArgs A;      // layer 0's pointers; x/residual: the stack input, out: its output
  uint64_t* xbuf;   // [kStackMax][NB][kLine]: layer l's output, one line per workgroup
  float* h_all;     // [nl][H] every layer's output, or null
  int nl;
  StackLayer st[kStackMax];
};

// the pointers of one layer as the kernel body uses them
struct LayerPtrs {
  const uint8_t* rbase;
  int64_t rstride;
  const uint8_t* sblk;
  const uint16_t* router;
  const uint16_t* g;
  const float* norm_w;
  uint64_t *logits, *flags, *hs, *hr;
  int32_t* idx_out;
  float* w_out;
};

__device__ __forceinline__ LayerPtrs ptrs_of(const LayerArgs& A) {
  return {A.rbase, A.rstride, A.sblk, A.router, A.g, A.norm_w, A.logits, A.flags, A.hs, A.hr,
          A.idx_out, A.w_out};
}


// The 2-bit planes of half a code word: thread t takes word t >> 1 and half
// h = t & 1, i.e. the 8 values that meet the codes of that half (elements 2k + h,
// k < 8); the planes and scale are those prep_x_word<2> builds for the whole word.
// A chunk (4 words x 2 halves) is 8 consecutive lanes, aligned to 8, and all 8
// must call this together.  Twice the threads of prep_x_word<2>, half the work
// each.
template <int STRIDE>
__device__ __forceinline__ void prep_x_half2(const float (&v)[8], bool valid, int t, uint32_t* planes,
                                             float* scl, float* xsum) {
  float m = fmaxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))),
                  fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7]))));
  float s = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  // the chunk's 8 lanes: two DPP quads, joined by the half-row mirror
  m = fmaxf(m, dpp_f<kDppXor1>(m));
  m = fmaxf(m, dpp_f<kDppXor2>(m));
  m = fmaxf(m, dpp_f<kDppHalfMirror>(m));
  s += dpp_f<kDppXor1>(s);
  s += dpp_f<kDppXor2>(s);
  s += dpp_f<kDppHalfMirror>(s);
  float f, scale;
  chunk_exp(m, f, scale);
  if (valid) {
    uint32_t u[8], p[6];
#pragma unroll
    for (int k = 0; k < 8; ++k) u[k] = to_u24(v[k], f);
    nibble_planes8(u, p);
    const int w = t >> 1, h = t & 1, c = w >> 2, i = w & 3;
#pragma unroll
    for (int d = 0; d < 6; ++d) planes[c * STRIDE + i * 12 + h * 6 + d] = p[d];
    if (i == 0 && h == 0) {
      scl[c] = scale * QTraits<2>::FACTOR;
      xsum[c] = s;
    }
  }
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

template <int BITS, int H, int I, bool STACK, class Args>
__device__ __forceinline__ void layer_body(const LayerArgs& A, const Args& P) {
  QMOE_PT_DECL;
  // ---- compile-time geometry
  constexpr int CH = H * BITS / 128;            // 16-byte chunks per gate/up row
  constexpr int LGH = CH >= 64 ? 64 : CH;       // lanes per gate/up row
  constexpr int CPLH = CH / LGH;                // chunks per lane
  constexpr int RPWH = 64 / LGH;                // gate/up rows per wave pass
  static_assert(LGH * CPLH == CH, "every chunk of a gate/up row has a lane");
  constexpr int GH = H / kGroup;
  constexpr int64_t RBH = (int64_t)H * BITS / 8;
  constexpr int CI = I * BITS / 128;            // 16-byte chunks per down row
  constexpr int LGI = CI;                       // one chunk per lane
  static_assert(CI <= 64, "down rows must fit one chunk per lane");
  constexpr int RPWI = 64 / LGI;                // down rows per wave pass
  constexpr int GI = I / kGroup;
  constexpr int64_t RBI = (int64_t)I * BITS / 8;
  constexpr int DITEMS = (kRB + RPWI - 1) / RPWI;  // down items per expert per workgroup
  static_assert(DITEMS <= kLW, "one shared down item per wave");
  static_assert(kRB % RPWI == 0, "a down pass never runs past the workgroup's rows");
  constexpr int MAXR = (kFusedMaxK * DITEMS + kLW - 1) / kLW;  // routed down items per wave
  constexpr int NSP = I / RPWH;                 // shared gate/up items
  constexpr int CRQ = H / 32;                   // 16-byte router chunks per quarter row
  constexpr int CPLR = (CRQ + 63) / 64;
  constexpr int PW = QTraits<BITS>::PW;
  // plane words per chunk as kept in LDS: 16 bytes of padding per chunk, so that the
  // 16-byte reads of consecutive lanes (one chunk each) fall in different banks
  constexpr int PWL = PW + 4;
  constexpr int PER_L = (kFusedMaxE + kLB - 1) / kLB;

  const int NB = gridDim.x, wg = blockIdx.x;
  int tx = threadIdx.x;
  // wave-uniform values go through readfirstlane so that their arithmetic (item,
  // expert and row selection, load addresses) runs on the scalar unit
  const int wv = __builtin_amdgcn_readfirstlane((int)(tx >> 6));
  int lane = tx & 63;
  const int rank = wv * NB + wg;
  const int W = NB * kLW;
  const int E = A.E, K = A.K;
  int glh = lane % LGH, subh = lane / LGH;
  int gli = lane % LGI, subi = lane / LGI;
  const int row0 = wg * kRB;

  __shared__ __align__(16) float s_x[H];          // the layer input x
  __shared__ __align__(16) uint32_t s_xp[CH * PWL];
  __shared__ float s_xsc[CH], s_xsum[CH];
  __shared__ __align__(16) uint32_t s_hp[(kFusedMaxK + 1) * CI * PWL];  // their planes
  __shared__ float s_hsc[(kFusedMaxK + 1) * CI], s_hsum[(kFusedMaxK + 1) * CI];
  __shared__ float s_y[kFusedMaxK + 1][kRB];
  __shared__ float s_part[kLW];
  __shared__ uint32_t s_tag;
  __shared__ float s_rv[kLW];
  __shared__ uint32_t s_wmax[kLW];             // top-K: largest key of each wave
  __shared__ uint32_t s_ncand;                 // number of candidates
  __shared__ uint64_t s_cand[kFusedMaxE];      // candidates: key << 32 | ~expert
  __shared__ uint64_t s_pick[kFusedMaxK];      // the picks, in rank order
  bool ok_all = true;
  LayerPtrs Lp = ptrs_of(A);  // layer 0 (a stack's first layer is described by A too)
  // a stack's layer table, copied to LDS once: read per layer from the kernel
  // arguments, the pointers would come through scalar loads that miss, and every
  // LDS wait after such a load waits for it too
  __shared__ uint64_t s_tab[STACK ? kStackMax * 6 : 1];
  uint64_t tab_v = 0;
  if constexpr (STACK) {
    static_assert(sizeof(StackLayer) == 6 * sizeof(uint64_t), "six words per layer");
    tab_v = reinterpret_cast<const uint64_t*>(P.st)[min((int)threadIdx.x, P.nl * 6 - 1)];
  }
  // word f of layer l's table entry, as a wave-uniform value
  auto tab = [&](int l, int f) -> uint64_t {
    const uint64_t v = s_tab[l * 6 + f];
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  };

  // ---- 1. loads: the epoch, x (once per workgroup, into LDS below), the
  //         shared-gate vector and the norm weight, then the router rows.  Every
  //         load of the kernel's straight-line parts is unconditional (clamped
  //         addresses; a lane with nothing to load reads a valid word it ignores):
  //         vector memory completes in issue order, and a straight run of loads
  //         lets each use below wait for its own data only (a conditional load
  //         makes the compiler wait for everything).
  QMOE_PT(0);
  const uint32_t epoch = __hip_atomic_load(A.ctrl + CTRL_EPOCH, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int xi = min((int)tx, H / 8 - 1);
  float gx[8], nw[8];
  uint4 gq;  // shared-gate vector chunk for gamma (step 8)
  {
    const float4 f0 = reinterpret_cast<const float4*>(A.x + 8 * xi)[0];
    const float4 f1 = reinterpret_cast<const float4*>(A.x + 8 * xi)[1];
    gx[0] = f0.x; gx[1] = f0.y; gx[2] = f0.z; gx[3] = f0.w;
    gx[4] = f1.x; gx[5] = f1.y; gx[6] = f1.z; gx[7] = f1.w;
    gq = reinterpret_cast<const uint4*>(Lp.g)[xi];
    const float* nwp = Lp.norm_w ? Lp.norm_w : A.x;  // no norm: a load that is ignored
    const float4 w0 = reinterpret_cast<const float4*>(nwp + 8 * xi)[0];
    const float4 w1 = reinterpret_cast<const float4*>(nwp + 8 * xi)[1];
    nw[0] = w0.x; nw[1] = w0.y; nw[2] = w0.z; nw[3] = w0.w;
    nw[4] = w1.x; nw[5] = w1.y; nw[6] = w1.z; nw[7] = w1.w;
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the rest
  const int quarter = wv & 3;
  uint4 rq[CPLR];
  // a row past E reads row E - 1 (not stored)
  auto router_fetch = [&](const uint16_t* rt, int row, uint4(&dst)[CPLR]) {
    const int rc = min(row, E - 1);
#pragma unroll
    for (int i = 0; i < CPLR; ++i) {
      const int cq = min(lane + 64 * i, CRQ - 1);
      dst[i] = ld_stream16(rt + (int64_t)rc * H + 8 * (quarter * CRQ + cq));
    }
  };
  router_fetch(Lp.router, wg * 2 + (wv >> 2), rq);

  const float resid_v = A.residual[row0 + min((int)tx, kRB - 1)];
  float resid = (int)tx < kRB ? resid_v : 0.f;
  // the shared expert's loads, into registers: one gate/up row pair per rank below
  // I/RPWH (another wave reads rows of item 0 that it ignores) ...
  const bool has_sp = rank < NSP;
  int jsp = rank * RPWH + subh;
  int nl_s = wv * RPWI + subi;
  RowDot<BITS, LGH, CPLH> dH;
  auto shared_fetch = [&](const uint8_t* sblk, uint4(&qd)[2][CPLH], uint32_t(&sd)[2][CPLH]) {
    const int j = has_sp ? jsp : subh;  // no item: rows of item 0, ignored
    const uint8_t* cr[2] = {sblk + A.off_g + j * RBH, sblk + A.off_u + j * RBH};
    const uint32_t* sr[2] = {reinterpret_cast<const uint32_t*>(sblk + A.off_gsb) + j * GH,
                             reinterpret_cast<const uint32_t*>(sblk + A.off_usb) + j * GH};
    dH.template fetch_always<2>(cr, sr, glh, qd, sd);
  };
  // ... and the wave's shared down item (waves below DITEMS; another wave reads
  // rows it ignores)
  auto shared_down_fetch = [&](const uint8_t* sblk, uint4& d0, uint32_t& s0) {
    // a wave-uniform row base plus a 32-bit lane offset
    const int rb = wv < DITEMS ? row0 + wv * RPWI : row0;
    d0 = ld_stream16(sblk + A.off_d + (int64_t)rb * RBI + (uint32_t)(subi * RBI + 16 * gli));
    s0 = ld_stream4(reinterpret_cast<const uint32_t*>(sblk + A.off_dsb) + (int64_t)rb * GI +
                    (uint32_t)(subi * GI + gli / QTraits<BITS>::CPG));
  };
  uint4 qsp[2][CPLH];
  uint32_t ssp[2][CPLH];
  uint4 dq[1 + MAXR];
  uint32_t dsc[1 + MAXR];
  // (the down item is issued in step 2, the gate/up pair in step 5)
  // the next layer's loads (stack only)
  uint4 gqN, rqN[CPLR];
  float nwN[8];
  if constexpr (STACK)
    if ((int)threadIdx.x < P.nl * 6) s_tab[threadIdx.x] = tab_v;  // seen after the next barrier

  for (int l = 0;;) {
  if constexpr (STACK)  // per-layer copies: addresses derived from them are not kept live across layers
    asm volatile("" : "+v"(tx), "+v"(lane), "+v"(glh), "+v"(subh), "+v"(gli), "+v"(subi), "+v"(xi), "+v"(jsp), "+v"(nl_s));
  if (Lp.norm_w) {
    // RMSNorm of the input stream, computed by every workgroup: x = h / sqrt(mean(h^2) + eps) * w
    float ss = 0.f;
    if ((int)tx < H / 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(gx[i], gx[i], ss);
    }
    ss = group_sum<64>(ss);
    if (lane == 0) s_part[wv] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kLW; ++w) tot += s_part[w];
    const float r = 1.0f / sqrtf(tot / (float)H + A.eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) gx[i] = gx[i] * r * nw[i];
    __syncthreads();  // s_part is reused by the router dots
  }
  if ((int)tx < H / 8) {
    reinterpret_cast<float4*>(s_x)[2 * tx] = make_float4(gx[0], gx[1], gx[2], gx[3]);
    reinterpret_cast<float4*>(s_x)[2 * tx + 1] = make_float4(gx[4], gx[5], gx[6], gx[7]);
  }
  __syncthreads();
  QMOE_PT(1);

  // ---- 2. router dots -> logits (every wave has read the epoch itself)
  // tag 0 is what a zero-filled workspace holds: skipped when the counter wraps
  uint32_t tag0 = (uint32_t)__builtin_amdgcn_readfirstlane(epoch) + 1u;
  if constexpr (STACK) {
    // layer l of a stack is call number epoch + 1 + l (the layers share the
    // buffers); a run of numbers that would reach 0 restarts at 1
    const uint32_t nl = (uint32_t)P.nl;
    tag0 = (tag0 == 0u || tag0 + nl - 1u < tag0) ? 1u + (uint32_t)l : tag0 + (uint32_t)l;
  } else {
    tag0 = tag0 ? tag0 : 1u;
  }
  auto router_rows = [&](int r0) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPLR; ++i) {
      const int cq = lane + 64 * i;
      if (cq < CRQ) {
        const float4* xp = reinterpret_cast<const float4*>(s_x) + 2 * (quarter * CRQ + cq);
        const float4 f0 = xp[0], f1 = xp[1];
        const float xr8[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
        acc += bf16_chunk_dot(rq[i], xr8);
      }
    }
    acc = group_sum_last<64>(acc);
    if (lane == 63) s_part[wv] = acc;
    __syncthreads();
    if (tx < 8) {  // rows r0, r0 + 1 and padding: one whole 64-byte store
      const bool real = tx < 2 && r0 + (int)tx < E;
      const float* pp = s_part + 4 * (tx & 1);
      const float v = real ? (pp[0] + pp[1]) + (pp[2] + pp[3]) : 0.f;
      tag_put(Lp.logits + (r0 >> 1) * kLine + tx, v, tag0);
    }
    __syncthreads();
  };
  // the first pair of rows was fetched in step 1 (outside the loop, so that the
  // dots wait for those rows only, not for every load issued after them)
  if (wg * 2 < E) router_rows(wg * 2);
  for (int r0 = wg * 2 + NB * 2; r0 < E; r0 += NB * 2) {
    router_fetch(Lp.router, r0 + (wv >> 2), rq);
    router_rows(r0);
  }
  QMOE_PT(2);
  // the shared down item goes out now, behind the logit stores: 2 MB that would
  // otherwise join the stream after the top-K, small enough not to hold up the
  // logits' visibility (measured against issuing it in step 5: 15.27 against 15.72
  // us per layer, 2-bit 14.74 against 14.92; in step 1, before the router dots or
  // after the first logit poll it gains less, and the shared gate rows issued here
  // as well lose part of the gain)
  shared_down_fetch(Lp.sblk, dq[0], dsc[0]);

  // ---- 3. x planes in LDS; the epoch goes to every thread through the barrier
  if constexpr (BITS == 2) {
    // half a code word per thread (8 values, elements 2k + h of word t >> 1)
    for (int t0 = 0; t0 < H / 8; t0 += kLB) {
      if (t0 + (int)wv * 64 >= H / 8) break;
      const int t = t0 + (int)tx;
      const bool valid = t < H / 8;
      const float4* xp = reinterpret_cast<const float4*>(s_x + 16 * (valid ? t >> 1 : 0));
      const float4 a = xp[0], b = xp[1], c = xp[2], d = xp[3];
      const bool odd = (t & 1) != 0;
      const float v[8] = {odd ? a.y : a.x, odd ? a.w : a.z, odd ? b.y : b.x, odd ? b.w : b.z,
                          odd ? c.y : c.x, odd ? c.w : c.z, odd ? d.y : d.x, odd ? d.w : d.z};
      float vz[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) vz[k] = valid ? v[k] : 0.f;
      prep_x_half2<PWL>(vz, valid, t, s_xp, s_xsc, s_xsum);
    }
  } else {
    prep_x_coop<BITS, PWL>(s_x, H, s_xp, s_xsc, s_xsum, tx, kLB);
  }
  if (tx == 0) {
    s_tag = tag0;
    s_ncand = 0;
  }
  if (tx < kFusedMaxK) s_pick[tx] = 0;  // no pick: key 0, expert ~0 = -1
  __syncthreads();
  QMOE_PT(3);
  const uint32_t tag = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_tag);

  uint64_t* hs = Lp.hs + (size_t)(tag % kSlotsH) * I;
  uint64_t* hr = Lp.hr + (size_t)(tag % kSlotsH) * kFusedMaxK * I;
  // h is kept word-transposed: value e of code-word-sized group w of a vector
  // lives at e * (words in the vector) + w, so that the thread that builds word
  // w's planes reads its values with loads that are contiguous across the wave.
  constexpr int kHsW = I / QTraits<BITS>::EPW, kHrW = kFusedMaxK * I / QTraits<BITS>::EPW;
  auto hpos = [](int j, int words) { return (j % QTraits<BITS>::EPW) * words + j / QTraits<BITS>::EPW; };
  // the first poll of logits 0..kLB-1 (step 5) goes out now, unconditionally (a
  // lane past E reads logit E - 1), so that its round trip overlaps the loading of
  // the x planes; logits from kLB on are first read by the poll loop of step 5
  uint64_t lraw[PER_L];
  uint32_t pending = 0;
  {
    const int ec = min((int)tx, E - 1);
    lraw[0] = tag_get(Lp.logits + (ec >> 1) * kLine + (ec & 1));
  }
#pragma unroll
  for (int j = 0; j < PER_L; ++j) {
    if (j) lraw[j] = 0;  // tag 0 is never current: polled in the loop
    if ((int)tx + j * kLB < E) pending |= 1u << j;
  }
  dH.template load_prepped<PWL>(s_xp, s_xsc, s_xsum, CH, glh);
  float hs_val = 0.f;
  QMOE_PT(4);
  // ---- 5. top-K.  Order: larger logit, then lower index; the keys are the
  //         logits' bits mapped to an order-preserving u32 (-0 counts as +0).
  //         (a) every thread polls its logits; the largest key of each wave;
  //         (b) L = the K-th largest of these 8 is at most the K-th largest key
  //             overall (K waves hold a key >= L), so the picks are among the keys
  //             >= L; those candidates -- a handful for spread-out logits, at most
  //             E -- are appended to an LDS list;
  //         (c) the last wave ranks them: each candidate counts those ahead of it
  //             (larger key, or equal key and lower index: stored as key << 32 |
  //             ~index, that is plain u64 order) and the one of rank r < K writes
  //             itself to pick slot r; the picks go to the other waves through LDS.
  {
    uint32_t key[PER_L];
#pragma unroll
    for (int j = 0; j < PER_L; ++j) key[j] = 0;
    for (uint32_t spins = 0;; ++spins) {
#pragma unroll
      for (int j = 0; j < PER_L; ++j)
        if (((pending >> j) & 1u) && (uint32_t)(lraw[j] >> 32) == tag) {
          key[j] = order_key((uint32_t)lraw[j]);
          pending &= ~(1u << j);
        }
      if (!pending) break;
      if (spins > kSpinLimit) {
        ok_all = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int j = 0; j < PER_L; ++j)
        if ((pending >> j) & 1u) {
          const int e = tx + j * kLB;
          lraw[j] = tag_get(Lp.logits + (e >> 1) * kLine + (e & 1));
        }
    }
    uint32_t lmax = 0;
#pragma unroll
    for (int j = 0; j < PER_L; ++j) lmax = max(lmax, key[j]);
    const uint32_t wmax = wave_max_u32(lmax);
    if (lane == 0) s_wmax[wv] = wmax;
    __syncthreads();
  QMOE_PT(5);
    // the shared expert's gate/up rows go out only now, once this workgroup's
    // logits have all arrived: issued with the router rows or right after them,
    // they flood the memory system while the logit stores of the slowest
    // workgroups are still becoming visible, and the poll above ends later
    // (measured); here they travel during the ranking, ahead of the routed rows
    shared_fetch(Lp.sblk, qsp, ssp);
    uint32_t L;
    {
      const uint32_t mi = lane < kLW ? s_wmax[lane] : 0u;
      int n = 0;  // how many wave maxima are >= mine
#pragma unroll
      for (int w = 0; w < kLW; ++w) n += (uint32_t)__builtin_amdgcn_readlane((int)mi, w) >= mi ? 1 : 0;
      L = wave_max_u32(lane < kLW && n >= K ? mi : 0u);
    }
#pragma unroll
    for (int j = 0; j < PER_L; ++j)
      if (key[j] != 0 && key[j] >= L) {
        const uint32_t slot = atomicAdd(&s_ncand, 1u);  // key, then the inverted index:
        s_cand[slot] = ((uint64_t)key[j] << 32) | ~(uint32_t)(tx + j * kLB);  // u64 order
      }
    __syncthreads();
  }
  if (wv == kLW - 1) {
    // one LDS round trip for the count, this lane's candidate and the first eight
    // (entries at or past nc are ignored); a candidate of rank r < K is pick r
    const int nc = (int)s_ncand;
    uint64_t o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = s_cand[u];
    const uint64_t cv0 = s_cand[lane];
    for (int c0 = 0; c0 < nc; c0 += 64) {
      const uint64_t cv = c0 == 0 ? cv0 : s_cand[c0 + lane];
      int rk = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) rk += (u < nc && o[u] > cv) ? 1 : 0;
      for (int c = 8; c < nc; c += 8) {  // more than eight candidates: rare
        uint64_t o2[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o2[u] = s_cand[c + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) rk += (c + u < nc && o2[u] > cv) ? 1 : 0;
      }
      if (c0 + lane < nc && rk < K) s_pick[rk] = cv;
    }
  }
  __syncthreads();
  QMOE_PT(6);
  int eidx[kFusedMaxK];
  float elog[kFusedMaxK];
#pragma unroll
  for (int r = 0; r < kFusedMaxK; ++r) {
    const uint64_t v = r < K ? s_pick[r] : 0ull;
    eidx[r] = __builtin_amdgcn_readfirstlane((int)~(uint32_t)v);
    elog[r] = key_value((uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32)));
  }
  // renormalised softmax over the K picks (uniform values)
  float wsel[kFusedMaxK];
  {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kFusedMaxK; ++k) {
      wsel[k] = k < K ? __expf(elog[k] - elog[0]) : 0.f;
      sum += wsel[k];
    }
    const float inv = 1.0f / sum;
#pragma unroll
    for (int k = 0; k < kFusedMaxK; ++k) wsel[k] *= inv;
  }
  if (wg == 0 && tx == 0) {
#pragma unroll
    for (int k = 0; k < kFusedMaxK; ++k)
      if (k < K) {
        __hip_atomic_store(Lp.idx_out + k, eidx[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(Lp.w_out + k, wsel[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  }

  // ---- 6. loads: two routed gate/up row pairs per wave
  const int n_rp = K * NSP;
  int it = rank;
  uint4 q[4][CPLH];
  uint32_t sq[4][CPLH];
  int kk[2], jj[2];
  bool eok[2];
  auto fetch_pairs = [&](int it0) {
    const uint8_t* cr[4];
    const uint32_t* sr[4];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int item = it0 + v * W;
      const bool valid = item < n_rp;
      kk[v] = valid ? item / NSP : 0;
      jj[v] = valid ? (item % NSP) * RPWH + subh : 0;
      int e = -1;
#pragma unroll
      for (int k = 0; k < kFusedMaxK; ++k)
        if (valid && kk[v] == k) e = eidx[k];
      eok[v] = (unsigned)e < (unsigned)E;
      const uint8_t* blk = Lp.rbase + (eok[v] ? (int64_t)e * Lp.rstride : 0);
      cr[2 * v] = blk + A.off_g + jj[v] * RBH;
      cr[2 * v + 1] = blk + A.off_u + jj[v] * RBH;
      sr[2 * v] = reinterpret_cast<const uint32_t*>(blk + A.off_gsb) + jj[v] * GH;
      sr[2 * v + 1] = reinterpret_cast<const uint32_t*>(blk + A.off_usb) + jj[v] * GH;
    }
    // unconditional: a row of a missing expert reads block 0 and is stored as NaN
    dH.template fetch_always<4>(cr, sr, glh, q, sq);
  };
  // unconditional, so that the waits below count exactly (a wave without items
  // reads rows of expert 0 that every such wave shares)
  fetch_pairs(it);
  // this wave's routed down rows of the workgroup's output rows, into registers:
  // MAXR items (known since the top-K; an unused one reads a valid row it
  // ignores).  Issued here, behind the gate/up rows, so that they arrive during
  // the gate/up dots: loads return in issue order per CU, so loads issued at the
  // end of step 7 would hold up the h reads of steps 8 and 9.  (The down
  // rows once went to LDS by DMA; after an LDS DMA the compiler makes the next use
  // of any loaded register wait for every load, DMA included.)
#pragma unroll
  for (int m = 0; m < MAXR; ++m) {
    const int t = wv * MAXR + m;
    const int k = t / DITEMS, d = t % DITEMS;
    const int e = (t < K * DITEMS && k < kFusedMaxK) ? eidx[k] : -1;
    // every output row of the pass lies inside H (H is a multiple of kRB), so a
    // valid expert reads rows row0 + d*RPWI + subi
    const bool ok = (unsigned)e < (unsigned)E;
    const uint8_t* blk = ok ? Lp.rbase + (int64_t)e * Lp.rstride : Lp.sblk;
    const int rb = ok ? row0 + d * RPWI : 0;
    dq[1 + m] = ld_stream16(blk + A.off_d + (int64_t)rb * RBI + (uint32_t)(subi * RBI + 16 * gli));
    dsc[1 + m] = ld_stream4(reinterpret_cast<const uint32_t*>(blk + A.off_dsb) + (int64_t)rb * GI +
                            (uint32_t)(subi * GI + gli / QTraits<BITS>::CPG));
  }
  QMOE_PT(7);
  // ---- 4. shared gate/up + SwiGLU -> hs (one item per wave at most): computed
  //         only here, while the routed rows of step 6 travel
  if (has_sp) {
    float p[2];
    dH.template dots<2>(qsp, ssp, p);
    const float a = group_sum_last<LGH>(p[0]);
    const float u = group_sum_last<LGH>(p[1]);
    hs_val = silu_f(a) * u;
    if (group_last<LGH>(lane)) tag_put(hs + hpos(jsp, kHsW), hs_val, tag);
  }
  // ---- 7. routed gate/up dots + SwiGLU -> hr, two row pairs per step (the first
  //         step outside the loop, so that its dots wait for their own rows only,
  //         not for the down rows issued after them)
  auto gate_up_step = [&](int it0) {
    float p[4];
    dH.template dots<4>(q, sq, p);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const float a = group_sum_last<LGH>(p[2 * v]);
      const float u = group_sum_last<LGH>(p[2 * v + 1]);
      if (group_last<LGH>(lane) && it0 + v * W < n_rp)
        tag_put(hr + hpos(kk[v] * I + jj[v], kHrW), eok[v] ? silu_f(a) * u : __builtin_nanf(""), tag);
    }
  };
  if (it < n_rp) gate_up_step(it);
  for (it += 2 * W; it < n_rp; it += 2 * W) {
    fetch_pairs(it);
    gate_up_step(it);
  }
  // the planes of n h values (n a multiple of a chunk) built straight from
  // registers: thread t reads the values of code word t, tagged words
  // src[e * stride + t] (e < EPW); one DPP quad holds a chunk; a wave with no word
  // in a pass skips it.
  // 2-bit: half a code word per thread instead (8 values: elements 2k + h of word
  // t >> 1, at stride 2 * stride from src[h * stride + (t >> 1)]), so that twice the
  // threads each read and convert half as many values.
  auto h_planes = [&](const uint64_t* src, int stride, int n, uint32_t* planes, float* scl, float* xsum) {
    if constexpr (BITS == 2) {
      const int halves = n / 8;
      for (int t0 = 0; t0 < halves; t0 += kLB) {
        if (t0 + (int)wv * 64 >= halves) break;
        const int t = t0 + (int)tx;
        const bool valid = t < halves;
        float v[8];
        read_tagged_strided<8>(src + (t & 1) * stride + (t >> 1), 2 * stride, valid, v, tag, ok_all);
        prep_x_half2<PWL>(v, valid, t, planes, scl, xsum);
      }
    } else {
      constexpr int EPW = QTraits<BITS>::EPW;
      const int words = n / EPW;
      for (int w0 = 0; w0 < words; w0 += kLB) {
        if (w0 + (int)wv * 64 >= words) break;
        const int w = w0 + (int)tx;
        const bool valid = w < words;
        float v[EPW];
        read_tagged_strided<EPW>(src + w, stride, valid, v, tag, ok_all);
        prep_x_word<BITS, PWL>(v, valid, w, planes, scl, xsum);
      }
    }
  };
  // completion: once every wave has issued its h stores, one tagged flag, written
  // as a whole 64-byte store into a line of its own.  A bare barrier: it orders
  // the issue only.  No reader waits for the flags (the h words carry their own
  // tags), but the barrier and the store keep this workgroup's h reads behind its
  // own h stores: without the barrier the layer took 15.45 us, with the barrier
  // alone 14.60, with both 14.51.
  QMOE_PT(8);
  __builtin_amdgcn_s_barrier();
  if (tx < 8) tag_put(Lp.flags + wg * kLine + tx, 0.f, tag);
  // ---- 8. the shared expert's h, read as soon as this workgroup's own routed dots
  //         are done: every workgroup runs its shared dots before its routed ones,
  //         so these words are nearly always current by now (each is checked by
  //         its tag and read again until it is).  Its planes, the shared down rows
  //         and gamma's dot then run before the wait for the routed h, not after it
  //         (measured: 14.91 against 15.28 us per layer, 2-bit 14.16 against 14.72;
  //         the routed planes then also fit one pass of the workgroup's threads).
  h_planes(hs, kHsW, I, s_hp + K * CI * PWL, s_hsc + K * CI, s_hsum + K * CI);
  __syncthreads();
  // (a thread past H/8 holds a copy of the last chunk: it adds nothing)
  const float gpart = group_sum_last<64>((int)tx < H / 8 ? bf16_chunk_dot(gq, gx) : 0.f);
  if (lane == 63) s_rv[wv] = gpart;
  if (wv < DITEMS) {  // the wave's shared down item
    RowDot<BITS, LGI, 1> dS;
    dS.template load_prepped<PWL>(s_hp + K * CI * PWL, s_hsc + K * CI, s_hsum + K * CI, CI, gli);
    const uint4 qs[1][1] = {{dq[0]}};
    const uint32_t ss[1][1] = {{dsc[0]}};
    float ps[1];
    dS.template dots<1>(qs, ss, ps);
    const float vs = group_sum_last<LGI>(ps[0]);
    if (group_last<LGI>(lane) && nl_s < kRB) s_y[kFusedMaxK][nl_s] = vs;
  }
  QMOE_PT(9);
  // ---- 9. read hr, each word until it carries this call's tag; the routed down
  //         rows (integer dots against the planes of h, codes in registers since
  //         step 6); combine.  No wait for the flags first: polling the h words
  //         themselves at this point measured faster (14.51 against 14.88 us per
  //         layer, 2-bit 13.57 against 14.27).
  QMOE_PT(10);
  h_planes(hr, kHrW, K * I, s_hp, s_hsc, s_hsum);
  QMOE_PT(11);
  if constexpr (STACK) {
    // the next layer's loads that do not depend on its input: the shared-gate
    // vector, the norm weight, the first router rows and the shared expert's rows.
    // They go out behind the h reads and arrive while the tail below computes.
    if (l + 1 < P.nl) {
      const uint16_t* rtN = reinterpret_cast<const uint16_t*>(tab(l + 1, 2));
      const uint16_t* gN = reinterpret_cast<const uint16_t*>(tab(l + 1, 3));
      const float* nwN_p = reinterpret_cast<const float*>(tab(l + 1, 4));
      gqN = reinterpret_cast<const uint4*>(gN)[xi];
      const float* nwp = nwN_p ? nwN_p : A.x;  // no norm: a load that is ignored
      const float4 w0 = reinterpret_cast<const float4*>(nwp + 8 * xi)[0];
      const float4 w1 = reinterpret_cast<const float4*>(nwp + 8 * xi)[1];
      nwN[0] = w0.x; nwN[1] = w0.y; nwN[2] = w0.z; nwN[3] = w0.w;
      nwN[4] = w1.x; nwN[5] = w1.y; nwN[6] = w1.z; nwN[7] = w1.w;
      router_fetch(rtN, wg * 2 + (wv >> 2), rqN);
    }
  }
  __syncthreads();
  // Every workgroup read the epoch before storing its h: advance it.
  if (wg == 0 && tx == 0)
    __hip_atomic_store(A.ctrl + CTRL_EPOCH, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  QMOE_PT(12);
  // routed down rows: the wave's MAXR items, which all belong to one expert kw, as
  // one branch-free block so that their dots and reductions interleave
  static_assert(DITEMS % MAXR == 0, "the routed down items of a wave share one expert");
  const int kw = (wv * MAXR) / DITEMS;
  if (kw < K) {
    RowDot<BITS, LGI, 1> dR;
    dR.template load_prepped<PWL>(s_hp + kw * CI * PWL, s_hsc + kw * CI, s_hsum + kw * CI, CI, gli);
    uint4 qr[MAXR][1];
    uint32_t sr[MAXR][1];
#pragma unroll
    for (int m = 0; m < MAXR; ++m) {
      qr[m][0] = dq[1 + m];
      sr[m][0] = dsc[1 + m];
    }
    float pr[MAXR];
    dR.template dots<MAXR>(qr, sr, pr);
    float vr[MAXR];
#pragma unroll
    for (int m = 0; m < MAXR; ++m) vr[m] = group_sum_last<LGI>(pr[m]);
    int ew = -1;
#pragma unroll
    for (int k = 0; k < kFusedMaxK; ++k)
      if (k == kw) ew = eidx[k];
    const bool eok_w = (unsigned)ew < (unsigned)E;
    if (group_last<LGI>(lane)) {
#pragma unroll
      for (int m = 0; m < MAXR; ++m) {
        const int nl = ((wv * MAXR + m) % DITEMS) * RPWI + subi;
        if (nl < kRB) s_y[kw][nl] = eok_w ? vr[m] : __builtin_nanf("");
      }
    }
  }
  __syncthreads();
  QMOE_PT(13);
  if ((int)tx < kRB && row0 + (int)tx < H) {
    float gs = 0.f;
#pragma unroll
    for (int w = 0; w < kLW; ++w) gs += s_rv[w];
    float acc = resid;
#pragma unroll
    for (int k = 0; k < kFusedMaxK; ++k)
      if (k < K) acc = fmaf(wsel[k], s_y[k][tx], acc);
    const float v = fmaf(sigmoid_f(gs), s_y[kFusedMaxK][tx], acc);
    // the output is written through to memory (agent-scope stores, as the tagged
    // words are), so the end of the launch finds no dirty L2 lines to write back
    // (measured: 13.99 -> 13.96 us per layer, 2-bit 12.53 -> 12.44)
    if constexpr (STACK) {
      if (P.h_all) P.h_all[(int64_t)l * H + row0 + tx] = v;
      if (l + 1 < P.nl) {  // the workgroup's rows fill one line: a single writer
        tag_put(P.xbuf + ((int64_t)l * NB + wg) * kLine + tx, v, tag);
        resid = v;
      } else {
        __hip_atomic_store(A.out + row0 + tx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      __hip_atomic_store(A.out + row0 + tx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if constexpr (!STACK) {
    break;
  } else {
    if (++l == P.nl) break;
    // ---- 10. (stack) the next layer's input: every workgroup's output line of this
    //         layer, polled word by word until each carries this call's tag; its
    //         other loads were issued in step 9
    {
      constexpr int XW = H / kLB;  // words per thread
      uint64_t* xl = P.xbuf + (int64_t)(l - 1) * NB * kLine;
      uint64_t xv[XW];
#pragma unroll
      for (int j = 0; j < XW; ++j) xv[j] = tag_get(xl + tx + j * kLB);
      uint32_t pend = 0;
      for (uint32_t spins = 0;; ++spins) {
#pragma unroll
        for (int j = 0; j < XW; ++j)
          if ((uint32_t)(xv[j] >> 32) != tag) pend |= 1u << j;
          else pend &= ~(1u << j);
        if (!pend) break;
        if (spins > kSpinLimit) {
          ok_all = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < XW; ++j)
          if ((pend >> j) & 1u) xv[j] = tag_get(xl + tx + j * kLB);
      }
#pragma unroll
      for (int j = 0; j < XW; ++j) s_x[tx + j * kLB] = __uint_as_float((uint32_t)xv[j]);
      __syncthreads();
      const float4 f0 = reinterpret_cast<const float4*>(s_x + 8 * xi)[0];
      const float4 f1 = reinterpret_cast<const float4*>(s_x + 8 * xi)[1];
      gx[0] = f0.x; gx[1] = f0.y; gx[2] = f0.z; gx[3] = f0.w;
      gx[4] = f1.x; gx[5] = f1.y; gx[6] = f1.z; gx[7] = f1.w;
    }
    Lp.rbase = reinterpret_cast<const uint8_t*>(tab(l, 0));
    Lp.sblk = reinterpret_cast<const uint8_t*>(tab(l, 1));
    Lp.router = reinterpret_cast<const uint16_t*>(tab(l, 2));
    Lp.g = reinterpret_cast<const uint16_t*>(tab(l, 3));
    Lp.norm_w = reinterpret_cast<const float*>(tab(l, 4));
    Lp.rstride = (int64_t)tab(l, 5);
    Lp.idx_out = A.idx_out + l * K;
    Lp.w_out = A.w_out + l * K;
    gq = gqN;
#pragma unroll
    for (int i = 0; i < 8; ++i) nw[i] = nwN[i];
#pragma unroll
    for (int i = 0; i < CPLR; ++i) rq[i] = rqN[i];
  }
  }  // layers
  QMOE_PT(14);
  if (!ok_all) flag_status(A.ctrl, 1u);
  QMOE_PT_STORE();
}

template <int BITS, int H, int I>
__global__ __launch_bounds__(kLB, 2) void k_layer(LayerArgs A) {
  layer_body<BITS, H, I, false>(A, A);
}

template <int BITS, int H, int I>
__global__ __launch_bounds__(kLB, 2) void k_stack(StackArgs S) {
  layer_body<BITS, H, I, true>(S.A, S);
}

struct FusedCfg {
  int nb = 0, rb = 0;
};

inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

struct WsLayout {
  int64_t ctrl, logits, flags, hs, hr, total;
};

WsLayout fused_ws(int E, int H, int I) {
  WsLayout w;
  w.ctrl = 0;
  w.logits = 256;
  w.flags = w.logits + align256((int64_t)((E + 1) / 2) * kLine * 8);
  w.hs = w.flags + align256((int64_t)(H / kRB) * kLine * 8);
  w.hr = w.hs + align256((int64_t)kSlotsH * I * 8);
  w.total = w.hr + align256((int64_t)kSlotsH * kFusedMaxK * I * 8);
  return w;
}

// unfused fallback: logits[E] | y_routed[K][H] | y_shared[H] | h[K][I] (ctrl block stays zero)
// | xn[H] (the normalised input, for the RMSNorm variant)
struct UnfusedWs {
  int64_t logits, yr, ys, h, xn, total;
};

UnfusedWs unfused_ws(int E, int K, int H, int I) {
  UnfusedWs u;
  u.logits = 256;
  u.yr = u.logits + align256((int64_t)E * 4);
  u.ys = u.yr + align256((int64_t)K * H * 4);
  u.h = u.ys + align256((int64_t)H * 4);
  u.xn = u.h + align256((int64_t)K * I * 4);
  u.total = u.xn + align256((int64_t)H * 4);
  return u;
}

using KernelFn = void (*)(LayerArgs);
using StackFn = void (*)(StackArgs);

template <bool ST>
using FnOf = typename std::conditional<ST, StackFn, KernelFn>::type;

template <bool ST, int BITS, int H, int I>
FnOf<ST> pick() {
  if constexpr (ST)
    return k_stack<BITS, H, I>;
  else
    return k_layer<BITS, H, I>;
}

template <bool ST, int BITS, int H>
FnOf<ST> pick_i(int I) {
  if (I == 256) return pick<ST, BITS, H, 256>();
  if (I == 512) return pick<ST, BITS, H, 512>();
  if (I == 1024) return pick<ST, BITS, H, 1024>();
  return nullptr;
}

template <bool ST, int BITS>
FnOf<ST> pick_h(int H, int I) {
  if (H == 1024) return pick_i<ST, BITS, 1024>(I);
  if (H == 2048) return pick_i<ST, BITS, 2048>(I);
  if (H == 4096) return pick_i<ST, BITS, 4096>(I);
  return nullptr;
}

// grid geometry for the fused kernel, or nb == 0 when the shape needs the fallback
FusedCfg fused_config(const qmoe_layer& L, const void* fn) {
  FusedCfg c;
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  if (!fn || K > kFusedMaxK || E > kFusedMaxE || H % kRB) return c;
  if (H / kRB > kLB) return c;  // at most kLB workgroups (one per CU, all co-resident)
  const int cus = device_cus();
  if (cus <= 0) return c;
  int blocks_per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks_per_cu, fn, kLB, 0) != hipSuccess ||
      blocks_per_cu < 1)
    return c;
  const int nb = H / kRB;
  if (nb > cus * blocks_per_cu) return c;  // every workgroup must be resident at once
  const int bits = L.routed.bits;
  const int ch = H * bits / 128;
  const int rpwh = 64 / (ch >= 64 ? 64 : ch);
  const int n_sp = I / rpwh;
  // one shared gate/up item per wave at most, and every workgroup must tag a routed
  // h row (rank == workgroup index) for the epoch hand-over
  if (n_sp > nb * kLW || K * n_sp < nb) return c;
  c.nb = nb;
  c.rb = kRB;
  return c;
}

template <bool ST>
FnOf<ST> fused_kernel(const qmoe_layer& L) {
  const int H = L.routed.hidden, I = L.routed.inter;
  return L.routed.bits == 4 ? pick_h<ST, 4>(H, I) : pick_h<ST, 2>(H, I);
}

LayerArgs layer_args(const qmoe_layer& L, const float* x, const float* norm_w, float eps,
                     const float* residual, float* out, int32_t* idx, float* w, uint8_t* wsb) {
  const int E = L.routed.num_experts, H = L.routed.hidden, I = L.routed.inter;
  const WsLayout wl = fused_ws(E, H, I);
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
  A.norm_w = norm_w;
  A.eps = eps;
  A.residual = residual;
  A.out = out;
  A.idx_out = idx;
  A.w_out = w;
  A.ctrl = reinterpret_cast<uint32_t*>(wsb + wl.ctrl);
  A.logits = reinterpret_cast<uint64_t*>(wsb + wl.logits);
  A.flags = reinterpret_cast<uint64_t*>(wsb + wl.flags);
  A.hs = reinterpret_cast<uint64_t*>(wsb + wl.hs);
  A.hr = reinterpret_cast<uint64_t*>(wsb + wl.hr);
  A.E = E;
  A.K = L.top_k;
  return A;
}

// stack workspace: the single layer's (every layer of a launch uses its buffers,
// each with its own call number), then the output lines of each layer
struct StackWs {
  int64_t xbuf, total;
};

StackWs stack_ws(const qmoe_layer& L, int n) {
  const WsLayout wl = fused_ws(L.routed.num_experts, L.routed.hidden, L.routed.inter);
  const int nl = n < kStackMax ? n : kStackMax;
  StackWs w;
  w.xbuf = wl.total;
  w.total = w.xbuf + align256((int64_t)nl * (L.routed.hidden / kRB) * kLine * 8);
  return w;
}

}  // namespace

size_t layer_workspace_bytes(const qmoe_layer& L) {
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  const WsLayout f = fused_ws(E, H, I);
  const UnfusedWs u = unfused_ws(E, K, H, I);
  return (size_t)(f.total > u.total ? f.total : u.total);
}

hipError_t launch_layer(const qmoe_layer& L, const float* x, const float* norm_w, float eps,
                        const float* residual, float* out, int32_t* idx, float* w, void* ws,
                        hipStream_t s) {
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  KernelFn fn = fused_kernel<false>(L);
  const FusedCfg cfg = fused_config(L, reinterpret_cast<const void*>(fn));
  if (cfg.nb > 0) {
    const LayerArgs A = layer_args(L, x, norm_w, eps, residual, out, idx, w, wsb);
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
  hipError_t err = hipSuccess;
  if (norm_w) {
    float* xn = reinterpret_cast<float*>(wsb + u.xn);
    err = launch_rmsnorm(x, norm_w, eps, H, xn, s);
    x = xn;
  }
  if (err == hipSuccess) err = launch_router_topk(L.router, x, 1, H, E, K, logits, idx, w, s);
  if (err == hipSuccess) err = launch_ffn(L.routed, idx, K, x, 0, yr, h, s);
  if (err == hipSuccess) err = launch_ffn(L.shared, zero_idx, 1, x, 0, ys, h, s);
  if (err == hipSuccess) err = launch_combine(yr, w, ys, L.shared_gate, x, residual, out, H, K, s);
  return err;
}

size_t stack_workspace_bytes(const qmoe_layer& L, int n_layers) {
  const size_t st = (size_t)stack_ws(L, n_layers).total;
  const size_t one = layer_workspace_bytes(L);
  return st > one ? st : one;
}

hipError_t launch_stack(const qmoe_layer* Ls, const float* const* norm_w, int n, float eps,
                        const float* h0, float* out, float* h_all, int32_t* idx, float* w, void* ws,
                        bool persistent, hipStream_t s) {
  const qmoe_layer& L0 = Ls[0];
  const int K = L0.top_k, H = L0.routed.hidden;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  StackFn fn = persistent ? fused_kernel<true>(L0) : nullptr;
  const FusedCfg cfg = fn ? fused_config(L0, reinterpret_cast<const void*>(fn)) : FusedCfg{};
  hipError_t err = hipSuccess;
  if (cfg.nb == 0) {  // one launch per layer: layer l reads layer l-1's output
    const float* cur = h0;
    for (int l = 0; l < n && err == hipSuccess; ++l) {
      float* dst = h_all ? h_all + (int64_t)l * H : out;
      err = launch_layer(Ls[l], cur, norm_w[l], eps, cur, dst, idx + l * K, w + l * K, ws, s);
      cur = dst;
    }
    if (err == hipSuccess && h_all)
      err = hipMemcpyAsync(out, cur, (size_t)H * 4, hipMemcpyDeviceToDevice, s);
    return err;
  }
  const StackWs sw = stack_ws(L0, n);
  // launches of up to kStackMax layers; a later launch reads its input from out
  // (every workgroup reads its input before any writes its rows of out)
  for (int c0 = 0; c0 < n; c0 += kStackMax) {
    const int nl = n - c0 < kStackMax ? n - c0 : kStackMax;
    const float* xin = c0 == 0 ? h0 : out;
    StackArgs S;
    S.A = layer_args(Ls[c0], xin, norm_w[c0], eps, xin, out, idx + (int64_t)c0 * K,
                     w + (int64_t)c0 * K, wsb);
    S.xbuf = reinterpret_cast<uint64_t*>(wsb + sw.xbuf);
    S.h_all = h_all ? h_all + (int64_t)c0 * H : nullptr;
    S.nl = nl;
    for (int i = 0; i < nl; ++i) {
      const qmoe_layer& Li = Ls[c0 + i];
      S.st[i].rbase = static_cast<const uint8_t*>(Li.routed.base);
      S.st[i].sblk = static_cast<const uint8_t*>(Li.shared.base);
      S.st[i].router = Li.router;
      S.st[i].g = Li.shared_gate;
      S.st[i].norm_w = norm_w[c0 + i];
      S.st[i].rstride = Li.routed.stride;
    }
    hipLaunchKernelGGL(fn, dim3(cfg.nb), dim3(kLB), 0, s, S);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace qmoe

#ifdef QMOE_PHASE_PROBE
// the recorded phase timestamps: [64 calls][512 workgroups][16 phases] of uint32
extern "C" int qmoe_phase_probe_read(void* dst) {
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(qmoe::g_phase), sizeof(qmoe::g_phase));
}
#endif
