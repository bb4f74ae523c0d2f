// One expert FFN with fused SwiGLU in a single launch: y = D (silu(G x) * (U x)).
//
// The page "flash-moe 소개" (discuss.pytorch.kr), section "손으로 작성한 Metal 컴퓨트
// 셰이더", lists the dequant matvec and the fused SwiGLU among the hand-written
// kernels.  The stand-alone path (kernels.hip) runs the gate/up rows and the down
// rows as two launches; here one launch does both and hands h from workgroup to
// workgroup as tagged words (qmoe_handoff.h), as the fused layer does for its
// shared expert:
//   NB = H/16 workgroups of 8 waves, all co-resident; workgroup b owns output rows
//   [16b, 16b+16); rank = wave * NB + workgroup numbers the waves so that
//   consecutive ranks sit on different CUs.
//   1. loads: x (thread t: code word t), the call counter, the expert index,
//      then (into registers) the wave's gate/up row pair (ranks below I/RPWH)
//      and its down rows of the workgroup's output rows;
//   2. x as fixed-point planes, built from registers into LDS, then in every
//      wave's registers;
//   3. gate/up dots + SwiGLU -> h (tagged stores);
//   4. h read by every workgroup straight into its planes (no LDS copy of the
//      values), each word until it carries this call's number; the down rows -> y.
// The down rows travel during steps 2-3 instead of being requested after a kernel
// boundary, and the boundary itself (launch gap, the second kernel's first load of
// h) becomes one read of tagged words.
#include "qmoe_device.h"
#include "qmoe_handoff.h"
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kFB = 512;       // threads per workgroup
constexpr int kFW = kFB / 64;  // waves per workgroup
constexpr int kFR = 16;        // output rows per workgroup

struct Ffn1Args {
  const uint8_t* base;  // the pool: expert e at base + e * stride
  int64_t stride;
  int E;
  const int32_t* idx;   // device: the expert
  int64_t off_g, off_u, off_d, off_gsb, off_usb, off_dsb;
  const float* x;
  float* y;
  uint32_t* ctrl;  // CTRL_EPOCH: calls so far; CTRL_STATUS: bit 0 set on a time-out
  uint64_t* h;     // [kSlotsH][H] tagged h values: see k_ffn1
};

template <int BITS, int H, int I>
__global__ __launch_bounds__(kFB, 2) void k_ffn1(Ffn1Args A) {
  // ---- compile-time geometry (as the fused layer's shared expert)
  constexpr int CH = H * BITS / 128;       // 16-byte chunks per gate/up row
  constexpr int LGH = CH >= 64 ? 64 : CH;  // lanes per gate/up row
  constexpr int CPLH = CH / LGH;           // chunks per lane
  constexpr int RPWH = 64 / LGH;           // gate/up rows per wave pass
  static_assert(LGH * CPLH == CH, "every chunk of a gate/up row has a lane");
  constexpr int GH = H / kGroup;
  constexpr int64_t RBH = (int64_t)H * BITS / 8;
  constexpr int CI = I * BITS / 128;       // 16-byte chunks per down row
  constexpr int LGI = CI;                  // one chunk per lane
  static_assert(CI <= 64, "down rows must fit one chunk per lane");
  constexpr int RPWI = 64 / LGI;           // down rows per wave pass
  constexpr int GI = I / kGroup;
  constexpr int64_t RBI = (int64_t)I * BITS / 8;
  constexpr int DITEMS = kFR / RPWI;       // down items per workgroup
  static_assert(kFR % RPWI == 0 && DITEMS <= kFW, "one down item per wave at most");
  constexpr int NSP = I / RPWH;            // gate/up items
  constexpr int PW = QTraits<BITS>::PW;
  // plane words per chunk as kept in LDS: 16 bytes of padding per chunk, so that the
  // 16-byte reads of consecutive lanes (one chunk each) fall in different banks
  constexpr int PWL = PW + 4;

  constexpr int NB = H / kFR;              // the grid (the host launches exactly this)
  static_assert(I <= H, "a workgroup's h words fit one line");
  const int wg = blockIdx.x;
  const int tx = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int lane = tx & 63;
  const int rank = wv * NB + wg;
  const int glh = lane % LGH, subh = lane / LGH;
  const int gli = lane % LGI, subi = lane / LGI;
  const int row0 = wg * kFR;

  __shared__ __align__(16) uint32_t s_xp[CH * PWL];
  __shared__ float s_xsc[CH], s_xsum[CH];
  __shared__ __align__(16) uint32_t s_hp[CI * PWL];
  __shared__ float s_hsc[CI], s_hsum[CI];
  bool ok = true;

  // ---- 1. loads, every one unconditional with a clamped address: vector memory
  //         completes in issue order, and a straight run of loads lets each use
  //         below wait for its own data only.  A bad index reads expert 0 and
  //         stores NaN.  x goes first: its loads depend on nothing, so their
  //         round trip overlaps the expert index's, which every row address
  //         waits for (issued after that wait, as the compiler placed them
  //         otherwise, the call took 7.47 against 6.27 us).  Thread t loads code
  //         word t of x (EPW values).
  constexpr int EPW = QTraits<BITS>::EPW;
  static_assert(H / EPW <= kFB, "one code word of x per thread");
  const bool xvalid = tx < H / EPW;
  float xv[EPW];
  {
    const float4* xp = reinterpret_cast<const float4*>(A.x + EPW * min(tx, H / EPW - 1));
#pragma unroll
    for (int k = 0; k < EPW; k += 4) {
      const float4 f = xp[k / 4];
      xv[k] = f.x;
      xv[k + 1] = f.y;
      xv[k + 2] = f.z;
      xv[k + 3] = f.w;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t epoch = __hip_atomic_load(A.ctrl + CTRL_EPOCH, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int e = __builtin_amdgcn_readfirstlane(A.idx[0]);
  const bool eok = (unsigned)e < (unsigned)A.E;
  const uint8_t* blk = A.base + (eok ? (int64_t)e * A.stride : 0);
  // h layout: workgroup b = e * Q + q owns the line b * kLine, whose word i holds
  // h value EPW * (SPW * q + i) + e (i < SPW): value e of code words SPW*q .. +SPW.
  // So each line has a single writer, and the thread that builds code word t's
  // planes reads its EPW values at one stride, the lanes of a wave in runs of SPW
  // contiguous words.
  constexpr int SPW = I / NB;              // h words per workgroup
  constexpr int Q = I / EPW / SPW;         // workgroups per value position e
  static_assert(SPW * NB == I && Q * EPW == NB && SPW % RPWH == 0, "h layout");
  const bool has = rank < NSP;  // item wv of this workgroup: words wv*RPWH .. +RPWH
  const int j = has ? EPW * (SPW * (wg % Q) + wv * RPWH + subh) + wg / Q : subh;  // no item: ignored
  RowDot<BITS, LGH, CPLH> dH;
  uint4 q[2][CPLH];
  uint32_t sq[2][CPLH];
  {
    const uint8_t* cr[2] = {blk + A.off_g + j * RBH, blk + A.off_u + j * RBH};
    const uint32_t* sr[2] = {reinterpret_cast<const uint32_t*>(blk + A.off_gsb) + j * GH,
                             reinterpret_cast<const uint32_t*>(blk + A.off_usb) + j * GH};
    dH.template fetch_always<2>(cr, sr, glh, q, sq);
  }
  // the wave's down rows (waves below DITEMS; another wave reads rows it ignores):
  // a wave-uniform row base plus a 32-bit lane offset
  const int rb = wv < DITEMS ? row0 + wv * RPWI : row0;
  const uint4 dq = ld_stream16(blk + A.off_d + (int64_t)rb * RBI + (uint32_t)(subi * RBI + 16 * gli));
  const uint32_t dsc = ld_stream4(reinterpret_cast<const uint32_t*>(blk + A.off_dsb) + (int64_t)rb * GI +
                                  (uint32_t)(subi * GI + gli / QTraits<BITS>::CPG));

  // ---- 2. x planes, built from registers into LDS (once per workgroup), then in
  //         every wave's registers
  if (wv * 64 < H / EPW) prep_x_word<BITS, PWL>(xv, xvalid, tx, s_xp, s_xsc, s_xsum);
  __syncthreads();
  dH.template load_prepped<PWL>(s_xp, s_xsc, s_xsum, CH, glh);
  // tag 0 is what a zero-filled workspace holds: skipped when the counter wraps
  uint32_t tag = (uint32_t)__builtin_amdgcn_readfirstlane((int)epoch) + 1u;
  tag = tag ? tag : 1u;
  // h lives in lines with a single writer, since such a line becomes visible to
  // other CUs sooner than one written by several (measured per call, 4096 x 1024
  // 4-bit: 7.40 us with the layout above read straight into planes; 8.03 with
  // single-writer lines read in buffer order into LDS; 8.46 with h in row order,
  // 16 writers per line; 8.27 for the two launches of kernels.hip)
  uint64_t* hb = A.h + (int64_t)(tag % kSlotsH) * H;

  // ---- 3. gate/up dots + SwiGLU -> h
  if (has) {
    float p[2];
    dH.template dots<2>(q, sq, p);
    const float a = group_sum_last<LGH>(p[0]);
    const float u = group_sum_last<LGH>(p[1]);
    if (group_last<LGH>(lane)) tag_put(hb + wg * kLine + wv * RPWH + subh, eok ? silu_f(a) * u : __builtin_nanf(""), tag);
  }

  // ---- 4. h read straight into its planes (the barrier keeps the reads behind
  //         this workgroup's own h stores): thread t takes code word t; the down
  //         rows
  __builtin_amdgcn_s_barrier();
  static_assert(I / EPW <= kFB, "one code word of h per thread");
  if (wv * 64 < I / EPW) {
    const bool valid = tx < I / EPW;
    float v[EPW];
    read_tagged_strided<EPW>(hb + (tx / SPW) * kLine + tx % SPW, Q * kLine, valid, v, tag, ok);
    prep_x_word<BITS, PWL>(v, valid, tx, s_hp, s_hsc, s_hsum);
  }
  __syncthreads();
  // Every workgroup read the counter before storing its h (each stores at least
  // one word: rank wg < I/RPWH): advance it.
  if (wg == 0 && tx == 0)
    __hip_atomic_store(A.ctrl + CTRL_EPOCH, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (wv < DITEMS) {
    RowDot<BITS, LGI, 1> dD;
    dD.template load_prepped<PWL>(s_hp, s_hsc, s_hsum, CI, gli);
    const uint4 qd[1][1] = {{dq}};
    const uint32_t sd[1][1] = {{dsc}};
    float p[1];
    dD.template dots<1>(qd, sd, p);
    const float v = group_sum_last<LGI>(p[0]);
    if (group_last<LGI>(lane)) A.y[row0 + wv * RPWI + subi] = eok ? v : __builtin_nanf("");
  }
  if (!ok) flag_status(A.ctrl, 1u);
}

using Ffn1Fn = void (*)(Ffn1Args);

template <int BITS, int H>
Ffn1Fn pick_ffn1_i(int I) {
  if (I == 256) return k_ffn1<BITS, H, 256>;
  if (I == 512) return k_ffn1<BITS, H, 512>;
  if (I == 1024) return k_ffn1<BITS, H, 1024>;
  return nullptr;
}

template <int BITS>
Ffn1Fn pick_ffn1_h(int H, int I) {
  if (H == 1024) return pick_ffn1_i<BITS, 1024>(I);
  if (H == 2048) return pick_ffn1_i<BITS, 2048>(I);
  if (H == 4096) return pick_ffn1_i<BITS, 4096>(I);
  return nullptr;
}

Ffn1Fn ffn1_kernel(const qmoe_expert_pool& pool) {
  return pool.bits == 4 ? pick_ffn1_h<4>(pool.hidden, pool.inter) : pick_ffn1_h<2>(pool.hidden, pool.inter);
}

inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

}  // namespace

// [0, 256): control words; then kSlotsH slots of H tagged h words (a line of 16 per
// workgroup, I/(H/16) of them used)
size_t ffn_fused_ws_bytes(const qmoe_expert_pool& pool) {
  return (size_t)(256 + align256((int64_t)kSlotsH * pool.hidden * 8));
}

bool ffn_fused_supported(const qmoe_expert_pool& pool) {
  const Ffn1Fn fn = ffn1_kernel(pool);
  if (!fn) return false;
  const int H = pool.hidden, I = pool.inter;
  const int nb = H / kFR;
  const int ch = H * pool.bits / 128;
  const int nsp = I / (64 / (ch >= 64 ? 64 : ch));
  // one gate/up item per wave at most, and one at least per workgroup (the counter
  // hand-over needs a word from every workgroup); a workgroup's h words in one line
  if (nsp > nb * kFW || nsp < nb || I > H) return false;
  const int cus = device_cus();
  int per_cu = 0;
  if (cus <= 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn),
                                                               kFB, 0) != hipSuccess || per_cu < 1)
    return false;
  return nb <= cus * per_cu;  // every workgroup resident at once
}

hipError_t launch_ffn_fused(const qmoe_expert_pool& pool, const int32_t* idx, const float* x, float* y,
                            void* ws, hipStream_t s) {
  const Ffn1Fn fn = ffn1_kernel(pool);
  if (!fn) return hipErrorInvalidValue;
  const qmoe_expert_offsets o = expert_offsets(pool.hidden, pool.inter, pool.bits);
  Ffn1Args A;
  A.base = static_cast<const uint8_t*>(pool.base);
  A.stride = pool.stride;
  A.E = pool.num_experts;
  A.idx = idx;
  A.off_g = o.gate_codes;
  A.off_u = o.up_codes;
  A.off_d = o.down_codes;
  A.off_gsb = o.gate_sb;
  A.off_usb = o.up_sb;
  A.off_dsb = o.down_sb;
  A.x = x;
  A.y = y;
  A.ctrl = static_cast<uint32_t*>(ws);
  A.h = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + 256);
  hipLaunchKernelGGL(fn, dim3(pool.hidden / kFR), dim3(kFB), 0, s, A);
  return hipGetLastError();
}

}  // namespace qmoe
