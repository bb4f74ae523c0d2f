// Host-tier expert offload: the routed experts of a layer live in pinned host
// memory and an LRU cache of expert slots in HBM holds the ones recently used.
//
// The page "flash-moe 소개" (discuss.pytorch.kr), sections "SSD 전문가 스트리밍과
// "OS 신뢰" 원칙" and "레이어당 파이프라인 상세 구조", streams the four selected
// experts of each layer from SSD with parallel reads after a host-side top-K and
// lets the OS page cache keep the popular ones; on its unified memory the reads and
// the GPU share one memory controller, so it runs them one after the other.  On a
// discrete GPU the copies travel over the host link and land in HBM by DMA, so here
// they overlap the compute of the same layer:
//   1. router + top-K on the GPU; the K indices go to pinned host memory;
//   2. the shared expert's FFN is enqueued at once (it needs no routing);
//   3. the host waits for the indices only, maps each expert to a slot (a hit, or
//      the least recently used slot not taken by this token), and enqueues one
//      host-to-device copy per miss on the copy stream, after the previous token's
//      expert FFN has released the slots it read;
//   4. the compute stream waits for the copies, then runs the routed FFN on the
//      slots and the combine.
// The cache state is host memory of this handle; the slot memory and the host pool
// are the caller's.  Calls on one handle must come from one host thread at a time.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "qmoe_internal.h"

struct qmoe_offload {
  qmoe_expert_pool host;  // base: pinned host memory
  uint8_t* slots;         // device, n_slots * host.stride bytes
  int32_t n_slots;
  int64_t block_bytes;
  std::vector<int32_t> slot_of;    // expert -> slot, -1 if not resident
  std::vector<int32_t> expert_in;  // slot -> expert, -1 if empty
  std::vector<uint64_t> last_use;  // slot -> tick of last use
  uint64_t tick = 0;
  int32_t* idx_host = nullptr;   // pinned [kMaxTopK]: the token's experts
  int32_t* slot_host = nullptr;  // pinned [kMaxTopK]: their slots
  hipEvent_t ev_idx = nullptr, ev_copies = nullptr, ev_ffn = nullptr;
  bool ffn_recorded = false;
  qmoe_offload_stats stats{};
};

namespace qmoe {

size_t offload_workspace_bytes(const qmoe_layer& L) {
  // logits[E] | y_routed[K][H] | y_shared[H] | h[K][I] | slot list[K] (256-B aligned parts)
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  return al(E * 4) + al(K * H * 4) + al(H * 4) + al(K * I * 4) + al(K * 4) + 256;
}

int offload_create(const qmoe_expert_pool& host, int32_t n_slots, void* slot_mem,
                   qmoe_offload** out) {
  qmoe_offload* o = new (std::nothrow) qmoe_offload();
  if (!o) return QMOE_EINVAL;
  o->host = host;
  o->slots = static_cast<uint8_t*>(slot_mem);
  o->n_slots = n_slots;
  o->block_bytes = expert_offsets(host.hidden, host.inter, host.bits).total;
  o->slot_of.assign(host.num_experts, -1);
  o->expert_in.assign(n_slots, -1);
  o->last_use.assign(n_slots, 0);
  hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&o->idx_host), 2 * kMaxTopK * sizeof(int32_t),
                               hipHostMallocDefault);
  if (e == hipSuccess) {
    o->slot_host = o->idx_host + kMaxTopK;
    e = hipEventCreateWithFlags(&o->ev_idx, hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&o->ev_copies, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&o->ev_ffn, hipEventDisableTiming);
  if (e != hipSuccess) {
    offload_destroy(o);
    return QMOE_EHIP;
  }
  *out = o;
  return QMOE_OK;
}

void offload_destroy(qmoe_offload* o) {
  if (!o) return;
  if (o->ev_idx) hipEventDestroy(o->ev_idx);
  if (o->ev_copies) hipEventDestroy(o->ev_copies);
  if (o->ev_ffn) hipEventDestroy(o->ev_ffn);
  if (o->idx_host) hipHostFree(o->idx_host);
  delete o;
}

void offload_stats(const qmoe_offload* o, qmoe_offload_stats* s) { *s = o->stats; }
const qmoe_expert_pool& offload_host_pool(const qmoe_offload* o) { return o->host; }
int32_t offload_slots(const qmoe_offload* o) { return o->n_slots; }

hipError_t offload_layer(qmoe_offload* o, const qmoe_layer& L, const float* x, const float* residual,
                         float* out, int32_t* idx, float* w, void* ws, hipStream_t s,
                         hipStream_t copy_stream) {
  const int E = L.routed.num_experts, K = L.top_k, H = L.routed.hidden, I = L.routed.inter;
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  float* logits = reinterpret_cast<float*>(wsb);
  float* yr = reinterpret_cast<float*>(wsb + al((size_t)E * 4));
  float* ys = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(yr) + al((size_t)K * H * 4));
  float* h = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ys) + al((size_t)H * 4));
  int32_t* slot_dev = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(h) + al((size_t)K * I * 4));
  int32_t* zero_dev = slot_dev + 64;  // the shared expert's index 0 (set below)

  // 1. routing on the GPU, the indices to the host
  hipError_t e = launch_router_topk(L.router, x, 1, H, E, K, logits, idx, w, s);
  if (e == hipSuccess) e = hipMemcpyAsync(o->idx_host, idx, (size_t)K * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipEventRecord(o->ev_idx, s);
  // 2. the shared expert meanwhile
  if (e == hipSuccess) e = hipMemsetAsync(zero_dev, 0, 4, s);
  if (e == hipSuccess) e = launch_ffn(L.shared, zero_dev, 1, x, 0, ys, h, s);
  if (e != hipSuccess) return e;
  // 3. the host maps the experts to slots; misses are copied on the copy stream
  if ((e = hipEventSynchronize(o->ev_idx)) != hipSuccess) return e;
  ++o->tick;
  bool copies = false;
  if (o->ffn_recorded && (e = hipStreamWaitEvent(copy_stream, o->ev_ffn, 0)) != hipSuccess) return e;
  for (int k = 0; k < K; ++k) {
    const int32_t ex = o->idx_host[k];
    if (ex < 0 || ex >= E) return hipErrorInvalidValue;  // cannot come from the router
    int32_t sl = o->slot_of[ex];
    if (sl >= 0) {
      ++o->stats.hits;
    } else {
      // the least recently used slot that this token does not use (empty slots first)
      int32_t best = -1;
      for (int32_t c = 0; c < o->n_slots; ++c) {
        if (o->last_use[c] == o->tick) continue;
        if (best < 0 || o->last_use[c] < o->last_use[best]) best = c;
      }
      sl = best;
      if (o->expert_in[sl] >= 0) o->slot_of[o->expert_in[sl]] = -1;
      o->expert_in[sl] = ex;
      o->slot_of[ex] = sl;
      e = hipMemcpyAsync(o->slots + (int64_t)sl * o->host.stride,
                         static_cast<const uint8_t*>(o->host.base) + (int64_t)ex * o->host.stride,
                         (size_t)o->block_bytes, hipMemcpyHostToDevice, copy_stream);
      if (e != hipSuccess) return e;
      copies = true;
      ++o->stats.misses;
      o->stats.bytes_copied += (uint64_t)o->block_bytes;
    }
    o->last_use[sl] = o->tick;
    o->slot_host[k] = sl;
  }
  // 4. the routed experts on their slots, then the combine
  if (copies) {
    if ((e = hipEventRecord(o->ev_copies, copy_stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(s, o->ev_copies, 0)) != hipSuccess) return e;
  }
  e = hipMemcpyAsync(slot_dev, o->slot_host, (size_t)K * 4, hipMemcpyHostToDevice, s);
  qmoe_expert_pool slot_pool = o->host;
  slot_pool.base = o->slots;
  slot_pool.num_experts = o->n_slots;
  if (e == hipSuccess) e = launch_ffn(slot_pool, slot_dev, K, x, 0, yr, h, s);
  if (e == hipSuccess) e = hipEventRecord(o->ev_ffn, s);
  if (e == hipSuccess) o->ffn_recorded = true;
  if (e == hipSuccess) e = launch_combine(yr, w, ys, L.shared_gate, x, residual, out, H, K, s);
  ++o->stats.calls;
  return e;
}

}  // namespace qmoe
