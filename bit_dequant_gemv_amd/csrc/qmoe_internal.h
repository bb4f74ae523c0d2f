// Internal host-side launch interface between the C ABI (api.cpp) and the
// kernel translation units.  Arguments arrive validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmoe.h"

namespace qmoe {

// largest input width kept in registers per lane group
constexpr int kMaxCols4 = 8192;
constexpr int kMaxCols2 = 16384;
constexpr int kMaxRouterH = 8192;
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 4096;
constexpr int kMaxBatch = 256;

hipError_t launch_qgemv(int bits, const uint8_t* codes, const uint32_t* sb, const float* x,
                        float* y, int rows, int cols, hipStream_t s);

hipError_t launch_ffn(const qmoe_expert_pool& pool, const int32_t* idx, int n, const float* x,
                      int64_t x_stride, float* y, float* h_ws, hipStream_t s);
// One expert's FFN in a single launch (ffn.hip), for the shapes ffn_fused_supported
// accepts.  ws: ffn_fused_ws_bytes(pool) bytes, zero-filled before its first use and
// kept between calls (a call counter and tagged h values).
bool ffn_fused_supported(const qmoe_expert_pool& pool);
size_t ffn_fused_ws_bytes(const qmoe_expert_pool& pool);
hipError_t launch_ffn_fused(const qmoe_expert_pool& pool, const int32_t* idx, const float* x, float* y,
                            void* ws, hipStream_t s);

// prep_bits = 4 or 2 with xplanes: the router may also write the fixed-point x
// planes of every token (pw words per token); *prepped says whether it did.
hipError_t launch_router_topk(const uint16_t* router, const float* x, int T, int H, int E, int K,
                              float* logits, int32_t* idx, float* w, hipStream_t s,
                              int prep_bits = 0, uint32_t* xplanes = nullptr, int pw = 0,
                              bool* prepped = nullptr);

hipError_t launch_combine(const float* y_routed, const float* w, const float* y_shared,
                          const uint16_t* g, const float* x, const float* residual, float* out,
                          int H, int K, hipStream_t s);

hipError_t launch_rmsnorm(const float* v, const float* w, float eps, int n, float* out,
                          hipStream_t s);

// fused single-launch layer (layer.hip)
size_t layer_workspace_bytes(const qmoe_layer& L);
// norm_w null: x is the layer input; else the input is rmsnorm(x) with weight norm_w
hipError_t launch_layer(const qmoe_layer& L, const float* x, const float* norm_w, float eps,
                        const float* residual, float* out, int32_t* idx, float* w, void* ws,
                        hipStream_t s);

// the fused layer with its workspace in a device-global array of
// kNoAllocScratchBytes per GPU instead of a caller's buffer (noalloc.hip); the
// layer's workspace size must not exceed it
constexpr size_t kNoAllocScratchBytes = (size_t)1 << 20;
hipError_t launch_layer_noalloc(const qmoe_layer& L, const float* x, const float* residual,
                                float* out, int32_t* idx, float* w, hipStream_t s);

// a decoder stack of n layers of one shape, h <- h + MoE_l(rmsnorm(h, norm_w[l])):
// one fused launch per layer, or (persistent) one launch per 32 layers (layer.hip)
size_t stack_workspace_bytes(const qmoe_layer& L, int n_layers);
hipError_t launch_stack(const qmoe_layer* layers, const float* const* norm_w, int n, float eps,
                        const float* h0, float* out, float* h_all, int32_t* idx, float* w, void* ws,
                        bool persistent, hipStream_t s);

// GatedDeltaNet recurrence, one decode step (gdn.hip); dk in {64, 128, 256}
hipError_t launch_gdn_step(float* S, const float* q, const float* k, const float* v, const float* alpha,
                           const float* beta, float* o, int heads, int dk, int dv, hipStream_t s);

// full-attention decode (attn.hip); D in {64, 128, 256}, Hq / Hkv <= 16
size_t attn_workspace_bytes(int Hq, int Hkv, int D, int Tmax);
// q_gate_rows: q rows hold 2D floats (query, then gate); q/k_norm_w: RMS weights or
// null; gate: where the gate halves go (q_gate_rows only), or null
hipError_t launch_attn_decode(const float* q, const float* k, const float* v, float* kc, float* vc,
                              int Hq, int Hkv, int D, int Tmax, int pos, float theta, int rot_dim,
                              float* o, void* ws, hipStream_t s, bool q_gate_rows = false,
                              const float* q_norm_w = nullptr, const float* k_norm_w = nullptr,
                              float eps = 0.f, float* gate = nullptr);

// batched decode (batched.hip)
size_t batched_workspace_bytes(const qmoe_layer& L, int T);
hipError_t launch_layer_batched(const qmoe_layer& L, const float* x, const float* residual,
                                float* out, int T, int32_t* idx, float* w, void* ws,
                                hipStream_t s);

// streaming-read calibration (stream.hip): reads bytes/16 16-byte words of buf
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t key, uint32_t* sink,
                              hipStream_t s);

// host-tier expert offload (offload.cpp)
size_t offload_workspace_bytes(const qmoe_layer& L);
int offload_create(const qmoe_expert_pool& host, int32_t n_slots, void* slot_mem, qmoe_offload** out);
void offload_destroy(qmoe_offload* o);
void offload_stats(const qmoe_offload* o, qmoe_offload_stats* s);
const qmoe_expert_pool& offload_host_pool(const qmoe_offload* o);
int32_t offload_slots(const qmoe_offload* o);
hipError_t offload_layer(qmoe_offload* o, const qmoe_layer& L, const float* x, const float* residual,
                         float* out, int32_t* idx, float* w, void* ws, hipStream_t s,
                         hipStream_t copy_stream);

// compute units of the current device (cached per device); 0 if it cannot be read
int device_cus();

// offsets of the canonical expert block
qmoe_expert_offsets expert_offsets(int hidden, int inter, int bits);

}  // namespace qmoe
