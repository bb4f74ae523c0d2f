// C ABI front end of libqmoe: validates every argument on the host, then
// enqueues the kernels on the caller's stream.  Nothing here allocates, frees
// or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "qmoe_internal.h"

static_assert(QMOE_NOALLOC_SCRATCH_BYTES == qmoe::kNoAllocScratchBytes,
              "the header states the allocation-free entry point's scratch size");

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return QMOE_OK;
  return fail(QMOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_vec(const void* p, const char* name) {
  if (!p) return fail(QMOE_EINVAL, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(QMOE_EALIGN, "%s must be 16-byte aligned", name);
  return QMOE_OK;
}

int check_pool(const qmoe_expert_pool* p, const char* name) {
  if (!p) return fail(QMOE_EINVAL, "%s is NULL", name);
  if (!p->base) return fail(QMOE_EINVAL, "%s.base is NULL", name);
  if (p->bits != 2 && p->bits != 4) return fail(QMOE_EINVAL, "%s.bits must be 2 or 4", name);
  if (p->num_experts < 1 || p->num_experts > qmoe::kMaxExperts)
    return fail(QMOE_ESHAPE, "%s.num_experts must be in [1, %d]", name, qmoe::kMaxExperts);
  if (p->hidden < 64 || p->inter < 64 || p->hidden % 64 || p->inter % 64)
    return fail(QMOE_ESHAPE, "%s: hidden and inter must be positive multiples of 64", name);
  const int maxc = p->bits == 4 ? qmoe::kMaxCols4 : qmoe::kMaxCols2;
  if (p->hidden > maxc || p->inter > maxc)
    return fail(QMOE_ESHAPE, "%s: hidden and inter must be at most %d at %d bits", name, maxc,
                p->bits);
  const qmoe_expert_offsets o = qmoe::expert_offsets(p->hidden, p->inter, p->bits);
  if (p->stride < o.total || p->stride % 256)
    return fail(QMOE_EALIGN, "%s.stride must be >= %lld and a multiple of 256", name,
                (long long)o.total);
  if (!aligned(p->base, 256)) return fail(QMOE_EALIGN, "%s.base must be 256-byte aligned", name);
  return QMOE_OK;
}

int check_layer(const qmoe_layer* L) {
  if (!L) return fail(QMOE_EINVAL, "layer is NULL");
  int rc = check_pool(&L->routed, "routed");
  if (rc) return rc;
  rc = check_pool(&L->shared, "shared");
  if (rc) return rc;
  if (L->shared.num_experts != 1) return fail(QMOE_ESHAPE, "shared.num_experts must be 1");
  if (L->shared.hidden != L->routed.hidden || L->shared.inter != L->routed.inter ||
      L->shared.bits != L->routed.bits)
    return fail(QMOE_ESHAPE, "shared and routed experts must have the same shape and bits");
  if (L->top_k < 1 || L->top_k > qmoe::kMaxTopK || L->top_k > L->routed.num_experts)
    return fail(QMOE_ESHAPE, "top_k must be in [1, min(E, %d)]", qmoe::kMaxTopK);
  if (L->routed.hidden > qmoe::kMaxRouterH)
    return fail(QMOE_ESHAPE, "hidden must be at most %d", qmoe::kMaxRouterH);
  if (!L->router || !aligned(L->router, 16)) return fail(QMOE_EALIGN, "router must be 16-byte aligned");
  if (!L->shared_gate || !aligned(L->shared_gate, 16))
    return fail(QMOE_EALIGN, "shared_gate must be 16-byte aligned");
  return QMOE_OK;
}

int check_qmat(const qmoe_qmat* W, int bits) {
  if (!W) return fail(QMOE_EINVAL, "W is NULL");
  if (W->rows < 0 || W->cols < 0) return fail(QMOE_EINVAL, "negative matrix size");
  if (W->cols < 64 || W->cols % 64) return fail(QMOE_ESHAPE, "cols must be a positive multiple of 64");
  const int maxc = bits == 4 ? qmoe::kMaxCols4 : qmoe::kMaxCols2;
  if (W->cols > maxc) return fail(QMOE_ESHAPE, "cols must be at most %d at %d bits", maxc, bits);
  if (W->rows > 0) {
    if (!W->codes || !W->sb) return fail(QMOE_EINVAL, "codes/sb is NULL");
    if (!aligned(W->codes, 16)) return fail(QMOE_EALIGN, "codes must be 16-byte aligned");
    if (!aligned(W->sb, 4)) return fail(QMOE_EALIGN, "sb must be 4-byte aligned");
  }
  return QMOE_OK;
}

}  // namespace

namespace qmoe {

int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];  // zero-initialised; 0 = not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

qmoe_expert_offsets expert_offsets(int hidden, int inter, int bits) {
  qmoe_expert_offsets o;
  const int64_t gu = (int64_t)inter * hidden * bits / 8;
  const int64_t dn = (int64_t)hidden * inter * bits / 8;
  const int64_t gsb = (int64_t)inter * (hidden / 64) * 4;
  const int64_t dsb = (int64_t)hidden * (inter / 64) * 4;
  o.gate_codes = 0;
  o.up_codes = gu;
  o.down_codes = 2 * gu;
  o.gate_sb = 2 * gu + dn;
  o.up_sb = o.gate_sb + gsb;
  o.down_sb = o.up_sb + gsb;
  o.total = o.down_sb + dsb;
  return o;
}

}  // namespace qmoe

extern "C" {

int qmoe_expert_layout(int32_t hidden, int32_t inter, int32_t bits, qmoe_expert_offsets* out) {
  if (!out) return fail(QMOE_EINVAL, "out is NULL");
  if (bits != 2 && bits != 4) return fail(QMOE_EINVAL, "bits must be 2 or 4");
  if (hidden < 64 || inter < 64 || hidden % 64 || inter % 64)
    return fail(QMOE_ESHAPE, "hidden and inter must be positive multiples of 64");
  *out = qmoe::expert_offsets(hidden, inter, bits);
  return QMOE_OK;
}

static int qgemv_common(const qmoe_qmat* W, const float* x, float* y, void* stream, int bits) {
  int rc = check_qmat(W, bits);
  if (rc) return rc;
  if (W->rows == 0) return QMOE_OK;
  if ((rc = check_vec(x, "x"))) return rc;
  if (!y) return fail(QMOE_EINVAL, "y is NULL");
  return hip_status(qmoe::launch_qgemv(bits, static_cast<const uint8_t*>(W->codes), W->sb, x, y,
                                       W->rows, W->cols, static_cast<hipStream_t>(stream)),
                    "qgemv launch");
}

int qgemv_w4(const qmoe_qmat* W, const float* x, float* y, void* stream) {
  return qgemv_common(W, x, y, stream, 4);
}

int qgemv_w2(const qmoe_qmat* W, const float* x, float* y, void* stream) {
  return qgemv_common(W, x, y, stream, 2);
}

int moe_router_topk(const uint16_t* router, const float* x, int32_t T, int32_t H, int32_t E,
                    int32_t K, float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  if (T < 0 || H < 0 || E < 0 || K < 0) return fail(QMOE_EINVAL, "negative size");
  if (H < 64 || H % 64 || H > qmoe::kMaxRouterH)
    return fail(QMOE_ESHAPE, "H must be a multiple of 64 in [64, %d]", qmoe::kMaxRouterH);
  if (E < 1 || E > qmoe::kMaxExperts) return fail(QMOE_ESHAPE, "E must be in [1, %d]", qmoe::kMaxExperts);
  if (K < 1 || K > E || K > qmoe::kMaxTopK) return fail(QMOE_ESHAPE, "K must be in [1, min(E, 8)]");
  if (T == 0) return QMOE_OK;
  if (!router || !aligned(router, 16)) return fail(QMOE_EALIGN, "router must be 16-byte aligned");
  int rc;
  if ((rc = check_vec(x, "x"))) return rc;
  if (!logits || !topk_idx || !topk_w) return fail(QMOE_EINVAL, "output pointer is NULL");
  return hip_status(qmoe::launch_router_topk(router, x, T, H, E, K, logits, topk_idx, topk_w,
                                             static_cast<hipStream_t>(stream)),
                    "router launch");
}

// [0, F): the single-launch path's state (F = ffn_fused_ws_bytes, a multiple of 256);
// [F, F + n*I*4): h of the two-launch path, so that calls with n > 1 never touch
// the state of the n == 1 calls that share the workspace
size_t qmoe_ffn_workspace_bytes(const qmoe_expert_pool* pool, int32_t n) {
  if (!pool || n < 0 || pool->inter < 0) return 0;
  return qmoe::ffn_fused_ws_bytes(*pool) + (size_t)n * (size_t)pool->inter * sizeof(float);
}

int expert_ffn_swiglu(const qmoe_expert_pool* pool, const int32_t* expert_idx, int32_t n,
                      const float* x, float* y, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_pool(pool, "pool");
  if (rc) return rc;
  if (n < 0) return fail(QMOE_EINVAL, "n must be >= 0");
  if (n > 65535) return fail(QMOE_ESHAPE, "n must be at most 65535");
  if (n == 0) return QMOE_OK;
  if (!expert_idx) return fail(QMOE_EINVAL, "expert_idx is NULL");
  if ((rc = check_vec(x, "x"))) return rc;
  if (!y) return fail(QMOE_EINVAL, "y is NULL");
  if (!ws || ws_bytes < qmoe_ffn_workspace_bytes(pool, n))
    return fail(QMOE_EWORKSPACE, "workspace needs %zu bytes", qmoe_ffn_workspace_bytes(pool, n));
  if (!aligned(ws, 16)) return fail(QMOE_EALIGN, "ws must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n == 1 && qmoe::ffn_fused_supported(*pool))
    return hip_status(qmoe::launch_ffn_fused(*pool, expert_idx, x, y, ws, s), "expert_ffn launch");
  float* h = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + qmoe::ffn_fused_ws_bytes(*pool));
  return hip_status(qmoe::launch_ffn(*pool, expert_idx, n, x, 0, y, h, s), "expert_ffn launch");
}

int moe_combine_residual_gate(const float* y_routed, const float* topk_w, const float* y_shared,
                              const uint16_t* shared_gate, const float* x, const float* residual,
                              float* out, int32_t H, int32_t K, void* stream) {
  if (H < 0 || K < 0) return fail(QMOE_EINVAL, "negative size");
  if (K > qmoe::kMaxTopK) return fail(QMOE_ESHAPE, "K must be at most %d", qmoe::kMaxTopK);
  if (H == 0) return QMOE_OK;
  if ((K > 0 && (!y_routed || !topk_w)) || !y_shared || !shared_gate || !x || !residual || !out)
    return fail(QMOE_EINVAL, "NULL pointer");
  return hip_status(qmoe::launch_combine(y_routed, topk_w, y_shared, shared_gate, x, residual, out,
                                         H, K, static_cast<hipStream_t>(stream)),
                    "combine launch");
}

size_t qmoe_workspace_bytes(const qmoe_layer* L, int32_t T) {
  if (!L || T < 1 || T > qmoe::kMaxBatch) return 0;
  if (T == 1) return qmoe::layer_workspace_bytes(*L);
  return qmoe::batched_workspace_bytes(*L, T);
}

int moe_layer_forward(const qmoe_layer* L, const float* x, const float* residual, float* out,
                      int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if ((rc = check_vec(x, "x"))) return rc;
  if (!residual || !out || !topk_idx || !topk_w) return fail(QMOE_EINVAL, "NULL pointer");
  if (out == x) return fail(QMOE_EINVAL, "out must not alias x");
  const size_t need = qmoe_workspace_bytes(L, 1);
  if (!ws || ws_bytes < need) return fail(QMOE_EWORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(QMOE_EALIGN, "ws must be 256-byte aligned");
  return hip_status(qmoe::launch_layer(*L, x, nullptr, 0.f, residual, out, topk_idx, topk_w, ws,
                                       static_cast<hipStream_t>(stream)),
                    "moe_layer_forward launch");
}

int moe_layer_forward_noalloc(const qmoe_layer* L, const float* x, const float* residual,
                              float* out, int32_t* topk_idx, float* topk_w, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if ((rc = check_vec(x, "x"))) return rc;
  if (!residual || !out || !topk_idx || !topk_w) return fail(QMOE_EINVAL, "NULL pointer");
  if (out == x) return fail(QMOE_EINVAL, "out must not alias x");
  const size_t need = qmoe_workspace_bytes(L, 1);
  if (need > qmoe::kNoAllocScratchBytes)
    return fail(QMOE_EWORKSPACE,
                "this layer needs %zu bytes of scratch; the allocation-free entry point has %zu "
                "(use moe_layer_forward with a workspace)",
                need, qmoe::kNoAllocScratchBytes);
  return hip_status(qmoe::launch_layer_noalloc(*L, x, residual, out, topk_idx, topk_w,
                                               static_cast<hipStream_t>(stream)),
                    "moe_layer_forward_noalloc launch");
}

int moe_layer_forward_norm(const qmoe_layer* L, const float* h, const float* norm_w, float eps,
                           float* out, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if ((rc = check_vec(h, "h"))) return rc;
  if ((rc = check_vec(norm_w, "norm_w"))) return rc;
  if (!(eps >= 0.0f)) return fail(QMOE_EINVAL, "eps must be >= 0");
  if (!out || !topk_idx || !topk_w) return fail(QMOE_EINVAL, "NULL pointer");
  const size_t need = qmoe_workspace_bytes(L, 1);
  if (!ws || ws_bytes < need) return fail(QMOE_EWORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(QMOE_EALIGN, "ws must be 256-byte aligned");
  return hip_status(qmoe::launch_layer(*L, h, norm_w, eps, h, out, topk_idx, topk_w, ws,
                                       static_cast<hipStream_t>(stream)),
                    "moe_layer_forward_norm launch");
}

size_t qmoe_stack_workspace_bytes(const qmoe_layer* layers, int32_t n_layers) {
  if (!layers || n_layers < 1) return 0;
  return qmoe::stack_workspace_bytes(layers[0], n_layers);
}

int moe_stack_forward(const qmoe_layer* layers, const float* const* norm_w, int32_t n_layers,
                      float eps, const float* h0, float* out, float* h_all, int32_t* topk_idx,
                      float* topk_w, int32_t flags, void* ws, size_t ws_bytes, void* stream) {
  if (!layers || !norm_w) return fail(QMOE_EINVAL, "layers or norm_w is NULL");
  if (flags & ~QMOE_STACK_PERSISTENT) return fail(QMOE_EINVAL, "unknown flags 0x%x", flags);
  if (n_layers < 1) return fail(QMOE_EINVAL, "n_layers must be >= 1");
  const qmoe_layer& L0 = layers[0];
  for (int l = 0; l < n_layers; ++l) {
    int rc = check_layer(&layers[l]);
    if (rc) return rc;
    const qmoe_layer& L = layers[l];
    if (L.routed.num_experts != L0.routed.num_experts || L.routed.hidden != L0.routed.hidden ||
        L.routed.inter != L0.routed.inter || L.routed.bits != L0.routed.bits ||
        L.top_k != L0.top_k)
      return fail(QMOE_ESHAPE, "layer %d differs in shape from layer 0", l);
    if ((rc = check_vec(norm_w[l], "norm_w[l]"))) return rc;
  }
  if (!(eps >= 0.0f)) return fail(QMOE_EINVAL, "eps must be >= 0");
  int rc = check_vec(h0, "h0");
  if (rc || (rc = check_vec(out, "out"))) return rc;
  if (h_all && (rc = check_vec(h_all, "h_all"))) return rc;
  if (h_all && (h_all == out || h_all == h0)) return fail(QMOE_EINVAL, "h_all must not alias h0 or out");
  if (!topk_idx || !topk_w) return fail(QMOE_EINVAL, "NULL pointer");
  const size_t need = qmoe_stack_workspace_bytes(layers, n_layers);
  if (!ws || ws_bytes < need) return fail(QMOE_EWORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(QMOE_EALIGN, "ws must be 256-byte aligned");
  return hip_status(qmoe::launch_stack(layers, norm_w, n_layers, eps, h0, out, h_all, topk_idx,
                                       topk_w, ws, (flags & QMOE_STACK_PERSISTENT) != 0,
                                       static_cast<hipStream_t>(stream)),
                    "moe_stack_forward launch");
}

int moe_layer_forward_batched(const qmoe_layer* L, const float* x, const float* residual,
                              float* out, int32_t T, int32_t* topk_idx, float* topk_w, void* ws,
                              size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 1 || T > qmoe::kMaxBatch) return fail(QMOE_ESHAPE, "T must be in [1, %d]", qmoe::kMaxBatch);
  if ((rc = check_vec(x, "x"))) return rc;
  if ((rc = check_vec(residual, "residual")) || (rc = check_vec(out, "out"))) return rc;
  if (!topk_idx || !topk_w) return fail(QMOE_EINVAL, "NULL pointer");
  if (out == x) return fail(QMOE_EINVAL, "out must not alias x");
  const size_t need = qmoe_workspace_bytes(L, T);
  if (!ws || ws_bytes < need) return fail(QMOE_EWORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(QMOE_EALIGN, "ws must be 256-byte aligned");
  return hip_status(qmoe::launch_layer_batched(*L, x, residual, out, T, topk_idx, topk_w, ws,
                                               static_cast<hipStream_t>(stream)),
                    "moe_layer_forward_batched launch");
}

int gdn_recurrent_step(float* state, const float* q, const float* k, const float* v, const float* alpha,
                       const float* beta, float* o, int32_t heads, int32_t dk, int32_t dv, void* stream) {
  if (heads < 0 || dv < 1) return fail(QMOE_ESHAPE, "heads must be >= 0 and dv >= 1");
  if (dk != 64 && dk != 128 && dk != 256) return fail(QMOE_ESHAPE, "dk must be 64, 128 or 256");
  if ((int64_t)heads * dv > (int64_t)1 << 30) return fail(QMOE_ESHAPE, "heads * dv too large");
  if (heads == 0) return QMOE_OK;
  int rc = check_vec(state, "state");
  if (rc || (rc = check_vec(q, "q")) || (rc = check_vec(k, "k"))) return rc;
  if (!v || !alpha || !beta || !o) return fail(QMOE_EINVAL, "NULL pointer");
  return hip_status(qmoe::launch_gdn_step(state, q, k, v, alpha, beta, o, heads, dk, dv,
                                          static_cast<hipStream_t>(stream)),
                    "gdn_recurrent_step launch");
}

static int check_attn_shape(int32_t Hq, int32_t Hkv, int32_t D, int32_t Tmax) {
  if (D != 64 && D != 128 && D != 256) return fail(QMOE_ESHAPE, "D must be 64, 128 or 256");
  if (Hkv < 1 || Hq < Hkv || Hq % Hkv || Hq / Hkv > 16)
    return fail(QMOE_ESHAPE, "Hq must be a multiple of Hkv, at most 16 query heads per KV head");
  if (Tmax < 1) return fail(QMOE_ESHAPE, "Tmax must be >= 1");
  return QMOE_OK;
}

size_t qmoe_attn_workspace_bytes(int32_t Hq, int32_t Hkv, int32_t D, int32_t Tmax) {
  if (check_attn_shape(Hq, Hkv, D, Tmax)) return 0;
  return qmoe::attn_workspace_bytes(Hq, Hkv, D, Tmax);
}

int attn_decode_step(const float* q, const float* k, const float* v, float* k_cache, float* v_cache,
                     int32_t Hq, int32_t Hkv, int32_t D, int32_t Tmax, int32_t pos, float theta,
                     int32_t rot_dim, float* o, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_attn_shape(Hq, Hkv, D, Tmax);
  if (rc) return rc;
  if (pos < 0 || pos >= Tmax) return fail(QMOE_ESHAPE, "pos must be in [0, Tmax)");
  if (rot_dim < 0 || rot_dim > D || rot_dim % 2) return fail(QMOE_ESHAPE, "rot_dim must be even, 0..D");
  if (!(theta > 0.0f)) return fail(QMOE_EINVAL, "theta must be > 0");
  if ((rc = check_vec(q, "q")) || (rc = check_vec(k, "k")) || (rc = check_vec(v, "v")) ||
      (rc = check_vec(k_cache, "k_cache")) || (rc = check_vec(v_cache, "v_cache")) ||
      (rc = check_vec(o, "o")))
    return rc;
  const size_t need = qmoe_attn_workspace_bytes(Hq, Hkv, D, Tmax);
  if (!ws || ws_bytes < need) return fail(QMOE_EWORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(QMOE_EALIGN, "ws must be 256-byte aligned");
  return hip_status(qmoe::launch_attn_decode(q, k, v, k_cache, v_cache, Hq, Hkv, D, Tmax, pos, theta,
                                             rot_dim, o, ws, static_cast<hipStream_t>(stream)),
                    "attn_decode_step launch");
}

int attn_decode_step_qgate(const float* qg, const float* k, const float* v, const float* q_norm_w,
                           const float* k_norm_w, float eps, float* k_cache, float* v_cache, int32_t Hq,
                           int32_t Hkv, int32_t D, int32_t Tmax, int32_t pos, float theta, int32_t rot_dim,
                           float* o, float* gate, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_attn_shape(Hq, Hkv, D, Tmax);
  if (rc) return rc;
  if (pos < 0 || pos >= Tmax) return fail(QMOE_ESHAPE, "pos must be in [0, Tmax)");
  if (rot_dim < 0 || rot_dim > D || rot_dim % 2) return fail(QMOE_ESHAPE, "rot_dim must be even, 0..D");
  if (!(theta > 0.0f)) return fail(QMOE_EINVAL, "theta must be > 0");
  if (!(eps >= 0.0f)) return fail(QMOE_EINVAL, "eps must be >= 0");
  if ((rc = check_vec(qg, "qg")) || (rc = check_vec(k, "k")) || (rc = check_vec(v, "v")) ||
      (rc = check_vec(k_cache, "k_cache")) || (rc = check_vec(v_cache, "v_cache")) ||
      (rc = check_vec(o, "o")))
    return rc;
  if ((q_norm_w && !aligned(q_norm_w, 4)) || (k_norm_w && !aligned(k_norm_w, 4)) || (gate && !aligned(gate, 4)))
    return fail(QMOE_EALIGN, "q_norm_w, k_norm_w and gate must be 4-byte aligned");
  const size_t need = qmoe_attn_workspace_bytes(Hq, Hkv, D, Tmax);
  if (!ws || ws_bytes < need) return fail(QMOE_EWORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(QMOE_EALIGN, "ws must be 256-byte aligned");
  return hip_status(qmoe::launch_attn_decode(qg, k, v, k_cache, v_cache, Hq, Hkv, D, Tmax, pos, theta,
                                             rot_dim, o, ws, static_cast<hipStream_t>(stream), true,
                                             q_norm_w, k_norm_w, eps, gate),
                    "attn_decode_step_qgate launch");
}

int rmsnorm_f32(const float* v, const float* w, float eps, int32_t n, float* out, void* stream) {
  if (n < 0) return fail(QMOE_EINVAL, "n must be >= 0");
  if (!(eps >= 0.0f)) return fail(QMOE_EINVAL, "eps must be >= 0");
  if (n == 0) return QMOE_OK;
  if (!v || !w || !out) return fail(QMOE_EINVAL, "NULL pointer");
  return hip_status(qmoe::launch_rmsnorm(v, w, eps, n, out, static_cast<hipStream_t>(stream)),
                    "rmsnorm launch");
}

int qmoe_stream_read(const void* buf, int64_t bytes, uint32_t key, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(QMOE_EINVAL, "bytes must be a non-negative multiple of 16");
  if (bytes == 0) return QMOE_OK;
  if (!buf || !aligned(buf, 16)) return fail(QMOE_EALIGN, "buf must be 16-byte aligned");
  if (!sink || !aligned(sink, 4)) return fail(QMOE_EALIGN, "sink must be 4-byte aligned");
  return hip_status(qmoe::launch_stream_read(buf, bytes, key, sink, static_cast<hipStream_t>(stream)),
                    "qmoe_stream_read launch");
}

int qmoe_offload_create(const qmoe_expert_pool* host_pool, int32_t n_slots, void* slot_mem,
                        qmoe_offload** out) {
  if (!out) return fail(QMOE_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_pool(host_pool, "host_pool");
  if (rc) return rc;
  if (n_slots < 1) return fail(QMOE_ESHAPE, "n_slots must be >= 1");
  if (!slot_mem) return fail(QMOE_EINVAL, "slot_mem is NULL");
  if (!aligned(slot_mem, 256)) return fail(QMOE_EALIGN, "slot_mem must be 256-byte aligned");
  rc = qmoe::offload_create(*host_pool, n_slots, slot_mem, out);
  if (rc) return fail(rc, "could not create the offload handle (pinned staging or events)");
  return QMOE_OK;
}

int qmoe_offload_destroy(qmoe_offload* handle) {
  if (!handle) return fail(QMOE_EINVAL, "handle is NULL");
  qmoe::offload_destroy(handle);
  return QMOE_OK;
}

int qmoe_offload_get_stats(const qmoe_offload* handle, qmoe_offload_stats* out) {
  if (!handle || !out) return fail(QMOE_EINVAL, "NULL pointer");
  qmoe::offload_stats(handle, out);
  return QMOE_OK;
}

size_t qmoe_offload_workspace_bytes(const qmoe_layer* L) {
  if (!L || L->top_k < 1 || L->routed.num_experts < 1 || L->routed.hidden < 1 || L->routed.inter < 1)
    return 0;
  return qmoe::offload_workspace_bytes(*L);
}

int moe_layer_forward_offload(qmoe_offload* handle, const qmoe_layer* L, const float* x,
                              const float* residual, float* out, int32_t* topk_idx, float* topk_w,
                              void* ws, size_t ws_bytes, void* stream, void* copy_stream) {
  if (!handle) return fail(QMOE_EINVAL, "handle is NULL");
  if (!L) return fail(QMOE_EINVAL, "layer is NULL");
  // the routed pool's base is unused (the experts are in the handle's host pool)
  qmoe_layer Lc = *L;
  Lc.routed.base = qmoe::offload_host_pool(handle).base;
  int rc = check_layer(&Lc);
  if (rc) return rc;
  const qmoe_expert_pool& hp = qmoe::offload_host_pool(handle);
  if (L->routed.num_experts != hp.num_experts || L->routed.hidden != hp.hidden ||
      L->routed.inter != hp.inter || L->routed.bits != hp.bits)
    return fail(QMOE_ESHAPE, "the layer's routed shape differs from the handle's host pool");
  if (L->top_k > qmoe::offload_slots(handle)) return fail(QMOE_ESHAPE, "n_slots must be >= top_k");
  if ((rc = check_vec(x, "x"))) return rc;
  if (!residual || !out || !topk_idx || !topk_w) return fail(QMOE_EINVAL, "NULL pointer");
  if (out == x) return fail(QMOE_EINVAL, "out must not alias x");
  const size_t need = qmoe_offload_workspace_bytes(L);
  if (!ws || ws_bytes < need) return fail(QMOE_EWORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(QMOE_EALIGN, "ws must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t cs = copy_stream ? static_cast<hipStream_t>(copy_stream) : s;
  return hip_status(qmoe::offload_layer(handle, Lc, x, residual, out, topk_idx, topk_w, ws, s, cs),
                    "moe_layer_forward_offload");
}

const char* qmoe_strerror(int status) {
  switch (status) {
    case QMOE_OK: return "ok";
    case QMOE_EINVAL: return "invalid argument";
    case QMOE_ESHAPE: return "unsupported shape";
    case QMOE_EALIGN: return "misaligned pointer or stride";
    case QMOE_EWORKSPACE: return "workspace too small";
    case QMOE_EHIP: return "HIP runtime error";
    case QMOE_EUNSUPPORTED: return "not supported";
    default: return "unknown status";
  }
}

const char* qmoe_last_error(void) { return g_last_error; }

}  // extern "C"
