/*
 * qmoe.h -- C ABI of libqmoe: batch-1 quantized mixture-of-experts expert forward
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are web pages about the Flash-MoE engine; cited by
 * page title and section):
 *   [PK] "flash-moe 소개", PyTorch Korea user group forum (discuss.pytorch.kr
 *        topic 9315): sections "FMA 최적화 역양자화 커널" (affine dequant
 *        w = nibble*scale + bias and its FMA rearrangement), "손으로 작성한 Metal
 *        컴퓨트 셰이더" (4/2-bit dequant matrix-vector kernels, fused SwiGLU,
 *        two-stage RMSNorm, fused MoE combine + residual + sigmoid gate),
 *        "레이어당 파이프라인 상세 구조" (router in the second command buffer,
 *        softmax + top-K, expert forward + combine deferred in the third) and
 *        "Qwen3.5-397B-A17B 모델 아키텍처" (512 experts, K=4 active plus one
 *        shared expert, hidden 4096).
 *
 * Conventions for every function below
 *   - Array pointers are DEVICE pointers owned by the caller (for example torch
 *     tensors); struct pointers (qmoe_qmat*, qmoe_layer*, ...) are HOST
 *     pointers read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously; no call synchronises the device, allocates or
 *     frees memory.  Scratch memory is a caller-provided workspace (except for
 *     moe_layer_forward_noalloc, whose scratch is a library-held device array).
 *   - Arguments are validated on the host before anything is enqueued; a
 *     negative qmoe_status is returned and nothing is launched.  A launch
 *     failure returns QMOE_EHIP.  Device faults surface at the caller's next
 *     synchronisation, as with any stream API.  qmoe_last_error() gives a
 *     thread-local text for the last failure.
 *   - Buffers must stay alive until the stream has passed the call.
 *   - Expert indices read on the device outside [0, E) are not dereferenced:
 *     the outputs that depend on them are set to NaN.
 *
 * Quantized matrix layout (the pages do not give one; this library's reading)
 *   codes : row-major, cols*bits/8 bytes per row; element k of a row is the
 *           unsigned code in bits (k*bits)%8 upward of byte (k*bits)/8
 *           (least-significant first).  16-byte aligned.
 *   sb    : uint32 [rows][cols/64]; bits 0-15 = bf16 scale, bits 16-31 = bf16
 *           bias of the group of 64 input columns.  4-byte aligned.
 *   value : W[n][k] = q[n][k] * scale[n][k/64] + bias[n][k/64]     ([PK] FMA section)
 *
 * Expert block (one expert, qmoe_expert_layout gives the offsets):
 *   gate codes, up codes, down codes, gate sb, up sb, down sb, in that order;
 *   gate and up are inter x hidden (out x in), down is hidden x inter.
 *   hidden 4096 / inter 1024: 7,077,888 B at 4 bits (the pages' ~6.75 MB per
 *   expert), 3,932,160 B at 2 bits.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QMOE_OK = 0,
  QMOE_EINVAL = -1,      /* null pointer, bad enum value, negative size */
  QMOE_ESHAPE = -2,      /* sizes not supported (not a multiple of 64, too large, K > E) */
  QMOE_EALIGN = -3,      /* a pointer or stride is not aligned as documented */
  QMOE_EWORKSPACE = -4,  /* workspace missing or smaller than qmoe_workspace_bytes() */
  QMOE_EHIP = -5,        /* the HIP runtime reported an error */
  QMOE_EUNSUPPORTED = -6 /* a valid request the library does not implement */
} qmoe_status;

/* Byte offsets of the six tensors inside one expert block, and its size. */
typedef struct {
  int64_t gate_codes, up_codes, down_codes, gate_sb, up_sb, down_sb, total;
} qmoe_expert_offsets;

/* One quantized matrix (rows = outputs, cols = inputs). */
typedef struct {
  const void* codes;   /* device, [rows][cols*bits/8] bytes, 16-byte aligned */
  const uint32_t* sb;  /* device, [rows][cols/64] scale|bias words */
  int32_t rows, cols;
} qmoe_qmat;

/* Experts resident in HBM: expert e's block starts at base + e*stride. */
typedef struct {
  const void* base;     /* device, 256-byte aligned */
  int64_t stride;       /* bytes between experts: >= block size, multiple of 256 */
  int32_t num_experts;  /* E */
  int32_t hidden;       /* H, multiple of 64 */
  int32_t inter;        /* I, multiple of 64 */
  int32_t bits;         /* 2 or 4 */
} qmoe_expert_pool;

/* One MoE layer: E routed experts, one shared expert, router and shared gate. */
typedef struct {
  qmoe_expert_pool routed;      /* E routed experts */
  qmoe_expert_pool shared;      /* num_experts must be 1; same hidden/inter/bits */
  const uint16_t* router;       /* device bf16 [E][H]: logits = router . x */
  const uint16_t* shared_gate;  /* device bf16 [H]: gamma = sigmoid(shared_gate . x) */
  int32_t top_k;                /* K, 1 <= K <= min(E, 8) */
} qmoe_layer;

/* Pure host: offsets of an expert block for (hidden, inter, bits).  No device use. */
int qmoe_expert_layout(int32_t hidden, int32_t inter, int32_t bits, qmoe_expert_offsets* out);

/*
 * y[rows] = W x with W 4-bit ([PK] "손으로 작성한 Metal 컴퓨트 셰이더": 4-bit dequant
 * matrix-vector product; "FMA 최적화 역양자화 커널": w = nibble*scale + bias).
 * x: device float[cols]; y: device float[rows] (written).  cols a multiple of 64
 * and at most 8192; rows >= 0.  fp32 accumulation.
 */
int qgemv_w4(const qmoe_qmat* W, const float* x, float* y, void* stream);

/* As qgemv_w4 for 2-bit codes (values 0..3); cols at most 16384. */
int qgemv_w2(const qmoe_qmat* W, const float* x, float* y, void* stream);

/*
 * Router GEMV + softmax + top-K for T tokens ([PK] "레이어당 파이프라인 상세 구조":
 * routing in the second command buffer, then softmax + top-K; here both on the GPU).
 *   router  : device bf16 [E][H]
 *   x       : device float [T][H]
 *   logits  : device float [T][E] (written; also the kernel's scratch)
 *   topk_idx: device int32 [T][K] (written): descending logit, ties to the lower index
 *   topk_w  : device float [T][K] (written): softmax over the K selected logits
 * 1 <= K <= min(E, 8), H a multiple of 64 (at most 8192), E <= 4096.
 */
int moe_router_topk(const uint16_t* router, const float* x, int32_t T, int32_t H, int32_t E,
                    int32_t K, float* logits, int32_t* topk_idx, float* topk_w, void* stream);

/*
 * Expert FFN with fused SwiGLU for n experts of a pool, chosen by a device index list
 * ([PK] Metal shaders: dequant matvec + fused SwiGLU):
 *   y[i] = D_e (silu(G_e x) * (U_e x)),  e = expert_idx[i]
 *   expert_idx: device int32 [n]; x: device float [H]; y: device float [n][H] (written);
 *   an index outside [0, num_experts) gives a row of NaN.
 *   ws: device workspace of at least qmoe_ffn_workspace_bytes(pool, n) bytes, 16-byte
 *   aligned, ZERO-FILLED before its first use.  With n == 1 and a shape the
 *   single-launch kernel takes (hidden 1024/2048/4096, inter 256/512/1024) the call
 *   is one launch that keeps state in the workspace from call to call (a call
 *   counter, values tagged with the call number, as moe_layer_forward does), so the
 *   caller must not write to its first qmoe_ffn_workspace_bytes(pool, 0) bytes
 *   afterwards; calls that share a workspace must be stream-ordered.  Word 1 (int32
 *   at byte offset 4) is then a status word: nonzero if a bounded wait inside the
 *   kernel ran out (the output of that call is undefined).  Otherwise two launches
 *   use the rest of the workspace as scratch.
 */
int expert_ffn_swiglu(const qmoe_expert_pool* pool, const int32_t* expert_idx, int32_t n,
                      const float* x, float* y, void* ws, size_t ws_bytes, void* stream);
size_t qmoe_ffn_workspace_bytes(const qmoe_expert_pool* pool, int32_t n);

/*
 * Fused combine ([PK] Metal shaders: MoE combine + residual + sigmoid gate, one kernel):
 *   out = residual + sum_i topk_w[i] * y_routed[i] + sigmoid(shared_gate . x) * y_shared
 *   y_routed: device float [K][H]; topk_w: device float [K]; y_shared, x, residual,
 *   out: device float [H]; shared_gate: device bf16 [H].  out may alias residual.
 */
int moe_combine_residual_gate(const float* y_routed, const float* topk_w, const float* y_shared,
                              const uint16_t* shared_gate, const float* x, const float* residual,
                              float* out, int32_t H, int32_t K, void* stream);

/*
 * One MoE layer at batch 1 in a single kernel launch: router GEMV -> top-K ->
 * K routed + 1 shared SwiGLU expert (expert-indexed, no host round trip) ->
 * combine with residual and sigmoid gate.  ([PK] "레이어당 파이프라인 상세 구조":
 * the routing, expert forward and combine the reference splits over two command
 * buffers and a host top-K.)
 *   x, residual: device float [H]; out: device float [H] (written; must not alias x,
 *   may alias residual); topk_idx/topk_w: device [K] (written).
 *   ws: device workspace of at least qmoe_workspace_bytes(L, 1) bytes, 256-byte
 *   aligned, ZERO-FILLED before its first use.  The library keeps state in it from
 *   call to call (a call counter, a status word, values tagged with the call
 *   number), so the caller must not write to it afterwards.  Calls that share a
 *   workspace must be stream-ordered.  Word 1 (int32 at byte offset 4) is a status
 *   word: nonzero if a bounded wait inside the kernel ran out (the output of that
 *   call is then undefined); the caller may read it after the stream passes.
 */
int moe_layer_forward(const qmoe_layer* L, const float* x, const float* residual, float* out,
                      int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward for callers that cannot allocate memory or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and result as moe_layer_forward without ws/ws_bytes:
 * the workspace is a device-global array of QMOE_NOALLOC_SCRATCH_BYTES (1 MiB) per
 * GPU, held by the library until the process ends.  Nothing is allocated or
 * freed by the call.  The first call on a device looks the array up (and, unless
 * the stream is being captured, enqueues a fill of zeros before the layer).
 * Errors: as moe_layer_forward; QMOE_EWORKSPACE if the layer's workspace
 * (qmoe_workspace_bytes(L, 1)) exceeds QMOE_NOALLOC_SCRATCH_BYTES.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * state (a call counter and values tagged with it): calls on one GPU must be
 * ordered (one stream, or event dependencies); calls that overlap race.
 */
#define QMOE_NOALLOC_SCRATCH_BYTES (1u << 20)
int moe_layer_forward_noalloc(const qmoe_layer* L, const float* x, const float* residual,
                              float* out, int32_t* topk_idx, float* topk_w, void* stream);

/*
 * The same layer with its input RMS-normalised inside the launch: a decoder
 * stack step h <- h + MoE(rmsnorm(h)) ([PK] Metal shaders: two-stage RMS
 * normalisation; "지연 GPU 전문가 실행 (Deferred CMD3)": the normalised combine
 * output feeds the next layer).  x = h / sqrt(mean(h^2) + eps) * norm_w,
 * residual = h.
 *   h: device float [H] (the residual stream); norm_w: device float [H];
 *   out: device float [H] (written; may alias h); topk_idx/topk_w as above;
 *   ws: as for moe_layer_forward (the same workspace may serve both).
 */
int moe_layer_forward_norm(const qmoe_layer* L, const float* h, const float* norm_w, float eps,
                           float* out, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * A decoder stack for one token: for l = 0 .. n_layers-1,
 * h <- h + MoE_l(rmsnorm(h, norm_w[l])), each layer as in moe_layer_forward_norm
 * ([PK] "지연 GPU 전문가 실행 (Deferred CMD3)": the combined, normalised output
 * of one layer is the next layer's input with no host round trip).
 *   layers: host array [n_layers]; every layer has the same E, H, I, bits and K;
 *   norm_w: host array [n_layers] of device float [H] (16-byte aligned);
 *   h0: device float [H], the input; out: device float [H], the output (may alias h0);
 *   h_all: device float [n_layers][H], each layer's output, or NULL (must not alias
 *   h0 or out);
 *   topk_idx/topk_w: device [n_layers][K] (written);
 *   flags: 0, or QMOE_STACK_PERSISTENT: up to 32 layers per launch, the workgroups
 *   staying resident from layer to layer (each layer's output reaches the next
 *   through the workspace; the next layer's router rows, gate vector and norm
 *   weight load during the current layer's tail).  Both give the same result bit
 *   for bit.  Without the flag each layer is one fused launch, which measures
 *   faster on MI355X: the device-side hand-off costs as much as a kernel boundary,
 *   and the layer loop compiles to a slower kernel;
 *   ws: at least qmoe_stack_workspace_bytes(layers, n_layers) bytes, 256-byte
 *   aligned, zero-filled before its first use; it may serve moe_layer_forward
 *   calls too, but no two calls may use it at the same time.
 * Errors: as moe_layer_forward_norm; QMOE_ESHAPE if a layer's shape differs from
 * layer 0's; QMOE_EINVAL for unknown flags.  Word 1 of the workspace is the status
 * word of moe_layer_forward.
 */
#define QMOE_STACK_PERSISTENT 1
int moe_stack_forward(const qmoe_layer* layers, const float* const* norm_w, int32_t n_layers,
                      float eps, const float* h0, float* out, float* h_all, int32_t* topk_idx,
                      float* topk_w, int32_t flags, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for moe_stack_forward (0 if layers is NULL or n_layers < 1). */
size_t qmoe_stack_workspace_bytes(const qmoe_layer* layers, int32_t n_layers);

/*
 * Batched decode of T tokens through one layer (row t equals moe_layer_forward on
 * token t): tokens are grouped per routed expert (histogram, scan, stable scatter)
 * so each active expert's weights are read once per batch.
 *   x, residual, out: device float [T][H], 16-byte aligned (out must not alias x; it
 *   may alias residual);
 *   topk_idx/topk_w: device [T][K] (written).
 *   ws: at least qmoe_workspace_bytes(L, T) bytes, 256-byte aligned, zero-filled
 *   before its first use (the same workspace may serve moe_layer_forward).
 *   1 <= T <= 256.
 */
int moe_layer_forward_batched(const qmoe_layer* L, const float* x, const float* residual,
                              float* out, int32_t T, int32_t* topk_idx, float* topk_w, void* ws,
                              size_t ws_bytes, void* stream);

/* Workspace bytes for moe_layer_forward (T == 1) or moe_layer_forward_batched. */
size_t qmoe_workspace_bytes(const qmoe_layer* L, int32_t T);

/*
 * One decode step of the GatedDeltaNet recurrence for every head ([PK] "Accelerate
 * BLAS를 이용한 선형 어텐션 가속": per linear-attention layer, 64 heads of a 128x128
 * state updated by a scale, a matrix-vector product and a rank-1 update).  With the state S of a head
 * as [dk][dv] (S^T k recalls the value stored at key k):
 *   S <- alpha S;  u = S^T k;  S <- S + k (beta (v - u))^T;  o = S^T q.
 *   state: device float [heads][dv][dk], updated in place; row j of head h holds
 *          column j of that head's S (contiguous over the keys), 16-byte aligned;
 *   q, k: device float [heads][dk] (16-byte aligned); v: device float [heads][dv];
 *   alpha, beta: device float [heads]; o: device float [heads][dv] (written).
 *   dk: 64, 128 or 256; dv >= 1; heads >= 0 (0: nothing is done).
 * q, k, v and the gates are taken as given: projections, normalisation and the
 * gates' nonlinearities come before the recurrence.  Errors: QMOE_ESHAPE for a bad
 * shape, QMOE_EINVAL / QMOE_EALIGN for a missing or misaligned pointer.
 */
int gdn_recurrent_step(float* state, const float* q, const float* k, const float* v,
                       const float* alpha, const float* beta, float* o, int32_t heads,
                       int32_t dk, int32_t dv, void* stream);

/*
 * One decode token of grouped-query attention with rotary position embedding
 * ([PK] Metal shaders: GPU attention -- Q@K^T, softmax, scores@V -- and RoPE;
 * architecture: 15 of the 60 layers are full attention):
 *   q, k <- rope(q, pos), rope(k, pos): on the first rot_dim dimensions, the pairs
 *           (x_i, x_{i + rot_dim/2}) turn by pos * theta^(-2i/rot_dim); the rest pass;
 *   k_cache[g][pos], v_cache[g][pos] <- k[g], v[g];
 *   o[h] = sum_{t <= pos} softmax_t(q[h] . k_cache[g][t] / sqrt(D)) v_cache[g][t],
 *          g = h / (Hq / Hkv).
 *   q: device float [Hq][D]; k, v: device float [Hkv][D] (this token's, before RoPE);
 *   k_cache, v_cache: device float [Hkv][Tmax][D], row pos written, rows < pos read;
 *   o: device float [Hq][D] (written); all 16-byte aligned.
 *   D: 64, 128 or 256; Hq a multiple of Hkv with Hq / Hkv <= 16; 0 <= pos < Tmax;
 *   rot_dim even, 0..D; theta > 0.
 *   ws: at least qmoe_attn_workspace_bytes(Hq, Hkv, D, Tmax) bytes, 256-byte aligned
 *   (scratch: no state is kept between calls).
 * Errors: QMOE_ESHAPE for a bad shape or position, QMOE_EINVAL / QMOE_EALIGN /
 * QMOE_EWORKSPACE for bad pointers, theta or workspace.
 */
int attn_decode_step(const float* q, const float* k, const float* v, float* k_cache,
                     float* v_cache, int32_t Hq, int32_t Hkv, int32_t D, int32_t Tmax, int32_t pos,
                     float theta, int32_t rot_dim, float* o, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * attn_decode_step from the query projection's output, with the steps the page
 * fuses into its RoPE kernel ([PK] "손으로 작성한 Metal 컴퓨트 셰이더": RoPE fused
 * with the Q de-interleave and the K normalisation):
 *   q[h], gate[h] <- qg[h][0:D], qg[h][D:2D]  (each head's row holds its D query
 *                                               values, then its D gate values);
 *   q[h] <- q[h] / sqrt(mean(q[h]^2) + eps) * q_norm_w   (if q_norm_w is not NULL);
 *   k[g] <- k[g] / sqrt(mean(k[g]^2) + eps) * k_norm_w   (if k_norm_w is not NULL);
 *   then RoPE, the cache append and the attention of attn_decode_step.
 *   qg: device float [Hq][2D], 16-byte aligned; q_norm_w, k_norm_w: device float [D] or
 *   NULL; gate: device float [Hq][D] (written: the de-interleaved gate halves, handed
 *   on unapplied) or NULL; every other argument as for attn_decode_step (the same
 *   workspace size).  eps >= 0.
 */
int attn_decode_step_qgate(const float* qg, const float* k, const float* v, const float* q_norm_w,
                           const float* k_norm_w, float eps, float* k_cache, float* v_cache, int32_t Hq,
                           int32_t Hkv, int32_t D, int32_t Tmax, int32_t pos, float theta, int32_t rot_dim,
                           float* o, float* gate, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for attn_decode_step (0 for a bad shape). */
size_t qmoe_attn_workspace_bytes(int32_t Hq, int32_t Hkv, int32_t D, int32_t Tmax);

/*
 * Host-tier expert offload ([PK] "SSD 전문가 스트리밍과 "OS 신뢰" 원칙" and
 * "레이어당 파이프라인 상세 구조": the selected experts of each layer are read from
 * storage after a host-side top-K, the popular ones kept by a cache).  For layers
 * whose routed experts do not fit in HBM: the routed pool lives in pinned host
 * memory, and an LRU cache of n_slots expert slots in HBM keeps the recently used
 * ones.  Per token: router + top-K on the GPU; the K indices come back to the host
 * (the only synchronisation, on an event); the shared expert's FFN runs meanwhile;
 * missing experts are copied host-to-device on copy_stream into the least recently
 * used slots; then the routed FFN on the slots and the combine.  The result equals
 * moe_layer_forward's up to rounding (the stand-alone kernels run, not the fused
 * one).
 *
 * qmoe_offload_create: host_pool describes the routed experts with base = a
 *   PINNED HOST pointer (hipHostMalloc), the same stride rules as a device pool;
 *   slot_mem: device memory of n_slots * host_pool->stride bytes, 256-byte aligned,
 *   owned by the caller; n_slots >= 1.  *out receives a handle (host memory the
 *   library allocates here, freed by qmoe_offload_destroy).
 * moe_layer_forward_offload: L->shared, L->router, L->shared_gate and L->top_k are
 *   used as in moe_layer_forward; L->routed must have the host pool's shape and
 *   its base is ignored.  x, residual, out, topk_idx, topk_w as in moe_layer_forward.
 *   ws: device, at least qmoe_offload_workspace_bytes(L), 256-byte aligned (scratch).
 *   copy_stream: a hipStream_t for the copies (NULL: stream).  The call waits on the
 *   host for the router's indices, so it cannot be captured in a graph.  Calls on
 *   one handle must come from one host thread at a time.  n_slots must be >= top_k.
 * Errors: QMOE_EINVAL / QMOE_EALIGN / QMOE_ESHAPE for bad arguments, QMOE_EHIP for a
 * runtime failure.  qmoe_offload_get_stats: calls, expert hits and misses, bytes
 * copied since creation.
 */
typedef struct qmoe_offload qmoe_offload;
typedef struct {
  uint64_t calls, hits, misses, bytes_copied;
} qmoe_offload_stats;
int qmoe_offload_create(const qmoe_expert_pool* host_pool, int32_t n_slots, void* slot_mem,
                        qmoe_offload** out);
int qmoe_offload_destroy(qmoe_offload* handle);
int qmoe_offload_get_stats(const qmoe_offload* handle, qmoe_offload_stats* out);
size_t qmoe_offload_workspace_bytes(const qmoe_layer* L);
int moe_layer_forward_offload(qmoe_offload* handle, const qmoe_layer* L, const float* x,
                              const float* residual, float* out, int32_t* topk_idx, float* topk_w,
                              void* ws, size_t ws_bytes, void* stream, void* copy_stream);

/*
 * RMSNorm ([PK] Metal shaders: two-stage RMS normalisation):
 *   out = v / sqrt(mean(v^2) + eps) * w;  v, w, out: device float [n]; out may alias v.
 */
int rmsnorm_f32(const float* v, const float* w, float eps, int32_t n, float* out, void* stream);

/*
 * Streaming-read calibration: one launch that reads `bytes` of buf with 16-byte
 * non-temporal loads and computes nothing, to measure the HBM bandwidth a
 * single launch can reach for a given number of bytes (the weight streams of
 * the layer kernels are read once per call, so their attainable rate depends on
 * the bytes per launch).  The xor of everything read is stored to sink[0] only
 * if it equals `key` (it keeps the loads alive; pass any value).
 *   buf: device, 16-byte aligned; bytes: a multiple of 16 (0: nothing is done);
 *   sink: device uint32 [1].
 */
int qmoe_stream_read(const void* buf, int64_t bytes, uint32_t key, uint32_t* sink, void* stream);

/* Static text for a status code; thread-local detail of the last failure. */
const char* qmoe_strerror(int status);
const char* qmoe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
