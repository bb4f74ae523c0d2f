"""CPU oracle for the batch-1 quantized MoE expert forward (TEST INFRASTRUCTURE).

This package is a plain, slow, obviously-correct float64 numpy statement of what
the HIP path computes.  It is test infrastructure: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It imports numpy and the standard library only, and shares no code,
tables or constants with the HIP library (``bit_dequant_gemv_amd``) or with the
input generators (``synth``).

Sources (web pages about Flash-MoE; cited by title and section):

* [PK] "flash-moe 소개" on the PyTorch Korea user group forum
  (discuss.pytorch.kr, topic 9315), sections "Qwen3.5-397B-A17B 모델 아키텍처"
  (model architecture), "FMA 최적화 역양자화 커널" (FMA-optimised dequant kernel),
  "손으로 작성한 Metal 컴퓨트 셰이더" (hand-written Metal shaders) and
  "레이어당 파이프라인 상세 구조" (per-layer pipeline).
* [GN] GeekNews topic 27758, "Flash-MoE - 노트북에서 3,970억 파라미터 모델을 실행",
  sections "모델 아키텍처" and "핵심 기술".
* [ML] mrlatte.net story "3970억 파라미터 AI를 48GB 맥북에서? …", section
  "기술적 인사이트" (technical insight).

Readings of the pages where they are silent (each listed in the design notes):

* The quantized layout is not described on the pages.  The canonical layout
  used here: codes row-major, element (n, k) in bits ``(k*bits) % 8`` upward
  of byte ``(k*bits)//8`` of row n (least-significant first); one u32 per
  (row, group of 64 input columns) holding the bf16 scale in bits 0-15 and the
  bf16 bias in bits 16-31.  Group size 64 along the input dimension.
* Codes are unsigned (0..2**bits-1) with no zero point: the page's formula is
  ``nibble * scale + bias``.
* Softmax + top-K: descending logit, ties to the lower expert index; weights
  are the softmax of the selected logits (the full softmax renormalised over
  the selection, which is the same number).
* SwiGLU: silu on the gate projection, times the up projection.
* Combine: ``out = residual + sum_i w_i * y_i + sigmoid(g . x) * y_shared``;
  the sigmoid gate scales the shared expert only.
* RMSNorm: ``v / sqrt(mean(v^2) + eps) * w``.
* GatedDeltaNet: the pages name a scale, a matrix-vector product and a rank-1
  update of a 128x128 state per head; read as the delta rule with a decay gate
  (``gdn_step``), with q, k, v and the two gates given.
* Full attention: the pages name Q@K^T, softmax, scores@V and RoPE.  Read as one
  decode token of grouped-query attention with scale 1/sqrt(D) over a key/value
  cache, rotate-half RoPE on the first rot_dim dimensions of q and k
  (``attn_decode``).

Parity status of each function is stated in its docstring; every function here
is pinned by a test in ``tests/test_oracle_pins.py`` against hand-built cases,
closed forms, brute force or exact rational arithmetic.
"""

from __future__ import annotations

import math

import numpy as np

GROUP = 64  # quantisation group along the input dimension (see module notes)

__all__ = [
    "GROUP",
    "bf16_bits_to_f64",
    "expert_offsets",
    "expert_bytes",
    "expert_views",
    "unpack_codes",
    "unpack_sb",
    "dequant",
    "qgemv",
    "router_logits",
    "router_topk",
    "topk_tolerance",
    "silu",
    "sigmoid",
    "expert_ffn",
    "combine_residual_gate",
    "moe_layer",
    "moe_layer_batched",
    "rmsnorm",
    "moe_stack",
    "gdn_step",
    "rope",
    "attn_decode",
    "deinterleave_q",
    "head_rmsnorm",
    "attn_decode_qgate",
    "rel_l2",
]


# --------------------------------------------------------------------------
# Exact conversions
# --------------------------------------------------------------------------

def bf16_bits_to_f64(u16) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 value is the upper half of an IEEE binary32 value, so shifting the
    16 bits into the top of a 32-bit word and reinterpreting is exact.
    """
    a = np.asarray(u16, dtype=np.uint16)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Expert block layout (canonical)
# --------------------------------------------------------------------------

def expert_offsets(hidden: int, inter: int, bits: int) -> dict:
    """Byte offsets of the six tensors inside one expert block.

    Order: gate codes, up codes, down codes, gate sb, up sb, down sb.
    gate/up are ``inter x hidden`` (out x in); down is ``hidden x inter``.
    The page [PK] "SSD 전문가 스트리밍" gives ~6.75 MB per 4-bit expert; with
    hidden 4096 and 4 bytes of scale+bias per group of 64 this pins inter=1024
    (checked in the tests).
    """
    if bits not in (2, 4):
        raise ValueError("bits must be 2 or 4")
    if hidden % GROUP or inter % GROUP:
        raise ValueError("hidden and inter must be multiples of 64")
    gu_codes = inter * hidden * bits // 8
    d_codes = hidden * inter * bits // 8
    gu_sb = inter * (hidden // GROUP) * 4
    d_sb = hidden * (inter // GROUP) * 4
    off = {}
    pos = 0
    for name, size in (("gate_codes", gu_codes), ("up_codes", gu_codes), ("down_codes", d_codes),
                       ("gate_sb", gu_sb), ("up_sb", gu_sb), ("down_sb", d_sb)):
        off[name] = (pos, size)
        pos += size
    off["total"] = pos
    return off


def expert_bytes(hidden: int, inter: int, bits: int) -> int:
    return expert_offsets(hidden, inter, bits)["total"]


def expert_views(block: np.ndarray, hidden: int, inter: int, bits: int) -> dict:
    """Split one expert block (uint8) into (codes, sb) for gate, up and down."""
    block = np.ascontiguousarray(block, dtype=np.uint8).reshape(-1)
    off = expert_offsets(hidden, inter, bits)
    if block.size < off["total"]:
        raise ValueError("expert block too small")

    def codes(name, rows, cols):
        o, s = off[name + "_codes"]
        return block[o:o + s].reshape(rows, cols * bits // 8)

    def sb(name, rows, cols):
        o, s = off[name + "_sb"]
        return block[o:o + s].view(np.uint32).reshape(rows, cols // GROUP)

    return {
        "gate": (codes("gate", inter, hidden), sb("gate", inter, hidden)),
        "up": (codes("up", inter, hidden), sb("up", inter, hidden)),
        "down": (codes("down", hidden, inter), sb("down", hidden, inter)),
    }


# --------------------------------------------------------------------------
# Dequantisation and GEMV   ([PK] "FMA 최적화 역양자화 커널")
# --------------------------------------------------------------------------

def unpack_codes(codes: np.ndarray, cols: int, bits: int) -> np.ndarray:
    """Unsigned codes q[n, k] from the packed bytes (canonical LSB-first order).

    q[n, k] = (byte[n, (k*bits)//8] >> ((k*bits) % 8)) & (2**bits - 1).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows = codes.shape[0]
    if codes.shape[1] * 8 != cols * bits:
        raise ValueError("codes row length does not match cols*bits/8")
    k = np.arange(cols)
    byte_idx = (k * bits) // 8
    shift = ((k * bits) % 8).astype(np.uint8)
    q = (codes[:, byte_idx] >> shift[None, :]) & np.uint8((1 << bits) - 1)
    assert q.shape == (rows, cols)
    return q.astype(np.int64)


def unpack_sb(sb: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-(row, group) scale and bias from the interleaved u32 words.

    Bits 0-15 hold the bf16 scale, bits 16-31 the bf16 bias.
    """
    sb = np.asarray(sb, dtype=np.uint32)
    scale = bf16_bits_to_f64((sb & np.uint32(0xFFFF)).astype(np.uint16))
    bias = bf16_bits_to_f64((sb >> np.uint32(16)).astype(np.uint16))
    return scale, bias


def dequant(codes: np.ndarray, sb: np.ndarray, cols: int, bits: int) -> np.ndarray:
    """W[n, k] = q[n, k] * scale[n, k // 64] + bias[n, k // 64]   (float64).

    This is the affine group dequantisation the page [PK] section
    "FMA 최적화 역양자화 커널" writes as ``nibble * scale + bias`` (unsigned code,
    no zero point).
    """
    q = unpack_codes(codes, cols, bits)
    scale, bias = unpack_sb(sb)
    if scale.shape != (q.shape[0], cols // GROUP):
        raise ValueError("sb shape must be [rows][cols/64]")
    g = np.arange(cols) // GROUP
    return q.astype(np.float64) * scale[:, g] + bias[:, g]


def qgemv(codes: np.ndarray, sb: np.ndarray, x: np.ndarray, bits: int) -> np.ndarray:
    """y = dequant(W) @ x in float64 -- the plain definition of the quantized GEMV.

    The page's FMA rearrangement ``fma(nibble, scale*x, bias*x)`` ([PK]
    "FMA 최적화 역양자화 커널") reaches the same value in exact arithmetic; the
    tests check that identity in rational arithmetic.
    """
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    W = dequant(codes, sb, x.size, bits)
    return W @ x


# --------------------------------------------------------------------------
# Router, softmax and top-K   ([PK] "레이어당 파이프라인 상세 구조": router in
# CMD2, then "softmax + topK" on the host)
# --------------------------------------------------------------------------

def router_logits(router_bf16: np.ndarray, x: np.ndarray) -> np.ndarray:
    """logits[e] = sum_h W_r[e, h] * x[h] with the router stored [E][H] (bf16)."""
    Wr = bf16_bits_to_f64(router_bf16)
    return Wr @ np.asarray(x, dtype=np.float64).reshape(-1)


def router_topk(logits: np.ndarray, k: int, decide_in=np.float32):
    """Top-k experts and their renormalised softmax weights.

    The selection order is descending logit with ties to the lower index.  The
    comparison is taken on the logits rounded to ``decide_in`` (float32, the
    precision the GPU decides in); the weights are the float64 softmax over the
    selected float64 logits, which equals the full softmax renormalised over
    the selection.
    Returns (idx int64[k], w float64[k]).
    """
    logits = np.asarray(logits, dtype=np.float64).reshape(-1)
    E = logits.size
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    key = logits.astype(decide_in) if decide_in is not None else logits
    order = sorted(range(E), key=lambda e: (-float(key[e]), e))
    idx = np.array(order[:k], dtype=np.int64)
    sel = logits[idx]
    ex = np.exp(sel - sel.max())
    return idx, ex / ex.sum()


def topk_tolerance(router_bf16: np.ndarray, x: np.ndarray, n_terms: int | None = None) -> np.ndarray:
    """Per-expert bound on the float32 error of a GPU logit.

    tau[e] = 4 * 2**-24 * sqrt(H) * sum_h |W_r[e, h] * x[h]|: a generous
    statistical bound for an fp32 dot product of H terms.  Two logits closer
    than tau may legitimately be ordered differently by an fp32 kernel.
    """
    Wr = bf16_bits_to_f64(router_bf16)
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    H = n_terms if n_terms is not None else x.size
    return 4.0 * 2.0 ** -24 * math.sqrt(H) * (np.abs(Wr) @ np.abs(x))


# --------------------------------------------------------------------------
# Expert FFN with SwiGLU   ([PK] "손으로 작성한 Metal 컴퓨트 셰이더": fused SwiGLU)
# --------------------------------------------------------------------------

def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """silu(z) = z * sigmoid(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def expert_ffn(block: np.ndarray, x: np.ndarray, hidden: int, inter: int, bits: int,
               return_intermediates: bool = False):
    """y = D @ (silu(G @ x) * (U @ x)) for one quantized expert (float64)."""
    v = expert_views(block, hidden, inter, bits)
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    a = qgemv(*v["gate"], x, bits)
    u = qgemv(*v["up"], x, bits)
    h = silu(a) * u
    y = qgemv(*v["down"], h, bits)
    if return_intermediates:
        return y, {"a": a, "u": u, "h": h}
    return y


# --------------------------------------------------------------------------
# Combine + residual + sigmoid gate   ([PK] "손으로 작성한 Metal 컴퓨트 셰이더":
# the combine of the weighted experts with the residual and the sigmoid gate is
# one fused kernel there)
# --------------------------------------------------------------------------

def combine_residual_gate(y_routed: np.ndarray, w: np.ndarray, y_shared: np.ndarray,
                          shared_gate_bf16: np.ndarray, x: np.ndarray,
                          residual: np.ndarray) -> np.ndarray:
    """out = residual + sum_i w_i * y_routed[i] + sigmoid(g . x) * y_shared."""
    y_routed = np.asarray(y_routed, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    g = bf16_bits_to_f64(shared_gate_bf16).reshape(-1)
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    gamma = sigmoid(g @ x)
    return (np.asarray(residual, dtype=np.float64).reshape(-1)
            + w @ y_routed.reshape(w.size, -1)
            + gamma * np.asarray(y_shared, dtype=np.float64).reshape(-1))


# --------------------------------------------------------------------------
# One MoE layer at batch 1
# --------------------------------------------------------------------------

def moe_layer(get_expert, shared_block: np.ndarray, router_bf16: np.ndarray,
              shared_gate_bf16: np.ndarray, x: np.ndarray, residual: np.ndarray,
              hidden: int, inter: int, bits: int, top_k: int,
              force_idx=None, return_details: bool = False):
    """Router -> softmax/top-K -> K routed experts + shared expert -> combine.

    ``get_expert(e)`` returns the uint8 block of routed expert ``e`` so that
    only the selected experts need to exist on the host.  ``force_idx`` runs
    the layer with a given expert set (used when an fp32 near-tie makes the
    set ambiguous); the weights are then the softmax over those logits.
    """
    logits = router_logits(router_bf16, x)
    if force_idx is None:
        idx, w = router_topk(logits, top_k)
    else:
        idx = np.asarray(force_idx, dtype=np.int64)
        sel = logits[idx]
        ex = np.exp(sel - sel.max())
        w = ex / ex.sum()
    ys = np.stack([expert_ffn(get_expert(int(e)), x, hidden, inter, bits) for e in idx])
    y_sh = expert_ffn(shared_block, x, hidden, inter, bits)
    out = combine_residual_gate(ys, w, y_sh, shared_gate_bf16, x, residual)
    if return_details:
        return out, {"logits": logits, "idx": idx, "w": w, "y_routed": ys, "y_shared": y_sh}
    return out


def moe_layer_batched(get_expert, shared_block, router_bf16, shared_gate_bf16, X, residual,
                      hidden, inter, bits, top_k):
    """Batched decode: row t is ``moe_layer`` on token t (grouping is not part
    of the definition; the GPU's per-expert token groups are an implementation
    detail)."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    R = np.atleast_2d(np.asarray(residual, dtype=np.float64))
    return np.stack([moe_layer(get_expert, shared_block, router_bf16, shared_gate_bf16,
                               X[t], R[t], hidden, inter, bits, top_k) for t in range(X.shape[0])])


# --------------------------------------------------------------------------
# RMSNorm   ([PK] "손으로 작성한 Metal 컴퓨트 셰이더": RMS normalisation in two
# passes, a sum-of-squares reduction and then the scaling)
# --------------------------------------------------------------------------

def rmsnorm(v: np.ndarray, w: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) * w."""
    v = np.asarray(v, dtype=np.float64).reshape(-1)
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    return v / math.sqrt(float(np.mean(v * v)) + eps) * w


def moe_stack(layers, h0: np.ndarray, hidden, inter, bits, top_k, eps=1e-6):
    """Decoder MoE stack at batch 1: for each layer, x = rmsnorm(h, w_l) and
    h = moe_layer_l(x, residual=h).  ``layers`` yields dicts with keys
    get_expert, shared_block, router, shared_gate, norm_w."""
    h = np.asarray(h0, dtype=np.float64).reshape(-1)
    for L in layers:
        x = rmsnorm(h, L["norm_w"], eps)
        h = moe_layer(L["get_expert"], L["shared_block"], L["router"], L["shared_gate"],
                      x, h, hidden, inter, bits, top_k)
    return h


# --------------------------------------------------------------------------
# GatedDeltaNet recurrence   ([PK] "Accelerate BLAS를 이용한 선형 어텐션 가속" /
# [GN] "핵심 기술", "Accelerate BLAS 활용":
# the linear-attention layers update a 128x128 state per head, 64 heads, with a
# scale, a matrix-vector product and a rank-1 update; [PK] architecture: 45 of
# the 60 layers are GatedDeltaNet layers)
# --------------------------------------------------------------------------

def gdn_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: np.ndarray,
             beta: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """One token of the gated delta rule for every head.

    S: [heads][dk][dv], the state: S[h]^T k is the value the head recalls for the
    key k.  q, k: [heads][dk]; v: [heads][dv]; alpha (decay) and beta (write
    strength): [heads].  Per head, in the order of the pages' three BLAS calls:
      S <- alpha S                      (scale)
      u  = S^T k                        (matrix-vector: what the key recalls now)
      S <- S + k (beta (v - u))^T       (rank-1 update: move that recall toward v)
      o  = S^T q                        (the read-out of the updated state)
    The pages name the operations only; this is the delta rule with a decay gate,
    taking q, k, v, alpha and beta as given (their projections, normalisation and
    the gates' nonlinearities come before the recurrence).  Returns (S', o).
    """
    S = np.array(S, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64).reshape(-1)
    beta = np.asarray(beta, dtype=np.float64).reshape(-1)
    heads = S.shape[0]
    o = np.zeros((heads, S.shape[2]))
    for h in range(heads):
        S[h] = alpha[h] * S[h]
        u = S[h].T @ k[h]
        S[h] = S[h] + np.outer(k[h], beta[h] * (v[h] - u))
        o[h] = S[h].T @ q[h]
    return S, o


# --------------------------------------------------------------------------
# Full-attention decode   ([PK] Metal shaders: GPU attention -- Q@K^T, softmax,
# scores@V -- and RoPE; architecture: 15 of the 60 layers are full attention)
# --------------------------------------------------------------------------

def rope(x: np.ndarray, pos: int, theta: float, rot_dim: int) -> np.ndarray:
    """Rotary position embedding of every row of x ([rows][D]) at position pos:
    the first rot_dim dimensions are split in halves (a, b) and each pair
    (a_i, b_i) is rotated by the angle pos * theta^(-2i/rot_dim); the other
    dimensions pass through."""
    x = np.array(x, dtype=np.float64)
    half = rot_dim // 2
    ang = pos * theta ** (-2.0 * np.arange(half) / rot_dim)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half].copy(), x[..., half:rot_dim].copy()
    x[..., :half] = a * c - b * s
    x[..., half:rot_dim] = b * c + a * s
    return x


def attn_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, K: np.ndarray, V: np.ndarray,
                pos: int, theta: float, rot_dim: int):
    """One decode token of grouped-query attention over a key/value cache.

    q: [Hq][D]; k, v: [Hkv][D] (this token's); K, V: [Hkv][T][D] caches with
    T > pos.  q and k are rotated at position pos, the rotated k and v go to row
    pos of the caches, and query head h attends to rows 0..pos of KV head
    h // (Hq / Hkv): o_h = sum_t softmax_t(q_h . K_t / sqrt(D)) V_t.
    Returns (o [Hq][D], K', V')."""
    q = rope(q, pos, theta, rot_dim)
    kr = rope(k, pos, theta, rot_dim)
    K = np.array(K, dtype=np.float64)
    V = np.array(V, dtype=np.float64)
    K[:, pos] = kr
    V[:, pos] = np.asarray(v, dtype=np.float64)
    hq, D = q.shape
    group = hq // K.shape[0]
    o = np.zeros((hq, D))
    for h in range(hq):
        g = h // group
        s = K[g, :pos + 1] @ q[h] / math.sqrt(D)
        p = np.exp(s - s.max())
        o[h] = (p / p.sum()) @ V[g, :pos + 1]
    return o, K, V


def deinterleave_q(qg: np.ndarray, D: int) -> tuple[np.ndarray, np.ndarray]:
    """The query projection's output with the query and its gate interleaved by
    head: row h of qg ([Hq][2D]) holds head h's D query values followed by its D
    gate values.  Returns (q [Hq][D], gate [Hq][D]).

    [PK] "손으로 작성한 Metal 컴퓨트 셰이더" lists RoPE fused with a
    de-interleave of Q; the page gives no layout, and this per-head
    [query | gate] split is the reading taken (the gate half is handed on, not
    applied: the page does not say what uses it)."""
    qg = np.asarray(qg, dtype=np.float64)
    if qg.shape[-1] != 2 * D:
        raise ValueError("qg rows must hold 2*D values")
    return qg[..., :D].copy(), qg[..., D:].copy()


def head_rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMS normalisation of every row of x ([rows][D]) over its D values:
    x / sqrt(mean(x^2) + eps) * w, with one weight vector w [D] for all rows
    ([PK] "손으로 작성한 Metal 컴퓨트 셰이더": the K normalisation fused with
    RoPE; the weight form is read as a plain multiply, as for the layer's RMSNorm)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def attn_decode_qgate(qg: np.ndarray, k: np.ndarray, v: np.ndarray, K: np.ndarray, V: np.ndarray,
                      pos: int, theta: float, rot_dim: int, q_norm_w=None, k_norm_w=None,
                      eps: float = 1e-6):
    """One decode token of grouped-query attention from the interleaved query
    projection: q and gate de-interleaved from qg, q and k RMS-normalised per head
    when a weight is given (None: no normalisation), then ``attn_decode`` (RoPE,
    cache append, attention).  Returns (o [Hq][D], gate [Hq][D], K', V')."""
    D = np.asarray(k).shape[-1]
    q, gate = deinterleave_q(qg, D)
    if q_norm_w is not None:
        q = head_rmsnorm(q, q_norm_w, eps)
    k = np.asarray(k, dtype=np.float64)
    if k_norm_w is not None:
        k = head_rmsnorm(k, k_norm_w, eps)
    o, K2, V2 = attn_decode(q, k, v, K, V, pos, theta, rot_dim)
    return o, gate, K2, V2


# --------------------------------------------------------------------------
# Comparison helpers
# --------------------------------------------------------------------------

def rel_l2(a, b) -> float:
    """||a - b||_2 / ||b||_2  (b is the reference)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    nb = float(np.linalg.norm(b))
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b)) / nb

