"""Python binding of libqmoe (batch-1 quantized MoE expert forward on MI355X).

A thin ctypes layer over the C ABI declared in ``include/qmoe.h``: the functions
here have the same names as the C entry points, take torch tensors that live
on the GPU, marshal pointers and the current HIP stream, and raise
``QmoeError`` on a non-zero status.  Every step of the computation runs in the
library's HIP kernels; nothing here computes.  Importing this module fails
loudly if the library has not been built (run ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QMOE_LIBRARY=probe loads the instrumented build (phase timestamps in the fused
# layer; see build.py --probe) instead of the product library
LIB_PATH = os.path.join(_HERE, "libqmoe_probe.so" if os.environ.get("QMOE_LIBRARY") == "probe"
                        else "libqmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950); there is no fallback")

_lib = ctypes.CDLL(LIB_PATH)

QMOE_OK, QMOE_EINVAL, QMOE_ESHAPE, QMOE_EALIGN, QMOE_EWORKSPACE, QMOE_EHIP, QMOE_EUNSUPPORTED = \
    0, -1, -2, -3, -4, -5, -6


class QmoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_lib.qmoe_strerror(status).decode()} ({status}): "
                         f"{_lib.qmoe_last_error().decode()}")


class ExpertOffsets(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("gate_codes", "up_codes", "down_codes", "gate_sb", "up_sb", "down_sb", "total")]


class QMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("sb", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class ExpertPoolC(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("stride", ctypes.c_int64),
                ("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("bits", ctypes.c_int32)]


class LayerC(ctypes.Structure):
    _fields_ = [("routed", ExpertPoolC), ("shared", ExpertPoolC), ("router", ctypes.c_void_p),
                ("shared_gate", ctypes.c_void_p), ("top_k", ctypes.c_int32)]


class OffloadStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("calls", "hits", "misses", "bytes_copied")]


_vp, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
_SIGS = {
    "qmoe_expert_layout": ([_i32, _i32, _i32, ctypes.POINTER(ExpertOffsets)], ctypes.c_int),
    "qgemv_w4": ([ctypes.POINTER(QMat), _vp, _vp, _vp], ctypes.c_int),
    "qgemv_w2": ([ctypes.POINTER(QMat), _vp, _vp, _vp], ctypes.c_int),
    "moe_router_topk": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
    "expert_ffn_swiglu": ([ctypes.POINTER(ExpertPoolC), _vp, _i32, _vp, _vp, _vp, _sz, _vp],
                          ctypes.c_int),
    "qmoe_ffn_workspace_bytes": ([ctypes.POINTER(ExpertPoolC), _i32], _sz),
    "moe_combine_residual_gate": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp], ctypes.c_int),
    "moe_layer_forward": ([ctypes.POINTER(LayerC), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                          ctypes.c_int),
    "moe_layer_forward_noalloc": ([ctypes.POINTER(LayerC), _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_layer_forward_norm": ([ctypes.POINTER(LayerC), _vp, _vp, _f32, _vp, _vp, _vp, _vp, _sz, _vp],
                               ctypes.c_int),
    "moe_layer_forward_batched": ([ctypes.POINTER(LayerC), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz,
                                   _vp], ctypes.c_int),
    "qmoe_workspace_bytes": ([ctypes.POINTER(LayerC), _i32], _sz),
    "moe_stack_forward": ([ctypes.POINTER(LayerC), ctypes.POINTER(_vp), _i32, _f32, _vp, _vp, _vp, _vp,
                           _vp, _i32, _vp, _sz, _vp], ctypes.c_int),
    "qmoe_stack_workspace_bytes": ([ctypes.POINTER(LayerC), _i32], _sz),
    "qmoe_offload_create": ([ctypes.POINTER(ExpertPoolC), _i32, _vp, ctypes.POINTER(_vp)], ctypes.c_int),
    "qmoe_offload_destroy": ([_vp], ctypes.c_int),
    "qmoe_offload_get_stats": ([_vp, ctypes.POINTER(OffloadStats)], ctypes.c_int),
    "qmoe_offload_workspace_bytes": ([ctypes.POINTER(LayerC)], _sz),
    "moe_layer_forward_offload": ([_vp, ctypes.POINTER(LayerC), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp],
                                  ctypes.c_int),
    "qmoe_stream_read": ([_vp, ctypes.c_int64, ctypes.c_uint32, _vp, _vp], ctypes.c_int),
    "attn_decode_step_qgate": ([_vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32,
                                _i32, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "rmsnorm_f32": ([_vp, _vp, _f32, _i32, _vp, _vp], ctypes.c_int),
    "gdn_recurrent_step": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp], ctypes.c_int),
    "attn_decode_step": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _sz,
                          _vp], ctypes.c_int),
    "qmoe_attn_workspace_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "qmoe_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "qmoe_last_error": ([], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


def _check(rc, where):
    if rc != QMOE_OK:
        raise QmoeError(rc, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# data structures
# ---------------------------------------------------------------------------

def qmoe_expert_layout(hidden: int, inter: int, bits: int) -> dict:
    o = ExpertOffsets()
    _check(_lib.qmoe_expert_layout(hidden, inter, bits, ctypes.byref(o)), "qmoe_expert_layout")
    return {n: getattr(o, n) for n, _ in ExpertOffsets._fields_}


class ExpertPool:
    """E expert blocks resident in one uint8 GPU tensor, expert e at byte e*stride."""

    def __init__(self, buf: torch.Tensor, num_experts: int, hidden: int, inter: int, bits: int,
                 stride: int | None = None):
        lay = qmoe_expert_layout(hidden, inter, bits)
        self.stride = stride if stride is not None else (lay["total"] + 255) // 256 * 256
        if buf.dtype != torch.uint8 or buf.numel() < self.stride * (num_experts - 1) + lay["total"]:
            raise ValueError("pool buffer must be uint8 and hold every expert")
        self.buf, self.num_experts, self.hidden, self.inter, self.bits = buf, num_experts, hidden, inter, bits
        self.layout = lay

    @staticmethod
    def allocate(num_experts, hidden, inter, bits, device="cuda"):
        lay = qmoe_expert_layout(hidden, inter, bits)
        stride = (lay["total"] + 255) // 256 * 256
        buf = torch.empty(stride * num_experts, dtype=torch.uint8, device=device)
        return ExpertPool(buf, num_experts, hidden, inter, bits, stride)

    def c(self) -> ExpertPoolC:
        return ExpertPoolC(self.buf.data_ptr(), self.stride, self.num_experts, self.hidden,
                           self.inter, self.bits)

    def expert_bytes(self, e: int) -> torch.Tensor:
        o = e * self.stride
        return self.buf[o:o + self.layout["total"]]


class Layer:
    """One MoE layer: routed pool, shared expert (pool of 1), router and shared gate."""

    def __init__(self, routed: ExpertPool, shared: ExpertPool, router: torch.Tensor,
                 shared_gate: torch.Tensor, top_k: int):
        self.routed, self.shared, self.router, self.shared_gate, self.top_k = \
            routed, shared, router, shared_gate, top_k
        _ptr(router, None, "router")          # bf16 bits (torch.int16 or torch.bfloat16)
        _ptr(shared_gate, None, "shared_gate")

    def c(self) -> LayerC:
        return LayerC(self.routed.c(), self.shared.c(), self.router.data_ptr(),
                      self.shared_gate.data_ptr(), self.top_k)


def qmoe_workspace_bytes(layer: Layer, T: int = 1) -> int:
    return int(_lib.qmoe_workspace_bytes(ctypes.byref(layer.c()), T))


def qmoe_ffn_workspace_bytes(pool: ExpertPool, n: int) -> int:
    return int(_lib.qmoe_ffn_workspace_bytes(ctypes.byref(pool.c()), n))


def alloc_workspace(layer: Layer, T: int = 1) -> torch.Tensor:
    """A zero-filled workspace (the fused layer kernel requires zero on first use)."""
    n = qmoe_workspace_bytes(layer, T)
    if n == 0:
        raise ValueError("bad layer or batch size")
    return torch.zeros(n, dtype=torch.uint8, device=layer.routed.buf.device)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def _qgemv(fn, bits, codes, sb, x, y, rows, cols):
    if y is None:
        y = torch.empty(rows, dtype=torch.float32, device=x.device)
    m = QMat(_ptr(codes, None, "codes").value, _ptr(sb, None, "sb").value, rows, cols)
    _check(fn(ctypes.byref(m), _ptr(x, torch.float32, "x"), _ptr(y, torch.float32, "y"), _stream()),
           f"qgemv_w{bits}")
    return y


def qgemv_w4(codes, sb, x, y=None):
    """y = W x for a 4-bit matrix (codes uint8 [rows][cols/2], sb int32/uint32 [rows][cols/64])."""
    return _qgemv(_lib.qgemv_w4, 4, codes, sb, x, y, codes.shape[0], x.numel())


def qgemv_w2(codes, sb, x, y=None):
    """y = W x for a 2-bit matrix (codes uint8 [rows][cols/4])."""
    return _qgemv(_lib.qgemv_w2, 2, codes, sb, x, y, codes.shape[0], x.numel())


def moe_router_topk(router, x, k, logits=None, idx=None, w=None):
    """Router GEMV + softmax top-k for x [T][H]; returns (idx int32 [T][k], w [T][k], logits)."""
    x2 = x.reshape(-1, router.shape[1])
    T, H = x2.shape
    E = router.shape[0]
    dev = x.device
    logits = logits if logits is not None else torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = idx if idx is not None else torch.empty(T, k, dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty(T, k, dtype=torch.float32, device=dev)
    _check(_lib.moe_router_topk(_ptr(router, None, "router"), _ptr(x2, torch.float32, "x"), T, H, E, k,
                                _ptr(logits, torch.float32, "logits"), _ptr(idx, torch.int32, "idx"),
                                _ptr(w, torch.float32, "w"), _stream()), "moe_router_topk")
    return idx, w, logits


def expert_ffn_swiglu(pool: ExpertPool, expert_idx, x, y=None, ws=None):
    """y[i] = D_e(silu(G_e x) * U_e x) for e = expert_idx[i] (device int32).  ws: a
    workspace zero-filled before its first use and kept between calls (a fresh
    zero-filled one when None)."""
    n = expert_idx.numel()
    y = y if y is not None else torch.empty(n, pool.hidden, dtype=torch.float32, device=x.device)
    need = qmoe_ffn_workspace_bytes(pool, n)
    ws = ws if ws is not None else torch.zeros(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(_lib.expert_ffn_swiglu(ctypes.byref(pool.c()), _ptr(expert_idx, torch.int32, "expert_idx"), n,
                                  _ptr(x, torch.float32, "x"), _ptr(y, torch.float32, "y"),
                                  _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream()),
           "expert_ffn_swiglu")
    return y


def moe_combine_residual_gate(y_routed, topk_w, y_shared, shared_gate, x, residual, out=None):
    H = x.numel()
    K = topk_w.numel()
    out = out if out is not None else torch.empty(H, dtype=torch.float32, device=x.device)
    _check(_lib.moe_combine_residual_gate(_ptr(y_routed, torch.float32, "y_routed"),
                                          _ptr(topk_w, torch.float32, "topk_w"),
                                          _ptr(y_shared, torch.float32, "y_shared"),
                                          _ptr(shared_gate, None, "shared_gate"),
                                          _ptr(x, torch.float32, "x"), _ptr(residual, torch.float32, "residual"),
                                          _ptr(out, torch.float32, "out"), H, K, _stream()),
           "moe_combine_residual_gate")
    return out


def moe_layer_forward(layer: Layer, x, residual=None, out=None, idx=None, w=None, ws=None):
    """One fused launch: returns (out [H], idx int32 [K], w [K])."""
    residual = residual if residual is not None else x
    dev = x.device
    out = out if out is not None else torch.empty_like(x)
    idx = idx if idx is not None else torch.empty(layer.top_k, dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty(layer.top_k, dtype=torch.float32, device=dev)
    if ws is None:
        raise ValueError("pass a persistent workspace from alloc_workspace(layer)")
    _check(_lib.moe_layer_forward(ctypes.byref(layer.c()), _ptr(x, torch.float32, "x"),
                                  _ptr(residual, torch.float32, "residual"), _ptr(out, torch.float32, "out"),
                                  _ptr(idx, torch.int32, "idx"), _ptr(w, torch.float32, "w"),
                                  _ptr(ws, None, "ws"), ws.numel(), _stream()), "moe_layer_forward")
    return out, idx, w


def moe_layer_forward_noalloc(layer: Layer, x, residual=None, out=None, idx=None, w=None):
    """moe_layer_forward with the library's own device scratch (no workspace, no
    allocation inside the call when out/idx/w are given): returns (out, idx, w)."""
    residual = residual if residual is not None else x
    dev = x.device
    out = out if out is not None else torch.empty_like(x)
    idx = idx if idx is not None else torch.empty(layer.top_k, dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty(layer.top_k, dtype=torch.float32, device=dev)
    _check(_lib.moe_layer_forward_noalloc(ctypes.byref(layer.c()), _ptr(x, torch.float32, "x"),
                                          _ptr(residual, torch.float32, "residual"),
                                          _ptr(out, torch.float32, "out"), _ptr(idx, torch.int32, "idx"),
                                          _ptr(w, torch.float32, "w"), _stream()),
           "moe_layer_forward_noalloc")
    return out, idx, w


def moe_layer_forward_norm(layer: Layer, h, norm_w, eps=1e-6, out=None, idx=None, w=None, ws=None):
    """One fused launch of h + MoE(rmsnorm(h)): returns (out [H], idx int32 [K], w [K]).
    out may be h itself (an in-place step of the residual stream)."""
    dev = h.device
    out = out if out is not None else torch.empty_like(h)
    idx = idx if idx is not None else torch.empty(layer.top_k, dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty(layer.top_k, dtype=torch.float32, device=dev)
    if ws is None:
        raise ValueError("pass a persistent workspace from alloc_workspace(layer)")
    _check(_lib.moe_layer_forward_norm(ctypes.byref(layer.c()), _ptr(h, torch.float32, "h"),
                                       _ptr(norm_w, torch.float32, "norm_w"), eps,
                                       _ptr(out, torch.float32, "out"), _ptr(idx, torch.int32, "idx"),
                                       _ptr(w, torch.float32, "w"), _ptr(ws, None, "ws"), ws.numel(),
                                       _stream()), "moe_layer_forward_norm")
    return out, idx, w


class Stack:
    """Layers of one shape with their RMSNorm weights, marshalled once for
    moe_stack_forward (the C structs and the pointer table live as long as this)."""

    def __init__(self, layers, norm_ws):
        if len(layers) != len(norm_ws) or not layers:
            raise ValueError("one RMSNorm weight per layer, at least one layer")
        self.layers, self.norm_ws = list(layers), list(norm_ws)
        self.n = len(self.layers)
        self.top_k = self.layers[0].top_k
        self._lc = (LayerC * self.n)(*[L.c() for L in self.layers])
        self._nw = (_vp * self.n)(*[_ptr(w, torch.float32, "norm_w").value for w in self.norm_ws])


def qmoe_stack_workspace_bytes(stack: Stack) -> int:
    return int(_lib.qmoe_stack_workspace_bytes(stack._lc, stack.n))


def alloc_stack_workspace(stack: Stack) -> torch.Tensor:
    """A zero-filled workspace for moe_stack_forward (it also serves moe_layer_forward)."""
    n = qmoe_stack_workspace_bytes(stack)
    if n == 0:
        raise ValueError("bad stack")
    return torch.zeros(n, dtype=torch.uint8, device=stack.layers[0].routed.buf.device)


QMOE_STACK_PERSISTENT = 1


def moe_stack_forward(stack: Stack, h0, eps=1e-6, out=None, h_all=None, idx=None, w=None, ws=None,
                      persistent=False):
    """h <- h + MoE_l(rmsnorm(h, norm_w[l])) through every layer of the stack: one
    fused launch per layer, or (persistent) one launch per 32 layers.  Returns
    (out [H], idx int32 [n, K], w [n, K]).  h_all: a float tensor [n, H] that
    receives every layer's output, or None."""
    dev = h0.device
    out = out if out is not None else torch.empty_like(h0)
    idx = idx if idx is not None else torch.empty(stack.n, stack.top_k, dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty(stack.n, stack.top_k, dtype=torch.float32, device=dev)
    if ws is None:
        raise ValueError("pass a persistent workspace from alloc_stack_workspace(stack)")
    ha = None if h_all is None else _ptr(h_all, torch.float32, "h_all")
    _check(_lib.moe_stack_forward(stack._lc, stack._nw, stack.n, eps, _ptr(h0, torch.float32, "h0"),
                                  _ptr(out, torch.float32, "out"), ha, _ptr(idx, torch.int32, "idx"),
                                  _ptr(w, torch.float32, "w"), QMOE_STACK_PERSISTENT if persistent else 0,
                                  _ptr(ws, None, "ws"), ws.numel(), _stream()),
           "moe_stack_forward")
    return out, idx, w


def moe_layer_forward_batched(layer: Layer, x, residual=None, out=None, idx=None, w=None, ws=None):
    """T tokens x [T][H]: returns (out [T][H], idx [T][K], w [T][K])."""
    T = x.shape[0]
    residual = residual if residual is not None else x
    dev = x.device
    out = out if out is not None else torch.empty_like(x)
    idx = idx if idx is not None else torch.empty(T, layer.top_k, dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty(T, layer.top_k, dtype=torch.float32, device=dev)
    if ws is None:
        raise ValueError("pass a persistent workspace from alloc_workspace(layer, T)")
    _check(_lib.moe_layer_forward_batched(ctypes.byref(layer.c()), _ptr(x, torch.float32, "x"),
                                          _ptr(residual, torch.float32, "residual"),
                                          _ptr(out, torch.float32, "out"), T,
                                          _ptr(idx, torch.int32, "idx"), _ptr(w, torch.float32, "w"),
                                          _ptr(ws, None, "ws"), ws.numel(), _stream()),
           "moe_layer_forward_batched")
    return out, idx, w


def gdn_recurrent_step(state, q, k, v, alpha, beta, o=None):
    """One GatedDeltaNet decode step for every head, state [heads][dv][dk] updated in
    place: returns o [heads][dv]."""
    heads, dv, dk = state.shape
    o = o if o is not None else torch.empty(heads, dv, dtype=torch.float32, device=state.device)
    for t, n, shp in ((q, "q", (heads, dk)), (k, "k", (heads, dk)), (v, "v", (heads, dv)),
                      (alpha, "alpha", (heads,)), (beta, "beta", (heads,)), (o, "o", (heads, dv))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    _check(_lib.gdn_recurrent_step(_ptr(state, torch.float32, "state"), _ptr(q, torch.float32, "q"),
                                   _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"),
                                   _ptr(alpha, torch.float32, "alpha"), _ptr(beta, torch.float32, "beta"),
                                   _ptr(o, torch.float32, "o"), heads, dk, dv, _stream()), "gdn_recurrent_step")
    return o


def qmoe_attn_workspace_bytes(Hq: int, Hkv: int, D: int, Tmax: int) -> int:
    return int(_lib.qmoe_attn_workspace_bytes(Hq, Hkv, D, Tmax))


def attn_decode_step(q, k, v, k_cache, v_cache, pos, theta=1e7, rot_dim=None, o=None, ws=None):
    """One decode token of grouped-query attention with RoPE: writes row pos of the
    caches ([Hkv][Tmax][D]) and returns o [Hq][D]."""
    Hq, D = q.shape
    Hkv, Tmax, D2 = k_cache.shape
    rot_dim = D if rot_dim is None else rot_dim
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(k.shape) != (Hkv, D) \
            or tuple(v.shape) != (Hkv, D):
        raise ValueError("q [Hq][D], k and v [Hkv][D], caches [Hkv][Tmax][D]")
    o = o if o is not None else torch.empty(Hq, D, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(256, qmoe_attn_workspace_bytes(Hq, Hkv, D, Tmax)), dtype=torch.uint8,
                         device=q.device)
    _check(_lib.attn_decode_step(_ptr(q, torch.float32, "q"), _ptr(k, torch.float32, "k"),
                                 _ptr(v, torch.float32, "v"), _ptr(k_cache, torch.float32, "k_cache"),
                                 _ptr(v_cache, torch.float32, "v_cache"), Hq, Hkv, D, Tmax, pos, theta,
                                 rot_dim, _ptr(o, torch.float32, "o"), _ptr(ws, None, "ws"), ws.numel(),
                                 _stream()), "attn_decode_step")
    return o


def attn_decode_step_qgate(qg, k, v, k_cache, v_cache, pos, theta=1e7, rot_dim=None, q_norm_w=None,
                           k_norm_w=None, eps=1e-6, o=None, gate=None, ws=None):
    """attn_decode_step from the interleaved query projection qg [Hq][2D] (per head:
    D query values, then D gate values), with optional per-head RMS normalisation
    of q and k.  Returns (o [Hq][D], gate [Hq][D])."""
    Hq, D2x = qg.shape
    Hkv, Tmax, D = k_cache.shape
    rot_dim = D if rot_dim is None else rot_dim
    if D2x != 2 * D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(k.shape) != (Hkv, D) \
            or tuple(v.shape) != (Hkv, D):
        raise ValueError("qg [Hq][2D], k and v [Hkv][D], caches [Hkv][Tmax][D]")
    for wgt in (q_norm_w, k_norm_w):
        if wgt is not None and tuple(wgt.shape) != (D,):
            raise ValueError("norm weights are [D]")
    o = o if o is not None else torch.empty(Hq, D, dtype=torch.float32, device=qg.device)
    gate = gate if gate is not None else torch.empty(Hq, D, dtype=torch.float32, device=qg.device)
    if ws is None:
        ws = torch.empty(max(256, qmoe_attn_workspace_bytes(Hq, Hkv, D, Tmax)), dtype=torch.uint8,
                         device=qg.device)
    _check(_lib.attn_decode_step_qgate(
        _ptr(qg, torch.float32, "qg"), _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"),
        _ptr(q_norm_w, torch.float32, "q_norm_w") if q_norm_w is not None else None,
        _ptr(k_norm_w, torch.float32, "k_norm_w") if k_norm_w is not None else None, eps,
        _ptr(k_cache, torch.float32, "k_cache"), _ptr(v_cache, torch.float32, "v_cache"), Hq, Hkv, D, Tmax,
        pos, theta, rot_dim, _ptr(o, torch.float32, "o"), _ptr(gate, torch.float32, "gate"),
        _ptr(ws, None, "ws"), ws.numel(), _stream()), "attn_decode_step_qgate")
    return o, gate


class Offload:
    """A host-tier expert cache: the routed experts in pinned host memory (an
    ExpertPool whose buf is a pinned CPU tensor) and n_slots expert slots in HBM.
    Destroyed with the object (or by close())."""

    def __init__(self, host_pool: ExpertPool, n_slots: int, slot_mem: torch.Tensor | None = None):
        if host_pool.buf.is_cuda or not host_pool.buf.is_pinned():
            raise ValueError("the host pool must be a pinned CPU tensor")
        self.host_pool = host_pool
        self.n_slots = n_slots
        self.slot_mem = slot_mem if slot_mem is not None else torch.empty(
            n_slots * host_pool.stride, dtype=torch.uint8, device="cuda")
        if self.slot_mem.numel() < n_slots * host_pool.stride:
            raise ValueError("slot_mem too small")
        h = _vp()
        _check(_lib.qmoe_offload_create(ctypes.byref(host_pool.c()), n_slots, _ptr(self.slot_mem, None, "slot_mem"),
                                        ctypes.byref(h)), "qmoe_offload_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            _lib.qmoe_offload_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def stats(self) -> dict:
        st = OffloadStats()
        _check(_lib.qmoe_offload_get_stats(self._h, ctypes.byref(st)), "qmoe_offload_get_stats")
        return {n: int(getattr(st, n)) for n, _ in OffloadStats._fields_}


def qmoe_offload_workspace_bytes(layer: Layer) -> int:
    return int(_lib.qmoe_offload_workspace_bytes(ctypes.byref(layer.c())))


def moe_layer_forward_offload(off: Offload, layer: Layer, x, residual=None, out=None, idx=None, w=None,
                              ws=None, copy_stream=None):
    """One layer whose routed experts are in off's host pool (layer.routed describes
    that pool).  Returns (out, idx, w).  Waits on the host for the routing."""
    residual = residual if residual is not None else x
    dev = x.device
    out = out if out is not None else torch.empty_like(x)
    idx = idx if idx is not None else torch.empty(layer.top_k, dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty(layer.top_k, dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(qmoe_offload_workspace_bytes(layer), dtype=torch.uint8, device=dev)
    cs = ctypes.c_void_p(copy_stream.cuda_stream) if copy_stream is not None else None
    _check(_lib.moe_layer_forward_offload(off._h, ctypes.byref(layer.c()), _ptr(x, torch.float32, "x"),
                                          _ptr(residual, torch.float32, "residual"),
                                          _ptr(out, torch.float32, "out"), _ptr(idx, torch.int32, "idx"),
                                          _ptr(w, torch.float32, "w"), _ptr(ws, None, "ws"), ws.numel(),
                                          _stream(), cs), "moe_layer_forward_offload")
    return out, idx, w


def qmoe_stream_read(buf, nbytes=None, key=0xA5A5A5A5, sink=None):
    """One read-only streaming launch over nbytes of buf (default: all of it);
    returns the sink tensor (written only if the xor of the data equals key)."""
    nbytes = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    sink = sink if sink is not None else torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check(_lib.qmoe_stream_read(_ptr(buf, None, "buf"), nbytes, key, _ptr(sink, None, "sink"), _stream()),
           "qmoe_stream_read")
    return sink


def rmsnorm_f32(v, weight, eps=1e-6, out=None):
    out = out if out is not None else torch.empty_like(v)
    _check(_lib.rmsnorm_f32(_ptr(v, torch.float32, "v"), _ptr(weight, torch.float32, "w"), eps, v.numel(),
                            _ptr(out, torch.float32, "out"), _stream()), "rmsnorm_f32")
    return out


def raw_lib():
    """The ctypes handle (for tests of the C ABI itself)."""
    return _lib
