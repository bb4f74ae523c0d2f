"""Seeded synthetic inputs for the quantized MoE layer (shared by both sides).

This module holds no arithmetic of the method: it only draws random numbers and
places them in the canonical expert layout.  Both the oracle side (tests) and
the GPU side (tests, bench) take their inputs from here.

Every tensor is a stream of the counter-based generator Philox4x32-10
(J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11), keyed by (seed, tensor id).  Word ``n``
of a stream is lane ``n % 4`` of the Philox output for counter
``(n // 4 low 32 bits, n // 4 high 32 bits, 0, 0)``.  The same definition is
implemented on the device in ``synth/csrc/synth.hip`` so that large pools can
be generated in HBM while the host regenerates only the experts it checks; a
GPU test checks the two implementations bit for bit.

Value mappings (all exactly reproducible on both sides):

* codes: the stream's bytes, little-endian within each word -- i.i.d. uniform
  nibbles / 2-bit codes whatever the packing;
* uniform(lo, hi): element i uses word i: ``u = (w >> 8) * 2**-24`` (exact),
  ``v = f32(lo) + f32(u * f32(hi - lo))`` with both operations rounded to
  binary32 separately (no fused multiply-add);
* normal(sigma): element i uses words 8i..8i+7, read as sixteen 16-bit
  halves; ``z = sum(halves) - 16 * 32767.5`` is an exact integer and
  ``v = f32(z) * f32(sigma / (65536 * sqrt(16/12)))``.  This is the
  Irwin-Hall sum of 16 uniforms: mean 0, standard deviation sigma, tails cut
  at sqrt(48) sigma (about 6.9 sigma) -- a stand-in for the ~N(0, sigma) inputs;
* bf16: round-to-nearest-even of the binary32 value, on the bit pattern.

Canonical expert block (per expert, in this order): gate codes, up codes,
down codes, gate sb, up sb, down sb.  gate/up are inter x hidden (out x in),
down is hidden x inter; codes row-major, element k of a row in bits
(k*bits) % 8 upward of byte (k*bits)//8; sb is one u32 per (row, group of 64
input columns), bf16 scale in bits 0-15 and bf16 bias in bits 16-31.
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np

# tensor kinds (tensor id = kind | expert << 8 | layer << 20)
K_GATE_CODES, K_UP_CODES, K_DOWN_CODES = 0, 1, 2
K_GATE_SCALE, K_UP_SCALE, K_DOWN_SCALE = 3, 4, 5
K_GATE_BIAS, K_UP_BIAS, K_DOWN_BIAS = 6, 7, 8
K_ROUTER, K_SHARED_GATE, K_X, K_NORM_W = 9, 10, 11, 12
K_GDN_STATE, K_GDN_Q, K_GDN_K, K_GDN_V, K_GDN_ALPHA, K_GDN_BETA = 13, 14, 15, 16, 17, 18
K_ATTN_Q, K_ATTN_K, K_ATTN_V, K_ATTN_KCACHE, K_ATTN_VCACHE = 19, 20, 21, 22, 23
K_ATTN_QG, K_ATTN_QNW, K_ATTN_KNW = 24, 25, 26

# distributions of the synthetic workload
SCALE_LO, SCALE_HI = 0.001, 0.02     # bf16 scale ~ U(0.001, 0.02)
BIAS_SIGMA = 0.05                    # bf16 bias ~ N(0, 0.05)
ROUTER_SIGMA = 0.02                  # bf16 router ~ N(0, 0.02)
SHARED_GATE_SIGMA = 0.02             # bf16 shared-expert gate vector ~ N(0, 0.02)
X_SIGMA = 1.0                        # fp32 activations ~ N(0, 1)
NORM_LO, NORM_HI = 0.9, 1.1          # fp32 RMSNorm weight ~ U(0.9, 1.1)
GDN_STATE_SIGMA = 0.1                # GatedDeltaNet state ~ N(0, 0.1)
GDN_ALPHA_LO, GDN_ALPHA_HI = 0.9, 1.0  # decay gate ~ U(0.9, 1)
GDN_BETA_LO, GDN_BETA_HI = 0.0, 1.0    # write strength ~ U(0, 1)

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def tensor_id(kind: int, expert: int = 0, layer: int = 0) -> int:
    if not (0 <= kind < 256 and 0 <= expert < 4096 and 0 <= layer < 4096):
        raise ValueError("tensor id field out of range")
    return kind | (expert << 8) | (layer << 20)


def philox4x32_10(ctr: np.ndarray, key) -> np.ndarray:
    """Philox4x32 with 10 rounds on an (n, 4) uint32 counter array."""
    c = np.asarray(ctr, dtype=np.uint32).reshape(-1, 4).astype(np.uint64)
    c0, c1, c2, c3 = c[:, 0], c[:, 1], c[:, 2], c[:, 3]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for r in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0)), lo1, (hi0 ^ c3 ^ np.uint64(k1)), lo0
        k0 = (k0 + _W0) & 0xFFFFFFFF
        k1 = (k1 + _W1) & 0xFFFFFFFF
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def words(seed: int, tid: int, n_words: int, start: int = 0) -> np.ndarray:
    """Words [start, start + n_words) of stream (seed, tid) as uint32."""
    if n_words <= 0:
        return np.zeros(0, dtype=np.uint32)
    b0 = start // 4
    b1 = (start + n_words + 3) // 4
    blocks = np.arange(b0, b1, dtype=np.uint64)
    ctr = np.zeros((blocks.size, 4), dtype=np.uint32)
    ctr[:, 0] = (blocks & _MASK32).astype(np.uint32)
    ctr[:, 1] = (blocks >> np.uint64(32)).astype(np.uint32)
    out = philox4x32_10(ctr, (seed, tid)).reshape(-1)
    off = start - b0 * 4
    return out[off:off + n_words]


def stream_bytes(seed: int, tid: int, n_bytes: int) -> np.ndarray:
    w = words(seed, tid, (n_bytes + 3) // 4)
    return w.astype("<u4").view(np.uint8)[:n_bytes].copy()


def uniform_f32(seed: int, tid: int, n: int, lo: float, hi: float) -> np.ndarray:
    w = words(seed, tid, n)
    u = (w >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)
    return np.float32(lo) + u * np.float32(hi - lo)


def normal_const(sigma: float) -> np.float32:
    return np.float32(sigma / (65536.0 * math.sqrt(16.0 / 12.0)))


def normal_f32(seed: int, tid: int, n: int, sigma: float) -> np.ndarray:
    w = words(seed, tid, 8 * n).astype("<u4")
    halves = w.view(np.uint16).reshape(n, 16).astype(np.int64)
    z = (halves.sum(axis=1) - 524280).astype(np.float32)
    return z * normal_const(sigma)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


# --------------------------------------------------------------------------
# Canonical expert layout (placement only)
# --------------------------------------------------------------------------

def expert_layout(hidden: int, inter: int, bits: int) -> dict:
    """name -> (offset, size) for the six tensors of one expert, plus 'total'."""
    gu = inter * hidden * bits // 8
    dn = hidden * inter * bits // 8
    gsb = inter * (hidden // 64) * 4
    dsb = hidden * (inter // 64) * 4
    sizes = [("gate_codes", gu), ("up_codes", gu), ("down_codes", dn),
             ("gate_sb", gsb), ("up_sb", gsb), ("down_sb", dsb)]
    lay, pos = {}, 0
    for name, s in sizes:
        lay[name] = (pos, s)
        pos += s
    lay["total"] = pos
    return lay


def sb_words(seed: int, scale_tid: int, bias_tid: int, n: int) -> np.ndarray:
    s = f32_to_bf16_bits(uniform_f32(seed, scale_tid, n, SCALE_LO, SCALE_HI)).astype(np.uint32)
    b = f32_to_bf16_bits(normal_f32(seed, bias_tid, n, BIAS_SIGMA)).astype(np.uint32)
    return s | (b << np.uint32(16))


def expert_block(seed: int, layer: int, expert: int, hidden: int, inter: int, bits: int) -> np.ndarray:
    """One expert's canonical block (uint8), exactly as the device fill writes it."""
    lay = expert_layout(hidden, inter, bits)
    blk = np.zeros(lay["total"], dtype=np.uint8)
    for i, m in enumerate(("gate", "up", "down")):
        o, s = lay[m + "_codes"]
        blk[o:o + s] = stream_bytes(seed, tensor_id(K_GATE_CODES + i, expert, layer), s)
        o, s = lay[m + "_sb"]
        blk[o:o + s] = sb_words(seed, tensor_id(K_GATE_SCALE + i, expert, layer),
                                tensor_id(K_GATE_BIAS + i, expert, layer), s // 4).view(np.uint8)
    return blk


def matrix(seed: int, layer: int, expert: int, which: int, rows: int, cols: int, bits: int):
    """A stand-alone quantized matrix (codes uint8 [rows][cols*bits/8], sb uint32
    [rows][cols/64]) drawn from the streams of projection ``which`` (0 gate, 1 up,
    2 down) of the given expert."""
    codes = stream_bytes(seed, tensor_id(K_GATE_CODES + which, expert, layer),
                         rows * cols * bits // 8).reshape(rows, cols * bits // 8)
    sb = sb_words(seed, tensor_id(K_GATE_SCALE + which, expert, layer),
                  tensor_id(K_GATE_BIAS + which, expert, layer), rows * (cols // 64))
    return codes, sb.reshape(rows, cols // 64)


def router(seed: int, layer: int, E: int, H: int) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed, tensor_id(K_ROUTER, 0, layer), E * H,
                                       ROUTER_SIGMA)).reshape(E, H)


def shared_gate(seed: int, layer: int, H: int) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed, tensor_id(K_SHARED_GATE, 0, layer), H, SHARED_GATE_SIGMA))


def activations(seed: int, token: int, H: int) -> np.ndarray:
    """x (or h0) for token ``token``: fp32 ~N(0, 1)."""
    return normal_f32(seed, tensor_id(K_X, token % 4096, token // 4096), H, X_SIGMA)


def norm_weight(seed: int, layer: int, H: int) -> np.ndarray:
    return uniform_f32(seed, tensor_id(K_NORM_W, 0, layer), H, NORM_LO, NORM_HI)


def gdn_state(seed: int, layer: int, heads: int, dk: int, dv: int) -> np.ndarray:
    """A GatedDeltaNet state, fp32 ~N(0, 0.1), as [heads][dv][dk] (the library's
    layout: row j of a head holds the values at index j over the keys)."""
    return normal_f32(seed, tensor_id(K_GDN_STATE, 0, layer), heads * dv * dk,
                      GDN_STATE_SIGMA).reshape(heads, dv, dk)


def attn_cache(seed: int, layer: int, Hkv: int, T: int, D: int):
    """Key and value caches [Hkv][T][D], fp32 ~N(0, 1)."""
    K = normal_f32(seed, tensor_id(K_ATTN_KCACHE, 0, layer), Hkv * T * D, 1.0).reshape(Hkv, T, D)
    V = normal_f32(seed, tensor_id(K_ATTN_VCACHE, 0, layer), Hkv * T * D, 1.0).reshape(Hkv, T, D)
    return K, V


def attn_token(seed: int, layer: int, token: int, Hq: int, Hkv: int, D: int):
    """q [Hq][D], k and v [Hkv][D] of one decode token, fp32 ~N(0, 1)."""
    t = token % 4096
    q = normal_f32(seed, tensor_id(K_ATTN_Q, t, layer), Hq * D, 1.0).reshape(Hq, D)
    k = normal_f32(seed, tensor_id(K_ATTN_K, t, layer), Hkv * D, 1.0).reshape(Hkv, D)
    v = normal_f32(seed, tensor_id(K_ATTN_V, t, layer), Hkv * D, 1.0).reshape(Hkv, D)
    return q, k, v


def attn_token_qg(seed: int, layer: int, token: int, Hq: int, Hkv: int, D: int):
    """The query projection's output qg [Hq][2D] (per head: query, then gate),
    fp32 ~N(0, 2), and this token's k ~N(0, 1) and v ~N(0, 1) [Hkv][D]."""
    t = token % 4096
    qg = normal_f32(seed, tensor_id(K_ATTN_QG, t, layer), Hq * 2 * D, 2.0).reshape(Hq, 2 * D)
    _, k, v = attn_token(seed, layer, token, 1, Hkv, D)
    return qg, k, v


def attn_norm_weights(seed: int, layer: int, D: int):
    """RMS-normalisation weights of q and k, fp32 ~U(0.9, 1.1) [D] each."""
    return (uniform_f32(seed, tensor_id(K_ATTN_QNW, 0, layer), D, NORM_LO, NORM_HI),
            uniform_f32(seed, tensor_id(K_ATTN_KNW, 0, layer), D, NORM_LO, NORM_HI))


def gdn_token(seed: int, layer: int, token: int, heads: int, dk: int, dv: int):
    """Inputs of one recurrence step: q and k ~N(0, 1) scaled to unit length per
    head, v ~N(0, 1), alpha ~U(0.9, 1), beta ~U(0, 1); all fp32."""
    t = token % 4096
    q = normal_f32(seed, tensor_id(K_GDN_Q, t, layer), heads * dk, 1.0).reshape(heads, dk)
    k = normal_f32(seed, tensor_id(K_GDN_K, t, layer), heads * dk, 1.0).reshape(heads, dk)
    q = (q / np.linalg.norm(q.astype(np.float64), axis=1, keepdims=True)).astype(np.float32)
    k = (k / np.linalg.norm(k.astype(np.float64), axis=1, keepdims=True)).astype(np.float32)
    v = normal_f32(seed, tensor_id(K_GDN_V, t, layer), heads * dv, 1.0).reshape(heads, dv)
    alpha = uniform_f32(seed, tensor_id(K_GDN_ALPHA, t, layer), heads, GDN_ALPHA_LO, GDN_ALPHA_HI)
    beta = uniform_f32(seed, tensor_id(K_GDN_BETA, t, layer), heads, GDN_BETA_LO, GDN_BETA_HI)
    return q, k, v, alpha, beta


# --------------------------------------------------------------------------
# Device-side fill (same streams, generated in HBM)
# --------------------------------------------------------------------------

_LIB = None
_LIBPATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmoe_synth.so")


def device_lib():
    """ctypes handle of the device generator library (built by __graft_entry__.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIBPATH):
            raise RuntimeError(f"{_LIBPATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIBPATH)
        vp, u32, u64, i32, i64, f32 = (ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64,
                                       ctypes.c_int32, ctypes.c_int64, ctypes.c_float)
        lib.synth_fill_bytes.argtypes = [vp, u64, u32, u32, vp]
        lib.synth_fill_uniform_f32.argtypes = [vp, u64, u32, u32, f32, f32, vp]
        lib.synth_fill_normal_f32.argtypes = [vp, u64, u32, u32, f32, vp]
        lib.synth_fill_normal_bf16.argtypes = [vp, u64, u32, u32, f32, vp]
        lib.synth_fill_expert_pool.argtypes = [vp, i64, i32, i32, i32, u32, i32, i32, i32,
                                               f32, f32, f32, vp]
        for f in (lib.synth_fill_bytes, lib.synth_fill_uniform_f32, lib.synth_fill_normal_f32,
                  lib.synth_fill_normal_bf16, lib.synth_fill_expert_pool):
            f.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def fill_expert_pool(buf, stride: int, n_experts: int, expert0: int, layer: int, seed: int,
                     hidden: int, inter: int, bits: int, stream=None):
    """Fill ``n_experts`` canonical expert blocks at ``buf`` (uint8 torch tensor on
    the GPU), expert j at byte ``j * stride`` drawing the streams of expert id
    ``expert0 + j``."""
    lib = device_lib()
    _check(lib.synth_fill_expert_pool(ctypes.c_void_p(buf.data_ptr()), stride, n_experts, expert0,
                                      layer, seed, hidden, inter, bits,
                                      np.float32(SCALE_LO), np.float32(SCALE_HI - SCALE_LO),
                                      normal_const(BIAS_SIGMA), _stream_handle(stream)),
           "synth_fill_expert_pool")


def fill_normal_bf16(t, seed: int, tid: int, sigma: float, stream=None):
    _check(device_lib().synth_fill_normal_bf16(ctypes.c_void_p(t.data_ptr()), t.numel(), seed, tid,
                                               normal_const(sigma), _stream_handle(stream)),
           "synth_fill_normal_bf16")


def fill_normal_f32(t, seed: int, tid: int, sigma: float, stream=None):
    _check(device_lib().synth_fill_normal_f32(ctypes.c_void_p(t.data_ptr()), t.numel(), seed, tid,
                                              normal_const(sigma), _stream_handle(stream)),
           "synth_fill_normal_f32")


def fill_uniform_f32(t, seed: int, tid: int, lo: float, hi: float, stream=None):
    _check(device_lib().synth_fill_uniform_f32(ctypes.c_void_p(t.data_ptr()), t.numel(), seed, tid,
                                               np.float32(lo), np.float32(hi - lo),
                                               _stream_handle(stream)),
           "synth_fill_uniform_f32")


def fill_bytes(t, seed: int, tid: int, stream=None):
    _check(device_lib().synth_fill_bytes(ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size(),
                                         seed, tid, _stream_handle(stream)),
           "synth_fill_bytes")
