"""C ABI checks that need no GPU: the library loads, exports every function that
include/qmoe.h declares, computes the expert layout on the host, and rejects
bad arguments before anything is launched."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_dequant_gemv_amd", "libqmoe.so")
HEADER = os.path.join(ROOT, "include", "qmoe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libqmoe.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    names = _declared_functions()
    assert len(names) >= 12, names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_expert_layout_matches_oracle_layout():
    import bit_dequant_gemv_amd as q
    for H, I, bits in [(4096, 1024, 4), (4096, 1024, 2), (128, 64, 4), (1024, 256, 2)]:
        lay = q.qmoe_expert_layout(H, I, bits)
        off = oracle.expert_offsets(H, I, bits)
        for name in ("gate_codes", "up_codes", "down_codes", "gate_sb", "up_sb", "down_sb"):
            assert lay[name] == off[name][0]
        assert lay["total"] == off["total"]
    assert q.qmoe_expert_layout(4096, 1024, 4)["total"] == 7_077_888


def test_invalid_arguments_are_rejected_before_launch():
    import bit_dequant_gemv_amd as q
    lib = q.raw_lib()
    # bad bits / shapes in the pure-host layout call
    o = q.ExpertOffsets()
    assert lib.qmoe_expert_layout(4096, 1024, 3, ctypes.byref(o)) == q.QMOE_EINVAL
    assert lib.qmoe_expert_layout(100, 1024, 4, ctypes.byref(o)) == q.QMOE_ESHAPE
    assert lib.qmoe_expert_layout(4096, 1024, 4, None) == q.QMOE_EINVAL
    # qgemv: null matrix, cols not a multiple of 64, misaligned codes
    assert lib.qgemv_w4(None, None, None, None) == q.QMOE_EINVAL
    m = q.QMat(16, 16, 4, 100)
    assert lib.qgemv_w4(ctypes.byref(m), 16, 16, None) == q.QMOE_ESHAPE
    m = q.QMat(17, 16, 4, 128)
    assert lib.qgemv_w4(ctypes.byref(m), 16, 16, None) == q.QMOE_EALIGN
    m = q.QMat(16, 16, 4, 16384)
    assert lib.qgemv_w4(ctypes.byref(m), 16, 16, None) == q.QMOE_ESHAPE     # > 8192 at 4 bits
    assert "multiple of 64" in lib.qmoe_last_error().decode() or "at most" in lib.qmoe_last_error().decode()
    # router: K > E, H not a multiple of 64
    assert lib.moe_router_topk(16, 16, 1, 4096, 4, 5, 16, 16, 16, None) == q.QMOE_ESHAPE
    assert lib.moe_router_topk(16, 16, 1, 100, 512, 4, 16, 16, 16, None) == q.QMOE_ESHAPE
    # expert pool: bad stride, bad bits
    pool = q.ExpertPoolC(256, 1000, 4, 4096, 1024, 4)
    assert lib.expert_ffn_swiglu(ctypes.byref(pool), 16, 1, 16, 16, 16, 1 << 20, None) == q.QMOE_EALIGN
    pool = q.ExpertPoolC(256, 7077888, 4, 4096, 1024, 3)
    assert lib.expert_ffn_swiglu(ctypes.byref(pool), 16, 1, 16, 16, 16, 1 << 20, None) == q.QMOE_EINVAL
    # layer: short workspace, top_k > 8
    routed = q.ExpertPoolC(256, 7077888, 512, 4096, 1024, 4)
    shared = q.ExpertPoolC(256, 7077888, 1, 4096, 1024, 4)
    L = q.LayerC(routed, shared, 256, 256, 4)
    need = lib.qmoe_workspace_bytes(ctypes.byref(L), 1)
    assert need > 0
    assert lib.moe_layer_forward(ctypes.byref(L), 256, 256, 512, 16, 16, 256, need - 1, None) == \
        q.QMOE_EWORKSPACE
    assert lib.moe_layer_forward(ctypes.byref(L), 256, 256, 256, 16, 16, 256, need, None) == \
        q.QMOE_EINVAL   # out aliases x
    L9 = q.LayerC(routed, shared, 256, 256, 9)
    assert lib.moe_layer_forward(ctypes.byref(L9), 256, 256, 512, 16, 16, 256, need, None) == q.QMOE_ESHAPE
    bad_shared = q.LayerC(routed, q.ExpertPoolC(256, 7077888, 2, 4096, 1024, 4), 256, 256, 4)
    assert lib.moe_layer_forward(ctypes.byref(bad_shared), 256, 256, 512, 16, 16, 256, need, None) == \
        q.QMOE_ESHAPE
    assert lib.moe_layer_forward_batched(ctypes.byref(L), 256, 256, 512, 0, 16, 16, 256, need, None) == \
        q.QMOE_ESHAPE
    # batched: residual and out are read and written as float4s
    need2 = lib.qmoe_workspace_bytes(ctypes.byref(L), 2)
    assert lib.moe_layer_forward_batched(ctypes.byref(L), 256, 260, 512, 2, 16, 16, 256, need2, None) == \
        q.QMOE_EALIGN
    assert lib.moe_layer_forward_batched(ctypes.byref(L), 256, 512, 516, 2, 16, 16, 256, need2, None) == \
        q.QMOE_EALIGN
    assert lib.rmsnorm_f32(16, 16, -1.0, 4, 16, None) == q.QMOE_EINVAL
    # attention decode: shapes, position, rotation, workspace
    na = lib.qmoe_attn_workspace_bytes(32, 2, 256, 4096)
    assert na > 0 and lib.qmoe_attn_workspace_bytes(32, 2, 100, 4096) == 0
    assert lib.qmoe_attn_workspace_bytes(34, 2, 256, 4096) == 0 and lib.qmoe_attn_workspace_bytes(34, 1, 256, 8) == 0
    def attn(Hq=32, Hkv=2, D=256, Tmax=4096, pos=5, theta=1e7, rot=64, ws=256, wsb=None):
        return lib.attn_decode_step(256, 256, 256, 256, 256, Hq, Hkv, D, Tmax, pos, theta, rot, 256, ws,
                                    na if wsb is None else wsb, None)
    assert attn(pos=4096) == q.QMOE_ESHAPE and attn(pos=-1) == q.QMOE_ESHAPE
    assert attn(rot=3) == q.QMOE_ESHAPE and attn(rot=258) == q.QMOE_ESHAPE
    assert attn(theta=0.0) == q.QMOE_EINVAL and attn(Hq=33) == q.QMOE_ESHAPE
    assert attn(wsb=na - 1) == q.QMOE_EWORKSPACE and attn(ws=272) == q.QMOE_EALIGN
    # GatedDeltaNet step: shapes, pointers (heads == 0 is a no-op: no launch)
    assert lib.gdn_recurrent_step(256, 256, 256, 256, 256, 256, 256, 64, 100, 128, None) == q.QMOE_ESHAPE
    assert lib.gdn_recurrent_step(256, 256, 256, 256, 256, 256, 256, 64, 128, 0, None) == q.QMOE_ESHAPE
    assert lib.gdn_recurrent_step(256, 256, 256, 256, 256, 256, 256, -1, 128, 128, None) == q.QMOE_ESHAPE
    assert lib.gdn_recurrent_step(None, None, None, None, None, None, None, 0, 128, 128, None) == q.QMOE_OK
    assert lib.gdn_recurrent_step(None, 256, 256, 256, 256, 256, 256, 64, 128, 128, None) == q.QMOE_EINVAL
    assert lib.gdn_recurrent_step(264, 256, 256, 256, 256, 256, 256, 64, 128, 128, None) == q.QMOE_EALIGN
    assert lib.gdn_recurrent_step(256, 256, 256, None, 256, 256, 256, 64, 128, 128, None) == q.QMOE_EINVAL
    assert lib.qmoe_workspace_bytes(ctypes.byref(L), 0) == 0
    # stack: no layers, shapes that differ between layers, a short workspace
    Ls = (q.LayerC * 2)(L, L)
    nw = (ctypes.c_void_p * 2)(256, 256)
    need_s = lib.qmoe_stack_workspace_bytes(Ls, 2)
    assert need_s >= need and lib.qmoe_stack_workspace_bytes(Ls, 0) == 0
    assert lib.qmoe_stack_workspace_bytes(None, 2) == 0
    assert lib.moe_stack_forward(Ls, nw, 0, 1e-6, 256, 512, None, 16, 16, 0, 256, need_s, None) == q.QMOE_EINVAL
    assert lib.moe_stack_forward(None, nw, 2, 1e-6, 256, 512, None, 16, 16, 0, 256, need_s, None) == q.QMOE_EINVAL
    assert lib.moe_stack_forward(Ls, nw, 2, 1e-6, 256, 512, None, 16, 16, 0, 256, need_s - 1, None) == \
        q.QMOE_EWORKSPACE
    assert lib.moe_stack_forward(Ls, nw, 2, 1e-6, 256, 512, 520, 16, 16, 0, 256, need_s, None) == q.QMOE_EALIGN
    assert lib.moe_stack_forward(Ls, nw, 2, 1e-6, 256, 512, None, 16, 16, 2, 256, need_s, None) == q.QMOE_EINVAL
    assert lib.moe_stack_forward(Ls, nw, 2, 1e-6, 256, 512, 512, 16, 16, 0, 256, need_s, None) == q.QMOE_EINVAL
    L2b = q.LayerC(q.ExpertPoolC(256, 3932160, 512, 4096, 1024, 2), q.ExpertPoolC(256, 3932160, 1, 4096, 1024, 2),
                   256, 256, 4)
    Lmix = (q.LayerC * 2)(L, L2b)
    assert lib.moe_stack_forward(Lmix, nw, 2, 1e-6, 256, 512, None, 16, 16, 0, 256, need_s, None) == q.QMOE_ESHAPE
    # more layers than one launch holds: the buffers of one launch's worth
    assert lib.qmoe_stack_workspace_bytes((q.LayerC * 40)(*([L] * 40)), 40) == \
        lib.qmoe_stack_workspace_bytes((q.LayerC * 32)(*([L] * 32)), 32)
    assert lib.qmoe_strerror(q.QMOE_EWORKSPACE) == b"workspace too small"


def test_workspace_grows_with_batch():
    import bit_dequant_gemv_amd as q
    lib = q.raw_lib()
    routed = q.ExpertPoolC(256, 7077888, 512, 4096, 1024, 4)
    shared = q.ExpertPoolC(256, 7077888, 1, 4096, 1024, 4)
    L = q.LayerC(routed, shared, 256, 256, 4)
    a = lib.qmoe_workspace_bytes(ctypes.byref(L), 1)
    b = lib.qmoe_workspace_bytes(ctypes.byref(L), 64)
    assert b > a > (512 + 1) * 8
    assert b % 256 == 0 and a % 256 == 0


def test_offload_handle_arguments_are_checked_on_the_host():
    import bit_dequant_gemv_amd as q
    lib = q.raw_lib()
    h = ctypes.c_void_p()
    pool = q.ExpertPoolC(0, 1 << 23, 4, 1024, 256, 4)  # null base
    assert lib.qmoe_offload_create(ctypes.byref(pool), 2, ctypes.c_void_p(256), ctypes.byref(h)) == q.QMOE_EINVAL
    pool = q.ExpertPoolC(4096, 1 << 23, 4, 1024, 256, 4)
    assert lib.qmoe_offload_create(ctypes.byref(pool), 0, ctypes.c_void_p(256), ctypes.byref(h)) == q.QMOE_ESHAPE
    assert lib.qmoe_offload_create(ctypes.byref(pool), 2, None, ctypes.byref(h)) == q.QMOE_EINVAL
    assert lib.qmoe_offload_create(ctypes.byref(pool), 2, ctypes.c_void_p(100), ctypes.byref(h)) == q.QMOE_EALIGN
    assert lib.qmoe_offload_create(ctypes.byref(pool), 2, ctypes.c_void_p(256), None) == q.QMOE_EINVAL
    assert lib.qmoe_offload_destroy(None) == q.QMOE_EINVAL
    assert lib.moe_layer_forward_offload(None, None, None, None, None, None, None, None, 0, None, None) \
        == q.QMOE_EINVAL
    L = q.LayerC(pool, q.ExpertPoolC(4096, 1 << 23, 1, 1024, 256, 4), 256, 256, 4)
    assert lib.qmoe_offload_workspace_bytes(ctypes.byref(L)) > 4 * 1024 * 4
