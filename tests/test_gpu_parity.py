"""Parity of the HIP path (through the C ABI) against the float64 CPU oracle.

Bars: expert indices equal the oracle's top-K (decided on fp32-rounded logits,
ties to the lower index) except exempted fp32 near-ties; floating-point outputs
within relative L2 error 1e-3 of the oracle (the stated bar), and within 1e-4
as a tighter fp32-accumulation check.  Inputs are seeded synthetic tensors
drawn by ``synth`` on the device and regenerated on the host for the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from qmoe_testlib import DeviceLayer, check_topk, device_x, host_x

pytestmark = pytest.mark.gpu

TOL = 1e-3       # relative L2 bar for fp32-accumulated outputs
TIGHT = 1e-4     # fp32 accumulation is ~1e-6 here; this catches real defects early


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def q():
    import bit_dequant_gemv_amd as q
    return q


def _rel(a, b):
    return oracle.rel_l2(np.asarray(a, dtype=np.float64), b)


# ---------------------------------------------------------------------------
# generators: device fill == host fill, bit for bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,I,bits,E", [(128, 64, 4, 3), (192, 128, 2, 2), (4096, 1024, 4, 1)])
def test_synth_device_matches_host(q, H, I, bits, E):
    say("synth pool", H, I, bits, E)
    pool = q.ExpertPool.allocate(E, H, I, bits)
    synth.fill_expert_pool(pool.buf, pool.stride, E, 5, 3, 77, H, I, bits)
    torch.cuda.synchronize()
    for e in range(E):
        dev = pool.expert_bytes(e).cpu().numpy()
        host = synth.expert_block(77, 3, 5 + e, H, I, bits)
        np.testing.assert_array_equal(dev, host)


def test_synth_device_value_streams(q):
    say("synth value streams")
    n = 10007
    t = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.fill_normal_bf16(t, 9, 123, 0.02)
    np.testing.assert_array_equal(t.cpu().numpy().view(np.uint16),
                                  synth.f32_to_bf16_bits(synth.normal_f32(9, 123, n, 0.02)))
    f = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.fill_normal_f32(f, 9, 124, 1.0)
    np.testing.assert_array_equal(f.cpu().numpy(), synth.normal_f32(9, 124, n, 1.0))
    synth.fill_uniform_f32(f, 9, 125, 0.9, 1.1)
    np.testing.assert_array_equal(f.cpu().numpy(), synth.uniform_f32(9, 125, n, 0.9, 1.1))
    b = torch.empty(4 * 1001, dtype=torch.uint8, device="cuda")
    synth.fill_bytes(b[:4003], 9, 126)
    np.testing.assert_array_equal(b[:4003].cpu().numpy(), synth.stream_bytes(9, 126, 4003))


# ---------------------------------------------------------------------------
# quantized GEMV
# ---------------------------------------------------------------------------

GEMV_SHAPES = [(1, 64), (63, 128), (64, 4096), (1000, 1024), (4096, 1024), (1024, 4096),
               (7, 8192), (129, 192), (33, 320)]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("rows,cols", GEMV_SHAPES)
def test_qgemv_parity(q, bits, rows, cols):
    say("qgemv", bits, rows, cols)
    seed = 1000 + rows * 7 + cols
    codes, sb = synth.matrix(seed, 0, 0, 0, rows, cols, bits)
    x = synth.normal_f32(seed, 99, cols, 1.0)
    fn = q.qgemv_w4 if bits == 4 else q.qgemv_w2
    y = fn(torch.from_numpy(codes).cuda(), torch.from_numpy(sb.view(np.int32)).cuda(),
           torch.from_numpy(x).cuda())
    ref = oracle.qgemv(codes, sb, x, bits)
    r = _rel(y.cpu().numpy(), ref)
    say("  rel_l2", r)
    assert r <= TOL and r <= TIGHT


def test_qgemv_empty_and_unit_vectors(q):
    say("qgemv empty / unit")
    codes, sb = synth.matrix(5, 0, 0, 0, 0, 128, 4)
    y = torch.full((1,), 7.0, device="cuda")
    q.qgemv_w4(torch.zeros(0, 64, dtype=torch.uint8, device="cuda"),
               torch.zeros(0, 2, dtype=torch.int32, device="cuda"),
               torch.zeros(128, device="cuda"), y=y)
    assert y.item() == 7.0     # nothing written for 0 rows
    codes, sb = synth.matrix(6, 0, 0, 0, 37, 256, 4)
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(sb.view(np.int32)).cuda()
    W = oracle.dequant(codes, sb, 256, 4)
    for k in (0, 1, 31, 32, 63, 64, 255):
        x = np.zeros(256, np.float32)
        x[k] = 1.0
        y = q.qgemv_w4(dc, ds, torch.from_numpy(x).cuda()).cpu().numpy()
        np.testing.assert_allclose(y, W[:, k], rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------------------
# expert FFN
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,I,bits,E,idx", [(256, 128, 4, 4, [2, 0, 2]), (256, 128, 2, 3, [1]),
                                            (4096, 1024, 4, 2, [1]), (4096, 1024, 4, 2, [0, 1, 1, 0, 1]),
                                            (4096, 1024, 2, 2, [1, 0]), (1024, 320, 4, 3, [2, 1])])
def test_expert_ffn_parity(q, H, I, bits, E, idx):
    say("expert_ffn", H, I, bits, E, idx)
    seed = 1000
    pool = q.ExpertPool.allocate(E, H, I, bits)
    synth.fill_expert_pool(pool.buf, pool.stride, E, 0, 0, seed, H, I, bits)
    x = host_x(seed, 0, H)
    y = q.expert_ffn_swiglu(pool, torch.tensor(idx, dtype=torch.int32, device="cuda"),
                            torch.from_numpy(x).cuda()).cpu().numpy()
    for i, e in enumerate(idx):
        ref = oracle.expert_ffn(synth.expert_block(seed, 0, e, H, I, bits), x, H, I, bits)
        r = _rel(y[i], ref)
        say("  slot", i, "expert", e, "rel_l2", r)
        assert r <= TOL and r <= TIGHT


# one expert per call on a shape the single-launch kernel takes (hidden 1024/2048/4096,
# inter 256/512/1024): gate/up, SwiGLU and down in one launch, h handed over as tagged
# words; both bit widths, the smallest and largest grids and both lane layouts
FUSED_FFN_CASES = [(1024, 256, 4, 3, 2), (2048, 512, 2, 2, 1), (4096, 1024, 2, 2, 0), (1024, 1024, 4, 2, 1),
                   (4096, 256, 4, 2, 1), (1024, 256, 2, 2, 1), (4096, 1024, 4, 3, 2)]


@pytest.mark.parametrize("H,I,bits,E,e", FUSED_FFN_CASES)
def test_expert_ffn_single_launch_parity(q, H, I, bits, E, e):
    """n = 1 takes the single-launch kernel: against the oracle, over nine calls on one
    workspace (the call counter passes the four h slots twice), with a call of three
    experts (the two-launch path, sharing the workspace) in the middle; the status
    word stays clear."""
    say("expert_ffn single launch", H, I, bits, E, e)
    seed = 1100 + H + I + bits
    pool = q.ExpertPool.allocate(E, H, I, bits)
    synth.fill_expert_pool(pool.buf, pool.stride, E, 0, 0, seed, H, I, bits)
    ws = torch.zeros(q.qmoe_ffn_workspace_bytes(pool, 3), dtype=torch.uint8, device="cuda")
    blocks = [synth.expert_block(seed, 0, k, H, I, bits) for k in range(E)]
    for call in range(9):
        x = host_x(seed, call, H)
        ek = (e + call) % E
        if call == 4:
            idx = [ek, (ek + 1) % E, ek]
            y = q.expert_ffn_swiglu(pool, torch.tensor(idx, dtype=torch.int32, device="cuda"),
                                    torch.from_numpy(x).cuda(), ws=ws).cpu().numpy()
        else:
            idx = [ek]
            y = q.expert_ffn_swiglu(pool, torch.tensor(idx, dtype=torch.int32, device="cuda"),
                                    torch.from_numpy(x).cuda(), ws=ws).cpu().numpy()
        for i, k in enumerate(idx):
            r = _rel(y[i], oracle.expert_ffn(blocks[k], x, H, I, bits))
            say("  call", call, "slot", i, "expert", k, "rel_l2", r)
            assert r <= TOL and r <= TIGHT
    assert int(ws[4:8].view(torch.int32).item()) == 0  # status word


def test_expert_ffn_single_launch_bad_index_gives_nan(q):
    say("expert_ffn single launch, bad index")
    pool = q.ExpertPool.allocate(2, 4096, 1024, 4)
    synth.fill_expert_pool(pool.buf, pool.stride, 2, 0, 0, 3, 4096, 1024, 4)
    ws = torch.zeros(q.qmoe_ffn_workspace_bytes(pool, 1), dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(host_x(3, 0, 4096)).cuda()
    for idx, finite in (([7], False), ([1], True), ([-1], False), ([0], True)):
        y = q.expert_ffn_swiglu(pool, torch.tensor(idx, dtype=torch.int32, device="cuda"), x, ws=ws)
        y = y.cpu().numpy()
        assert np.isfinite(y).all() if finite else np.isnan(y).all()
    assert int(ws[4:8].view(torch.int32).item()) == 0


def test_expert_ffn_single_launch_counter_wraps(q):
    """The one-launch FFN's call counter wraps past 2^32 - 1 without taking a
    zero-filled h word for a current one."""
    say("expert_ffn single launch, counter wrap")
    H, I, bits, E, seed = 2048, 512, 4, 2, 1234
    pool = q.ExpertPool.allocate(E, H, I, bits)
    synth.fill_expert_pool(pool.buf, pool.stride, E, 0, 0, seed, H, I, bits)
    ws = torch.zeros(q.qmoe_ffn_workspace_bytes(pool, 1), dtype=torch.uint8, device="cuda")
    ws[0:4].view(torch.int32).fill_(-2)  # counter = 0xFFFFFFFE
    for call in range(3):
        x = host_x(seed, call, H)
        y = q.expert_ffn_swiglu(pool, torch.tensor([call % E], dtype=torch.int32, device="cuda"),
                                torch.from_numpy(x).cuda(), ws=ws).cpu().numpy()
        ref = oracle.expert_ffn(synth.expert_block(seed, 0, call % E, H, I, bits), x, H, I, bits)
        assert _rel(y[0], ref) <= TIGHT
    # 0xFFFFFFFE -> 0xFFFFFFFF -> 1 (0 skipped) -> 2
    assert int(ws[0:4].view(torch.int32).item()) == 2
    assert int(ws[4:8].view(torch.int32).item()) == 0


def test_expert_ffn_bad_index_gives_nan(q):
    say("expert_ffn bad index")
    pool = q.ExpertPool.allocate(2, 256, 128, 4)
    synth.fill_expert_pool(pool.buf, pool.stride, 2, 0, 0, 3, 256, 128, 4)
    y = q.expert_ffn_swiglu(pool, torch.tensor([1, 7, -1], dtype=torch.int32, device="cuda"),
                            torch.from_numpy(host_x(3, 0, 256)).cuda()).cpu().numpy()
    assert np.isfinite(y[0]).all() and np.isnan(y[1]).all() and np.isnan(y[2]).all()


# ---------------------------------------------------------------------------
# router + top-K, combine, RMSNorm
# ---------------------------------------------------------------------------

# T >= 8 takes the token-tiled router (ragged expert and token tiles included) and,
# for E <= 1024, the wave-per-token top-K
@pytest.mark.parametrize("E,H,K,T", [(512, 4096, 4, 5), (64, 1024, 8, 3), (10, 256, 3, 2), (4096, 512, 2, 1),
                                     (512, 4096, 4, 64), (1000, 1024, 8, 9), (2048, 512, 2, 20)])
def test_router_topk_parity(q, E, H, K, T):
    say("router_topk", E, H, K, T)
    seed = 2000 + E
    R = synth.router(seed, 0, E, H)
    X = np.stack([host_x(seed, t, H) for t in range(T)])
    idx, w, logits = q.moe_router_topk(torch.from_numpy(R.view(np.int16)).cuda(),
                                       torch.from_numpy(X).cuda(), K)
    idx, w, logits = idx.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()
    for t in range(T):
        ref_l = oracle.router_logits(R, X[t])
        assert _rel(logits[t], ref_l) <= TIGHT
        tau = oracle.topk_tolerance(R, X[t])
        ex = check_topk(idx[t], ref_l, tau, K)
        sel = ref_l[idx[t]]
        ref_w = np.exp(sel - sel.max())
        ref_w /= ref_w.sum()
        assert _rel(w[t], ref_w) <= TIGHT
        say("  token", t, "near-tie exemptions", ex)


@pytest.mark.parametrize("T", [1, 8])
def test_router_exact_ties_go_to_lower_index(q, T):
    say("router ties", T)
    E, H = 512, 4096
    R = synth.router(31, 0, E, H).copy()
    X = host_x(31, 0, H)
    # a dominant row (parallel to x) copied to three experts: identical fp32 logits
    R[7] = synth.f32_to_bf16_bits((0.02 * X).astype(np.float32))
    R[300] = R[7]
    R[450] = R[7]
    idx, w, _ = q.moe_router_topk(torch.from_numpy(R.view(np.int16)).cuda(),
                                  torch.from_numpy(np.tile(X, (T, 1))).cuda(), 4)
    for t in range(T):
        got = idx.cpu().numpy()[t].tolist()
        assert got[:3] == [7, 300, 450], got
        np.testing.assert_allclose(w.cpu().numpy()[t][:3], w.cpu().numpy()[t][0], rtol=0)


def test_combine_parity(q):
    say("combine")
    H, K = 4096, 4
    rng = np.random.default_rng(5)
    yr = rng.standard_normal((K, H)).astype(np.float32)
    w = rng.dirichlet(np.ones(K)).astype(np.float32)
    ys = rng.standard_normal(H).astype(np.float32)
    g = synth.shared_gate(5, 0, H)
    x = host_x(5, 0, H)
    r = rng.standard_normal(H).astype(np.float32)
    c = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = q.moe_combine_residual_gate(c(yr), c(w), c(ys), c(g.view(np.int16)), c(x), c(r)).cpu().numpy()
    ref = oracle.combine_residual_gate(yr, w, ys, g, x, r)
    assert _rel(out, ref) <= TIGHT
    # out aliasing the residual
    rr = c(r)
    q.moe_combine_residual_gate(c(yr), c(w), c(ys), c(g.view(np.int16)), c(x), rr, out=rr)
    assert _rel(rr.cpu().numpy(), ref) <= TIGHT


@pytest.mark.parametrize("n", [1, 64, 4096, 5000])
def test_rmsnorm_parity(q, n):
    say("rmsnorm", n)
    v = synth.normal_f32(8, 1, n, 1.0)
    w = synth.uniform_f32(8, 2, n, 0.9, 1.1)
    out = q.rmsnorm_f32(torch.from_numpy(v).cuda(), torch.from_numpy(w).cuda(), 1e-6).cpu().numpy()
    assert _rel(out, oracle.rmsnorm(v, w, 1e-6)) <= TIGHT
    vv = torch.from_numpy(v).cuda()
    q.rmsnorm_f32(vv, torch.from_numpy(w).cuda(), 1e-6, out=vv)
    assert _rel(vv.cpu().numpy(), oracle.rmsnorm(v, w, 1e-6)) <= TIGHT


# ---------------------------------------------------------------------------
# one MoE layer
# ---------------------------------------------------------------------------

def _status(ws):
    return int(ws[4:8].view(torch.int32).item())


def _epoch(ws):
    return int(ws[0:4].view(torch.int32).item())


def _check_layer_token(D, x, out, idx, w, residual=None):
    residual = x if residual is None else residual
    R = D.host_router()
    logits = oracle.router_logits(R, x)
    tau = oracle.topk_tolerance(R, x)
    ex = check_topk(idx, logits, tau, D.K)
    ref = oracle.moe_layer(D.host_expert, D.host_shared(), R, D.host_gate(), x, residual,
                           D.H, D.I, D.bits, D.K, force_idx=idx if ex else None)
    r = _rel(out, ref)
    say("  idx", list(idx), "near-ties", ex, "rel_l2", r)
    assert r <= TOL and r <= TIGHT
    sel = logits[np.asarray(idx)]
    ref_w = np.exp(sel - sel.max())
    assert _rel(w, ref_w / ref_w.sum()) <= TIGHT
    return ex


LAYER_CASES = [  # (E, H, I, bits, K)  -- fused shapes, plus shapes served by the fallback chain
    (64, 1024, 256, 4, 4), (64, 1024, 256, 2, 4), (100, 2048, 512, 4, 3), (33, 1024, 512, 4, 1),
    (16, 192, 128, 4, 2), (512, 4096, 1024, 4, 8),
    # 2-bit planes built from half code words: routed h of 3 and 1 experts (192 and 64
    # half words, whole waves), and a 2048-wide x (256 half words)
    (100, 2048, 512, 2, 3), (33, 1024, 512, 2, 1),
]


@pytest.mark.parametrize("E,H,I,bits,K", LAYER_CASES)
def test_layer_parity(q, E, H, I, bits, K):
    say("layer", E, H, I, bits, K)
    D = DeviceLayer(3000 + E, 0, E, H, I, bits, K)
    ws = q.alloc_workspace(D.L)
    for tok in range(2):
        x = host_x(D.seed, tok, H)
        out, idx, w = q.moe_layer_forward(D.L, torch.from_numpy(x).cuda(), ws=ws)
        torch.cuda.synchronize()
        assert _status(ws) == 0
        _check_layer_token(D, x, out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy())


@pytest.mark.parametrize("bits", [4, 2])
def test_layer_full_config(q, bits):
    """The workload layer: 512 experts (4096 x 1024, group 64), top-4, shared expert."""
    say("layer full config bits", bits)
    seed = 1001 if bits == 4 else 1002
    D = DeviceLayer(seed, 0, 512, 4096, 1024, bits, 4)
    ws = q.alloc_workspace(D.L)
    resid = host_x(seed, 1000, 4096)
    for tok in range(3):
        x = host_x(seed, tok, 4096)
        # residual distinct from x on one token (the stack passes the pre-norm h)
        r = resid if tok == 2 else x
        out, idx, w = q.moe_layer_forward(D.L, torch.from_numpy(x).cuda(), torch.from_numpy(r).cuda(),
                                          ws=ws)
        torch.cuda.synchronize()
        assert _status(ws) == 0
        _check_layer_token(D, x, out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), residual=r)


def test_layer_fused_equals_unfused_chain_and_is_deterministic(q):
    say("fused vs unfused chain")
    D = DeviceLayer(1001, 0, 512, 4096, 1024, 4, 4)
    ws = q.alloc_workspace(D.L)
    xs = device_x(1001, [11, 12, 13], 4096)
    for t in range(3):
        x = xs[t].contiguous()
        e0 = _epoch(ws)
        out1, idx1, w1 = q.moe_layer_forward(D.L, x, ws=ws)
        out2, idx2, w2 = q.moe_layer_forward(D.L, x, ws=ws)
        torch.cuda.synchronize()
        assert _epoch(ws) == e0 + 2 and _status(ws) == 0
        assert torch.equal(out1, out2) and torch.equal(idx1, idx2) and torch.equal(w1, w2)
        # the same layer through the stand-alone entry points
        idx, w, _ = q.moe_router_topk(D.router, x, 4)
        assert torch.equal(idx[0], idx1)
        yr = q.expert_ffn_swiglu(D.routed, idx[0].contiguous(), x)
        ys = q.expert_ffn_swiglu(D.shared, torch.zeros(1, dtype=torch.int32, device="cuda"), x)
        out3 = q.moe_combine_residual_gate(yr, w[0].contiguous(), ys[0].contiguous(), D.gate, x, x)
        r = _rel(out1.cpu().numpy(), out3.cpu().numpy().astype(np.float64))
        say("  fused vs chain rel_l2", r)
        assert r <= 1e-5


def test_layer_output_may_alias_residual(q):
    say("layer out aliases residual")
    D = DeviceLayer(4001, 0, 64, 1024, 256, 4, 4)
    ws = q.alloc_workspace(D.L)
    x = host_x(D.seed, 0, 1024)
    r = host_x(D.seed, 5, 1024)
    rr = torch.from_numpy(r).cuda()
    out, idx, w = q.moe_layer_forward(D.L, torch.from_numpy(x).cuda(), rr, out=rr, ws=ws)
    torch.cuda.synchronize()
    _check_layer_token(D, x, rr.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), residual=r)


@pytest.mark.parametrize("E,H,I,bits,K", [(512, 4096, 1024, 4, 4), (64, 1024, 256, 2, 4),
                                          (16, 192, 128, 4, 2)])
def test_layer_norm_variant(q, E, H, I, bits, K):
    """h <- h + MoE(rmsnorm(h)) in one launch (fused shapes) or through the fallback
    chain (the last shape): against the oracle, and against rmsnorm_f32 followed by
    moe_layer_forward; out written in place over h."""
    say("layer norm variant", E, H, I, bits, K)
    D = DeviceLayer(6000 + E + bits, 3, E, H, I, bits, K)
    ws = q.alloc_workspace(D.L)
    nw = synth.norm_weight(D.seed, 3, H)
    dnw = torch.from_numpy(nw).cuda()
    for tok in range(2):
        h0 = host_x(D.seed, 20 + tok, H)
        h = torch.from_numpy(h0).cuda()
        # the two-call chain on a copy
        xn = q.rmsnorm_f32(h.clone(), dnw, 1e-6)
        ref_out, ref_idx, _ = q.moe_layer_forward(D.L, xn, h.clone(), ws=ws)
        out, idx, w = q.moe_layer_forward_norm(D.L, h, dnw, 1e-6, out=h, ws=ws)
        torch.cuda.synchronize()
        assert _status(ws) == 0
        assert out.data_ptr() == h.data_ptr()
        xr = oracle.rmsnorm(h0, nw, 1e-6)
        _check_layer_token(D, xr, h.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), residual=h0)
        if torch.equal(idx, ref_idx):
            r = _rel(h.cpu().numpy(), ref_out.cpu().numpy().astype(np.float64))
            say("  norm variant vs chain rel_l2", r)
            assert r <= 1e-5


def test_layer_call_counter_wraps(q):
    """The call tag in the workspace wraps past 2^32 - 1 without being mistaken for
    a zero-filled word."""
    say("call counter wrap")
    D = DeviceLayer(4001, 0, 64, 1024, 256, 4, 4)
    ws = q.alloc_workspace(D.L)
    ws[0:4].view(torch.int32).fill_(-2)  # counter = 0xFFFFFFFE
    x = host_x(D.seed, 3, 1024)
    for t in range(3):
        out, idx, w = q.moe_layer_forward(D.L, torch.from_numpy(x).cuda(), ws=ws)
        torch.cuda.synchronize()
        assert _status(ws) == 0
        _check_layer_token(D, x, out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy())
    # 0xFFFFFFFE -> 0xFFFFFFFF -> 1 (0 skipped) -> 2
    assert _epoch(ws) == 2


# ---------------------------------------------------------------------------
# batched decode (tokens grouped per expert)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("E,H,I,bits,K,T", [(64, 1024, 256, 4, 4, 16), (512, 4096, 1024, 4, 4, 64),
                                            (512, 4096, 1024, 2, 4, 8), (8, 256, 128, 4, 8, 5),
                                            # every expert gets 40 pairs: chunks of 32 and 8
                                            (4, 256, 128, 4, 4, 40),
                                            # other row-block shapes of the shared expert's
                                            # matrix-core chunks: 16 lanes per row and 3 blocks
                                            # of 64 rows; a block of 256 rows over I = 64 (its
                                            # last 12 tiles empty); ragged token chunks
                                            (16, 512, 192, 4, 4, 20), (8, 256, 64, 2, 2, 37)])
def test_batched_parity(q, E, H, I, bits, K, T):
    say("batched", E, H, I, bits, K, T)
    D = DeviceLayer(1004 if E == 512 else 5000 + E, 0, E, H, I, bits, K)
    X = device_x(D.seed, range(T), H)
    ws = q.alloc_workspace(D.L, T)
    out, idx, w = q.moe_layer_forward_batched(D.L, X, ws=ws)
    torch.cuda.synchronize()
    out, idx, w = out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    Xh = X.cpu().numpy()
    # every row: routing against the oracle's logits
    R = D.host_router()
    for t in range(T):
        check_topk(idx[t], oracle.router_logits(R, Xh[t]), oracle.topk_tolerance(R, Xh[t]), K)
    # sampled rows against the full oracle layer
    for t in sorted({0, T // 2, T - 1}):
        say("  token", t)
        _check_layer_token(D, Xh[t], out[t], idx[t], w[t])
    # batch invariance: each row equals the single-token fused layer
    if E <= 512:
        ws1 = q.alloc_workspace(D.L)
        for t in range(0, T, max(1, T // 8)):
            o1, i1, _ = q.moe_layer_forward(D.L, X[t].contiguous(), ws=ws1)
            if (i1.cpu().numpy() == idx[t]).all():
                assert _rel(out[t], o1.cpu().numpy().astype(np.float64)) <= 1e-5


# ---------------------------------------------------------------------------
# layer stack (RMSNorm before every layer, residual = pre-norm h)
# ---------------------------------------------------------------------------

def _chain(q, layers, dnorm, h0, ws):
    """One moe_layer_forward_norm launch per layer, in place: each layer's output, idx, w."""
    h = h0.clone()
    outs, idxs, wts = [], [], []
    for l, D in enumerate(layers):
        _, idx, w = q.moe_layer_forward_norm(D.L, h, dnorm[l], 1e-6, out=h, ws=ws)
        outs.append(h.clone())
        idxs.append(idx.clone())
        wts.append(w.clone())
    return torch.stack(outs), torch.stack(idxs), torch.stack(wts)


def _stack_case(q, seed, E, H, I, bits, K, nl, tokens, oracle_layers):
    layers = [DeviceLayer(seed, l, E, H, I, bits, K) for l in range(nl)]
    norm_w = [synth.norm_weight(seed, l, H) for l in range(nl)]
    dnorm = [torch.from_numpy(w).cuda() for w in norm_w]
    S = q.Stack([D.L for D in layers], dnorm)
    ws = q.alloc_stack_workspace(S)
    ws_chain = q.alloc_workspace(layers[0].L)
    for tok in tokens:  # later calls run with the next call number on the same workspace
        h0 = host_x(seed, tok, H)
        hd = torch.from_numpy(h0).cuda()
        co, ci, cw = _chain(q, layers, dnorm, hd, ws_chain)
        for persistent in (False, True):
            h_all = torch.full((nl, H), float("nan"), dtype=torch.float32, device="cuda")
            out, idx, w = q.moe_stack_forward(S, hd, 1e-6, h_all=h_all, ws=ws, persistent=persistent)
            out2, idx2, _ = q.moe_stack_forward(S, hd, 1e-6, ws=ws, persistent=persistent)  # no h_all
            torch.cuda.synchronize()
            assert _status(ws) == 0 and _status(ws_chain) == 0
            # the same arithmetic as one launch per layer: equal bit for bit
            same = [bool(torch.equal(co[l], h_all[l])) for l in range(nl)]
            say("  token", tok, "persistent" if persistent else "per layer",
                "layers equal to the single-layer launches:", sum(same), "of", nl)
            assert torch.equal(ci, idx) and torch.equal(cw, w) and torch.equal(idx2, idx)
            assert all(same) and torch.equal(out, h_all[-1]) and torch.equal(out2, out)
        # the oracle, fed the GPU's input to each checked layer
        HA, IDX, W = h_all.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
        for l in oracle_layers:
            hprev = (h0 if l == 0 else HA[l - 1]).astype(np.float64)
            xr = oracle.rmsnorm(hprev, norm_w[l], 1e-6)
            _check_layer_token(layers[l], xr, HA[l], IDX[l], W[l], residual=hprev)


STACK_CASES = [  # (E, H, I, bits, K, layers) -- fused shapes, then one the fallback chain serves
    (64, 1024, 256, 4, 4, 5), (64, 1024, 256, 2, 4, 3), (100, 2048, 512, 4, 3, 3), (16, 192, 128, 4, 2, 3),
]


@pytest.mark.parametrize("E,H,I,bits,K,nl", STACK_CASES)
def test_stack_kernel_matches_layer_launches_and_oracle(q, E, H, I, bits, K, nl):
    say("stack kernel", E, H, I, bits, K, nl)
    _stack_case(q, 1003, E, H, I, bits, K, nl, tokens=(0, 1), oracle_layers=range(nl))


def test_stack_kernel_more_layers_than_one_launch(q):
    """34 layers: two launches (32 + 2); the oracle checks the layers around the seam."""
    say("stack kernel, 34 layers")
    _stack_case(q, 1003, 64, 1024, 256, 4, 4, 34, tokens=(0,), oracle_layers=(0, 30, 31, 32, 33))


def test_stack_parity(q):
    """A 3-layer stack at the workload's per-layer shape, 2 tokens, end to end: one
    launch per layer against the oracle, and the stack kernel against both."""
    L_, E, H, I, K = 3, 512, 4096, 1024, 4
    seed = 1003
    say("stack", L_, "layers")
    layers = [DeviceLayer(seed, l, E, H, I, 4, K) for l in range(L_)]
    norm_w = [synth.norm_weight(seed, l, H) for l in range(L_)]
    dnorm = [torch.from_numpy(w).cuda() for w in norm_w]
    ws = [q.alloc_workspace(D.L) for D in layers]
    S = q.Stack([D.L for D in layers], dnorm)
    ws_s = q.alloc_stack_workspace(S)
    for tok in range(2):
        h0 = host_x(seed, tok, H)
        h = torch.from_numpy(h0).cuda()
        out_s, idx_s, _ = q.moe_stack_forward(S, h.clone(), 1e-6, ws=ws_s, persistent=True)
        gpu_idx = []
        for l, D in enumerate(layers):
            # one launch per layer, in place: h <- h + MoE(rmsnorm(h))
            _, idx, _ = q.moe_layer_forward_norm(D.L, h, dnorm[l], 1e-6, out=h, ws=ws[l])
            gpu_idx.append(idx.cpu().numpy())
        torch.cuda.synchronize()
        assert _status(ws_s) == 0
        assert torch.equal(out_s, h) and (idx_s.cpu().numpy() == np.stack(gpu_idx)).all()
        # oracle end to end; a near-tie is resolved the way the GPU did after checking validity
        hr = h0.astype(np.float64)
        for l, D in enumerate(layers):
            xr = oracle.rmsnorm(hr, norm_w[l], 1e-6)
            R = D.host_router()
            ex = check_topk(gpu_idx[l], oracle.router_logits(R, xr), oracle.topk_tolerance(R, xr), K)
            hr = oracle.moe_layer(D.host_expert, D.host_shared(), R, D.host_gate(), xr, hr, H, I, 4, K,
                                  force_idx=gpu_idx[l] if ex else None)
        r = _rel(h.cpu().numpy(), hr)
        say("  token", tok, "stack rel_l2", r)
        assert r <= TOL and r <= TIGHT


# ---------------------------------------------------------------------------
# GatedDeltaNet recurrence (one decode step per call, state updated in place)
# ---------------------------------------------------------------------------

GDN_CASES = [  # (heads, dk, dv, steps) -- ragged column counts, every dk, the model's full size
    (3, 64, 5, 3), (2, 128, 7, 3), (1, 256, 3, 3), (5, 128, 1, 2), (64, 128, 128, 4),
]


@pytest.mark.parametrize("heads,dk,dv,steps", GDN_CASES)
def test_gdn_step_parity(q, heads, dk, dv, steps):
    say("gdn", heads, dk, dv, steps)
    seed = 1005
    S0 = synth.gdn_state(seed, 0, heads, dk, dv)            # [heads][dv][dk]
    state = torch.from_numpy(S0).cuda()
    Sref = S0.transpose(0, 2, 1).astype(np.float64)         # the oracle's [heads][dk][dv]
    for t in range(steps):
        qq, kk, vv, al, be = synth.gdn_token(seed, 0, t, heads, dk, dv)
        o = q.gdn_recurrent_step(state, *(torch.from_numpy(a).cuda() for a in (qq, kk, vv, al, be)))
        Sref, oref = oracle.gdn_step(Sref, qq, kk, vv, al, be)
        torch.cuda.synchronize()
        rs = _rel(state.cpu().numpy().transpose(0, 2, 1), Sref)
        ro = _rel(o.cpu().numpy(), oref)
        say("  step", t, "state rel_l2", rs, "o rel_l2", ro)
        assert rs <= 1e-5 and ro <= 1e-5


def test_gdn_zero_heads_and_untouched_tail(q):
    """heads = 0 does nothing; a step writes only the state and o it owns (guard
    words around both stay as they were)."""
    st = torch.full((2, 3, 64), 7.0, device="cuda")
    o = q.gdn_recurrent_step(st[:0], *(torch.zeros(s, device="cuda") for s in ((0, 64), (0, 64), (0, 3), (0,), (0,))))
    assert o.numel() == 0 and bool((st == 7.0).all())
    big = torch.full((2 * 3 * 64 + 64,), -1.0, device="cuda")
    state = big[:2 * 3 * 64].view(2, 3, 64)
    state.fill_(0.5)
    ob = torch.full((2 * 3 + 16,), -2.0, device="cuda")
    qq, kk, vv, al, be = synth.gdn_token(1005, 1, 0, 2, 64, 3)
    q.gdn_recurrent_step(state, *(torch.from_numpy(a).cuda() for a in (qq, kk, vv, al, be)), o=ob[:6].view(2, 3))
    torch.cuda.synchronize()
    assert bool((big[2 * 3 * 64:] == -1.0).all()) and bool((ob[6:] == -2.0).all())
    Sref, oref = oracle.gdn_step(np.full((2, 64, 3), 0.5), qq, kk, vv, al, be)
    assert _rel(state.cpu().numpy().transpose(0, 2, 1), Sref) <= 1e-5
    assert _rel(ob[:6].cpu().numpy().reshape(2, 3), oref) <= 1e-5


# ---------------------------------------------------------------------------
# full-attention decode (RoPE, cache append, grouped-query attention)
# ---------------------------------------------------------------------------

ATTN_CASES = [  # (Hq, Hkv, D, Tmax, pos, rot_dim, theta) -- ragged tiles, one key, 16:1 groups,
    (4, 2, 64, 40, 37, 64, 1e4),        # partial and no rotation, the full 4096-key context
    (3, 1, 128, 100, 0, 128, 1e4), (16, 1, 256, 300, 299, 64, 1e7), (8, 8, 128, 65, 64, 0, 1e4),
    (32, 2, 256, 4096, 4095, 64, 1e7),
    (32, 2, 256, 8192, 8191, 64, 1e7),  # the benchmark's shape and launch: 128 ranges per KV head
    (8, 1, 128, 16384, 16383, 128, 1e6),  # 256 ranges: the merge takes its loads in two batches
]


def _attn_check(q, Hq, Hkv, D, Tmax, pos, rot, theta, tokens, seed=1006):
    K0, V0 = synth.attn_cache(seed, 0, Hkv, Tmax, D)
    kc, vc = torch.from_numpy(K0).cuda(), torch.from_numpy(V0).cuda()
    kc[:, pos + 1:] = float("nan")  # rows past the token must never be read
    vc[:, pos + 1:] = float("nan")
    ws = torch.empty(q.qmoe_attn_workspace_bytes(Hq, Hkv, D, Tmax), dtype=torch.uint8, device="cuda")
    for i in range(tokens):
        p = pos + i
        Kh, Vh = kc.cpu().numpy(), vc.cpu().numpy()  # the caches as the GPU holds them before the token
        qq, kk, vv = synth.attn_token(seed, 0, p, Hq, Hkv, D)
        o = q.attn_decode_step(*(torch.from_numpy(a).cuda() for a in (qq, kk, vv)), kc, vc, p, theta, rot, ws=ws)
        torch.cuda.synchronize()
        oref, Kref, Vref = oracle.attn_decode(qq, kk, vv, np.nan_to_num(Kh), np.nan_to_num(Vh), p, theta, rot)
        r = _rel(o.cpu().numpy(), oref)
        say("  pos", p, "o rel_l2", r)
        assert r <= 1e-4
        K2, V2 = kc.cpu().numpy(), vc.cpu().numpy()
        assert _rel(K2[:, p], Kref[:, p]) <= 1e-6 and np.array_equal(V2[:, p], vv)
        assert np.array_equal(K2[:, :p], Kh[:, :p]) and np.array_equal(V2[:, :p], Vh[:, :p])
        assert np.isnan(K2[:, p + 1:]).all() and np.isnan(V2[:, p + 1:]).all()


@pytest.mark.parametrize("Hq,Hkv,D,Tmax,pos,rot,theta", ATTN_CASES)
def test_attn_decode_parity(q, Hq, Hkv, D, Tmax, pos, rot, theta):
    say("attention decode", Hq, Hkv, D, Tmax, pos, rot, theta)
    _attn_check(q, Hq, Hkv, D, Tmax, pos, rot, theta, tokens=1)


def test_attn_decode_consecutive_tokens(q):
    """Three tokens in a row: each appends its key and value and sees the earlier ones."""
    say("attention decode, 3 tokens")
    _attn_check(q, 8, 2, 128, 200, 60, 128, 1e6, tokens=3)


QGATE_CASES = [  # (Hq, Hkv, D, Tmax, pos, rot_dim, theta, q norm, k norm)
    (4, 2, 64, 40, 37, 64, 1e4, True, True), (16, 1, 256, 300, 299, 64, 1e7, True, True),
    (8, 8, 128, 65, 0, 0, 1e4, False, True), (32, 2, 256, 4096, 4095, 64, 1e7, True, False),
    (3, 1, 128, 100, 50, 128, 1e4, False, False),
]


@pytest.mark.parametrize("Hq,Hkv,D,Tmax,pos,rot,theta,qn,kn", QGATE_CASES)
def test_attn_decode_qgate_parity(q, Hq, Hkv, D, Tmax, pos, rot, theta, qn, kn):
    """The query projection's rows de-interleaved into query and gate, q and k
    RMS-normalised per head (when weighted), then RoPE, cache append and attention:
    against the oracle, three tokens in a row."""
    say("attention decode qgate", Hq, Hkv, D, Tmax, pos, rot, theta, qn, kn)
    seed = 1007
    K0, V0 = synth.attn_cache(seed, 0, Hkv, Tmax, D)
    kc, vc = torch.from_numpy(K0).cuda(), torch.from_numpy(V0).cuda()
    kc[:, pos + 1:] = float("nan")
    vc[:, pos + 1:] = float("nan")
    wq, wk = synth.attn_norm_weights(seed, 0, D)
    dwq = torch.from_numpy(wq).cuda() if qn else None
    dwk = torch.from_numpy(wk).cuda() if kn else None
    for i in range(min(3, Tmax - pos)):
        p = pos + i
        Kh, Vh = kc.cpu().numpy(), vc.cpu().numpy()
        qg, kk, vv = synth.attn_token_qg(seed, 0, p, Hq, Hkv, D)
        o, gate = q.attn_decode_step_qgate(*(torch.from_numpy(a).cuda() for a in (qg, kk, vv)), kc, vc, p,
                                           theta, rot, q_norm_w=dwq, k_norm_w=dwk, eps=1e-6)
        torch.cuda.synchronize()
        oref, gref, Kref, Vref = oracle.attn_decode_qgate(qg, kk, vv, np.nan_to_num(Kh), np.nan_to_num(Vh), p,
                                                          theta, rot, wq if qn else None, wk if kn else None,
                                                          1e-6)
        r = _rel(o.cpu().numpy(), oref)
        say("  pos", p, "o rel_l2", r)
        assert r <= 1e-4
        assert np.array_equal(gate.cpu().numpy(), gref.astype(np.float32))
        K2, V2 = kc.cpu().numpy(), vc.cpu().numpy()
        assert _rel(K2[:, p], Kref[:, p]) <= 1e-6 and np.array_equal(V2[:, p], vv)
        assert np.array_equal(K2[:, :p], Kh[:, :p]) and np.array_equal(V2[:, :p], Vh[:, :p])
        assert np.isnan(K2[:, p + 1:]).all() and np.isnan(V2[:, p + 1:]).all()
