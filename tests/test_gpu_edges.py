"""Edge cases of the HIP path against the float64 CPU oracle (through the C ABI).

* exact ties inside the fused layer's own ranking (all logits equal: every
  expert is a candidate; three identical dominant router rows);
* the batched layer row by row against the single-token layer, and on sampled
  rows spanning both of the shared expert's token chunks against the oracle;
* activations that stress the 24-bit block fixed point the kernels read x in
  (magnitudes 1e4 and 1e-4 in one 32-element chunk, an all-zero chunk, a chunk
  in the fp32 denormal range, non-finite values);
* the shape limits: the fused layer at E = 1000 and 2048, qgemv_w2 at 16384
  columns and qgemv_w4 at 8192.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from qmoe_testlib import DeviceLayer, check_topk, device_x, host_x

pytestmark = pytest.mark.gpu

TOL = 1e-3
TIGHT = 1e-4


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def q():
    import bit_dequant_gemv_amd as q
    return q


def _rel(a, b):
    return oracle.rel_l2(np.asarray(a, dtype=np.float64), b)


def _status(ws):
    return int(ws[4:8].view(torch.int32).item())


def _set_router(D, R):
    """Replace a device layer's router (bf16 bits [E][H]) on both sides."""
    D.router.copy_(torch.from_numpy(np.ascontiguousarray(R).view(np.int16)))
    D._cache["router"] = np.ascontiguousarray(R)


def _layer_vs_oracle(D, x, out, idx, w, residual=None):
    residual = x if residual is None else residual
    R = D.host_router()
    logits = oracle.router_logits(R, x)
    ex = check_topk(idx, logits, oracle.topk_tolerance(R, x), D.K)
    ref = oracle.moe_layer(D.host_expert, D.host_shared(), R, D.host_gate(), x, residual,
                           D.H, D.I, D.bits, D.K, force_idx=idx if ex else None)
    r = _rel(out, ref)
    err = float(np.max(np.abs(np.asarray(out, np.float64) - ref)))
    say("  idx", list(idx), "near-ties", ex, "rel_l2", r, "max abs err", err,
        "max |ref|", float(np.max(np.abs(ref))))
    assert r <= TOL and r <= TIGHT
    sel = logits[np.asarray(idx)]
    ref_w = np.exp(sel - sel.max())
    assert _rel(w, ref_w / ref_w.sum()) <= TIGHT
    return ex


# ---------------------------------------------------------------------------
# exact ties in the fused layer's ranking
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("E,bits", [(512, 4), (2048, 4), (512, 2)])
def test_layer_all_logits_equal(q, E, bits):
    """A zero router: E equal logits, so every expert is a candidate of the fused
    kernel's ranking (its loops past 8 and past 64 candidates).  The picks are the
    K lowest indices with equal weights, in the single-token and batched paths."""
    say("layer, all logits equal", E, bits)
    D = DeviceLayer(7100 + E + bits, 0, E, 4096, 1024, bits, 4)
    _set_router(D, np.zeros((E, 4096), np.uint16))
    ws = q.alloc_workspace(D.L)
    for tok in range(2):
        x = host_x(D.seed, tok, 4096)
        out, idx, w = q.moe_layer_forward(D.L, torch.from_numpy(x).cuda(), ws=ws)
        torch.cuda.synchronize()
        assert _status(ws) == 0
        assert idx.cpu().numpy().tolist() == [0, 1, 2, 3]
        assert w.cpu().numpy().tolist() == [0.25] * 4
        _layer_vs_oracle(D, x, out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy())
    if E == 512:
        T = 8
        X = device_x(D.seed, range(T), 4096)
        wsb = q.alloc_workspace(D.L, T)
        outb, idxb, wb = q.moe_layer_forward_batched(D.L, X, ws=wsb)
        torch.cuda.synchronize()
        assert (idxb.cpu().numpy() == np.arange(4)[None, :]).all()
        assert (wb.cpu().numpy() == 0.25).all()
        _layer_vs_oracle(D, X[5].cpu().numpy(), outb[5].cpu().numpy(), idxb[5].cpu().numpy(),
                         wb[5].cpu().numpy())


def test_layer_identical_dominant_rows(q):
    """One router row parallel to x copied to experts 7, 300 and 450: three equal
    largest logits, picked in index order with equal weights by the fused layer
    and by the batched layer."""
    say("layer, three identical dominant rows")
    E, H = 512, 4096
    D = DeviceLayer(7200, 0, E, H, 1024, 4, 4)
    x = host_x(D.seed, 0, H)
    R = D.host_router().copy()
    R[7] = synth.f32_to_bf16_bits((0.02 * x).astype(np.float32))
    R[300] = R[7]
    R[450] = R[7]
    _set_router(D, R)
    ws = q.alloc_workspace(D.L)
    out, idx, w = q.moe_layer_forward(D.L, torch.from_numpy(x).cuda(), ws=ws)
    torch.cuda.synchronize()
    got, wt = idx.cpu().numpy(), w.cpu().numpy()
    assert got[:3].tolist() == [7, 300, 450], got
    assert wt[0] == wt[1] == wt[2]
    _layer_vs_oracle(D, x, out.cpu().numpy(), got, wt)
    X = torch.from_numpy(np.tile(x, (4, 1))).cuda()
    wsb = q.alloc_workspace(D.L, 4)
    outb, idxb, wb = q.moe_layer_forward_batched(D.L, X, ws=wsb)
    torch.cuda.synchronize()
    for t in range(4):
        assert idxb[t].cpu().numpy().tolist() == got.tolist()
        wbt = wb[t].cpu().numpy()
        assert wbt[0] == wbt[1] == wbt[2]
        # another kernel's softmax: equal up to rounding
        assert _rel(wbt, wt.astype(np.float64)) <= 1e-6
        assert _rel(outb[t].cpu().numpy(), out.cpu().numpy().astype(np.float64)) <= 1e-5


# ---------------------------------------------------------------------------
# batched decode, every row
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("E,H,I,bits,K,T", [(512, 4096, 1024, 4, 4, 64), (512, 4096, 1024, 2, 4, 40),
                                            (64, 1024, 256, 4, 4, 64), (8, 256, 128, 4, 8, 33)])
def test_batched_every_row(q, E, H, I, bits, K, T):
    """Every row of a batch against the single-token fused layer (same selection:
    within 1e-5; a different one only at an exempted near-tie, at most two rows),
    and rows spanning both 32-token chunks of the shared expert (every row for the
    small shapes, every fourth for the workload's) against the oracle."""
    say("batched every row", E, H, I, bits, K, T)
    D = DeviceLayer(7300 + E + bits + T, 0, E, H, I, bits, K)
    X = device_x(D.seed, range(T), H)
    ws = q.alloc_workspace(D.L, T)
    out, idx, w = q.moe_layer_forward_batched(D.L, X, ws=ws)
    torch.cuda.synchronize()
    out, idx, w = out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    Xh = X.cpu().numpy()
    R = D.host_router()
    ws1 = q.alloc_workspace(D.L)
    differ = 0
    worst = 0.0
    for t in range(T):
        o1, i1, w1 = q.moe_layer_forward(D.L, X[t].contiguous(), ws=ws1)
        i1 = i1.cpu().numpy()
        if (i1 == idx[t]).all():
            r = _rel(out[t], o1.cpu().numpy().astype(np.float64))
            worst = max(worst, r)
            assert r <= 1e-5, (t, r)
            assert _rel(w[t], w1.cpu().numpy().astype(np.float64)) <= 1e-6
        else:  # both selections must be valid for the oracle's logits
            differ += 1
            lg = oracle.router_logits(R, Xh[t])
            tau = oracle.topk_tolerance(R, Xh[t])
            check_topk(idx[t], lg, tau, K)
            check_topk(i1, lg, tau, K)
    say("  rows vs single-token layer: worst rel_l2", worst, "selections differing", differ)
    assert differ <= 2
    rows = range(T) if E < 512 else range(0, T, 4)
    for t in rows:
        _layer_vs_oracle(D, Xh[t], out[t], idx[t], w[t])


# ---------------------------------------------------------------------------
# activations that stress the block fixed point of x
# ---------------------------------------------------------------------------

def _stress_x(n, seed, chunk=32):
    """N(0,1) except: chunk 0 alternates +-1e4 and 1e-4 magnitudes, chunk 1 is all
    zero, chunk 2 lies in the fp32 denormal range (|x| ~ 1e-39), chunk 3 mixes
    1e-30 and 1.0."""
    x = synth.normal_f32(seed, 1, n, 1.0).copy()
    c0 = np.where(np.arange(chunk) % 2 == 0, 1e4, 1e-4) * np.where(np.arange(chunk) % 3 == 0, -1, 1)
    x[0:chunk] = c0
    x[chunk:2 * chunk] = 0.0
    x[2 * chunk:3 * chunk] = (synth.normal_f32(seed, 2, chunk, 1.0) * np.float32(1e-39)).astype(np.float32)
    x[3 * chunk:4 * chunk] = np.where(np.arange(chunk) % 2 == 0, 1e-30, 1.0)
    return x.astype(np.float32)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("rows,cols", [(256, 4096), (33, 1024)])
def test_qgemv_block_fixed_point_edges(q, bits, rows, cols):
    say("qgemv x edges", bits, rows, cols)
    codes, sb = synth.matrix(8800 + rows, 0, 0, 0, rows, cols, bits)
    chunk = 32 if bits == 4 else 64
    x = _stress_x(cols, 8801, chunk)
    fn = q.qgemv_w4 if bits == 4 else q.qgemv_w2
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(sb.view(np.int32)).cuda()
    y = fn(dc, ds, torch.from_numpy(x).cuda()).cpu().numpy()
    ref = oracle.qgemv(codes, sb, x, bits)
    r = _rel(y, ref)
    err = np.abs(y.astype(np.float64) - ref)
    say("  rel_l2", r, "max abs err", float(err.max()), "max rel err per row",
        float(np.max(err / np.abs(ref))))
    assert r <= TIGHT
    # the same matrix with the large chunk removed: the small chunks alone
    x2 = x.copy()
    x2[:chunk] = 0.0
    y2 = fn(dc, ds, torch.from_numpy(x2).cuda()).cpu().numpy()
    r2 = _rel(y2, oracle.qgemv(codes, sb, x2, bits))
    say("  without the 1e4 chunk: rel_l2", r2)
    assert r2 <= TIGHT


@pytest.mark.parametrize("bits", [4, 2])
def test_qgemv_non_finite_input(q, bits):
    """A NaN or an infinity in x makes every output non-finite, as in the oracle
    (the GPU's value is NaN: the chunk's scale becomes NaN)."""
    say("qgemv non-finite", bits)
    rows, cols = 64, 512
    codes, sb = synth.matrix(8900, 0, 0, 0, rows, cols, bits)
    fn = q.qgemv_w4 if bits == 4 else q.qgemv_w2
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(sb.view(np.int32)).cuda()
    for bad in (np.nan, np.inf, -np.inf):
        x = synth.normal_f32(8901, 0, cols, 1.0).copy()
        x[200] = bad
        y = fn(dc, ds, torch.from_numpy(x).cuda()).cpu().numpy()
        with np.errstate(invalid="ignore"):
            ref = oracle.qgemv(codes, sb, x, bits)
        assert not np.isfinite(ref).any()
        assert np.isnan(y).all(), bad


def test_layer_block_fixed_point_edges(q):
    """The fused layer on an input with the stress chunks (the router and every
    expert's gate/up read it; the down rows read h, whose chunks then hold very
    different magnitudes too)."""
    say("layer x edges")
    for (E, H, I, bits) in [(64, 1024, 256, 4), (64, 1024, 256, 2), (512, 4096, 1024, 4)]:
        D = DeviceLayer(9000 + E + bits, 0, E, H, I, bits, 4)
        ws = q.alloc_workspace(D.L)
        x = _stress_x(H, 9001 + H, 32 if bits == 4 else 64)
        out, idx, w = q.moe_layer_forward(D.L, torch.from_numpy(x).cuda(), ws=ws)
        torch.cuda.synchronize()
        assert _status(ws) == 0
        say(" ", E, H, I, bits)
        _layer_vs_oracle(D, x, out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy())


# ---------------------------------------------------------------------------
# shape limits
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("E", [1000, 2048])
def test_layer_many_experts(q, E):
    """The fused layer at E = 1000 (a partial last pass of router rows, logits
    past the first 512 polled in the loop) and at its limit of 2048."""
    say("layer many experts", E)
    D = DeviceLayer(9100 + E, 0, E, 4096, 1024, 4, 4)
    ws = q.alloc_workspace(D.L)
    for tok in range(2):
        x = host_x(D.seed, tok, 4096)
        out, idx, w = q.moe_layer_forward(D.L, torch.from_numpy(x).cuda(), ws=ws)
        torch.cuda.synchronize()
        assert _status(ws) == 0
        _layer_vs_oracle(D, x, out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy())


@pytest.mark.parametrize("bits,rows,cols", [(2, 100, 16384), (2, 1, 16384), (4, 300, 8192)])
def test_qgemv_column_limit(q, bits, rows, cols):
    say("qgemv column limit", bits, rows, cols)
    codes, sb = synth.matrix(9200 + rows, 0, 0, 0, rows, cols, bits)
    x = synth.normal_f32(9201, 0, cols, 1.0)
    fn = q.qgemv_w4 if bits == 4 else q.qgemv_w2
    y = fn(torch.from_numpy(codes).cuda(), torch.from_numpy(sb.view(np.int32)).cuda(),
           torch.from_numpy(x).cuda()).cpu().numpy()
    r = _rel(y, oracle.qgemv(codes, sb, x, bits))
    say("  rel_l2", r)
    assert r <= TIGHT
