"""The allocation-free layer entry point (moe_layer_forward_noalloc) against
moe_layer_forward, which runs the same kernel on a caller's workspace: two
calls in a row, the second on a smaller layer, each with equal results."""
import sys

import numpy as np
import pytest
import torch

from qmoe_testlib import DeviceLayer, host_x

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _run_both(q, D, x):
    ws = q.alloc_workspace(D.L)
    xd = torch.from_numpy(x).cuda()
    ref_out, ref_idx, ref_w = q.moe_layer_forward(D.L, xd, ws=ws)
    out = torch.full_like(xd, float("nan"))
    idx = torch.full((D.K,), -7, dtype=torch.int32, device="cuda")
    w = torch.full((D.K,), float("nan"), device="cuda")
    q.moe_layer_forward_noalloc(D.L, xd, xd, out, idx, w)
    torch.cuda.synchronize()
    assert int(ws[4:8].view(torch.int32).item()) == 0
    return (ref_out, ref_idx, ref_w), (out, idx, w)


def test_noalloc_matches_workspace_entry_point_twice(q=None):
    import bit_dequant_gemv_amd as q
    cases = [(512, 4096, 1024, 4, 4, 1001), (64, 1024, 256, 2, 4, 4001)]  # second: smaller
    for E, H, I, bits, K, seed in cases:
        say("noalloc layer", E, H, I, bits, K)
        D = DeviceLayer(seed, 0, E, H, I, bits, K)
        for tok in range(2):
            (ro, ri, rw), (o, i, w) = _run_both(q, D, host_x(seed, tok, H))
            say("  token", tok, "idx", i.cpu().numpy().tolist(), "ref", ri.cpu().numpy().tolist())
            assert torch.equal(i, ri) and torch.equal(w, rw)
            assert torch.equal(o, ro), float((o - ro).abs().max())


def test_noalloc_rejects_too_large_a_layer():
    """A layer whose workspace exceeds the 1 MiB scratch is refused before launch."""
    import bit_dequant_gemv_amd as q
    say("noalloc too large")
    big = DeviceLayer(4002, 0, 4, 1024, 8192, 4, 2)  # inter 8192: 1.3 MiB of h slots
    need = q.qmoe_workspace_bytes(big.L)
    assert need > 1 << 20
    x = torch.zeros(big.H, device="cuda")
    with pytest.raises(q.QmoeError) as ei:
        q.moe_layer_forward_noalloc(big.L, x)
    assert ei.value.status == q.QMOE_EWORKSPACE
