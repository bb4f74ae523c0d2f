"""Host-tier expert offload (moe_layer_forward_offload): routed experts in pinned
host memory, an LRU cache of expert slots in HBM.  Each token's output and routing
against the layer with every expert resident (moe_layer_forward) and against the
oracle; the cache's hit and miss counts against an LRU model of the same
sequence."""
import sys
from collections import OrderedDict

import numpy as np
import pytest
import torch

import oracle
from qmoe_testlib import DeviceLayer, check_topk, host_x

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _host_copy(q, D):
    """The routed pool of a device layer copied into pinned host memory."""
    buf = torch.empty(D.routed.buf.numel(), dtype=torch.uint8, pin_memory=True)
    buf.copy_(D.routed.buf)
    return q.ExpertPool(buf, D.E, D.H, D.I, D.bits, D.routed.stride)


class LruModel:
    """Which experts hit: a slot cache of n entries, least recently used out, the
    experts of one token never evicting each other."""

    def __init__(self, n):
        self.n, self.d = n, OrderedDict()

    def token(self, experts):
        hits = misses = 0
        seen = set()  # this token's experts handled so far: never evicted by it
        for e in experts:
            if e in self.d:
                hits += 1
                self.d.move_to_end(e)
            else:
                misses += 1
                if len(self.d) >= self.n:
                    for old in self.d:  # least recently used first
                        if old not in seen:
                            del self.d[old]
                            break
                self.d[e] = True
            seen.add(e)
        return hits, misses


@pytest.mark.parametrize("E,H,I,bits,K,slots,tokens", [(64, 1024, 256, 4, 4, 8, 24), (16, 256, 128, 2, 3, 3, 12),
                                                        (512, 4096, 1024, 4, 4, 64, 6)])
def test_offload_matches_resident_layer_and_oracle(E, H, I, bits, K, slots, tokens):
    import bit_dequant_gemv_amd as q
    say("offload", E, H, I, bits, K, slots, tokens)
    D = DeviceLayer(8100 + E + bits, 0, E, H, I, bits, K)
    hp = _host_copy(q, D)
    torch.cuda.synchronize()
    off = q.Offload(hp, slots)
    L_off = q.Layer(hp, D.shared, D.router, D.gate, K)
    ws_res = q.alloc_workspace(D.L)
    copy_stream = torch.cuda.Stream()
    model = LruModel(slots)
    R = D.host_router()
    seq = list(range(tokens)) + [tokens - 1]  # the last token again: all hits
    for n, t in enumerate(seq):
        x = host_x(D.seed, t, H)
        xd = torch.from_numpy(x).cuda()
        out, idx, w = q.moe_layer_forward_offload(off, L_off, xd, copy_stream=copy_stream)
        ref_out, ref_idx, ref_w = q.moe_layer_forward(D.L, xd, ws=ws_res)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        lg = oracle.router_logits(R, x)
        ex = check_topk(got, lg, oracle.topk_tolerance(R, x), K)
        if torch.equal(idx, ref_idx):
            r = oracle.rel_l2(out.cpu().numpy().astype(np.float64), ref_out.cpu().numpy().astype(np.float64))
            assert r <= 1e-5, (t, r)
        if n % 4 == 0 or n == len(seq) - 1:
            ref = oracle.moe_layer(D.host_expert, D.host_shared(), R, D.host_gate(), x, x, H, I, bits, K,
                                   force_idx=got if ex else None)
            r = oracle.rel_l2(out.cpu().numpy(), ref)
            say("  token", t, "idx", got.tolist(), "rel_l2 vs oracle", r)
            assert r <= 1e-4
        h, m = model.token([int(e) for e in got])
        st = off.stats()
        assert st["calls"] == n + 1
        model.hits = getattr(model, "hits", 0) + h
        model.misses = getattr(model, "misses", 0) + m
        assert (st["hits"], st["misses"]) == (model.hits, model.misses), (st, model.hits, model.misses)
    st = off.stats()
    say("  stats", st)
    assert st["bytes_copied"] == st["misses"] * q.qmoe_expert_layout(H, I, bits)["total"]
    off.close()


def test_offload_rejects_bad_arguments():
    import bit_dequant_gemv_amd as q
    say("offload bad arguments")
    D = DeviceLayer(8200, 0, 16, 256, 128, 4, 4)
    hp = _host_copy(q, D)
    with pytest.raises(q.QmoeError):
        q.Offload(hp, 0)  # no slots
    off = q.Offload(hp, 2)  # fewer slots than top-K
    L_off = q.Layer(hp, D.shared, D.router, D.gate, 4)
    with pytest.raises(q.QmoeError) as ei:
        q.moe_layer_forward_offload(off, L_off, torch.zeros(256, device="cuda"))
    assert ei.value.status == q.QMOE_ESHAPE
    off.close()
