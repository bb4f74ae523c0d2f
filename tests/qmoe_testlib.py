"""Shared helpers of the GPU tests: build a layer in HBM from the seeded
generators, and regenerate on the host whatever the oracle needs."""
from __future__ import annotations

import numpy as np
import torch

import synth

SEEDS = {"config0": 1000, "config1": 1001, "config2": 1002, "config3": 1003, "config4": 1004}


class DeviceLayer:
    """A MoE layer generated in HBM plus the recipe to regenerate it on the host."""

    def __init__(self, seed, layer, E, H, I, bits, K, device="cuda"):
        import bit_dequant_gemv_amd as q
        self.seed, self.layer, self.E, self.H, self.I, self.bits, self.K = seed, layer, E, H, I, bits, K
        self.routed = q.ExpertPool.allocate(E, H, I, bits, device)
        self.shared = q.ExpertPool.allocate(1, H, I, bits, device)
        synth.fill_expert_pool(self.routed.buf, self.routed.stride, E, 0, layer, seed, H, I, bits)
        synth.fill_expert_pool(self.shared.buf, self.shared.stride, 1, E, layer, seed, H, I, bits)
        self.router = torch.empty(E, H, dtype=torch.int16, device=device)
        synth.fill_normal_bf16(self.router, seed, synth.tensor_id(synth.K_ROUTER, 0, layer),
                               synth.ROUTER_SIGMA)
        self.gate = torch.empty(H, dtype=torch.int16, device=device)
        synth.fill_normal_bf16(self.gate, seed, synth.tensor_id(synth.K_SHARED_GATE, 0, layer),
                               synth.SHARED_GATE_SIGMA)
        self.L = q.Layer(self.routed, self.shared, self.router, self.gate, K)
        self._cache = {}

    # host side (oracle inputs), regenerated from the seeds -- never read back
    def host_expert(self, e):
        if e not in self._cache:
            self._cache[e] = synth.expert_block(self.seed, self.layer, e, self.H, self.I, self.bits)
        return self._cache[e]

    def host_shared(self):
        return self.host_expert(self.E)

    def host_router(self):
        if "router" not in self._cache:
            self._cache["router"] = synth.router(self.seed, self.layer, self.E, self.H)
        return self._cache["router"]

    def host_gate(self):
        return synth.shared_gate(self.seed, self.layer, self.H)


def host_x(seed, token, H):
    return synth.activations(seed, token, H)


def device_x(seed, tokens, H, device="cuda"):
    return torch.from_numpy(np.stack([host_x(seed, t, H) for t in tokens])).to(device)


def check_topk(gpu_idx, oracle_logits, tau, K):
    """Expert ids must equal the oracle's top-K unless an fp32 near-tie makes the
    choice ambiguous (gap below tau); returns the number of exempted near-ties."""
    gpu_idx = [int(v) for v in gpu_idx]
    key = oracle_logits.astype(np.float32).astype(np.float64)
    order = sorted(range(key.size), key=lambda e: (-key[e], e))
    want = order[:K]
    if gpu_idx == want:
        return 0
    # every selected expert must be within tau of the boundary where it differs
    kth = key[want[-1]]
    nxt = key[order[K]] if K < key.size else -np.inf
    exempt = 0
    assert len(set(gpu_idx)) == K, gpu_idx
    for pos, (g, o) in enumerate(zip(gpu_idx, want)):
        if g == o:
            continue
        if abs(key[g] - key[o]) <= tau[g] + tau[o]:
            exempt += 1
            continue
        raise AssertionError(f"top-K mismatch at {pos}: gpu {gpu_idx} oracle {want} "
                             f"(logits {key[g]} vs {key[o]}, kth {kth}, next {nxt})")
    return exempt
