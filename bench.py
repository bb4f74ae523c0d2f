"""Benchmark of the batch-1 quantized MoE hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]

Workloads (all weights 4-bit unless noted; H = 4096, I = 1024, group 64):
  --config 1 (default)  one MoE layer at batch 1: router over 512 resident experts,
                        top-4 + shared expert, SwiGLU, combine; a step is one token
  --config 2            the same layer with 2-bit experts
  --config 0            one expert FFN call (gate, up, SwiGLU, down) on an expert
                        picked from 256 resident ones; a step is one call
  --config 3            a 60-layer stack (218 GB resident), RMSNorm before each
                        layer; a step is one token through all 60 layers
  --config 4            batched decode of 64 tokens through the config-1 layer;
                        a step is one batch
  --config 5            one GatedDeltaNet recurrence step (64 heads x 128x128
                        fp32 state) on a ring of 128 resident states; a step is
                        one call
  --config 6            one full-attention decode token (32 query heads over 2 KV
                        heads of 256, context 8192, fp32 caches) on a ring of 16
                        caches; a step is one call
  --config 7            the config-1 layer with its routed experts in pinned host
                        memory and a 256-slot HBM cache (host-tier offload); a step
                        is one token
Inputs are synthetic (seeded Philox streams generated in HBM); weights and
activations are resident in HBM before the timed region starts.  Steps are
enqueued as replays of HIP graphs, so the host never synchronises inside the
timed region.

Prints one JSON line.  `roofline.achieved` is the algorithmic bytes of one launch
of the dominant kernel (for configs 0 and 4: of one call, all its kernels) divided
by its average duration over the timed region (HIP events on the launch stream);
`cpu_baseline` times the float64 oracle on a bounded sample of the same workload
on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("4-bit expert GEMV effective GB/s (% of HBM peak); MoE-layer tokens/s at batch 1")
HBM_PEAK_GBPS = 8000.0

H, I, E, K = 4096, 1024, 512, 4


def expert_bytes(bits: int) -> int:
    """Bytes of one expert block: gate, up (I x H) and down (H x I) codes plus one
    u32 scale/bias word per row and group of 64."""
    gu = I * H * bits // 8
    return 2 * gu + H * I * bits // 8 + 4 * (2 * I * (H // 64) + H * (I // 64))


def layer_bytes(bits: int) -> int:
    """Algorithmic HBM bytes of one batch-1 layer evaluation: router (bf16 E x H),
    K routed + 1 shared expert blocks, shared-gate vector (bf16 H), and x, residual
    and out (fp32 H each)."""
    return E * H * 2 + (K + 1) * expert_bytes(bits) + H * 2 + 3 * H * 4


# the kernel sources each counter record depends on (a change elsewhere leaves it valid)
TRAFFIC_SOURCES = {
    "k_layer_w4": ["layer.hip", "qmoe_handoff.h", "qmoe_device.h"],
    "k_layer_w2": ["layer.hip", "qmoe_handoff.h", "qmoe_device.h"],
    "k_layer_w4_stack60": ["layer.hip", "qmoe_handoff.h", "qmoe_device.h"],
    "expert_ffn_w4": ["ffn.hip", "qmoe_handoff.h", "qmoe_device.h"],
    "batched64_w4": ["batched.hip", "kernels.hip", "qmoe_device.h"],
    "k_gdn": ["gdn.hip"],
    "k_attn_mma": ["attn.hip"],
}


def sources_sha(files=None) -> str:
    """Hash of the kernel sources' code (all of csrc/, or the given files):
    comment-only lines and blank lines are left out, so editing a comment does not
    invalidate counters taken on the same code."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_dequant_gemv_amd", "csrc")
    for f in sorted(files if files is not None else os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            for line in open(os.path.join(csrc, f), encoding="utf-8"):
                t = line.strip()
                if t and not t.startswith("//"):
                    h.update(t.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current sources of that kernel; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        rec = d.get(kernel_key)
        if rec and rec.get("sources_sha") == sources_sha(TRAFFIC_SOURCES.get(kernel_key)):
            return rec.get("bytes_per_launch")
    except Exception:
        return None
    return None


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

class LayerWorkload:
    def __init__(self, seed, layer, bits, torch, q, synth):
        self.bits = bits
        self.seed = seed
        self.layer = layer
        self.routed = q.ExpertPool.allocate(E, H, I, bits)
        self.shared = q.ExpertPool.allocate(1, H, I, bits)
        synth.fill_expert_pool(self.routed.buf, self.routed.stride, E, 0, layer, seed, H, I, bits)
        synth.fill_expert_pool(self.shared.buf, self.shared.stride, 1, E, layer, seed, H, I, bits)
        self.router = torch.empty(E, H, dtype=torch.int16, device="cuda")
        synth.fill_normal_bf16(self.router, seed, synth.tensor_id(synth.K_ROUTER, 0, layer), synth.ROUTER_SIGMA)
        self.gate = torch.empty(H, dtype=torch.int16, device="cuda")
        synth.fill_normal_bf16(self.gate, seed, synth.tensor_id(synth.K_SHARED_GATE, 0, layer),
                               synth.SHARED_GATE_SIGMA)
        self.L = q.Layer(self.routed, self.shared, self.router, self.gate, K)
        self.ws = q.alloc_workspace(self.L)


def make_x_ring(torch, synth, seed, n):
    X = torch.empty(n, H, dtype=torch.float32, device="cuda")
    for t in range(n):
        synth.fill_normal_f32(X[t], seed, synth.tensor_id(synth.K_X, t % 4096, t // 4096), 1.0)
    return X


def capture_graphs(torch, fn_list, per_graph):
    """Capture the callables in fn_list into graphs of per_graph consecutive launches."""
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fn_list[:per_graph]:  # warm-up on the side stream (library state, allocator)
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for g0 in range(0, len(fn_list), per_graph):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fn_list[g0:g0 + per_graph]:
                f()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def warm_for(torch, fn, seconds):
    """Run fn repeatedly for at least `seconds` of wall time (then synchronise), so
    that a bandwidth measurement starts in steady state."""
    import time
    t0 = time.perf_counter()
    while True:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def time_graphs(torch, graphs, n_replays, warmup_replays, tail=None):
    """Replay graphs round-robin (plus one optional tail graph) between two
    synchronisations; returns the seconds between the events around the timed
    replays, recorded on the stream the graphs run on."""
    for i in range(warmup_replays):
        graphs[i % len(graphs)].replay()
    if tail is not None:  # a graph's first replay carries one-time costs: not in the timed region
        tail.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(n_replays):
        graphs[i % len(graphs)].replay()
    if tail is not None:
        tail.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3


def cpu_oracle_layer(seed, layer, bits, tokens, target_s=15.0):
    """Time the oracle on host-resident inputs for a few tokens (bounded sample)."""
    import numpy as np

    import oracle
    import synth
    R = synth.router(seed, layer, E, H)
    g = synth.shared_gate(seed, layer, H)
    shared = synth.expert_block(seed, layer, E, H, I, bits)
    prepared = []
    for t in tokens:
        x = synth.activations(seed, t, H)
        idx, _ = oracle.router_topk(oracle.router_logits(R, x), K)
        blocks = {int(e): synth.expert_block(seed, layer, int(e), H, I, bits) for e in idx}
        prepared.append((x, blocks))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        pass
    done = 0
    t0 = time.perf_counter()
    for x, blocks in prepared:
        oracle.moe_layer(blocks.__getitem__, shared, R, g, x, x, H, I, bits, K)
        done += 1
        if time.perf_counter() - t0 > target_s:
            break
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": done / dt, "unit": "tokens/s", "cores": threads or cores, "kind": "oracle",
            "sample": f"{done} tokens of the same layer (float64 numpy oracle, host-resident inputs; "
                      f"{cores} host cores visible, BLAS threads {threads})"}


def run_layer_bench(args, torch, q, synth, bits):
    seed = 1001 if bits == 4 else 1002
    W = LayerWorkload(seed, 0, bits, torch, q, synth)
    n_ring = 4096
    X = make_x_ring(torch, synth, seed, n_ring)
    out = torch.empty(H, dtype=torch.float32, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    per_graph = 256
    calls = [(lambda t=t: q.moe_layer_forward(W.L, X[t], X[t], out, idx, w, W.ws)) for t in range(n_ring)]
    graphs = capture_graphs(torch, calls, per_graph)
    steps = max(1, args.steps)
    tail = None
    if steps % per_graph:
        tail = capture_graphs(torch, calls[:steps % per_graph], per_graph)[0]
    warm = (max(0, args.warmup) + per_graph - 1) // per_graph
    dt = time_graphs(torch, graphs, steps // per_graph, warm, tail)
    spread = launch_spread(torch, graphs, per_graph)
    status = int(W.ws[4:8].view(torch.int32).item())
    if status != 0:
        raise RuntimeError(f"fused layer kernel reported status {status}")
    tok_s = steps / dt
    launch_s = dt / steps
    lb = layer_bytes(bits)
    achieved = lb / launch_s / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profiles(f"k_layer_w{bits}")}
    eb = (K + 1) * expert_bytes(bits)
    extra = {"kernel": "k_layer (fused router+top-K+experts+combine, one launch per token)",
             "bytes_per_launch": lb, "avg_launch_us": round(launch_s * 1e6, 3),
             "launch_spread": spread,
             "expert_bytes_per_launch": eb,
             # the expert GEMVs' weight bytes over the fused launch that reads them
             "expert_gemv_GBps_in_layer": round(eb / launch_s / 1e9, 1)}
    if bits == 4:
        gbps5, us5 = run_expert_ffn5(torch, q, synth, W.routed, seed + 77)
        extra["expert_ffn_swiglu_5experts_GBps"] = round(gbps5, 1)
        extra["expert_ffn_swiglu_5experts_avg_call_us"] = round(us5, 3)
    del W, X, graphs
    torch.cuda.empty_cache()
    return tok_s, steps, dt, roof, extra, (seed, bits)


def run_qgemv_stream(torch, q, synth):
    """Sustained bandwidth of the stand-alone 4-bit GEMV: two 131072 x 4096 matrices
    (288 MB each with scale/bias, together above the 256 MB last-level cache) read
    alternately.  Returns (GB/s of algorithmic bytes, average launch in us)."""
    rows, cols, n = 131072, 4096, 2
    codes = torch.empty(n, rows, cols // 2, dtype=torch.uint8, device="cuda")
    sb = torch.empty(n, rows, cols // 64, dtype=torch.int32, device="cuda")
    synth.fill_bytes(codes, 7, 1)
    synth.fill_bytes(sb, 7, 2)
    sb &= 0x3FFF3FFF  # finite bf16 halves
    x = torch.empty(cols, dtype=torch.float32, device="cuda")
    synth.fill_normal_f32(x, 7, 3, 1.0)
    y = torch.empty(n, rows, dtype=torch.float32, device="cuda")
    calls = [(lambda i=i: q.qgemv_w4(codes[i % n], sb[i % n], x, y[i % n])) for i in range(16)]
    graphs = capture_graphs(torch, calls, 16)
    warm_for(torch, lambda: graphs[0].replay(), 0.1)  # clocks and page translations settle
    reps = 32
    dt = time_graphs(torch, graphs, reps, 2)
    per = rows * cols // 2 + rows * (cols // 64) * 4 + cols * 4 + rows * 4
    launches = 16 * reps
    del codes, sb
    return per * launches / dt / 1e9, dt / launches * 1e6


def run_stream_calibration(torch, q, sizes):
    """Attainable read bandwidth of ONE launch as a function of its bytes: the
    read-only streaming kernel (qmoe_stream_read) over a ring of distinct regions
    of an 8 GiB buffer, so no launch finds its bytes in a cache.  Returns
    {bytes: GB/s}."""
    total = 8 << 30
    buf = torch.empty(total // 4, dtype=torch.int32, device="cuda")
    buf.fill_(0x5A5A5A5A)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for nb in sizes:
        nb = (nb + 255) // 256 * 256
        n_reg = max(2, min(64, total // nb))
        step = (total - nb) // (n_reg - 1) // 256 * 256
        views = [buf[(i * step) // 4:(i * step + nb) // 4] for i in range(n_reg)]
        calls = [(lambda v=v: q.qmoe_stream_read(v, nb, sink=sink)) for v in views]
        graphs = capture_graphs(torch, calls, n_reg)
        warm_for(torch, lambda: graphs[0].replay(), 0.1)
        reps = max(4, int(8e9 // (nb * n_reg)))
        dt = time_graphs(torch, graphs, reps, 1)
        out[nb] = nb * n_reg * reps / dt / 1e9
    del buf
    torch.cuda.empty_cache()
    return out


def launch_spread(torch, graphs, launches_per_graph, repeats=25):
    """Average launch time of each of `repeats` graph replays (launches_per_graph
    launches each), as median, p10 and p90 in microseconds."""
    import statistics
    per = []
    st = torch.cuda.current_stream()
    for r in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        graphs[r % len(graphs)].replay()
        e1.record(st)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / launches_per_graph)
    per.sort()
    q10 = per[max(0, int(0.1 * (len(per) - 1)))]
    q90 = per[min(len(per) - 1, int(round(0.9 * (len(per) - 1))))]
    return {"repeats": repeats, "launches_each": launches_per_graph,
            "median_us": round(statistics.median(per), 3), "p10_us": round(q10, 3),
            "p90_us": round(q90, 3)}


def run_expert_ffn5(torch, q, synth, pool, seed):
    """The expert-GEMV work of one layer as a stand-alone call: expert_ffn_swiglu
    over 5 experts of the resident pool per call (indices drawn per call, a ring of
    256 sets), 5 x 7,077,888 B of weights.  Returns (GB/s, average call in us)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    n_ring = 256
    idx = torch.from_numpy(np.stack([rng.choice(pool.num_experts, 5, replace=False)
                                     for _ in range(n_ring)]).astype(np.int32)).cuda()
    X = make_x_ring(torch, synth, seed, 64)
    Y = torch.empty(5, H, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(256, q.qmoe_ffn_workspace_bytes(pool, 5)), dtype=torch.uint8, device="cuda")
    calls = [(lambda t=t: q.expert_ffn_swiglu(pool, idx[t], X[t % 64], Y, ws)) for t in range(n_ring)]
    dt = timed_steps(torch, calls, 4 * n_ring, n_ring, n_ring)
    per = 5 * expert_bytes(4) + H * 4 + 5 * H * 4
    return per * 4 * n_ring / dt / 1e9, dt / (4 * n_ring) * 1e6


def run_copy(torch):
    """Device-to-device copy of 1 GiB (read + write): the attainable-bandwidth
    reference for this machine, and the known-size kernel that scales the HBM
    byte counters."""
    n = 1 << 28
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    warm_for(torch, lambda: b.copy_(a), 0.1)
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record(st)
    for _ in range(reps):
        b.copy_(a)
    e1.record(st)
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    return 2 * 4 * n / dt / 1e9


def timed_steps(torch, calls, steps, warmup, per_graph):
    """Capture calls (one per step, cycled) into graphs of per_graph steps and time
    exactly `steps` of them.  Returns seconds."""
    per_graph = max(1, min(per_graph, len(calls)))
    n = (len(calls) // per_graph) * per_graph
    graphs = capture_graphs(torch, calls[:n], per_graph)
    tail = None
    if steps % per_graph:
        tail = capture_graphs(torch, calls[:steps % per_graph], per_graph)[0]
    warm = (max(0, warmup) + per_graph - 1) // per_graph
    return time_graphs(torch, graphs, steps // per_graph, warm, tail)


def run_ffn_bench(args, torch, q, synth):
    """One expert FFN per step on an expert drawn from 256 resident ones (1.8 GB)."""
    seed, n_exp = 1000, 256
    pool = q.ExpertPool.allocate(n_exp, H, I, 4)
    synth.fill_expert_pool(pool.buf, pool.stride, n_exp, 0, 0, seed, H, I, 4)
    n_ring = 1024
    X = make_x_ring(torch, synth, seed, n_ring)
    # a fixed pseudo-random walk over the experts (every expert visited, no repeats in a row)
    order = torch.tensor([(t * 97 + 13) % n_exp for t in range(n_ring)], dtype=torch.int32, device="cuda")
    Y = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(256, q.qmoe_ffn_workspace_bytes(pool, 1)), dtype=torch.uint8, device="cuda")
    calls = [(lambda t=t: q.expert_ffn_swiglu(pool, order[t:t + 1], X[t], Y.view(1, H), ws))
             for t in range(n_ring)]
    steps = max(1, args.steps)
    dt = timed_steps(torch, calls, steps, args.warmup, 256)
    per_call = expert_bytes(4) + 2 * H * 4
    launch_s = dt / steps
    roof = {"bound": "hbm", "achieved": round(per_call / launch_s / 1e9, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(per_call / launch_s / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profiles("expert_ffn_w4")}
    extra = {"kernel": "expert_ffn_swiglu (k_ffn1: gate/up, SwiGLU and down in one launch), roofline over the call",
             "bytes_per_call": per_call, "avg_call_us": round(launch_s * 1e6, 3)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_oracle_ffn(seed, n_exp, args.cpu_seconds)
    return {"value": steps / dt, "unit": "expert FFN calls/s", "steps": steps, "dt": dt, "roof": roof,
            "extra": extra, "cpu": cpu, "workload": "expert_ffn_batch1_4bit", "bits": 4,
            "cfg": {"experts_resident": n_exp}}


def run_gdn_bench(args, torch, q, synth):
    """One GatedDeltaNet decode step per step (64 heads x 128x128 fp32 state), on a
    state taken in turn from a ring of 128 (512 MB, more than the last-level cache)."""
    import numpy as np
    heads, dk, dv, ring, n_tok = 64, 128, 128, 128, 64
    seed = 1005
    states = torch.empty(ring, heads, dv, dk, dtype=torch.float32, device="cuda")
    synth.fill_normal_f32(states, seed, synth.tensor_id(synth.K_GDN_STATE, 0, 0), synth.GDN_STATE_SIGMA)
    toks = [synth.gdn_token(seed, 0, t, heads, dk, dv) for t in range(n_tok)]
    Qs, Ks, Vs, As, Bs = (torch.from_numpy(np.stack([t[i] for t in toks])).cuda() for i in range(5))
    o = torch.empty(heads, dv, dtype=torch.float32, device="cuda")
    calls = [(lambda i=i: q.gdn_recurrent_step(states[i % ring], Qs[i % n_tok], Ks[i % n_tok], Vs[i % n_tok],
                                               As[i % n_tok], Bs[i % n_tok], o=o)) for i in range(ring)]
    steps = max(1, args.steps)
    dt = timed_steps(torch, calls, steps, args.warmup, ring)
    if not bool(torch.isfinite(states).all()):
        raise RuntimeError("GatedDeltaNet state went non-finite")
    # the same bytes moved by a plain device copy (4 MB read + 4 MB written), timed alike
    copies = [(lambda i=i: states[(i + 1) % ring].copy_(states[i])) for i in range(ring)]
    copy_s = timed_steps(torch, copies, 1024, 128, ring) / 1024
    per_step = 2 * heads * dv * dk * 4 + (2 * heads * dk + 2 * heads * dv + 2 * heads) * 4
    launch_s = dt / steps
    roof = {"bound": "hbm", "achieved": round(per_step / launch_s / 1e9, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(per_step / launch_s / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profiles("k_gdn")}
    extra = {"kernel": "gdn_recurrent_step (k_gdn<128>)", "bytes_per_step": per_step,
             "avg_step_us": round(launch_s * 1e6, 3), "copy_4MB_us": round(copy_s * 1e6, 3),
             "copy_4MB_GBps": round(2 * heads * dk * dv * 4 / copy_s / 1e9, 1)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_oracle_gdn(seed, heads, dk, dv, args.cpu_seconds)
    return {"value": steps / dt, "unit": "recurrence steps/s", "steps": steps, "dt": dt, "roof": roof,
            "extra": extra, "cpu": cpu, "workload": "gdn_decode_step_64x128x128", "bits": None,
            "metric": "GatedDeltaNet decode steps/s (64 heads x 128x128 fp32 state), batch 1",
            "config": {"workload": "gdn_decode_step_64x128x128", "heads": heads, "dk": dk, "dv": dv,
                       "state_ring": ring, "state_ring_MB": ring * heads * dk * dv * 4 >> 20}}


def run_attn_bench(args, torch, q, synth):
    """One full-attention decode token (RoPE, cache append, grouped-query attention)
    at context 8192: 32 query heads over 2 KV heads of 256, fp32 caches, on a ring of
    16 layers' caches (512 MB, more than the last-level cache)."""
    import numpy as np
    Hq, Hkv, D, T, ring, rot, theta = 32, 2, 256, 8192, 16, 64, 1e7
    seed = 1006
    KC = torch.empty(ring, Hkv, T, D, dtype=torch.float32, device="cuda")
    VC = torch.empty_like(KC)
    synth.fill_normal_f32(KC, seed, synth.tensor_id(synth.K_ATTN_KCACHE, 0, 0), 1.0)
    synth.fill_normal_f32(VC, seed, synth.tensor_id(synth.K_ATTN_VCACHE, 0, 0), 1.0)
    toks = [synth.attn_token(seed, 0, t, Hq, Hkv, D) for t in range(16)]
    Qs, Ks, Vs = (torch.from_numpy(np.stack([t[i] for t in toks])).cuda() for i in range(3))
    o = torch.empty(Hq, D, dtype=torch.float32, device="cuda")
    ws = torch.empty(q.qmoe_attn_workspace_bytes(Hq, Hkv, D, T), dtype=torch.uint8, device="cuda")
    calls = [(lambda i=i: q.attn_decode_step(Qs[i % 16], Ks[i % 16], Vs[i % 16], KC[i % ring], VC[i % ring],
                                             T - 1, theta, rot, o=o, ws=ws)) for i in range(ring)]
    steps = max(1, args.steps)
    dt = timed_steps(torch, calls, steps, args.warmup, ring)
    if not bool(torch.isfinite(o).all()):
        raise RuntimeError("attention output is not finite")
    per_step = 2 * Hkv * T * D * 4 + 2 * Hq * D * 4 + 2 * Hkv * D * 4
    launch_s = dt / steps
    roof = {"bound": "hbm", "achieved": round(per_step / launch_s / 1e9, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(per_step / launch_s / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profiles("k_attn_mma")}
    extra = {"kernel": "attn_decode_step (k_attn_mma<256>, k_attn_combine<256>)",
             "bytes_per_step": per_step, "avg_step_us": round(launch_s * 1e6, 3)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_oracle_attn(seed, Hq, Hkv, D, T, rot, theta, args.cpu_seconds)
    return {"value": steps / dt, "unit": "decode tokens/s (one attention layer)", "steps": steps, "dt": dt,
            "roof": roof, "extra": extra, "cpu": cpu, "workload": "attn_decode_32q_2kv_d256_ctx8192",
            "bits": None, "metric": "full-attention decode tokens/s per layer (GQA 32/2, D 256, context 8192, fp32 cache), batch 1",
            "config": {"workload": "attn_decode_32q_2kv_d256_ctx8192", "q_heads": Hq, "kv_heads": Hkv,
                       "head_dim": D, "context": T, "rot_dim": rot, "theta": theta, "cache_ring": ring,
                       "cache_ring_MB": ring * 2 * Hkv * T * D * 4 >> 20}}


def cpu_oracle_attn(seed, Hq, Hkv, D, T, rot, theta, target_s):
    """The oracle's attention decode (float64, numpy) on the host, repeated for about
    target_s seconds on one cache."""
    import oracle
    import synth
    K, V = synth.attn_cache(seed, 0, Hkv, T, D)
    toks = [synth.attn_token(seed, 0, t, Hq, Hkv, D) for t in range(4)]
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < target_s:
        oracle.attn_decode(*toks[n % 4], K, V, T - 1, theta, rot)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "decode tokens/s (one attention layer)",
            "cores": blas_threads(), "kind": "oracle", "sample": f"{n} tokens at context {T}"}


def cpu_oracle_gdn(seed, heads, dk, dv, target_s):
    """The oracle's recurrence step (float64, numpy) on the host, repeated for about
    target_s seconds on one state."""
    import oracle
    import synth
    S = synth.gdn_state(seed, 0, heads, dk, dv).transpose(0, 2, 1).astype("float64")
    toks = [synth.gdn_token(seed, 0, t, heads, dk, dv) for t in range(8)]
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < target_s:
        S, _ = oracle.gdn_step(S, *toks[n % 8])
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "recurrence steps/s", "cores": blas_threads(),
            "kind": "oracle", "sample": f"{n} steps of 64 heads x 128x128 on one state"}


def cpu_oracle_ffn(seed, n_exp, target_s):
    import oracle
    import synth
    blocks = [synth.expert_block(seed, 0, e, H, I, 4) for e in range(4)]
    xs = [synth.activations(seed, t, H) for t in range(8)]
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < target_s and done < 4096:
        oracle.expert_ffn(blocks[done % 4], xs[done % 8], H, I, 4)
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "expert FFN calls/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} calls on 4 experts (float64 numpy oracle, host-resident inputs)"}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def run_stack_bench(args, torch, q, synth):
    """60 layers of the config-1 layer, RMSNorm before each; 256 sequential tokens."""
    seed, n_layers, n_tok = 1003, 60, 256
    layers = [LayerWorkload(seed, l, 4, torch, q, synth) for l in range(n_layers)]
    norm = []
    for l in range(n_layers):
        w = torch.empty(H, dtype=torch.float32, device="cuda")
        synth.fill_uniform_f32(w, seed, synth.tensor_id(synth.K_NORM_W, 0, l), synth.NORM_LO, synth.NORM_HI)
        norm.append(w)
    H0 = make_x_ring(torch, synth, seed, n_tok)
    h = torch.empty(H, dtype=torch.float32, device="cuda")
    idx = torch.empty(n_layers, K, dtype=torch.int32, device="cuda")
    w = torch.empty(n_layers, K, dtype=torch.float32, device="cuda")
    S = q.Stack([W.L for W in layers], norm)
    ws = q.alloc_stack_workspace(S)

    def token(t):  # h <- h + MoE_l(rmsnorm(h)) for the 60 layers
        q.moe_stack_forward(S, H0[t], 1e-6, out=h, idx=idx, w=w, ws=ws, persistent=args.persistent)

    calls = [(lambda t=t: token(t)) for t in range(n_tok)]
    steps = max(1, min(args.steps, 4096))
    dt = timed_steps(torch, calls, steps, args.warmup, 8)
    for wsp in [ws]:
        if int(wsp[4:8].view(torch.int32).item()) != 0:
            raise RuntimeError("fused layer kernel reported a time-out")
    per_tok = n_layers * (layer_bytes(4) + H * 4)  # + the RMSNorm weight
    tok_s = steps / dt
    # per launch (one layer): its bytes over the average layer time; the same ratio
    # as a whole token's bytes over the token's time
    roof = {"bound": "hbm", "achieved": round(per_tok * tok_s / 1e9, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(per_tok * tok_s / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profiles("k_layer_w4_stack60")}
    kern = ("k_stack, 32 + 28 layers per launch" if args.persistent else "k_layer x60 per token")
    eb = (K + 1) * expert_bytes(4)  # the 5 experts' weight bytes of one layer
    extra = {"kernel": kern + ", RMSNorm fused (roofline per layer launch; traffic per launch)",
             "bytes_per_token": per_tok, "layer_evals_per_s": round(tok_s * n_layers, 1),
             "expert_bytes_per_layer": eb,
             # the expert GEMVs' weight bytes over the layer launch that reads them
             "expert_gemv_GBps_in_layer": round(eb * tok_s * n_layers / 1e9, 1),
             "resident_GB": round(sum(W.routed.buf.numel() + W.shared.buf.numel() for W in layers) / 1e9, 1)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_oracle_stack(seed, n_layers, args.cpu_seconds)
    return {"value": tok_s, "unit": "tokens/s (60-layer stack)", "steps": steps, "dt": dt, "roof": roof,
            "extra": extra, "cpu": cpu, "workload": "moe_stack60_batch1_4bit", "bits": 4,
            "cfg": {"layers": n_layers, "tokens": n_tok, "rmsnorm_eps": 1e-6}}


def cpu_oracle_stack(seed, n_layers, target_s):
    """Oracle layers of one token through the stack, as many as fit in target_s;
    extrapolated to the 60 layers of a token."""
    import numpy as np

    import oracle
    import synth
    h = synth.activations(seed, 0, H).astype(np.float64)
    done, spent, wall0 = 0, 0.0, time.perf_counter()
    for l in range(n_layers):
        if done and time.perf_counter() - wall0 > 3 * target_s:  # input generation counts here
            break
        R = synth.router(seed, l, E, H)
        g = synth.shared_gate(seed, l, H)
        shared = synth.expert_block(seed, l, E, H, I, 4)
        nw = synth.norm_weight(seed, l, H)
        x = oracle.rmsnorm(h, nw, 1e-6)
        idx, _ = oracle.router_topk(oracle.router_logits(R, x), K)
        blocks = {int(e): synth.expert_block(seed, l, int(e), H, I, 4) for e in idx}
        t0 = time.perf_counter()
        x = oracle.rmsnorm(h, nw, 1e-6)
        h = oracle.moe_layer(blocks.__getitem__, shared, R, g, x, h, H, I, 4, K)
        spent += time.perf_counter() - t0
        done += 1
        if spent > target_s:
            break
    per_layer = spent / done
    return {"value": 1.0 / (per_layer * n_layers), "unit": "tokens/s (60-layer stack)",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} layers of one token (float64 numpy oracle, host-resident inputs), "
                      f"extrapolated to {n_layers} layers"}


def run_batched_bench(args, torch, q, synth):
    """64 tokens per step through the config-1 layer, grouped per expert."""
    seed, T = 1004, 64
    W = LayerWorkload(seed, 0, 4, torch, q, synth)
    n_ring = 64
    X = make_x_ring(torch, synth, seed, n_ring * T).view(n_ring, T, H)
    out = torch.empty(T, H, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    ws = q.alloc_workspace(W.L, T)
    calls = [(lambda b=b: q.moe_layer_forward_batched(W.L, X[b], X[b], out, idx, w, ws)) for b in range(n_ring)]
    steps = max(1, min(args.steps, 8192))
    dt = timed_steps(torch, calls, steps, args.warmup, 64)
    # distinct experts per batch, averaged over the ring (read back after timing)
    distinct = []
    for b in range(n_ring):
        q.moe_layer_forward_batched(W.L, X[b], X[b], out, idx, w, ws)
        distinct.append(len(set(idx.cpu().numpy().ravel().tolist())))
    d_avg = sum(distinct) / len(distinct)
    per_batch = E * H * 2 + (d_avg + 1) * expert_bytes(4) + H * 2 + 3 * T * H * 4
    batch_s = dt / steps
    roof = {"bound": "hbm", "achieved": round(per_batch / batch_s / 1e9, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(per_batch / batch_s / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profiles("batched64_w4")}
    extra = {"kernel": "moe_layer_forward_batched (router, grouping, grouped gate/up, down, combine), "
                       "roofline over the whole call", "distinct_experts_avg": round(d_avg, 1),
             "bytes_per_batch": int(per_batch), "avg_batch_us": round(batch_s * 1e6, 2)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_oracle_layer(seed, 0, 4, list(range(64)), args.cpu_seconds)
    return {"value": steps * T / dt, "unit": "tokens/s", "steps": steps, "dt": dt, "roof": roof,
            "extra": extra, "cpu": cpu, "workload": f"moe_layer_batched{T}_4bit", "bits": 4,
            "cfg": {"batch": T}}


PHASES = ["start", "x in LDS", "router dots done", "x planes in LDS", "x planes in registers",
          "logits polled", "top-K ranked", "shared and routed rows issued",
          "shared + routed gate/up done (wave 0)", "shared h, planes and down rows", "routed h read starts",
          "routed h read into planes", "epoch advanced (barrier)", "routed down rows", "end"]


def run_phase_probe(args, torch, q, synth):
    """Phase timeline of the fused layer from the instrumented library: thread 0 of
    every workgroup stamps the 100 MHz real-time counter at each phase boundary.
    Prints, per phase, the median over the last 64 calls of the p10 / median / max
    over the workgroups, in microseconds from the earliest workgroup start."""
    import numpy as np
    import ctypes
    bits = 4 if args.config == 1 else 2
    seed = 1001 if bits == 4 else 1002
    W = LayerWorkload(seed, 0, bits, torch, q, synth)
    n = 256
    X = make_x_ring(torch, synth, seed, n)
    out = torch.empty(H, dtype=torch.float32, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    calls = [(lambda t=t: q.moe_layer_forward(W.L, X[t], X[t], out, idx, w, W.ws)) for t in range(n)]
    graphs = capture_graphs(torch, calls, n)
    dt = time_graphs(torch, graphs, 16, 16)
    buf = np.zeros(64 * 512 * 16, dtype=np.uint32)
    rc = q.raw_lib().qmoe_phase_probe_read(ctypes.c_void_p(buf.ctypes.data))
    if rc != 0:
        raise RuntimeError(f"qmoe_phase_probe_read failed ({rc})")
    nb = H // 16
    P = buf.reshape(64, 512, 16)[:, :nb, :len(PHASES)].astype(np.int64)
    stats = np.zeros((64, len(PHASES), 3))
    for c in range(64):
        t0 = P[c, :, 0].min()
        d = ((P[c] - t0) % (1 << 32)) * 0.01  # 100 MHz ticks -> us
        stats[c] = np.stack([np.percentile(d, 10, axis=0), np.median(d, axis=0), d.max(axis=0)], axis=1)
    med = np.median(stats, axis=0)
    print(f"fused layer, {bits}-bit, E={E} H={H} I={I} K={K}: {dt / (16 * n) * 1e6:.3f} us per launch (events)")
    print(f"{'phase':40s} {'p10':>7s} {'median':>7s} {'max':>7s}  (us from the first workgroup's start)")
    for k, name in enumerate(PHASES):
        print(f"{name:40s} {med[k, 0]:7.2f} {med[k, 1]:7.2f} {med[k, 2]:7.2f}")
    print(json.dumps({"phase_probe": True, "bits": bits, "avg_launch_us": round(dt / (16 * n) * 1e6, 3),
                      "phases_median_us": {name: round(float(med[k, 1]), 3) for k, name in enumerate(PHASES)},
                      "phases_max_us": {name: round(float(med[k, 2]), 3) for k, name in enumerate(PHASES)}}))


def launch_bytes(config):
    """Algorithmic bytes of one launch (or call) of the config's dominant kernel
    path, the size at which the read-only calibration stream is run."""
    if config in (1, 2, 3):
        return layer_bytes(4 if config != 2 else 2)
    if config == 0:
        return expert_bytes(4) + 2 * H * 4
    if config == 4:
        return E * H * 2 + 203 * expert_bytes(4) + H * 2 + 3 * 64 * H * 4
    if config == 5:
        return 2 * 64 * 128 * 128 * 4 + (2 * 64 * 128 * 2 + 2 * 64) * 4
    if config == 6:
        return 2 * 2 * 8192 * 256 * 4 + 2 * 32 * 256 * 4 + 2 * 2 * 256 * 4
    return None


def device_info():
    """GPU name (gfx target) and clocks from rocminfo, read before this process
    initialises the GPU; empty fields if the tool is not there."""
    import re
    import subprocess
    info = {}
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
    except Exception:
        return info
    for block in txt.split("*******"):
        m = re.search(r"Name:\s+(gfx\w+)", block)
        if not m:
            continue
        info["gfx"] = m.group(1)
        mk = re.search(r"Marketing Name:[ \t]*(\S[^\n]*)", block)
        if mk:
            info["marketing_name"] = mk.group(1).strip()
        mc = re.search(r"Max Clock Freq\. \(MHz\):[ \t]*(\d+)", block)
        if mc:
            info["max_sclk_MHz"] = int(mc.group(1))
        cu = re.search(r"Compute Unit:[ \t]*(\d+)", block)
        if cu:
            info["compute_units"] = int(cu.group(1))
        break
    try:
        txt = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30).stdout
        for key in ("sclk", "mclk", "fclk"):
            m = re.search(key + r" clock level: \d+: \((\d+)Mhz\)", txt)
            if m:
                info[key + "_MHz_now"] = int(m.group(1))
    except Exception:
        pass
    return info


def run_offload_bench(args, torch, q, synth):
    """Host-tier offload: the config-1 layer with its 512 routed experts in pinned
    host memory and an HBM cache of 256 expert slots (half the layer: a model twice
    the size of HBM).  A step is one token (fresh x each), waiting on the host for
    its routing as the offload path does.  Also measured: the host-to-device copy
    rate alone, the resident fused layer alone, and the two at once on separate
    streams (whether DMA and compute slow each other on this GPU)."""
    import numpy as np
    seed, slots = 1001, 256
    W = LayerWorkload(seed, 0, 4, torch, q, synth)
    hbuf = torch.empty(W.routed.buf.numel(), dtype=torch.uint8, pin_memory=True)
    hbuf.copy_(W.routed.buf)
    torch.cuda.synchronize()
    hp = q.ExpertPool(hbuf, E, H, I, 4, W.routed.stride)
    off = q.Offload(hp, slots)
    L_off = q.Layer(hp, W.shared, W.router, W.gate, K)
    n_tok = 256
    X = make_x_ring(torch, synth, seed, n_tok)
    out = torch.empty(H, dtype=torch.float32, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    ws = torch.empty(q.qmoe_offload_workspace_bytes(L_off), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    warm = min(max(args.warmup, 64), n_tok)
    for t in range(warm):  # fills the cache to its steady state
        q.moe_layer_forward_offload(off, L_off, X[t % n_tok], out=out, idx=idx, w=w, ws=ws, copy_stream=cs)
    torch.cuda.synchronize()
    st0 = off.stats()
    steps = max(1, min(args.steps, 4096))
    t0 = time.perf_counter()
    for t in range(steps):
        q.moe_layer_forward_offload(off, L_off, X[t % n_tok], out=out, idx=idx, w=w, ws=ws, copy_stream=cs)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st1 = off.stats()
    hits, misses = st1["hits"] - st0["hits"], st1["misses"] - st0["misses"]
    copied = st1["bytes_copied"] - st0["bytes_copied"]
    # the copy rate alone: 64 expert blocks host -> HBM slots on the copy stream
    eb = hp.layout["total"]
    rng = np.random.default_rng(7)
    picks = rng.integers(0, E, 64)

    def copies(stream):
        with torch.cuda.stream(stream):
            for i, e in enumerate(picks):
                off.slot_mem[(i % slots) * hp.stride:(i % slots) * hp.stride + eb].copy_(
                    hbuf[int(e) * hp.stride:int(e) * hp.stride + eb], non_blocking=True)

    def timed(fn, stream):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        return e0, e1

    copies(cs)
    torch.cuda.synchronize()
    c0, c1 = timed(lambda: copies(cs), cs)
    torch.cuda.synchronize()
    copy_alone = 64 * eb / (c0.elapsed_time(c1) / 1e3) / 1e9
    # the resident fused layer alone, then together with the copies
    calls = [(lambda t=t: q.moe_layer_forward(W.L, X[t], X[t], out, idx, w, W.ws)) for t in range(n_tok)]
    graphs = capture_graphs(torch, calls, n_tok)
    graphs[0].replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    g0, g1 = timed(lambda: [graphs[0].replay() for _ in range(8)], cur)
    torch.cuda.synchronize()
    layer_alone = g0.elapsed_time(g1) * 1e3 / (8 * n_tok)
    c0, c1 = timed(lambda: copies(cs), cs)
    g0, g1 = timed(lambda: [graphs[0].replay() for _ in range(8)], cur)
    torch.cuda.synchronize()
    copy_both = 64 * eb / (c0.elapsed_time(c1) / 1e3) / 1e9
    layer_both = g0.elapsed_time(g1) * 1e3 / (8 * n_tok)
    off.close()
    per_tok = layer_bytes(4)
    tok_s = steps / dt
    roof = {"bound": "hbm", "achieved": round(per_tok * tok_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(per_tok * tok_s / 1e9 / HBM_PEAK_GBPS, 5), "traffic": None}
    extra = {"kernel": "moe_layer_forward_offload (router + top-K, host wait, copies on a second stream, "
                       "shared and routed expert FFN, combine)",
             "slots": slots, "hit_rate": round(hits / max(1, hits + misses), 4),
             "misses_per_token": round(misses / steps, 3),
             "host_to_device_GBps_in_run": round(copied / dt / 1e9, 2),
             "avg_token_us": round(dt / steps * 1e6, 2),
             "copy_alone_GBps": round(copy_alone, 2), "copy_with_layer_running_GBps": round(copy_both, 2),
             "fused_layer_alone_us": round(layer_alone, 3), "fused_layer_with_copies_us": round(layer_both, 3)}
    return {"value": tok_s, "unit": "tokens/s (one offloaded layer)", "steps": steps, "dt": dt, "roof": roof,
            "extra": extra, "cpu": None, "workload": "moe_layer_offload_4bit_512experts_256slots", "bits": 4,
            "metric": "MoE-layer tokens/s at batch 1, routed experts in pinned host memory (256-slot HBM cache)",
            "cfg": {"slots": slots, "host_pool_GB": round(hbuf.numel() / 1e9, 2)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16384)
    ap.add_argument("--warmup", type=int, default=1024)
    ap.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 3, 4, 5, 6, 7])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--persistent", action="store_true",
                    help="config 3: the persistent stack kernel (32 layers per launch) instead of "
                         "one fused launch per layer")
    ap.add_argument("--phase-probe", action="store_true",
                    help="configs 1/2: load the instrumented library (build.py --probe) and print the "
                         "fused layer's phase timeline instead of the benchmark line")
    ap.add_argument("--no-device-info", action="store_true",
                    help="skip the rocminfo / rocm-smi child processes (for runs under a profiler, "
                         "whose preloaded library has initialised the GPU before this process starts)")
    args = ap.parse_args()
    if args.phase_probe:
        os.environ["QMOE_LIBRARY"] = "probe"
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)

    dev_info = {} if args.no_device_info else device_info()
    import torch
    import bit_dequant_gemv_amd as q
    import synth
    torch.cuda.set_device(0)
    if args.phase_probe:
        if args.config not in (1, 2):
            raise SystemExit("--phase-probe covers configs 1 and 2")
        run_phase_probe(args, torch, q, synth)
        return
    extra0 = {}
    if args.config in (1, 2):
        # stand-alone GEMV stream and copy reference first, on an otherwise empty device
        gbps, us = run_qgemv_stream(torch, q, synth)
        extra0["qgemv_w4_131072x4096_GBps"] = round(gbps, 1)
        extra0["qgemv_w4_131072x4096_frac_of_peak"] = round(gbps / HBM_PEAK_GBPS, 4)
        extra0["qgemv_w4_131072x4096_avg_launch_us"] = round(us, 2)
        extra0["copy_1GiB_GBps"] = round(run_copy(torch), 1)
        torch.cuda.empty_cache()
        bits = 4 if args.config == 1 else 2
        lb = layer_bytes(bits)
        stream = run_stream_calibration(torch, q, [4 << 20, lb, 40 << 20, 400 << 20, 4 << 30])
        extra0["stream_read_GBps_by_bytes_per_launch"] = {str(k): round(v, 1) for k, v in stream.items()}
        tok_s, steps, dt, roof, extra, (seed, _) = run_layer_bench(args, torch, q, synth, bits)
        att = stream[(lb + 255) // 256 * 256]
        extra0["attainable_GBps_same_bytes_per_launch"] = round(att, 1)
        extra0["frac_of_attainable_same_bytes"] = round(roof["achieved"] / att, 4)
        cpu = None
        if not args.no_cpu_baseline:
            cpu = cpu_oracle_layer(seed, 0, bits, list(range(64)), args.cpu_seconds)
            try:
                from threadpoolctl import threadpool_limits
                with threadpool_limits(limits=1):
                    one = cpu_oracle_layer(seed, 0, bits, list(range(8)), min(10.0, args.cpu_seconds))
                extra0["cpu_oracle_1thread_tokens_per_s"] = round(one["value"], 3)
            except ImportError:
                pass
        r = {"value": tok_s, "unit": "tokens/s", "steps": steps, "dt": dt, "roof": roof, "extra": extra,
             "cpu": cpu, "workload": f"moe_layer_batch1_{bits}bit", "bits": bits, "cfg": {}}
    elif args.config == 0:
        r = run_ffn_bench(args, torch, q, synth)
    elif args.config == 3:
        r = run_stack_bench(args, torch, q, synth)
    elif args.config == 5:
        r = run_gdn_bench(args, torch, q, synth)
    elif args.config == 6:
        r = run_attn_bench(args, torch, q, synth)
    elif args.config == 7:
        r = run_offload_bench(args, torch, q, synth)
    else:
        r = run_batched_bench(args, torch, q, synth)
    if "attainable_GBps_same_bytes_per_launch" not in extra0 and r["roof"].get("unit") == "GB/s" \
            and launch_bytes(args.config):
        nb = launch_bytes(args.config)
        att = list(run_stream_calibration(torch, q, [nb]).values())[0]
        extra0["attainable_GBps_same_bytes_per_launch"] = round(att, 1)
        extra0["attainable_bytes_per_launch"] = nb
        extra0["frac_of_attainable_same_bytes"] = round(r["roof"]["achieved"] / att, 4)
    r["extra"].update(extra0)
    config = r.get("config") or {"workload": r["workload"], "experts": E, "hidden": H, "inter": I,
                                 "top_k": K, "shared_experts": 1, "group": 64, "bits": r["bits"]}
    config.update(r.get("cfg", {}))
    config["device"] = dev_info.get("marketing_name") or torch.cuda.get_device_name(0)
    config["gfx"] = dev_info.get("gfx") or getattr(torch.cuda.get_device_properties(0), "gcnArchName", None)
    r["extra"]["device_info"] = dev_info
    line = {
        "metric": r.get("metric", METRIC), "value": round(r["value"], 1), "unit": r["unit"], "n_gpus": 1,
        "steps": r["steps"], "warmup": args.warmup, "ms_per_step": round(r["dt"] * 1e3 / r["steps"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": config,
        "roofline": r["roof"], "cpu_baseline": r["cpu"], "detail": r["extra"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
