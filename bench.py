#!/usr/bin/env python3
"""Benchmark of the routed MoE layer on one MI355X.

A step is one whole layer call (route, group, quantise, gate/up, down, combine: every
row of the hot path) over one batch of T synthetic tokens, on the stacked layer
l = step mod L, so that consecutive steps stream different weights (the stack is
larger than the 256 MB Infinity Cache). Inputs are resident in HBM before the timed
region. Default workload: the GLM-5.2-scale decode layer (hidden 6144, expert FFN
2048, 256 routed experts + 1 shared, top-8 of 8 groups / 4 kept, routed scaling 2.5,
int4 per-row weights, Q8_0 activations), 8 stacked layers (about 39 GB), T = 16 as
the headline (exactly --steps timed layer calls); T = 1, 4 and 16 are reported in
"sweep" (at least 64 timed calls each), and the GLM-scale batch-union prefill
(T = 2048, Zipf-skewed router bias) under "prefill" with its int8 TOP/s.

Prints ONE JSON line (rank 0). Extra detail goes to stderr.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD public specification
INT8_PEAK_TOPS = 5000.0        # dense int8 MFMA, AMD public specification
DOMINANT_STAGE = "ffn_gate_up"
METRIC = "MoE-layer tokens/s + int4 weight GB/s vs HBM peak (decode); int8 TOPS (prefill)"
KERNEL_SOURCES = ["quantized_moe_sigmoid_amd/csrc/coli_internal.h", "quantized_moe_sigmoid_amd/csrc/ffn_gemv_impl.h",
                  "quantized_moe_sigmoid_amd/csrc/select_impl.h", "quantized_moe_sigmoid_amd/csrc/ffn_gemv_w4.hip",
                  "quantized_moe_sigmoid_amd/csrc/ffn_mfma.hip"]
LOCAL_GROUP_MAX_P = 512         # batches above this many (token, expert) pairs take the grouped-GEMM path


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, T: int):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 PMC
    summary, or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"gateup_{workload}_T{T}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


class Stack:
    """L stacked layers of one workload, resident on the device."""

    def __init__(self, wl_index: int, layers: int, wbits: int | None = None, scale_group: int = 0,
                 topp: float = 0.0):
        import numpy as np
        import torch
        import quantized_moe_sigmoid_amd as q
        import synth
        import synth.device

        self.wl = dict(synth.WORKLOADS[wl_index])
        if wbits is not None:
            self.wl["wbits"] = wbits
        if wbits == synth.W_MXFP4:  # MXFP4: E8M0 scale bytes, one per 32 inputs
            scale_group = 32
            self.wl["name"] += "_mxfp4"
        if scale_group:
            self.wl["scale_group"] = scale_group
            if scale_group != 32:
                self.wl["name"] += f"_gs{scale_group}"
        if topp:
            self.wl["topp"] = topp
            self.wl["name"] += f"_topp{topp:g}"
        wl = self.wl
        self.cfg = q.make_cfg(**wl)
        self.blob = q.blob_bytes(self.cfg)
        self.L = layers
        self.dev = torch.device("cuda:0")
        ne = wl["n_experts"] + (1 if wl["has_shared"] else 0)
        self.ne = ne
        self.layers = []
        for l in range(layers):
            seed = synth.workload_seed(wl_index, l)
            blobs = torch.empty(ne * self.blob, dtype=torch.uint8, device=self.dev)
            synth.device.fill_blobs(blobs, seed, l, 0, ne, self.blob, wl["wbits"])
            inp = synth.layer_inputs(seed, l, tokens=1, hidden=wl["hidden"], ffn=wl["ffn"],
                                     n_experts=wl["n_experts"], has_shared=wl["has_shared"], wbits=wl["wbits"],
                                     zipf=wl.get("zipf", False), with_blobs=False,
                                     scale_group=wl.get("scale_group", 0))
            up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)
            w = q.Weights(blobs, up(inp["scales"]), up(inp["router_w"]), up(inp["router_bias"]))
            self.layers.append((seed, w))
        torch.cuda.synchronize()

    def inputs(self, T: int):
        import torch
        import synth
        xs = []
        for l, (seed, _) in enumerate(self.layers):
            xs.append(torch.from_numpy(synth.activations(seed, l, T, self.wl["hidden"])).to(self.dev))
        return xs

    def union_sizes(self, xs):
        """Distinct routed experts U of each layer for these inputs, and the routed pairs kept
        (fewer than T * k with adaptive top-p), from the library's own route and grouping."""
        import torch
        import quantized_moe_sigmoid_amd as q
        T = xs[0].shape[0]
        E, k = self.wl["n_experts"], self.wl["top_k"]
        ws = q.alloc_workspace(self.cfg, T, self.dev)
        idx = torch.empty((T, k), dtype=torch.int32, device=self.dev)
        tw = torch.empty((T, k), dtype=torch.float32, device=self.dev)
        cnt = torch.empty(E, dtype=torch.int32, device=self.dev)
        off = torch.empty(E + 1, dtype=torch.int32, device=self.dev)
        perm = torch.empty(T * k, dtype=torch.int32, device=self.dev)
        act = torch.empty(E, dtype=torch.int32, device=self.dev)
        na = torch.empty(1, dtype=torch.int32, device=self.dev)
        us, pairs = [], []
        for (seed, w), x in zip(self.layers, xs):
            q.route(self.cfg, w, x, idx, tw, ws)
            q.group(self.cfg, idx, T, cnt, off, perm, act, na)
            us.append(int(na.item()))
            pairs.append(int(off[E].item()))
        return us, pairs


def _packed_row_bytes(wl, n_inputs: int) -> int:
    """Packed weight bytes of one row (MXFP4: 4-bit codes)."""
    return n_inputs // 2 if wl["wbits"] == 40 else n_inputs * wl["wbits"] // 8


def _row_scale_bytes(wl, n_inputs: int) -> int:
    """Scale bytes of one weight row of n_inputs: one fp32 per row or per group; MXFP4 one
    E8M0 byte per 32 inputs."""
    g = wl.get("scale_group", 0)
    if wl["wbits"] == 40:
        return n_inputs // 32
    return 4 if g == 0 else 4 * (n_inputs // g)


def gateup_bytes(wl, U: int, T: int, pairs: int | None = None) -> int:
    """Algorithmic HBM bytes of one gate/up launch: the packed gate and up rows plus their
    fp32 scales of the U routed (+ shared) experts, the Q8_0 activations read once, and
    the requantised h written once."""
    H, F, k = wl["hidden"], wl["ffn"], wl["top_k"]
    S = 1 if wl["has_shared"] else 0
    nexp = U + S
    weights = nexp * 2 * F * (_packed_row_bytes(wl, H) + _row_scale_bytes(wl, H))
    acts = T * (H + 4 * (H // 32))   # Q8_0 codes + one fp32 scale per 32 values
    rows_out = (T * k if pairs is None else pairs) + S * T
    hout = rows_out * (F + 4 * (F // 32))
    return weights + acts + hout


def layer_weight_bytes(wl, U: int) -> int:
    """Packed weights + per-row scales of the experts one layer call streams."""
    H, F = wl["hidden"], wl["ffn"]
    nexp = U + (1 if wl["has_shared"] else 0)
    return nexp * (2 * F * (_packed_row_bytes(wl, H) + _row_scale_bytes(wl, H)) +
                   H * (_packed_row_bytes(wl, F) + _row_scale_bytes(wl, F)))


def run_T(stack, T: int, n_calls: int, warmup: int, use_graph: bool, n_prof: int | None = None):
    """Time exactly n_calls layer calls at T tokens (call i on stacked layer i mod L),
    after `warmup` untimed calls. With use_graph the n_calls calls are captured as one
    HIP graph and replayed once inside the timed region (the launches cost no host
    time); the region is bracketed by device synchronisations. A second pass of n_prof
    calls records HIP events between the stages of each call (per-stage durations)."""
    import torch
    import quantized_moe_sigmoid_amd as q
    xs = stack.inputs(T)
    L = stack.L
    ws = q.alloc_workspace(stack.cfg, T, stack.dev)
    outs = [torch.empty((T, stack.wl["hidden"]), dtype=torch.float32, device=stack.dev) for _ in range(L)]
    stream = torch.cuda.Stream(stack.dev)

    def step(i):
        l = i % L
        q.layer(stack.cfg, stack.layers[l][1], xs[l], outs[l], ws, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(max(warmup, 1)):
            step(i)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(n_calls):
                step(i)
        torch.cuda.synchronize()
        graph.replay()  # untimed: the first replay uploads the graph
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        if use_graph:
            graph.replay()
        else:
            for i in range(n_calls):
                step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / n_calls
    del graph

    # Per-stage durations: HIP events (no system-scope fence, so recording them costs no
    # cache flush) recorded on the launch stream between the stages of each layer call.
    ns = q.num_stages()
    names = [q.stage_name(i) for i in range(ns)]
    acc = [0.0] * ns
    nprof = n_prof if n_prof is not None else 4 * L
    ev = q.TimingEvents(ns + 1)
    with torch.cuda.stream(stream):
        for i in range(nprof):
            l = i % L
            q.layer_profiled(stack.cfg, stack.layers[l][1], xs[l], outs[l], ws, ev, stream=stream)
            stream.synchronize()
            for s in range(ns):
                acc[s] += ev.elapsed_ms(s, s + 1)
    ev.close()
    stage_ms = {names[s]: acc[s] / nprof for s in range(ns)}
    us, pairs = stack.union_sizes(xs)
    return dict(T=T, ms=ms, calls=n_calls, stage_ms=stage_ms, stage_calls=nprof, U=us, pairs=pairs)


def copy_bandwidth(mbytes: int, reps: int):
    """Streaming copy of mbytes MiB (synth.device.copy, 16-byte loads and stores):
    the traffic-calibration kernel of the hardware byte counters and a measured
    read+write bandwidth beside the HBM peak. Returns GB/s of (read + write)."""
    import torch
    import synth.device
    n = mbytes << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    synth.device.copy(src, dst)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        synth.device.copy(src, dst)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del src, dst
    return 2 * n / dt / 1e9


def read_bandwidth(mbytes: int, reps: int):
    """Streaming read of mbytes MiB (synth.device.read: 16-byte loads, four in flight per
    thread, nothing written but one word per wavefront): the measured read-bandwidth
    ceiling of the device beside the 8 TB/s specification. Returns GB/s."""
    import torch
    import synth.device
    n = mbytes << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(3)
    sink = synth.device.read_sink(src.device)
    torch.cuda.synchronize()
    synth.device.read(src, sink)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        synth.device.read(src, sink)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del src, sink
    return n / dt / 1e9


def scaled_mfma_ceiling(iters: int = 2000, reps: int = 3):
    """int8 TOP/s of synth.device.scaled_mfma: v_mfma_i32_32x32x32_i8 with each int32 result
    converted to fp32 and multiply-added with a scale, in registers only. The rate at which
    the device can produce exactly scaled Q8_0 block dots: the ceiling of a grouped GEMM
    that keeps every block dot exact. Median of `reps` launches timed with HIP events on
    the launch stream."""
    import torch
    import synth.device
    out = synth.device.scaled_mfma_out(torch.device("cuda:0"))
    synth.device.scaled_mfma(out, 10)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        synth.device.scaled_mfma(out, iters)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    dt = sorted(ts)[len(ts) // 2]
    return synth.device.scaled_mfma_ops(iters) / dt / 1e12


def h2d_bandwidth(mbytes: int = 256, reps: int = 5) -> float:
    """Host->device copy rate from pinned host memory (GB/s): the practical PCIe peak
    beside which the expert tier's copies are measured."""
    import torch
    n = mbytes << 20
    src = torch.empty(n, dtype=torch.uint8).pin_memory()
    dst = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    return n * reps / (time.perf_counter() - t0) / 1e9


def run_tier(args):
    """The expert residency tier: every layer's experts in pinned host RAM, a pool of
    `--tier-slots` HBM slots per layer managed by the LRU planner, misses copied host->HBM
    inside the timed region. One step = one layer call on each of L stacked layers, with
    coli_moe_layer_tiered (route, route to the host, plan, misses copied on a second stream
    while the resident pairs compute, then the missing pairs and the combine); the inputs
    cycle over 16 seeded batches per layer so that routes (and misses) change."""
    import numpy as np
    import torch
    import quantized_moe_sigmoid_amd as q
    import synth
    import synth.device

    wl = dict(synth.WORKLOADS[args.config])
    if args.wbits is not None:
        wl["wbits"] = args.wbits
        if args.wbits == 40:
            wl["scale_group"] = 32
    if args.scale_group:
        wl["scale_group"] = args.scale_group
    T = int(args.tokens.split(",")[-1]) if args.tokens else wl["tokens"][-1]
    E, H, slots, L = wl["n_experts"], wl["hidden"], args.tier_slots, args.layers
    S = 1 if wl["has_shared"] else 0
    if not 1 <= slots <= E:
        raise SystemExit(f"--tier-slots must lie in 1..{E}")
    cfg = q.make_cfg(**wl)
    pcfg = q.make_cfg(**dict(wl, n_experts=slots, n_group=1, topk_group=1))
    blob, nsc = q.blob_bytes(cfg), q.scales_per_expert(cfg)
    d = torch.device("cuda:0")
    h2d = h2d_bandwidth()
    log(f"host->device copies from pinned memory: {h2d:.1f} GB/s")
    layers = []
    for l in range(L):
        seed = synth.workload_seed(args.config, l)
        tmp = torch.empty((E + S) * blob, dtype=torch.uint8, device=d)
        synth.device.fill_blobs(tmp, seed, l, 0, E + S, blob, wl["wbits"])
        hb = torch.empty((E + S) * blob, dtype=torch.uint8, pin_memory=True)
        hb.copy_(tmp)
        del tmp
        inp = synth.layer_inputs(seed, l, tokens=1, hidden=H, ffn=wl["ffn"], n_experts=E, has_shared=wl["has_shared"],
                                 wbits=wl["wbits"], zipf=wl.get("zipf", False), with_blobs=False,
                                 scale_group=wl.get("scale_group", 0))
        sc = np.ascontiguousarray(inp["scales"]).reshape(-1)
        hs = torch.empty(sc.shape, dtype=torch.from_numpy(sc[:1]).dtype, pin_memory=True)
        hs.copy_(torch.from_numpy(sc))
        pool_b = torch.empty((slots + S) * blob, dtype=torch.uint8, device=d)
        pool_s = torch.empty((slots + S) * nsc, dtype=hs.dtype, device=d)
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
        rw, rb = up(inp["router_w"]), up(inp["router_bias"])
        tier = q.Tier(E, slots)
        if S:
            q.tier_stage(cfg, slots, hb, hs, [E], [slots], pool_b, pool_s)
        if args.tier_residual > 0:
            # a synthetic residual stream: layer l's input is layer l-1's plus sigma * noise
            seed0 = synth.workload_seed(args.config, 0)
            xs = []
            for i in range(16):
                xv = synth.activations(seed0, 0, T, H, index=100 + i)
                for j in range(1, l + 1):
                    xv = xv + args.tier_residual * synth.activations(seed0, j, T, H, index=200 + i)
                xs.append(up(xv.astype(np.float32)))
        else:
            xs = [up(synth.activations(seed, l, T, H, index=100 + i)) for i in range(16)]
        layers.append(dict(hb=hb, hs=hs, tier=tier, pool=q.Weights(pool_b, pool_s, rw, rb),
                           resident=q.Weights(None, None, rw, rb), xs=xs))
    tws = q.alloc_tier_workspace(cfg, slots, T, d)
    pfws = q.alloc_tier_workspace(cfg, slots, T, d)  # the lookahead's own route scratch
    rs = torch.cuda.Stream(d)                          # the lookahead's router stream
    out = torch.empty((T, H), dtype=torch.float32, device=d)
    cs = torch.cuda.Stream(d)
    ev = q.HipEvent()
    stats = dict(loads=0, unions=0, prefetched=0)

    def layer_call(lay, step, nxt=None):
        x = lay["xs"][step % 16]
        tier = lay["tier"]
        prev = tier.slot_of.copy()
        try:
            q.layer_tiered(cfg, lay["pool"], tier, lay["hb"], lay["hs"], lay["pool"].experts, lay["pool"].scales, x,
                           out, tws, cs, ev)
        except q.ColiError as e:
            raise SystemExit(f"the batch union does not fit in {slots} slots ({e}); use more --tier-slots")
        stats["loads"] += int(((tier.slot_of >= 0) & (prev < 0)).sum())      # experts copied in this call
        stats["unions"] += int((tier.last_use == tier.c.clock).sum())        # slots this batch used
        if nxt is not None:  # lookahead: the next layer's router on this layer's input, on its own stream
            try:
                stats["prefetched"] += q.tier_prefetch(cfg, nxt["pool"], nxt["tier"], nxt["hb"], nxt["hs"],
                                                       nxt["pool"].experts, nxt["pool"].scales, x, pfws, cs, stream=rs)
            except q.ColiError:
                pass  # a predicted union that does not fit is not prefetched

    def step_all(st):
        for li, lay in enumerate(layers):
            nxt = layers[li + 1] if args.tier_lookahead and li + 1 < L else None
            layer_call(lay, st, nxt)

    for w in range(args.warmup):
        step_all(w)
    torch.cuda.synchronize()
    stats.update(loads=0, unions=0, prefetched=0)
    t0 = time.perf_counter()
    for st in range(args.steps):
        step_all(args.warmup + st)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    calls = args.steps * L
    per_call = dt / calls
    copy_bytes = (stats["loads"] + stats["prefetched"]) * (blob + nsc * (1 if wl["wbits"] == 40 else 4))
    achieved = copy_bytes / dt / 1e9
    hit = 1.0 - stats["loads"] / max(1, stats["unions"])
    log(f"tier: {slots}/{E} slots, T={T}: {per_call * 1e6:.1f} us/layer call, {T / per_call:.0f} tok/s, "
        f"hit rate {hit:.3f}, {stats['loads'] / calls:.1f} expert loads/call on demand, "
        f"{stats['prefetched'] / calls:.1f} prefetched/call, copies {achieved:.1f} GB/s")
    line = {
        "metric": "MoE-layer tokens/s (decode, expert tier: host RAM -> HBM slots)",
        "value": round(T / per_call, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(per_call * L * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "int8x" + {2: "int2", 4: "int4", 8: "int8", 40: "mxfp4"}[wl["wbits"]],
        "data": "synthetic (seeded SplitMix64); experts in pinned host RAM, copies inside the timed region",
        "config": {"workload": wl["name"] + "_tier" + ("_lookahead" if args.tier_lookahead else ""), "tokens": T,
                   "slots": slots, "n_experts": E, "stacked_layers": L, "scale_group": wl.get("scale_group", 0),
                   "residual_sigma": args.tier_residual},
        "roofline": {"bound": "pcie", "achieved": round(achieved, 2), "peak": round(h2d, 2), "unit": "GB/s",
                     "frac": round(achieved / h2d, 4), "traffic": None,
                     "kernel": "host->HBM expert copies (hipMemcpyAsync, overlapped with the resident pairs' FFN)", "bytes_per_step": copy_bytes // args.steps},
        "tier": {"hit_rate": round(hit, 4), "loads_per_call": round(stats["loads"] / calls, 2),
                 "prefetched_per_call": round(stats["prefetched"] / calls, 2),
                 "union_per_call": round(stats["unions"] / calls, 2)},
    }
    print(json.dumps(line), flush=True)


def gateup_ops(wl, T: int, pairs: float | None = None) -> int:
    """int8 multiply-add operations (x2) of one gate/up launch: every (token, expert)
    pair and every shared-expert row against 2F weight rows of H inputs."""
    rows = (T * wl["top_k"] if pairs is None else pairs) + (T if wl["has_shared"] else 0)
    return 2 * rows * 2 * wl["ffn"] * wl["hidden"]


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_sample(wl, seed: int, T: int):
    """Inputs of the oracle for T tokens of layer 0, with host copies of only the experts
    these tokens route to (the route is computed once here to find them)."""
    import numpy as np
    import oracle
    import synth
    inp = synth.layer_inputs(seed, 0, tokens=T, hidden=wl["hidden"], ffn=wl["ffn"], n_experts=wl["n_experts"],
                             has_shared=wl["has_shared"], wbits=wl["wbits"], zipf=wl.get("zipf", False),
                             with_blobs=False, scale_group=wl.get("scale_group", 0))
    cfg = oracle.make_cfg(**wl)
    ridx, _ = oracle.route(cfg, inp["router_w"], inp["router_bias"], inp["x"])
    E, S = wl["n_experts"], 1 if wl["has_shared"] else 0
    need = sorted(set(int(e) for e in ridx.ravel() if e >= 0))
    remap = np.full(E + 1, -1, np.int32)
    remap[need] = np.arange(len(need), dtype=np.int32)
    rows = need + ([E] if S else [])
    blobs = np.stack([synth.expert_blob(seed, 0, e, wl["hidden"], wl["ffn"], wl["wbits"]) for e in rows])
    scales = np.ascontiguousarray(inp["scales"][rows])
    sub = oracle.make_cfg(**dict(wl, n_experts=len(need), n_group=1, topk_group=1))
    return dict(cfg=cfg, sub=sub, inp=inp, blobs=blobs, scales=scales, remap=remap)


def _time_oracle(smp, budget_s: float):
    """Oracle layer calls (route, then the FFN of the routed experts and the combine) until
    budget_s has passed; returns (calls, seconds)."""
    import oracle
    inp = smp["inp"]
    calls = 0
    t0 = time.perf_counter()
    while True:
        idx, w = oracle.route(smp["cfg"], inp["router_w"], inp["router_bias"], inp["x"])
        oracle.ffn(smp["sub"], smp["blobs"], smp["scales"], inp["x"], smp["remap"][idx], w)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return calls, el


def cpu_baseline(stack, T: int, budget_s: float, budget_1t_s: float):
    """The oracle (plain C, OpenMP over tokens, untuned) timed on the host cores on layer 0
    of the same workload and inputs: at the headline T with every OpenMP thread, and at
    T = 1 on a single thread (each a bounded sample of about the given seconds)."""
    import oracle
    wl = stack.wl
    seed, _ = stack.layers[0]
    Tm = min(T, 64)
    threads = oracle.threads()
    calls, el = _time_oracle(_oracle_sample(wl, seed, Tm), budget_s)
    res = dict(value=Tm * calls / el, unit="tokens/s", cores=threads, kind="oracle",
               sample=f"{calls} oracle calls of layer 0 at T={Tm} on {threads} threads ({el:.1f} s wall)",
               cpu_model=_cpu_model(), nproc=os.cpu_count(), omp_num_threads=os.environ.get("OMP_NUM_THREADS"))
    if budget_1t_s > 0:
        smp1 = _oracle_sample(wl, seed, 1)
        oracle.set_threads(1)
        try:
            c1, e1 = _time_oracle(smp1, budget_1t_s)
        finally:
            oracle.set_threads(threads)
        res["single_thread"] = dict(value=c1 / e1, unit="tokens/s", cores=1,
                                    sample=f"{c1} oracle calls of layer 0 at T=1 on 1 thread ({e1:.1f} s wall)")
    return res


def _csv_rows(path_or_dir: str, suffix: str):
    import csv
    import glob
    if os.path.isdir(path_or_dir):
        files = sorted(glob.glob(os.path.join(path_or_dir, "**", "*" + suffix), recursive=True))
    else:
        files = [path_or_dir]
    if not files:
        raise SystemExit(f"no *{suffix} under {path_or_dir}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_stats(stats_csv: str, out: str, cmd: str):
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel summary."""
    rows = _csv_rows(stats_csv, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel summary", "", f"Command: `{cmd}`", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(fetch_dir: str, write_dir: str, out: str, calib_mb: int, cmd: str):
    """Per-launch HBM bytes of the dominant kernel from two rocprofv3 --pmc runs.
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for the
    copy kernel of known size (calib_mb MiB read and written per launch)."""
    def per_kernel(rows, counter):
        acc = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            a = acc.setdefault(r["Kernel_Name"], [0.0, 0])
            a[0] += float(r["Counter_Value"])
            a[1] += 1
        return {k: (v[0] / v[1], v[1]) for k, v in acc.items()}

    fetch = per_kernel(_csv_rows(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    write = per_kernel(_csv_rows(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    calib_bytes = calib_mb << 20
    copy_name = next(k for k in fetch if "copy_kernel" in k)
    f_fetch = calib_bytes / (fetch[copy_name][0] * 1024.0)
    f_write = calib_bytes / (write[copy_name][0] * 1024.0)
    ffn = [k for k in fetch if "gemv" in k or ("mfma_kernel" in k and "logits" not in k)]
    dom = max(ffn, key=lambda k: fetch[k][0])  # gate/up reads two matrices per expert
    fb = fetch[dom][0] * 1024.0 * f_fetch
    wb = write[dom][0] * 1024.0 * f_write
    d = {"kernel": dom, "command": cmd, "calib_copy_MiB": calib_mb,
         "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4),
         "fetch_kib_per_dispatch": round(fetch[dom][0], 1), "write_kib_per_dispatch": round(write[dom][0], 1),
         "dispatches": fetch[dom][1], "hbm_read_bytes_per_launch": int(fb), "hbm_write_bytes_per_launch": int(wb),
         "hbm_bytes_per_launch": int(fb + wb), "kernel_source_sha256_16": kernel_source_hash(),
         "all_kernels_fetch_kib": {k: round(v[0], 1) for k, v in fetch.items()},
         "all_kernels_write_kib": {k: round(v[0], 1) for k, v in write.items()}}
    with open(out, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    print(json.dumps(d, indent=1))


def down_ops(wl, T: int, pairs: float | None = None) -> int:
    """int8 operations (x2) of one down launch: every pair row against H rows of F inputs."""
    rows = (T * wl["top_k"] if pairs is None else pairs) + (T if wl["has_shared"] else 0)
    return 2 * rows * wl["hidden"] * wl["ffn"]


def summarize_T(wl, r):
    """Derived figures of one run_T result: tokens/s, gate/up bytes and GB/s, layer weight
    bytes and GB/s (the int4 weights + scales the call streams, against the HBM peak)."""
    U = sum(r["U"]) / len(r["U"])
    r["U_mean"] = U
    r["tok_s"] = r["T"] / (r["ms"] * 1e-3)
    gu_ms = r["stage_ms"][DOMINANT_STAGE]
    gb = sum(gateup_bytes(wl, u, r["T"], pr) for u, pr in zip(r["U"], r["pairs"])) / len(r["U"])
    r["gateup_bytes"] = gb
    r["gateup_gbs"] = gb / (gu_ms * 1e-3) / 1e9
    lw = sum(layer_weight_bytes(wl, u) for u in r["U"]) / len(r["U"])
    r["layer_weight_bytes"] = lw
    r["layer_weight_gbs"] = lw / (r["ms"] * 1e-3) / 1e9
    return r


def sweep_entry(r):
    return {"T": r["T"], "calls": r["calls"], "tokens_per_s": round(r["tok_s"], 1),
            "us_per_step": round(r["ms"] * 1e3, 2), "U_mean": r["U_mean"],
            "pairs_mean": sum(r["pairs"]) / len(r["pairs"]), "gate_up_GBps": round(r["gateup_gbs"], 1),
            "layer_weight_GBps": round(r["layer_weight_gbs"], 1),
            "layer_weight_frac": round(r["layer_weight_gbs"] / HBM_PEAK_GBS, 4),
            "stage_calls": r["stage_calls"], "stage_us": {k: round(v * 1e3, 2) for k, v in r["stage_ms"].items()}}


def prefill_leg(args, n_calls: int):
    """The batch-union prefill workload (T = 2048 on one layer whose 4.9 GB of weights
    exceed every cache), timed in the same run: tokens/s per layer and int8 TOP/s of the
    gate/up and down grouped GEMMs against the 5.0 POP/s dense int8 peak."""
    import synth
    stack = Stack(args.prefill_config, 1, args.wbits, args.scale_group, args.topp)
    wl = stack.wl
    T = wl["tokens"][-1]
    r = summarize_T(wl, run_T(stack, T, n_calls, args.warmup, not args.no_graph, n_prof=8))
    pairs = sum(r["pairs"]) / len(r["pairs"])
    gu_ms, dn_ms = r["stage_ms"][DOMINANT_STAGE], r["stage_ms"]["ffn_down"]
    gops, dops = gateup_ops(wl, T, pairs), down_ops(wl, T, pairs)
    gtops, dtops = gops / (gu_ms * 1e-3) / 1e12, dops / (dn_ms * 1e-3) / 1e12
    ceil_tops = scaled_mfma_ceiling()
    log(f"exactly scaled int8 MFMA loop: {ceil_tops:.0f} TOP/s ({ceil_tops / INT8_PEAK_TOPS:.3f} of the int8 peak)")
    ceiling = {"kernel": "synth scaled_mfma (v_mfma_i32_32x32x32_i8 + v_cvt_f32_i32 + v_fma_f32 per result, "
                         "registers only)", "TOPs": round(ceil_tops, 1),
               "frac_of_peak": round(ceil_tops / INT8_PEAK_TOPS, 4),
               "gate_up_frac_of_ceiling": round(gtops / ceil_tops, 4)}
    layer_tops = (gops + dops) / (r["ms"] * 1e-3) / 1e12
    log(f"prefill T={T}: {r['ms']*1e3:.1f} us/step, {r['tok_s']:.0f} tok/s, U={r['U_mean']:.1f}, gate/up "
        f"{gu_ms*1e3:.1f} us = {gtops:.0f} TOP/s, down {dn_ms*1e3:.1f} us = {dtops:.0f} TOP/s; stages(us) " +
        ", ".join(f"{k}={v*1e3:.1f}" for k, v in r["stage_ms"].items()))
    out = {"workload": wl["name"], "tokens": T, "calls": n_calls, "tokens_per_s": round(r["tok_s"], 1),
           "us_per_step": round(r["ms"] * 1e3, 2), "U_mean": r["U_mean"], "pairs_mean": pairs,
           "gate_up": {"kernel": "mfma_kernel (grouped GEMM, v_mfma_i32_32x32x32_i8)", "ops_per_launch": int(gops),
                       "avg_launch_us": round(gu_ms * 1e3, 2), "achieved_TOPs": round(gtops, 1),
                       "peak_TOPs": INT8_PEAK_TOPS, "frac": round(gtops / INT8_PEAK_TOPS, 4),
                       "traffic": read_traffic(wl["name"], T), "weight_GBps": round(r["gateup_gbs"], 1)},
           "down": {"ops_per_launch": int(dops), "avg_launch_us": round(dn_ms * 1e3, 2),
                    "achieved_TOPs": round(dtops, 1), "frac": round(dtops / INT8_PEAK_TOPS, 4)},
           "layer_TOPs": round(layer_tops, 1), "layer_frac": round(layer_tops / INT8_PEAK_TOPS, 4),
           "scaled_mfma_ceiling": ceiling,
           "layer_weight_GBps": round(r["layer_weight_gbs"], 1),
           "stage_calls": r["stage_calls"], "stage_us": {k: round(v * 1e3, 2) for k, v in r["stage_ms"].items()}}
    del stack
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed layer calls at the headline T")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4],
                    help="workload: 1 OLMoE-scale decode, 2 GLM-scale decode (default), 3 GLM-scale prefill, "
                         "4 verify / low-bit")
    ap.add_argument("--prefill-config", type=int, default=3, choices=[0, 3],
                    help="prefill leg timed in the same run (0: none)")
    ap.add_argument("--wbits", type=int, default=None, choices=[2, 4, 8, 40],
                    help="weight format: int2/int4/int8, or 40 = MXFP4 (E2M1 codes, E8M0 scale per 32 inputs)")
    ap.add_argument("--topp", type=float, default=0.0,
                    help="adaptive expert top-p (0: plain top-k); changes the router's result")
    ap.add_argument("--scale-group", type=int, default=0, choices=[0, 64],
                    help="64: group-scaled weights, one fp32 scale per 64 inputs of a row")
    ap.add_argument("--tokens", type=str, default=None, help="comma list of T; the last is the headline")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--sweep-calls", type=int, default=64, help="timed calls per T of the sweep (at least)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--cpu-budget-1t", type=float, default=8.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-mb", type=int, default=1024,
                    help="MiB moved by the copy and read kernels (byte-counter calibration, bandwidth ceilings; 0: skip)")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "OUT"),
                    help="write a short text summary of a rocprofv3 --stats kernel table and exit")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into the traffic summary and exit")
    ap.add_argument("--cmd", type=str, default="", help="the command that produced the profiler output")
    ap.add_argument("--tier-slots", type=int, default=0,
                    help="measure the expert tier instead: experts in pinned host RAM, this many HBM slots per layer")
    ap.add_argument("--tier-lookahead", action="store_true",
                    help="with --tier-slots: prefetch each next layer's predicted union (router lookahead)")
    ap.add_argument("--tier-residual", type=float, default=0.0,
                    help="with --tier-slots: inputs form a synthetic residual stream, x_l = x_(l-1) + sigma * noise")
    args = ap.parse_args()

    if args.summarize_stats:
        summarize_stats(args.summarize_stats[0], args.summarize_stats[1], args.cmd)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.summarize_pmc[2], args.calib_mb, args.cmd)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's sharding across GPUs "
              "is a design note, not built", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        raise SystemExit("--steps must be at least 1")

    if args.tier_slots:
        run_tier(args)
        return

    import synth
    copy_gbs = read_gbs = None
    if args.calib_mb > 0:
        copy_gbs = copy_bandwidth(args.calib_mb, 5)
        read_gbs = read_bandwidth(args.calib_mb, 5)
        log(f"copy kernel ({args.calib_mb} MiB): {copy_gbs:.0f} GB/s read+write; read kernel: {read_gbs:.0f} GB/s")
    wl0 = synth.WORKLOADS[args.config]
    Ts = [int(t) for t in args.tokens.split(",")] if args.tokens else list(wl0["tokens"])
    layers = args.layers if len(wl0["tokens"]) > 1 or wl0["tokens"][0] < 1024 else 1
    stack = Stack(args.config, layers, args.wbits, args.scale_group, args.topp)
    wl = stack.wl
    results = []
    for T in Ts:
        r = summarize_T(wl, run_T(stack, T, max(args.steps, args.sweep_calls), args.warmup, not args.no_graph))
        results.append(r)
        log(f"T={T}: {r['ms']*1e3:.1f} us/step over {r['calls']} calls, {r['tok_s']:.0f} tok/s, U={r['U_mean']:.1f}, "
            f"gate/up {r['stage_ms'][DOMINANT_STAGE]*1e3:.1f} us = {r['gateup_gbs']:.0f} GB/s, layer weights "
            f"{r['layer_weight_gbs']:.0f} GB/s ({r['layer_weight_gbs'] / HBM_PEAK_GBS:.2f} of peak); stages(us) " +
            ", ".join(f"{k}={v*1e3:.1f}" for k, v in r["stage_ms"].items()))
    # the headline: exactly --steps timed layer calls at the last T
    T = Ts[-1]
    head = summarize_T(wl, run_T(stack, T, args.steps, args.warmup, not args.no_graph))
    log(f"headline T={T}: {head['ms']*1e3:.1f} us/step over exactly {args.steps} calls, {head['tok_s']:.0f} tok/s")
    gemm = T * wl["top_k"] > LOCAL_GROUP_MAX_P
    gu_ms = head["stage_ms"][DOMINANT_STAGE]
    traffic = read_traffic(wl["name"], T)
    if gemm:
        ops = int(gateup_ops(wl, T, sum(head["pairs"]) / len(head["pairs"])))
        ach = ops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(ach / INT8_PEAK_TOPS, 4), "traffic": traffic,
                "kernel": "mfma_kernel (gate/up grouped GEMM, v_mfma_i32_32x32x32_i8)",
                "ops_per_launch": ops, "avg_launch_us": round(gu_ms * 1e3, 2),
                "scaled_mfma_ceiling_TOPs": round(scaled_mfma_ceiling(), 1)}
    else:
        ach = head["gateup_gbs"]
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "gate/up GEMV (fused SiLU*up + Q8_0 requantisation)",
                "bytes_per_launch": int(head["gateup_bytes"]), "avg_launch_us": round(gu_ms * 1e3, 2)}
    roof.update({"launches_timed": head["stage_calls"],
                 "measured_copy_GBps": None if copy_gbs is None else round(copy_gbs, 1),
                 "measured_read_GBps": None if read_gbs is None else round(read_gbs, 1),
                 "layer_weight_GBps": round(head["layer_weight_gbs"], 1),
                 "layer_weight_frac": round(head["layer_weight_gbs"] / HBM_PEAK_GBS, 4)})
    prefill = None
    if args.prefill_config and not gemm:
        prefill = prefill_leg(args, max(args.steps // 4, 50))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(stack, T, args.cpu_budget, args.cpu_budget_1t)
        log(f"cpu baseline: {cpu}")
    line = {
        "metric": METRIC,
        "value": round(head["tok_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8x" + {2: "int2", 4: "int4", 8: "int8", 40: "mxfp4"}[wl["wbits"]],
        "data": "synthetic (seeded SplitMix64; random int weights, N(0,1) activations)",
        "config": {"workload": wl["name"], "hidden": wl["hidden"], "ffn": wl["ffn"], "n_experts": wl["n_experts"],
                   "top_k": wl["top_k"], "n_group": wl["n_group"], "topk_group": wl["topk_group"],
                   "rsf": wl["rsf"], "has_shared": wl["has_shared"], "wbits": wl["wbits"],
                   "scale_group": wl.get("scale_group", 0), "topp": wl.get("topp", 0.0), "tokens": T,
                   "stacked_layers": stack.L, "graph": not args.no_graph, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "sweep": [sweep_entry(r) for r in results],
        "prefill": prefill,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
