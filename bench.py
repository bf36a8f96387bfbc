#!/usr/bin/env python3
"""MoE-layer throughput of the expert-cached layer on one MI355X.

One step = one pass of the layer's GPU path over one decode batch: router softmax
+ top-k and permutation (moe_route), then the SwiGLU experts of the step over the
expert slots with the gate-weighted un-permute and merge of their outputs in one
call (moe_expert_ffn_merge; token lists from the host copy of the step's ids, as
the cached pipeline has them; bit-identical to moe_expert_ffn + moe_merge_partial,
whose step time is reported beside it).  K steps are captured once in a HIP graph;
the graph is replayed R_rep times and the median replay gives ``value``.  Inputs
(logits, activations, expert slots) are resident in HBM before the timed region.

``value`` is the largest decode shape that fits one GPU (hidden 4096, 256 routed
experts + 1 shared, top-6, bf16; batch 1) with every expert resident (C = E): the
step excludes the ids copy to the host, the cache plan, PCIe fills and the CPU
experts, which the cached pipeline (``pipeline``) includes.  The expert set of each
step comes from the library's own planner (moe_lru_replay).  Slot pools are
replicated and the steps rotate over the replicas (emulated layers), so every
step's weights come from HBM rather than from the 256 MB last-level cache.

Reported besides ``value``:
  roofline      the decode expert FFN of the headline (moe_expert_ffn: k_decode_gate_up +
                k_decode_down), algorithmic bytes / time per call, timed with HIP events on
                the replay stream around a graph of those calls alone (rotating over the
                pool replicas); ``traffic`` is the counter-measured HBM bytes per call,
                recorded while the decode kernel sources are unchanged, else null;
  configs       per workload and batch: the same step (tokens/s, median and spread), its
                FFN roofline, and the cache-limited GPU step (C = 47 / 28 slots, GPU experts
                = hits + fills of the q* plan, with the GPU share of the step's experts);
                the 8192-token prefill chunks with their MFMA fractions; the trace's sha256,
                measured reuse and Zipf fit;
  prefill       8K chunks with the pool resident, and streamed through emulated layers with
                one and two layer buffers at 4k / 8k / 16k tokens (the single-buffer ablation);
  pipeline      the full cached decode step (GPU route -> ids to the host -> plan with q* ->
                PCIe fills on a side stream + CPU experts -> GPU experts -> merge) at the
                pages' B_P:B_H and at the ratio measured here (B_H at 6 threads pinned to the
                GPU's NUMA node), the ids-copy + plan latency, and the miss statistics of a
                cache shared by a stack of layers; host-link bound, context only;
  cpu_baseline  the fp64 oracle timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (decode, 8K prefill) + % HBM/MFMA roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP4_PEAK_TFLOPS = 10100.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="decode steps per timed graph (K)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replays", type=int, default=10, help="timed replays of each graph (median reported)")
    ap.add_argument("--workload", default="v4flash_decode_bf16", help="decode workload of `value`")
    ap.add_argument("--batch", type=int, default=1, help="decode batch of `value`")
    ap.add_argument("--decode", default="v4flash_decode_bf16:1,2,4,8;a3b_decode_bf16:1,4,8;v4flash_mxfp4:1,2,4,8;"
                                        "tiny_fp32:1",
                    help="decode workloads and batches of the per-config table ('' for none)")
    ap.add_argument("--replicas", type=int, default=0, help="slot-pool replicas (0: enough to defeat the 256 MB cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pipeline", action="store_true")
    ap.add_argument("--pipeline-steps", type=int, default=400)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-reps", type=int, default=10)
    ap.add_argument("--stream-layers", type=int, default=4,
                    help="emulated layers of the streamed prefill chunk (0: skip streaming)")
    ap.add_argument("--stream-tokens", default="4096,8192,16384", help="chunk sizes of the streamed ablation")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain 256 MiB read + 256 MiB write elementwise kernel (torch.neg), "
                         "whose byte counters calibrate FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def payload_bytes(wl):
    """Algorithmic bytes of one expert's weights (codes + scales for MXFP4)."""
    n = 3 * wl.H * wl.I
    return {"f32": 4 * n, "bf16": 2 * n, "mxfp4": n // 2 + n // 32}[wl.wdtype]


# HBM traffic of the decode FFN kernels from hardware counters (rocprofv3 --pmc FETCH_SIZE, then
# --pmc WRITE_SIZE, over the commands in profiles/decode_ffn_and_prefill_gemm_hbm_traffic.md), in KiB per dispatch
# as the counters read them, averaged over the calls of the rotating FFN graph and summed over
# k_decode_gate_up and k_decode_down of one moe_expert_ffn call at batch 1 (every call has the
# same expert count, so the record matches the timed calls).  The same runs read the plain
# 256 MiB read + 256 MiB write kernel of --copy-probe, whose readings give the scale factors.
# A record applies only while the decode kernel sources hash to the value it was taken with.
DECODE_SOURCES = ("ffn_decode.hip", "ffn_common.h", "device_common.h")
_SRC = "fc1b332b1d545db72d1aa9024d3c5ee75f62f084a3a547cc89756564aa3b9168"
TRAFFIC = {
    ("v4flash_decode_bf16", 1): {"sha256": _SRC, "fetch_kib": 86070.0 + 43117.0, "write_kib": 84.0 + 56.0},
    ("a3b_decode_bf16", 1): {"sha256": _SRC, "fetch_kib": 24618.0 + 12358.0, "write_kib": 48.0 + 32.0},
    ("v4flash_mxfp4", 1): {"sha256": _SRC, "fetch_kib": 22925.0 + 11551.0, "write_kib": 42.0 + 56.0},
}
FETCH_FACTOR = 262144.0 / 131080.0
WRITE_FACTOR = 1.0


class _phase:
    """A named range around a bench phase (roctx through torch's marker API), so that a kernel
    trace taken with rocprofv3 --marker-trace can be split by phase."""

    def __init__(self, name):
        self.name = name

    def __enter__(self):
        try:
            import torch
            torch.cuda.nvtx.range_push(self.name)
            self.on = True
        except Exception:
            self.on = False

    def __exit__(self, *exc):
        if self.on:
            import torch
            torch.cuda.synchronize()
            torch.cuda.nvtx.range_pop()


def decode_sources_sha256():
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "expert_cached_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gpu_numa_cpus():
    """CPUs of the GPU's NUMA node within this process's affinity mask, and the node: the node
    from the PCI device of cuda:0 in sysfs (bus id from torch's device properties)."""
    import torch
    allowed = sorted(os.sched_getaffinity(0))
    p = torch.cuda.get_device_properties(0)
    bus, dev, dom = (getattr(p, n, None) for n in ("pci_bus_id", "pci_device_id", "pci_domain_id"))
    node = None
    if bus is not None and dev is not None:
        path = f"/sys/bus/pci/devices/{int(dom or 0):04x}:{int(bus):02x}:{int(dev):02x}.0/numa_node"
        try:
            with open(path) as f:
                node = int(f.read().strip())
        except (OSError, ValueError):
            node = None
    if node is None or node < 0:
        return allowed, node
    try:
        with open(f"/sys/devices/system/node/node{node}/cpulist") as f:
            spec = f.read().strip()
    except OSError:
        return allowed, node
    cpus = set()
    for part in spec.split(","):
        a, _, b = part.partition("-")
        cpus.update(range(int(a), int(b or a) + 1))
    mine = [c for c in allowed if c in cpus]
    return (mine or allowed), node


def timed_replays(graph, stream, n_rep):
    """Replay a captured graph once to warm up, then n_rep times with HIP events recorded on
    the replay stream around each replay; returns the replay times in ms."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_rep)]
    with torch.cuda.stream(stream):
        graph.replay()
        torch.cuda.synchronize()
        for r in range(n_rep):
            ev[2 * r].record(stream)
            graph.replay()
            ev[2 * r + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[2 * r].elapsed_time(ev[2 * r + 1]) for r in range(n_rep)]


def trace_info(wl, sets, ids_all):
    """sha256 of the routed ids, measured reuse, top-decile share and the Zipf exponent fitted to
    the experts' frequency-rank curve (least squares of log frequency on log rank)."""
    import synth
    st = synth.trace_stats(sets, wl.E)
    freq = np.sort(np.bincount(sets.ravel(), minlength=wl.E))[::-1].astype(np.float64)
    n = max(2, int((freq > 0).sum()) // 2)
    r = np.arange(1, n + 1, dtype=np.float64)
    slope = float(np.polyfit(np.log(r), np.log(freq[:n]), 1)[0])
    return {"ids_sha256": hashlib.sha256(np.ascontiguousarray(ids_all, np.int32).tobytes()).hexdigest(),
            "steps": int(ids_all.shape[0]), "reuse": round(st["reuse"], 4),
            "top_decile_share": round(st["top_decile_share"], 4), "zipf_fit_s": round(-slope, 3),
            "zipf_fit_ranks": n}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    table = [(args.workload, [args.batch])]
    if args.decode:
        for item in args.decode.split(";"):
            name, _, bs = item.partition(":")
            table.append((name.strip(), [int(v) for v in bs.split(",") if v.strip()]))
    # one pass per workload (weights drawn once), the headline batch first
    order = []
    for name, bs in table:
        for n_, b in ((name, b) for b in bs):
            if (n_, b) not in order:
                order.append((n_, b))
    configs, head = {}, None
    by_wl = {}
    for name, b in order:
        by_wl.setdefault(name, []).append(b)
    for name, batches in by_wl.items():
        wl = synth.workload(name)
        t0 = time.time()
        experts = synth.expert_weights_many(wl, range(wl.E + wl.n_shared), threads=16)
        log(f"{name}: expert weights drawn in {time.time() - t0:.1f}s")
        entry = configs.setdefault(name, {"hidden": wl.H, "inter": wl.I, "experts": wl.E, "top_k": wl.k,
                                          "shared_experts": wl.n_shared, "weights": wl.wdtype, "slots": wl.C,
                                          "decode": {}})
        for b in batches:
            with _phase(f"decode {name} batch {b}"):
                d = decode(args, wl, b, experts)
            if name == args.workload and b == args.batch:
                head = d
            entry["decode"][str(b)] = {k_: d[k_] for k_ in ("tokens_per_s", "ms_per_step", "ms_per_step_min",
                                                            "ms_per_step_max", "two_calls_ms_per_step",
                                                            "gpu_experts_per_step", "replicas", "roofline",
                                                            "cache_limited", "trace")}
        if name == args.workload:
            head_experts = experts
        else:
            del experts

    wl = synth.workload(args.workload)
    d = head
    Bt = args.batch
    result = {"metric": METRIC, "value": d["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": d["ms_per_step"], "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": wl.wdtype, "data": "synthetic",
              "config": {"workload": f"{wl.name} decode, batch {Bt}", "hidden": wl.H, "inter": wl.I,
                         "experts": wl.E, "top_k": wl.k, "shared_experts": wl.n_shared, "batch": Bt,
                         "n_slots": wl.E, "residency": "all experts resident (C = E)",
                         "replicas": d["replicas"], "gpu_experts_per_step": d["gpu_experts_per_step"],
                         "replays": args.replays,
                         "ms_per_step_min_max": [d["ms_per_step_min"], d["ms_per_step_max"]],
                         "step": "route+permute, then experts+merge in one call (moe_expert_ffn_merge); HIP graph of "
                                 "K steps, median of the replays; excludes the ids copy to the host, the cache "
                                 "plan, PCIe fills and CPU experts (see pipeline)"},
              "roofline": d["roofline"]}

    # ---------------------------------------------------------------- 8K prefill chunks
    if not args.no_prefill:
        torch.cuda.empty_cache()
        result["prefill"] = {}
        for name in ("a3b_prefill8k_bf16", "v4flash_mxfp4"):
            with _phase(f"prefill {name}"):
                result["prefill"][name] = prefill(args, name)
            configs.setdefault(name, {})["prefill8k"] = {
                k_: result["prefill"][name][k_] for k_ in ("tokens_per_s", "ms_per_chunk", "gemm_ms", "gemm_tflops",
                                                           "mfma_frac_bf16_peak", "mfma_frac_fp4_peak")
                if k_ in result["prefill"][name]}
    result["configs"] = configs

    # ---------------------------------------------------------------- full cached pipeline (context)
    if not args.no_pipeline:
        with _phase("cached decode pipeline"):
            wl_pipe = synth.workload("a3b_decode_bf16")
            result["pipeline"] = pipeline(args, wl_pipe, synth.expert_weights_many(wl_pipe, range(wl_pipe.E),
                                                                                   threads=16))
            result["pipeline"]["layer_stack"] = layer_stack_stats()

    # ---------------------------------------------------------------- CPU baseline: the oracle
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, wl, head_experts, d["logits"], d["x"])
    print(json.dumps(result), flush=True)


def decode(args, wl, Bt, experts):
    """Decode steps at batch Bt: planner replay, pools, the graph of K timed steps, the FFN
    roofline (a graph of FFN calls alone, rotating over the pool replicas) and the
    cache-limited GPU step."""
    import torch
    import synth
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool
    K, W, NR = args.steps, args.warmup, args.replays
    dt = {"f32": B.MOE_W_F32, "bf16": B.MOE_W_BF16, "mxfp4": B.MOE_W_MXFP4}[wl.wdtype]
    E, k, H = wl.E, wl.k, wl.H
    n_trace = wl.steps

    # ---------------------------------------------------------------- inputs
    if wl.name == "tiny_fp32":
        import oracle
        x = synth.activations(wl, n_trace * Bt, tag=21)
        logits = oracle.router_logits(x, synth.router_weights(wl)).reshape(n_trace, Bt, E)
        sets = None
    else:
        logits, sets = synth.zipf_reuse_trace(wl, Bt, n_trace)
        x = synth.activations(wl, n_trace * Bt, tag=11)

    # routing of every trace step on the GPU, copied back once for the planner
    cfg_res = B.make_config(wl.H, wl.I, E, k, wl.n_shared, E, 1, dt, 1, 0, 1.0, 1.0)
    L = LayerBuffers(cfg_res, Bt)
    d_logits = torch.from_numpy(np.ascontiguousarray(logits.reshape(n_trace * Bt, E))).cuda()
    ids_all = np.empty((n_trace, Bt, k), np.int32)
    for s in range(n_trace):
        L.route(d_logits[s * Bt:(s + 1) * Bt], Bt)
        ids_all[s] = L.ids[: Bt * k].view(Bt, k).cpu().numpy()

    def plan_sets(cfg):
        """GPU experts (hits + fills) and their slots of every trace step under cfg's cache."""
        planner = B.moe_create(cfg)
        cap = min(E, Bt * k)
        plans = [B.Plan(cap, E) for _ in range(n_trace)]
        st = B.moe_lru_replay(planner, 0, ids_all, n_trace, Bt, plans)
        B.moe_destroy(planner)
        ex = [np.concatenate([p.get("hit"), p.get("fill")]).astype(np.int32) for p in plans]
        sl = [np.concatenate([p.get("hit_slot"), p.get("fill_slot")]).astype(np.int32) for p in plans]
        nd = [int(p.c.n_distinct) for p in plans]
        return ex, sl, nd, st

    # all-resident plan: C = E slots, every miss filled (B_P = B_H)
    step_experts, step_slots, n_distinct, _ = plan_sets(cfg_res)
    mean_distinct = float(np.mean([len(e) for e in step_experts]))
    planner = B.moe_create(cfg_res)
    B.moe_lru_replay(planner, 0, ids_all, n_trace, Bt)
    slot_of = B.moe_lru_slots(planner, 0, E)
    B.moe_destroy(planner)

    # pool laid out by the planner's slots; replicas defeat the last-level cache
    order = [int(np.where(slot_of == s)[0][0]) if (slot_of == s).any() else 0 for s in range(E)]
    host_pool = pack_pool(cfg_res, [experts[e] for e in order], pin=False)
    step_bytes = mean_distinct * payload_bytes(wl) + (payload_bytes(wl) if wl.n_shared else 0)
    R = args.replicas or max(1, math.ceil(4 * MALL_BYTES / step_bytes))
    R = min(R, max(K, 100), max(1, int((48 << 30) // host_pool.numel())))
    pools = [host_pool.cuda() for _ in range(R)]
    del host_pool
    shared = None
    if wl.n_shared:
        sh = pack_pool(cfg_res, [experts[E]], pin=False)
        shared = [sh.cuda() for _ in range(R)]
    d_x = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
    out = torch.empty(Bt * H, dtype=torch.int16 if wl.act_dtype == "bf16" else torch.float32, device="cuda")
    with_shared = 1 if wl.n_shared else 0
    torch.cuda.synchronize()
    log(f"{wl.name} batch {Bt}: pool {B.moe_expert_bytes(cfg_res) * E / 1e9:.2f} GB x {R} replicas, "
        f"mean GPU experts/step {mean_distinct:.2f}")

    stream = torch.cuda.Stream()
    h_ids_steps = [np.ascontiguousarray(ids_all[t]) for t in range(n_trace)]

    def ffn_merge(s_idx, exps, slts, rotate=True):
        t, r = s_idx % n_trace, (s_idx % R if rotate else 0)
        L.ffn_merge(d_x[t * Bt:(t + 1) * Bt], Bt, pools[r], exps[t], slts[t], h_ids_steps[t],
                    shared[r] if shared else None, with_shared, None, out, torch.cuda.current_stream())

    def ffn(s_idx, rotate=True):
        """The step's experts alone (moe_expert_ffn: the pair outputs)."""
        t, r = s_idx % n_trace, (s_idx % R if rotate else 0)
        L.ffn(d_x[t * Bt:(t + 1) * Bt], Bt, pools[r], step_experts[t], step_slots[t],
              shared[r] if shared else None, with_shared, torch.cuda.current_stream(), h_ids=h_ids_steps[t])

    def enqueue(s_idx, exps=step_experts, slts=step_slots):
        t = s_idx % n_trace
        L.route(d_logits[t * Bt:(t + 1) * Bt], Bt, torch.cuda.current_stream())
        ffn_merge(s_idx, exps, slts)

    def enqueue_two_calls(s_idx):
        """The same step through moe_expert_ffn (pair outputs) and moe_merge_partial."""
        t, r = s_idx % n_trace, s_idx % R
        st = torch.cuda.current_stream()
        L.route(d_logits[t * Bt:(t + 1) * Bt], Bt, st)
        L.ffn(d_x[t * Bt:(t + 1) * Bt], Bt, pools[r], step_experts[t], step_slots[t],
              shared[r] if shared else None, with_shared, st, h_ids=h_ids_steps[t])
        L.merge(step_experts[t], with_shared, None, Bt, out, st)

    def graph_ms(body, n, n_rep=NR, name="graph"):
        """Capture body(W + s) for s < n; per-iteration ms of each timed replay.  The replays run
        inside a marker range of their own (``name``), so a kernel trace taken with
        --marker-trace attributes every dispatch to the graph it belongs to."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s in range(n):
                body(W + s)
        with _phase(f"{wl.name} b{Bt} {name}"):
            ts = timed_replays(g, stream, n_rep)
        del g
        return [t / n for t in ts]

    with torch.cuda.stream(stream):
        for s in range(min(W, 64)):                        # eager warm-up (code objects, caches)
            enqueue(s)
    torch.cuda.synchronize()
    step_ms = graph_ms(enqueue, K, name="step")
    ms_per_step = float(np.median(step_ms))
    value = Bt / (ms_per_step / 1e3)
    two_calls_ms = float(np.median(graph_ms(enqueue_two_calls, K, name="two-call step")))


    # ---------------------------------------------------------------- decode FFN roofline
    # The expert FFN calls (moe_expert_ffn: the HBM-streaming kernels) of n_prof consecutive
    # steps alone in one graph: each call reads its experts from the next pool replica, so the
    # weights come from HBM, and the per-call time is the two kernels' durations back to back.
    n_prof = max(K, 100)
    ffn_ms = float(np.median(graph_ms(ffn, n_prof, name="ffn roofline")))
    warm_ms = float(np.median(graph_ms(lambda s_idx: ffn(s_idx, rotate=False), n_prof, 3, name="ffn warm")))
    fused_ms = float(np.median(graph_ms(lambda s_idx: ffn_merge(s_idx, step_experts, step_slots), n_prof,
                                        name="ffn+merge call")))
    pairs = Bt * k + (Bt if with_shared else 0)
    act = 2 if wl.act_dtype == "bf16" else 4
    w_bytes = 0.0
    for s in range(n_prof):
        w_bytes += (len(step_experts[(W + s) % n_trace]) + with_shared) * payload_bytes(wl)
    w_bytes /= n_prof
    ffn_bytes = w_bytes + Bt * H * act + pairs * H * act              # weights, x, pair outputs
    fused_bytes = w_bytes + Bt * H * act + Bt * H * act + pairs * 8   # weights, x, layer output, ids + gates
    achieved = ffn_bytes / (ffn_ms / 1e3) / 1e9
    rec = TRAFFIC.get((wl.name, Bt))
    traffic = None
    if rec is not None and rec["sha256"] == decode_sources_sha256():
        traffic = round((rec["fetch_kib"] * FETCH_FACTOR + rec["write_kib"] * WRITE_FACTOR) * 1024)
    roofline = {"bound": "hbm", "kernel": "moe_expert_ffn, decode (k_decode_gate_up + k_decode_down)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_source": "recorded rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of these decode kernel sources "
                                  "(null when the sources changed since)",
                "ffn_us": round(ffn_ms * 1e3, 3), "bytes_per_launch": round(ffn_bytes), "launches_timed": n_prof,
                "warm_r1": {"ffn_us": round(warm_ms * 1e3, 3),
                            "achieved": round(ffn_bytes / (warm_ms / 1e3) / 1e9, 1)},
                "step_call": {"call": "moe_expert_ffn_merge (k_decode_gate_up + k_decode_down_merge when the "
                                      "list has at most 8 entries, else + k_decode_down + k_merge)",
                              "us": round(fused_ms * 1e3, 3), "bytes_per_launch": round(fused_bytes),
                              "achieved": round(fused_bytes / (fused_ms / 1e3) / 1e9, 1),
                              "frac": round(fused_bytes / (fused_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}}

    # ---------------------------------------------------------------- cache-limited GPU step
    # The q* plan of the workload's C slots at the pages' 52.7 : 77.3: the GPU computes the hits
    # and the fills of each step (timing does not depend on which expert a slot holds, so the
    # replicated pool's first C slots stand in for the cache's contents).
    cache_limited = None
    if wl.C < E:
        cfg_c = B.make_config(wl.H, wl.I, E, k, wl.n_shared, wl.C, 1, dt, 1, 0, 52.7, 77.3)
        ce, cs, cnd, cst = plan_sets(cfg_c)
        gpu_share = float(np.sum([len(e) for e in ce]) / max(1, np.sum(cnd)))
        c_ms = float(np.median(graph_ms(lambda s_idx: enqueue(s_idx, ce, cs), K, name="cache-limited step")))
        cache_limited = {"slots": wl.C, "bp_bh": [52.7, 77.3], "tokens_per_s": round(Bt / (c_ms / 1e3), 1),
                         "ms_per_step": round(c_ms, 5),
                         "gpu_experts_per_step": round(float(np.mean([len(e) for e in ce])), 3),
                         "gpu_share_of_step_experts": round(gpu_share, 4),
                         "miss_rate": round(cst.misses / max(1, cst.distinct), 4),
                         "host_experts_per_step": round(cst.host / n_trace, 3),
                         "note": "GPU part of the cached step only: the CPU experts and PCIe fills run beside it "
                                 "(see pipeline)"}
    log(f"{wl.name} batch {Bt}: {ms_per_step * 1e3:.2f} us/step, {value:.0f} tok/s; FFN {ffn_ms * 1e3:.2f} us, "
        f"{achieved:.0f} GB/s")
    L.close()
    del pools, shared, d_logits, d_x
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(value, 1), "ms_per_step": round(ms_per_step, 5),
            "ms_per_step_min": round(float(np.min(step_ms)), 5), "ms_per_step_max": round(float(np.max(step_ms)), 5),
            "replicas": R, "two_calls_ms_per_step": round(two_calls_ms, 5),
            "gpu_experts_per_step": round(mean_distinct, 3), "roofline": roofline, "cache_limited": cache_limited,
            "trace": trace_info(wl, sets, ids_all) if sets is not None else None,
            "logits": logits, "x": x}


def prefill(args, name):
    """One 8192-token chunk through route + grouped GEMMs + merge with the layer's pool
    resident in HBM, captured in a graph and replayed; MFMA roofline of the two GEMMs; the
    chunk streamed through emulated layers at several chunk sizes."""
    import torch
    import synth
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool
    wl = synth.workload(name)
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    dt = {"f32": B.MOE_W_F32, "bf16": B.MOE_W_BF16, "mxfp4": B.MOE_W_MXFP4}[wl.wdtype]
    cfg = B.make_config(H, I, E, k, wl.n_shared, 0, 1, dt)
    experts = synth.expert_weights_many(wl, range(E + wl.n_shared), threads=16)
    host_pool = pack_pool(cfg, [experts[e] for e in range(E)], pin=args.stream_layers > 0)
    pool = host_pool.cuda()
    shared = pack_pool(cfg, [experts[E]], pin=False).cuda() if wl.n_shared else None
    del experts
    L = LayerBuffers(cfg, T)
    d_logits = torch.from_numpy(synth.iid_logits(wl, T)).cuda()
    x = synth.activations(wl, T, tag=3)
    d_x = torch.from_numpy(x.view(np.int16)).cuda()
    out = torch.empty(T * H, dtype=torch.int16, device="cuda")
    allx = np.arange(E, dtype=np.int32)
    ws = 1 if wl.n_shared else 0
    stream = torch.cuda.Stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def step(events=False):
        L.route(d_logits, T, stream)
        if events:
            ev[0].record(stream)
        L.ffn(d_x, T, pool, allx, allx, shared, ws, stream)
        if events:
            ev[1].record(stream)
        L.merge(allx, ws, None, T, out, stream)

    with torch.cuda.stream(stream):
        for _ in range(3):
            step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(args.prefill_reps):
            step()
    with _phase(f"prefill {name} chunk graph"):
        chunk_ms = [t / args.prefill_reps for t in timed_replays(g, stream, 5)]
    ms = float(np.median(chunk_ms))
    del g
    # FFN alone (events around the grouped GEMMs of eager chunks)
    gemm_ms = []
    with _phase(f"prefill {name} gemm timing"), torch.cuda.stream(stream):
        for _ in range(7):
            step(events=True)
            torch.cuda.synchronize()
            gemm_ms.append(ev[0].elapsed_time(ev[1]))
    gms = float(np.median(gemm_ms[1:]))
    # router logits of the chunk (moe_router_logits), context: the chunk itself starts from logits
    d_wr = torch.from_numpy(np.ascontiguousarray(synth.router_weights(wl).T)).cuda()
    lg = torch.empty(T * E, dtype=torch.float32, device="cuda")
    rl_ms = []
    with torch.cuda.stream(stream):
        for _ in range(5):
            ev[0].record(stream)
            B.moe_router_logits(L.ctx, d_x, T, d_wr, lg, stream)
            ev[1].record(stream)
            torch.cuda.synchronize()
            rl_ms.append(ev[0].elapsed_time(ev[1]))
    del d_wr, lg
    flops = 6.0 * T * k * H * I + (6.0 * T * H * I if wl.n_shared else 0.0)
    tflops = flops / (gms / 1e3) / 1e12
    nb = B.moe_expert_bytes(cfg)
    res = {"tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_chunk": round(ms, 4),
           "ms_per_chunk_min_max": [round(min(chunk_ms), 4), round(max(chunk_ms), 4)], "tokens": T,
           "gemm_ms": round(gms, 4), "gemm_tflops": round(tflops, 1),
           "router_logits_ms": round(float(np.median(rl_ms)), 4),
           "mfma_frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4), "gflop": round(flops / 1e9, 1),
           "pool_gb": round(nb * E / 1e9, 3), "weights": wl.wdtype,
           "note": "layer pool resident in HBM"}
    if wl.wdtype == "mxfp4":
        res["mfma_frac_fp4_peak"] = round(tflops / FP4_PEAK_TFLOPS, 4)
        res["note"] += "; MXFP4 weights dequantised to bf16 MFMA operands (bf16 MFMA), so the FP4 fraction " \
                       "is against a peak this path does not use"
    del pool
    L.close()
    if args.stream_layers > 0:
        res["streamed"] = {}
        sizes = [int(v) for v in args.stream_tokens.split(",") if v.strip()] if wl.wdtype == "bf16" else [T]
        for Ts in sizes:
            res["streamed"][str(Ts)] = stream_chunk(args, wl, cfg, host_pool, shared, Ts)
    return res


def stream_chunk(args, wl, cfg, host_pool, shared, T):
    """A T-token chunk through n emulated layers whose pools upload from pinned host memory
    (moe_prefill_stream), with two layer buffers and with one (the single-buffer ablation),
    against the overlap model built from the measured upload and compute."""
    import torch
    import synth
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import LayerBuffers
    n, E = args.stream_layers, wl.E
    nb = B.moe_expert_bytes(cfg)
    layer_bytes = nb * E
    scfg = B.make_config(wl.H, wl.I, E, wl.k, wl.n_shared, 0, n, cfg.w_dtype)
    ctx = B.moe_create(scfg)
    L = LayerBuffers(cfg, T)
    d_logits = torch.from_numpy(synth.iid_logits(wl, T)).cuda()
    d_x = torch.from_numpy(synth.activations(wl, T, tag=3).view(np.int16)).cuda()
    # every emulated layer streams a full layer pool (the layers hold copies of one pool:
    # the transfer and the kernels do not depend on the values)
    hp = torch.empty(n * layer_bytes, dtype=torch.uint8, pin_memory=True)
    for l in range(n):
        hp[l * layer_bytes:(l + 1) * layer_bytes].copy_(host_pool)
    B.moe_bind_pools(ctx, None, 0, hp, n * E)
    bufs = torch.empty(2 * layer_bytes, dtype=torch.uint8, device="cuda")
    logits_n = d_logits.repeat(n, 1).contiguous()
    sh_n = shared.repeat(n).contiguous() if shared is not None else None
    out = torch.empty(n * T * wl.H, dtype=torch.int16, device="cuda")
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # B_P: one layer pool, pinned host -> device, on the upload stream
    ups = []
    for _ in range(3):
        e0.record(side)
        B.moe_upload(ctx, bufs, hp, layer_bytes, side)
        e1.record(side)
        torch.cuda.synchronize()
        ups.append(e0.elapsed_time(e1))
    up_ms = float(np.median(ups))
    # compute of one layer with its pool resident (the first buffer holds a pool now)
    allx = np.arange(E, dtype=np.int32)
    ws = 1 if wl.n_shared else 0
    comp = []
    for _ in range(4):
        e0.record(main)
        L.route(d_logits, T, main)
        L.ffn(d_x, T, bufs, allx, allx, shared, ws, main)
        L.merge(allx, ws, None, T, out, main)
        e1.record(main)
        torch.cuda.synchronize()
        comp.append(e0.elapsed_time(e1))
    compute_ms = float(np.median(comp[1:]))

    def chunk(n_buf):
        times = []
        for _ in range(3):
            e0.record(main)
            B.moe_prefill_stream(ctx, bufs, n_buf, logits_n, d_x, T, sh_n, L.ids, L.w, L.counts, L.offsets,
                                 L.perm, L.inv, L.o, L.ws, out, main, side)
            e1.record(main)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return float(np.median(times))

    double_ms, single_ms = chunk(2), chunk(1)
    B.moe_destroy(ctx)
    L.close()
    del hp, bufs
    torch.cuda.empty_cache()
    pred2 = up_ms + (n - 1) * max(up_ms, compute_ms) + compute_ms
    pred1 = n * (up_ms + compute_ms)
    return {"layers": n, "tokens": T, "layer_gb": round(layer_bytes / 1e9, 3),
            "bp_gbps": round(layer_bytes / (up_ms / 1e3) / 1e9, 2),
            "layer_upload_ms": round(up_ms, 3), "layer_compute_ms": round(compute_ms, 4),
            "compute_over_upload": round(compute_ms / up_ms, 4),
            "double_ms": round(double_ms, 3), "single_ms": round(single_ms, 3),
            "double_pred_ms": round(pred2, 3), "single_pred_ms": round(pred1, 3),
            "chunk_tokens_per_s_double": round(T / (double_ms / 1e3), 1),
            "single_buffer_penalty": round(1.0 - double_ms / single_ms, 4),
            "note": "PCIe-inclusive; prediction: double = U + (n-1) max(U, C) + C, single = n (U + C)"}


def measure_bandwidths(B, ctx_cfg, host_pool, slots, nb, wl, side, n_exp=16):
    """The pages' two rates on this machine: B_P, pinned host -> device copies of single
    expert blobs (as fills are issued), and B_H, the rate at which the CPU experts
    (moe_host_ffn) stream expert weights from the pinned pool: at 6 threads pinned to the
    GPU's NUMA node (the pages' edge emulation), at 6 unpinned threads and at all threads."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_exp = min(n_exp, wl.E, wl.C)
    ctx = B.moe_create(ctx_cfg)
    B.moe_bind_pools(ctx, slots, wl.C, host_pool, wl.E)

    def timed(per_blob):
        ts = []
        for rep in range(6):                              # the first pass warms the path up
            e0.record(side)
            if per_blob:
                for i in range(n_exp):
                    B.moe_upload(ctx, slots[i * nb:(i + 1) * nb], host_pool[i * nb:(i + 1) * nb], nb, side)
            else:
                B.moe_upload(ctx, slots[: n_exp * nb], host_pool[: n_exp * nb], n_exp * nb, side)
            e1.record(side)
            torch.cuda.synchronize()
            if rep:
                ts.append(e0.elapsed_time(e1))
        return n_exp * nb / (float(np.median(ts)) / 1e3) / 1e9

    bp = timed(True)
    bp_batched = timed(False)
    B.moe_destroy(ctx)
    k = wl.k
    T = (n_exp + k - 1) // k
    ids = np.array([[(t * k + j) % n_exp if t * k + j < n_exp else (t * k + j) % wl.E for j in range(k)]
                    for t in range(T)], np.int32)
    host = sorted(set(ids.ravel().tolist()))
    h_x = torch.zeros(T * wl.H, dtype=torch.int16 if wl.act_dtype == "bf16" else torch.float32)
    h_w = np.full((T, k), 1.0 / k, np.float32)
    h_y = torch.zeros(T * wl.H, dtype=torch.float32)
    numa_cpus, node = gpu_numa_cpus()
    all_cpus = sorted(os.sched_getaffinity(0))

    def bh(nt, cpus):
        """B_H with nt threads created under the affinity mask cpus (a fresh context, so its
        worker threads are created under the mask)."""
        os.sched_setaffinity(0, cpus)
        try:
            c = B.moe_create(ctx_cfg)
            B.moe_bind_pools(c, None, 0, host_pool, wl.E)
            plan = B.Plan(len(host), wl.E)
            plan.arrays["host"][: len(host)] = host
            plan.c.n_host = len(host)
            plan.c.layer = 0
            ts = []
            for _ in range(6):
                t0 = time.perf_counter()
                B.moe_host_ffn(c, h_x, T, ids, h_w, plan, h_y, nt)
                ts.append(time.perf_counter() - t0)
            B.moe_destroy(c)
        finally:
            os.sched_setaffinity(0, all_cpus)
        return round(len(host) * payload_bytes(wl) / float(np.median(ts[1:])) / 1e9, 2)

    n_all = len(all_cpus)
    nt_pipe = min(16, n_all)
    out = {"bp_gbps": round(bp, 2), "bp_gbps_one_copy": round(bp_batched, 2),
           "bh_gbps_6_threads_numa_pinned": bh(6, numa_cpus[:6] if len(numa_cpus) >= 6 else numa_cpus),
           "bh_gbps_6_threads": bh(6, all_cpus), "bh_gbps_all_threads": bh(n_all, all_cpus),
           "bh_gbps_pipeline_threads": bh(nt_pipe, all_cpus),
           "gpu_numa_node": node, "numa_cpus_used": (numa_cpus[:6] if len(numa_cpus) >= 6 else numa_cpus),
           "threads_all": n_all, "threads_pipeline": nt_pipe, "cpu_model": cpu_model()}
    b_h = out["bh_gbps_pipeline_threads"]
    out["qstar_at_measured_ratio"] = {m: B.moe_qstar(m, bp, b_h, 0) for m in range(1, 9)}
    return out


def pipeline(args, wl, experts):
    """Cached decode of the a3b shape at batch 1: route on the GPU, plan on the host (global
    LRU + q*), upload the fills on a side stream while the hits run, CPU experts in parallel,
    merge.  Run at the pages' B_P:B_H and at the ratio measured on this machine."""
    import torch
    import synth
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import pack_pool
    E = wl.E
    dt = {"f32": B.MOE_W_F32, "bf16": B.MOE_W_BF16, "mxfp4": B.MOE_W_MXFP4}[wl.wdtype]
    cfg0 = B.make_config(wl.H, wl.I, E, wl.k, wl.n_shared, wl.C, 1, dt, 1, 0, 52.7, 77.3)
    nb = B.moe_expert_bytes(cfg0)
    host_pool = pack_pool(cfg0, [experts[e] for e in range(E)], pin=True)
    slots = torch.empty(wl.C * nb, dtype=torch.uint8, device="cuda")
    shared = pack_pool(cfg0, [experts[E]], pin=False).cuda() if wl.n_shared else None
    bw = measure_bandwidths(B, cfg0, host_pool, slots, nb, wl, torch.cuda.Stream())
    Bt = 1
    logits, _ = synth.zipf_reuse_trace(wl, Bt, wl.steps)
    x = synth.activations(wl, wl.steps * Bt, tag=11)
    res = run_pipeline(args, wl, Bt, logits, x, dt, host_pool, slots, shared, 52.7, 77.3)
    res["measured"] = bw
    res["at_measured_ratio"] = run_pipeline(args, wl, Bt, logits, x, dt, host_pool, slots, shared, bw["bp_gbps"],
                                            bw["bh_gbps_pipeline_threads"])
    res["workload"] = f"{wl.name} decode, batch {Bt}, {wl.C} slots"
    return res


def run_pipeline(args, wl, Bt, logits, x, dt, host_pool, slots, shared, bp, bh):
    import torch
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import LayerBuffers
    E, k, H = wl.E, wl.k, wl.H
    cfg = B.make_config(wl.H, wl.I, E, k, wl.n_shared, wl.C, 1, dt, 1, 0, bp, bh)
    L = LayerBuffers(cfg, Bt)
    B.moe_bind_pools(L.ctx, slots, wl.C, host_pool, E)
    n_trace = wl.steps
    d_logits = torch.from_numpy(logits.reshape(n_trace * Bt, E)).cuda()
    d_x = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
    h_ids = torch.empty(Bt * k, dtype=torch.int32, pin_memory=True)
    h_w = torch.empty(Bt * k, dtype=torch.float32, pin_memory=True)
    h_x = torch.empty(Bt * H, dtype=d_x.dtype, pin_memory=True)
    h_y = torch.zeros(Bt * H, dtype=torch.float32, pin_memory=True)
    d_y = torch.empty(Bt * H, dtype=torch.float32, device="cuda")
    out = torch.empty(Bt * H, dtype=d_x.dtype, device="cuda")
    plan = B.Plan(min(E, Bt * k), E)
    main_s, side = torch.cuda.current_stream(), torch.cuda.Stream()
    ws = 1 if wl.n_shared else 0
    nthreads = min(16, os.cpu_count() or 1)
    lat = []

    def step(s, record=False):
        t = s % n_trace
        L.route(d_logits[t * Bt:(t + 1) * Bt], Bt, main_s)
        t0 = time.perf_counter()
        h_ids.copy_(L.ids[: Bt * k], non_blocking=True)
        h_w.copy_(L.w[: Bt * k], non_blocking=True)
        h_x.copy_(d_x[t * Bt:(t + 1) * Bt].view(-1), non_blocking=True)
        main_s.synchronize()
        B.moe_lru_step(L.ctx, 0, h_ids.numpy().reshape(Bt, k), Bt, plan)
        if record:
            lat.append(time.perf_counter() - t0)
        B.moe_fill(L.ctx, plan, side)
        hits, hslots = plan.get("hit").copy(), plan.get("hit_slot").copy()
        fills, fslots = plan.get("fill").copy(), plan.get("fill_slot").copy()
        ids_np = h_ids.numpy().reshape(Bt, k)
        L.ffn(d_x[t * Bt:(t + 1) * Bt], Bt, slots, hits, hslots, shared, ws, main_s, h_ids=ids_np)
        B.moe_fill_wait(L.ctx, main_s)
        L.ffn(d_x[t * Bt:(t + 1) * Bt], Bt, slots, fills, fslots, None, 0, main_s, h_ids=ids_np)
        have_host = plan.c.n_host > 0
        if have_host:
            B.moe_host_ffn(L.ctx, h_x, Bt, h_ids, h_w, plan, h_y, nthreads)
            d_y.copy_(h_y, non_blocking=True)
        gpu = np.concatenate([hits, fills]).astype(np.int32)
        L.merge(gpu, ws, d_y if have_host else None, Bt, out, main_s)

    for s in range(64):
        step(s)
    torch.cuda.synchronize()
    B.moe_lru_reset(L.ctx)
    n = args.pipeline_steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(n):
        step(s, record=True)
    torch.cuda.synchronize()
    dt_s = time.perf_counter() - t0
    st = B.moe_lru_stats(L.ctx)
    L.close()
    return {"tokens_per_s": round(Bt * n / dt_s, 1), "steps": n, "ms_per_step": round(dt_s * 1e3 / n, 4),
            "ids_copy_and_plan_us": round(float(np.median(lat)) * 1e6, 2),
            "slots": wl.C, "bp_bh": [bp, bh], "miss_rate": round(st.misses / max(1, st.distinct), 4),
            "fills_per_step": round(st.fills / n, 3), "host_experts_per_step": round(st.host / n, 3),
            "cold_start": True, "note": "includes host-link fills and CPU experts; context only"}


def layer_stack_stats(steps=1024):
    """One cache over a stack of L layers (key = (layer, expert)), capacity the workload's
    fraction of the whole pool (37 % / 11 % of L * E), each layer routed by its own Zipf trace,
    every step planning layer 0 .. L-1: miss rate, fills and CPU experts per layer-step, from
    the library's planner at the pages' 52.7 : 77.3."""
    import synth
    import oracle
    from expert_cached_moe_amd import binding as B
    out = {}
    for name, Bt in (("a3b_decode_bf16", 1), ("v4flash_decode_bf16", 1)):
        wl = synth.workload(name)
        res = {}
        for NL in (1, 4, 8):
            C = int(round(wl.C / wl.E * NL * wl.E))
            cfg = B.make_config(wl.H, wl.I, wl.E, wl.k, wl.n_shared, C, NL, B.MOE_W_BF16, 1, 0, 52.7, 77.3)
            ctx = B.moe_create(cfg)
            traces = [synth.zipf_reuse_trace(wl, Bt, steps, tag=100 + l)[0] for l in range(NL)]
            ids = [np.stack([oracle.route(tr[s], wl.k)[0] for s in range(steps)]) for tr in traces]
            p = B.Plan(min(wl.E, Bt * wl.k), wl.E)
            t0 = time.perf_counter()
            for s in range(steps):
                for l in range(NL):
                    B.moe_lru_step(ctx, l, ids[l][s], Bt, p)
            plan_us = (time.perf_counter() - t0) / (steps * NL) * 1e6
            st = B.moe_lru_stats(ctx)
            B.moe_destroy(ctx)
            res[str(NL)] = {"slots": C, "miss_rate": round(st.misses / max(1, st.distinct), 4),
                            "fills_per_layer_step": round(st.fills / (steps * NL), 3),
                            "host_experts_per_layer_step": round(st.host / (steps * NL), 3),
                            "plan_us_per_layer_step": round(plan_us, 2)}
        out[name] = {"batch": Bt, "steps": steps, "capacity_fraction": round(wl.C / wl.E, 4), "layers": res}
    return out


def cpu_baseline(args, wl, experts, logits, x):
    """The fp64 oracle on the host cores: route + layer for as many steps as fit in about
    --cpu-seconds of timed work; each expert's weights decoded to fp64 once, outside the timed
    part (resident, like the GPU's)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    Bt, k = args.batch, wl.k
    W64 = {}
    shared = oracle.expert_f64(experts[wl.E], wl.wdtype) if wl.n_shared else None
    xf = oracle.act_f64(x, wl.act_dtype)
    n, spent = 0, 0.0
    while spent < args.cpu_seconds and n < wl.steps:
        ids, _ = oracle.route(logits[n], k)
        for e in set(ids.ravel().tolist()):
            if e not in W64:
                W64[e] = oracle.expert_f64(experts[e], wl.wdtype)
        t0 = time.perf_counter()
        ids, gates = oracle.route(logits[n], k)
        oracle.moe_layer(xf[n * Bt:(n + 1) * Bt], ids, gates, W64, shared=shared)
        spent += time.perf_counter() - t0
        n += 1
    return {"value": round(Bt * n / spent, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {n} decode steps of the {wl.name} trace (batch {Bt}), fp64 numpy, "
                      f"weights decoded to fp64 before timing"}


if __name__ == "__main__":
    main()
