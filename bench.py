#!/usr/bin/env python3
"""MoE-layer throughput of the expert-cached layer on one MI355X.

One step = one pass of the layer's GPU path over one decode batch: router
softmax + top-k and permutation (moe_route), then the SwiGLU experts of the step over
the expert slots with the gate-weighted un-permute and merge of their outputs
(moe_expert_ffn_merge, token lists from the host copy of the step's ids, as the
cached pipeline has them; bit-identical to moe_expert_ffn + moe_merge_partial, whose
step time is reported beside it).  The K timed steps are captured once in a HIP graph and
replayed; inputs (logits, activations, expert slots) are resident in HBM before
the timed region.  The step's expert set comes from the library's own cache
planner (moe_lru_replay).  Expert slot pools are replicated R times and the steps
rotate over the replicas (R emulated layers), so each step's weights come from
HBM rather than from the 256 MB last-level cache.

Reported besides ``value``:
  roofline     decode expert FFN (moe_expert_ffn: the HBM-streaming kernels) algorithmic
               bytes / time per call, timed with HIP events around a graph of those calls alone
               that rotate over
               the pool replicas; ``traffic`` is the counter-measured HBM bytes per
               call while the decode kernels are unchanged since the counters;
               ``warm_r1`` is the same graph on one replica (weights partly served by
               the last-level cache), reported apart; ``step_call`` times the call the
               step makes (moe_expert_ffn_merge: the same gate/up kernel, then down and
               merge fused) the same way;
  batches      the same step at the other decode batch sizes of the workload;
  decode_other the same step and FFN roofline on the other decode shapes (hidden 4096,
               256 experts + 1 shared, top-6; bf16 and MXFP4 weights);
  cpu_baseline the fp64 oracle timed on the host cores on a bounded sample;
  pipeline     the full cached decode step (GPU route -> host plan with q* ->
               PCIe fills on a side stream + CPU experts -> GPU experts -> merge),
               which includes host-link transfers and is context, not ``value``.
"""
from __future__ import annotations

import argparse
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
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="a3b_decode_bf16")
    ap.add_argument("--batch", type=int, default=1, help="decode batch of `value`")
    ap.add_argument("--extra-batches", default="4,8", help="further decode batches reported beside `value` ('' for none)")
    ap.add_argument("--other-decode", default="v4flash_decode_bf16:1,8;v4flash_mxfp4:1,8",
                    help="further decode workloads with their batches, reported beside `value` ('' for none)")
    ap.add_argument("--replicas", type=int, default=0, help="slot-pool replicas (0: enough to defeat the 256 MB cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pipeline", action="store_true")
    ap.add_argument("--pipeline-steps", type=int, default=400)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--stream-layers", type=int, default=4,
                    help="emulated layers of the streamed prefill chunk (0: skip streaming)")
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
# --pmc WRITE_SIZE, over `bench.py --steps 50 --warmup 5 --no-cpu-baseline --no-pipeline
# --prefill-reps 3 --stream-layers 0 --copy-probe`), in KiB per dispatch as the counters read
# them, averaged over the 100 calls of the rotating FFN graph and summed over k_decode_gate_up
# and k_decode_down of one moe_expert_ffn call at batch 1 (every call has the same expert
# count, so the record matches the timed calls).  The same runs read the plain 256 MiB read +
# 256 MiB write kernel of --copy-probe as FETCH_SIZE 131080 KiB and WRITE_SIZE 262144 KiB, so
# fetch counts are scaled by 262144 / 131080 and write counts by 1.  A record applies only
# while the decode kernel sources hash to the value it was taken with.
DECODE_SOURCES = ("ffn_decode.hip", "ffn_common.h", "device_common.h")
_SRC = "c31eea7f69972adaa28a1454f7bed36214747ab19e32da27628381b4c0d8c7b5"
TRAFFIC = {
    ("a3b_decode_bf16", 1): {"sha256": _SRC, "fetch_kib": 24613.0 + 12361.0, "write_kib": 48.0 + 32.0},
    ("v4flash_decode_bf16", 1): {"sha256": _SRC, "fetch_kib": 86072.0 + 43113.0, "write_kib": 84.0 + 56.0},
    ("v4flash_mxfp4", 1): {"sha256": _SRC, "fetch_kib": 22922.5 + 11552.0, "write_kib": 42.0 + 56.0},
}
FETCH_FACTOR = 262144.0 / 131080.0
WRITE_FACTOR = 1.0


class _phase:
    """A named range around a bench phase (roctx through torch's marker API when the build
    has it), so that a kernel trace taken with rocprofv3 --marker-trace can be split by phase."""

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
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "expert_cached_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
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
    wl = synth.workload(args.workload)
    if wl.wdtype == "mxfp4" or not wl.batches:
        raise SystemExit(f"decode bench needs a decode workload, got {wl.name}")
    t0 = time.time()
    experts = synth.expert_weights_many(wl, range(wl.E + wl.n_shared), threads=16)
    log(f"expert weights drawn in {time.time() - t0:.1f}s")

    with _phase(f"decode batch {args.batch}"):
        d = decode(args, wl, args.batch, experts)
    Bt = args.batch
    result = {"metric": METRIC, "value": d["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": d["ms_per_step"], "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": wl.wdtype, "data": "synthetic",
              "config": {"workload": f"{wl.name} decode, batch {Bt}", "hidden": wl.H, "inter": wl.I,
                         "experts": wl.E, "top_k": wl.k, "shared_experts": wl.n_shared, "batch": Bt,
                         "replicas": d["replicas"], "gpu_experts_per_step": d["gpu_experts_per_step"],
                         "step": "route+permute, then ffn+merge in one call; HIP graph"},
              "roofline": d["roofline"]}
    extra = [int(b) for b in args.extra_batches.split(",") if b.strip()] if args.extra_batches else []
    if extra:
        result["batches"] = {}
        for b in extra:
            with _phase(f"decode batch {b}"):
                e = decode(args, wl, b, experts)
            result["batches"][str(b)] = {k_: e[k_] for k_ in ("tokens_per_s", "ms_per_step", "two_calls_ms_per_step",
                                                               "gpu_experts_per_step", "replicas")} | \
                {"roofline": e["roofline"]}

    # ---------------------------------------------------------------- other decode shapes (context)
    if args.other_decode:
        result["decode_other"] = {}
        for item in args.other_decode.split(";"):
            name, _, bs = item.partition(":")
            wl2 = synth.workload(name.strip())
            ex2 = synth.expert_weights_many(wl2, range(wl2.E + wl2.n_shared), threads=16)
            res = {"hidden": wl2.H, "inter": wl2.I, "experts": wl2.E, "top_k": wl2.k,
                   "shared_experts": wl2.n_shared, "dtype": wl2.wdtype, "batches": {}}
            for b in [int(v) for v in bs.split(",") if v.strip()]:
                with _phase(f"decode {wl2.name} batch {b}"):
                    e = decode(args, wl2, b, ex2)
                res["batches"][str(b)] = {k_: e[k_] for k_ in ("tokens_per_s", "ms_per_step", "two_calls_ms_per_step",
                                                                "gpu_experts_per_step", "replicas")} | \
                    {"roofline": e["roofline"]}
            result["decode_other"][wl2.name] = res
            del ex2

    # ---------------------------------------------------------------- 8K prefill chunks (context)
    if not args.no_prefill:
        torch.cuda.empty_cache()
        result["prefill"] = {}
        for name in ("a3b_prefill8k_bf16", "v4flash_mxfp4"):
            with _phase(f"prefill {name}"):
                result["prefill"][name] = prefill(args, name)

    # ---------------------------------------------------------------- full cached pipeline (context)
    logits, x = d["logits"], d["x"]
    dt = d["w_dtype"]
    if not args.no_pipeline:
        with _phase("cached decode pipeline"):
            result["pipeline"] = pipeline(args, wl, experts, logits, x, dt)

    # ---------------------------------------------------------------- CPU baseline: the oracle
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, wl, experts, logits, x)
    print(json.dumps(result), flush=True)


def decode(args, wl, Bt, experts):
    """Decode steps at batch Bt: planner replay, pools, the graph of K timed steps, and the
    FFN roofline (a graph of FFN calls alone, rotating over the pool replicas)."""
    import torch
    import synth
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool
    K, W = args.steps, args.warmup
    dt = {"f32": B.MOE_W_F32, "bf16": B.MOE_W_BF16, "mxfp4": B.MOE_W_MXFP4}[wl.wdtype]
    E, k, H, I = wl.E, wl.k, wl.H, wl.I
    n_trace = wl.steps

    # ---------------------------------------------------------------- inputs
    logits, _ = synth.zipf_reuse_trace(wl, Bt, n_trace)
    x = synth.activations(wl, n_trace * Bt, tag=11)

    # all-resident plan from the library's planner: C = E slots, every miss filled
    cfg_res = B.make_config(H, I, E, k, wl.n_shared, E, 1, dt, 1, 0, 1.0, 1.0)
    planner = B.moe_create(cfg_res)
    cap = min(E, Bt * k)
    # routing of every trace step on the GPU, copied back once for the planner
    L = LayerBuffers(cfg_res, Bt)
    d_logits = torch.from_numpy(logits.reshape(n_trace * Bt, E)).cuda()
    ids_all = np.empty((n_trace, Bt, k), np.int32)
    for s in range(n_trace):
        L.route(d_logits[s * Bt:(s + 1) * Bt], Bt)
        ids_all[s] = L.ids[: Bt * k].view(Bt, k).cpu().numpy()
    plans = [B.Plan(cap, E) for _ in range(n_trace)]
    B.moe_lru_replay(planner, 0, ids_all, n_trace, Bt, plans)
    slot_of = B.moe_lru_slots(planner, 0, E)
    B.moe_destroy(planner)
    step_experts, step_slots = [], []
    for p in plans:
        step_experts.append(np.concatenate([p.get("hit"), p.get("fill")]).astype(np.int32))
        step_slots.append(np.concatenate([p.get("hit_slot"), p.get("fill_slot")]).astype(np.int32))
    mean_distinct = float(np.mean([len(e) for e in step_experts]))

    # pool laid out by the planner's slots; replicas defeat the last-level cache
    order = [int(np.where(slot_of == s)[0][0]) if (slot_of == s).any() else 0 for s in range(E)]
    host_pool = pack_pool(cfg_res, [experts[e] for e in order], pin=True)
    step_bytes = mean_distinct * payload_bytes(wl) + (payload_bytes(wl) if wl.n_shared else 0)
    R = args.replicas or max(1, math.ceil(4 * MALL_BYTES / step_bytes))
    R = min(R, max(1, int((48 << 30) // host_pool.numel())))
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
    log(f"batch {Bt}: pool {B.moe_expert_bytes(cfg_res) * E / 1e9:.2f} GB x {R} replicas, "
        f"mean GPU experts/step {mean_distinct:.2f}")

    # ---------------------------------------------------------------- graph of the timed steps
    stream = torch.cuda.Stream()
    h_ids_steps = [np.ascontiguousarray(ids_all[t]) for t in range(n_trace)]

    def ffn_merge(s_idx, rotate=True):
        """The step's experts and the merge of their outputs (moe_expert_ffn_merge)."""
        t, r = s_idx % n_trace, (s_idx % R if rotate else 0)
        L.ffn_merge(d_x[t * Bt:(t + 1) * Bt], Bt, pools[r], step_experts[t], step_slots[t], h_ids_steps[t],
                    shared[r] if shared else None, with_shared, None, out, torch.cuda.current_stream())

    def ffn(s_idx, rotate=True):
        """The step's experts alone (moe_expert_ffn: the pair outputs)."""
        t, r = s_idx % n_trace, (s_idx % R if rotate else 0)
        L.ffn(d_x[t * Bt:(t + 1) * Bt], Bt, pools[r], step_experts[t], step_slots[t],
              shared[r] if shared else None, with_shared, torch.cuda.current_stream(), h_ids=h_ids_steps[t])

    def enqueue(s_idx):
        t = s_idx % n_trace
        L.route(d_logits[t * Bt:(t + 1) * Bt], Bt, torch.cuda.current_stream())
        ffn_merge(s_idx)

    def enqueue_two_calls(s_idx):
        """The same step through moe_expert_ffn (pair outputs) and moe_merge_partial."""
        t, r = s_idx % n_trace, s_idx % R
        st = torch.cuda.current_stream()
        L.route(d_logits[t * Bt:(t + 1) * Bt], Bt, st)
        L.ffn(d_x[t * Bt:(t + 1) * Bt], Bt, pools[r], step_experts[t], step_slots[t],
              shared[r] if shared else None, with_shared, st, h_ids=h_ids_steps[t])
        L.merge(step_experts[t], with_shared, None, Bt, out, st)

    def timed_graph(body, n):
        """Capture body(W + s) for s < n, replay once to warm up, then time one replay with
        HIP events recorded on the replay stream; returns milliseconds per iteration."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s in range(n):
                body(W + s)
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):                    # replay runs on the current stream
            g.replay()
            torch.cuda.synchronize()
            t_start.record(stream)
            g.replay()
            t_end.record(stream)
        torch.cuda.synchronize()
        del g
        return t_start.elapsed_time(t_end) / n

    with torch.cuda.stream(stream):
        for s in range(min(W, 64)):                        # eager warm-up (code objects, caches)
            enqueue(s)
    torch.cuda.synchronize()
    ms_per_step = timed_graph(enqueue, K)
    value = Bt / (ms_per_step / 1e3)

    # ---------------------------------------------------------------- decode FFN roofline
    two_calls_ms = timed_graph(enqueue_two_calls, K)

    # The expert FFN calls (moe_expert_ffn: the HBM-streaming kernels) of n_prof consecutive
    # steps alone in one graph: each call reads its experts from the next pool replica, so the
    # weights come from HBM, and the per-call time is the two kernels' durations back to back.
    # The step itself runs the same gate/up kernel, then down and merge fused (timed apart).
    n_prof = min(K, 1000)
    ffn_ms = timed_graph(ffn, n_prof)
    # warm: every call reads replica 0, so weights the last-level cache still holds are reused
    warm_ms = timed_graph(lambda s_idx: ffn(s_idx, rotate=False), n_prof)
    fused_ms = timed_graph(ffn_merge, n_prof)
    pairs = Bt * k + (Bt if with_shared else 0)
    act = 2 if wl.act_dtype == "bf16" else 4
    w_bytes = 0.0
    for s in range(n_prof):
        w_bytes += (len(step_experts[(W + s) % n_trace]) + with_shared) * payload_bytes(wl)
    w_bytes /= n_prof
    ffn_bytes = w_bytes + Bt * H * act + pairs * H * act              # weights, x, pair outputs
    fused_bytes = w_bytes + Bt * H * act + Bt * H * act + pairs * 8   # weights, x, layer output, gates
    achieved = ffn_bytes / (ffn_ms / 1e3) / 1e9
    rec = TRAFFIC.get((wl.name, Bt))
    traffic = None
    if rec is not None and rec["sha256"] == decode_sources_sha256():
        traffic = round((rec["fetch_kib"] * FETCH_FACTOR + rec["write_kib"] * WRITE_FACTOR) * 1024)
    roofline = {"bound": "hbm", "kernel": "moe_expert_ffn, decode (k_decode_gate_up + k_decode_down)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "ffn_us": round(ffn_ms * 1e3, 3), "bytes_per_launch": round(ffn_bytes), "launches_timed": n_prof,
                "warm_r1": {"ffn_us": round(warm_ms * 1e3, 3),
                            "achieved": round(ffn_bytes / (warm_ms / 1e3) / 1e9, 1)},
                "step_call": {"call": "moe_expert_ffn_merge (k_decode_gate_up + k_decode_down_merge when the "
                                      "list has at most 8 entries, else + k_decode_down + k_merge)",
                              "us": round(fused_ms * 1e3, 3), "bytes_per_launch": round(fused_bytes),
                              "achieved": round(fused_bytes / (fused_ms / 1e3) / 1e9, 1)}}
    log(f"batch {Bt}: {ms_per_step * 1e3:.2f} us/step, {value:.0f} tok/s; FFN {ffn_ms * 1e3:.2f} us, "
        f"{achieved:.0f} GB/s")
    L.close()
    del pools, shared, d_logits, d_x
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(value, 1), "ms_per_step": round(ms_per_step, 5), "replicas": R,
            "two_calls_ms_per_step": round(two_calls_ms, 5),
            "gpu_experts_per_step": round(mean_distinct, 3), "roofline": roofline,
            "logits": logits, "x": x, "w_dtype": dt}


def prefill(args, name):
    """One 8192-token chunk through route + grouped GEMMs + merge with the layer's pool
    resident in HBM, captured in a graph and replayed; MFMA roofline of the two GEMMs."""
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
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

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
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        ev[2].record(stream)
        g.replay()
        ev[3].record(stream)
    torch.cuda.synchronize()
    ms = ev[2].elapsed_time(ev[3]) / args.prefill_reps
    # FFN alone (events around the grouped GEMMs of eager chunks)
    gemm_ms = []
    with torch.cuda.stream(stream):
        for _ in range(5):
            step(events=True)
            torch.cuda.synchronize()
            gemm_ms.append(ev[0].elapsed_time(ev[1]))
    gms = float(np.median(gemm_ms))
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
    del g
    res = {"tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_chunk": round(ms, 4), "tokens": T,
           "gemm_ms": round(gms, 4), "gemm_tflops": round(tflops, 1),
           "router_logits_ms": round(float(np.median(rl_ms)), 4),
           "mfma_frac_bf16_peak": round(tflops / 2500.0, 4), "gflop": round(flops / 1e9, 1),
           "pool_gb": round(nb * E / 1e9, 3), "weights": wl.wdtype,
           "note": "layer pool resident in HBM; MXFP4 weights dequantised to bf16 MFMA inputs"}
    del pool
    if args.stream_layers > 0:
        res["streamed"] = stream_chunk(args, wl, cfg, host_pool, shared, d_logits, d_x, L, ms)
    L.close()
    return res


def stream_chunk(args, wl, cfg, host_pool, shared, d_logits, d_x, L, compute_ms):
    """The chunk through n emulated layers whose pools upload from pinned host memory
    (moe_prefill_stream), with two layer buffers and with one (the single-buffer
    ablation), against the overlap model built from the measured upload and compute."""
    import torch
    from expert_cached_moe_amd import binding as B
    n, T, E = args.stream_layers, wl.T, wl.E
    nb = B.moe_expert_bytes(cfg)
    layer_bytes = nb * E
    scfg = B.make_config(wl.H, wl.I, E, wl.k, wl.n_shared, 0, n, cfg.w_dtype)
    ctx = B.moe_create(scfg)
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
    pred2 = up_ms + (n - 1) * max(up_ms, compute_ms) + compute_ms
    pred1 = n * (up_ms + compute_ms)
    return {"layers": n, "layer_gb": round(layer_bytes / 1e9, 3), "bp_gbps": round(layer_bytes / (up_ms / 1e3) / 1e9, 2),
            "layer_upload_ms": round(up_ms, 3), "layer_compute_ms": round(compute_ms, 4),
            "double_ms": round(double_ms, 3), "single_ms": round(single_ms, 3),
            "double_pred_ms": round(pred2, 3), "single_pred_ms": round(pred1, 3),
            "chunk_tokens_per_s_double": round(T / (double_ms / 1e3), 1),
            "single_buffer_penalty": round(1.0 - double_ms / single_ms, 4),
            "note": "PCIe-inclusive; prediction: double = U + (n-1) max(U, C) + C, single = n (U + C)"}


def measure_bandwidths(B, ctx, host_pool, slots, nb, wl, side, n_exp=16):
    """The pages' two rates on this machine: B_P, pinned host -> device copies of single
    expert blobs (as fills are issued), and B_H, the rate at which the CPU experts
    (moe_host_ffn) stream expert weights from the pinned pool, at 6 threads (the pages'
    setting) and at all threads."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_exp = min(n_exp, wl.E, wl.C)

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
    k = wl.k
    T = (n_exp + k - 1) // k
    ids = np.array([[(t * k + j) % n_exp if t * k + j < n_exp else (t * k + j) % wl.E for j in range(k)]
                    for t in range(T)], np.int32)
    host = sorted(set(ids.ravel().tolist()))
    plan = B.Plan(len(host), wl.E)
    plan.arrays["host"][: len(host)] = host
    plan.c.n_host = len(host)
    plan.c.layer = 0
    h_x = torch.zeros(T * wl.H, dtype=torch.int16 if wl.act_dtype == "bf16" else torch.float32)
    h_w = np.full((T, k), 1.0 / k, np.float32)
    h_y = torch.zeros(T * wl.H, dtype=torch.float32)
    out = {}
    for label, nt in (("bh_gbps_6_threads", 6), ("bh_gbps_all_threads", os.cpu_count() or 1)):
        ts = []
        for _ in range(5):
            t0 = time.perf_counter()
            B.moe_host_ffn(ctx, h_x, T, ids, h_w, plan, h_y, nt)
            ts.append(time.perf_counter() - t0)
        out[label] = round(len(host) * payload_bytes(wl) / float(np.median(ts)) / 1e9, 2)
    nt = min(16, os.cpu_count() or 1)
    ts = []
    for _ in range(5):
        t0 = time.perf_counter()
        B.moe_host_ffn(ctx, h_x, T, ids, h_w, plan, h_y, nt)
        ts.append(time.perf_counter() - t0)
    out["bh_gbps_pipeline_threads"] = round(len(host) * payload_bytes(wl) / float(np.median(ts)) / 1e9, 2)
    out = {"bp_gbps": round(bp, 2), "bp_gbps_one_copy": round(bp_batched, 2), **out,
           "threads_all": os.cpu_count() or 1, "threads_pipeline": nt}
    bh = out["bh_gbps_pipeline_threads"]
    out["qstar_at_measured_ratio"] = {m: B.moe_qstar(m, bp, bh, 0) for m in range(1, 9)}
    return out


def pipeline(args, wl, experts, logits, x, dt):
    """Cached decode: route on the GPU, plan on the host (global LRU + q*), upload the
    fills on a side stream while the hits run, CPU experts in parallel, merge.  Run at the
    pages' B_P:B_H and at the ratio measured on this machine (per-blob fills, and the CPU
    experts at the pipeline's own thread count)."""
    import torch
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import pack_pool
    E = wl.E
    cfg0 = B.make_config(wl.H, wl.I, E, wl.k, wl.n_shared, wl.C, 1, dt, 1, 0, 52.7, 77.3)
    nb = B.moe_expert_bytes(cfg0)
    host_pool = pack_pool(cfg0, [experts[e] for e in range(E)], pin=True)
    slots = torch.empty(wl.C * nb, dtype=torch.uint8, device="cuda")
    shared = pack_pool(cfg0, [experts[E]], pin=False).cuda() if wl.n_shared else None
    ctx0 = B.moe_create(cfg0)
    B.moe_bind_pools(ctx0, slots, wl.C, host_pool, E)
    bw = measure_bandwidths(B, ctx0, host_pool, slots, nb, wl, torch.cuda.Stream())
    B.moe_destroy(ctx0)
    res = run_pipeline(args, wl, logits, x, dt, host_pool, slots, shared, 52.7, 77.3)
    res["measured"] = bw
    res["at_measured_ratio"] = run_pipeline(args, wl, logits, x, dt, host_pool, slots, shared, bw["bp_gbps"],
                                            bw["bh_gbps_pipeline_threads"])
    return res


def run_pipeline(args, wl, logits, x, dt, host_pool, slots, shared, bp, bh):
    import torch
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import LayerBuffers
    Bt, E, k, H = args.batch, wl.E, wl.k, wl.H
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

    def step(s):
        t = s % n_trace
        L.route(d_logits[t * Bt:(t + 1) * Bt], Bt, main_s)
        h_ids.copy_(L.ids[: Bt * k], non_blocking=True)
        h_w.copy_(L.w[: Bt * k], non_blocking=True)
        h_x.copy_(d_x[t * Bt:(t + 1) * Bt].view(-1), non_blocking=True)
        main_s.synchronize()
        B.moe_lru_step(L.ctx, 0, h_ids.numpy().reshape(Bt, k), Bt, plan)
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
        step(s)
    torch.cuda.synchronize()
    dt_s = time.perf_counter() - t0
    st = B.moe_lru_stats(L.ctx)
    L.close()
    return {"tokens_per_s": round(Bt * n / dt_s, 1), "steps": n, "ms_per_step": round(dt_s * 1e3 / n, 4),
            "slots": wl.C, "bp_bh": [bp, bh], "miss_rate": round(st.misses / max(1, st.distinct), 4),
            "fills_per_step": round(st.fills / n, 3), "host_experts_per_step": round(st.host / n, 3),
            "cold_start": True, "note": "includes host-link fills and CPU experts; context only"}


def cpu_baseline(args, wl, experts, logits, x):
    """The fp64 oracle on the host cores: route + layer for as many steps as fit in
    about --cpu-seconds; weights pre-decoded to fp64 (resident, like the GPU's)."""
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
            "sample": f"first {n} decode steps of the same trace (batch {Bt}), fp64 numpy, weights pre-decoded"}


if __name__ == "__main__":
    main()
