#!/usr/bin/env python3
"""MoE-layer throughput of the expert-cached layer on one MI355X.

One step = one pass of the layer's GPU path over one decode batch: router
softmax + top-k and permutation (moe_route), the SwiGLU experts of the step over
the expert slots (moe_expert_ffn, token lists from the host copy of the step's
ids, as the cached pipeline has them), and the gate-weighted un-permute and merge
(moe_merge_partial).  The K timed steps are captured once in a HIP graph and
replayed; inputs (logits, activations, expert slots) are resident in HBM before
the timed region.  The step's expert set comes from the library's own cache
planner (moe_lru_replay).  Expert slot pools are replicated R times and the steps
rotate over the replicas (R emulated layers), so each step's weights come from
HBM rather than from the 256 MB last-level cache.

Reported besides ``value``:
  roofline     decode FFN (moe_expert_ffn) bytes / time, timed with HIP events
               around the FFN of eager steps that each follow a 1 GiB fill (the
               fill hides the host enqueue time and evicts the last-level cache);
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
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--replicas", type=int, default=0, help="slot-pool replicas (0: enough to defeat the 256 MB cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pipeline", action="store_true")
    ap.add_argument("--pipeline-steps", type=int, default=400)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-reps", type=int, default=20)
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def payload_bytes(wl):
    """Algorithmic bytes of one expert's weights (codes + scales for MXFP4)."""
    n = 3 * wl.H * wl.I
    return {"f32": 4 * n, "bf16": 2 * n, "mxfp4": n // 2 + n // 32}[wl.wdtype]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = synth.workload(args.workload)
    if wl.wdtype == "mxfp4" or not wl.batches:
        raise SystemExit(f"decode bench needs a decode workload, got {wl.name}")
    Bt, K, W = args.batch, args.steps, args.warmup
    dt = {"f32": B.MOE_W_F32, "bf16": B.MOE_W_BF16, "mxfp4": B.MOE_W_MXFP4}[wl.wdtype]
    E, k, H, I = wl.E, wl.k, wl.H, wl.I
    n_trace = wl.steps

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    logits, _ = synth.zipf_reuse_trace(wl, Bt, n_trace)
    x = synth.activations(wl, n_trace * Bt, tag=11)
    experts = synth.expert_weights_many(wl, range(E + wl.n_shared), threads=16)
    log(f"inputs drawn in {time.time() - t0:.1f}s")

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
    step_experts, step_slots = [], []
    for p in plans:
        ex_ = np.concatenate([p.get("hit"), p.get("fill")]).astype(np.int32)
        sl_ = np.concatenate([p.get("hit_slot"), p.get("fill_slot")]).astype(np.int32)
        step_experts.append(ex_)
        step_slots.append(sl_)
    mean_distinct = float(np.mean([len(e) for e in step_experts]))

    # pool laid out by the planner's slots; replicas defeat the last-level cache
    nb = B.moe_expert_bytes(cfg_res)
    order = [int(np.where(slot_of == s)[0][0]) if (slot_of == s).any() else 0 for s in range(E)]
    host_pool = pack_pool(cfg_res, [experts[e] for e in order], pin=True)
    step_bytes = mean_distinct * payload_bytes(wl) + (payload_bytes(wl) if wl.n_shared else 0)
    R = args.replicas or max(1, math.ceil(4 * MALL_BYTES / step_bytes))
    R = min(R, max(1, int((48 << 30) // host_pool.numel())))
    pools = [host_pool.cuda() for _ in range(R)]
    shared = None
    if wl.n_shared:
        sh = pack_pool(cfg_res, [experts[E]], pin=False)
        shared = [sh.cuda() for _ in range(R)]
    d_x = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
    out = torch.empty(Bt * H, dtype=torch.int16 if wl.act_dtype == "bf16" else torch.float32, device="cuda")
    with_shared = 1 if wl.n_shared else 0
    torch.cuda.synchronize()
    log(f"pool {nb * E / 1e9:.2f} GB x {R} replicas, mean GPU experts/step {mean_distinct:.2f}")

    # ---------------------------------------------------------------- graph of the timed steps
    stream = torch.cuda.Stream()
    h_ids_steps = [np.ascontiguousarray(ids_all[t]) for t in range(n_trace)]

    def enqueue(s_idx, st, events=None):
        t = s_idx % n_trace
        r = s_idx % R
        L.route(d_logits[t * Bt:(t + 1) * Bt], Bt, st)
        if events is not None:
            events[0].record(st)
        L.ffn(d_x[t * Bt:(t + 1) * Bt], Bt, pools[r], step_experts[t], step_slots[t],
              shared[r] if shared else None, with_shared, st, h_ids=h_ids_steps[t])
        if events is not None:
            events[1].record(st)
        L.merge(step_experts[t], with_shared, None, Bt, out, st)

    with torch.cuda.stream(stream):
        for s in range(min(W, 64)):                     # eager warm-up (code objects, caches)
            enqueue(s, stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for s in range(K):
            enqueue(W + s, torch.cuda.current_stream())
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):                        # replay runs on the current stream
        g.replay()                                         # warm-up replay
        torch.cuda.synchronize()
        t_start.record(stream)
        g.replay()
        t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    value = Bt * K / (total_ms / 1e3)
    del g

    # ---------------------------------------------------------------- decode FFN roofline
    # Eager steps, each preceded by a 1 GiB fill on the same stream: the fill keeps the
    # GPU busy while the host enqueues route, event, FFN, event (so the events bracket
    # the FFN kernels only) and evicts the last-level cache like other layers would.
    n_prof = min(K, 400)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_prof)]
    with torch.cuda.stream(stream):
        for s in range(n_prof):
            flush.fill_(float(s))
            enqueue(W + s, stream, ev[s])
    torch.cuda.synchronize()
    ffn_ms = sum(a.elapsed_time(b) for a, b in ev) / n_prof
    ffn_bytes = 0.0
    for s in range(n_prof):
        t = (W + s) % n_trace
        ne = len(step_experts[t])
        pairs = Bt * k + (Bt if with_shared else 0)
        ffn_bytes += (ne + with_shared) * payload_bytes(wl) + Bt * H * (2 if wl.act_dtype == "bf16" else 4) + pairs * H * 4
    achieved = ffn_bytes / n_prof / (ffn_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "kernel": "moe_expert_ffn (k_decode_gate_up + k_decode_down)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "ffn_us": round(ffn_ms * 1e3, 2), "bytes_per_launch": round(ffn_bytes / n_prof),
                "launches_timed": n_prof}
    del flush
    log(f"GPU path: {ms_per_step * 1e3:.2f} us/step, {value:.0f} tok/s; FFN {ffn_ms * 1e3:.2f} us, "
        f"{achieved:.0f} GB/s")

    result = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
              "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": wl.wdtype, "data": "synthetic",
              "config": {"workload": f"{wl.name} decode, batch {Bt}", "hidden": H, "inter": I, "experts": E,
                         "top_k": k, "shared_experts": wl.n_shared, "batch": Bt, "replicas": R,
                         "gpu_experts_per_step": round(mean_distinct, 3), "step": "route+permute+ffn+merge, HIP graph"},
              "roofline": roofline}

    # ---------------------------------------------------------------- 8K prefill chunks (context)
    if not args.no_prefill:
        del pools
        torch.cuda.empty_cache()
        result["prefill"] = {name: prefill(args, name) for name in ("a3b_prefill8k_bf16", "v4flash_mxfp4")}

    # ---------------------------------------------------------------- full cached pipeline (context)
    if not args.no_pipeline:
        result["pipeline"] = pipeline(args, wl, experts, logits, x, dt)

    # ---------------------------------------------------------------- CPU baseline: the oracle
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, wl, experts, logits, x)
    B.moe_destroy(planner)
    print(json.dumps(result), flush=True)


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
    pool = pack_pool(cfg, [experts[e] for e in range(E)], pin=False).cuda()
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
    flops = 6.0 * T * k * H * I + (6.0 * T * H * I if wl.n_shared else 0.0)
    tflops = flops / (gms / 1e3) / 1e12
    nb = B.moe_expert_bytes(cfg)
    del g
    L.close()
    return {"tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_chunk": round(ms, 4), "tokens": T,
            "gemm_ms": round(gms, 4), "gemm_tflops": round(tflops, 1),
            "mfma_frac_bf16_peak": round(tflops / 2500.0, 4), "gflop": round(flops / 1e9, 1),
            "pool_gb": round(nb * E / 1e9, 3), "weights": wl.wdtype,
            "note": "layer pool resident in HBM; MXFP4 weights dequantised to bf16 MFMA inputs"}


def pipeline(args, wl, experts, logits, x, dt):
    """Cached decode: route on the GPU, plan on the host (global LRU + q*), upload the
    fills on a side stream while the hits run, CPU experts in parallel, merge."""
    import torch
    from expert_cached_moe_amd import binding as B
    from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool
    Bt, E, k, H = args.batch, wl.E, wl.k, wl.H
    cfg = B.make_config(wl.H, wl.I, E, k, wl.n_shared, wl.C, 1, dt, 1, 0, 52.7, 77.3)
    L = LayerBuffers(cfg, Bt)
    nb = B.moe_expert_bytes(cfg)
    host_pool = pack_pool(cfg, [experts[e] for e in range(E)], pin=True)
    slots = torch.empty(wl.C * nb, dtype=torch.uint8, device="cuda")
    shared = pack_pool(cfg, [experts[E]], pin=False).cuda() if wl.n_shared else None
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
            "slots": wl.C, "bp_bh": [52.7, 77.3], "miss_rate": round(st.misses / max(1, st.distinct), 4),
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
