"""GPU parity of the two pipelines around the layer kernels, through the C ABI.

Cached decode: the GPU router, the host cache planner (global LRU + q*), the fills
of the planned misses into the slot pool over PCIe on a side stream, the GPU
experts over hits and fills, the CPU experts of the host set and the exact merge.
Every step's output is checked against the oracle's unpartitioned layer, and every
plan bit for bit against the oracle's cache.  Slots start poisoned and the host
pool holds real weights only for the experts the trace uses (0xFF = NaN elsewhere),
so a read of a slot before its fill, or of the wrong expert, fails the step.

Prefill streaming: a chunk through several layers whose pools upload from pinned
host memory into two (or one) device layer buffers; every layer must be bit-identical
to the same layer computed with its pool resident, and match the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import Experts, TOL, config, dev_act, out_f64, rel_err_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from expert_cached_moe_amd import binding
    return binding


def _act_tensor(wl, n):
    return torch.empty(n, dtype=torch.float32 if wl.act_dtype == "f32" else torch.int16, device="cuda")


# ---------------------------------------------------------------- cached decode
def _decode_inputs(wl, Bt, n_steps, layer=0):
    if wl.name == "tiny_fp32":
        # the tiny layer routes with its own router: logits = x . W_r, one token per step
        x = synth.activations(wl, n_steps * Bt, tag=21)
        logits = oracle.router_logits(x, synth.router_weights(wl)).astype(np.float32)
        return logits.reshape(n_steps, Bt, wl.E), x
    logits, _ = synth.zipf_reuse_trace(wl, Bt, n_steps, tag=0 if layer == 0 else 100 + layer)
    return logits, synth.activations(wl, n_steps * Bt, tag=11)


@pytest.mark.parametrize("name,Bt,n_steps", [("tiny_fp32", 1, 64), ("a3b_decode_bf16", 4, 24),
                                             ("a3b_decode_bf16", 1, 32), ("v4flash_decode_bf16", 1, 6),
                                             ("v4flash_mxfp4", 2, 6)])
def test_cached_decode_pipeline(B, name, Bt, n_steps):
    _run_pipeline(B, name, Bt, n_steps)


def test_cached_decode_pipeline_resize(B):
    """Elastic slot pool under the pipeline ([B] "Elastic Memory"): shrink 47 -> 20 slots
    before step 8 (moves copied inside the device pool, freed slots poisoned, pool rebound
    smaller), grow back to 47 before step 16 (the new slots are poisoned until filled)."""
    _run_pipeline(B, "a3b_decode_bf16", 4, 24, resizes={8: 20, 16: 47})


@pytest.mark.parametrize("name,n_layers,Bt,n_steps", [("a3b_decode_bf16", 4, 1, 10), ("v4flash_mxfp4", 4, 2, 4)])
def test_cached_decode_pipeline_layer_stack(B, name, n_layers, Bt, n_steps):
    """One cache over a stack of MoE layers ([A] "Abandoning fixed offloading ...": a single
    LRU spans the experts of all layers): the slot pool holds the workload's fraction of the
    whole pool (37 % or 11 % of n_layers * E blobs), the host pool every (layer, expert) blob
    in key order, each layer has its own weights and routing trace, and every decode step
    runs layer 0 .. n_layers-1 through the pipeline with plans keyed (layer, expert)."""
    _run_pipeline(B, name, Bt, n_steps, n_layers=n_layers)


def _run_pipeline(B, name, Bt, n_steps, resizes=None, n_layers=1):
    from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool
    print(f"[pipeline] {name} B={Bt} steps={n_steps} layers={n_layers} resizes={resizes}", flush=True)
    wl = synth.workload(name)
    E, k, H, NL = wl.E, wl.k, wl.H, n_layers
    C = wl.C if NL == 1 else int(round(wl.C / E * NL * E))
    inputs = [_decode_inputs(wl, Bt, n_steps, layer=l) for l in range(NL)]
    logits = [inp[0] for inp in inputs]
    x = inputs[0][1]                                   # every layer takes the same x
    routes = [[oracle.route(logits[l][s], k) for s in range(n_steps)] for l in range(NL)]
    exs = []
    for l in range(NL):
        used = sorted({int(e) for s in range(n_steps) for e in routes[l][s][0].ravel()})
        ex = Experts(wl, layer=l)
        ex.prefetch(used + ([E] if wl.n_shared else []), threads=16)
        exs.append((ex, set(used)))
    cfg = config(wl, n_slots=C, n_layers=NL)
    nb = B.moe_expert_bytes(cfg)
    host_pool = pack_pool(cfg, [ex.raw(e) if e in used else None for ex, used in exs for e in range(E)], pin=True)
    slots = torch.full((C * nb,), 0xFF, dtype=torch.uint8, device="cuda")
    shared = [pack_pool(cfg, [ex.raw(E)], pin=False).cuda() for ex, _ in exs] if wl.n_shared else None
    ws = 1 if wl.n_shared else 0
    L = LayerBuffers(cfg, Bt)
    B.moe_bind_pools(L.ctx, slots, C, host_pool, NL * E)
    d_logits = [torch.from_numpy(np.ascontiguousarray(lg.reshape(n_steps * Bt, E), np.float32)).cuda()
                for lg in logits]
    d_x = dev_act(x)
    h_x = torch.empty(Bt * H, dtype=d_x.dtype, pin_memory=True)
    h_y = torch.zeros(Bt * H, dtype=torch.float32, pin_memory=True)
    d_y = torch.empty(Bt * H, dtype=torch.float32, device="cuda")
    out = _act_tensor(wl, Bt * H)
    plan = B.Plan(min(E, Bt * k), E)
    ref_cache = oracle.LRUCache(C, E, n_layers=NL)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    xf = oracle.act_f64(x, wl.act_dtype)
    worst, n_host, n_fill = 0.0, 0, 0
    for s in range(n_steps):
        if resizes and s in resizes:
            newC = resizes[s]
            r = B.Resize(256)
            B.moe_lru_resize(L.ctx, newC, r)
            want_r = ref_cache.resize(newC)
            assert r.moves() == want_r["moves"] and r.evicted() == want_r["evicted"], s
            B.moe_move_slots(L.ctx, r, main)
            if newC < C:
                slots[newC * nb:C * nb].fill_(0xFF)          # freed slots: any later read shows up as NaN
            B.moe_bind_pools(L.ctx, slots, newC, host_pool, NL * E)
            C = newC
        for l in range(NL):
            ex = exs[l][0]
            L.route(d_logits[l][s * Bt:(s + 1) * Bt], Bt, main)
            ids = L.ids[: Bt * k].cpu().numpy().reshape(Bt, k)          # synchronises the route
            gates = L.w[: Bt * k].cpu().numpy().reshape(Bt, k)
            rids, rgates = routes[l][s]
            assert np.array_equal(ids, rids), f"step {s} layer {l}: routing"
            assert np.abs(gates - rgates).max() <= 1e-6 * np.abs(rgates).max(), f"step {s} layer {l}: gates"
            B.moe_lru_step(L.ctx, l, ids, Bt, plan)
            want = ref_cache.step(rids, 52.7, 77.3, layer=l)
            for f in ("hit", "hit_slot", "fill", "fill_slot", "fill_victim", "host"):
                assert plan.get(f).tolist() == list(want[f]), f"step {s} layer {l}: plan field {f}"
            B.moe_fill(L.ctx, plan, side)
            hits, hsl = plan.get("hit").copy(), plan.get("hit_slot").copy()
            fills, fsl = plan.get("fill").copy(), plan.get("fill_slot").copy()
            sh = shared[l] if ws else None
            L.ffn(d_x[s * Bt:(s + 1) * Bt], Bt, slots, hits, hsl, sh, ws, main, h_ids=ids)
            B.moe_fill_wait(L.ctx, main)
            L.ffn(d_x[s * Bt:(s + 1) * Bt], Bt, slots, fills, fsl, None, 0, main, h_ids=ids)
            host = plan.c.n_host > 0
            if host:
                h_x.copy_(d_x[s * Bt:(s + 1) * Bt].reshape(-1))
                B.moe_host_ffn(L.ctx, h_x, Bt, ids, np.ascontiguousarray(gates), plan, h_y, 8)
                d_y.copy_(h_y)
            gpu = np.concatenate([hits, fills]).astype(np.int32)
            L.merge(gpu, ws, d_y if host else None, Bt, out, main)
            y = out_f64(out, wl, Bt)
            ref = oracle.moe_layer(xf[s * Bt:(s + 1) * Bt], rids, rgates, ex, shared=ex.f64(E) if ws else None)
            err = rel_err_rows(y, ref).max()
            assert np.isfinite(y).all() and err <= TOL[wl.wdtype], f"step {s} layer {l}: rel err {err}"
            worst = max(worst, err)
            n_host += len(want["host"])
            n_fill += len(want["fill"])
    print(f"[pipeline] {name}: worst rel err {worst:.2e}, fills {n_fill}, host experts {n_host}", flush=True)
    for l in range(NL):
        assert np.array_equal(B.moe_lru_slots(L.ctx, l, E), ref_cache.slot_table(l))
    assert n_fill > 0
    L.close()


# ---------------------------------------------------------------- prefill layer streaming
def _stream_workload(case):
    base = {"f32_gemv": "tiny_fp32", "bf16_gemm": "tiny_fp32", "mxfp4_shared": "tiny_fp32",
            "a3b_layer": "a3b_prefill8k_bf16"}[case]
    wl = synth.workload(base)
    if case == "bf16_gemm":
        wl = dataclasses.replace(wl, name="tiny_bf16_e16", wdtype="bf16", E=16, k=4)
    elif case == "mxfp4_shared":
        wl = dataclasses.replace(wl, name="tiny_mxfp4_e16_shared", wdtype="mxfp4", E=16, k=4, n_shared=1)
    return wl


@pytest.mark.parametrize("case,T,n_layers", [("f32_gemv", 16, 3), ("bf16_gemm", 64, 3), ("mxfp4_shared", 48, 2),
                                             ("a3b_layer", 40, 2), ("a3b_layer", 8192, 2)])
def test_prefill_stream(B, case, T, n_layers):
    """A chunk streamed through n_layers layers (double- and single-buffered) is bit-identical
    to each layer run with its pool resident, and matches the oracle on sampled tokens.  The
    8192-token case streams two full a3b layer pools (1.2 GB each) through the same path the
    bench times."""
    from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool
    print(f"[stream] {case} T={T} layers={n_layers}", flush=True)
    wl = _stream_workload(case)
    E, H, Lk = wl.E, wl.H, n_layers
    cfg = config(wl, n_slots=0, n_layers=Lk)
    nb = B.moe_expert_bytes(cfg)
    n_all = E + wl.n_shared
    exs = [synth.expert_weights_many(wl, range(n_all), threads=16, layer=l) for l in range(Lk)]
    host_pool = pack_pool(cfg, [exs[l][e] for l in range(Lk) for e in range(E)], pin=True)
    shared = pack_pool(cfg, [exs[l][E] for l in range(Lk)], pin=False).cuda() if wl.n_shared else None
    ws = 1 if wl.n_shared else 0
    logits = np.stack([synth.iid_logits(wl, T, tag=100 + l) for l in range(Lk)])
    x = synth.activations(wl, T, tag=5)
    Lb = LayerBuffers(cfg, T)
    B.moe_bind_pools(Lb.ctx, None, 0, host_pool, Lk * E)
    d_logits = torch.from_numpy(logits).cuda()
    d_x = dev_act(x)
    bufs = torch.empty(2 * E * nb, dtype=torch.uint8, device="cuda")
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    outs = {}
    for n_buf in (2, 1):
        bufs.fill_(0xFF)
        o = _act_tensor(wl, Lk * T * H)
        o.fill_(0)
        B.moe_prefill_stream(Lb.ctx, bufs, n_buf, d_logits, d_x, T, shared, Lb.ids, Lb.w, Lb.counts, Lb.offsets,
                             Lb.perm, Lb.inv, Lb.o, Lb.ws, o, main, side)
        torch.cuda.synchronize()
        outs[n_buf] = o
    assert torch.equal(outs[1], outs[2]), "single- and double-buffered chunks differ"

    allx = np.arange(E, dtype=np.int32)
    res = _act_tensor(wl, T * H)
    xf = oracle.act_f64(x, wl.act_dtype)
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(T, 6), replace=False)]))
    for l in range(Lk):
        pool_l = host_pool[l * E * nb:(l + 1) * E * nb].cuda()
        sh_l = shared[l * nb:(l + 1) * nb] if ws else None
        Lb.route(d_logits[l], T, main)
        Lb.ffn(d_x, T, pool_l, allx, allx, sh_l, ws, main)
        Lb.merge(allx, ws, None, T, res, main)
        torch.cuda.synchronize()
        got = outs[2][l * T * H:(l + 1) * T * H]
        assert torch.equal(got, res), f"layer {l}: streamed output differs from the resident layer"
        ids = Lb.ids[: T * wl.k].cpu().numpy().reshape(T, wl.k)
        rids, g = oracle.route(logits[l], wl.k)
        assert np.array_equal(ids, rids)
        gw = Lb.w[: T * wl.k].cpu().numpy().reshape(T, wl.k)
        assert np.abs(gw - g).max() <= 1e-6 * np.abs(g).max()
        f64 = {}

        def expert(e, l=l, f64=f64):
            if e not in f64:
                f64[e] = oracle.expert_f64(exs[l][e], wl.wdtype)
            return f64[e]

        ref = oracle.moe_layer(xf[sample], rids[sample], g[sample], expert, shared=expert(E) if ws else None)
        err = rel_err_rows(out_f64(got, wl, T)[sample], ref).max()
        assert err <= TOL[wl.wdtype], f"layer {l}: rel err {err}"
        del pool_l
    Lb.close()


def test_prefill_stream_rejects_bad_arguments(B):
    """Validation happens before anything is enqueued (and needs no upload)."""
    from expert_cached_moe_amd.runtime import LayerBuffers
    wl = synth.workload("tiny_fp32")
    cfg = config(wl, n_slots=0, n_layers=2)
    Lb = LayerBuffers(cfg, 16)
    bufs = torch.zeros(2 * wl.E * B.moe_expert_bytes(cfg), dtype=torch.uint8, device="cuda")
    out = torch.empty(2 * 16 * wl.H, dtype=torch.float32, device="cuda")
    args = lambda nbuf, s, side: (Lb.ctx, bufs, nbuf, torch.zeros(2 * 16 * wl.E, device="cuda"),
                                  torch.zeros(16 * wl.H, device="cuda"), 16, None, Lb.ids, Lb.w, Lb.counts,
                                  Lb.offsets, Lb.perm, Lb.inv, Lb.o, Lb.ws, out, s, side)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    with pytest.raises(B.MoeError, match="host pool"):
        B.moe_prefill_stream(*args(2, main, side))                     # no host pool bound
    host = torch.zeros(2 * wl.E * B.moe_expert_bytes(cfg), dtype=torch.uint8, pin_memory=True)
    B.moe_bind_pools(Lb.ctx, None, 0, host, 2 * wl.E)
    with pytest.raises(B.MoeError, match="n_buffers"):
        B.moe_prefill_stream(*args(3, main, side))
    with pytest.raises(B.MoeError, match="stream of their own"):
        B.moe_prefill_stream(*args(2, main, main))
    Lb.close()
