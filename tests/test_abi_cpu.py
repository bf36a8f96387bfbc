"""C-ABI checks that need no GPU: the library loads and exports every declared
symbol; the host parts of the path (q*, the global LRU planner, the CPU expert
FFN, blob packing, validation) match the oracle.  No GPU compute is called."""
import os
import re

import numpy as np
import pytest

import oracle
import synth
from helpers import Experts, TOL, config, rel_err_rows

B = pytest.importorskip("expert_cached_moe_amd.binding")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_match_header():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        hdr = f.read()
    declared = sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(moe_\w+)\s*\(", hdr, re.M)))
    assert declared, "no declarations parsed"
    assert sorted(declared) == sorted(B.EXPORTS)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    syms = set(re.findall(r"\sT\s(moe_\w+)$", out, re.M))
    for name in declared:
        assert name in syms, name
    assert B.exported_symbols() == B.EXPORTS


def test_qstar_matches_oracle_and_table():
    for bp, bh in [(52.7, 77.3), (11.8, 47.5), (30.0, 30.0), (60.0, 40.0), (1.0, 3.0)]:
        for m in range(0, 65):
            for rnd, name in [(0, "nearest"), (1, "argmin")]:
                assert B.moe_qstar(m, bp, bh, rnd) == oracle.qstar(m, bp, bh, name), (bp, bh, m, rnd)
    assert B.moe_qstar(-3, 52.7, 77.3, 0) == 0


def test_config_validation():
    ok = B.make_config(256, 128, 8, 2, 0, 3, 1, 0)
    B.moe_destroy(B.moe_create(ok))
    bad = [
        dict(hidden=100), dict(hidden=96), dict(hidden=224, w_dtype=2), dict(inter=48), dict(n_experts=0), dict(n_experts=513), dict(top_k=9),
        dict(top_k=0), dict(n_shared=2), dict(n_slots=-1), dict(n_layers=0), dict(w_dtype=7),
        dict(renormalize=2), dict(q_round=5), dict(bp_gbps=0.0), dict(bh_gbps=float("nan")),
    ]
    for b in bad:
        kw = dict(hidden=256, inter=128, n_experts=8, top_k=2, n_shared=0, n_slots=3, n_layers=1, w_dtype=0)
        kw.update(b)
        cfg = B.make_config(**kw)
        with pytest.raises(B.MoeError):
            B.moe_create(cfg)
        assert B._lib.moe_expert_bytes(B.ctypes.byref(cfg)) < 0


def test_blob_sizes():
    for name in synth.WORKLOADS:
        wl = synth.workload(name)
        nb = B.moe_expert_bytes(config(wl))
        assert nb % 256 == 0
        elems = 3 * wl.H * wl.I
        payload = {"f32": elems * 4, "bf16": elems * 2, "mxfp4": elems // 2 + elems // 32}[wl.wdtype]
        assert payload <= nb < payload + 4 * 256
        assert B.moe_pair_rows(config(wl), 5) == 5 * wl.k + (5 if wl.n_shared else 0)


def _plan_dict(p):
    return {"distinct": p.get("distinct").tolist(), "hit": p.get("hit").tolist(),
            "hit_slot": p.get("hit_slot").tolist(), "fill": p.get("fill").tolist(),
            "fill_slot": p.get("fill_slot").tolist(), "fill_victim": p.get("fill_victim").tolist(),
            "host": p.get("host").tolist()}


def _replay_compare(wl, ids_steps, C, bp, bh, q_round=0):
    """C++ planner vs the oracle LRU, bit-exact per step (plans and slot tables)."""
    cfg = config(wl, n_slots=C, bp=bp, bh=bh, q_round=q_round)
    ctx = B.moe_create(cfg)
    try:
        ref = oracle.LRUCache(C, wl.E)
        n_steps, T = len(ids_steps), ids_steps[0].shape[0]
        cap = min(wl.E, T * wl.k)
        plans = [B.Plan(cap, wl.E) for _ in range(n_steps)]
        st = B.moe_lru_replay(ctx, 0, np.stack(ids_steps), n_steps, T, plans)
        tot = {"m": 0, "q": 0, "n": 0}
        for s in range(n_steps):
            want = ref.step(ids_steps[s], bp, bh, "argmin" if q_round else "nearest")
            got = _plan_dict(plans[s])
            for key in got:
                assert got[key] == want[key], (wl.name, s, key)
            assert np.array_equal(plans[s].get("slot_of_expert"), want["slot_of_expert"])
            tot["m"] += want["m"]
            tot["q"] += want["q"]
            tot["n"] += len(want["distinct"])
        assert (st.steps, st.misses, st.fills, st.distinct) == (n_steps, tot["m"], tot["q"], tot["n"])
        assert np.array_equal(B.moe_lru_slots(ctx, 0, wl.E), ref.slot_table(0))
    finally:
        B.moe_destroy(ctx)
    return tot


def test_planner_hand_traces():
    import os
    gold = os.path.join(ROOT, "tests", "golden", "lru_traces.txt")
    lines = [ln.strip() for ln in open(gold) if ln.strip() and not ln.startswith("#")]
    traces, cur = [], None
    for ln in lines:
        if ln.startswith("trace"):
            _, name, E, C, k, bp, bh = ln.split()
            cur = dict(E=int(E), C=int(C), k=int(k), bp=float(bp), bh=float(bh), steps=[])
            traces.append(cur)
        else:
            f = [p.strip() for p in ln.split("|")]
            toks = np.array([[int(v) for v in t.split(",")] for t in f[0].split(";")], np.int32)
            want = [[] if v == "-" else [int(x) for x in v.split(",")] for v in f[1:]]
            cur["steps"].append((toks, want))
    for tr in traces:
        cfg = B.make_config(64, 32, tr["E"], tr["k"], 0, tr["C"], 1, 0, 1, 0, tr["bp"], tr["bh"])
        ctx = B.moe_create(cfg)
        for toks, want in tr["steps"]:
            p = B.Plan(tr["E"], tr["E"])
            B.moe_lru_step(ctx, 0, toks, toks.shape[0], p)
            got = [p.get(f).tolist() for f in ("distinct", "hit", "hit_slot", "fill", "fill_slot", "fill_victim",
                                               "host")]
            assert got == want
        B.moe_destroy(ctx)


@pytest.mark.parametrize("name,B_,steps", [("tiny_fp32", 1, 64), ("a3b_decode_bf16", 1, 4096),
                                          ("a3b_decode_bf16", 4, 1024), ("a3b_decode_bf16", 8, 1024),
                                          ("v4flash_decode_bf16", 1, 4096), ("v4flash_decode_bf16", 8, 1024)])
def test_planner_matches_oracle_lru(name, B_, steps):
    wl = synth.workload(name)
    if name == "tiny_fp32":
        x = synth.activations(wl, steps, tag=1)
        logits = oracle.router_logits(x, synth.router_weights(wl))[:, None, :]
    else:
        logits, _ = synth.zipf_reuse_trace(wl, B_, steps)
    ids_steps = [oracle.route(logits[s], wl.k)[0] for s in range(steps)]
    tot = _replay_compare(wl, ids_steps, wl.C, 52.7, 77.3)
    assert tot["q"] <= tot["m"]
    _replay_compare(wl, ids_steps, wl.C, 52.7, 77.3, q_round=1)
    _replay_compare(wl, ids_steps[: min(steps, 512)], wl.C, 1.0, 1.0)          # pure LRU (q = m)


def test_planner_mattson_every_capacity():
    """Pure LRU (B_P = B_H): the C++ planner's misses equal the stack-distance counts at every C."""
    wl = synth.workload("a3b_decode_bf16")
    logits, _ = synth.zipf_reuse_trace(wl, 2, 600, tag=3)
    ids_steps = [oracle.route(logits[s], wl.k)[0] for s in range(600)]
    order = [oracle.step_order(s) for s in ids_steps]
    mat = oracle.mattson_misses(order, wl.E)
    smax = max(len(s) for s in order)
    for C in [smax, smax + 1, 24, 47, 64, 100, wl.E]:
        ctx = B.moe_create(config(wl, n_slots=C, bp=1.0, bh=1.0))
        st = B.moe_lru_replay(ctx, 0, np.stack(ids_steps), 600, 2)
        assert st.misses == mat[C], C
        B.moe_destroy(ctx)


def test_planner_errors_leave_state_untouched():
    wl = synth.workload("a3b_decode_bf16")
    ctx = B.moe_create(config(wl))
    p = B.Plan(wl.E, wl.E)
    good = np.arange(8, dtype=np.int32)[None, :]
    B.moe_lru_step(ctx, 0, good, 1, p)
    before = B.moe_lru_stats(ctx).misses, B.moe_lru_slots(ctx, 0, wl.E).copy()
    for bad in (np.array([[0, 1, 2, 3, 4, 5, 6, 200]], np.int32), np.array([[0, 1, 2, 3, 4, 5, 6, 6]], np.int32)):
        with pytest.raises(B.MoeError):
            B.moe_lru_step(ctx, 0, bad, 1, p)
    with pytest.raises(B.MoeError):
        B.moe_lru_step(ctx, 0, good + 8, 1, B.Plan(2, wl.E))          # capacity too small
    with pytest.raises(B.MoeError):
        B.moe_lru_step(ctx, 1, good, 1, p)                               # layer out of range
    assert (B.moe_lru_stats(ctx).misses, ) == (before[0], )
    assert np.array_equal(B.moe_lru_slots(ctx, 0, wl.E), before[1])
    B.moe_lru_reset(ctx)
    assert B.moe_lru_stats(ctx).steps == 0 and (B.moe_lru_slots(ctx, 0, wl.E) == -1).all()
    B.moe_destroy(ctx)


@pytest.mark.parametrize("bp,bh", [(52.7, 77.3), (1.0, 1.0)])
def test_planner_resize_matches_oracle(bp, bh):
    """C++ planner vs the oracle with resizes at random safe points (shrinks, grows, down to
    zero slots): every plan, every move and eviction list, and the slot tables bit-exact."""
    wl = synth.workload("a3b_decode_bf16")
    Bt, n = 4, 400
    logits, _ = synth.zipf_reuse_trace(wl, Bt, n)
    ids_steps = [oracle.route(logits[t], wl.k)[0] for t in range(n)]
    rng = np.random.default_rng(5)
    events = {int(t): int(c) for t, c in zip(rng.choice(n, 12, replace=False), rng.integers(0, 80, 12))}
    events[200] = 0
    cfg = config(wl, n_slots=wl.C, bp=bp, bh=bh)
    ctx = B.moe_create(cfg)
    try:
        ref = oracle.LRUCache(wl.C, wl.E)
        plan = B.Plan(min(wl.E, Bt * wl.k), wl.E)
        for t in range(n):
            if t in events:
                r = B.Resize(128)
                B.moe_lru_resize(ctx, events[t], r)
                want = ref.resize(events[t])
                assert r.moves() == want["moves"] and r.evicted() == want["evicted"], t
                assert np.array_equal(B.moe_lru_slots(ctx, 0, wl.E), ref.slot_table(0)), t
            B.moe_lru_step(ctx, 0, ids_steps[t], Bt, plan)
            want = ref.step(ids_steps[t], bp, bh)
            got = _plan_dict(plan)
            for key in got:
                assert got[key] == want[key], (t, key)
            assert np.array_equal(plan.get("slot_of_expert"), want["slot_of_expert"]), t
    finally:
        B.moe_destroy(ctx)


def test_resize_errors_leave_state_untouched():
    wl = synth.workload("tiny_fp32")
    ctx = B.moe_create(config(wl, n_slots=4, bp=1.0, bh=1.0))
    try:
        plan = B.Plan(2, wl.E)
        for ids in ([0, 1], [2, 3], [4, 5], [1, 6]):
            B.moe_lru_step(ctx, 0, np.array([ids], np.int32), 1, plan)
        before = B.moe_lru_slots(ctx, 0, wl.E).copy()
        with pytest.raises(B.MoeError):
            B.moe_lru_resize(ctx, -1, B.Resize(8))
        with pytest.raises(B.MoeError):
            B.moe_lru_resize(ctx, 2, B.Resize(1))          # two moves and two evictions
        assert np.array_equal(B.moe_lru_slots(ctx, 0, wl.E), before)
        r = B.Resize(2)
        B.moe_lru_resize(ctx, 2, r)
        assert r.moves() == [(2, 0), (3, 1)] and r.evicted() == [5, 4]
        with pytest.raises(B.MoeError):                   # a pool larger than the resized cache is refused
            B.moe_bind_pools(ctx, 1, 3, None, 0)
    finally:
        B.moe_destroy(ctx)


def test_multilayer_keys():
    """Two layers share one cache; keys are (layer, expert)."""
    wl = synth.workload("tiny_fp32")
    cfg = config(wl, n_slots=3, bp=1.0, bh=1.0, n_layers=2)
    ctx = B.moe_create(cfg)
    ref = oracle.LRUCache(3, wl.E, n_layers=2)
    rng = np.random.default_rng(1)
    for s in range(200):
        layer = s % 2
        ids = np.stack([rng.permutation(wl.E)[:2]]).astype(np.int32)
        p = B.Plan(8, wl.E)
        B.moe_lru_step(ctx, layer, ids, 1, p)
        want = ref.step(ids, 1.0, 1.0, layer=layer)
        assert p.get("fill_victim").tolist() == want["fill_victim"]
        assert p.get("hit").tolist() == want["hit"]
        assert np.array_equal(p.get("slot_of_expert"), want["slot_of_expert"])
    B.moe_destroy(ctx)


@pytest.mark.parametrize("name,n_layers,B_,steps", [("a3b_decode_bf16", 4, 1, 384), ("v4flash_decode_bf16", 4, 2, 256),
                                                    ("a3b_decode_bf16", 8, 1, 128)])
def test_multilayer_stack_matches_oracle(name, n_layers, B_, steps):
    """A stack of n_layers MoE layers shares one cache whose capacity is the workload's fraction
    of the whole pool (37 % or 11 % of n_layers * E), keyed (layer, expert) ([A] "Abandoning
    fixed offloading ...": one LRU over the experts of all layers).  Each layer routes by its own
    Zipf trace; every decode step plans layer 0 .. n_layers-1 in order.  Every plan, the slot
    tables and the statistics match the oracle's cache bit for bit."""
    wl = synth.workload(name)
    frac = wl.C / wl.E
    C = int(round(frac * n_layers * wl.E))
    cfg = config(wl, n_slots=C, n_layers=n_layers)
    ctx = B.moe_create(cfg)
    ref = oracle.LRUCache(C, wl.E, n_layers=n_layers)
    traces = [synth.zipf_reuse_trace(wl, B_, steps, tag=100 + l)[0] for l in range(n_layers)]
    p = B.Plan(min(wl.E, B_ * wl.k), wl.E)
    misses = distinct = 0
    for s in range(steps):
        for l in range(n_layers):
            ids = oracle.route(traces[l][s], wl.k)[0]
            B.moe_lru_step(ctx, l, ids, B_, p)
            want = ref.step(ids, 52.7, 77.3, layer=l)
            for f in ("distinct", "hit", "hit_slot", "fill", "fill_slot", "fill_victim", "host"):
                assert p.get(f).tolist() == list(want[f]), (s, l, f)
            assert np.array_equal(p.get("slot_of_expert"), want["slot_of_expert"]), (s, l)
            misses += want["m"]
            distinct += len(want["distinct"])
    for l in range(n_layers):
        assert np.array_equal(B.moe_lru_slots(ctx, l, wl.E), ref.slot_table(l))
    st = B.moe_lru_stats(ctx)
    assert (st.misses, st.distinct, st.steps) == (misses, distinct, steps * n_layers)
    B.moe_destroy(ctx)


def _host_pool(cfg, ex, E):
    from expert_cached_moe_amd.runtime import pack_pool
    return pack_pool(cfg, [ex.raw(e) for e in range(E)], pin=False)


@pytest.mark.parametrize("name,T,n_host", [("tiny_fp32", 5, 3), ("a3b_decode_bf16", 4, 3),
                                          ("v4flash_mxfp4", 2, 2), ("v4flash_decode_bf16", 1, 2)])
def test_host_ffn_matches_oracle(name, T, n_host):
    """The CPU side of the split: y_host = sum over the plan's host experts (no GPU)."""
    wl = synth.workload(name)
    ex = Experts(wl)
    rng = np.random.default_rng(T)
    logits = rng.standard_normal((T, wl.E)).astype(np.float32)
    ids, gates = oracle.route(logits, wl.k)
    present = sorted(set(ids.ravel().tolist()))
    host = present[:n_host]
    # host pool holding only the needed experts: other blobs stay zero
    cfg = config(wl)
    nb = B.moe_expert_bytes(cfg)
    pool = np.zeros(wl.E * nb, np.uint8)
    for e in host:
        w = ex.raw(e)
        B.moe_pack_expert(cfg, w["wg"], w["wu"], w["wd"], w.get("sg"), w.get("su"), w.get("sd"),
                          pool[e * nb:(e + 1) * nb])
    ctx = B.moe_create(cfg)
    B.moe_bind_pools(ctx, None, 0, pool, wl.E)
    p = B.Plan(wl.E, wl.E)
    p.arrays["host"][: len(host)] = host
    p.c.n_host = len(host)
    x = synth.activations(wl, T, tag=7)
    y = np.full((T, wl.H), np.nan, np.float32)
    w32 = gates.astype(np.float32)
    for nt in (1, 3, 0):
        B.moe_host_ffn(ctx, x, T, ids.astype(np.int32), w32, p, y, nt)
        xf = oracle.act_f64(x, wl.act_dtype)
        ref = oracle.moe_layer(xf, ids, w32.astype(np.float64), ex, subset=set(host))
        err = rel_err_rows(y, ref)
        assert err.max() <= min(TOL[wl.wdtype], 1e-4), (nt, err.max())
        if nt == 1:
            y1 = y.copy()
        else:
            assert np.array_equal(y, y1)            # independent of the thread count
    B.moe_destroy(ctx)


def test_pack_rejects_nan_scale():
    wl = synth.workload("v4flash_mxfp4")
    cfg = config(wl)
    w = synth.expert_weights(wl, 0)
    sg = w["sg"].copy()
    sg[3, 1] = 0xFF
    blob = np.full(B.moe_expert_bytes(cfg), 7, np.uint8)
    with pytest.raises(B.MoeError):
        B.moe_pack_expert(cfg, w["wg"], w["wu"], w["wd"], sg, w["su"], w["sd"], blob)
    assert (blob == 7).all()                    # no side effect on error


def test_ffn_merge_argument_errors():
    """moe_expert_ffn_merge rejects what it cannot run before touching the GPU: batches
    above the decode size, a missing host copy of the ids, bad or repeated expert ids,
    a shared expert the config does not have.  (The addresses are never dereferenced.)"""
    wl = synth.workload("a3b_decode_bf16")
    cfg = config(wl)
    ctx = B.moe_create(cfg)
    ids = np.arange(wl.k, dtype=np.int32)[None, :]
    ex = np.arange(wl.k, dtype=np.int32)
    good = dict(d_x=64, T=1, h_topk_ids=ids, d_topk_ids=64, d_topk_w=64, d_slot_base=64, h_experts=ex,
                h_slots=ex, n=wl.k, d_shared=None, with_shared=0, d_y_host=None, d_out=64, d_ws=64)

    def status(**kw):
        args = dict(good, **kw)
        with pytest.raises(B.MoeError) as ei:
            B.moe_expert_ffn_merge(ctx, **args)
        return ei.value.status

    assert status(T=9, h_topk_ids=np.zeros((9, wl.k), np.int32)) == B.MOE_ESHAPE
    assert status(h_topk_ids=None) == B.MOE_EINVAL
    assert status(d_topk_w=None) == B.MOE_EINVAL
    assert status(h_experts=np.array([0, 1, 2, 3, 4, 5, 6, wl.E], np.int32)) == B.MOE_EINVAL
    assert status(h_experts=np.array([0, 1, 2, 3, 4, 5, 6, 6], np.int32)) == B.MOE_EINVAL
    assert status(h_topk_ids=np.array([[0, 1, 2, 3, 4, 5, 6, -1]], np.int32)) == B.MOE_EINVAL
    assert status(h_topk_ids=np.array([[0, 1, 2, 3, 4, 5, 6, 6]], np.int32)) == B.MOE_EINVAL
    assert status(with_shared=1, d_shared=64) == B.MOE_EINVAL
    B.moe_destroy(ctx)


def test_noalloc_rejects_oversized_batch():
    """moe_expert_ffn_merge_noalloc refuses a decode batch whose scratch exceeds the library's
    array (MXFP4, hidden = inter = 16384, 512 experts top-16 + shared: 8.9 MB at T = 8) before
    any GPU work; the same layer at T = 7 fits.  (The addresses are never dereferenced.)"""
    cfg = B.make_config(16384, 16384, 512, 16, 1, 0, 1, B.MOE_W_MXFP4)
    assert B.moe_workspace_bytes(cfg, 8) > B.moe_noalloc_scratch_bytes() >= B.moe_workspace_bytes(cfg, 7)
    ctx = B.moe_create(cfg)
    ids = np.arange(8 * 16, dtype=np.int32).reshape(8, 16)
    with pytest.raises(B.MoeError) as ei:
        B.moe_expert_ffn_merge_noalloc(ctx, 256, 8, ids, 256, 256, 256, np.arange(128), np.arange(128), 128, 256, 1,
                                       None, 256, None)
    assert ei.value.status == B.MOE_ECAPACITY
    assert "exceeds" in B.moe_last_error(ctx)
    B.moe_destroy(ctx)
