"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
fixtures under tests/golden/ (each citing its page), closed forms, textbook
algorithms (Mattson's stack distances, subset enumeration, dense evaluation of
every expert) and special cases.  No HIP code is involved.
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def _ints(s):
    s = s.strip()
    return [] if s == "-" else [int(v) for v in s.split(",")]


# ------------------------------------------------------------------ routing
def test_route_tie_fixture():
    for ln in _lines("route_ties.txt"):
        lg, k, want = [p.strip() for p in ln.split("|")]
        l = np.array([[float(v) for v in lg.split()]], dtype=np.float32)
        ids, _ = oracle.route(l, int(k))
        assert ids[0].tolist() == [int(v) for v in want.split()], ln


def _router_cases():
    cases, cur = [], None
    for ln in _lines("router_logits.txt"):
        tag, *vals = ln.split()
        if tag == "case":
            cur = {"name": vals[0], "x": [], "wr": [], "l": []}
        elif tag == "end":
            cases.append(cur)
        else:
            cur[tag].append([float.fromhex(v) if "0x" in v else float(v) for v in vals])
    return cases


def test_router_logits_fixture():
    """Hand-worked logits, bit for bit: a scaled, transposed or partly dropped product fails
    the first case; accumulating in fp32 (instead of one rounding of the exact sum) fails the
    other two."""
    cases = _router_cases()
    assert len(cases) == 3
    for c in cases:
        x = np.array(c["x"], np.float32)
        wr = np.array(c["wr"], np.float32)
        want = np.array(c["l"], np.float32)
        got = oracle.router_logits(x, wr)
        assert got.dtype == np.float32 and got.shape == want.shape, c["name"]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (c["name"], got, want)


def _dominance_topk(row, k):
    """Brute force: the unique ordered k-list whose members beat every non-member."""
    E = len(row)

    def beats(a, b):        # a ranks before b
        return row[a] > row[b] or (row[a] == row[b] and a < b)

    found = []
    for sub in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in sub]
        if all(beats(a, b) for a in sub for b in rest):
            ordered = list(sub)
            for i in range(len(ordered)):          # selection by pairwise comparison
                for j in range(i + 1, len(ordered)):
                    if beats(ordered[j], ordered[i]):
                        ordered[i], ordered[j] = ordered[j], ordered[i]
            found.append(ordered)
    assert len(found) == 1
    return found[0]


def test_route_subset_bruteforce():
    rng = np.random.default_rng(7)
    for trial in range(200):
        E = int(rng.integers(1, 8))
        k = int(rng.integers(1, E + 1))
        row = rng.integers(-3, 4, size=E).astype(np.float32) * np.float32(0.5)   # many ties
        ids, _ = oracle.route(row[None, :], k)
        assert ids[0].tolist() == _dominance_topk(row.tolist(), k)


def test_gates_closed_forms():
    # k = 2: the renormalised softmax of two logits is a logistic function of their difference
    rng = np.random.default_rng(3)
    l = rng.standard_normal((64, 5)).astype(np.float32)
    ids, g = oracle.route(l, 2)
    a = np.take_along_axis(l, ids, 1).astype(np.float64)
    np.testing.assert_allclose(g[:, 0], expit(a[:, 0] - a[:, 1]), rtol=1e-15, atol=0)
    np.testing.assert_allclose(g[:, 1], expit(a[:, 1] - a[:, 0]), rtol=1e-15, atol=0)
    # k = E: renormalised gates are the full softmax, listed in routed order
    ids, g = oracle.route(l, 5)
    sm = softmax(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(g, np.take_along_axis(sm, ids, 1), rtol=1e-14)
    # renormalize=False: gates are the full softmax entries of the routed experts
    ids, g = oracle.route(l, 2, renormalize=False)
    np.testing.assert_allclose(g, np.take_along_axis(sm, ids, 1), rtol=1e-14)
    # three equal top logits, k = 3: each gate is exactly 1/3
    _, g = oracle.route(np.array([[1.0, 3.0, 3.0, -2.0, 3.0]], np.float32), 3)
    np.testing.assert_allclose(g, [[1 / 3, 1 / 3, 1 / 3]], rtol=1e-15)
    # shift invariance
    _, g1 = oracle.route(l, 3)
    _, g2 = oracle.route(l + np.float32(8.0), 3)
    np.testing.assert_allclose(g1, g2, rtol=1e-5)


def test_route_rejects_nan():
    with pytest.raises(ValueError):
        oracle.route(np.array([[0.0, np.nan]], np.float32), 1)


def test_permute_bruteforce():
    rng = np.random.default_rng(11)
    for T, E, k in [(1, 4, 2), (7, 8, 3), (33, 16, 4), (100, 5, 5), (0, 4, 2)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else \
            np.zeros((0, k), np.int32)
        counts, offsets, perm, inv = oracle.permute(ids, E)
        flat = ids.ravel().tolist()
        assert counts.tolist() == [flat.count(e) for e in range(E)]
        assert offsets[0] == 0 and offsets[-1] == len(flat)
        for e in range(E):
            assert perm[offsets[e]:offsets[e + 1]].tolist() == [p for p in range(len(flat)) if flat[p] == e]
        assert all(inv[perm[i]] == i for i in range(len(flat)))


# ------------------------------------------------------------------ expert and layer
def _dense_layer(x, logits, k, W_all, shared=None):
    """All experts on all tokens, weighted by a dense gate vector (zero off the top-k)."""
    T, E = logits.shape
    G = np.zeros((T, E))
    for t in range(T):
        top = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        z = [math.exp(float(logits[t, e]) - float(logits[t, top[0]])) for e in top]
        for e, v in zip(top, z):
            G[t, e] = v / sum(z)
    Wg = np.stack([w[0] for w in W_all])        # [E, I, H]
    Wu = np.stack([w[1] for w in W_all])
    Wd = np.stack([w[2] for w in W_all])        # [E, H, I]
    g = np.einsum("th,eih->tei", x, Wg)
    u = np.einsum("th,eih->tei", x, Wu)
    h = g * expit(g) * u
    o = np.einsum("tei,ehi->teh", h, Wd)
    y = np.einsum("te,teh->th", G, o)
    if shared is not None:
        gs = x @ shared[0].T
        y += (gs * expit(gs) * (x @ shared[1].T)) @ shared[2].T
    return y


@pytest.fixture(scope="module")
def tiny():
    wl = synth.workload("tiny_fp32")
    x = synth.activations(wl, wl.T)
    logits = oracle.router_logits(x, synth.router_weights(wl))
    W = {e: oracle.expert_f64(synth.expert_weights(wl, e), "f32") for e in range(wl.E)}
    return wl, x.astype(np.float64), logits, W


def test_layer_dense_bruteforce(tiny):
    wl, x, logits, W = tiny
    ids, gates = oracle.route(logits, wl.k)
    y = oracle.moe_layer(x, ids, gates, W)
    yd = _dense_layer(x, logits, wl.k, [W[e] for e in range(wl.E)])
    assert np.abs(y - yd).max() <= 1e-12 * np.abs(yd).max()
    # with a shared expert (always on, gate 1)
    y2 = oracle.moe_layer(x, ids, gates, W, shared=W[0])
    yd2 = _dense_layer(x, logits, wl.k, [W[e] for e in range(wl.E)], shared=W[0])
    assert np.abs(y2 - yd2).max() <= 1e-12 * np.abs(yd2).max()


def test_layer_bf16_and_mxfp4_dense():
    for name in ("a3b_decode_bf16", "v4flash_mxfp4"):
        wl = synth.workload(name)
        sub = 4                                     # 4 experts, reduced K slices keep this fast
        W = [oracle.expert_f64(synth.expert_weights(wl, e), wl.wdtype) for e in range(sub)]
        x = oracle.bf16_bits_to_f64(synth.activations(wl, 3))
        logits = np.array([[0.3, -1.0, 2.0, 0.1], [1.0, 1.0, 1.0, 1.0], [-2.0, 0.5, 0.0, 4.0]], np.float32)
        ids, gates = oracle.route(logits, 2)
        y = oracle.moe_layer(x, ids, gates, dict(enumerate(W)))
        yd = _dense_layer(x, logits, 2, W)
        assert np.abs(y - yd).max() <= 1e-12 * np.abs(yd).max()


def test_expert_special_cases(tiny):
    wl, x, logits, W = tiny
    ids, gates = oracle.route(logits, 1)
    assert np.allclose(gates, 1.0)
    # k = 1: the layer is the selected expert itself
    y = oracle.moe_layer(x, ids, gates, W)
    for t in range(x.shape[0]):
        wg, wu, wd = W[int(ids[t, 0])]
        g = wg @ x[t]
        want = wd @ (g * expit(g) * (wu @ x[t]))
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-15)
    # Wu = 0 -> exactly zero output; Wg = 0 -> silu(0) = 0 -> exactly zero
    ids2, g2 = oracle.route(logits, 2)
    Wz = {e: (w[0], np.zeros_like(w[1]), w[2]) for e, w in W.items()}
    assert not np.any(oracle.moe_layer(x, ids2, g2, Wz))
    Wz = {e: (np.zeros_like(w[0]), w[1], w[2]) for e, w in W.items()}
    assert not np.any(oracle.moe_layer(x, ids2, g2, Wz))
    # identical experts: gates sum to one, so the layer equals that expert
    Wsame = {e: W[0] for e in W}
    ys = oracle.moe_layer(x, ids2, g2, Wsame)
    gg = x @ W[0][0].T
    want = (gg * expit(gg) * (x @ W[0][1].T)) @ W[0][2].T
    np.testing.assert_allclose(ys, want, rtol=1e-12, atol=1e-14)
    # silu -> identity for large positive gate pre-activations: y = Wd((Wg x) * (Wu x))
    wg, wu, wd = W[3]
    xs = np.abs(x[:2])
    big = np.abs(wg) * 2000.0
    g = xs @ big.T
    assert g.min() > 40
    o = oracle.expert_ffn((big, wu, wd), xs)
    np.testing.assert_allclose(o, (g * (xs @ wu.T)) @ wd.T, rtol=1e-12)
    # ... and -> 0 for large negative ones
    o = oracle.expert_ffn((-big, wu, wd), xs)
    assert np.abs(o).max() < 1e-12


def test_partition_invariant_exhaustive(tiny):
    """The GPU and CPU partial sums add up to the plain layer for every split of the
    routed experts ([B] "The q* Policy": the partial sums merge exactly)."""
    wl, x, logits, W = tiny
    ids, gates = oracle.route(logits, wl.k)
    y = oracle.moe_layer(x, ids, gates, W, shared=W[5])
    experts = sorted(set(ids.ravel().tolist()))
    for r in range(len(experts) + 1):
        for cache in itertools.combinations(experts, r):
            yc, yh = oracle.moe_layer_partitioned(x, ids, gates, W, cache, shared=W[5])
            assert np.abs(yc + yh - y).max() <= 1e-12 * np.abs(y).max()
    # nothing cached, no shared expert: the GPU part is exactly zero
    yc, yh = oracle.moe_layer_partitioned(x, ids, gates, W, [])
    assert not np.any(yc)


# ------------------------------------------------------------------ q*
def test_qstar_table():
    for ln in _lines("qstar_table.txt"):
        bp, bh, rnd, *qs = ln.split()
        got = [oracle.qstar(m, float(bp), float(bh), rnd) for m in range(9)]
        assert got == [int(q) for q in qs], ln


def test_qstar_makespan_derivation():
    """At the continuous optimum the DMA time of the filled experts equals the CPU time
    of the rest on the residual bandwidth B_H - B_P, and both equal m / B_H."""
    for bp, bh in [(52.7, 77.3), (11.8, 47.5)]:
        for m in range(1, 9):
            grid = np.linspace(0, m, 200001)
            cost = np.maximum(grid / bp, (m - grid) / (bh - bp))
            qc = grid[np.argmin(cost)]
            assert abs(qc - m * bp / bh) < 1e-4
            assert abs(cost.min() - m / bh) < 1e-6
            # the integer 'argmin' reading attains the integer minimum
            qi = oracle.qstar(m, bp, bh, "argmin")
            ci = [max(q / bp, (m - q) / (bh - bp)) for q in range(m + 1)]
            assert ci[qi] == min(ci)
    assert oracle.qstar(5, 80.0, 60.0) == 5          # no residual CPU bandwidth: fill all
    assert oracle.qstar(0, 52.7, 77.3) == 0


# ------------------------------------------------------------------ LRU
def _traces():
    out, cur = [], None
    for ln in _lines("lru_traces.txt"):
        if ln.startswith("trace"):
            _, name, E, C, k, bp, bh = ln.split()
            cur = {"name": name, "E": int(E), "C": int(C), "k": int(k), "bp": float(bp),
                   "bh": float(bh), "steps": []}
            out.append(cur)
        else:
            f = [p.strip() for p in ln.split("|")]
            toks = [_ints(t) for t in f[0].split(";")]
            cur["steps"].append((toks, *[_ints(v) for v in f[1:]]))
    return out


def test_lru_hand_traces():
    for tr in _traces():
        cache = oracle.LRUCache(tr["C"], tr["E"])
        for toks, dist, hit, hslot, fill, fslot, victim, host in tr["steps"]:
            p = cache.step(np.array(toks), tr["bp"], tr["bh"])
            got = (p["distinct"], p["hit"], p["hit_slot"], p["fill"], p["fill_slot"],
                   p["fill_victim"], p["host"])
            assert got == (dist, hit, hslot, fill, fslot, victim, host), (tr["name"], toks)
            tab = p["slot_of_expert"]
            for e, s in zip(hit + fill, hslot + fslot):
                assert tab[e] == s


def _random_step_sets(rng, E, k, B, n):
    sets = []
    for _ in range(n):
        ids = np.stack([rng.choice(E, size=k, replace=False, p=None) for _ in range(B)])
        sets.append(ids)
    return sets


@pytest.mark.parametrize("E,k,B", [(12, 2, 1), (16, 3, 2), (20, 4, 3), (10, 1, 4)])
def test_lru_equals_mattson_stack(E, k, B):
    """With every miss filled (B_P = B_H) the slot cache is a stack algorithm: its
    misses at every size C >= the largest step equal Mattson's stack-distance count."""
    rng = np.random.default_rng(E * 100 + k * 10 + B)
    pz = 1.0 / np.arange(1, E + 1) ** 1.1
    steps = [np.stack([rng.choice(E, size=k, replace=False, p=pz / pz.sum()) for _ in range(B)])
             for _ in range(300)]
    order = [oracle.step_order(s) for s in steps]
    mat = oracle.mattson_misses(order, E + 2)
    smax = max(len(s) for s in order)
    prev = None
    for C in range(smax, E + 3):
        cache = oracle.LRUCache(C, E)
        miss = sum(cache.step(s, 1.0, 1.0)["m"] for s in steps)
        assert miss == mat[C], C
        if prev is not None:
            assert miss <= prev
        prev = miss
    # C >= E: only first references miss
    assert mat[E] == len(set(np.concatenate([s.ravel() for s in steps]).tolist()))


def test_lru_plan_invariants():
    """q* split bookkeeping on a Zipf/reuse trace: sets partition the step, slots stay consistent."""
    wl = synth.workload("a3b_decode_bf16")
    for B in (1, 8):
        logits, _ = synth.zipf_reuse_trace(wl, B, 200)
        cache = oracle.LRUCache(wl.C, wl.E)
        for t in range(200):
            ids, _ = oracle.route(logits[t], wl.k)
            p = cache.step(ids, 52.7, 77.3)
            assert sorted(p["hit"] + p["fill"] + p["host"]) == sorted(p["distinct"])
            assert p["q"] == len(p["fill"]) <= wl.C - len(p["hit"])
            assert p["q"] == min(oracle.qstar(p["m"], 52.7, 77.3), wl.C - len(p["hit"]))
            tab = p["slot_of_expert"]
            occupied = tab[tab >= 0]
            assert len(set(occupied.tolist())) == occupied.size <= wl.C
            assert all(tab[e] < 0 for e in p["host"])


def test_resize_hand_case():
    """Hand-derived ([B] "Elastic Memory" reading: keep the most recent, move survivors down).
    C = 4, every miss filled.  Steps {0,1}, {2,3}: slots 0..3 = e0, e1, e2, e3 with recency
    (1,2) (1,1) (2,2) (2,1).  Step {4,5}: victims e1 (1,1) then e0 (1,2): slot 1 = e4 (3,2),
    slot 0 = e5 (3,1).  Step {1,6}: victims e3 (2,1), e2 (2,2): slot 3 = e1 (4,2), slot 2 =
    e6 (4,1).  Shrink to 2: keep e1, e6 (the two most recent), drop e5 (slot 0) and e4
    (slot 1), move slot 2 -> 0 and slot 3 -> 1."""
    c = oracle.LRUCache(4, 8)
    for ids in ([0, 1], [2, 3], [4, 5], [1, 6]):
        c.step(np.array([ids]), 1.0, 1.0)
    assert c.slot_table().tolist() == [-1, 3, -1, -1, 1, 0, 2, -1]
    r = c.resize(2)
    assert r == {"moves": [(2, 0), (3, 1)], "evicted": [5, 4]}
    assert c.slot_table().tolist() == [-1, 1, -1, -1, -1, -1, 0, -1]
    # the next step hits e6 and e1 in their new slots; a miss now evicts the older of the two
    p = c.step(np.array([[6, 7]]), 1.0, 1.0)
    assert (p["hit"], p["hit_slot"], p["fill"], p["fill_slot"], p["fill_victim"]) == ([6], [0], [7], [1], [1])


@pytest.mark.parametrize("E,k,B,C,C2", [(16, 2, 1, 8, 3), (24, 3, 1, 12, 5), (20, 2, 2, 10, 6), (12, 1, 3, 9, 4)])
def test_resize_shrink_equals_smaller_cache(E, k, B, C, C2):
    """With every miss filled the cache is a stack algorithm: a cache of size C shrunk to C2
    at any step holds exactly the C2 most recent keys, which is what a cache that had size
    C2 all along holds, so from then on both take the same hits and misses."""
    rng = np.random.default_rng(E + 7 * C + C2)
    pz = 1.0 / np.arange(1, E + 1) ** 1.1
    steps = [np.stack([rng.choice(E, size=k, replace=False, p=pz / pz.sum()) for _ in range(B)])
             for _ in range(120)]
    assert max(len(oracle.step_order(s)) for s in steps) <= C2
    for cut in (0, 1, 17, 60, 119):
        big, small = oracle.LRUCache(C, E), oracle.LRUCache(C2, E)
        for t, s in enumerate(steps):
            if t == cut:
                big.resize(C2)
                keys_big = sorted(x for x in big.key_of_slot if x >= 0)
                keys_small = sorted(x for x in small.key_of_slot if x >= 0)
                assert keys_big == keys_small, (cut, keys_big, keys_small)
            pb, ps = big.step(s, 1.0, 1.0), small.step(s, 1.0, 1.0)
            if t >= cut:
                assert sorted(pb["hit"]) == sorted(ps["hit"]) and sorted(pb["fill"]) == sorted(ps["fill"]), (cut, t)


def test_resize_grow_then_shrink_back_is_identity():
    wl = synth.workload("a3b_decode_bf16")
    logits, _ = synth.zipf_reuse_trace(wl, 4, 60)
    c = oracle.LRUCache(wl.C, wl.E)
    for t in range(60):
        c.step(oracle.route(logits[t], wl.k)[0], 52.7, 77.3)
    before = (list(c.key_of_slot), list(c.recency))
    assert c.resize(wl.C + 30) == {"moves": [], "evicted": []}
    assert c.resize(wl.C) == {"moves": [], "evicted": []}
    assert (c.key_of_slot, c.recency) == before


# ------------------------------------------------------------------ MXFP4
def test_mxfp4_table_and_packing():
    table = {int(c): float(v) for c, v in (ln.split() for ln in _lines("mxfp4_codes.txt"))}
    codes = np.array([[c | (c << 4) for c in range(16)] * 2], dtype=np.uint8)    # 32 bytes = 64 elements
    val = oracle.mxfp4_decode(codes, np.array([[127, 127]], np.uint8))
    for c in range(16):
        assert val[0, 2 * c] == table[c] and val[0, 2 * c + 1] == table[c]
        assert math.copysign(1.0, val[0, 2 * c]) == math.copysign(1.0, table[c])
    # low nibble is the even element
    b = np.zeros((1, 16), np.uint8)
    b[0, 0] = 0x21
    v = oracle.mxfp4_decode(b, np.array([[127]], np.uint8))
    assert v[0, 0] == 0.5 and v[0, 1] == 1.0
    # scale: 2^(X-127)
    b[0, 0] = 0x02
    assert oracle.mxfp4_decode(b, np.array([[128]], np.uint8))[0, 0] == 2.0
    assert oracle.mxfp4_decode(b, np.array([[120]], np.uint8))[0, 0] == 2.0 ** -7
    with pytest.raises(ValueError):
        oracle.mxfp4_decode(b, np.array([[255]], np.uint8))


def test_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3F81, 0x7F7F], np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 1.0 + 2.0 ** -7, (2 - 2.0 ** -7) * 2.0 ** 127]
    assert oracle.bf16_bits_to_f64(bits).tolist() == want
    # rounding mirror: ties to even at bf16 precision
    assert oracle.round_to_bf16(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8])).tolist() == \
        [1.0, 1.0 + 2.0 ** -6]


# ------------------------------------------------------------------ prefill stream model
def test_prefill_worked_arithmetic():
    d = {}
    for ln in _lines("prefill_stream.txt"):
        key, *vals = ln.split()
        d[key] = [float(v) for v in vals]
    t = oracle.stream_time(d["pool_bytes"][0], d["link_bytes_per_s"][0])
    assert round(t, 2) == d["chunk_seconds_max"][0]                  # 1.2220 s -> "1.22"
    assert d["chunk_seconds_min"][0] <= t <= d["chunk_seconds_max"][0] + 0.005
    assert abs(d["chunk_tokens"][0] / t - d["tokens_per_s"][0]) / d["tokens_per_s"][0] < 0.01
    # transfer-bound pipeline: the chunk costs one pool stream plus the last layer's compute
    L = 40
    for pen in d["single_buffer_penalty"]:
        r = pen / (1 - pen)                      # compute/transfer ratio implied by the penalty
        assert 0 < r < 1                         # i.e. compute hides behind transfer
        xfer, comp = [1.0] * L, [r] * L
        db = oracle.prefill_pipeline_time(xfer, comp, True)
        sb = oracle.prefill_pipeline_time(xfer, comp, False)
        assert abs(db - (L + r)) < 1e-12 and abs(sb - L * (1 + r)) < 1e-12
        assert abs((1 - db / sb) - pen) < 0.03   # large-L limit of the penalty is r/(1+r)


def test_pipeline_model_bounds():
    rng = np.random.default_rng(5)
    for _ in range(50):
        L = int(rng.integers(1, 10))
        x, c = rng.random(L).tolist(), rng.random(L).tolist()
        db = oracle.prefill_pipeline_time(x, c, True)
        sb = oracle.prefill_pipeline_time(x, c, False)
        assert max(sum(x), sum(c)) - 1e-12 <= db <= sb + 1e-12
        assert abs(sb - sum(x) - sum(c)) < 1e-12
    assert oracle.prefill_pipeline_time([0.0] * 3, [1.0, 2.0, 3.0]) == 6.0
