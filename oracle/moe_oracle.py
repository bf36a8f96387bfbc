"""Oracle: one MoE layer over a slot-limited expert cache, in fp64 on the CPU.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run this module.  It shares no
code, table or constant with the HIP library: inputs reach both sides from the
``synth`` generators and from nowhere else.

Sources (the FreeToken pages):
  [A] asapai.co.kr, "Running 753B GLM-5.2 on a single workstation GPU: FreeToken
      doubles llama.cpp's throughput"
  [B] banandre.com, "The 284B Model on a 32GB GPU Trick: How FreeToken Proves
      Hardware Is a Software Problem"
  [Z] zubnet.ai, news item on FreeToken and Unsloth GGUF (formats, mechanisms)

What the layer computes.  A router picks a few experts per token ([B] "Sparsity
Is a Lie"); each expert is a small feed-forward network.  On a cache miss the
scheduler either copies the expert to the GPU or computes it on the CPU, with
q* ~= m*B_P/B_H of the m misses filled ([B] "The q* Policy"); the GPU and CPU
partial sums are added after the layer and the result is exactly the plain
layer output, with no approximation ([B] "The q* Policy").  The decode cache is
one LRU updated on misses ([A] "Abandoning fixed offloading ..."; [B]
"Semantic-Aware Caching"), and it starts empty ([B] "Elastic Memory").

Readings taken where the pages leave a step open (the pages name none of these):
  * expert = SwiGLU without biases: Wd (silu(Wg x) * (Wu x)), silu(z) = z/(1+e^-z);
  * router = softmax over the logits, top-k by (logit descending, expert id
    ascending), gates renormalised over the k (``renormalize=False`` keeps the
    softmax over all experts);
  * the always-on shared expert has gate 1, lives outside the cache and is a
    GPU expert;
  * q = floor(m*B_P/B_H + 1/2) computed in IEEE double in that operation order,
    clamped to [0, m] and to the slots not holding a hit (C - h);
  * the experts of a step are taken in "step order": more tokens first, then
    lower id; the first q misses in step order are filled, the rest go to the CPU
    and are not inserted into the cache;
  * recency key of an expert used in a step = (step counter, n - rank), rank in
    step order, larger = more recent; a fill takes the lowest free slot, else the
    slot of the resident with the smallest key that is not used in this step;
  * miss rate = misses / distinct (expert, step) reads.

Pins (tests/test_oracle_pins.py, tests/golden/): dense brute force over all
experts, closed-form special cases, subset brute force for top-k, the
partition invariant, the q* table and its makespan derivation, the Mattson
stack-distance algorithm for the LRU, hand-worked LRU traces, the OCP MX e2m1
table, and the pages' worked prefill arithmetic.  The pages' measured miss rates
(16 % / 39 %) stay unpinned: their routing traces are not published.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "round_to_bf16", "mxfp4_decode", "expert_f64", "act_f64",
    "router_logits", "route", "permute", "silu", "expert_ffn", "moe_layer",
    "moe_layer_partitioned", "qstar", "step_order", "LRUCache", "mattson_misses",
    "stream_time", "prefill_pipeline_time", "E2M1_VALUES",
]


# ------------------------------------------------------------------ element formats
def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64 values: the 16 bits are the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """fp64 -> nearest fp32 -> nearest-even bf16, returned as fp64 (optional mirror of GPU h rounding)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# OCP Microscaling Formats (MX) v1.0: FP4 E2M1 magnitudes by the 3 low code bits.
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def mxfp4_decode(codes, scales) -> np.ndarray:
    """MXFP4 rows -> fp64.  The pages list MXFP4 among the weight formats ([Z]); the
    element rule is OCP MX v1.0: value = (-1)^s * e2m1(c) * 2^(X - 127), one e8m0
    X per 32 consecutive elements along K; element 2i sits in the low nibble of
    byte i.  X = 255 (NaN) is rejected."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if np.any(scales == 255):
        raise ValueError("e8m0 scale 0xFF is NaN")
    R, half = codes.shape
    K = 2 * half
    nib = np.empty((R, K), dtype=np.uint8)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    mag = np.asarray(E2M1_VALUES, dtype=np.float64)[nib & 7]
    sign = np.where(nib & 8, -1.0, 1.0)
    scale = np.exp2(scales.astype(np.float64) - 127.0)
    return sign * mag * np.repeat(scale, 32, axis=1)


def expert_f64(w: dict, wdtype: str):
    """(Wg [I,H], Wu [I,H], Wd [H,I]) in fp64 from the stored format ('f32'|'bf16'|'mxfp4')."""
    if wdtype == "f32":
        return tuple(np.asarray(w[n], dtype=np.float64) for n in ("wg", "wu", "wd"))
    if wdtype == "bf16":
        return tuple(bf16_bits_to_f64(w[n]) for n in ("wg", "wu", "wd"))
    if wdtype == "mxfp4":
        return (mxfp4_decode(w["wg"], w["sg"]), mxfp4_decode(w["wu"], w["su"]),
                mxfp4_decode(w["wd"], w["sd"]))
    raise ValueError(wdtype)


def act_f64(x, act_dtype: str) -> np.ndarray:
    return np.asarray(x, dtype=np.float64) if act_dtype == "f32" else bf16_bits_to_f64(x)


# ------------------------------------------------------------------ router
def router_logits(x, wr) -> np.ndarray:
    """l = x . W_r in fp64, rounded once to fp32 (the tiny layer's routing input)."""
    return (np.asarray(x, np.float64) @ np.asarray(wr, np.float64)).astype(np.float32)


def route(logits, k: int, renormalize: bool = True):
    """Top-k experts per token and their gates ([B] "Sparsity Is a Lie": a small router
    picks a handful of experts per token).

    Order: logit descending, expert id ascending on equal logits.  Gates: softmax
    in fp64, renormalised over the selected k (or over all experts).
    Returns (ids int32 [T,k], gates fp64 [T,k])."""
    l = np.asarray(logits, dtype=np.float32)
    if not np.all(np.isfinite(l)):
        raise ValueError("router logits must be finite")
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-l, axis=1, kind="stable")       # stable: equal logits keep id order
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l, order[:, :k], axis=1).astype(np.float64)
    if renormalize:
        ex = np.exp(sel - sel[:, :1])
        gates = ex / ex.sum(axis=1, keepdims=True)
    else:
        lf = l.astype(np.float64)
        mx = lf.max(axis=1, keepdims=True)
        gates = np.exp(sel - mx) / np.exp(lf - mx).sum(axis=1, keepdims=True)
    return ids, gates


def permute(ids, E: int):
    """Token-by-expert grouping: stable counting sort of the pairs p = t*k + j by expert.

    Returns counts [E], offsets [E+1] (exclusive prefix sum), perm [T*k] (pair
    indices grouped by expert, ascending p inside a group) and inv (inv[perm[i]] = i)."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    np.cumsum(counts, out=offsets[1:])
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return counts, offsets, perm, inv


# ------------------------------------------------------------------ experts and layer
def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(W, x, round_h: bool = False) -> np.ndarray:
    """SwiGLU expert on rows x [n, H]: Wd (silu(Wg x) * (Wu x)), fp64 throughout."""
    wg, wu, wd = W
    x = np.asarray(x, dtype=np.float64)
    h = silu(x @ wg.T) * (x @ wu.T)
    if round_h:
        h = round_to_bf16(h)
    return h @ wd.T


def moe_layer(x, ids, gates, experts, shared=None, subset=None, round_h=False) -> np.ndarray:
    """y_t = sum_j g_tj FFN_{e_tj}(x_t) [+ FFN_shared(x_t)] in fp64, by sparse dispatch.

    ``experts`` maps an expert id to its fp64 (Wg, Wu, Wd) (a dict or a callable);
    ``subset`` restricts the routed sum to a set of experts (a partition part)."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    T = x.shape[0]
    H = x.shape[1]
    y = np.zeros((T, H), dtype=np.float64)
    get = experts if callable(experts) else experts.__getitem__
    for e in np.unique(ids):
        if subset is not None and int(e) not in subset:
            continue
        t, j = np.nonzero(ids == e)
        y[t] += gates[t, j][:, None] * expert_ffn(get(int(e)), x[t], round_h)
    if shared is not None:
        y += expert_ffn(shared, x, round_h)
    return y


def moe_layer_partitioned(x, ids, gates, experts, cache_set, shared=None, round_h=False):
    """The two partial sums of [B] "The q* Policy": GPU part (cache experts + shared)
    and CPU part (the remaining routed experts).  Their sum is the layer output."""
    ids = np.asarray(ids)
    cache_set = set(int(e) for e in cache_set)
    host_set = set(int(e) for e in np.unique(ids)) - cache_set
    y_cache = moe_layer(x, ids, gates, experts, shared, subset=cache_set, round_h=round_h)
    y_host = moe_layer(x, ids, gates, experts, None, subset=host_set, round_h=round_h)
    return y_cache, y_host


# ------------------------------------------------------------------ q* split
def qstar(m: int, bp: float, bh: float, rounding: str = "nearest") -> int:
    """Number of the m misses to fill into the GPU cache ([B] "The q* Policy").

    DMA and CPU expert reads share the host memory, so with the link saturated
    the CPU keeps B_H - B_P; q* ~= m*B_P/B_H.  'nearest': floor(m*B_P/B_H + 1/2)
    in double, clamped to [0, m].  'argmin': the integer q minimising
    max(q/B_P, (m - q)/(B_H - B_P)), ties to the smaller q.  With B_H <= B_P the
    CPU has no residual bandwidth and every miss is filled."""
    if m <= 0:
        return 0
    if bh <= bp:
        return m
    if rounding == "nearest":
        q = int(np.floor(float(m) * bp / bh + 0.5))
        return max(0, min(m, q))
    if rounding == "argmin":
        best, bq = None, 0
        for q in range(m + 1):
            c = max(q / bp, (m - q) / (bh - bp))
            if best is None or c < best:
                best, bq = c, q
        return bq
    raise ValueError(rounding)


# ------------------------------------------------------------------ global LRU
def step_order(step_ids) -> list:
    """Distinct experts of one decode step, more tokens first, then lower id."""
    flat = np.asarray(step_ids, dtype=np.int64).ravel()
    vals, cnt = np.unique(flat, return_counts=True)
    order = sorted(range(len(vals)), key=lambda i: (-cnt[i], vals[i]))
    return [int(vals[i]) for i in order]


class LRUCache:
    """Slot cache shared by all MoE layers, keyed by (layer, expert), updated on
    every filled miss; it starts empty ([A] "Abandoning fixed offloading ...",
    [B] "Semantic-Aware Caching", [B] "Elastic Memory").  Plain Python lists."""

    def __init__(self, n_slots: int, n_experts: int, n_layers: int = 1):
        self.C = int(n_slots)
        self.E = int(n_experts)
        self.L = int(n_layers)
        self.key_of_slot = [-1] * self.C          # cache key (layer*E + e) held by a slot
        self.recency = [None] * self.C            # (step counter, n - rank)
        self.counter = 0

    def slot_of(self, key: int) -> int:
        for s in range(self.C):
            if self.key_of_slot[s] == key:
                return s
        return -1

    def slot_table(self, layer: int = 0) -> np.ndarray:
        tab = np.full(self.E, -1, dtype=np.int32)
        for s, key in enumerate(self.key_of_slot):
            if key >= 0 and key // self.E == layer:
                tab[key % self.E] = s
        return tab

    def step(self, step_ids, bp: float, bh: float, rounding: str = "nearest", layer: int = 0) -> dict:
        S = step_order(step_ids)
        keys = [layer * self.E + e for e in S]
        n = len(S)
        hit = [e for e, key in zip(S, keys) if self.slot_of(key) >= 0]
        miss = [e for e, key in zip(S, keys) if self.slot_of(key) < 0]
        m = len(miss)
        q = min(qstar(m, bp, bh, rounding), self.C - len(hit))
        fill, host = miss[:q], miss[q:]
        self.counter += 1
        rank = {e: r for r, e in enumerate(S)}
        in_step = set(keys)
        hit_slot = []
        for e in hit:
            s = self.slot_of(layer * self.E + e)
            self.recency[s] = (self.counter, n - rank[e])
            hit_slot.append(s)
        fill_slot, fill_victim = [], []
        for e in fill:
            free = [s for s in range(self.C) if self.key_of_slot[s] < 0]
            if free:
                s, victim = free[0], -1
            else:
                cands = [s for s in range(self.C) if self.key_of_slot[s] not in in_step]
                s = min(cands, key=lambda c: self.recency[c])
                victim = self.key_of_slot[s]
            self.key_of_slot[s] = layer * self.E + e
            self.recency[s] = (self.counter, n - rank[e])
            fill_slot.append(s)
            fill_victim.append(victim)
        return {"distinct": S, "hit": hit, "hit_slot": hit_slot, "fill": fill,
                "fill_slot": fill_slot, "fill_victim": fill_victim, "host": host,
                "m": m, "q": q, "slot_of_expert": self.slot_table(layer)}

    def resize(self, new_C: int) -> dict:
        """Rebuild the cache under a new slot count at a safe point, keeping the host pool
        ([B] "Elastic Memory").  Shrinking keeps the new_C most recently used entries and
        drops the rest; a kept entry whose slot no longer exists takes the lowest free slot
        (sources in ascending slot order).  Growing keeps every entry and adds free slots."""
        new_C = int(new_C)
        moves, evicted = [], []
        if new_C < self.C:
            resident = [s for s in range(self.C) if self.key_of_slot[s] >= 0]
            newest_first = sorted(resident, key=lambda s: self.recency[s], reverse=True)
            kept = set(newest_first[:new_C])
            evicted = [self.key_of_slot[s] for s in resident if s not in kept]
            for s in resident:
                if s not in kept:
                    self.key_of_slot[s] = -1
                    self.recency[s] = None
            free = [s for s in range(new_C) if s not in kept]
            for src in sorted(s for s in kept if s >= new_C):
                dst = free.pop(0)
                self.key_of_slot[dst], self.recency[dst] = self.key_of_slot[src], self.recency[src]
                self.key_of_slot[src], self.recency[src] = -1, None
                moves.append((src, dst))
            self.key_of_slot = self.key_of_slot[:new_C]
            self.recency = self.recency[:new_C]
        else:
            self.key_of_slot += [-1] * (new_C - self.C)
            self.recency += [None] * (new_C - self.C)
        self.C = new_C
        return {"moves": moves, "evicted": evicted}


def mattson_misses(step_sets, max_C: int) -> np.ndarray:
    """Stack-distance pass (Mattson et al., 1970): misses of an LRU cache of every
    size C = 0..max_C in one pass over a trace of per-step expert lists in step
    order.  A reference misses at size C iff its depth in the recency stack before
    the step is >= C.  Equals the slot cache's misses when every miss is filled and
    C is at least the largest step."""
    stack: list = []
    misses = np.zeros(max_C + 1, dtype=np.int64)
    for S in step_sets:
        for e in S:
            d = stack.index(e) if e in stack else max_C + 1
            misses[: min(d, max_C) + 1] += 1          # a miss for every C <= d
        stack = list(S) + [e for e in stack if e not in set(S)]
    return misses


# ------------------------------------------------------------------ prefill stream model
def stream_time(pool_bytes: float, bp_bytes_per_s: float) -> float:
    """Time to stream an expert pool once over the host link ([A] "Abandoning fixed
    offloading ...": an 8,192-token chunk takes the time of one pool stream)."""
    return pool_bytes / bp_bytes_per_s


def prefill_pipeline_time(xfer, compute, double_buffer: bool = True) -> float:
    """Makespan of streaming layer weights and computing layers in order.

    With two buffers the upload of layer l+1 overlaps the compute of layer l and
    may start once the compute of layer l-1 has freed its buffer ([A]
    "Abandoning fixed offloading ...", [B] "Semantic-Aware Caching"); with one
    buffer each upload waits for the previous layer's compute."""
    x_end, c_end = [], []
    for l, (x, c) in enumerate(zip(xfer, compute)):
        if double_buffer:
            start = max(x_end[l - 1] if l >= 1 else 0.0, c_end[l - 2] if l >= 2 else 0.0)
        else:
            start = c_end[l - 1] if l >= 1 else 0.0
        x_end.append(start + x)
        c_end.append(max(c_end[l - 1] if l >= 1 else 0.0, x_end[l]) + c)
    return c_end[-1] if c_end else 0.0
