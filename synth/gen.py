"""Seeded generators (numpy PCG64, only ``random`` and ``standard_normal``).

Workloads
---------
The shapes are those of the MoE layers the FreeToken pages measure on
(asapai.co.kr "Running 753B GLM-5.2 on a single workstation GPU", sections
"Abandoning fixed offloading in favor of measured bandwidth" and "35B on an 8GB
laptop, 753B on a 96GB workstation"; banandre.com "The 284B Model on a 32GB GPU
Trick", section "Sparsity Is a Lie"), at per-layer sizes:

* ``tiny_fp32``            H=256,  I=128,  E=8,   k=2, fp32, 3 slots
* ``a3b_decode_bf16``      H=2048, I=768,  E=128, k=8, bf16, 47 slots (37 %)
* ``v4flash_decode_bf16``  H=4096, I=1536, E=256 (+1 shared), k=6, bf16, 28 slots (11 %)
* ``a3b_prefill8k_bf16``   T=8192, H=2048, I=768, E=128, k=8, bf16
* ``v4flash_mxfp4``        v4flash shapes with MXFP4 expert weights, decode and
                           an 8192-token prefill chunk

Recipes
-------
* weights: N(0, 0.02) drawn in fp32, stored as the workload's element format
  (fp32; bf16 by round-to-nearest-even; MXFP4 by the OCP MX v1.0 conversion:
  shared exponent floor(log2 amax) - 2 per 32 elements along K, e2m1 values by
  round-to-nearest-even, saturating at 6).  Every expert has its own seed, so
  any subset of a pool can be drawn without drawing the rest.
* activations: N(0, 1), stored in the activation format (fp32 or bf16).
* decode routing: Zipf(s=1.1) expert popularity, each of the previous step's k
  experts of a sequence kept with probability 0.7, the rest sampled without
  replacement in proportion to popularity (Gumbel top-n).  Logits are written
  so that the sampled set is the unique top-k with no ties.
* prefill routing: i.i.d. N(0, 1) logits (near-uniform, every expert is hit).
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "seed_root", "bf16_bits_from_f32",
    "f32_from_bf16_bits", "expert_weights", "shared_expert_weights",
    "activations", "iid_logits", "expert_weights_many", "zipf_reuse_trace", "mxfp4_quantize",
    "router_weights", "trace_stats",
]

W_F32, W_BF16, W_MXFP4 = "f32", "bf16", "mxfp4"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed index: SeedSequence(1000 + index)
    H: int
    I: int
    E: int
    k: int
    n_shared: int
    C: int              # device expert slots of the LRU cache
    wdtype: str
    batches: tuple      # decode batch sizes (tokens per step)
    steps: int          # decode steps per trace
    T: int              # prefill chunk / layer-check tokens

    @property
    def act_dtype(self):
        return W_F32 if self.wdtype == W_F32 else W_BF16


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", 1, 256, 128, 8, 2, 0, 3, W_F32, (1,), 64, 16),
        Workload("a3b_decode_bf16", 2, 2048, 768, 128, 8, 0, 47, W_BF16, (1, 4, 8), 4096, 8),
        Workload("v4flash_decode_bf16", 3, 4096, 1536, 256, 6, 1, 28, W_BF16, (1, 2, 4, 8), 4096, 8),
        Workload("a3b_prefill8k_bf16", 4, 2048, 768, 128, 8, 0, 128, W_BF16, (), 0, 8192),
        Workload("v4flash_mxfp4", 5, 4096, 1536, 256, 6, 1, 28, W_MXFP4, (1, 2, 4, 8), 4096, 8192),
    ]
}

# substream tags
_WEIGHTS, _ACT, _TRACE, _ROUTER, _PREFILL = 0, 1, 2, 3, 4


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def seed_root(wl: Workload) -> int:
    return 1000 + wl.index


def _rng(wl_or_seed, *key) -> np.random.Generator:
    base = seed_root(wl_or_seed) if isinstance(wl_or_seed, Workload) else int(wl_or_seed)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(base, spawn_key=tuple(key))))


# ---------------------------------------------------------------- formats
def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))   # finite inputs: no wrap-around
    return (u >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def mxfp4_quantize(w: np.ndarray):
    """OCP MX v1.0 conversion of fp32 rows [R, K] (K % 32 == 0) to MXFP4.

    Shared exponent X = floor(log2(amax)) - 2 of each block of 32 (from frexp, so
    exact), elements |w| / 2^X rounded to the nearest e2m1 magnitude with ties to
    the even code, saturating at 6.  Returns (codes uint8 [R, K/2] with the even
    element in the low nibble, scales uint8 [R, K/32] = X + 127)."""
    w = np.asarray(w, dtype=np.float32)
    R, K = w.shape
    assert K % 32 == 0
    blk = w.reshape(R, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)                      # amax = m * 2^ex, m in [0.5, 1)
    x = np.where(amax > 0, ex.astype(np.int32) - 1 - 2, -127)
    x = np.clip(x, -127, 127)
    scaled = np.ldexp(np.abs(blk), (-x)[:, :, None])
    idx = np.zeros(scaled.shape, dtype=np.uint8)
    tie_odd = np.zeros(scaled.shape, dtype=bool)
    for i, mid in enumerate(_E2M1_MID):
        idx += scaled > mid
        if i % 2 == 1:
            tie_odd |= scaled == mid
    idx += tie_odd
    idx = np.minimum(idx, 7)
    code = (idx | np.where(np.signbit(blk), np.uint8(8), np.uint8(0))).reshape(R, K)
    codes = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    scales = (x + 127).astype(np.uint8)
    return codes, scales


# ---------------------------------------------------------------- weights
def _draw_expert(wl: Workload, e: int, layer: int = 0):
    # layer 0 keeps the single-layer stream; deeper layers get substreams of their own
    rng = _rng(wl, _WEIGHTS, e) if layer == 0 else _rng(wl, _WEIGHTS, e, layer)
    H, I = wl.H, wl.I
    wg = rng.standard_normal((I, H), dtype=np.float32) * np.float32(0.02)
    wu = rng.standard_normal((I, H), dtype=np.float32) * np.float32(0.02)
    wd = rng.standard_normal((H, I), dtype=np.float32) * np.float32(0.02)
    return wg, wu, wd


def expert_weights(wl: Workload, e: int, layer: int = 0) -> dict:
    """Natural-layout weights of routed expert ``e`` (``e == E`` is the shared one) of MoE
    layer ``layer``.

    Keys: ``wg`` [I,H], ``wu`` [I,H], ``wd`` [H,I] in the storage format
    (float32, or uint16 bf16 bits, or MXFP4 codes) and, for MXFP4, ``sg``,
    ``su``, ``sd`` (e8m0 scales, one per 32 along K)."""
    wg, wu, wd = _draw_expert(wl, e, layer)
    if wl.wdtype == W_F32:
        return {"wg": wg, "wu": wu, "wd": wd}
    if wl.wdtype == W_BF16:
        return {"wg": bf16_bits_from_f32(wg), "wu": bf16_bits_from_f32(wu), "wd": bf16_bits_from_f32(wd)}
    cg, sg = mxfp4_quantize(wg)
    cu, su = mxfp4_quantize(wu)
    cd, sd = mxfp4_quantize(wd)
    return {"wg": cg, "wu": cu, "wd": cd, "sg": sg, "su": su, "sd": sd}


def expert_weights_many(wl: Workload, experts, threads: int = 8, layer: int = 0) -> dict:
    """expert_weights for several experts, drawn on a thread pool (numpy releases the GIL)."""
    import concurrent.futures as cf
    experts = list(experts)
    with cf.ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return dict(zip(experts, ex.map(lambda e: expert_weights(wl, e, layer), experts)))


def shared_expert_weights(wl: Workload):
    return expert_weights(wl, wl.E) if wl.n_shared else None


def router_weights(wl: Workload) -> np.ndarray:
    """Router matrix W_r [H, E], N(0, 0.02) fp32 (tiny layer only)."""
    return _rng(wl, _ROUTER).standard_normal((wl.H, wl.E), dtype=np.float32) * np.float32(0.02)


# ---------------------------------------------------------------- activations / logits
def activations(wl: Workload, T: int, tag: int = 0) -> np.ndarray:
    """x [T, H] ~ N(0, 1) in the activation format (float32 or bf16 bits)."""
    x = _rng(wl, _ACT, tag, T).standard_normal((T, wl.H), dtype=np.float32)
    return x if wl.act_dtype == W_F32 else bf16_bits_from_f32(x)


def iid_logits(wl: Workload, T: int, tag: int = 0) -> np.ndarray:
    """Prefill router logits [T, E] ~ N(0, 1) fp32."""
    return _rng(wl, _PREFILL, tag, T).standard_normal((T, wl.E), dtype=np.float32)


def zipf_reuse_trace(wl: Workload, B: int, n_steps: int | None = None, s: float = 1.1,
                     reuse: float = 0.7, noise: float = 0.1, gap: float = 0.25, tag: int = 0):
    """Decode routing trace: logits [n_steps, B, E] fp32 and the drawn sets [n_steps, B, k].

    Each of B independent sequences keeps each of its previous k experts with
    probability ``reuse``; the remaining picks are drawn without replacement,
    from the experts outside the previous set, with probability proportional to
    the Zipf popularity (Gumbel top-n), so the expected overlap is ``reuse``.  Non-picked
    logits are log-popularity plus ``noise`` N(0,1); picked logits sit above
    the largest non-picked one, spaced by ``gap`` in a random order."""
    n_steps = wl.steps if n_steps is None else n_steps
    E, k = wl.E, wl.k
    rng = _rng(wl, _TRACE, B, tag)
    rank = np.argsort(rng.random(E), kind="stable")          # random rank of each expert
    logp = -s * np.log(rank + 1.0)
    logp -= np.log(np.exp(logp).sum())
    logits = np.empty((n_steps, B, E), dtype=np.float32)
    sets = np.empty((n_steps, B, k), dtype=np.int32)
    prev = None
    for t in range(n_steps):
        u_keep = rng.random((B, k))
        u_gum = rng.random((B, E))
        z = rng.standard_normal((B, E))
        u_ord = rng.random((B, k))
        for b in range(B):
            chosen = np.zeros(E, dtype=bool)
            if prev is not None:
                kept = prev[b][u_keep[b] < reuse]
            else:
                kept = np.empty(0, dtype=np.int64)
            need = k - kept.size
            if need:
                with np.errstate(divide="ignore"):
                    g = logp - np.log(-np.log(u_gum[b]))
                if prev is not None:
                    g[prev[b]] = -np.inf        # dropped experts are not re-drawn: reuse stays at `reuse`
                new = np.argsort(-g, kind="stable")[:need]
                sel = np.concatenate([kept, new])
            else:
                sel = kept
            chosen[sel] = True
            base = (logp + noise * z[b]).astype(np.float32)
            top = base[~chosen].max()
            order = sel[np.argsort(u_ord[b], kind="stable")]
            row = base.copy()
            for r, e in enumerate(order):
                row[e] = np.float32(top + gap * (k - r))
            logits[t, b] = row
            sets[t, b] = sel
        prev = sets[t].astype(np.int64)
    return logits, sets


def trace_stats(sets: np.ndarray, E: int) -> dict:
    """Observed reuse fraction and popularity of a drawn trace (reporting only)."""
    n, B, k = sets.shape
    kept = 0
    for t in range(1, n):
        for b in range(B):
            kept += np.intersect1d(sets[t, b], sets[t - 1, b]).size
    freq = np.bincount(sets.ravel(), minlength=E)
    return {"reuse": kept / max(1, (n - 1) * B * k), "top_decile_share":
            float(np.sort(freq)[::-1][: max(1, E // 10)].sum() / freq.sum())}
