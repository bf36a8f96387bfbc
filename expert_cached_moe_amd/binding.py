"""ctypes binding of libmoecache (include/moe.h): argument marshalling only.

Every function keeps the C name and order of arguments.  Device buffers are
passed as torch tensors (or raw integer addresses), host buffers as numpy arrays
or pinned torch tensors, streams as ``torch.cuda.Stream`` (or an integer
``hipStream_t``; 0 = the null stream).  A non-zero status raises ``MoeError``
carrying ``moe_last_error``.  The library must be built
(``python -m expert_cached_moe_amd.build``); importing fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # noqa: F401  -- load torch's HIP runtime first so the library binds to the same one

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoecache.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m expert_cached_moe_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_ECAPACITY, MOE_EHIP, MOE_EUNSUPPORTED, MOE_ESTATE = 0, -1, -2, -3, -4, -5, -6
MOE_W_F32, MOE_W_BF16, MOE_W_MXFP4 = 0, 1, 2
MOE_Q_NEAREST, MOE_Q_ARGMIN = 0, 1

c_i32p = ctypes.POINTER(ctypes.c_int32)
c_f32p = ctypes.POINTER(ctypes.c_float)
c_u8p = ctypes.POINTER(ctypes.c_uint8)
vp = ctypes.c_void_p

EXPORTS = [
    "moe_create", "moe_destroy", "moe_last_error", "moe_status_string", "moe_expert_bytes",
    "moe_workspace_bytes", "moe_pair_rows", "moe_pack_expert", "moe_bind_pools", "moe_route",
    "moe_qstar", "moe_lru_step", "moe_lru_replay", "moe_lru_reset", "moe_lru_slots", "moe_lru_stats",
    "moe_fill", "moe_fill_wait", "moe_upload", "moe_expert_ffn", "moe_host_ffn", "moe_merge_partial",
    "moe_expert_ffn_merge",
    "moe_prefill_stream", "moe_router_logits", "moe_lru_resize", "moe_move_slots",
    "moe_expert_ffn_merge_noalloc", "moe_noalloc_scratch_bytes",
]


class moe_resize(ctypes.Structure):
    _fields_ = [("cap", ctypes.c_int32), ("n_move", ctypes.c_int32), ("n_evict", ctypes.c_int32),
                ("move_src", ctypes.POINTER(ctypes.c_int32)), ("move_dst", ctypes.POINTER(ctypes.c_int32)),
                ("evicted", ctypes.POINTER(ctypes.c_int32))]


class moe_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("q_round", ctypes.c_int32), ("bp_gbps", ctypes.c_double), ("bh_gbps", ctypes.c_double)]


class moe_plan(ctypes.Structure):
    _fields_ = [("cap", ctypes.c_int32), ("n_distinct", ctypes.c_int32), ("n_hit", ctypes.c_int32),
                ("n_miss", ctypes.c_int32), ("n_fill", ctypes.c_int32), ("n_host", ctypes.c_int32),
                ("layer", ctypes.c_int32), ("distinct", c_i32p), ("hit", c_i32p), ("hit_slot", c_i32p),
                ("fill", c_i32p), ("fill_slot", c_i32p), ("fill_victim", c_i32p), ("host", c_i32p),
                ("slot_of_expert", c_i32p)]


class moe_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("steps", "distinct", "hits", "misses", "fills", "host", "evictions")]


_P = ctypes.POINTER
_sig = {
    "moe_create": (ctypes.c_int, [_P(moe_config), _P(vp)]),
    "moe_destroy": (None, [vp]),
    "moe_last_error": (ctypes.c_char_p, [vp]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_expert_bytes": (ctypes.c_int64, [_P(moe_config)]),
    "moe_workspace_bytes": (ctypes.c_int64, [_P(moe_config), ctypes.c_int32]),
    "moe_pair_rows": (ctypes.c_int64, [_P(moe_config), ctypes.c_int32]),
    "moe_pack_expert": (ctypes.c_int, [_P(moe_config), vp, vp, vp, vp, vp, vp, vp]),
    "moe_bind_pools": (ctypes.c_int, [vp, vp, ctypes.c_int32, vp, ctypes.c_int32]),
    "moe_route": (ctypes.c_int, [vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp]),
    "moe_router_logits": (ctypes.c_int, [vp, vp, ctypes.c_int32, vp, vp, vp]),
    "moe_qstar": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_int32]),
    "moe_lru_step": (ctypes.c_int, [vp, ctypes.c_int32, vp, ctypes.c_int32, _P(moe_plan)]),
    "moe_lru_replay": (ctypes.c_int, [vp, ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32, vp, _P(moe_stats)]),
    "moe_lru_reset": (ctypes.c_int, [vp]),
    "moe_lru_slots": (ctypes.c_int, [vp, ctypes.c_int32, vp]),
    "moe_lru_stats": (ctypes.c_int, [vp, _P(moe_stats)]),
    "moe_lru_resize": (ctypes.c_int, [vp, ctypes.c_int32, _P(moe_resize)]),
    "moe_move_slots": (ctypes.c_int, [vp, _P(moe_resize), vp]),
    "moe_fill": (ctypes.c_int, [vp, _P(moe_plan), vp]),
    "moe_fill_wait": (ctypes.c_int, [vp, vp]),
    "moe_upload": (ctypes.c_int, [vp, vp, vp, ctypes.c_int64, vp]),
    "moe_prefill_stream": (ctypes.c_int, [vp, vp, ctypes.c_int32, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, vp]),
    "moe_expert_ffn": (ctypes.c_int, [vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp,
                                      ctypes.c_int32, vp, vp, vp]),
    "moe_host_ffn": (ctypes.c_int, [vp, vp, ctypes.c_int32, vp, vp, _P(moe_plan), vp, ctypes.c_int32]),
    "moe_merge_partial": (ctypes.c_int, [vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, vp,
                                         ctypes.c_int32, vp, vp]),
    "moe_expert_ffn_merge": (ctypes.c_int, [vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp,
                                            ctypes.c_int32, vp, vp, vp, vp]),
    "moe_expert_ffn_merge_noalloc": (ctypes.c_int, [vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                                    vp, ctypes.c_int32, vp, vp, vp]),
    "moe_noalloc_scratch_bytes": (ctypes.c_int64, []),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_lib.moe_status_string(status).decode()}: {msg}")
        self.status = status


def _ptr(x):
    """Address of a tensor / array / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(ctx, st):
    if st != MOE_OK:
        raise MoeError(st, _lib.moe_last_error(ctx).decode() if ctx else "")
    return st


def make_config(hidden, inter, n_experts, top_k, n_shared=0, n_slots=0, n_layers=1, w_dtype=MOE_W_BF16,
                renormalize=1, q_round=MOE_Q_NEAREST, bp_gbps=52.7, bh_gbps=77.3) -> moe_config:
    return moe_config(hidden, inter, n_experts, top_k, n_shared, n_slots, n_layers, w_dtype, renormalize,
                      q_round, bp_gbps, bh_gbps)


# ------------------------------------------------------------------ entry points (C names)
def moe_create(cfg: moe_config) -> int:
    out = vp()
    st = _lib.moe_create(ctypes.byref(cfg), ctypes.byref(out))
    if st != MOE_OK:
        raise MoeError(st, "moe_create")
    return out.value


def moe_destroy(ctx: int) -> None:
    _lib.moe_destroy(ctx)


def moe_last_error(ctx: int) -> str:
    return _lib.moe_last_error(ctx).decode()


def moe_status_string(st: int) -> str:
    return _lib.moe_status_string(st).decode()


def moe_expert_bytes(cfg: moe_config) -> int:
    v = _lib.moe_expert_bytes(ctypes.byref(cfg))
    if v < 0:
        raise MoeError(int(v), "moe_expert_bytes")
    return v


def moe_workspace_bytes(cfg: moe_config, max_T: int) -> int:
    v = _lib.moe_workspace_bytes(ctypes.byref(cfg), max_T)
    if v < 0:
        raise MoeError(int(v), "moe_workspace_bytes")
    return v


def moe_pair_rows(cfg: moe_config, T: int) -> int:
    v = _lib.moe_pair_rows(ctypes.byref(cfg), T)
    if v < 0:
        raise MoeError(int(v), "moe_pair_rows")
    return v


def moe_pack_expert(cfg, wg, wu, wd, sg, su, sd, blob) -> None:
    arrs = [np.ascontiguousarray(a) if a is not None else None for a in (wg, wu, wd, sg, su, sd)]
    st = _lib.moe_pack_expert(ctypes.byref(cfg), *[_ptr(a) for a in arrs], _ptr(blob))
    if st != MOE_OK:
        raise MoeError(st, "moe_pack_expert")


def moe_bind_pools(ctx, d_slots, n_slots, h_pool, n_pool) -> None:
    _check(ctx, _lib.moe_bind_pools(ctx, _ptr(d_slots), n_slots, _ptr(h_pool), n_pool))


def moe_router_logits(ctx, d_x, T, d_wr, d_logits, s=None) -> None:
    _check(ctx, _lib.moe_router_logits(ctx, _ptr(d_x), T, _ptr(d_wr), _ptr(d_logits), _stream(s)))


def moe_route(ctx, d_logits, T, d_topk_ids, d_topk_w, d_counts, d_offsets, d_perm, d_inv, d_ws, s=None) -> None:
    _check(ctx, _lib.moe_route(ctx, _ptr(d_logits), T, _ptr(d_topk_ids), _ptr(d_topk_w), _ptr(d_counts),
                               _ptr(d_offsets), _ptr(d_perm), _ptr(d_inv), _ptr(d_ws), _stream(s)))


def moe_qstar(m, bp, bh, rounding=MOE_Q_NEAREST) -> int:
    return _lib.moe_qstar(m, bp, bh, rounding)


class Plan:
    """Host arrays of one decode-step plan and the moe_plan struct pointing at them."""

    FIELDS = ("distinct", "hit", "hit_slot", "fill", "fill_slot", "fill_victim", "host")

    def __init__(self, cap: int, n_experts: int):
        self.arrays = {f: np.zeros(cap, np.int32) for f in self.FIELDS}
        self.arrays["slot_of_expert"] = np.zeros(n_experts, np.int32)
        self.c = moe_plan(cap, 0, 0, 0, 0, 0, 0,
                          *[self.arrays[f].ctypes.data_as(c_i32p) for f in self.FIELDS + ("slot_of_expert",)])

    def get(self, f):
        n = {"distinct": self.c.n_distinct, "hit": self.c.n_hit, "hit_slot": self.c.n_hit,
             "fill": self.c.n_fill, "fill_slot": self.c.n_fill, "fill_victim": self.c.n_fill,
             "host": self.c.n_host}
        return self.arrays[f] if f == "slot_of_expert" else self.arrays[f][: n[f]]


def moe_lru_step(ctx, layer, h_topk_ids, T, plan: Plan) -> None:
    ids = np.ascontiguousarray(h_topk_ids, dtype=np.int32)
    _check(ctx, _lib.moe_lru_step(ctx, layer, _ptr(ids), T, ctypes.byref(plan.c)))


def moe_lru_replay(ctx, layer, h_topk_ids, n_steps, T, plans=None) -> moe_stats:
    """plans: None or a list of n_steps Plan objects."""
    ids = np.ascontiguousarray(h_topk_ids, dtype=np.int32)
    st = moe_stats()
    arr = None
    if plans is not None:
        arr = (moe_plan * n_steps)(*[p.c for p in plans])
    _check(ctx, _lib.moe_lru_replay(ctx, layer, _ptr(ids), n_steps, T,
                                    ctypes.cast(arr, vp) if arr is not None else None, ctypes.byref(st)))
    if plans is not None:                       # copy the counts back into the Plan structs
        for p, c in zip(plans, arr):
            p.c = c
    return st


def moe_lru_reset(ctx) -> None:
    _check(ctx, _lib.moe_lru_reset(ctx))


def moe_lru_slots(ctx, layer, n_experts) -> np.ndarray:
    out = np.zeros(n_experts, np.int32)
    _check(ctx, _lib.moe_lru_slots(ctx, layer, _ptr(out)))
    return out


def moe_lru_stats(ctx) -> moe_stats:
    st = moe_stats()
    _check(ctx, _lib.moe_lru_stats(ctx, ctypes.byref(st)))
    return st


class Resize:
    """Host arrays of a cache resize and the moe_resize struct pointing at them."""

    def __init__(self, cap: int):
        self.arrays = {f: np.zeros(max(cap, 1), np.int32) for f in ("move_src", "move_dst", "evicted")}
        c_i32p = ctypes.POINTER(ctypes.c_int32)
        self.c = moe_resize(cap, 0, 0, *[self.arrays[f].ctypes.data_as(c_i32p) for f in ("move_src", "move_dst",
                                                                                         "evicted")])

    def moves(self):
        n = self.c.n_move
        return list(zip(self.arrays["move_src"][:n].tolist(), self.arrays["move_dst"][:n].tolist()))

    def evicted(self):
        return self.arrays["evicted"][: self.c.n_evict].tolist()


def moe_lru_resize(ctx, new_slots, r: Resize) -> None:
    _check(ctx, _lib.moe_lru_resize(ctx, new_slots, ctypes.byref(r.c)))


def moe_move_slots(ctx, r: Resize, s=None) -> None:
    _check(ctx, _lib.moe_move_slots(ctx, ctypes.byref(r.c), _stream(s)))


def moe_fill(ctx, plan: Plan, side=None) -> None:
    _check(ctx, _lib.moe_fill(ctx, ctypes.byref(plan.c), _stream(side)))


def moe_fill_wait(ctx, s=None) -> None:
    _check(ctx, _lib.moe_fill_wait(ctx, _stream(s)))


def moe_upload(ctx, d_dst, h_src, nbytes, side=None) -> None:
    _check(ctx, _lib.moe_upload(ctx, _ptr(d_dst), _ptr(h_src), nbytes, _stream(side)))


def moe_expert_ffn(ctx, d_x, T, h_topk_ids, d_offsets, d_perm, d_slot_base, h_experts, h_slots, n, d_shared,
                   with_shared, d_o, d_ws, s=None) -> None:
    he = np.ascontiguousarray(h_experts, dtype=np.int32) if h_experts is not None else None
    hs = np.ascontiguousarray(h_slots, dtype=np.int32) if h_slots is not None else None
    hi = h_topk_ids
    if isinstance(hi, np.ndarray):
        hi = np.ascontiguousarray(hi, dtype=np.int32)
    _check(ctx, _lib.moe_expert_ffn(ctx, _ptr(d_x), T, _ptr(hi), _ptr(d_offsets), _ptr(d_perm), _ptr(d_slot_base),
                                    _ptr(he), _ptr(hs), n, _ptr(d_shared), with_shared, _ptr(d_o), _ptr(d_ws),
                                    _stream(s)))


def moe_host_ffn(ctx, h_x, T, h_topk_ids, h_topk_w, plan: Plan, h_y, n_threads=0) -> None:
    _check(ctx, _lib.moe_host_ffn(ctx, _ptr(h_x), T, _ptr(h_topk_ids), _ptr(h_topk_w), ctypes.byref(plan.c),
                                  _ptr(h_y), n_threads))


def moe_merge_partial(ctx, d_o, d_topk_ids, d_topk_w, h_gpu_experts, n_gpu, with_shared, d_y_host, T, d_out,
                      s=None) -> None:
    ge = np.ascontiguousarray(h_gpu_experts, dtype=np.int32) if h_gpu_experts is not None else None
    _check(ctx, _lib.moe_merge_partial(ctx, _ptr(d_o), _ptr(d_topk_ids), _ptr(d_topk_w), _ptr(ge), n_gpu,
                                       with_shared, _ptr(d_y_host), T, _ptr(d_out), _stream(s)))


def moe_expert_ffn_merge(ctx, d_x, T, h_topk_ids, d_topk_ids, d_topk_w, d_slot_base, h_experts, h_slots, n,
                         d_shared, with_shared, d_y_host, d_out, d_ws, s=None) -> None:
    he = np.ascontiguousarray(h_experts, dtype=np.int32) if h_experts is not None else None
    hs = np.ascontiguousarray(h_slots, dtype=np.int32) if h_slots is not None else None
    hi = h_topk_ids
    if isinstance(hi, np.ndarray):
        hi = np.ascontiguousarray(hi, dtype=np.int32)
    _check(ctx, _lib.moe_expert_ffn_merge(ctx, _ptr(d_x), T, _ptr(hi), _ptr(d_topk_ids), _ptr(d_topk_w),
                                          _ptr(d_slot_base), _ptr(he), _ptr(hs), n, _ptr(d_shared), with_shared,
                                          _ptr(d_y_host), _ptr(d_out), _ptr(d_ws), _stream(s)))


def moe_expert_ffn_merge_noalloc(ctx, d_x, T, h_topk_ids, d_topk_ids, d_topk_w, d_slot_base, h_experts, h_slots, n,
                                 d_shared, with_shared, d_y_host, d_out, s=None) -> None:
    he = np.ascontiguousarray(h_experts, dtype=np.int32) if h_experts is not None else None
    hs = np.ascontiguousarray(h_slots, dtype=np.int32) if h_slots is not None else None
    hi = h_topk_ids
    if isinstance(hi, np.ndarray):
        hi = np.ascontiguousarray(hi, dtype=np.int32)
    _check(ctx, _lib.moe_expert_ffn_merge_noalloc(ctx, _ptr(d_x), T, _ptr(hi), _ptr(d_topk_ids), _ptr(d_topk_w),
                                                  _ptr(d_slot_base), _ptr(he), _ptr(hs), n, _ptr(d_shared),
                                                  with_shared, _ptr(d_y_host), _ptr(d_out), _stream(s)))


def moe_noalloc_scratch_bytes() -> int:
    return int(_lib.moe_noalloc_scratch_bytes())


def moe_prefill_stream(ctx, d_layer_bufs, n_buffers, d_logits, d_x, T, d_shared, d_topk_ids, d_topk_w, d_counts,
                       d_offsets, d_perm, d_inv, d_o, d_ws, d_out, s=None, side=None) -> None:
    _check(ctx, _lib.moe_prefill_stream(ctx, _ptr(d_layer_bufs), n_buffers, _ptr(d_logits), _ptr(d_x), T,
                                        _ptr(d_shared), _ptr(d_topk_ids), _ptr(d_topk_w), _ptr(d_counts),
                                        _ptr(d_offsets), _ptr(d_perm), _ptr(d_inv), _ptr(d_o), _ptr(d_ws),
                                        _ptr(d_out), _stream(s), _stream(side)))


def exported_symbols() -> list:
    """Names of include/moe.h entry points found in the loaded library."""
    return [n for n in EXPORTS if hasattr(_lib, n)]
