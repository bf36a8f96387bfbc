"""Shared plumbing for the tests: workload configs and synthetic inputs for both sides."""
import numpy as np

import oracle
import synth

DT = {"f32": 0, "bf16": 1, "mxfp4": 2}
TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp4": 2e-2}


def config(wl, n_slots=None, bp=52.7, bh=77.3, n_layers=1, q_round=0, renormalize=1):
    from expert_cached_moe_amd import binding as B
    return B.make_config(wl.H, wl.I, wl.E, wl.k, wl.n_shared, wl.C if n_slots is None else n_slots, n_layers,
                         DT[wl.wdtype], renormalize, q_round, bp, bh)


class Experts:
    """Lazily drawn expert weights of one MoE layer of a workload (natural layout and fp64 for the oracle)."""

    def __init__(self, wl, layer=0):
        self.wl = wl
        self.layer = layer
        self._raw = {}
        self._f64 = {}

    def prefetch(self, es, threads=8):
        need = [e for e in es if e not in self._raw]
        if need:
            self._raw.update(synth.expert_weights_many(self.wl, need, threads, layer=self.layer))

    def raw(self, e):
        if e not in self._raw:
            self._raw[e] = synth.expert_weights(self.wl, e, layer=self.layer)
        return self._raw[e]

    def f64(self, e):
        if e not in self._f64:
            self._f64[e] = oracle.expert_f64(self.raw(e), self.wl.wdtype)
        return self._f64[e]

    def __call__(self, e):
        return self.f64(e)


def rel_err_rows(y, ref):
    """Per-token max_i |y - ref| / max_i |ref| (rows of ref that are all zero must match exactly)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max(axis=1)
    num = np.abs(y - ref).max(axis=1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return out


def step_ids(logits_step, k):
    ids, gates = oracle.route(logits_step, k)
    return ids, gates


def dev_act(x):
    """Activations to the device: fp32 as is, bf16 bits as int16 storage."""
    import torch
    if x.dtype == np.float32:
        return torch.from_numpy(x).cuda()
    return torch.from_numpy(x.view(np.int16)).cuda()


def out_f64(t, wl, T):
    """Layer output tensor (fp32, or bf16 bits in int16 storage) as fp64 [T][H]."""
    a = t.cpu().numpy()
    if wl.act_dtype == "f32":
        return a.reshape(T, wl.H).astype(np.float64)
    return oracle.bf16_bits_to_f64(a.view(np.uint16)).reshape(T, wl.H)
