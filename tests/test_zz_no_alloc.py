"""moe_expert_ffn_merge_noalloc, the decode experts + merge with the library's own scratch
array (for callers that cannot allocate device memory), against moe_expert_ffn_merge with a
caller workspace: bit for bit, on two calls in a row on the same GPU, the second with a smaller
batch (the scratch array keeps the first call's contents), plus the oracle on the first call."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, dev_act, out_f64, rel_err_rows
from test_gpu_parity import GpuLayer, check_route

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from expert_cached_moe_amd import binding
    return binding


def _call_pair(B, G, wl, T, seed, frac):
    """One step: route, then both entry points on the same inputs; returns both outputs and the
    oracle's reference."""
    lg, _ = synth.zipf_reuse_trace(wl, T, 2, tag=seed)
    logits = lg[1]
    G.L.route(torch.from_numpy(np.ascontiguousarray(logits)).cuda(), T)
    ids, gates = check_route(G, logits, T)
    present = sorted(set(ids.ravel().tolist()))
    rng = np.random.default_rng(seed)
    gpu = sorted(rng.permutation(present)[: max(1, int(round(frac * len(present))))].tolist())
    slots = [G.slot[e] for e in gpu]
    ws = 1 if wl.n_shared else 0
    x = synth.activations(wl, T, tag=seed)
    dx = dev_act(x)
    yh = torch.from_numpy(rng.standard_normal(T * wl.H).astype(np.float32)).cuda() if frac < 1 else None
    dt = torch.float32 if wl.act_dtype == "f32" else torch.int16
    want = torch.full((T * wl.H,), 3, dtype=dt, device="cuda")
    got = torch.full((T * wl.H,), 5, dtype=dt, device="cuda")
    G.L.ffn_merge(dx, T, G.pool, gpu, slots, ids, G.shared, ws, yh, want)
    B.moe_expert_ffn_merge_noalloc(G.L.ctx, dx, T, ids, G.L.ids, G.L.w, G.pool, gpu, slots, len(gpu), G.shared, ws,
                                   yh, got, torch.cuda.current_stream())
    torch.cuda.synchronize()
    xf = oracle.act_f64(x, wl.act_dtype)
    ref = oracle.moe_layer(xf, ids, gates, G.ex, shared=G.ex.f64(wl.E) if ws else None, subset=set(gpu))
    if yh is not None:
        ref = ref + yh.cpu().numpy().astype(np.float64).reshape(T, wl.H)
    return want, got, ref


@pytest.mark.parametrize("name,T1,T2", [("a3b_decode_bf16", 8, 2), ("v4flash_mxfp4", 4, 1), ("tiny_fp32", 8, 3)])
def test_noalloc_matches_workspace_entry_point(B, name, T1, T2):
    print(f"[noalloc] {name} T={T1} then T={T2}", flush=True)
    wl = synth.workload(name)
    pool = list(range(wl.E)) if wl.E <= 8 else None
    if pool is None:
        used = set()
        for T, seed in ((T1, 1), (T2, 2)):
            lg, _ = synth.zipf_reuse_trace(wl, T, 2, tag=seed)
            used |= set(oracle.route(lg[1], wl.k)[0].ravel().tolist())
        pool = sorted(used)
    G = GpuLayer(B, wl, pool, max(T1, T2))
    for T, seed, frac in ((T1, 1, 1.0), (T2, 2, 0.5)):
        want, got, ref = _call_pair(B, G, wl, T, seed, frac)
        assert torch.equal(got, want), (name, T)
        err = rel_err_rows(out_f64(got, wl, T), ref).max()
        assert err <= TOL[wl.wdtype], (name, T, err)
    G.L.close()
