"""GPU parity at the edges of the method's input space, through the C ABI.

- routing at the largest supported sizes (512 experts, top-16) on all three kernel paths;
- a prefill batch whose expert list includes experts no token chose (zero-row groups);
- decode batches where every token picks the same experts, and where no two tokens share one;
- a streamed prefill chunk of zero tokens.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, config, dev_act, out_f64, rel_err_rows
from test_gpu_parity import GpuLayer, _route_case, check_route

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from expert_cached_moe_amd import binding
    return binding


@pytest.mark.parametrize("T", [2, 200, 1000])
def test_route_max_experts_and_k(B, T):
    """E = 512, k = 16: T = 2 takes the one-wave path (32 pairs), T = 200 the single-
    workgroup path (3,200 pairs), T = 1000 the multi-kernel path (16,000 pairs)."""
    print(f"[route-max] E=512 k=16 T={T}", flush=True)
    wl = dataclasses.replace(synth.workload("tiny_fp32"), name="e512_k16", E=512, k=16)
    logits = synth.iid_logits(wl, T, tag=T)
    logits[:, ::7] = np.round(logits[:, ::7], 1)          # many exact ties
    _route_case(B, wl, logits)


def test_prefill_listed_experts_without_tokens(B):
    """Every expert listed, most of them with no token at T = 24: zero-row groups add no
    tiles and leave the output unchanged."""
    wl = synth.workload("a3b_prefill8k_bf16")
    T = 24
    logits = synth.iid_logits(wl, T, tag=77)
    ids, _ = oracle.route(logits, wl.k)
    allx = list(range(wl.E))
    G = GpuLayer(B, wl, allx, T)
    x = synth.activations(wl, T, tag=77)
    out = G.run(logits, x, allx, 0)
    ids, gates = check_route(G, logits, T)
    y = out_f64(out, wl, T)
    ref = oracle.moe_layer(oracle.act_f64(x, wl.act_dtype), ids, gates, G.ex)
    assert rel_err_rows(y, ref).max() <= TOL[wl.wdtype]
    assert len(set(ids.ravel().tolist())) < wl.E                # some listed experts had no token
    G.L.close()


@pytest.mark.parametrize("name,mode", [("a3b_decode_bf16", "same"), ("a3b_decode_bf16", "disjoint"),
                                       ("v4flash_mxfp4", "same"), ("tiny_fp32", "disjoint")])
def test_decode_overlap_extremes(B, name, mode):
    """T = 8 (fp32 tiny: T = 4): all tokens on the same k experts (each expert sees every
    token), or on pairwise disjoint ones (every expert sees one token)."""
    wl = synth.workload(name)
    T = 8 if wl.E >= 8 * wl.k else 4
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((T, wl.E)).astype(np.float32)
    if mode == "same":
        top = rng.choice(wl.E, wl.k, replace=False)
        logits[:, top] += 20.0 + np.arange(wl.k, dtype=np.float32)
    else:
        perm = rng.permutation(wl.E)
        for t in range(T):
            logits[t, perm[t * wl.k:(t + 1) * wl.k]] += 20.0 + np.arange(wl.k, dtype=np.float32)
    ids, _ = oracle.route(logits, wl.k)
    present = sorted(set(ids.ravel().tolist()))
    assert len(present) == (wl.k if mode == "same" else T * wl.k)
    G = GpuLayer(B, wl, present, T)
    x = synth.activations(wl, T, tag=5)
    ws = 1 if wl.n_shared else 0
    out = G.run(logits, x, present, ws)
    ids, gates = check_route(G, logits, T)
    y = out_f64(out, wl, T)
    ref = oracle.moe_layer(oracle.act_f64(x, wl.act_dtype), ids, gates, G.ex, shared=G.ex.f64(wl.E) if ws else None)
    assert rel_err_rows(y, ref).max() <= TOL[wl.wdtype]
    G.L.close()


@pytest.mark.parametrize("T", [1, 8])
def test_decode_lists_every_expert(B, T):
    """The caller lists all 512 experts of a layer (every one resident) for a decode batch of
    top-16 routing: only experts some token uses are computed (at most T * k = 128 of them),
    the listed experts without a token add nothing and their pair rows stay unwritten; the
    one-call path (experts + merge) is bit-identical to the two calls."""
    print(f"[decode-every-expert] E=512 k=16 T={T}", flush=True)
    from test_gpu_parity import pair_rows_written
    base = synth.workload("a3b_decode_bf16")
    wl = dataclasses.replace(base, name="bf16_512x256_e512_k16", H=512, I=256, E=512, k=16, C=512)
    logits = synth.iid_logits(wl, T, tag=40 + T)
    allx = list(range(wl.E))
    G = GpuLayer(B, wl, allx, T)
    x = synth.activations(wl, T, tag=40 + T)
    out = G.run(logits, x, allx, 0)
    ids, gates = check_route(G, logits, T)
    o = pair_rows_written(G, T, ids, set(allx), 0)
    y = out_f64(out, wl, T)
    xf = oracle.act_f64(x, wl.act_dtype)
    ref = oracle.moe_layer(xf, ids, gates, G.ex)
    assert rel_err_rows(y, ref).max() <= TOL[wl.wdtype]
    assert np.isfinite(o).all()
    dx = dev_act(x)
    one = torch.full_like(out, 7)
    G.L.ffn_merge(dx, T, G.pool, allx, allx, ids, None, 0, None, one)
    torch.cuda.synchronize()
    assert torch.equal(one, out)
    G.L.close()


def test_prefill_stream_zero_tokens(B):
    """A chunk of no tokens still streams every layer's pool and computes nothing."""
    from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool
    wl = synth.workload("tiny_fp32")
    n_layers = 2
    cfg = config(wl, n_slots=0, n_layers=n_layers)
    nb = B.moe_expert_bytes(cfg)
    ex = synth.expert_weights_many(wl, range(wl.E), threads=4)
    host = pack_pool(cfg, [ex[e] for _ in range(n_layers) for e in range(wl.E)], pin=True)
    L = LayerBuffers(cfg, 1)
    B.moe_bind_pools(L.ctx, None, 0, host, n_layers * wl.E)
    bufs = torch.zeros(2 * wl.E * nb, dtype=torch.uint8, device="cuda")
    out = torch.full((4,), 7.0, dtype=torch.float32, device="cuda")
    B.moe_prefill_stream(L.ctx, bufs, 2, torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda"), 0, None,
                         L.ids, L.w, L.counts, L.offsets, L.perm, L.inv, L.o, L.ws, out,
                         torch.cuda.current_stream(), torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full((4,), 7.0, device="cuda"))
    # the last layer's pool is in buffer (n_layers - 1) % 2
    last = (n_layers - 1) % 2
    assert torch.equal(bufs[last * wl.E * nb:(last + 1) * wl.E * nb].cpu(), host[(n_layers - 1) * wl.E * nb:])
    L.close()
