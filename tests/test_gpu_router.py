"""GPU parity of the router logits l = x . W_r (moe_router_logits) against the oracle.

The oracle's logits are fp64 rounded once to fp32; the kernel accumulates in fp32 in its
own order.  Recursive summation of H products is within H * 2^-24 * sum_h |x_h w_h| of
the exact dot product, and the oracle's rounding adds half an ulp, so each logit is held
to that bound (computed from the data), not to a guessed tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import config, dev_act

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from expert_cached_moe_amd import binding
    return binding


def _logits(B, wl, x, T):
    from expert_cached_moe_amd.runtime import LayerBuffers
    cfg = config(wl)
    L = LayerBuffers(cfg, max(T, 1))
    wr = synth.router_weights(wl)                                   # [H, E]
    d_wr = torch.from_numpy(np.ascontiguousarray(wr.T)).cuda()      # [E, H]: one row per expert
    d_x = dev_act(x) if T else torch.zeros(1, device="cuda")
    out = torch.full((max(T, 1) * wl.E,), float("nan"), dtype=torch.float32, device="cuda")
    B.moe_router_logits(L.ctx, d_x, T, d_wr, out)
    torch.cuda.synchronize()
    return L, wr, out


@pytest.mark.parametrize("name,T", [("tiny_fp32", 16), ("tiny_fp32", 3), ("tiny_fp32", 0), ("a3b_decode_bf16", 1),
                                    ("a3b_decode_bf16", 8), ("a3b_prefill8k_bf16", 200), ("v4flash_decode_bf16", 8),
                                    ("v4flash_mxfp4", 45)])
def test_router_logits_parity(B, name, T):
    print(f"[router] {name} T={T}", flush=True)
    wl = synth.workload(name)
    x = synth.activations(wl, max(T, 1), tag=31)[:T]
    L, wr, out = _logits(B, wl, x, T)
    if T == 0:
        assert torch.isnan(out).all()                                # nothing written
        L.close()
        return
    got = out.cpu().numpy().reshape(T, wl.E).astype(np.float64)
    xf = oracle.act_f64(x, wl.act_dtype)
    ref = oracle.router_logits(xf, wr).astype(np.float64)
    bound = wl.H * 2.0 ** -24 * (np.abs(xf) @ np.abs(wr.astype(np.float64))) + 2.0 ** -24 * np.abs(ref)
    err = np.abs(got - ref)
    assert (err <= bound).all(), float((err / bound).max())
    L.close()


def test_router_then_route_tiny(B):
    """The tiny layer's own routing on the GPU: logits from moe_router_logits, top-k from
    moe_route, against the oracle's route of the oracle's logits for every token whose first
    k+1 logits are pairwise further apart than twice the logit bound (so neither the picks
    nor their order can depend on rounding)."""
    wl = synth.workload("tiny_fp32")
    T = 64
    x = synth.activations(wl, T, tag=21)
    L, wr, out = _logits(B, wl, x, T)
    L.route(out, T)
    torch.cuda.synchronize()
    ids = L.ids[: T * wl.k].cpu().numpy().reshape(T, wl.k)
    xf = oracle.act_f64(x, wl.act_dtype)
    ref = oracle.router_logits(xf, wr)
    rids, _ = oracle.route(ref, wl.k)
    bound = (wl.H * 2.0 ** -24 * (np.abs(xf) @ np.abs(wr.astype(np.float64))) + 2.0 ** -24 * np.abs(ref)).max(axis=1)
    srt = -np.sort(-ref.astype(np.float64), axis=1)
    gaps = srt[:, :wl.k] - srt[:, 1:wl.k + 1]                      # order of the picks and the cut
    clear = (gaps > 2 * bound[:, None]).all(axis=1)
    assert clear.sum() >= T // 2
    assert np.array_equal(ids[clear], rids[clear])
    L.close()
