"""Every pair output of the full-size prefill grouped GEMM against a plain PyTorch fp32
reference of the same products on the GPU.

The oracle checks a sample of tokens of the 8192-token chunk one by one; this test
covers every pair row (every row tile, column tile and ragged expert tail, and the
shared expert's rows) with torch matmuls in fp32 over the same weights and activations:
per expert, g = A Wg^T, u = A Wu^T, h = bf16(silu(g) u), o = h Wd^T.  MXFP4 weights are
decoded here from their definition (e2m1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign
bit, low nibble first, times 2^(scale - 127) per 32 values along K).  A wrong tile, lane
or row shows up as an error of order one; the bound is the two bf16 roundings (h and o).
A second call must reproduce the first bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from helpers import config

pytestmark = pytest.mark.gpu

_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16).float()


def _mxfp4(codes: np.ndarray, scales: np.ndarray) -> torch.Tensor:
    c = torch.from_numpy(np.ascontiguousarray(codes)).cuda().long()
    lut = torch.tensor(_E2M1, device="cuda")
    v = torch.stack([lut[c & 15], lut[c >> 4]], dim=-1).reshape(c.shape[0], -1)     # low nibble first
    s = torch.from_numpy(np.ascontiguousarray(scales)).cuda().double()
    sc = torch.pow(2.0, s - 127.0).float().repeat_interleave(32, dim=1)
    return v * sc


def _weights(wl, w):
    if wl.wdtype == "bf16":
        return _bf16(w["wg"]), _bf16(w["wu"]), _bf16(w["wd"])
    return _mxfp4(w["wg"], w["sg"]), _mxfp4(w["wu"], w["su"]), _mxfp4(w["wd"], w["sd"])


def _ref(x, wl, w):
    wg, wu, wd = _weights(wl, w)
    h = (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)).bfloat16().float()
    return h @ wd.T


@pytest.mark.parametrize("name", ["a3b_prefill8k_bf16", "v4flash_mxfp4"])
def test_prefill_every_pair_row(name):
    from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool
    print(f"[gemm-full] {name}", flush=True)
    wl = synth.workload(name)
    T, E, k, H = wl.T, wl.E, wl.k, wl.H
    cfg = config(wl)
    ex = synth.expert_weights_many(wl, range(E + wl.n_shared), threads=16)
    pool = pack_pool(cfg, [ex[e] for e in range(E)], pin=False).cuda()
    shared = pack_pool(cfg, [ex[E]], pin=False).cuda() if wl.n_shared else None
    L = LayerBuffers(cfg, T)
    L.route(torch.from_numpy(synth.iid_logits(wl, T)).cuda(), T)
    d_x = torch.from_numpy(synth.activations(wl, T, tag=3).view(np.int16)).cuda()
    allx = np.arange(E, dtype=np.int32)
    rows = T * k + (T if wl.n_shared else 0)
    L.ffn(d_x, T, pool, allx, allx, shared, wl.n_shared)
    torch.cuda.synchronize()
    o = L.o[: rows * H].view(torch.bfloat16).float().view(rows, H).clone()
    L.o.fill_(0)
    L.ffn(d_x, T, pool, allx, allx, shared, wl.n_shared)
    torch.cuda.synchronize()
    same = torch.equal(o, L.o[: rows * H].view(torch.bfloat16).float().view(rows, H))
    x = d_x.view(torch.bfloat16).float()
    off = L.offsets.cpu().numpy()
    perm = L.perm[: T * k].long()
    groups = [(e, perm[off[e]:off[e + 1]], perm[off[e]:off[e + 1]] // k) for e in range(E)]
    if wl.n_shared:
        t_all = torch.arange(T, device="cuda")
        groups.append((E, T * k + t_all, t_all))
    worst, bad = 0.0, []
    for e, p, tok in groups:
        if p.numel() == 0:
            continue
        ref = _ref(x[tok], wl, ex[e])
        rel = (o[p] - ref).abs().amax(dim=1) / ref.abs().amax(dim=1)
        wrong = torch.nonzero(~(rel <= 2e-2)).flatten()
        if wrong.numel():
            d = (o[p[wrong[0]]] - ref[wrong[0]]).abs()
            cols = torch.nonzero(d > 2e-2 * ref[wrong[0]].abs().max()).flatten()
            bad.append(f"expert {e} ({p.numel()} rows): {wrong.numel()} bad rows, positions {wrong.min().item()}.."
                       f"{wrong.max().item()}, first bad row's columns {cols[:8].tolist()} ({cols.numel()})")
        worst = max(worst, rel.max().item())
    print(f"[gemm-full] worst per-row relative error {worst:.2e}; repeat call bitwise equal: {same}", flush=True)
    for b in bad[:16]:
        print("[gemm-full]", b, flush=True)
    assert not bad, f"{len(bad)} experts with wrong pair rows"
    assert same
    L.close()
