"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Integer outputs (top-k ids, counts, offsets, permutation and its inverse, cache
plans) must match bit for bit; gates within 1e-6 relative; layer outputs within
the per-token relative error max|y - y_ref| / max|y_ref| of 1e-5 (fp32) or 2e-2
(bf16, MXFP4), with a tighter secondary bound where the arithmetic allows it.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import Experts, TOL, config, dev_act, out_f64, rel_err_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from expert_cached_moe_amd import binding
    return binding


_dev_act, _out_f64 = dev_act, out_f64


def _route_case(B, wl, logits, renorm=1):
    from expert_cached_moe_amd.runtime import LayerBuffers
    T = logits.shape[0]
    cfg = config(wl, renormalize=renorm)
    L = LayerBuffers(cfg, max(T, 1))
    dl = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda() if T else torch.empty(1).cuda()
    L.route(dl, T)
    torch.cuda.synchronize()
    n = T * wl.k
    ids = L.ids[:n].cpu().numpy().reshape(T, wl.k)
    w = L.w[:n].cpu().numpy().reshape(T, wl.k)
    counts, offsets = L.counts.cpu().numpy(), L.offsets.cpu().numpy()
    perm, inv = L.perm[:n].cpu().numpy(), L.inv[:n].cpu().numpy()
    rids, rg = oracle.route(logits, wl.k, renormalize=bool(renorm)) if T else (np.zeros((0, wl.k), np.int32), None)
    rc, ro, rp, ri = oracle.permute(rids, wl.E)
    assert np.array_equal(ids, rids)
    assert np.array_equal(counts, rc) and np.array_equal(offsets, ro)
    assert np.array_equal(perm, rp) and np.array_equal(inv, ri)
    if T:
        assert np.abs(w - rg).max() <= 1e-6 * np.abs(rg).max() + 1e-12
    L.close()


@pytest.mark.parametrize("case", ["tiny", "a3b_b1", "a3b_b8", "v4_b8", "prefill_a3b", "prefill_v4", "ragged513",
                                  "t1", "t0", "ties", "no_renorm", "e8_k8", "decode_ties", "decode_no_renorm"])
def test_route_parity(B, case):
    print(f"[route] {case}", flush=True)
    if case == "tiny":
        wl = synth.workload("tiny_fp32")
        logits = oracle.router_logits(synth.activations(wl, wl.T), synth.router_weights(wl))
        _route_case(B, wl, logits)
    elif case in ("a3b_b1", "a3b_b8"):
        wl = synth.workload("a3b_decode_bf16")
        b = 1 if case == "a3b_b1" else 8
        lg, _ = synth.zipf_reuse_trace(wl, b, 16)
        for s in range(16):
            _route_case(B, wl, lg[s])
    elif case == "v4_b8":
        wl = synth.workload("v4flash_decode_bf16")
        lg, _ = synth.zipf_reuse_trace(wl, 8, 8)
        for s in range(8):
            _route_case(B, wl, lg[s])
    elif case == "prefill_a3b":
        wl = synth.workload("a3b_prefill8k_bf16")
        _route_case(B, wl, synth.iid_logits(wl, 8192))
    elif case == "prefill_v4":
        wl = synth.workload("v4flash_mxfp4")
        _route_case(B, wl, synth.iid_logits(wl, 8192))
    elif case == "ragged513":
        wl = synth.workload("a3b_prefill8k_bf16")
        _route_case(B, wl, synth.iid_logits(wl, 513, tag=5))       # 4104 pairs: multi-chunk path, ragged tail
    elif case == "t1":
        wl = synth.workload("v4flash_mxfp4")
        _route_case(B, wl, synth.iid_logits(wl, 1, tag=2))
    elif case == "t0":
        wl = synth.workload("a3b_decode_bf16")
        _route_case(B, wl, np.zeros((0, wl.E), np.float32))
    elif case == "ties":
        wl = synth.workload("a3b_prefill8k_bf16")
        rng = np.random.default_rng(4)
        lg = (rng.integers(-3, 3, size=(700, wl.E)) * 0.5).astype(np.float32)
        lg[::7] = 0.0
        lg[1::7] = -0.0
        _route_case(B, wl, lg)
    elif case == "no_renorm":
        wl = synth.workload("v4flash_decode_bf16")
        _route_case(B, wl, synth.iid_logits(wl, 37, tag=3), renorm=0)
    elif case in ("decode_ties", "decode_no_renorm"):
        # decode batch sizes (the one-workgroup route and grouping): exact ties, -0 == +0,
        # and the softmax over all experts
        wl = synth.workload("a3b_decode_bf16")
        rng = np.random.default_rng(11)
        for T in (1, 3, 8):
            lg = (rng.integers(-3, 3, size=(T, wl.E)) * 0.5).astype(np.float32)
            lg[:, ::5] = 0.0
            lg[:, 1::5] = -0.0
            _route_case(B, wl, lg, renorm=0 if case == "decode_no_renorm" else 1)
    elif case == "e8_k8":
        import dataclasses
        wl = dataclasses.replace(synth.workload("tiny_fp32"), k=8)
        _route_case(B, wl, np.random.default_rng(0).standard_normal((9, 8)).astype(np.float32))


# bf16 / fp32-high-half bit pattern of a quiet NaN, written into the pair outputs before a call
POISON = 0x7FC1


def check_route(G, logits, T):
    """The GPU's ids of the last route equal the oracle's bit for bit and its gates agree within
    1e-6 relative; returns the oracle's (ids, gates), from which every reference is built."""
    k = G.wl.k
    ids = G.L.ids[: T * k].cpu().numpy().reshape(T, k)
    w = G.L.w[: T * k].cpu().numpy().reshape(T, k)
    rids, rg = oracle.route(logits, k)
    assert np.array_equal(ids, rids), "top-k ids differ from the oracle"
    assert np.abs(w - rg).max() <= 1e-6 * np.abs(rg).max() + 1e-12, "gates differ from the oracle"
    return rids, rg


def pair_rows_written(G, T, ids, gpu, with_shared):
    """Pair-output rows of listed experts (and the shared expert's rows) as fp64; asserts every
    other row still holds the poison pattern (the call writes only its listed experts' pairs)."""
    wl = G.wl
    rows = T * wl.k + (T if with_shared else 0)
    raw = G.L.o.view(torch.int16)[: rows * wl.H * (2 if wl.act_dtype == "f32" else 1)].cpu().numpy()
    raw = raw.reshape(rows, -1)
    listed = np.zeros(rows, bool)
    for t in range(T):
        for j in range(wl.k):
            listed[t * wl.k + j] = int(ids[t, j]) in gpu
    listed[T * wl.k:] = True
    assert (raw[~listed] == POISON).all(), "pair rows of unlisted experts were written"
    out = np.full((rows, wl.H), np.nan)
    got = np.ascontiguousarray(raw[listed])
    if wl.act_dtype == "f32":
        out[listed] = got.view(np.float32).astype(np.float64)
    else:
        out[listed] = oracle.bf16_bits_to_f64(got.view(np.uint16))
    return out


class GpuLayer:
    """Device pool of packed experts (slot = position in ``experts``) and buffers."""

    def __init__(self, B, wl, experts, max_T, ex=None):
        from expert_cached_moe_amd.runtime import LayerBuffers, pack_pool
        self.wl, self.ex = wl, ex or Experts(wl)
        self.cfg = config(wl)
        self.L = LayerBuffers(self.cfg, max_T)
        self.experts = list(experts)
        self.slot = {e: i for i, e in enumerate(self.experts)}
        self.ex.prefetch(self.experts + ([wl.E] if wl.n_shared else []))
        host = pack_pool(self.cfg, [self.ex.raw(e) for e in self.experts], pin=False)
        self.pool = host.cuda()
        self.shared = None
        if wl.n_shared:
            self.shared = pack_pool(self.cfg, [self.ex.raw(wl.E)], pin=False).cuda()

    def run(self, logits, x, gpu_experts, with_shared, y_host=None, host_ids=True):
        """host_ids: decode token lists from the host copy of the ids (else from the router's
        device offsets/permutation).  The pair-output buffer is filled with POISON first, so
        rows the call must not write can be checked afterwards."""
        T = logits.shape[0]
        wl, L = self.wl, self.L
        L.o.view(torch.int16).fill_(POISON)
        L.route(torch.from_numpy(np.ascontiguousarray(logits)).cuda(), T)
        h_ids = L.ids[: T * wl.k].cpu().numpy().reshape(T, wl.k) if host_ids else None
        dx = _dev_act(x)
        slots = [self.slot[e] for e in gpu_experts]
        L.ffn(dx, T, self.pool, gpu_experts, slots, self.shared, with_shared, h_ids=h_ids)
        out = torch.empty(T * wl.H, dtype=torch.float32 if wl.act_dtype == "f32" else torch.int16, device="cuda")
        L.merge(gpu_experts, with_shared, y_host, T, out)
        torch.cuda.synchronize()
        return out


def _decode_case(B, name, T, frac, seed, host_ids=True, wl=None):
    wl = wl or synth.workload(name)
    lg, _ = synth.zipf_reuse_trace(wl, T, 3, tag=seed)
    logits = lg[2]
    ids, gates = oracle.route(logits, wl.k)
    present = sorted(set(ids.ravel().tolist()))
    rng = np.random.default_rng(seed)
    gpu = sorted(rng.permutation(present)[: max(1, int(round(frac * len(present))))].tolist())
    # slots in a shuffled order with unused slots between them
    pool_order = rng.permutation(present + [e for e in range(wl.E) if e not in present][:3]).tolist()
    G = GpuLayer(B, wl, pool_order, T)
    x = synth.activations(wl, T, tag=seed)
    ws = 1 if wl.n_shared else 0
    out = G.run(logits, x, gpu, ws, host_ids=host_ids)
    check_route(G, logits, T)
    y = _out_f64(out, wl, T)
    xf = oracle.act_f64(x, wl.act_dtype)
    shared = G.ex.f64(wl.E) if wl.n_shared else None
    ref = oracle.moe_layer(xf, ids, gates, G.ex, shared=shared, subset=set(gpu))
    err = rel_err_rows(y, ref)
    tol = TOL[wl.wdtype]
    assert err.max() <= tol, (name, T, err.max())
    # per-pair expert outputs (activation dtype, before the gate-weighted sum): tighter bound;
    # rows of experts not on the GPU must be untouched
    o = pair_rows_written(G, T, ids, set(gpu), ws)
    if ws:
        r = oracle.expert_ffn(shared, xf)
        pe = rel_err_rows(o[T * wl.k:], r).max()
        assert pe <= (1e-5 if wl.wdtype == "f32" else 1.5e-2), (name, "shared", pe)
    for t in range(T):
        for j in range(wl.k):
            e = int(ids[t, j])
            if e not in gpu:
                continue
            r = oracle.expert_ffn(G.ex.f64(e), xf[t:t + 1])
            pe = rel_err_rows(o[t * wl.k + j][None, :], r)[0]
            assert pe <= (1e-5 if wl.wdtype == "f32" else 1.5e-2), (name, t, j, pe)
    # bitwise run-to-run determinism
    out2 = G.run(logits, x, gpu, ws, host_ids=host_ids)
    assert torch.equal(out, out2)
    if host_ids:
        # experts and merge in one call (moe_expert_ffn_merge) against the two calls, bit for
        # bit, with a host part when some experts are on the host
        yh = torch.from_numpy(np.random.default_rng(seed + 7).standard_normal(T * wl.H).astype(np.float32)).cuda() \
            if frac < 1 else None
        slots = [G.slot[e] for e in gpu]
        h_ids = G.L.ids[: T * wl.k].cpu().numpy().reshape(T, wl.k)
        dx = _dev_act(x)
        two, one = torch.empty_like(out), torch.full_like(out, 7)
        G.L.ffn(dx, T, G.pool, gpu, slots, G.shared, ws, h_ids=h_ids)
        G.L.merge(gpu, ws, yh, T, two)
        G.L.ffn_merge(dx, T, G.pool, gpu, slots, h_ids, G.shared, ws, yh, one)
        torch.cuda.synchronize()
        assert torch.equal(one, two), (name, T, frac)
    G.L.close()
    return err.max()


@pytest.mark.parametrize("name,T", [("tiny_fp32", 1), ("tiny_fp32", 8), ("a3b_decode_bf16", 1),
                                    ("a3b_decode_bf16", 4), ("a3b_decode_bf16", 8), ("v4flash_decode_bf16", 1),
                                    ("v4flash_decode_bf16", 8), ("v4flash_mxfp4", 1), ("v4flash_mxfp4", 8)])
@pytest.mark.parametrize("frac", [1.0, 0.5])
def test_decode_ffn_merge_parity(B, name, T, frac):
    print(f"[decode] {name} T={T} frac={frac}", flush=True)
    _decode_case(B, name, T, frac, seed=T * 10 + int(frac * 2))


@pytest.mark.parametrize("wdtype,H,I,T", [("f32", 512, 256, 1), ("f32", 512, 256, 5), ("bf16", 1024, 512, 1),
                                          ("bf16", 1024, 512, 8), ("mxfp4", 2048, 1024, 1), ("mxfp4", 8192, 512, 8),
                                          ("mxfp4", 16384, 512, 2)])
def test_decode_other_shapes(B, wdtype, H, I, T):
    """Decode at hidden/intermediate sizes other than the workloads' (16 experts, top-4):
    the kernels pick their lanes-per-row and chunks-per-lane from the shape.  MXFP4 at
    hidden 8192 stages two token rows of x per group in LDS, so the shared expert's 8
    tokens take four groups; at hidden 16384 a gate/up lane holds 8 chunks, so the block
    scales of its rows span two 64-dword pieces, and one token row fills the staging LDS."""
    print(f"[decode-other-shapes] {wdtype} H={H} I={I} T={T}", flush=True)
    import dataclasses
    base = synth.workload({"f32": "tiny_fp32", "bf16": "a3b_decode_bf16", "mxfp4": "v4flash_mxfp4"}[wdtype])
    wl = dataclasses.replace(base, name=f"{wdtype}_{H}x{I}", H=H, I=I, E=16, k=4, C=16, batches=(T,))
    _decode_case(B, None, T, 0.75, seed=T + 300, wl=wl)


@pytest.mark.parametrize("name,T", [("tiny_fp32", 3), ("a3b_decode_bf16", 8), ("v4flash_mxfp4", 2)])
def test_decode_device_lists_parity(B, name, T):
    """Decode with the token lists taken from the router's device outputs."""
    print(f"[decode-device-lists] {name} T={T}", flush=True)
    _decode_case(B, name, T, 0.75, seed=T + 100, host_ids=False)


def test_decode_no_gpu_experts_is_host_only(B):
    """q = 0 and no hits: the GPU part is exactly zero and the output is the host part."""
    wl = synth.workload("a3b_decode_bf16")
    G = GpuLayer(B, wl, [0, 1], 2)
    logits = synth.iid_logits(wl, 2, tag=9)
    x = synth.activations(wl, 2, tag=9)
    yh = torch.randn(2 * wl.H, device="cuda")
    out = G.run(logits, x, [], 0, y_host=yh)
    want = yh.cpu().numpy().astype(np.float32)
    got = _out_f64(out, wl, 2).ravel()
    assert np.abs(got - want).max() <= 2 ** -8 * np.abs(want).max()
    G.L.close()


@pytest.mark.parametrize("name,T", [("a3b_prefill8k_bf16", 40), ("tiny_fp32", 100), ("v4flash_mxfp4", 24)])
def test_small_prefill_parity(B, name, T):
    """Ragged prefill-sized batches (T > 8: the grouped path) at sizes the oracle finishes quickly."""
    print(f"[prefill-small] {name} T={T}", flush=True)
    wl = synth.workload(name)
    logits = synth.iid_logits(wl, T, tag=T)
    ids, _ = oracle.route(logits, wl.k)
    present = sorted(set(ids.ravel().tolist()))
    G = GpuLayer(B, wl, present, T)
    x = synth.activations(wl, T, tag=T)
    ws = 1 if wl.n_shared else 0
    out = G.run(logits, x, present, ws)
    ids, gates = check_route(G, logits, T)
    y = _out_f64(out, wl, T)
    ref = oracle.moe_layer(oracle.act_f64(x, wl.act_dtype), ids, gates, G.ex,
                           shared=G.ex.f64(wl.E) if ws else None)
    err = rel_err_rows(y, ref)
    assert err.max() <= TOL[wl.wdtype], err.max()
    G.L.close()


@pytest.mark.parametrize("H,I", [(8192, 512), (512, 4224)])
def test_prefill_mxfp4_register_staged(B, H, I):
    """MXFP4 GEMM shapes the large-tile kernel does not take run the register-staged kernel:
    a gate/up reduction of K = 8192 (the tile's scales would not fit its LDS region) and a
    down reduction of K = 4224 (the same).  Ragged 40-token batch, shared expert included."""
    print(f"[prefill-mxfp4-staged] H={H} I={I}", flush=True)
    base = synth.workload("v4flash_mxfp4")
    wl = dataclasses.replace(base, name=f"mxfp4_{H}x{I}", H=H, I=I, E=8, k=2, C=8, T=40)
    T = wl.T
    logits = synth.iid_logits(wl, T, tag=T)
    present = sorted(set(oracle.route(logits, wl.k)[0].ravel().tolist()))
    G = GpuLayer(B, wl, present, T)
    x = synth.activations(wl, T, tag=T)
    out = G.run(logits, x, present, 1)
    ids, gates = check_route(G, logits, T)
    y = _out_f64(out, wl, T)
    ref = oracle.moe_layer(oracle.act_f64(x, wl.act_dtype), ids, gates, G.ex, shared=G.ex.f64(wl.E))
    err = rel_err_rows(y, ref)
    assert err.max() <= TOL[wl.wdtype], err.max()
    assert np.median(err) <= 6e-3, np.median(err)
    G.L.close()


def test_prefill_bf16_large_tile_down(B):
    """bf16 prefill with an intermediate size of 2048: both GEMMs run the large-tile kernel
    (K = I = 2048 for the down GEMM, K = H = 1024 for gate/up) on a ragged 40-token batch with
    a shared expert, so every tile ends part way, the down GEMM skips the A loads of dead row
    groups and its pair-output rows come from the row table."""
    print("[prefill-bf16-big-down] H=1024 I=2048", flush=True)
    base = synth.workload("v4flash_decode_bf16")
    wl = dataclasses.replace(base, name="bf16_1024x2048", H=1024, I=2048, E=8, k=2, C=8, T=40)
    T = wl.T
    logits = synth.iid_logits(wl, T, tag=T + 7)
    present = sorted(set(oracle.route(logits, wl.k)[0].ravel().tolist()))
    G = GpuLayer(B, wl, present, T)
    x = synth.activations(wl, T, tag=T + 7)
    out = G.run(logits, x, present, 1)
    ids, gates = check_route(G, logits, T)
    y = _out_f64(out, wl, T)
    ref = oracle.moe_layer(oracle.act_f64(x, wl.act_dtype), ids, gates, G.ex, shared=G.ex.f64(wl.E))
    err = rel_err_rows(y, ref)
    assert err.max() <= TOL[wl.wdtype], err.max()
    assert np.median(err) <= 6e-3, np.median(err)
    G.L.close()


@pytest.mark.parametrize("name,n_sample,T", [("a3b_prefill8k_bf16", 24, 8192), ("v4flash_mxfp4", 8, 8192),
                                            ("a3b_prefill8k_bf16", 12, 16384)])
def test_prefill_full_size_sampled(B, name, n_sample, T):
    """Prefill chunks at full size (8192 tokens, and the 16384-token chunk of the streamed
    ablation) through the grouped GEMM; the oracle checks a sample of tokens (first, last and
    random ones) one by one."""
    print(f"[prefill-full] {name} T={T}", flush=True)
    wl = synth.workload(name)
    ex = Experts(wl)
    logits = synth.iid_logits(wl, T)
    G = GpuLayer(B, wl, list(range(wl.E)), T, ex=ex)
    x = synth.activations(wl, T, tag=3)
    ws = 1 if wl.n_shared else 0
    out = G.run(logits, x, list(range(wl.E)), ws)
    y = _out_f64(out, wl, T)
    rids, rg = check_route(G, logits, T)
    rng = np.random.default_rng(0)
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, n_sample - 2, replace=False)]))
    xs = oracle.act_f64(x[sample], wl.act_dtype)
    conv = lambda e: oracle.expert_f64(ex.raw(e), wl.wdtype)          # no fp64 cache: bounded memory
    ref = oracle.moe_layer(xs, rids[sample], rg[sample], conv, shared=conv(wl.E) if ws else None)
    err = rel_err_rows(y[sample], ref)
    assert err.max() <= TOL[wl.wdtype], err.max()
    # typical error of two bf16 roundings (h, then each pair output, up to 2^-9 relative
    # each), well under the bound
    assert np.median(err) <= 6e-3, np.median(err)
    G.L.close()
