"""GPU parity over layer shapes other than the workloads': one case per kernel variant.

The decode kernels are instantiated per (weight format, 16-byte chunks a lane in the gate/up
rows, lanes and chunks per down row), the grouped GEMMs per (weight format, kernel chosen from
N and K).  The cases below pick hidden and intermediate sizes so that every instantiation the
dispatch can reach is run at least once against the oracle, with ragged token counts, expert
subsets on the GPU, and a shared expert in some of them.  The checks are those of the workload
tests: route bit-exact, layer output within the per-format tolerance, pair outputs of listed
experts only, run-to-run bit identity and, for decode, the one-call entry point bit-identical to
the two calls.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from helpers import TOL, out_f64, rel_err_rows
from test_gpu_parity import B, GpuLayer, _decode_case, check_route  # noqa: F401  (B is a fixture)

pytestmark = pytest.mark.gpu

BASE = {"f32": "tiny_fp32", "bf16": "a3b_decode_bf16", "mxfp4": "v4flash_mxfp4"}


def _shape(wdtype, H, I, E, k, shared, name):
    return dataclasses.replace(synth.workload(BASE[wdtype]), name=name, H=H, I=I, E=E, k=k, C=E,
                               n_shared=1 if shared else 0)


# (format, H, I, E, k, T, GPU share of the step's experts, shared expert).  Chunks a lane in the
# gate/up rows: H/8 (bf16), H/32 (MXFP4), H/4 (fp32) over 64 lanes; lanes x chunks per down row
# from I (32 lanes where the row allows, else 16, else 64).
DECODE = [
    ("bf16", 512, 384, 16, 4, 3, 0.75, False),      # gate/up 1 chunk a lane; down 16 x 3
    ("bf16", 1024, 128, 12, 2, 5, 1.0, False),      # 2; down 16 x 1
    ("bf16", 2048, 3072, 8, 2, 2, 0.75, False),     # 4; down 64 x 6
    ("bf16", 4096, 2048, 8, 3, 7, 1.0, True),       # 8; down 32 x 8
    ("bf16", 1024, 1536, 64, 6, 8, 0.5, True),      # 2; down 32 x 6, more list entries than the fused kernel takes
    ("mxfp4", 2048, 512, 16, 4, 4, 0.75, False),    # 1; down 16 x 1
    ("mxfp4", 4096, 1024, 8, 2, 8, 1.0, False),     # 2; down 32 x 1
    ("mxfp4", 2048, 3072, 8, 2, 1, 1.0, True),      # 1; down 32 x 3
    ("mxfp4", 2048, 6144, 8, 1, 6, 0.75, False),    # 1; down 32 x 6
    ("f32", 256, 192, 32, 8, 8, 0.75, False),       # 1; down 16 x 3
    ("f32", 1024, 64, 10, 3, 2, 1.0, True),         # 4; down 16 x 1
    ("f32", 2048, 1024, 8, 2, 5, 0.75, False),      # 8; down 32 x 8
]


@pytest.mark.parametrize("wdtype,H,I,E,k,T,frac,shared", DECODE)
def test_decode_shape_sweep(B, wdtype, H, I, E, k, T, frac, shared):
    name = f"{wdtype}_{H}x{I}_E{E}k{k}{'s' if shared else ''}"
    print(f"[decode-sweep] {name} T={T} gpu share {frac}", flush=True)
    wl = _shape(wdtype, H, I, E, k, shared, name)
    _decode_case(B, name, T, frac, seed=H + I + T, wl=wl)


# Grouped GEMM kernels: large tile for MXFP4 when K <= 4096 and K % 128 == 0, for bf16 when
# K >= 512; for the other bf16 GEMMs the three-stage kernel, or the pipelined kernel when K
# has fewer than three slices of 64.  GEMM 1 has N = 2I, K = H; GEMM 2 N = H, K = I.  The
# three-stage kernel's ring position moves by K / 64 mod 3 per tile: 4 and 6 slices below
# give 1 and 0 (the only K it takes are 256 and 384).
PREFILL = [
    ("bf16", 512, 128, 8, 2, 37, False),       # large tile (K = 512) / pipelined (K = 128)
    ("bf16", 2048, 256, 16, 4, 300, True),     # large tile (K = 2048) / three-stage (K = 256)
    ("bf16", 1536, 640, 8, 3, 130, False),     # large tile / large tile, 5 and 6 column tiles
    ("bf16", 256, 384, 8, 2, 12288, True),     # three-stage (K = 256) / three-stage (K = 384); 864 and 288 tiles: several a workgroup
    ("mxfp4", 1024, 384, 8, 2, 77, False),     # large tile / large tile, K = 1024 and 384
    ("mxfp4", 4096, 2048, 8, 2, 50, True),     # large tile / large tile, K = 4096 and 2048
    ("mxfp4", 512, 1152, 8, 2, 65, False),     # large tile / large tile, 9 column tiles of GEMM 1
]


@pytest.mark.parametrize("wdtype,H,I,E,k,T,shared", PREFILL)
def test_prefill_shape_sweep(B, wdtype, H, I, E, k, T, shared):
    name = f"{wdtype}_{H}x{I}_E{E}k{k}{'s' if shared else ''}"
    print(f"[prefill-sweep] {name} T={T}", flush=True)
    wl = dataclasses.replace(_shape(wdtype, H, I, E, k, shared, name), T=T)
    logits = synth.iid_logits(wl, T, tag=H + I)
    present = sorted(set(oracle.route(logits, wl.k)[0].ravel().tolist()))
    G = GpuLayer(B, wl, present, T)
    x = synth.activations(wl, T, tag=H + I)
    ws = 1 if shared else 0
    out = G.run(logits, x, present, ws)
    ids, gates = check_route(G, logits, T)
    y = out_f64(out, wl, T)
    ref = oracle.moe_layer(oracle.act_f64(x, wl.act_dtype), ids, gates, G.ex,
                           shared=G.ex.f64(wl.E) if ws else None)
    err = rel_err_rows(y, ref)
    assert err.max() <= TOL[wl.wdtype], err.max()
    assert np.median(err) <= 6e-3, np.median(err)
    out2 = G.run(logits, x, present, ws)
    assert bool((out == out2).all()), "prefill output differs between two runs"
    G.L.close()
