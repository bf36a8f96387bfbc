"""Device buffers for one MoE layer, allocated with torch (memory and streams only).

``LayerBuffers`` owns the context and the device scratch a layer needs up to
``max_T`` tokens and forwards to the C entry points; ``pack_pool`` packs expert
weights into a (pinned) host pool of blobs with ``moe_pack_expert``.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


class LayerBuffers:
    def __init__(self, cfg: B.moe_config, max_T: int, device: str = "cuda"):
        self.cfg = cfg
        self.ctx = B.moe_create(cfg)
        self.E, self.k, self.H, self.I = cfg.n_experts, cfg.top_k, cfg.hidden, cfg.inter
        self.max_T = max_T
        self.blob_bytes = B.moe_expert_bytes(cfg)
        dev = torch.device(device)
        self.ws = torch.empty(B.moe_workspace_bytes(cfg, max_T), dtype=torch.uint8, device=dev)
        n = max(1, max_T * self.k)
        self.ids = torch.empty(n, dtype=torch.int32, device=dev)
        self.w = torch.empty(n, dtype=torch.float32, device=dev)
        self.counts = torch.empty(self.E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
        self.perm = torch.empty(n, dtype=torch.int32, device=dev)
        self.inv = torch.empty(n, dtype=torch.int32, device=dev)
        # pair outputs in the activation dtype: fp32 for fp32 weights, bf16 bits (int16 storage) otherwise
        o_dtype = torch.float32 if cfg.w_dtype == B.MOE_W_F32 else torch.int16
        self.o = torch.empty(max(1, B.moe_pair_rows(cfg, max_T)) * self.H, dtype=o_dtype, device=dev)

    def close(self):
        if self.ctx:
            B.moe_destroy(self.ctx)
            self.ctx = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def route(self, logits: torch.Tensor, T: int, stream=None):
        B.moe_route(self.ctx, logits, T, self.ids, self.w, self.counts, self.offsets, self.perm, self.inv,
                    self.ws, stream)

    def ffn(self, x, T, slot_base, experts, slots, shared=None, with_shared=0, stream=None, h_ids=None):
        """h_ids: host copy of the step's top-k ids (decode: the kernels then skip the router's
        device outputs); None: the token lists come from this buffer set's last route."""
        n = len(experts)
        B.moe_expert_ffn(self.ctx, x, T, h_ids, self.offsets, self.perm, slot_base, experts, slots, n, shared,
                         with_shared, self.o, self.ws, stream)

    def ffn_merge(self, x, T, slot_base, experts, slots, h_ids, shared=None, with_shared=0, y_host=None, out=None,
                  stream=None):
        """Decode (T <= 8): the experts and the merge of their pair outputs in one call, from
        this buffer set's last route (ids and gates) and the host copy h_ids of its ids."""
        B.moe_expert_ffn_merge(self.ctx, x, T, h_ids, self.ids, self.w, slot_base, experts, slots, len(experts), shared,
                               with_shared, y_host, out, self.ws, stream)

    def merge(self, gpu_experts, with_shared, y_host, T, out, stream=None):
        B.moe_merge_partial(self.ctx, self.o, self.ids, self.w, gpu_experts, len(gpu_experts), with_shared,
                            y_host, T, out, stream)


def pack_pool(cfg: B.moe_config, experts, pin: bool = True) -> torch.Tensor:
    """Pack a sequence of natural-layout expert dicts (wg, wu, wd[, sg, su, sd]) into
    one contiguous uint8 tensor of blobs (pinned host memory when ``pin``).  A ``None``
    entry leaves its blob filled with 0xFF bytes (NaN in every weight format)."""
    experts = list(experts)
    nb = B.moe_expert_bytes(cfg)
    pool = torch.empty(len(experts) * nb, dtype=torch.uint8, pin_memory=pin)
    view = pool.numpy()
    for i, w in enumerate(experts):
        if w is None:
            view[i * nb:(i + 1) * nb] = 0xFF
            continue
        B.moe_pack_expert(cfg, w["wg"], w["wu"], w["wd"], w.get("sg"), w.get("su"), w.get("sd"),
                          view[i * nb:(i + 1) * nb])
    return pool
