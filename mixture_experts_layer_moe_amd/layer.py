"""One GPU's share of an MoE layer: the four library calls on preallocated buffers.

Marshalling only: buffers are allocated once with torch, and `run()` enqueues
moe_route_topk -> moe_permute -> moe_grouped_ffn -> moe_combine on one stream
with no host synchronisation in between (every data-dependent size stays on
the device), so the whole layer can also be captured in a HIP graph.  With
fused_gather=True the permute writes indices only and moe_grouped_ffn_gather
reads layer0's token rows straight from x (no x_perm).  With signalled=True
the grouped FFN and the combine run as one launch with tile-level signals
(moe_ffn_combine_fused; 256-row tiles).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import ffi
from .workloads import MoEConfig


class MoELayer:
    def __init__(self, cfg: MoEConfig, x: torch.Tensor, logits: torch.Tensor,
                 src_rank: Optional[torch.Tensor], w0: torch.Tensor, w0_up: Optional[torch.Tensor],
                 w1: torch.Tensor, tile_m: Optional[int] = None, renormalize: bool = True,
                 fused_gather: bool = False, signalled: bool = False):
        self.cfg = cfg
        self.fused_gather = fused_gather
        self.signalled = signalled
        self.tile_m = tile_m or cfg.tile_m
        self.renormalize = renormalize
        self.x, self.logits, self.src_rank = x, logits, src_rank
        self.w0, self.w0_up, self.w1 = w0, w0_up, w1
        dev = x.device
        T, H, k, El = cfg.T, cfg.H, cfg.k, cfg.n_local
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.perm = ffi.alloc_permuted(T, H, k, El, self.tile_m, dev, rows=not fused_gather)
        nbytes = ffi.permute_workspace_bytes(T, k, El, cfg.num_ranks)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        self.act_buf = torch.empty((self.perm.R_cap, cfg.F_loc), dtype=torch.bfloat16, device=dev)
        self.y_perm = torch.empty((self.perm.R_cap, H), dtype=torch.float32, device=dev)
        ffn_bytes = ffi.grouped_ffn_workspace_bytes(self.tile_m, H)
        self.ffn_ws = torch.empty(ffn_bytes, dtype=torch.uint8, device=dev) if ffn_bytes else None
        self.out = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.fused_ws = ffi.alloc_fused_workspace(self.perm.tiles_cap, H, dev) if signalled else None

    @classmethod
    def from_inputs(cls, cfg: MoEConfig, inputs: dict, **kw) -> "MoELayer":
        return cls(cfg, inputs["x"], inputs["logits"], inputs["src_rank"], inputs["w0"],
                   inputs["w0_up"], inputs["w1"], **kw)

    def route(self, stream=None):
        ffi.moe_route_topk(self.logits, self.cfg.k, self.renormalize, self.topk_idx, self.topk_w, stream)

    def permute(self, stream=None):
        c = self.cfg
        ffi.moe_permute(self.x, self.topk_idx, self.src_rank, c.E, c.expert_begin, c.n_local,
                        c.num_ranks, self.tile_m, out=self.perm, ws=self.ws, stream=stream,
                        copy_rows=not self.fused_gather)

    def ffn(self, stream=None):
        if self.fused_gather:
            ffi.moe_grouped_ffn_gather(self.x, self.perm, self.w0, self.w0_up, self.w1, self.cfg.act,
                                       self.act_buf, self.y_perm, self.ffn_ws, stream, use_workspace=False)
        else:
            ffi.moe_grouped_ffn(self.perm, self.w0, self.w0_up, self.w1, self.cfg.act,
                                self.act_buf, self.y_perm, self.ffn_ws, stream, use_workspace=False)

    def combine(self, stream=None):
        ffi.moe_combine(self.y_perm, self.perm.inv_perm, self.topk_w, self.out, stream)

    def ffn_combine(self, stream=None):
        """The grouped FFN and the combine as one launch with tile-level signals."""
        ffi.moe_ffn_combine_fused(self.perm, self.w0, self.w0_up, self.w1, self.cfg.act, self.topk_w,
                                  self.fused_ws, self.act_buf, self.y_perm, self.out, stream)

    def run(self, stream=None) -> torch.Tensor:
        self.route(stream)
        self.permute(stream)
        if self.signalled:
            self.ffn_combine(stream)
        else:
            self.ffn(stream)
            self.combine(stream)
        return self.out
