"""moe_permute_noalloc (the library's fixed scratch) against moe_permute (a caller workspace).

Both run the same kernels; only where the per-(bucket, chunk) counts and
per-pair ranks live differs, so every output must be bit-identical: counts,
offsets, row_src, inv_perm, the tile list and the copied rows.  Two calls in a
row share the fixed scratch, the second with a smaller input (it must not see
anything the first left behind), and a third runs index-only.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_moe_amd import ffi
from mixture_experts_layer_moe_amd import workloads as W

import parity_helpers as P

pytestmark = pytest.mark.gpu


def bits16(t):
    return t.contiguous().view(torch.int16)


def same_outputs(a: ffi.Permuted, b: ffi.Permuted, rows: bool):
    for name in ("expert_counts", "expert_offsets", "row_src", "inv_perm", "num_tiles"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    nt = int(a.num_tiles.item())
    assert torch.equal(a.tiles[:nt], b.tiles[:nt])
    if rows:
        real = (a.row_src >= 0).nonzero().squeeze(1)
        assert torch.equal(bits16(a.x_perm[real]), bits16(b.x_perm[real]))
    return nt


@pytest.mark.parametrize("order", ["large_then_small"])
def test_permute_noalloc_matches_workspace_call(order):
    dev = P.require_gpu()
    ffi.lib()
    cases = [
        # the expert-parallel share's routing (16384 tokens, 8 source ranks, 8 of 64 experts, top-8)
        W.CONFIGS["ep_share"].with_(H=512),
        # then a smaller, different layer: fewer tokens, more buckets, other tile size
        W.MoEConfig("s", T=700, H=256, F=256, E=16, k=4, act="swiglu", logits="normal", tile_m=32,
                    expert_begin=2, E_loc=10, num_ranks=3),
    ]
    for i, cfg in enumerate(cases):
        d = W.make_inputs(cfg, dev, weights=False)
        idx, _ = ffi.moe_route_topk(d["logits"], cfg.k)
        ref = ffi.moe_permute(d["x"], idx, d["src_rank"], cfg.E, cfg.expert_begin, cfg.n_local, cfg.num_ranks,
                              cfg.tile_m)
        out = ffi.alloc_permuted(cfg.T, cfg.H, cfg.k, cfg.n_local, cfg.tile_m, dev)
        for t in (out.expert_counts, out.expert_offsets, out.row_src, out.inv_perm, out.tiles, out.num_tiles):
            t.fill_(-5)
        torch.cuda.synchronize()
        st = ffi.moe_permute_noalloc(d["x"], idx, d["src_rank"], cfg.H, cfg.E, cfg.expert_begin, cfg.n_local,
                                     cfg.num_ranks, cfg.tile_m, out)
        assert st == 0, ffi.lib().moe_status_str(st)
        torch.cuda.synchronize()
        nt = same_outputs(ref, out, rows=True)
        print(f"[no-alloc] call {i}: T {cfg.T}, {nt} tiles, identical to the workspace call", flush=True)
        # index-only form on the same scratch
        io = ffi.alloc_permuted(cfg.T, cfg.H, cfg.k, cfg.n_local, cfg.tile_m, dev, rows=False)
        st = ffi.moe_permute_noalloc(None, idx, d["src_rank"], cfg.H, cfg.E, cfg.expert_begin, cfg.n_local,
                                     cfg.num_ranks, cfg.tile_m, io)
        assert st == 0
        torch.cuda.synchronize()
        same_outputs(ref, io, rows=False)
    # beyond the fixed scratch: refused on the host, nothing launched
    big = ffi.alloc_permuted(1, 8, 1, 1, 16, dev, rows=False)
    idx_big = torch.zeros((300000, 8), dtype=torch.int32, device=dev)
    assert ffi.moe_permute_noalloc(None, idx_big, None, 8, 8, 0, 8, 1, 64, big) == 3   # MOE_ERR_WORKSPACE
