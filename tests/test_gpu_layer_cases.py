"""The whole layer through the C ABI on the method's edge cases and on every scheduling path.

Comet (section 2.1) defines the layer for any routing: each token's top-k
experts, each selected expert's FFN, the weighted sum.  These tests run the
four calls (route -> permute -> grouped FFN -> combine) end to end and compare
with the oracle:

  * degenerate routings (one token, one expert, k = E, every token on one
    expert, no local pair) on both tile paths (16- and 256-row tiles) and in
    both layer0 forms (permuted copy and fused gather);
  * the grouped GEMMs' last scheduling round after whole rounds: on a stream
    limited to one XCD (32 CUs) the persistent grid is 32 workgroups, so small
    layers have more items than workgroups; the left-over items are split
    along K into fp32 partial tiles that a second kernel sums (SwiGLU and
    GELU, 128- and 256-row tiles), and every real row is checked;
  * a stream limited to 7 of the 8 XCDs (the grid sized to its CU mask);
  * the expert-parallel partition at the expert-parallel share's real shape:
    8 ranks of 8 experts each sum to the 64-expert layer.

Inputs are the seeded generators; expected values come only from the oracle.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_moe_amd import ffi
from mixture_experts_layer_moe_amd import workloads as W
from mixture_experts_layer_moe_amd.layer import MoELayer
from oracle import moe_oracle as O

import parity_helpers as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = P.require_gpu()
    ffi.lib()
    return d


def bits16(t):
    return t.contiguous().view(torch.int16)


def edge_inputs(case: str, dev):
    """(cfg, inputs) of one degenerate routing; logits are drawn, then biased on the host."""
    T, H, F, E, k, e0, El, R = 200, 256, 256, 8, 2, 0, None, 1
    if case == "one_token":
        T = 1
    if case == "single_expert":
        E, k = 1, 1
    if case == "k_equals_E":
        E, k = 4, 4
    if case == "all_to_one_expert":
        k = 1
    if case == "no_local_pairs":
        e0, El, R = 4, 4, 3
    cfg = W.MoEConfig(case, T=T, H=H, F=F, E=E, k=k, act="swiglu", logits="normal", tile_m=16,
                      expert_begin=e0, E_loc=El, num_ranks=R)
    d = W.make_inputs(cfg, dev)
    lg = d["logits"].cpu()
    if case == "all_to_one_expert":
        lg[:, 3] += 100.0
    if case == "no_local_pairs":
        lg[:, :4] += 100.0   # the top-2 of every token lie in experts 0..3, none in the local 4..7
    d["logits"] = lg.to(dev)
    return cfg, d


EDGE_CASES = ["one_token", "single_expert", "k_equals_E", "all_to_one_expert", "no_local_pairs"]


@pytest.mark.parametrize("fused_gather", [False, True], ids=["x_perm", "gather"])
@pytest.mark.parametrize("tile_m", [16, 256])
@pytest.mark.parametrize("case", EDGE_CASES)
def test_layer_edge_cases(dev, case, tile_m, fused_gather):
    cfg, d = edge_inputs(case, dev)
    layer = MoELayer.from_inputs(cfg, d, tile_m=tile_m, fused_gather=fused_gather)
    layer.out.fill_(float("nan"))
    out = layer.run()
    torch.cuda.synchronize()
    idx, w = P.oracle_route(d["logits"], cfg.k)
    assert np.array_equal(layer.topk_idx.cpu().numpy(), idx)
    np.testing.assert_allclose(layer.topk_w.cpu().numpy(), w, rtol=2e-6, atol=1e-7)
    ref = P.oracle_permute(idx, d["src_rank"], cfg, tile_m)
    assert np.array_equal(layer.perm.inv_perm.cpu().numpy(), ref["inv_perm"])
    assert layer.perm.expert_counts.cpu().numpy().tolist() == ref["counts"].tolist()
    nt = int(layer.perm.num_tiles.item())
    assert [tuple(r) for r in layer.perm.tiles[:nt].cpu().numpy().tolist()] == [tuple(t) for t in ref["tiles"]]
    if case == "single_expert":
        assert np.all(w == 1.0) and np.all(idx == 0)
    if case == "k_equals_E":
        assert np.all(np.sort(idx, axis=1) == np.arange(4))
    if case == "all_to_one_expert":
        assert np.all(idx == 3) and ref["counts"].tolist() == [0, 0, 0, cfg.T, 0, 0, 0, 0]
    got = out.cpu().double().numpy()
    if case == "no_local_pairs":
        assert nt == 0 and np.all(ref["inv_perm"] == -1)
        assert np.all(got == 0.0), "a token with no local pair must get a zero row"
        return
    ref_out = O.moe_layer_expert_major(P.to_np64(d["x"]), cfg.k, P.host_weights64(d), cfg.act, (idx, w),
                                       list(range(cfg.T)), cfg.expert_begin, cfg.n_local)
    P.assert_output_close(got, ref_out, f"{case} tile_m {tile_m}" + (" gather" if fused_gather else ""))
    real = np.nonzero(ref["row_src"] >= 0)[0]
    P.check_ffn_rows(cfg, d, ref, layer.act_buf, layer.y_perm, real, f"{case} tile_m {tile_m}")


# ---------------------------------------------------------------------------
# whole rounds, then the last round split along K (one-XCD stream: 32 workgroups)
# ---------------------------------------------------------------------------

SPLIT_LAYERS = {
    # 8 row tiles: layer0 6 column blocks (48 items: 32 whole, 16 in 2 K slices), layer1 5 (40: 32, 8 in 4)
    128: dict(T=300, H=1280, F=768),
    # 6 row tiles: layer0 36 items (32 whole, 4 in 8 K slices), layer1 36 (same)
    256: dict(T=500, H=1536, F=768),
}


@pytest.mark.parametrize("fused_gather", [False, True], ids=["x_perm", "gather"])
@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("tile_m", [128, 256])
def test_split_k_after_whole_rounds(dev, tile_m, act, fused_gather):
    cfg = W.MoEConfig("split", E=4, k=2, act=act, logits="normal", tile_m=tile_m, **SPLIT_LAYERS[tile_m])
    d = W.make_inputs(cfg, dev)
    idx, w = P.oracle_route(d["logits"], cfg.k)
    ref = P.oracle_permute(idx, None, cfg, tile_m)
    nt = len(ref["tiles"])
    tcap = ffi.tiles_capacity(cfg.T, cfg.k, cfg.n_local, tile_m)
    sched = P.ffn_schedule(nt, tcap, cfg.H, cfg.F, tile_m, 32)
    for name, s in sched.items():
        print(f"[schedule] {name}: G {s['G']}, items {s['total']}, whole {s['full']}, K slices {s['S']}, "
              f"last-round tiles {s['last_tiles']}", flush=True)
        assert s["G"] == 32 and s["full"] > 0 and s["S"] >= 2, (name, s)
    h, stream = P.cu_masked_stream(range(32), dev)
    try:
        layer = MoELayer.from_inputs(cfg, d, fused_gather=fused_gather)
        layer.act_buf.fill_(-7.0)
        layer.y_perm.fill_(-7.0)
        torch.cuda.synchronize()
        out = layer.run(stream)
        torch.cuda.synchronize()
    finally:
        P.destroy_stream(h)
    assert [tuple(r) for r in layer.perm.tiles[:nt].cpu().numpy().tolist()] == [tuple(t) for t in ref["tiles"]]
    real = np.nonzero(ref["row_src"] >= 0)[0]
    pad = np.setdiff1d(np.arange(layer.perm.R_cap), real)
    padt = torch.from_numpy(pad).to(dev)
    assert torch.all(layer.act_buf[padt] == -7.0) and torch.all(layer.y_perm[padt] == -7.0)
    # every real row (a superset of the rows of the tiles the split last round touches)
    what = f"split {act} tile_m {tile_m}" + (" gather" if fused_gather else "")
    P.check_ffn_rows(cfg, d, ref, layer.act_buf, layer.y_perm, real, what)
    ref_out = O.moe_layer_expert_major(P.to_np64(d["x"]), cfg.k, P.host_weights64(d), cfg.act, (idx, w),
                                       list(range(cfg.T)))
    P.assert_output_close(out.cpu().double().numpy(), ref_out, what + " out")


# ---------------------------------------------------------------------------
# whole rounds, then more than half a grid of items left and no K split: the last round runs whole
# items (two half-width pieces each would take two rounds); without a workspace the other GEMM's
# few left-over items run as half-width pieces
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("use_ws", [True, False], ids=["workspace", "no_workspace"])
def test_whole_last_round(dev, use_ws):
    # 6 row tiles of 256: layer0 9 column blocks (54 items: 32 whole, 22 left, 22 > 32 / 2 so no
    # split and no half-width pieces), layer1 6 (36: 32 whole, 4 left: K slices or half-width pieces)
    cfg = W.MoEConfig("whole", T=500, H=1536, F=1152, E=4, k=2, act="swiglu", logits="normal", tile_m=256)
    d = W.make_inputs(cfg, dev)
    idx, w = P.oracle_route(d["logits"], cfg.k)
    ref = P.oracle_permute(idx, None, cfg, cfg.tile_m)
    nt = len(ref["tiles"])
    tcap = ffi.tiles_capacity(cfg.T, cfg.k, cfg.n_local, cfg.tile_m)
    sched = P.ffn_schedule(nt, tcap, cfg.H, cfg.F, cfg.tile_m, 32)
    l0 = sched["layer0"]
    print(f"[schedule] {sched}", flush=True)
    assert l0["G"] == 32 and l0["full"] > 0 and l0["S"] == 1 and 2 * (l0["total"] - l0["full"]) > l0["G"], l0
    h, stream = P.cu_masked_stream(range(32), dev)
    try:
        layer = MoELayer.from_inputs(cfg, d)
        layer.route(stream)
        layer.permute(stream)
        layer.act_buf.fill_(-7.0)
        layer.y_perm.fill_(-7.0)
        torch.cuda.synchronize()
        ffi.moe_grouped_ffn(layer.perm, layer.w0, layer.w0_up, layer.w1, cfg.act, layer.act_buf, layer.y_perm,
                            layer.ffn_ws if use_ws else None, stream, use_workspace=use_ws)
        layer.combine(stream)
        torch.cuda.synchronize()
    finally:
        P.destroy_stream(h)
    real = np.nonzero(ref["row_src"] >= 0)[0]
    pad = np.setdiff1d(np.arange(layer.perm.R_cap), real)
    padt = torch.from_numpy(pad).to(dev)
    assert torch.all(layer.act_buf[padt] == -7.0) and torch.all(layer.y_perm[padt] == -7.0)
    what = "whole last round" + (" workspace" if use_ws else " no workspace")
    P.check_ffn_rows(cfg, d, ref, layer.act_buf, layer.y_perm, real, what)
    ref_out = O.moe_layer_expert_major(P.to_np64(d["x"]), cfg.k, P.host_weights64(d), cfg.act, (idx, w),
                                       list(range(cfg.T)))
    P.assert_output_close(layer.out.cpu().double().numpy(), ref_out, what + " out")


def test_layer_on_seven_xcds(dev):
    # The persistent grid follows the stream's CU mask: 224 CUs -> 224 workgroups.  Layer0 then has
    # 224 whole items and 32 left over (7 K slices); layer1 has fewer items than CUs (grid of 80).
    cfg = W.CONFIGS["mixtral"].with_(T=1536, H=1024, F=2048)
    d = W.make_inputs(cfg, dev)
    idx, w = P.oracle_route(d["logits"], cfg.k)
    ref = P.oracle_permute(idx, None, cfg, cfg.tile_m)
    nt = len(ref["tiles"])
    tcap = ffi.tiles_capacity(cfg.T, cfg.k, cfg.n_local, cfg.tile_m)
    n = torch.cuda.get_device_properties(dev).multi_processor_count
    cus = list(range(n // 8, n))
    sched = P.ffn_schedule(nt, tcap, cfg.H, cfg.F, cfg.tile_m, len(cus))
    print(f"[schedule] {sched}", flush=True)
    assert sched["layer0"]["full"] > 0 and sched["layer0"]["S"] >= 2
    h, stream = P.cu_masked_stream(cus, dev)
    try:
        layer = MoELayer.from_inputs(cfg, d)
        torch.cuda.synchronize()
        out = layer.run(stream)
        torch.cuda.synchronize()
    finally:
        P.destroy_stream(h)
    # all rows of the tiles the last round of either GEMM touches, plus a seeded sample of the rest
    tiles = ref["tiles"]
    rows = set()
    for t in sched["layer0"]["last_tiles"] + sched["layer1"]["last_tiles"]:
        le, r0 = tiles[t]
        rows.update(range(r0, min(r0 + cfg.tile_m, ref["offsets"][le] + ref["counts"][le])))
    real = np.nonzero(ref["row_src"] >= 0)[0]
    rows.update(np.random.default_rng(1).choice(real, size=96, replace=False).tolist())
    P.check_ffn_rows(cfg, d, ref, layer.act_buf, layer.y_perm, rows, "seven XCDs")
    toks = sorted({int(ref["row_src"][r]) // cfg.k for r in list(rows)[:64]})
    ref_out = O.moe_layer_expert_major(P.to_np64(d["x"]), cfg.k, P.host_weights64(d), cfg.act, (idx, w), toks)
    P.assert_output_close(out[torch.tensor(toks, device=dev)].cpu().double().numpy(), ref_out, "seven XCDs out")


# ---------------------------------------------------------------------------
# expert-parallel partition at the expert-parallel share's shape
# ---------------------------------------------------------------------------

def test_expert_parallel_partition_real_shape(dev):
    # 16384 tokens, 64 experts top-8, hidden 4096, FFN 2048: the 64-expert layer on one GPU, and
    # the 8 shares of 8 experts each (what 8 ranks of an expert-parallel group compute).  The sum of
    # the shares is the full layer: up to the fp32 order of the top-k reduce, and, where a GEMM's
    # split last round rounds an activation the other way, one bf16 ulp carried through W1.
    base = W.CONFIGS["ep_share"]
    full_cfg = base.with_(E_loc=64, num_ranks=8)
    dfull = W.make_inputs(full_cfg, dev)
    full = MoELayer.from_inputs(full_cfg, dfull)
    full.run()
    torch.cuda.synchronize()
    idx, w = P.oracle_route(dfull["logits"], full_cfg.k)
    assert np.array_equal(full.topk_idx.cpu().numpy(), idx)
    # the 64-expert layer against the oracle on sampled tokens
    toks = P.sample_tokens(full_cfg.T, 2, idx, 0, 64, seed=3)
    xs = np.zeros((full_cfg.T, full_cfg.H))
    xs[toks] = P.to_np64(dfull["x"][torch.tensor(toks, device=dev)])
    ref = O.moe_layer_expert_major(xs, full_cfg.k, P.host_weights64(dfull), full_cfg.act, (idx, w), toks, 0, 64)
    P.assert_output_close(full.out[torch.tensor(toks, device=dev)].cpu().double().numpy(), ref, "64-expert layer")
    del dfull
    full_inv = full.perm.inv_perm.reshape(-1)
    acc = torch.zeros_like(full.out)
    for r in range(8):
        c = base.with_(expert_begin=8 * r, E_loc=8)
        dr = W.make_inputs(c, dev)
        lay = MoELayer.from_inputs(c, dr)
        lay.run()
        torch.cuda.synchronize()
        real = (lay.perm.row_src >= 0).nonzero().squeeze(1)
        rows_full = full_inv[lay.perm.row_src[real].long()].long()
        a, b = lay.act_buf[real].float(), full.act_buf[rows_full].float()
        assert torch.all((a - b).abs() <= torch.maximum(a.abs(), b.abs()) * 2.0 ** -7 + 1e-5), r
        acc += lay.out
        del lay, dr
    torch.cuda.synchronize()
    f = full.out
    err = (acc - f).abs().max().item()
    print(f"[parity] 8 expert-parallel shares vs the 64-expert layer: max |err| {err:.3e}, "
          f"max |out| {f.abs().max().item():.3e}", flush=True)
    assert err <= 2e-3 * f.abs().max().item()
