"""Parity of the HIP path with the CPU oracle, call by call and for the whole layer.

Every case runs through the C ABI (libmoe.so via the ctypes binding).  Inputs
are the seeded synthetic workloads; expected values come from the oracle
only.  Routing indices, the permutation, the tile list and the reorganised
rows must be bit-exact; floating-point outputs must meet max |err| <= 2e-2 and
relative Frobenius error <= 1e-2 (bf16 inputs, fp32 accumulation).

Full-size workloads run in the launch configuration the benchmark uses (the
workload's own tile_m); their outputs are checked on sampled tokens that the
oracle computes one by one, and their routing and permutation in full.
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

TILE_MS = [16, 32, 64, 128, 256]


@pytest.fixture(scope="module")
def dev():
    d = P.require_gpu()
    ffi.lib()  # loud failure if the library is missing
    return d


def bits16(t):
    return t.contiguous().view(torch.int16)


# ---------------------------------------------------------------------------
# input generators: bit-identical on both sides
# ---------------------------------------------------------------------------

def test_generators_bit_identical_on_gpu(dev):
    a = W.normal_tensor((333, 129), 0.02, seed=0, tid=W.TID_W0, expert=5)
    b = W.normal_tensor((333, 129), 0.02, seed=0, tid=W.TID_W0, expert=5, device=dev)
    assert torch.equal(bits16(a), bits16(b).cpu())
    for name in ["tiny", "fine_grained", "ep_share"]:
        cfg = W.CONFIGS[name].with_(T=77)
        hc = W.make_inputs(cfg.with_(H=128, F=128), "cpu", weights=False)
        gc = W.make_inputs(cfg.with_(H=128, F=128), dev, weights=False)
        assert torch.equal(bits16(hc["x"]), bits16(gc["x"]).cpu())
        assert torch.equal(hc["logits"].view(torch.int32), gc["logits"].cpu().view(torch.int32))
        if hc["src_rank"] is not None:
            assert torch.equal(hc["src_rank"], gc["src_rank"].cpu())


# ---------------------------------------------------------------------------
# moe_route_topk
# ---------------------------------------------------------------------------

def check_route(logits_cpu, k, renormalize, dev):
    idx_o, w_o = P.oracle_route(logits_cpu, k, renormalize)
    idx_g, w_g = ffi.moe_route_topk(logits_cpu.to(dev), k, renormalize)
    assert np.array_equal(idx_g.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w_g.cpu().numpy(), w_o, rtol=2e-6, atol=1e-7)
    return idx_o


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_route_full_size(dev, name):
    cfg = W.CONFIGS[name]
    logits = W.make_logits(cfg, dev).cpu()
    check_route(logits, cfg.k, True, dev)


@pytest.mark.parametrize("T,E,k,kind,renorm", [
    (1, 8, 2, "normal", True),
    (130, 1, 1, "normal", True),          # single expert
    (200, 6, 6, "normal", True),          # k = E
    (257, 8, 2, "ties", True),            # many equal logits: lower id first
    (100, 65, 3, "ties", True),           # E not a multiple of the wave
    (64, 64, 8, "ties", True),            # four lanes per token (E <= 64, k <= 8): merged top-k lists
    (50, 64, 4, "ties", False),           # same, full-softmax gate
    (300, 50, 5, "ties", True),           # E not a multiple of 4: scalar logit loads
    (70, 64, 12, "ties", True),           # k > 8 with E <= 64: one logit per lane, ballot tie-break
    (33, 17, 9, "normal", False),         # same, full-softmax gate
    (64, 1024, 32, "normal", True),       # largest supported E and k
    (300, 16, 4, "normal", False),        # full-softmax weights
])
def test_route_edge_cases(dev, T, E, k, kind, renorm):
    g = torch.Generator().manual_seed(T * 1000 + E)
    if kind == "ties":
        logits = torch.randint(-2, 3, (T, E), generator=g).to(torch.float32)
    else:
        logits = torch.randn((T, E), generator=g, dtype=torch.float32)
    check_route(logits, k, renorm, dev)


# ---------------------------------------------------------------------------
# moe_permute (inputs: oracle routing of seeded logits)
# ---------------------------------------------------------------------------

def check_permute(x, idx_np, src_rank, E, expert_begin, E_loc, num_ranks, tile_m, dev):
    T, H = x.shape
    k = idx_np.shape[1]
    ranks_np = None if src_rank is None else src_rank.cpu().numpy()
    ref = O.permute(idx_np, ranks_np, expert_begin, E_loc, tile_m)
    xd = x.to(dev)
    p = ffi.moe_permute(xd, torch.from_numpy(idx_np.astype(np.int32)).to(dev),
                        None if src_rank is None else src_rank.to(dev),
                        E, expert_begin, E_loc, num_ranks, tile_m)
    torch.cuda.synchronize()
    off = ref["offsets"]
    assert p.expert_counts.cpu().numpy().tolist() == ref["counts"].tolist()
    assert p.expert_offsets.cpu().numpy().tolist() == off.tolist()
    rs = p.row_src.cpu().numpy()
    assert np.array_equal(rs[:off[-1]], ref["row_src"])
    assert np.all(rs[off[-1]:] == -1)
    assert np.array_equal(p.inv_perm.cpu().numpy(), ref["inv_perm"])
    nt = int(p.num_tiles.item())
    assert nt == len(ref["tiles"])
    assert [tuple(r) for r in p.tiles[:nt].cpu().numpy().tolist()] == [tuple(t) for t in ref["tiles"]]
    real = np.nonzero(ref["row_src"] >= 0)[0]
    if len(real):
        rows = torch.from_numpy(real).to(dev)
        toks = torch.from_numpy(ref["row_src"][real] // k).to(dev)
        assert torch.equal(bits16(p.x_perm[rows]), bits16(xd[toks]))
    return ref, p


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_permute_full_size(dev, name):
    cfg = W.CONFIGS[name]
    d = W.make_inputs(cfg, dev, weights=False)
    idx, _ = P.oracle_route(d["logits"], cfg.k)
    check_permute(d["x"], idx, d["src_rank"], cfg.E, cfg.expert_begin, cfg.n_local, cfg.num_ranks,
                  cfg.tile_m, dev)


@pytest.mark.parametrize("tile_m", TILE_MS)
def test_permute_tile_sizes_with_ranks(dev, tile_m):
    cfg = W.MoEConfig("t", T=333, H=64, F=128, E=16, k=4, act="swiglu", logits="normal",
                      tile_m=tile_m, expert_begin=4, E_loc=6, num_ranks=5)
    d = W.make_inputs(cfg, dev, weights=False)
    idx, _ = P.oracle_route(d["logits"], cfg.k)
    check_permute(d["x"], idx, d["src_rank"], cfg.E, 4, 6, 5, tile_m, dev)


def test_permute_many_tiles_with_ranks(dev):
    # More than 4096 tiles with source ranks: each tile's place in the list comes from per-(priority,
    # expert) tile counts over many tiles of every expert; the order must be the oracle's.
    cfg = W.MoEConfig("m", T=8300, H=64, F=128, E=64, k=8, act="swiglu", logits="normal",
                      tile_m=16, num_ranks=4)
    d = W.make_inputs(cfg, dev, weights=False)
    idx, _ = P.oracle_route(d["logits"], cfg.k)
    assert ffi.tiles_capacity(cfg.T, cfg.k, cfg.n_local, 16) > 4096
    check_permute(d["x"], idx, d["src_rank"], cfg.E, 0, 64, 4, 16, dev)


def test_permute_large_histogram(dev):
    # 4096 (expert, rank) buckets x 47 chunks of 256 tokens: too many per-chunk counts to copy into every
    # placing block (placing blocks x buckets x chunks > 2^23 at every tokens-per-wave choice), so the
    # single-block scan runs between the count and place launches.
    cfg = W.MoEConfig("m", T=12000, H=64, F=128, E=512, k=4, act="swiglu", logits="normal",
                      tile_m=32, num_ranks=8)
    d = W.make_inputs(cfg, dev, weights=False)
    idx, _ = P.oracle_route(d["logits"], cfg.k)
    nb, nc = 512 * 8, (cfg.T + 255) // 256
    assert (1 + (cfg.T + 255) // 256) * nb * nc > 1 << 23
    check_permute(d["x"], idx, d["src_rank"], cfg.E, 0, 512, 8, 32, dev)


@pytest.mark.parametrize("case", ["one_token", "all_to_one_expert", "max_buckets", "k_equals_E",
                                  "no_local_pairs", "exact_tile_multiple"])
def test_permute_edge_cases(dev, case):
    g = torch.Generator().manual_seed(7)
    T, H, E, k, e0, El, R, tm = 200, 64, 8, 2, 0, 8, 1, 32
    if case == "one_token":
        T = 1
    if case == "max_buckets":
        T, E, k, El, R, tm = 300, 64, 4, 64, 64, 16
    if case == "k_equals_E":
        E, k, El = 4, 4, 4
    logits = torch.randn((T, E), generator=g)
    if case == "all_to_one_expert":
        logits[:, 3] += 100.0
        k = 1
    if case == "no_local_pairs":
        logits[:, :4] += 100.0          # top-2 always among experts 0..3
        e0, El = 4, 4
    if case == "exact_tile_multiple":
        T, k, tm = 64, 1, 16
        logits = torch.zeros((T, E))
        logits[torch.arange(T), torch.arange(T) % 4] = 1.0   # 16 tokens on each of experts 0..3
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    ranks = torch.randint(0, R, (T,), generator=g, dtype=torch.int32) if R > 1 else None
    idx, _ = O.route_topk(logits.numpy(), k)
    ref, p = check_permute(x, idx, ranks, E, e0, El, R, tm, dev)
    if case == "no_local_pairs":
        assert int(p.num_tiles.item()) == 0 and np.all(p.inv_perm.cpu().numpy() == -1)


# ---------------------------------------------------------------------------
# moe_grouped_ffn (inputs: oracle reorganisation of seeded tokens)
# ---------------------------------------------------------------------------

def host_reorganised(cfg, x, idx, src_rank, tile_m, dev):
    """x_perm / counts / offsets / tiles built on the host from the oracle's permutation.

    Padding rows and the unused tail are NaN, so a leak of a padding row into
    a real output would show.
    """
    T, k = idx.shape
    ref = P.oracle_permute(idx, src_rank, cfg, tile_m)
    R_cap = ffi.rows_capacity(T, k, cfg.n_local, tile_m)
    tcap = ffi.tiles_capacity(T, k, cfg.n_local, tile_m)
    x_perm = torch.full((R_cap, cfg.H), float("nan"), dtype=torch.bfloat16, device=dev)
    real = np.nonzero(ref["row_src"] >= 0)[0]
    if len(real):
        x_perm[torch.from_numpy(real).to(dev)] = x.to(dev)[torch.from_numpy(ref["row_src"][real] // k).to(dev)]
    i32 = lambda a: torch.tensor(np.asarray(a, dtype=np.int32), device=dev)
    tiles = torch.full((tcap, 2), -1, dtype=torch.int32, device=dev)
    if ref["tiles"]:
        tiles[:len(ref["tiles"])] = i32(ref["tiles"])
    perm = ffi.Permuted(x_perm=x_perm, expert_counts=i32(ref["counts"]), expert_offsets=i32(ref["offsets"]),
                        row_src=i32(np.concatenate([ref["row_src"], -np.ones(R_cap - len(ref["row_src"]))])),
                        inv_perm=i32(ref["inv_perm"]), tiles=tiles, num_tiles=i32([len(ref["tiles"])]),
                        tile_m=tile_m, R_cap=R_cap, tiles_cap=tcap)
    return ref, perm


def check_grouped_ffn(cfg, tile_m, dev, max_rows=None):
    d = W.make_inputs(cfg, dev)
    idx, _ = P.oracle_route(d["logits"], cfg.k)
    ref, perm = host_reorganised(cfg, d["x"], idx, d["src_rank"], tile_m, dev)
    act_buf = torch.full((perm.R_cap, cfg.F_loc), -7.0, dtype=torch.bfloat16, device=dev)
    y_perm = torch.full((perm.R_cap, cfg.H), -7.0, dtype=torch.float32, device=dev)
    ffi.moe_grouped_ffn(perm, d["w0"], d["w0_up"], d["w1"], cfg.act, act_buf, y_perm)
    torch.cuda.synchronize()
    real = np.nonzero(ref["row_src"] >= 0)[0]
    pad = np.setdiff1d(np.arange(perm.R_cap), real)
    # padding rows are never written
    if len(pad):
        padt = torch.from_numpy(pad).to(dev)
        assert torch.all(act_buf[padt] == -7.0) and torch.all(y_perm[padt] == -7.0)
    rows = real if max_rows is None else np.random.default_rng(0).choice(real, size=min(max_rows, len(real)),
                                                                          replace=False)
    xs = P.to_np64(d["x"])
    wh = P.HostWeights(d["w0"], d["w0_up"], d["w1"])
    le_of = np.searchsorted(ref["offsets"], rows, side="right") - 1
    y_ref = np.zeros((len(rows), cfg.H))
    a_ref = np.zeros((len(rows), cfg.F_loc))
    cache = {}
    for i, (r, le) in enumerate(zip(rows, le_of)):
        if le not in cache:
            cache.clear()
            cache[le] = wh(int(le))
        w0, w0u, w1 = cache[le]
        xr = xs[ref["row_src"][r] // cfg.k]
        g = w0.astype(np.float64) @ xr
        u = None if w0u is None else w0u.astype(np.float64) @ xr
        a_ref[i] = O.activation(cfg.act, g, u)
        y_ref[i] = O.expert_ffn(xr, w0, w0u, w1, cfg.act)
    rt = torch.from_numpy(rows).to(dev)
    a_got = P.to_np64(act_buf[rt])
    # the activation is stored in bf16 (round to nearest even): within 2^-8 relative plus fp32 noise
    tol = 2.0 ** -8 * np.abs(a_ref) + 1e-4 * np.sqrt(np.mean(a_ref ** 2))
    assert np.all(np.abs(a_got - a_ref) <= tol), float(np.max(np.abs(a_got - a_ref) - tol))
    P.assert_output_close(P.to_np64(y_perm[rt]), y_ref, "y_perm")


def test_grouped_ffn_tiny_gelu(dev):
    check_grouped_ffn(W.CONFIGS["tiny"], 64, dev)


@pytest.mark.parametrize("tile_m", TILE_MS)
def test_grouped_ffn_swiglu_tile_sizes(dev, tile_m):
    cfg = W.MoEConfig("s", T=160, H=256, F=384, E=4, k=2, act="swiglu", logits="normal", tile_m=tile_m)
    check_grouped_ffn(cfg, tile_m, dev)


@pytest.mark.parametrize("tile_m", [16, 128])
def test_grouped_ffn_gelu_ranks_and_ragged(dev, tile_m):
    cfg = W.MoEConfig("g", T=211, H=384, F=256, E=12, k=3, act="gelu", logits="normal", tile_m=tile_m,
                      expert_begin=2, E_loc=5, num_ranks=3)
    check_grouped_ffn(cfg, tile_m, dev)


@pytest.mark.parametrize("tile_m", TILE_MS)
@pytest.mark.parametrize("H,F", [(128, 128), (128, 256), (256, 128)])
def test_grouped_ffn_shortest_k(dev, tile_m, H, F):
    # K of 128 or 256 is 2 or 4 stages of 64: shorter than the load pipelines (the register stage
    # loads two stages ahead, the small-tile ring keeps three in flight), so their prologue and
    # end-of-K handling run without a steady state in between.
    cfg = W.MoEConfig("k", T=300, H=H, F=F, E=6, k=2, act="swiglu", logits="normal", tile_m=tile_m)
    check_grouped_ffn(cfg, tile_m, dev)


def test_grouped_ffn_zipf_uneven_experts(dev):
    cfg = W.CONFIGS["fine_grained"].with_(T=512, H=256, F=256)
    check_grouped_ffn(cfg, cfg.tile_m, dev)


# ---------------------------------------------------------------------------
# moe_combine (inputs: seeded y rows, oracle routing and permutation)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_combine_full_size(dev, name):
    cfg = W.CONFIGS[name]
    logits = W.make_logits(cfg, dev)
    idx, w = P.oracle_route(logits, cfg.k)
    src = W.make_src_rank(cfg, dev)
    ref = P.oracle_permute(idx, src, cfg, cfg.tile_m)
    R_cap = ffi.rows_capacity(cfg.T, cfg.k, cfg.n_local, cfg.tile_m)
    y = W.normal_tensor((R_cap, cfg.H), 1.0, cfg.seed, 99, device=dev, dtype=torch.float32)
    w32 = w.astype(np.float32)
    out = ffi.moe_combine(y, torch.from_numpy(ref["inv_perm"].astype(np.int32)).to(dev),
                          torch.from_numpy(w32).to(dev))
    torch.cuda.synchronize()
    toks = np.arange(cfg.T) if cfg.T <= 4096 else np.arange(0, cfg.T, 4)
    inv_s = ref["inv_perm"][toks]
    # Only the rows the sampled tokens use go to the host, renumbered compactly
    # (the reduce does not depend on where a row is stored).
    used = np.unique(inv_s[inv_s >= 0])
    y_host = np.zeros((len(used), cfg.H))
    if len(used):
        y_host[:] = P.to_np64(y[torch.from_numpy(used).to(dev)])
    compact = np.where(inv_s >= 0, np.searchsorted(used, inv_s), -1)
    expect = O.combine(y_host, compact, w32.astype(np.float64)[toks])
    got = P.to_np64(out[torch.from_numpy(toks).to(dev)])
    np.testing.assert_allclose(got, expect, rtol=1e-5, atol=1e-5)
    none = ~(inv_s >= 0).any(axis=1)
    assert np.all(got[none] == 0.0)


# ---------------------------------------------------------------------------
# the whole layer through the four calls
# ---------------------------------------------------------------------------

def run_layer(cfg, dev, tile_m=None, fused_gather=False):
    d = W.make_inputs(cfg, dev)
    layer = MoELayer.from_inputs(cfg, d, tile_m=tile_m, fused_gather=fused_gather)
    out = layer.run()
    torch.cuda.synchronize()
    return d, layer, out


def check_layer_routing_and_permutation(cfg, d, layer):
    idx, w = P.oracle_route(d["logits"], cfg.k)
    assert np.array_equal(layer.topk_idx.cpu().numpy(), idx)
    np.testing.assert_allclose(layer.topk_w.cpu().numpy(), w, rtol=2e-6, atol=1e-7)
    ref = P.oracle_permute(idx, d["src_rank"], cfg, layer.tile_m)
    assert np.array_equal(layer.perm.inv_perm.cpu().numpy(), ref["inv_perm"])
    nt = int(layer.perm.num_tiles.item())
    assert [tuple(r) for r in layer.perm.tiles[:nt].cpu().numpy().tolist()] == [tuple(t) for t in ref["tiles"]]
    return idx, w


SMALL_LAYERS = {
    "tiny": W.CONFIGS["tiny"],
    "mixtral_small": W.CONFIGS["mixtral"].with_(T=300, H=512, F=640, tile_m=64),
    "fine_grained_small": W.CONFIGS["fine_grained"].with_(T=700, H=256, F=384, tile_m=32),
    "ep_share_small": W.CONFIGS["ep_share"].with_(T=900, H=256, F=256, tile_m=64),
    "decode_small": W.CONFIGS["decode"].with_(T=64, H=512, F=256, E=64),
}


@pytest.mark.parametrize("fused_gather", [False, True], ids=["x_perm", "gather"])
@pytest.mark.parametrize("name", list(SMALL_LAYERS))
def test_layer_small_full_check(dev, name, fused_gather):
    cfg = SMALL_LAYERS[name]
    d, layer, out = run_layer(cfg, dev, fused_gather=fused_gather)
    idx, w = check_layer_routing_and_permutation(cfg, d, layer)
    wh = P.HostWeights(d["w0"], d["w0_up"], d["w1"])
    ref = O.moe_layer_expert_major(P.to_np64(d["x"]), cfg.k, wh, cfg.act, (idx, w), list(range(cfg.T)),
                                   cfg.expert_begin, cfg.n_local)
    P.assert_output_close(out.cpu().double().numpy(), ref, name + (" (fused gather)" if fused_gather else ""))


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_fused_gather_matches_permuted_copy(dev, name):
    # Layer0 reading its rows from x through row_src (index-only permute, no x_perm) must give the
    # same activation, layer1 output and layer output, bit for bit, as reading the permuted copy: the
    # operand values and the accumulation order are the same.
    cfg = W.CONFIGS[name]
    d = W.make_inputs(cfg, dev)
    a = MoELayer.from_inputs(cfg, d)
    b = MoELayer.from_inputs(cfg, d, fused_gather=True)
    a.run()
    b.run()
    torch.cuda.synchronize()
    assert b.perm.x_perm is None
    for t in ("expert_counts", "expert_offsets", "row_src", "inv_perm", "num_tiles"):
        assert torch.equal(getattr(a.perm, t), getattr(b.perm, t)), t
    nt = int(a.perm.num_tiles.item())
    assert torch.equal(a.perm.tiles[:nt], b.perm.tiles[:nt])
    real = (a.perm.row_src >= 0).nonzero().squeeze(1)
    assert torch.equal(bits16(a.act_buf[real]), bits16(b.act_buf[real]))
    assert torch.equal(a.y_perm[real].view(torch.int32), b.y_perm[real].view(torch.int32))
    assert torch.equal(a.out.view(torch.int32), b.out.view(torch.int32))


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_layer_full_size_sampled(dev, name):
    cfg = W.CONFIGS[name]
    d, layer, out = run_layer(cfg, dev)
    idx, w = check_layer_routing_and_permutation(cfg, d, layer)
    toks = set(P.sample_tokens(cfg.T, 6, idx, cfg.expert_begin, cfg.n_local))
    if layer.tile_m >= 128:
        # Besides the seeded sample: the tokens of the first and last real row of every row tile that
        # the last scheduling round of either GEMM touches (split along K into partial tiles summed by
        # a second kernel), derived from the item order on the host.
        ref = P.oracle_permute(idx, d["src_rank"], cfg, layer.tile_m)
        n_cus = torch.cuda.get_device_properties(dev).multi_processor_count
        sched = P.ffn_schedule(len(ref["tiles"]), layer.perm.tiles_cap, cfg.H, cfg.F_loc, layer.tile_m, n_cus)
        last = sorted(set(sched["layer0"]["last_tiles"]) | set(sched["layer1"]["last_tiles"]))
        print(f"[schedule] {name}: {sched}", flush=True)
        for ti in last:
            le, r0 = ref["tiles"][ti]
            r1 = min(r0 + layer.tile_m, ref["offsets"][le] + ref["counts"][le]) - 1
            toks.update({int(ref["row_src"][r0]) // cfg.k, int(ref["row_src"][r1]) // cfg.k})
    toks = sorted(toks)
    wh = P.HostWeights(d["w0"], d["w0_up"], d["w1"])
    xs = P.to_np64(d["x"][torch.tensor(toks, device=dev)])
    xfull = np.zeros((cfg.T, cfg.H))
    xfull[toks] = xs
    ref = O.moe_layer_expert_major(xfull, cfg.k, wh, cfg.act, (idx, w), toks, cfg.expert_begin, cfg.n_local)
    got = out[torch.tensor(toks, device=dev)].cpu().double().numpy()
    P.assert_output_close(got, ref, name)


def test_layer_is_deterministic(dev):
    cfg = W.CONFIGS["fine_grained"].with_(T=2048, H=512, F=384)
    d = W.make_inputs(cfg, dev)
    layer = MoELayer.from_inputs(cfg, d)
    a = layer.run().clone()
    y1 = layer.y_perm.clone()
    b = layer.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(y1.view(torch.int32), layer.y_perm.view(torch.int32))


def test_layer_graph_capture_replays_match_eager(dev):
    # The four calls need no host synchronisation, so the layer can be captured and replayed.
    cfg = W.CONFIGS["ep_share"].with_(T=1024, H=256, F=256, tile_m=64)
    d = W.make_inputs(cfg, dev)
    layer = MoELayer.from_inputs(cfg, d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.run()
    torch.cuda.current_stream().wait_stream(s)
    eager = layer.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.run()
    for _ in range(3):
        layer.out.fill_(123.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out.view(torch.int32), eager.view(torch.int32))


def test_tensor_parallel_partials_sum_to_full_layer(dev):
    # Each tensor-parallel rank computes its FFN column slice of every local expert; the partial
    # outputs over all ranks sum to the full layer's output.  The activations of a slice are
    # bitwise those of the full layer's columns (same rows, same K order), so the sum differs from
    # the full output only by the fp32 order of layer1's F reduction.
    cfg = W.CONFIGS["ep_share"].with_(T=1024, H=256, F=512, tile_m=64)
    full = MoELayer.from_inputs(cfg, W.make_inputs(cfg, dev))
    full.run()
    parts = []
    for r in range(4):
        c = cfg.with_(tp=4, tp_rank=r)
        lay = MoELayer.from_inputs(c, W.make_inputs(c, dev))
        lay.run()
        torch.cuda.synchronize()
        cols = slice(r * c.F_loc, (r + 1) * c.F_loc)
        real = (lay.perm.row_src >= 0).nonzero().squeeze(1)
        assert torch.equal(bits16(lay.act_buf[real]), bits16(full.act_buf[real][:, cols]))
        parts.append(lay.out.clone())
    torch.cuda.synchronize()
    f = full.out
    err = (sum(parts) - f).abs().max().item()
    print(f"[parity] tp=4 partial sum vs full layer: max |err| {err:.3e}, max |out| {f.abs().max().item():.3e}")
    assert err <= 1e-5 * f.abs().max().item()


@pytest.mark.parametrize("tile_m", [64, 256])
def test_expert_parallel_shares_sum_to_full_layer(dev, tile_m):
    # Expert parallelism on one GPU: each of 4 ranks runs the layer over its own 2 of the 8 experts
    # (the tokens' other slots are not local to it); the rank outputs sum to the full layer's.  A
    # rank's rows are the full layer's rows of its experts, so their activations agree bitwise and
    # the sum differs from the full output only by the fp32 order of the top-k reduce.  With 256-row
    # tiles the last scheduling round of each GEMM is split along K and summed in another fp32
    # order, and which items fall in that round differs between a rank and the full layer: there an
    # activation may differ by a bf16 ulp (or by fp32 noise near zero), and the outputs by what such
    # flips carry through W1.
    cfg = W.CONFIGS["mixtral"].with_(T=1024, H=256, F=512, tile_m=tile_m)
    split = tile_m >= 128
    full = MoELayer.from_inputs(cfg, W.make_inputs(cfg, dev))
    full.run()
    full_inv = full.perm.inv_perm.reshape(-1)
    parts = []
    for r in range(4):
        c = cfg.with_(expert_begin=2 * r, E_loc=2)
        lay = MoELayer.from_inputs(c, W.make_inputs(c, dev))
        lay.run()
        torch.cuda.synchronize()
        real = (lay.perm.row_src >= 0).nonzero().squeeze(1)
        full_rows = full_inv[lay.perm.row_src[real].long()].long()
        a, b = lay.act_buf[real], full.act_buf[full_rows]
        if split:
            # an ulp of the larger magnitude, plus an absolute floor for activations near zero
            af, bf = a.float(), b.float()
            assert torch.all((af - bf).abs() <= torch.maximum(af.abs(), bf.abs()) * 2.0 ** -7 + 1e-5)
        else:
            assert torch.equal(bits16(a), bits16(b))
        parts.append(lay.out.clone())
    torch.cuda.synchronize()
    f = full.out
    err = (sum(parts) - f).abs().max().item()
    print(f"[parity] ep=4 share sum vs full layer (tile_m {tile_m}): max |err| {err:.3e}, "
          f"max |out| {f.abs().max().item():.3e}")
    assert err <= (2e-3 if split else 1e-5) * f.abs().max().item()


@pytest.mark.parametrize("name,over", [
    ("mixtral", {}),
    # GELU (one layer0 matrix): 35 row tiles x 32 column blocks = 1120 layer0 items, 96 left for the last round
    ("mixtral", {"act": "gelu", "H": 1024, "F": 4096}),
])
def test_grouped_ffn_split_k_last_round(dev, name, over):
    # Mixtral shape: 35 row tiles x 112 layer0 / 16 layer1 column blocks on 256 CUs leave 80 layer0 and 48
    # layer1 items for the last round, which with the workspace run as K slices (3 and 5 of them) summed by
    # a second kernel, without it as half-width pieces.  The two must agree to fp32 summation-order noise
    # (layer0: an ulp of the bf16 activation where the rounding flips), and the split path must be bitwise
    # reproducible.
    cfg = W.CONFIGS[name].with_(**over)
    d = W.make_inputs(cfg, dev)
    layer = MoELayer.from_inputs(cfg, d)
    layer.route()
    layer.permute()
    a1, y1 = ffi.moe_grouped_ffn(layer.perm, d["w0"], d["w0_up"], d["w1"], cfg.act, use_workspace=False)
    a2, y2 = ffi.moe_grouped_ffn(layer.perm, d["w0"], d["w0_up"], d["w1"], cfg.act)
    a3, y3 = ffi.moe_grouped_ffn(layer.perm, d["w0"], d["w0_up"], d["w1"], cfg.act)
    torch.cuda.synchronize()
    real = (layer.perm.row_src >= 0).nonzero().squeeze(1)
    a1r, a2r, a3r = a1[real], a2[real], a3[real]
    assert torch.equal(bits16(a2r), bits16(a3r))
    # An ulp of the larger magnitude, plus an absolute floor far above the fp32 summation noise for the
    # activations that pass near zero (where an ulp is tiny).
    a1f, a2f = a1r.float(), a2r.float()
    da = (a1f - a2f).abs()
    bound = torch.maximum(a1f.abs(), a2f.abs()) * 2.0 ** -7 + 1e-5
    worst = int(torch.argmax(da - bound))
    r, c = divmod(worst, a1f.shape[1])
    assert torch.all(da <= bound), (f"layer0 split differs by more than a bf16 ulp at row {r} col {c}: "
                                    f"{a1f[r, c].item()} vs {a2f[r, c].item()}")
    assert (da > 0).float().mean().item() < 1e-2
    y1r, y2r, y3r = y1[real], y2[real], y3[real]
    assert torch.equal(y2r.view(torch.int32), y3r.view(torch.int32))
    # y: fp32 summation-order noise, plus what the flipped activations carry through W1 (|da| . |W1|^T,
    # exact bound of the layer1 difference the activation difference can cause).
    scale = y1r.abs().max().item()
    dact = (a1.float() - a2.float()).abs()
    dact[layer.perm.row_src < 0] = 0
    carried = torch.zeros_like(y1)
    offs = layer.perm.expert_offsets.cpu().tolist()
    for e in range(cfg.n_local):
        lo, hi = offs[e], offs[e + 1]
        if hi > lo and bool(dact[lo:hi].any()):
            carried[lo:hi] = dact[lo:hi] @ d["w1"][e].float().abs().t().contiguous()
    assert torch.all((y2r - y1r).abs() <= carried[real] * 1.001 + 1e-5 * scale)
