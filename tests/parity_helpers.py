"""Shared helpers of the GPU parity tests: seeded inputs on both sides, oracle calls, tolerances.

Inputs come only from the seeded generators (mixture_experts_layer_moe_amd.workloads),
which are bit-identical on the CPU and the GPU; expected values come only from
the oracle.  Nothing here feeds a HIP result into the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

from mixture_experts_layer_moe_amd import workloads as W
from oracle import moe_oracle as O

# Output bar for bf16 inputs with fp32 accumulation: max |err| and relative Frobenius error.
MAX_ABS_ERR = 2e-2
REL_FROB_ERR = 1e-2


def require_gpu() -> torch.device:
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return torch.device("cuda:0")


def to_np64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16/fp32 tensor to a float64 numpy array on the host."""
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_route(logits: torch.Tensor, k: int, renormalize: bool = True):
    return O.route_topk(logits.detach().cpu().numpy(), k, renormalize)


def oracle_permute(idx: np.ndarray, src_rank, cfg: W.MoEConfig, tile_m: int):
    ranks = None if src_rank is None else src_rank.detach().cpu().numpy()
    return O.permute(idx, ranks, cfg.expert_begin, cfg.n_local, tile_m)


def assert_output_close(got: np.ndarray, ref: np.ndarray, what: str = "output"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    max_err = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / denom if denom > 0 else float(np.linalg.norm(got))
    print(f"[parity] {what}: max |err| {max_err:.3e}, rel-Frobenius {rel:.3e}", flush=True)
    assert max_err <= MAX_ABS_ERR, f"{what}: max |err| {max_err:.3e} > {MAX_ABS_ERR}"
    assert rel <= REL_FROB_ERR, f"{what}: relative Frobenius error {rel:.3e} > {REL_FROB_ERR}"
    return max_err, rel


class HostWeights:
    """Expert weights on the host as float32 numpy arrays (exact copies of the bf16 values).

    Fetched from the device tensors one expert at a time, so a sampled check of
    a large layer only moves the experts it needs.
    """

    def __init__(self, w0: torch.Tensor, w0_up, w1: torch.Tensor):
        self.w0, self.w0_up, self.w1 = w0, w0_up, w1

    def __call__(self, le: int):
        f = lambda t: None if t is None else t[le].detach().to("cpu", torch.float32).numpy()
        return f(self.w0), f(self.w0_up), f(self.w1)


def sample_tokens(T: int, n: int, idx: np.ndarray, expert_begin: int, E_loc: int, seed: int = 0):
    """First and last token, a few seeded ones, and (if any) one with no local slot."""
    rng = np.random.default_rng(seed)
    toks = {0, T - 1}
    toks.update(int(t) for t in rng.choice(T, size=min(n, T), replace=False))
    local = (idx >= expert_begin) & (idx < expert_begin + E_loc)
    none = np.nonzero(~local.any(axis=1))[0]
    if len(none):
        toks.add(int(none[0]))
    return sorted(toks)


def host_weights64(d: dict):
    """Per-expert float64 host copies of the layer's weights (exact widening of the bf16 values)."""
    f = lambda t, le: None if t is None else t[le].detach().to("cpu", torch.float64).numpy()
    return lambda le: (f(d["w0"], le), f(d["w0_up"], le), f(d["w1"], le))


def check_ffn_rows(cfg: W.MoEConfig, d: dict, perm_ref: dict, act_buf: torch.Tensor, y_perm: torch.Tensor,
                   rows, what: str):
    """Stored activation and layer-1 output of the given reorganised rows against the oracle.

    perm_ref is the oracle's permutation (its row_src names the token and slot
    of every row).  The activation is stored in bf16 (round to nearest even), so
    it must be within 2^-8 relative of the oracle's plus fp32 accumulation noise;
    the layer-1 output must meet the output bar.
    """
    rows = np.asarray(sorted(rows), dtype=np.int64)
    assert len(rows) and np.all(perm_ref["row_src"][rows] >= 0), "rows must be real rows"
    dev = act_buf.device
    xs = to_np64(d["x"])
    le_of = np.searchsorted(perm_ref["offsets"], rows, side="right") - 1
    wget = host_weights64(d)
    a_ref = np.zeros((len(rows), act_buf.shape[1]))
    y_ref = np.zeros((len(rows), y_perm.shape[1]))
    for le in np.unique(le_of):
        w0, w0u, w1 = wget(int(le))
        sel = np.nonzero(le_of == le)[0]
        for i in sel:
            xr = xs[perm_ref["row_src"][rows[i]] // cfg.k]
            g = w0 @ xr
            u = None if w0u is None else w0u @ xr
            a_ref[i] = O.activation(cfg.act, g, u)
            y_ref[i] = O.expert_ffn(xr, w0, w0u, w1, cfg.act)
    rt = torch.from_numpy(rows).to(dev)
    a_got = to_np64(act_buf[rt])
    tol = 2.0 ** -8 * np.abs(a_ref) + 1e-4 * np.sqrt(np.mean(a_ref ** 2))
    bad = np.abs(a_got - a_ref) - tol
    assert np.all(bad <= 0), f"{what}: activation off by {float(bad.max()):.3e} beyond its bound"
    assert_output_close(to_np64(y_perm[rt]), y_ref, what + " y_perm")


def ffn_schedule(nt: int, tiles_cap: int, H: int, F: int, tile_m: int, cus: int):
    """Host mirror of the grouped GEMMs' persistent schedule for tile_m >= 128.

    For layer0 (items = row tiles x 128-column blocks of F, ordered in groups
    of 8 tiles, column block major inside a group) and layer1 (row tiles x
    256-column blocks of H, or 128 when 256 does not divide H, ordered in
    groups of 4 column blocks, tile major inside a group): the grid G (one
    workgroup per usable CU rounded down to a multiple of 8, fewer if the
    capacity has fewer items), the item count, the items run in whole rounds,
    the K-slice count S of the last round (1 = none) and the tile indices
    (positions in the tile list) that the last round touches.
    """
    assert tile_m >= 128
    out = {}
    for layer, nbn, K, group, order_m in (("layer0", F // 128, H, 8, True),
                                          ("layer1", H // (256 if H % 256 == 0 else 128), F, 4, False)):
        max_items = tiles_cap * nbn
        G = cus // 8 * 8
        if max_items < G:
            G = -(-max_items // 8) * 8
        G = max(G, 8)
        total = nt * nbn
        full = total // G * G
        rem = total - full
        S = 1 if rem == 0 else max(1, min(8, G // rem, K // 64))
        tiles = set()
        for item in range(full, total):
            if order_m:
                per = group * nbn
                grp, r = divmod(item, per)
                gsize = min(group, nt - grp * group)
                tiles.add(grp * group + r % gsize)
            else:
                per = nt * group
                g, r = divmod(item, per)
                gsize = min(group, nbn - g * group)
                tiles.add(r // gsize)
        out[layer] = {"G": G, "total": total, "full": full, "S": S, "last_tiles": sorted(tiles)}
    return out


def cu_masked_stream(cus, dev):
    """A stream whose kernels may use only the listed CUs (default priority); returns (handle, stream)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    n = torch.cuda.get_device_properties(dev).multi_processor_count
    words = (n + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for c in cus:
        mask[c // 32] |= 1 << (c % 32)
    h = ctypes.c_void_p()
    err = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(words), mask)
    assert err == 0, f"hipExtStreamCreateWithCUMask failed ({err})"
    return h, torch.cuda.ExternalStream(h.value, device=dev)


def destroy_stream(h):
    import ctypes
    torch.cuda.synchronize()
    assert ctypes.CDLL("libamdhip64.so").hipStreamDestroy(h) == 0
