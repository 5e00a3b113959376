"""Seeded synthetic MoE-layer workloads: shapes and input generators.

This module only *makes inputs*. It holds none of the layer's arithmetic
(no routing, no sorting, no expert FFN, no reduction), so both the CPU oracle
side and the HIP side can draw from it without sharing any of the method.

Generator design
----------------
Every element is a pure function of (seed, tensor id, expert, element index):

    h   = lowbias32((q * K1 + K2) mod 2^32)      q = element-pair counter
    u16 = high or low 16 bits of h               (two elements per hash)
    val = QUANTILE_TABLE[u16] * std              (fp32 multiply, then RNE cast)

`lowbias32` is Chris Wellons' 32-bit integer hash ("Prospecting for Hash
Functions", 2018).  All hash steps are exact int64 tensor operations (no
product ever exceeds 2^63), the table lookup is a gather, and the only float
operation is one correctly-rounded fp32 multiply followed by a
round-to-nearest-even cast.  The values are therefore bit-identical whether
the generator runs on the CPU or on a GPU, which lets a full-size layer be
generated on the device in well under a second while the oracle regenerates
exactly the same values for the experts it samples on the host.

Distributions: the quantile tables hold the inverse CDF of N(0,1) (or of the
standard Gumbel law) at the midpoints of 2^16 (x, weights) or 2^20 (logits)
equal-probability cells, i.e. a discretised normal whose resolution is far
finer than bf16's 8-bit mantissa and whose tails reach about 4.3 sigma
(2^16 cells) or 4.9 sigma (2^20 cells).

Workload shapes follow the MoE-layer problem statement (tokens x hidden, E
experts, top-k, per-expert FFN weights) of "Comet: Fine-grained
Computation-communication Overlapping for Mixture-of-Experts", section 2.1
(MoE Structure).  The expert-parallel share (source-rank labels, a local
expert range) follows the same page's section 2.1 (expert parallelism) and
section 3.1.2 (tokens sorted by source rank).

Weight storage is output-major per expert: the layer-0 matrices are stored as
[F, H] (row f holds the H input weights of FFN unit f) and the layer-1 matrix
as [H, F].  Mathematically the layer computes x . W with W of shape H x F and
F x H; the stored arrays are those matrices transposed, which makes the
reduction (K) dimension contiguous for both GEMM operands.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import torch

_M32 = 0xFFFFFFFF

# Tensor ids used to derive per-tensor keys.
TID_X = 1
TID_LOGITS = 2
TID_RANK = 3
TID_ROUTER = 4
TID_W0 = 10      # W_gate (SwiGLU) or W1 (GELU), stored [F, H]
TID_W0_UP = 11   # W_up (SwiGLU only), stored [F, H]
TID_W1 = 12      # W_down (SwiGLU) or W2 (GELU), stored [H, F]


def _lowbias32_int(x: int) -> int:
    """lowbias32 on a Python int (used for key derivation only)."""
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 tensors holding values in [0, 2^32).

    The product is split into 16-bit halves of x so that no intermediate
    exceeds 2^48: exact, overflow-free int64 arithmetic on any device.
    """
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + ((hi * c) & 0xFFFF) * 65536) & _M32


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _keys(seed: int, tid: int, expert: int):
    base = _lowbias32_int((seed * 0x9E3779B1 + tid * 0x85EBCA6B + 0x165667B1) & _M32)
    k1 = (_lowbias32_int(base ^ ((expert * 0xC2B2AE35 + 0x27D4EB2F) & _M32)) & 0x7FFFFFFF) | 1
    k2 = _lowbias32_int(k1 ^ 0x61C88647)
    return k1, k2


def _hash32(n: int, seed: int, tid: int, expert: int, device) -> torch.Tensor:
    """n 32-bit hash values (int64 tensor), counter 0..n-1."""
    k1, k2 = _keys(seed, tid, expert)
    q = torch.arange(n, dtype=torch.int64, device=device)
    # q < 2^31 and k1 < 2^31, so q * k1 < 2^62: exact.
    return _lowbias32((q * k1 + k2) & _M32)


def _u16(n: int, seed: int, tid: int, expert: int, device) -> torch.Tensor:
    """n uniform 16-bit integers; each hash supplies two of them."""
    h = _hash32((n + 1) // 2, seed, tid, expert, device)
    return torch.stack((h >> 16, h & 0xFFFF), dim=1).reshape(-1)[:n]


def _u20(n: int, seed: int, tid: int, expert: int, device) -> torch.Tensor:
    """n uniform 20-bit integers, one hash each."""
    return _hash32(n, seed, tid, expert, device) >> 12


@functools.lru_cache(maxsize=None)
def _table_cpu(kind: str, bits: int) -> torch.Tensor:
    """Quantiles at cell midpoints (j + 1/2) / 2^bits, computed in fp64, stored fp32."""
    n = 1 << bits
    p = (torch.arange(n, dtype=torch.float64) + 0.5) / n
    if kind == "normal":
        q = torch.special.ndtri(p)
    elif kind == "gumbel":
        q = -torch.log(-torch.log(p))
    else:
        raise ValueError(kind)
    return q.to(torch.float32)


_TABLE_DEV: Dict = {}


def _table(kind: str, bits: int, device) -> torch.Tensor:
    device = torch.device(device)
    if device.type == "cpu":
        return _table_cpu(kind, bits)
    key = (kind, bits, str(device))
    if key not in _TABLE_DEV:
        _TABLE_DEV[key] = _table_cpu(kind, bits).to(device)
    return _TABLE_DEV[key]


def normal_tensor(shape, std: float, seed: int, tid: int, expert: int = 0,
                  device="cpu", dtype=torch.bfloat16, fine: bool = False) -> torch.Tensor:
    """Discretised N(0, std^2) tensor, bit-identical on every device."""
    n = math.prod(shape)
    if fine:
        u = _u20(n, seed, tid, expert, device)
        tab = _table("normal", 20, device)
    else:
        u = _u16(n, seed, tid, expert, device)
        tab = _table("normal", 16, device)
    v = tab[u]
    if std != 1.0:
        v = v * torch.tensor(std, dtype=torch.float32, device=v.device)
    return v.to(dtype).reshape(shape)


def gumbel_tensor(shape, seed: int, tid: int, device="cpu") -> torch.Tensor:
    n = math.prod(shape)
    u = _u20(n, seed, tid, 0, device)
    return _table("gumbel", 20, device)[u].reshape(shape)


def uniform_int_tensor(shape, high: int, seed: int, tid: int, device="cpu") -> torch.Tensor:
    """Integers uniform in [0, high) (exactly uniform when high divides 2^32)."""
    n = math.prod(shape)
    return (_hash32(n, seed, tid, 0, device) % high).to(torch.int32).reshape(shape)


# ---------------------------------------------------------------------------
# Workload configurations
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class MoEConfig:
    """One MoE layer's share on one GPU.

    T tokens of width H; E experts in the router, of which the local range
    [expert_begin, expert_begin + E_loc) is computed here; top-k routing;
    FFN width F; act is "swiglu" (three matrices per expert) or "gelu" (two).
    num_ranks > 1 tags every token with a source-rank label in [0, num_ranks)
    (rank 0 = this GPU).  tile_m is the row-tile the reorganised tensors are
    padded to.  tp > 1 makes this GPU one tensor-parallel rank (tp_rank) of
    the layer: it holds FFN columns [tp_rank * F / tp, (tp_rank + 1) * F / tp)
    of every local expert (F_loc of them) and its output is that slice's
    partial sum, which a reduce-scatter over the tp ranks would complete.
    """
    name: str
    T: int
    H: int
    F: int
    E: int
    k: int
    act: str
    logits: str            # "router" | "normal" | "zipf"
    tile_m: int
    expert_begin: int = 0
    E_loc: Optional[int] = None
    num_ranks: int = 1
    tp: int = 1
    tp_rank: int = 0
    zipf_s: float = 1.1
    w_std: float = 0.02
    seed: int = 0
    description: str = field(default="", compare=False)

    @property
    def n_local(self) -> int:
        return self.E if self.E_loc is None else self.E_loc

    @property
    def F_loc(self) -> int:
        """FFN columns per expert held here (F / tp)."""
        assert self.F % self.tp == 0 and 0 <= self.tp_rank < self.tp, (self.F, self.tp, self.tp_rank)
        return self.F // self.tp

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig(
        "tiny", T=256, H=512, F=1024, E=8, k=2, act="gelu", logits="router", tile_m=64,
        description="256 tokens, hidden 512, FFN 1024, 8 experts top-2, GELU; logits from a "
                    "random 512x8 router"),
    "mixtral": MoEConfig(
        "mixtral", T=4096, H=4096, F=14336, E=8, k=2, act="swiglu", logits="normal", tile_m=256,
        description="Mixtral-shaped layer: 4096 tokens, hidden 4096, FFN 14336, SwiGLU, "
                    "8 experts top-2"),
    "fine_grained": MoEConfig(
        "fine_grained", T=8192, H=2048, F=1408, E=64, k=6, act="swiglu", logits="zipf",
        tile_m=256,
        description="fine-grained MoE: 8192 tokens, hidden 2048, FFN 1408, SwiGLU, 64 experts "
                    "top-6, Zipf(1.1)-biased router"),
    "ep_share": MoEConfig(
        "ep_share", T=16384, H=4096, F=2048, E=64, k=8, act="swiglu", logits="normal",
        tile_m=256, expert_begin=0, E_loc=8, num_ranks=8,
        description="expert-parallel share: 16384 tokens with source ranks 0..7, experts 0..7 "
                    "of a 64-expert top-8 router, hidden 4096, FFN 2048, SwiGLU"),
    "tp2_share": MoEConfig(
        "tp2_share", T=16384, H=4096, F=2048, E=64, k=8, act="swiglu", logits="normal",
        tile_m=256, expert_begin=0, E_loc=8, num_ranks=8, tp=2,
        description="tensor-parallel rank 0 of 2 of the expert-parallel share: FFN columns "
                    "0..1023 of each local expert, partial output"),
    "tp4_share": MoEConfig(
        "tp4_share", T=16384, H=4096, F=2048, E=64, k=8, act="swiglu", logits="normal",
        tile_m=256, expert_begin=0, E_loc=8, num_ranks=8, tp=4,
        description="tensor-parallel rank 0 of 4 of the expert-parallel share: FFN columns "
                    "0..511 of each local expert, partial output"),
    "tp8_share": MoEConfig(
        "tp8_share", T=16384, H=4096, F=2048, E=64, k=8, act="swiglu", logits="normal",
        tile_m=256, expert_begin=0, E_loc=8, num_ranks=8, tp=8,
        description="tensor-parallel rank 0 of 8 of the expert-parallel share: FFN columns "
                    "0..255 of each local expert, partial output"),
    "decode": MoEConfig(
        "decode", T=64, H=7168, F=2048, E=256, k=8, act="swiglu", logits="normal", tile_m=16,
        description="decode-sized layer: 64 tokens, hidden 7168, FFN 2048, SwiGLU, "
                    "256 experts top-8"),
}


def make_logits(cfg: MoEConfig, device="cpu", x: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Router logits [T, E] fp32.

    "normal": N(0,1) drawn directly.  "zipf": ln p_e + Gumbel(0,1) noise with
    p_e proportional to (e+1)^-s, so that the first choice of every token is
    exactly Zipf(s)-distributed.  "router": a random H x E router applied to x
    on the host in fp64 and rounded once to fp32 (input synthesis only; the
    layer itself starts from the logits).
    """
    T, E = cfg.T, cfg.E
    if cfg.logits == "normal":
        return normal_tensor((T, E), 1.0, cfg.seed, TID_LOGITS, device=device,
                             dtype=torch.float32, fine=True)
    if cfg.logits == "zipf":
        e = torch.arange(E, dtype=torch.float64)
        w = (e + 1.0) ** (-cfg.zipf_s)
        logp = torch.log(w / w.sum()).to(torch.float32).to(device)
        g = gumbel_tensor((T, E), cfg.seed, TID_LOGITS, device=device)
        return g + logp[None, :]
    if cfg.logits == "router":
        if x is None:
            x = make_x(cfg, device="cpu")
        wr = normal_tensor((cfg.H, E), cfg.w_std, cfg.seed, TID_ROUTER,
                           dtype=torch.float32, fine=True)
        lg = (x.to("cpu", torch.float64) @ wr.to(torch.float64)).to(torch.float32)
        return lg.to(device)
    raise ValueError(cfg.logits)


def make_x(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    return normal_tensor((cfg.T, cfg.H), 1.0, cfg.seed, TID_X, device=device)


def make_src_rank(cfg: MoEConfig, device="cpu") -> Optional[torch.Tensor]:
    if cfg.num_ranks <= 1:
        return None
    return uniform_int_tensor((cfg.T,), cfg.num_ranks, cfg.seed, TID_RANK, device=device)


def expert_weights(cfg: MoEConfig, local_expert: int, device="cpu"):
    """(w0, w0_up, w1) of one local expert as bf16 tensors.

    w0 = W_gate^T or W1^T  [F_loc, H];  w0_up = W_up^T [F_loc, H] or None;
    w1 = W_down^T or W2^T  [H, F_loc].  The expert's global id keys the
    generator, so a local range sees the same weights as the full layer, and a
    tensor-parallel rank gets its column slice of the full expert's weights.
    """
    e = cfg.expert_begin + local_expert
    w0 = normal_tensor((cfg.F, cfg.H), cfg.w_std, cfg.seed, TID_W0, e, device)
    w0u = (normal_tensor((cfg.F, cfg.H), cfg.w_std, cfg.seed, TID_W0_UP, e, device)
           if cfg.act == "swiglu" else None)
    w1 = normal_tensor((cfg.H, cfg.F), cfg.w_std, cfg.seed, TID_W1, e, device)
    if cfg.tp > 1:
        c0, c1 = cfg.tp_rank * cfg.F_loc, (cfg.tp_rank + 1) * cfg.F_loc
        w0 = w0[c0:c1].contiguous()
        w0u = None if w0u is None else w0u[c0:c1].contiguous()
        w1 = w1[:, c0:c1].contiguous()
    return w0, w0u, w1


def make_weights(cfg: MoEConfig, device="cpu"):
    """Stacked per-expert weights (w0 [E_loc,F,H], w0_up [E_loc,F,H] | None, w1 [E_loc,H,F])."""
    El = cfg.n_local
    w0 = torch.empty((El, cfg.F_loc, cfg.H), dtype=torch.bfloat16, device=device)
    w0u = (torch.empty((El, cfg.F_loc, cfg.H), dtype=torch.bfloat16, device=device)
           if cfg.act == "swiglu" else None)
    w1 = torch.empty((El, cfg.H, cfg.F_loc), dtype=torch.bfloat16, device=device)
    for le in range(El):
        a, b, c = expert_weights(cfg, le, device)
        w0[le].copy_(a)
        if w0u is not None:
            w0u[le].copy_(b)
        w1[le].copy_(c)
    return w0, w0u, w1


def make_inputs(cfg: MoEConfig, device="cpu", weights: bool = True) -> dict:
    x = make_x(cfg, device)
    d = {
        "x": x,
        "logits": make_logits(cfg, device, x=x if cfg.logits == "router" else None),
        "src_rank": make_src_rank(cfg, device),
    }
    if weights:
        d["w0"], d["w0_up"], d["w1"] = make_weights(cfg, device)
    return d


def flops(cfg: MoEConfig, R: int) -> int:
    """Algorithmic FLOPs of the two grouped GEMMs for R routed (token, expert) rows."""
    n_mats = 3 if cfg.act == "swiglu" else 2
    return 2 * R * cfg.H * cfg.F_loc * n_mats
