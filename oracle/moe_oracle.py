"""CPU oracle for one GPU's share of a Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and
this module imports nothing from the product path.

It is a plain, slow, obviously-correct restatement of what the layer computes,
in float64, one token at a time:

  * routing -- "Comet: Fine-grained Computation-communication Overlapping for
    Mixture-of-Experts" (paperlayer.ai summary), section 2.1 "MoE Structure":
    each token activates only its top-k experts chosen by the router;
  * expert FFN -- same section: each selected expert applies its
    feed-forward network to the token;
  * combine -- same section: expert outputs are gathered back and reduced
    over the token's top-k choices;
  * reorganisation -- section 3.1.2 ("How to reschedule the decomposed shared
    tensor?"): the shared tensor is regrouped into GEMM-tile-aligned
    sub-tensors, tokens are sorted by source rank, and tiles holding local
    tokens are prioritised; section 2.2.1: data reorganisation exposes only
    the data each tile needs.

Readings of what the pages leave open (all listed with reasons in the design
notes):
  R1 gate: softmax over the k selected logits (full softmax renormalised over
     the top-k); renormalize=False gives the full softmax at the selected
     experts.
  R3 top-k order: logits descending, equal logits -> lower expert id first;
     slot j follows that order.
  R5 dropless: every (token, local expert) pair is computed.
  R6 FFN: no biases; GELU is the exact erf form; SwiGLU is
     silu(x.Wg) * (x.Wu) then . Wd, with silu(z) = z / (1 + e^-z).
  R10 expert-parallel share: only pairs whose expert lies in the local range
     [expert_begin, expert_begin + E_loc) contribute; tokens with no local
     pair give a zero row.
  R11 permutation key: (local expert, source rank, token); each expert's rows
     are padded up to a multiple of tile_m.
  R12 tile priority: the source rank of the tile's last real row (the
     largest rank in the tile); tiles ordered by (priority, expert, m-tile).

Weight storage is output-major: w0 / w0_up are [F, H] (x . W_gate ==
w0 @ x) and w1 is [H, F] (a . W_down == w1 @ a).

Every function here is pinned by tests against brute force, closed forms,
library routines and invariants (tests/test_oracle_pins.py).
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf


# ---------------------------------------------------------------------------
# Routing (section 2.1; readings R1, R3)
# ---------------------------------------------------------------------------

def route_topk(logits: np.ndarray, k: int, renormalize: bool = True):
    """Top-k expert ids and gate weights for every token.

    Returns (idx int32 [T, k], w float64 [T, k]).  idx[t] lists the k largest
    logits of token t in descending order, equal logits taken lower id first.
    With renormalize the weights are softmax over the k selected logits, so
    each row sums to 1; without it they are the full softmax over all E
    experts evaluated at the selected ones.
    """
    logits = np.asarray(logits)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        row = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))
        sel = order[:k]
        top = row[sel[0]]
        z = [math.exp(row[e] - top) for e in sel]
        if renormalize:
            denom = math.fsum(z)
        else:
            denom = math.fsum(math.exp(v - top) for v in row)
        for j, e in enumerate(sel):
            idx[t, j] = e
            w[t, j] = z[j] / denom
    return idx, w


# ---------------------------------------------------------------------------
# Reorganisation into expert-contiguous, tile-aligned sub-tensors
# (section 3.1.2, section 2.2.1; readings R10, R11, R12)
# ---------------------------------------------------------------------------

def permute(topk_idx: np.ndarray, src_rank: Optional[np.ndarray], expert_begin: int,
            E_loc: int, tile_m: int) -> dict:
    """Expert-contiguous, source-rank-ordered, tile-padded row order.

    Pairs (t, j) whose expert e = topk_idx[t, j] is local are sorted by
    (e - expert_begin, src_rank[t], t).  Returns:
      counts   [E_loc]     real rows per local expert
      offsets  [E_loc+1]   padded start row of each expert (multiples of tile_m)
      row_src  [offsets[-1]]  t*k + j for a real row, -1 for a padding row
      row_rank [offsets[-1]]  source rank of each real row, -1 on padding
      inv_perm [T, k]      row of pair (t, j), -1 if its expert is not local
      tiles    list of (local_expert, row_begin), in schedule order
      tile_prio list of the tiles' priorities (same order)
    """
    topk_idx = np.asarray(topk_idx)
    T, k = topk_idx.shape
    ranks = np.zeros(T, dtype=np.int64) if src_rank is None else np.asarray(src_rank)
    pairs = []
    for t in range(T):
        for j in range(k):
            le = int(topk_idx[t, j]) - expert_begin
            if 0 <= le < E_loc:
                pairs.append((le, int(ranks[t]), t, j))
    pairs.sort()

    counts = [0] * E_loc
    for le, _, _, _ in pairs:
        counts[le] += 1
    offsets = [0]
    for le in range(E_loc):
        offsets.append(offsets[-1] + -(-counts[le] // tile_m) * tile_m)

    total = offsets[-1]
    row_src = np.full(total, -1, dtype=np.int64)
    row_rank = np.full(total, -1, dtype=np.int64)
    inv_perm = np.full((T, k), -1, dtype=np.int64)
    fill = [0] * E_loc
    for le, r, t, j in pairs:
        p = offsets[le] + fill[le]
        fill[le] += 1
        row_src[p] = t * k + j
        row_rank[p] = r
        inv_perm[t, j] = p

    keyed = []
    for le in range(E_loc):
        for m in range(-(-counts[le] // tile_m)):
            begin = offsets[le] + m * tile_m
            last = offsets[le] + min(counts[le], (m + 1) * tile_m) - 1
            keyed.append((int(row_rank[last]), le, m, begin))
    keyed.sort()
    return {
        "counts": np.array(counts, dtype=np.int64),
        "offsets": np.array(offsets, dtype=np.int64),
        "row_src": row_src,
        "row_rank": row_rank,
        "inv_perm": inv_perm,
        "tiles": [(le, begin) for (_, le, _, begin) in keyed],
        "tile_prio": [p for (p, _, _, _) in keyed],
    }


def gather_rows(x: np.ndarray, row_src: np.ndarray, k: int) -> np.ndarray:
    """Reorganised activations: row p holds x[row_src[p] // k]; padding rows are NaN."""
    out = np.full((len(row_src), x.shape[1]), np.nan)
    for p, s in enumerate(row_src):
        if s >= 0:
            out[p] = x[s // k]
    return out


# ---------------------------------------------------------------------------
# Expert feed-forward network (section 2.1; reading R6)
# ---------------------------------------------------------------------------

def silu(z):
    return z / (1.0 + np.exp(-z))


def gelu(h):
    return 0.5 * h * (1.0 + _erf(h / math.sqrt(2.0)))


def activation(act: str, g: np.ndarray, u: Optional[np.ndarray]) -> np.ndarray:
    """The FFN's nonlinearity applied to the layer-0 outputs of one row."""
    if act == "swiglu":
        return silu(g) * u
    if act == "gelu":
        return gelu(g)
    raise ValueError(act)


def expert_ffn(x_row: np.ndarray, w0: np.ndarray, w0_up: Optional[np.ndarray],
               w1: np.ndarray, act: str) -> np.ndarray:
    """One expert applied to one token row: layer0, activation, layer1."""
    x_row = np.asarray(x_row, dtype=np.float64)
    g = np.asarray(w0, dtype=np.float64) @ x_row
    u = None if w0_up is None else np.asarray(w0_up, dtype=np.float64) @ x_row
    a = activation(act, g, u)
    return np.asarray(w1, dtype=np.float64) @ a


# ---------------------------------------------------------------------------
# Combine (section 2.1, gather + top-k reduce; reading R10)
# ---------------------------------------------------------------------------

def combine(y_rows: np.ndarray, inv_perm: np.ndarray, topk_w: np.ndarray) -> np.ndarray:
    """out[t] = sum over slots j (in order) with inv_perm[t, j] >= 0 of w[t, j] * y_rows[inv_perm[t, j]]."""
    T, k = inv_perm.shape
    out = np.zeros((T, y_rows.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            p = int(inv_perm[t, j])
            if p >= 0:
                out[t] += float(topk_w[t, j]) * np.asarray(y_rows[p], dtype=np.float64)
    return out


# ---------------------------------------------------------------------------
# The whole layer, token by token
# ---------------------------------------------------------------------------

ExpertWeights = Callable[[int], tuple]


def moe_layer(x: np.ndarray, logits: np.ndarray, k: int, weights, act: str,
              expert_begin: int = 0, E_loc: Optional[int] = None,
              renormalize: bool = True, tokens: Optional[Sequence[int]] = None,
              route=None) -> np.ndarray:
    """Route every token, run each selected local expert on it, sum the weighted outputs.

    weights(le) (or weights[le]) returns (w0, w0_up, w1) of local expert le.
    tokens restricts the output to those token rows (routing is per token, so
    a subset gives exactly those rows of the full result).  route may pass a
    precomputed (idx, w) from route_topk.
    """
    x = np.asarray(x)
    T, E = np.asarray(logits).shape
    if E_loc is None:
        E_loc = E
    idx, w = route if route is not None else route_topk(logits, k, renormalize)
    get = weights if callable(weights) else weights.__getitem__
    tokens = range(T) if tokens is None else tokens
    out = np.zeros((len(tokens), x.shape[1]), dtype=np.float64)
    for i, t in enumerate(tokens):
        for j in range(k):
            le = int(idx[t, j]) - expert_begin
            if not 0 <= le < E_loc:
                continue
            w0, w0u, w1 = get(le)
            out[i] += float(w[t, j]) * expert_ffn(x[t], w0, w0u, w1, act)
    return out


def moe_layer_expert_major(x: np.ndarray, k: int, weights, act: str, route,
                           tokens: Sequence[int], expert_begin: int = 0,
                           E_loc: Optional[int] = None) -> np.ndarray:
    """The same sum as moe_layer, visiting experts in the outer loop.

    For large layers only a few token rows are checked, and each local
    expert's weights are fetched once (weights(le) is called at most once per
    expert, and only for experts some listed token selected).  route is the
    (idx, w) pair of route_topk.  Row i of the result is token tokens[i].
    """
    x = np.asarray(x)
    idx, w = route
    T, _ = idx.shape
    if E_loc is None:
        E_loc = int(idx.max()) + 1 - expert_begin
    get = weights if callable(weights) else weights.__getitem__
    users = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            le = int(idx[t, j]) - expert_begin
            if 0 <= le < E_loc:
                users.setdefault(le, []).append((i, t, j))
    out = np.zeros((len(tokens), x.shape[1]), dtype=np.float64)
    for le in sorted(users):
        w0, w0u, w1 = get(le)
        for i, t, j in users[le]:
            out[i] += float(w[t, j]) * expert_ffn(x[t], w0, w0u, w1, act)
    return out
