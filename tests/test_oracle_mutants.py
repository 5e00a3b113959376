"""The oracle's pins have teeth: plant plausible mistakes in a copy of the oracle.

Each mutant is the oracle's source with one edit, loaded as a separate module
(the real oracle is untouched).  At least one of the listed pins must fail on
it.  All of this runs on the CPU.
"""
import inspect
import types

import pytest

import test_oracle_pins as P
from oracle import moe_oracle

SRC = inspect.getsource(moe_oracle)

# (name, original text, planted mistake, pins that must catch it)
MUTANTS = [
    ("silu sign", "z / (1.0 + np.exp(-z))", "z / (1.0 + np.exp(z))",
     [("test_single_expert_top1_is_dense_ffn", {"act": "swiglu"})]),
    ("gelu tanh approximation", "0.5 * h * (1.0 + _erf(h / math.sqrt(2.0)))",
     "0.5 * h * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (h + 0.044715 * h ** 3)))",
     [("test_single_expert_top1_is_dense_ffn", {"act": "gelu"})]),
    ("gate and up swapped", "return silu(g) * u", "return silu(u) * g",
     [("test_single_expert_top1_is_dense_ffn", {"act": "swiglu"})]),
    ("tie-break to higher id", "key=lambda e: (-row[e], e)", "key=lambda e: (-row[e], -e)",
     [("test_topk1_is_argmax_with_ties", {}), ("test_topk_matches_bruteforce", {"E": 5})]),
    ("gate not renormalised", "denom = math.fsum(z)", "denom = math.fsum(math.exp(v - top) for v in row)",
     [("test_gate_weights_sum_to_one_and_ratios", {})]),
    ("layer drops the gate weight", "w0, w0u, w1 = get(le)\n            out[i] += float(w[t, j]) * expert_ffn",
     "w0, w0u, w1 = get(le)\n            out[i] += expert_ffn",
     [("test_layer_matches_dense_mixture", {"act": "swiglu", "renorm": True, "E": 4, "k": 2})]),
    ("expert-major layer drops the gate weight",
     "for i, t, j in users[le]:\n            out[i] += float(w[t, j]) * expert_ffn",
     "for i, t, j in users[le]:\n            out[i] += expert_ffn",
     [("test_expert_major_layer_matches_dense_mixture", {"act": "gelu"})]),
    ("expert-major layer ignores expert_begin", "le = int(idx[t, j]) - expert_begin\n            if 0 <= le < E_loc:\n                users",
     "le = int(idx[t, j])\n            if 0 <= le < E_loc:\n                users",
     [("test_expert_major_layer_matches_dense_mixture", {"act": "swiglu"})]),
    ("combine drops the gate weight", "out[t] += float(topk_w[t, j]) * np.asarray", "out[t] += np.asarray",
     [("test_combine_and_permute_reassemble_the_layer", {})]),
    ("transposed layer-1 weight", "return np.asarray(w1, dtype=np.float64) @ a",
     "return np.asarray(w1, dtype=np.float64).T[:len(x_row)] @ a[:len(x_row)]",
     [("test_single_expert_top1_is_dense_ffn", {"act": "gelu"})]),
    ("sort ignores source rank", "pairs.append((le, int(ranks[t]), t, j))", "pairs.append((le, 0, t, j))",
     [("test_permute_hand_example", {})]),
    ("padding rounds up one tile too many", "-(-counts[le] // tile_m) * tile_m",
     "(counts[le] // tile_m + 1) * tile_m",
     [("test_permute_exact_tile_multiple_has_no_padding", {})]),
    ("tile priority from the first row", "last = offsets[le] + min(counts[le], (m + 1) * tile_m) - 1",
     "last = offsets[le] + m * tile_m",
     [("test_permute_invariants", {"T": 500, "k": 8, "E": 64, "e0": 8, "El": 8, "R": 8, "tm": 64})]),
    ("local range ignores expert_begin", "le = int(idx[t, j]) - expert_begin\n            if not 0",
     "le = int(idx[t, j])\n            if not 0",
     [("test_rank_partition_invariance", {})]),
]


def _mutant_module(old, new):
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, old, new, pins):
    monkeypatch.setattr(P, "O", _mutant_module(old, new))
    caught = False
    for fn, kw in pins:
        try:
            getattr(P, fn)(**kw)
        except Exception:
            caught = True
    assert caught, f"planted mistake '{name}' passed every listed pin"


def test_unmutated_oracle_passes_the_same_pins():
    for _, _, _, pins in MUTANTS:
        for fn, kw in pins:
            getattr(P, fn)(**kw)
