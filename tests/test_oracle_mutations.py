"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutant below is a copy of one oracle function with a single bug; the
pins of test_oracle.py must fail on it.  This shows the pins are sharp enough
to notice a dropped term, a wrong sign or tie-break, or a swapped operand.
"""
import numpy as np
import pytest

import oracle
from oracle import dsa_oracle as O
import tests.test_oracle as P


# the real functions, for mutants that wrap them
_REAL_INDEXER = O.indexer_scores
_REAL_ATTENTION = O.sparse_attention
_REAL_GEOMETRY = O.row_geometry


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _no_relu(q8, q_scale, w, k8, k_scale):
    q, k = O.decode_e4m3fn(q8), O.decode_e4m3fn(k8)
    qs = 1.0 if q_scale is None else float(q_scale)
    ks = np.ones(k.shape[0]) if k_scale is None else np.asarray(k_scale, dtype=np.float64)
    return ((np.asarray(w) * qs) @ (q @ k.T)) * ks


def _no_kscale(q8, q_scale, w, k8, k_scale):
    return _REAL_INDEXER(q8, q_scale, w, k8, None)


def _abs_instead_of_relu(q8, q_scale, w, k8, k_scale):
    q, k = O.decode_e4m3fn(q8), O.decode_e4m3fn(k8)
    qs = 1.0 if q_scale is None else float(q_scale)
    ks = np.ones(k.shape[0]) if k_scale is None else np.asarray(k_scale, dtype=np.float64)
    return ((np.asarray(w) * qs) @ np.abs(q @ k.T)) * ks


def _tie_index_desc(scores, k):
    scores = np.asarray(scores)
    n = scores.shape[0]
    out = np.full(k, -1, dtype=np.int32)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    order = np.lexsort((-np.arange(n), -scores.astype(np.float64)))
    out[:] = np.sort(order[:k])
    return out


def _unsorted_output(scores, k):
    scores = np.asarray(scores)
    n = scores.shape[0]
    out = np.full(k, -1, dtype=np.int32)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    out[:] = np.lexsort((np.arange(n), -scores.astype(np.float64)))[:k]
    return out


def _signed_zero_ordered(scores, k):
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    out = np.full(k, -1, dtype=np.int32)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    key = -scores + np.where(np.signbit(scores) & (scores == 0), 1e-300, 0.0)
    out[:] = np.sort(np.lexsort((np.arange(n), key))[:k])
    return out


def _value_is_key(q, K, V, scale):
    return _REAL_ATTENTION(q, K, K[:, : V.shape[1]], scale)


def _lse_without_max(q, K, V, scale):
    x = scale * (q @ K.T)
    mx = x.max(axis=1, keepdims=True)
    p = np.exp(x - mx)
    den = p.sum(axis=1, keepdims=True)
    return (p @ V) / den, np.log(den[:, 0])


def _transposed_scores(q, K, V, scale):
    x = scale * (q @ K.T)
    x = x[:, ::-1]                           # logits paired with the wrong rows
    mx = x.max(axis=1, keepdims=True)
    p = np.exp(x - mx)
    den = p.sum(axis=1, keepdims=True)
    return (p @ V) / den, mx[:, 0] + np.log(den[:, 0])


def _exclusive_causality(seq_lens, q_start, num_rows):
    return [(b, max(p - 1, 0)) for b, p in _REAL_GEOMETRY(seq_lens, q_start, num_rows)]



PIN_RUNS = {
    "indexer": [P.test_indexer_hand_golden,
                lambda: [P.test_indexer_bruteforce_exact_rationals(s) for s in range(12)],
                P.test_indexer_integer_inputs_give_integer_scores],
    "topk": [P.test_topk_hand_golden_ties,
             lambda: [P.test_topk_pairwise_rank_bruteforce(s) for s in range(20)],
             lambda: [P.test_topk_invariants(s) for s in range(8)]],
    "attention": [P.test_attention_hand_golden, P.test_attention_bruteforce_loops,
                  P.test_attention_closed_forms, P.test_sparse_equals_dense_when_k_covers_context],
    "geometry": [P.test_sparse_equals_dense_when_k_covers_context, P.test_row_geometry],
}

MUTANTS = [
    ("indexer_scores", _no_relu, "indexer"),
    ("indexer_scores", _no_kscale, "indexer"),
    ("indexer_scores", _abs_instead_of_relu, "indexer"),
    ("topk_indices", _tie_index_desc, "topk"),
    ("topk_indices", _unsorted_output, "topk"),
    ("topk_indices", _signed_zero_ordered, "topk"),
    ("sparse_attention", _value_is_key, "attention"),
    ("sparse_attention", _lse_without_max, "attention"),
    ("sparse_attention", _transposed_scores, "attention"),
    ("row_geometry", _exclusive_causality, "geometry"),
]


@pytest.mark.parametrize("fn_name,mutant,group", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, fn_name, mutant, group):
    _patch(monkeypatch, fn_name, mutant)
    caught = 0
    for pin in PIN_RUNS[group]:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"no pin noticed the planted mistake {mutant.__name__}"
