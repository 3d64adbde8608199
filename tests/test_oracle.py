"""Pins of the CPU oracle against things other than itself (CPU only).

Each check rests on something the oracle does not compute: torch's own dtype
casts, exact rational arithmetic in scalar loops, subset enumeration, closed
forms, hand-worked fixtures under tests/golden/, and torch's SDPA for the
dense identity.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    if isinstance(x, str):
        return {"-0.0": -0.0, "ln3": math.log(3), "ln4": math.log(4), "ln2": math.log(2)}[x]
    return float(x)


# ---------------------------------------------------------------- formats

def test_e4m3fn_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3fn(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e4m3fn_known_points():
    assert O.e4m3fn_value(0x38) == 1.0
    assert O.e4m3fn_value(0x7E) == 448.0
    assert O.e4m3fn_value(0x01) == 2.0 ** -9
    assert O.e4m3fn_value(0xC0) == -2.0
    assert math.isnan(O.e4m3fn_value(0x7F))


def test_bf16_matches_torch_cast():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode_bf16(bits.numpy().view(np.uint16))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


# ---------------------------------------------------------------- indexer

def test_indexer_hand_golden():
    g = _load("indexer_hand.json")
    s = oracle.indexer_scores(np.array(g["q8"], np.uint8), g["q_scale"], np.array(g["w"]),
                              np.array(g["k8"], np.uint8), np.array(g["k_scale"]))
    assert s.tolist() == g["expected_scores"]
    for k, exp in g["expected_topk"].items():
        assert oracle.topk_indices(s, int(k)).tolist() == exp


def _finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c.astype(np.uint8)


def _exact_fp8(code):
    # independent decode through Fraction: mantissa/exponent fields of the byte
    sign = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 64)
    return sign * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


@pytest.mark.parametrize("seed", range(12))
def test_indexer_bruteforce_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    H_I, d_I, n = rng.integers(1, 6), rng.integers(1, 9), rng.integers(1, 13)
    q8 = _finite_codes(rng, (H_I, d_I))
    k8 = _finite_codes(rng, (n, d_I))
    w = rng.normal(size=H_I).astype(np.float32)
    qs = np.float32(rng.uniform(0.01, 3.0))
    ks = rng.uniform(0.01, 3.0, size=n).astype(np.float32)
    got = oracle.indexer_scores(q8, qs, w, k8, ks)
    for s in range(n):
        tot = Fraction(0)
        for j in range(H_I):
            dot = sum(_exact_fp8(int(q8[j, d])) * _exact_fp8(int(k8[s, d])) for d in range(d_I))
            if dot > 0:
                tot += Fraction(float(w[j])) * Fraction(float(qs)) * Fraction(float(ks[s])) * dot
        ref = float(tot)
        assert abs(got[s] - ref) <= 1e-12 * max(1.0, abs(ref)), (s, got[s], ref)


def test_indexer_integer_inputs_give_integer_scores():
    rng = np.random.default_rng(7)
    H_I, d_I, n = 4, 32, 50
    qi = rng.integers(-3, 4, size=(H_I, d_I))
    ki = rng.integers(-3, 4, size=(n, d_I))
    wi = rng.integers(-2, 3, size=H_I)
    to_codes = lambda a: torch.tensor(a, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.indexer_scores(to_codes(qi), None, wi.astype(np.float32), to_codes(ki), None)
    for s in range(n):
        ref = sum(int(wi[j]) * max(int(np.dot(qi[j], ki[s])), 0) for j in range(H_I))
        assert got[s] == ref


def test_indexer_per_token_scale_is_a_factor():
    # ReLU(c*x) = c*ReLU(x) for c > 0: scaling one key's scale scales only its score
    rng = np.random.default_rng(3)
    q8, k8 = _finite_codes(rng, (3, 5)), _finite_codes(rng, (6, 5))
    w = rng.normal(size=3)
    ks = np.ones(6)
    a = oracle.indexer_scores(q8, 1.0, w, k8, ks)
    ks2 = ks.copy()
    ks2[2] = 4.0
    b = oracle.indexer_scores(q8, 1.0, w, k8, ks2)
    assert b[2] == 4.0 * a[2]
    assert np.array_equal(np.delete(a, 2), np.delete(b, 2))


# ---------------------------------------------------------------- top-k

def test_topk_hand_golden_ties():
    g = _load("topk_ties.json")
    s = np.array([_num(x) for x in g["scores"]])
    assert np.signbit(s[3]) and not np.signbit(s[4])
    for k, exp in g["expected"].items():
        assert oracle.topk_indices(s, int(k)).tolist() == exp
        assert oracle.topk_indices(s.astype(np.float32), int(k)).tolist() == exp


def _rank_select(scores, k):
    n = len(scores)
    sel = []
    for s in range(n):
        better = sum(1 for t in range(n) if scores[t] > scores[s] or (scores[t] == scores[s] and t < s))
        if better < k:
            sel.append(s)
    return sel


@pytest.mark.parametrize("seed", range(20))
def test_topk_pairwise_rank_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 41))
    k = int(rng.integers(1, 45))
    scores = rng.integers(-4, 5, size=n).astype(np.float64) * (0.5 if seed % 2 else 1.0)
    if seed % 3 == 0:
        scores[rng.random(n) < 0.3] = -0.0
    got = oracle.topk_indices(scores, k)
    sel = _rank_select(scores.tolist(), k)
    assert got[: len(sel)].tolist() == sel
    assert (got[len(sel):] == -1).all()


@pytest.mark.parametrize("seed", range(10))
def test_topk_subset_enumeration(seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(1, 11))
    k = int(rng.integers(1, 5))
    scores = rng.integers(-2, 3, size=n).astype(np.float64)
    if k >= n:
        best = list(range(n))
    else:
        keyed = lambda sub: sorted((-scores[i], i) for i in sub)
        best = sorted(min(itertools.combinations(range(n), k), key=keyed))
    got = oracle.topk_indices(scores, k)
    assert got[: len(best)].tolist() == list(best)


@pytest.mark.parametrize("seed", range(8))
def test_topk_invariants(seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 5000))
    k = int(rng.choice([1, 7, 64, 2048]))
    scores = rng.normal(size=n).astype(np.float32)
    if seed % 2:
        scores = np.round(scores * 3).astype(np.float32)   # heavy ties
    idx = oracle.topk_indices(scores, k)
    m = min(k, n)
    sel = idx[:m]
    assert (idx[m:] == -1).all()
    assert (sel >= 0).all() and (sel < n).all()
    assert (np.diff(sel) > 0).all()                       # ascending, no duplicates
    mask = np.zeros(n, bool)
    mask[sel] = True
    if m < n:
        lo = scores[mask].min()
        hi = scores[~mask].max()
        assert lo >= hi
        if lo == hi:                                      # ties at the threshold: lower index wins
            tied_sel = np.nonzero(mask & (scores == lo))[0]
            tied_out = np.nonzero(~mask & (scores == lo))[0]
            assert tied_sel.max() < tied_out.min()


def test_topk_n_le_k_is_identity():
    for n in (1, 5, 64):
        idx = oracle.topk_indices(np.random.default_rng(n).normal(size=n), 64)
        assert idx[:n].tolist() == list(range(n)) and (idx[n:] == -1).all()


# ---------------------------------------------------------------- attention

def test_attention_hand_golden():
    g = _load("attention_hand.json")
    q = np.array(g["q"])
    K = np.array([[_num(x) for x in r] for r in g["K"]])
    V = np.array(g["V"])
    out, lse = oracle.sparse_attention(q, K, V, g["scale"])
    assert np.allclose(out, np.array(g["expected_out"]), rtol=0, atol=1e-14)
    assert np.allclose(lse, [_num(x) for x in g["expected_lse"]], rtol=0, atol=1e-14)


def test_attention_bruteforce_loops():
    rng = np.random.default_rng(5)
    H, m, D, Dv = 3, 7, 5, 4
    q, K, V = rng.normal(size=(H, D)), rng.normal(size=(m, D)), rng.normal(size=(m, Dv))
    out, lse = oracle.sparse_attention(q, K, V, 0.7)
    for h in range(H):
        logits = [0.7 * sum(q[h, d] * K[i, d] for d in range(D)) for i in range(m)]
        den = sum(math.exp(x) for x in logits)
        assert abs(lse[h] - math.log(den)) < 1e-12
        for d in range(Dv):
            ref = sum(math.exp(logits[i]) * V[i, d] for i in range(m)) / den
            assert abs(out[h, d] - ref) < 1e-12


def test_attention_closed_forms():
    rng = np.random.default_rng(6)
    q = rng.normal(size=(4, 6))
    K = rng.normal(size=(9, 6))
    V = rng.normal(size=(9, 5))
    out, _ = oracle.sparse_attention(q, K[:1], V[:1], 0.3)          # one row: out = V[0]
    assert np.array_equal(out, np.repeat(V[:1], 4, axis=0))
    out, lse = oracle.sparse_attention(np.zeros_like(q), K, V, 0.3)  # q = 0: mean of V
    assert np.allclose(out, V.mean(axis=0)[None].repeat(4, 0), atol=1e-14)
    assert np.allclose(lse, math.log(9), atol=1e-14)
    Keq = np.repeat(K[:1], 9, axis=0)                                 # equal keys: mean of V
    out, _ = oracle.sparse_attention(q, Keq, V, 0.3)
    assert np.allclose(out, V.mean(axis=0)[None].repeat(4, 0), atol=1e-14)
    u = rng.normal(size=6)
    u = u - (q @ u)[:, None].mean() * 0                               # shift all keys by one vector
    out1, lse1 = oracle.sparse_attention(q, K, V, 0.3)
    out2, lse2 = oracle.sparse_attention(q, K + u[None], V, 0.3)
    assert np.allclose(out1, out2, atol=1e-12)
    assert np.allclose(lse2 - lse1, 0.3 * (q @ u), atol=1e-12)
    perm = rng.permutation(9)                                         # order of the subset is irrelevant
    out3, lse3 = oracle.sparse_attention(q, K[perm], V[perm], 0.3)
    assert np.allclose(out1, out3, atol=1e-13) and np.allclose(lse1, lse3, atol=1e-13)


def test_dense_causal_matches_torch_sdpa():
    rng = np.random.default_rng(8)
    L, H, D, Dv = 11, 3, 8, 6
    q, K, V = rng.normal(size=(L, H, D)), rng.normal(size=(L, D)), rng.normal(size=(L, Dv))
    mine = oracle.dense_causal_attention(q, K, V, 0.4)
    tq = torch.tensor(q).permute(1, 0, 2)                 # [H, L, D]
    tk = torch.tensor(K)[None].expand(H, L, D)
    tv = torch.tensor(V)[None].expand(H, L, Dv)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.4)
    assert np.allclose(mine, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def _int_codes(a):
    return torch.tensor(a, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_sparse_equals_dense_when_k_covers_context():
    # with k >= L every row selects all of its causal prefix, so the whole path
    # must reduce to dense causal attention
    rng = np.random.default_rng(9)
    L, H_I, d_I, H, D, Dv = 23, 2, 4, 3, 8, 8
    a = dict(q8=_int_codes(rng.integers(-3, 4, size=(L, H_I, d_I))), q_scale=None,
             w=rng.integers(-2, 3, size=(L, H_I)).astype(np.float32),
             k8=_int_codes(rng.integers(-3, 4, size=(1, L, d_I))), k_scale=None,
             q_f=rng.normal(size=(L, H, D)), kv_f=rng.normal(size=(1, L, D)),
             v_f=rng.normal(size=(1, L, Dv)), seq_lens=[L], q_start=[0, L],
             k=32, scale=0.35, D_v=Dv)
    res = oracle.run_rows(a, range(L))
    dense = oracle.dense_causal_attention(a["q_f"], a["kv_f"][0], a["v_f"][0], 0.35)
    for t in range(L):
        assert res["idx"][t][: t + 1].tolist() == list(range(t + 1))
        assert np.allclose(res["out"][t], dense[t], atol=1e-12)


def test_shared_latent_value_is_prefix_of_row():
    # without a separate V cache, V is the first D_v dims of each latent row
    rng = np.random.default_rng(10)
    L, D, Dv = 9, 6, 4
    bits = lambda x: torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kvf = rng.normal(size=(1, L, D))
    a = dict(q8=_int_codes(np.ones((L, 1, 2))), q_scale=None, w=np.ones((L, 1), np.float32),
             k8=_int_codes(np.ones((1, L, 2))), k_scale=None,
             q=bits(rng.normal(size=(L, 2, D))), kv=bits(kvf), v=None,
             seq_lens=[L], q_start=[0, L], k=16, scale=0.5, D_v=Dv)
    res = oracle.run_rows(a, [L - 1])
    Kd = oracle.decode_bf16(a["kv"][0])
    ref, _ = oracle.sparse_attention(oracle.decode_bf16(a["q"][L - 1]), Kd, Kd[:, :Dv], 0.5)
    assert np.array_equal(res["out"][0], ref)


# ---------------------------------------------------------------- geometry / paging

def test_paged_rows_equal_contiguous_rows():
    rng = np.random.default_rng(11)
    lens, bs, d = [70, 5, 129], 16, 3
    cont = rng.normal(size=(3, 130, d))
    nblk = [(L + bs - 1) // bs for L in lens]
    perm = rng.permutation(sum(nblk))
    pool = np.zeros((sum(nblk), bs, d))
    table = np.full((3, max(nblk)), -1)
    off = 0
    for b, L in enumerate(lens):
        for i in range(nblk[b]):
            table[b, i] = perm[off + i]
            for sl in range(bs):
                if i * bs + sl < L:
                    pool[perm[off + i], sl] = cont[b, i * bs + sl]
        off += nblk[b]
    for b, L in enumerate(lens):
        assert np.array_equal(oracle.token_rows(pool, b, L, table, bs), cont[b, :L])


def test_row_geometry():
    assert oracle.row_geometry([5, 9], None, 2) == [(0, 4), (1, 8)]
    assert oracle.row_geometry([3], [0, 3], 3) == [(0, 0), (0, 1), (0, 2)]
    # a chunk of 2 query rows at the end of a 6-token cache
    assert oracle.row_geometry([6], [0, 2], 2) == [(0, 4), (0, 5)]


def test_abs_terms_are_scores_with_absolute_weights():
    # the absolute-term sum (the tolerance scale of a score) is the score the
    # same row would get with every head weight replaced by its magnitude
    rng = np.random.default_rng(12)
    H_I, d_I, n = 5, 16, 40
    q8 = _finite_codes(rng, (H_I, d_I))
    k8 = _finite_codes(rng, (n, d_I))
    w = rng.normal(size=H_I).astype(np.float32)
    ks = rng.uniform(0.1, 2.0, size=n).astype(np.float32)
    sc, ab = oracle.indexer_scores(q8, 0.7, w, k8, ks, with_abs=True)
    assert np.array_equal(sc, oracle.indexer_scores(q8, 0.7, w, k8, ks))
    assert np.allclose(ab, oracle.indexer_scores(q8, 0.7, np.abs(w), k8, ks), rtol=1e-15, atol=0)
    assert (ab >= np.abs(sc) - 1e-12 * ab).all()
