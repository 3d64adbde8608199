"""GPU parity of the streaming prefill selection (dsa_prefill_streaming).

The streaming path never stores the score matrix: a per-row threshold from the
scores of every 32nd token filters what leaves the indexer, and the exact
top-k is selected among the survivors (rows left with too few or too many
survivors are recomputed).  Its scores are the indexer's own, so its
selection, and the attention over it, must equal dsa_prefill's bit for bit;
on top of that it is checked against the oracle on sampled rows.  Crafted
inputs force every branch: rows that keep every token (n <= capacity), rows
thresholded on the sample, rows with fewer survivors than k, rows with more
survivors than the capacity, and rows whose scores all tie.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_long_06_amd as dsa
from tests.gpu_helpers import (DEV, announce, arrays_of, check_attention, check_rows, check_topk_swaps,
                               oracle_rows, to_np)

pytestmark = pytest.mark.gpu

STRIDE = 32                                   # sampled tokens: every 32nd


def _rank(k):
    return max((k + 15) // 16, 64)


def _cap(k):
    return 56 * _rank(k)


def _both(inp):
    wl = inp.wl
    batch = dsa.Batch.from_inputs(inp)
    idx_p = torch.empty((inp.num_rows, wl.k), dtype=torch.int32, device=DEV)
    idx_s = torch.empty_like(idx_p)
    out_p, lse_p, _ = dsa.prefill(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q, inp.kv,
                                  inp.v, wl.scale, idx_out=idx_p, D_v=wl.D_v)
    out_s, lse_s, _ = dsa.prefill_streaming(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q,
                                            inp.kv, inp.v, wl.scale, idx_out=idx_s, D_v=wl.D_v)
    torch.cuda.synchronize()
    return (idx_p, out_p, lse_p), (idx_s, out_s, lse_s)


def _assert_same(p, s, what):
    idx_p, out_p, lse_p = p
    idx_s, out_s, lse_s = s
    bad = (idx_p != idx_s).any(dim=1).nonzero().flatten().tolist()
    assert not bad, f"{what}: rows {bad[:8]} select differently ({len(bad)} rows)"
    assert torch.equal(out_p.view(torch.int16), out_s.view(torch.int16)), f"{what}: attention output differs"
    assert torch.equal(lse_p, lse_s), f"{what}: lse differs"


def _oracle_check(inp, idx, out, lse, rows, exact):
    a = arrays_of(inp)
    ref = oracle_rows(a, rows, need=("scores", "idx", "out"))
    if exact:
        for i, r in enumerate(rows):
            assert np.array_equal(idx[r], ref["idx"][i]), f"row {r}: selection not exact"
    check_rows(a, rows, idx[rows], out[rows], lse[rows], ref, inp.wl.k, inp.wl.name,
               min_same=1.0 if exact else 0.9)
    return ref


CASES = [
    # every row keeps every token (n <= capacity 7168)
    W.SMALL_PREFILL,
    # rows past the capacity take the sampled threshold; ragged last row tile and key chunk
    W.PREFILL_32K.replace(name="prefill_L12003", seq_len=12003, seed=31, sample_rows=0),
    # k = 512 (rank 64, capacity 3584), 8 indexer heads
    W.PREFILL_32K.replace(name="prefill_L6000_k512_hi8", seq_len=6000, k=512, H_I=8, seed=32, sample_rows=0),
    # two sequences behind a 64-token page table (sampled keys gathered through it)
    W.PREFILL_32K.replace(name="prefill_b2_L9000_paged64", seqs=2, seq_len=9000, paged=True, block_size=64,
                          seed=33, sample_rows=0),
    # integer indexer: many exactly tied scores, selection bit-exact against the oracle
    W.PREFILL_32K.replace(name="prefill_L9000_int", seq_len=9000, seed=34, sample_rows=0, integer_indexer=True),
    # the other head-tile counts of the filtered kernel: 16 heads with k = 64 (rank 64, capacity 3584), 48 heads
    # with k = 1024 (rank 64, capacity 3584)
    W.PREFILL_32K.replace(name="prefill_L5000_k64_hi16", seq_len=5000, k=64, H_I=16, seed=37, sample_rows=0),
    W.PREFILL_32K.replace(name="prefill_L7000_k1024_hi48", seq_len=7000, k=1024, H_I=48, seed=38, sample_rows=0),
    # k = 1 on integer scores: one winner per row among many exact ties (rank 64, capacity 3584)
    W.PREFILL_32K.replace(name="prefill_L5000_int_k1", seq_len=5000, k=1, seed=43, sample_rows=0,
                          integer_indexer=True),
    # 32 indexer heads (the remaining head-tile count) behind 16-token pages (smaller than a 64-key slot)
    W.PREFILL_32K.replace(name="prefill_L8500_hi32_paged16", seq_len=8500, H_I=32, paged=True, block_size=16,
                          seed=42, sample_rows=0),
]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_streaming_equals_prefill_and_oracle(wl):
    announce("streaming prefill", wl.name)
    inp = W.generate(wl, DEV)
    p, s = _both(inp)
    _assert_same(p, s, wl.name)
    idx, out, lse = (to_np(x) for x in s)
    n_rows = inp.num_rows
    cap = _cap(wl.k)
    always = [0, wl.k - 1, wl.k, min(cap, n_rows - 1), min(cap + 1, n_rows - 1), n_rows - 1]
    rows = W.sample_rows(wl, n_rows, 24, always=tuple(r for r in always if r < n_rows))
    _oracle_check(inp, idx, out, lse, rows, exact=wl.integer_indexer)


FP8_CASES = [CASES[1], CASES[4], CASES[6], CASES[8]]


@pytest.mark.parametrize("wl", FP8_CASES, ids=[w.name for w in FP8_CASES])
def test_fp8_filter_equals_exact_filter(wl):
    """With dsa_set_indexer_fp8(1) the filtered pass keeps every pair whose
    FP8 matrix-core estimate plus its error bound reaches the threshold, and
    only the pairs whose bounds straddle the row's k-th score are scored
    exactly afterwards (the 16x16x32 kernels' arithmetic).  The selection, and
    the attention over it, must equal the stored-score path's bit for bit, and
    the oracle's."""
    announce("fp8 filter vs stored scores", wl.name)
    inp = W.generate(wl, DEV)
    try:
        dsa.set_indexer_fp8(True)
        p, s = _both(inp)
    finally:
        dsa.set_indexer_fp8(False)
    _assert_same(p, s, wl.name + " fp8")
    idx, out, lse = (to_np(x) for x in s)
    rows = W.sample_rows(wl, inp.num_rows, 12, always=(0, wl.k, inp.num_rows - 1))
    _oracle_check(inp, idx, out, lse, rows, exact=wl.integer_indexer)


def _near_tie_inputs(wl, nclust, seed):
    """Seeded inputs whose index keys hold a cluster of ``nclust`` near-copies
    of one key (two dims moved by one e4m3fn code step each, never onto the
    NaN code) with a key scale four times the largest, so that many rows'
    sampled thresholds and k-th scores fall inside a dense run of scores that
    differ by less than the FP8 filter's error margin."""
    inp = W.generate(wl, "cpu")
    g = np.random.default_rng(seed)
    L = inp.seq_lens_host[0]
    k8 = inp.k8.numpy().copy()
    ks = inp.k_scale.numpy().copy()
    base = k8[0, int(g.integers(0, L))].copy()
    toks = g.choice(L, size=nclust, replace=False)
    for s in toks:
        c = base.copy()
        for d in g.choice(c.shape[0], size=2, replace=False):
            x = int(c[d]) ^ 1
            if (x & 0x7F) == 0x7F:
                x = int(c[d]) - 1
            c[d] = x
        k8[0, s] = c
    ks[0, toks] = ks[0, toks].max() * 4.0
    inp.k8 = torch.from_numpy(k8)
    inp.k_scale = torch.from_numpy(ks)
    return inp.to(DEV)


def test_fp8_filter_near_ties_inside_margin():
    """The FP8 filter where its margin matters: 9000 of 16000 keys are
    near-copies of one key, so the sampled thresholds and the k-th scores of
    the thresholded rows sit in runs of hundreds to thousands of scores within
    1% of each other (checked below on the oracle's scores), and the FP8
    estimate cannot order them; only the exact rescoring can.  The selection
    and attention must equal the stored-score path's bit for bit with the
    filter on and off, and the oracle's on sampled thresholded rows."""
    wl = W.PREFILL_32K.replace(name="prefill_L16000_near_ties", seq_len=16000, seed=35, sample_rows=0)
    announce("fp8 filter, near ties inside the margin", wl.name)
    inp = _near_tie_inputs(wl, 9000, 5)
    try:
        dsa.set_indexer_fp8(True)
        p, s8 = _both(inp)
    finally:
        dsa.set_indexer_fp8(False)
    _assert_same(p, s8, wl.name + " fp8")
    batch = dsa.Batch.from_inputs(inp)
    idx_e = torch.empty_like(s8[0])
    out_e, lse_e, _ = dsa.prefill_streaming(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q,
                                            inp.kv, inp.v, wl.scale, idx_out=idx_e, D_v=wl.D_v)
    torch.cuda.synchronize()
    _assert_same(p, (idx_e, out_e, lse_e), wl.name + " exact filter")
    idx, out, lse = (to_np(x) for x in s8)
    rows = list(range(7200, 16000, 880)) + [inp.num_rows - 1]
    ref = _oracle_check(inp, idx, out, lse, rows, exact=False)
    dense = 0
    for i in range(len(rows)):
        sc = np.asarray(ref["scores"][i])
        tau = np.sort(sc)[::-1][wl.k - 1]
        dense += int(np.count_nonzero(np.abs(sc - tau) <= 0.01 * abs(tau)) >= 100)
    assert dense >= 3, f"only {dense} checked rows have a dense run of scores at their k-th"


def test_streaming_chunked_prefill_late_chunk():
    """A chunk whose rows sit at positions 7500..9999 of a growing cache."""
    wl = W.CHUNKED_128K.replace(name="chunked_prefill_L10000_c2500", seq_len=10000, chunk=2500, seed=35,
                                sample_rows=0)
    announce("streaming chunked prefill", wl.name, "chunk 3")
    inp = W.generate(wl, DEV, chunk_index=3)
    p, s = _both(inp)
    _assert_same(p, s, wl.name)
    idx, out, lse = (to_np(x) for x in s)
    rows = W.sample_rows(wl, inp.num_rows, 16, always=(0, inp.num_rows - 1))
    _oracle_check(inp, idx, out, lse, rows, exact=False)


# ------------------------------------------------------------------ crafted rows for every fallback

_INT = W.PREFILL_32K.replace(name="prefill_L9000_int_crafted", seq_len=9000, seed=36, sample_rows=0,
                             integer_indexer=True)


def _e4m3(v):
    return torch.tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()


def _crafted(kind):
    """Integer inputs with q8 = +1 and w = +1 everywhere (score = H_I * ReLU(sum_d k8[s, d])), then:
    'underfill': sampled tokens (s % 32 == 0) score far above all others, so only
                 rank < k tokens reach the sampled threshold;
    'overflow':  sampled tokens score 0 and most others score > 0, so far more
                 than the capacity reach it;
    'zero_rows': every other query row is all zeros (every score 0: one big tie)."""
    inp = W.generate(_INT, DEV)
    one, three, mthree = _e4m3(1.0), _e4m3(3.0), _e4m3(-3.0)
    if kind in ("underfill", "overflow"):
        inp.q8.fill_(one)
        inp.w.fill_(1.0)
        k8 = inp.k8.view(-1, inp.k8.shape[-1])
        sampled = torch.arange(k8.shape[0], device=DEV) % STRIDE == 0
        if kind == "underfill":
            # others: integers in [-1, 1] (row sums <= 128); sampled: all +3 (sum 384)
            k8.copy_(torch.where(k8.view(torch.float8_e4m3fn).float().abs() > 1,
                                 torch.full_like(k8, one), k8))
            k8[sampled] = three
        else:
            # others: |values| so that most row sums are positive; sampled: all -3 (ReLU -> 0)
            k8.copy_(k8.view(torch.float8_e4m3fn).float().abs().to(torch.float8_e4m3fn).view(torch.uint8))
            k8[sampled] = mthree
    elif kind == "zero_rows":
        inp.q8[1::2] = 0
    return inp


@pytest.mark.parametrize("fp8", [False, True], ids=["exact_filter", "fp8_filter"])
@pytest.mark.parametrize("kind", ["underfill", "overflow", "zero_rows"])
def test_streaming_fallbacks_bit_exact(kind, fp8):
    """Crafted rows that leave the finalize too few candidates, too many, or
    none but ties, so that the fallback recomputes them; with the FP8 filter
    the exactify launch must leave such rows to it (and send there any row
    whose k-th lower bound does not clear the threshold)."""
    announce("streaming prefill crafted", kind, "fp8" if fp8 else "exact")
    inp = _crafted(kind)
    wl = inp.wl
    try:
        dsa.set_indexer_fp8(fp8)
        p, s = _both(inp)
    finally:
        dsa.set_indexer_fp8(False)
    _assert_same(p, s, f"crafted {kind}")
    idx, out, lse = (to_np(x) for x in s)
    n_rows = inp.num_rows
    cap = _cap(wl.k)
    rows = [0, 1, wl.k - 1, wl.k, wl.k + 1, cap - 1, cap, cap + 1, cap + 2, n_rows - 2, n_rows - 1]
    ref = _oracle_check(inp, idx, out, lse, rows, exact=True)
    # the construction does what it claims on the rows past the capacity
    for i, r in enumerate(rows):
        n = r + 1
        if n <= cap:
            continue
        sc = ref["scores"][i]
        samp = np.arange(n) % STRIDE == 0
        if kind == "underfill":
            assert sc[~samp].max() < sc[samp].min() and _rank(wl.k) < wl.k
        elif kind == "overflow":
            assert (sc[samp] == 0).all() and (sc[~samp] > 0).all()
            if n >= n_rows - 1:                       # 31/32 of 9000 tokens beat the sampled threshold
                assert (sc[~samp] > 0).sum() > cap
        elif r % 2 == 1:
            assert (sc == 0).all()
            assert np.array_equal(idx[r], np.arange(wl.k))


def test_streaming_long_context_chunk():
    """The last 320 rows of a 200000-token sequence (about 200 segments per row, 6250 sampled scores per
    threshold)."""
    wl = W.CHUNKED_128K.replace(name="chunked_prefill_L200000_c512", seq_len=200000, chunk=512, seed=41,
                                sample_rows=0)
    c = (wl.seq_len + wl.chunk - 1) // wl.chunk - 1
    announce("streaming chunked prefill", wl.name, "chunk", c)
    inp = W.generate(wl, DEV, chunk_index=c)
    p, s = _both(inp)
    _assert_same(p, s, wl.name)
    idx, out, lse = (to_np(x) for x in s)
    _oracle_check(inp, idx, out, lse, [0, inp.num_rows // 2, inp.num_rows - 1], exact=False)


def test_streaming_mixed_sequences():
    """Two sequences of different lengths with different numbers of query rows
    (positions 6000..8999 of a 9000-token sequence, 2000..6999 of a 7000-token
    one): per-row positions, thresholds and lists across sequences."""
    import dataclasses
    wl = W.PREFILL_32K.replace(name="prefill_b2_L9000_mixed", seqs=2, seq_len=9000, seed=39, sample_rows=0)
    announce("streaming prefill", wl.name, "lens 9000/7000, rows 3000/5000")
    full = W.generate(wl, DEV)
    sel = torch.cat([torch.arange(6000, 9000), torch.arange(9000, 14000)]).to(DEV)
    pick = lambda t: None if t is None else t[sel].contiguous()  # noqa: E731
    i32 = dict(dtype=torch.int32, device=DEV)
    inp = dataclasses.replace(full, seq_lens=torch.tensor([9000, 7000], **i32),
                              q_start=torch.tensor([0, 3000, 8000], **i32), num_rows=8000, max_q=5000, max_len=9000,
                              seq_lens_host=[9000, 7000], q_start_host=[0, 3000, 8000], q8=pick(full.q8),
                              q_scale=pick(full.q_scale), w=pick(full.w), q=pick(full.q))
    p, s = _both(inp)
    _assert_same(p, s, wl.name)
    idx, out, lse = (to_np(x) for x in s)
    # seq 0 rows 0..2999 (n = 6001..9000; the capacity 7168 is crossed at rows 1167/1168); seq 1 rows
    # 3000..7999 (n = 2001..7000, all under the capacity; k = 2048 is crossed at rows 3047/3048)
    rows = [0, 1167, 1168, 2999, 3000, 3046, 3047, 3048, 7999]
    rows = sorted(set(rows) | set(W.sample_rows(wl, 8000, 12, always=())))
    _oracle_check(inp, idx, out, lse, rows, exact=False)


def test_streaming_repeatable():
    """Two calls give bit-identical results (the list order from atomics never shows)."""
    wl = CASES[1]
    announce("streaming prefill repeat", wl.name)
    inp = W.generate(wl, DEV)
    batch = dsa.Batch.from_inputs(inp)
    res = []
    for _ in range(2):
        idx = torch.empty((inp.num_rows, wl.k), dtype=torch.int32, device=DEV)
        out, lse, _ = dsa.prefill_streaming(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q,
                                            inp.kv, inp.v, wl.scale, idx_out=idx, D_v=wl.D_v)
        torch.cuda.synchronize()
        res.append((idx, out, lse))
    _assert_same(res[0], res[1], "repeat")


def test_streaming_short_context_is_dense():
    wl = W.DENSE_PREFILL
    announce("streaming prefill dense", wl.name)
    inp = W.generate(wl, DEV)
    p, s = _both(inp)
    _assert_same(p, s, wl.name)
