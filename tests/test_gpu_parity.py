"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Rules (see tests/gpu_helpers.py): integer-exact inputs must give bit-exact
scores and indices; otherwise scores within 1e-4 of their absolute-term
scale, top-k swaps only among near-ties of the k-th score (bit-exact when
both sides select from the same fp32 scores), attention within
2e-2 + 1e-2*|ref|.  No oracle input comes from the HIP path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_long_06_amd as dsa
from tests.gpu_helpers import (DEV, announce, arrays_of, check_attention, check_rows, check_scores,
                               gpu_staged, oracle_rows, to_np)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ tiny prefill (integer-exact indexer)

def test_tiny_prefill_bit_exact_selection_and_attention():
    wl = W.TINY_PREFILL
    announce("tiny_prefill_L256 staged", wl)
    inp = W.generate(wl, "cpu")
    scores, idx, out, lse = gpu_staged(inp.to(DEV))
    scores, idx, out, lse = to_np(scores), to_np(idx), to_np(out), to_np(lse)

    a = arrays_of(inp)
    rows = list(range(wl.seq_len))
    ref = oracle.run_rows(a, rows)
    for r in rows:
        assert np.array_equal(scores[r, : r + 1].astype(np.float64), ref["scores"][r]), f"scores row {r}"
        assert np.array_equal(idx[r], ref["idx"][r]), f"top-k row {r}"
        check_attention(out[r], lse[r], ref["out"][r], ref["lse"][r], f"row {r}")
    # against the fp32 originals the bf16 rounding of q/k/v is the only difference
    ref32 = oracle.run_rows(arrays_of(inp, use_fp32_originals=True), rows[::17])
    for i, r in enumerate(rows[::17]):
        check_attention(out[r], None, ref32["out"][i], None, f"fp32 originals row {r}")


# ------------------------------------------------------------------ production shapes, small contexts

SMALL = [W.SMALL_DECODE, W.SMALL_PAGED, W.SMALL_PREFILL]


def _rows_for(inp):
    if inp.wl.kind == "decode":
        return list(range(inp.num_rows))
    return W.sample_rows(inp.wl, inp.num_rows, 160,
                         always=(0, 1, 2, 2046, 2047, 2048, 2049, inp.num_rows - 1))


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_end_to_end(wl):
    announce("end-to-end", wl.name)
    inp = W.generate(wl, DEV)
    scores, idx, out, lse = gpu_staged(inp)
    scores, idx, out, lse = to_np(scores), to_np(idx), to_np(out), to_np(lse)
    a = arrays_of(inp)
    rows = _rows_for(inp)
    ref = oracle_rows(a, rows)
    check_scores(scores, ref["scores"], ref["abs"], rows)
    check_rows(a, rows, idx[rows], out[rows], lse[rows], ref, wl.k, wl.name)


# Budget and head-shape variants: other k, other indexer head counts, the
# d_I = 32 indexer layout at production attention shapes, through the fused
# entry points.
VARIANTS = [
    W.SMALL_DECODE.replace(name="decode_b3_ctx5000_k512_hi32", k=512, H_I=32, seed=21),
    W.SMALL_DECODE.replace(name="decode_b3_ctx5000_k1024_hi48", k=1024, H_I=48, seed=22),
    W.SMALL_DECODE.replace(name="decode_b3_ctx5000_k4096_hi16_di32", k=4096, H_I=16, d_I=32, seed=23),
    W.SMALL_PAGED.replace(name="paged_decode_b5_mixed100_6000_k1024", k=1024, seed=24),
    W.SMALL_PREFILL.replace(name="prefill_L2500_k512_hi8", k=512, H_I=8, seed=25),
    # paged caches under the prefill layout: the prefill indexer's page lookups
    # (8-key groups, ragged ends) and the attention gather through the table
    W.SMALL_PREFILL.replace(name="prefill_b2_L2300_paged64", seqs=2, seq_len=2300, paged=True, block_size=64,
                            seed=26),
    W.SMALL_PREFILL.replace(name="prefill_L2100_paged16", seq_len=2100, paged=True, block_size=16, seed=27),
    # a wider length range than the 4K-128K paged batch: 1000 to 262144 tokens per sequence
    W.PAGED_DECODE_MIXED.replace(name="paged_decode_b6_mixed1k_256k", seqs=6, seq_len=262144, min_len=1000,
                                 seed=40),
]


@pytest.mark.parametrize("wl", VARIANTS, ids=[w.name for w in VARIANTS])
def test_budget_and_shape_variants(wl):
    announce("variant", wl.name)
    inp = W.generate(wl, DEV)
    batch = dsa.Batch.from_inputs(inp)
    idx = torch.empty((inp.num_rows, wl.k), dtype=torch.int32, device=DEV)
    call = dsa.prefill if inp.q_start is not None else dsa.decode
    out, lse, _ = call(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q, inp.kv, inp.v,
                       wl.scale, idx_out=idx, D_v=wl.D_v)
    scores = dsa.indexer(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale)
    torch.cuda.synchronize()
    idx, out, lse, scores = to_np(idx), to_np(out), to_np(lse), to_np(scores)
    a = arrays_of(inp)
    rows = list(range(inp.num_rows)) if wl.kind == "decode" else W.sample_rows(
        wl, inp.num_rows, 96, always=(0, wl.k - 1, wl.k, inp.num_rows - 1))
    ref = oracle_rows(a, rows)
    check_scores(scores, ref["scores"], ref["abs"], rows)
    check_rows(a, rows, idx[rows], out[rows], lse[rows], ref, wl.k, wl.name)


def test_small_chunked_prefill():
    wl = W.SMALL_CHUNKED
    first = W.generate(wl, DEV, chunk_index=0)
    cache = W.cache_of(first)
    nchunks = (wl.seq_len + wl.chunk - 1) // wl.chunk
    for c in range(nchunks):
        announce("chunked prefill", wl.name, "chunk", c)
        inp = first if c == 0 else W.generate(wl, DEV, chunk_index=c, cache=cache)
        scores, idx, out, lse = (to_np(x) for x in gpu_staged(inp))
        a = arrays_of(inp)
        rows = W.sample_rows(wl, inp.num_rows, 40, always=(0, inp.num_rows - 1))
        ref = oracle_rows(a, rows)
        check_scores(scores, ref["scores"], ref["abs"], rows)
        check_rows(a, rows, idx[rows], out[rows], lse[rows], ref, wl.k, f"{wl.name} chunk {c}")


# ------------------------------------------------------------------ attention stage on the oracle's index sets

@pytest.mark.parametrize("wl", [W.SMALL_DECODE, W.SMALL_PAGED, W.SMALL_PREFILL], ids=lambda w: w.name)
def test_attention_stage_on_oracle_indices(wl):
    announce("attention stage", wl.name)
    inp = W.generate(wl, DEV)
    a = arrays_of(inp)
    rows = list(range(inp.num_rows)) if inp.num_rows <= 16 else W.sample_rows(wl, inp.num_rows, 64, always=(0, 2047, inp.num_rows - 1))
    ref = oracle.run_rows(a, rows)
    idx_full = np.full((inp.num_rows, wl.k), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        idx_full[r] = ref["idx"][i]
    batch = dsa.Batch.from_inputs(inp)
    out, lse = dsa.sparse_attn(batch, inp.q, inp.kv, inp.v, wl.scale, torch.from_numpy(idx_full).to(DEV),
                               D_v=wl.D_v)
    out, lse = to_np(out), to_np(lse)
    for i, r in enumerate(rows):
        check_attention(out[r], lse[r], ref["out"][i], ref["lse"][i], f"{wl.name} row {r}")
    # rows given no index at all: zero output, lse = -inf
    empty = [r for r in range(inp.num_rows) if r not in set(rows)][:3]
    for r in empty:
        assert np.all(out[r] == 0) and np.all(np.isneginf(lse[r]))


def test_attention_ragged_and_padded_index_sets():
    # index sets shorter than k (-1 padded), unsorted, and a single token
    wl = W.SMALL_DECODE
    announce("attention ragged sets", wl.name)
    inp = W.generate(wl, DEV)
    a = arrays_of(inp)
    rng = np.random.default_rng(5)
    idx = np.full((inp.num_rows, wl.k), -1, dtype=np.int32)
    sets = []
    for r, L in enumerate(inp.seq_lens_host):
        m = [1, 777, 2048][r % 3]
        s = rng.choice(L, size=m, replace=False).astype(np.int32)
        idx[r, rng.permutation(wl.k)[:m]] = s
        sets.append(np.sort(s))
    batch = dsa.Batch.from_inputs(inp)
    out, lse = dsa.sparse_attn(batch, inp.q, inp.kv, inp.v, wl.scale, torch.from_numpy(idx).to(DEV), D_v=wl.D_v)
    out, lse = to_np(out), to_np(lse)
    for r, s in enumerate(sets):
        K = oracle.decode_bf16(a["kv"][r, s])
        ro, rl = oracle.sparse_attention(oracle.decode_bf16(a["q"][r]), K, K[:, : wl.D_v], wl.scale)
        check_attention(out[r], lse[r], ro, rl, f"row {r} m={len(s)}")


def test_attention_split_counts_agree():
    """The split-K form of the online softmax: one decode input attended with 1,
    2, 4 and 8 splits per row (dsa_set_attn_splits; 2 and 4 splits take the
    merge kernel that handles several items per thread).  Each split writes its
    normalised partial output in bf16 (relative rounding 2^-9) and its lse in
    fp32; the merge weights sum to one, so two split counts differ by at most
    two bf16 roundings of the partials plus one of the output: |a - b| <=
    2^-7 (|a| + |b|) + 2^-9 * max|partial|, bounded here by 2^-7 * max|out| * 4.
    The lse values differ only by fp32 rounding of the merge.  Every count is
    bit-identical across two runs."""
    wl = W.SMALL_DECODE
    announce("attention split counts", wl.name)
    inp = W.generate(wl, DEV)
    batch = dsa.Batch.from_inputs(inp)
    scores = dsa.indexer(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale)
    idx = dsa.topk(batch, scores, wl.k)
    res = {}
    try:
        for ns in (1, 2, 4, 8):
            dsa.set_attn_splits(ns)
            runs = [dsa.sparse_attn(batch, inp.q, inp.kv, inp.v, wl.scale, idx, D_v=wl.D_v) for _ in range(2)]
            torch.cuda.synchronize()
            assert torch.equal(runs[0][0].view(torch.int16), runs[1][0].view(torch.int16)), f"nsplit {ns}: not deterministic"
            assert torch.equal(runs[0][1], runs[1][1]), f"nsplit {ns}: lse not deterministic"
            res[ns] = (to_np(runs[0][0]).astype(np.float64), to_np(runs[0][1]).astype(np.float64))
    finally:
        dsa.set_attn_splits(0)
    o1, l1 = res[1]
    scale = np.abs(o1).max()
    for ns in (2, 4, 8):
        o, l = res[ns]
        assert np.abs(o - o1).max() <= 4 * 2.0 ** -7 * scale, f"nsplit {ns}: {np.abs(o - o1).max()} vs {scale}"
        assert np.allclose(l, l1, rtol=0, atol=1e-5), f"nsplit {ns}: lse off {np.abs(l - l1).max()}"
    # and the unsplit result is the oracle's within the attention rule
    a = arrays_of(inp)
    rows = list(range(inp.num_rows))
    ref = oracle.run_rows(a, rows, idx_override={r: to_np(idx)[r] for r in rows})
    for r in rows:
        check_attention(o1[r], l1[r], ref["out"][r], ref["lse"][r], f"nsplit 1 row {r}")


# ------------------------------------------------------------------ top-k kernel on shared fp32 scores (bit-exact)

def _decode_batch(lens):
    t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return dsa.Batch(seq_lens=t, num_rows=len(lens), max_q=1, max_len=max(lens))


def _prefill_batch(L):
    return dsa.Batch(seq_lens=torch.tensor([L], dtype=torch.int32, device=DEV), num_rows=L, max_q=L, max_len=L,
                     q_start=torch.tensor([0, L], dtype=torch.int32, device=DEV))


def _check_topk_rows(scores, lens_of_row, k, idx):
    s = scores.cpu().numpy()
    g = idx.cpu().numpy()
    for r, n in enumerate(lens_of_row):
        ref = oracle.topk_indices(s[r, :n], k)
        assert np.array_equal(g[r], ref), f"row {r} (n={n}, k={k}): first diff at {np.argmax(g[r] != ref)}"


@pytest.mark.parametrize("kind", ["normal", "ties", "signed_zeros", "all_equal", "sparse_ones"])
@pytest.mark.parametrize("k", [1, 64, 2048, 4096])
def test_topk_split_mode_bit_exact(kind, k):
    announce("topk split mode", kind, k)
    lens = [100, 2048, 2049, 5000, 20000, 33333, 4096 + 1, 9000]
    batch = _decode_batch(lens)
    scores = W.synthetic_scores(len(lens), (max(lens) + 3) // 4 * 4, kind, seed=k, device=DEV)
    idx = dsa.topk(batch, scores, k)
    torch.cuda.synchronize()
    _check_topk_rows(scores, lens, k, idx)


@pytest.mark.parametrize("kind", ["normal", "ties", "all_equal"])
def test_topk_split_mode_many_mixed_rows(kind):
    # 200 rows of 2049-40000 candidates: split mode with 16 slices per row, so
    # the short rows leave most of their slices empty
    announce("topk split mode mixed rows", kind)
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(2049, 40001, size=200)]
    lens[0], lens[1] = 40000, 2049
    batch = _decode_batch(lens)
    scores = W.synthetic_scores(len(lens), 40000, kind, seed=23, device=DEV)
    idx = dsa.topk(batch, scores, 2048)
    torch.cuda.synchronize()
    _check_topk_rows(scores, lens, 2048, idx)


@pytest.mark.parametrize("kind", ["normal", "ties", "signed_zeros", "sparse_ones"])
def test_topk_row_mode_bit_exact(kind):
    announce("topk row mode", kind)
    L = 3000
    batch = _prefill_batch(L)
    scores = W.synthetic_scores(L, L, kind, seed=7, device=DEV)
    idx = dsa.topk(batch, scores, 2048)
    torch.cuda.synchronize()
    _check_topk_rows(scores, [r + 1 for r in range(L)], 2048, idx)


@pytest.mark.parametrize("kind", ["all_equal", "sparse_ones", "normal"])
def test_topk_row_mode_long_rows(kind):
    # > 512 rows of up to 20000 candidates: row mode, including the path where
    # the boundary bin overflows the LDS candidate buffer
    announce("topk row mode long rows", kind)
    lens = [20000 - 17 * i for i in range(600)]
    batch = _decode_batch(lens)
    scores = W.synthetic_scores(len(lens), 20000, kind, seed=3, device=DEV)
    idx = dsa.topk(batch, scores, 2048)
    torch.cuda.synchronize()
    _check_topk_rows(scores, lens, 2048, idx)


@pytest.mark.parametrize("kind", ["normal", "ties", "signed_zeros", "all_equal", "sparse_ones"])
@pytest.mark.parametrize("k", [64, 2048, 4096])
def test_topk_row_mode_40k_rows(kind, k):
    # > 512 rows of 17000-40000 candidates (row mode) for every score pattern
    # and budget: boundary bins from a few keys (normal) to the whole row
    # (all equal), candidates staged in LDS or read from global memory
    announce("topk row mode 40k rows", kind, k)
    lens = [40000 - 45 * i for i in range(520)]
    batch = _decode_batch(lens)
    scores = W.synthetic_scores(len(lens), 40000, kind, seed=11 + k, device=DEV)
    idx = dsa.topk(batch, scores, k)
    torch.cuda.synchronize()
    _check_topk_rows(scores, lens, k, idx)


# ------------------------------------------------------------------ fused decode

@pytest.mark.parametrize("wl", [W.SMALL_DECODE, W.SMALL_PAGED], ids=lambda w: w.name)
def test_fused_decode_matches_staged_bitwise(wl):
    announce("fused decode vs staged", wl.name)
    inp = W.generate(wl, DEV)
    scores, idx_s, out_s, lse_s = gpu_staged(inp)
    batch = dsa.Batch.from_inputs(inp)
    idx_f = torch.empty_like(idx_s)
    out_f, lse_f, _ = dsa.decode(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q, inp.kv,
                                 inp.v, wl.scale, idx_out=idx_f, D_v=wl.D_v)
    out_g, lse_g, _ = dsa.decode(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q, inp.kv,
                                 inp.v, wl.scale, D_v=wl.D_v)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_s)
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(lse_f, lse_s)
    # a second fused call (no index output) is bit-identical too: no races, no float atomics
    assert torch.equal(out_g.view(torch.int16), out_f.view(torch.int16))
    assert torch.equal(lse_g, lse_f)


def _decode_against_staged_and_oracle(inp, what, exact):
    wl = inp.wl
    batch = dsa.Batch.from_inputs(inp)
    idx_f = torch.empty((inp.num_rows, wl.k), dtype=torch.int32, device=DEV)
    out_f, lse_f, _ = dsa.decode(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q, inp.kv,
                                 inp.v, wl.scale, idx_out=idx_f, D_v=wl.D_v)
    scores, idx_s, out_s, lse_s = gpu_staged(inp)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_s), f"{what}: fused selection differs from the staged top-k"
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16)), f"{what}: output differs"
    a = arrays_of(inp)
    rows = list(range(inp.num_rows))
    ref = oracle_rows(a, rows)
    g_idx, g_out, g_lse = to_np(idx_f), to_np(out_f), to_np(lse_f)
    if exact:
        for r in rows:
            assert np.array_equal(g_idx[r], ref["idx"][r]), f"{what} row {r}: selection not exact"
    check_rows(a, rows, g_idx, g_out, g_lse, ref, wl.k, what, min_same=1.0 if exact else 0.9)


def test_fused_decode_chunk_holding_the_top_k():
    """Integer indexer inputs where 3000 consecutive tokens of every sequence
    score far above the rest (and tie among themselves): the decode chunks
    they fill hold more of the top-k than their candidate lists keep, so the
    fused selection must notice the cut and select those rows again from
    their full scores; the result is the exact top-k (lowest tokens among
    the ties)."""
    wl = W.SMALL_DECODE.replace(name="decode_b3_ctx5000_int_dominant_run", integer_indexer=True, seed=61)
    announce("fused decode, dominant token run", wl.name)
    inp = W.generate(wl, "cpu")
    three = torch.tensor(3.0).to(torch.float8_e4m3fn).view(torch.uint8)
    inp.q8[:, 0, :] = three                      # head 0: all +3
    inp.w[:, 0] = 2.0
    inp.w[:, 1:] = 0.0
    inp.k8[:, 1000:4000, :] = three              # z = 128 * 9 for these tokens, |z| <= 128 * 9 elsewhere
    inp.k8[:, :1000, :] = 0
    inp.k8[:, 4000:, :] = 0
    _decode_against_staged_and_oracle(inp.to(DEV), wl.name, exact=True)


def test_fused_decode_integer_ties():
    """Integer scores with many exact ties at the k-th key: cut chunks whose
    smallest kept key ties the k-th key are selected again from the scores."""
    wl = W.SMALL_DECODE.replace(name="decode_b3_ctx5000_int", integer_indexer=True, seed=62)
    announce("fused decode, integer ties", wl.name)
    _decode_against_staged_and_oracle(W.generate(wl, "cpu").to(DEV), wl.name, exact=True)


# ------------------------------------------------------------------ fused prefill

@pytest.mark.parametrize("wl", [W.TINY_PREFILL, W.SMALL_PREFILL, W.SMALL_CHUNKED], ids=lambda w: w.name)
def test_fused_prefill_matches_staged_bitwise(wl):
    announce("fused prefill vs staged", wl.name)
    inp = W.generate(wl, DEV, chunk_index=1) if wl.chunk else W.generate(wl, DEV)
    scores, idx_s, out_s, lse_s = gpu_staged(inp)
    batch = dsa.Batch.from_inputs(inp)
    idx_f = torch.empty_like(idx_s)
    out_f, lse_f, _ = dsa.prefill(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q, inp.kv,
                                  inp.v, wl.scale, idx_out=idx_f, D_v=wl.D_v)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_s)
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(lse_f, lse_s)


@pytest.mark.parametrize("wl", [W.DENSE_PREFILL, W.DENSE_DECODE], ids=lambda w: w.name)
def test_short_context_is_dense_attention(wl):
    """max_len <= k: the fused entry points skip the indexer; the result is
    dense causal attention over every prior token (checked against the oracle,
    whose selection keeps every token when k >= t + 1)."""
    announce("short-context dense path", wl.name)
    inp = W.generate(wl, DEV)
    batch = dsa.Batch.from_inputs(inp)
    idx = torch.empty((inp.num_rows, wl.k), dtype=torch.int32, device=DEV)
    call = dsa.prefill if inp.q_start is not None else dsa.decode
    out, lse, _ = call(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q, inp.kv, inp.v,
                       wl.scale, idx_out=idx, D_v=wl.D_v)
    torch.cuda.synchronize()
    _, pos = inp.row_positions()
    g_idx = to_np(idx)
    for r, p in enumerate(pos):
        assert g_idx[r][: p + 1].tolist() == list(range(p + 1))
        assert (g_idx[r][p + 1:] == -1).all()
    rows = list(range(inp.num_rows)) if inp.num_rows <= 64 else W.sample_rows(wl, inp.num_rows, 64, always=(0, inp.num_rows - 1))
    a = arrays_of(inp)
    ref = oracle.run_rows(a, rows)
    g_out, g_lse = to_np(out), to_np(lse)
    for i, r in enumerate(rows):
        check_attention(g_out[r], g_lse[r], ref["out"][i], ref["lse"][i], f"{wl.name} row {r}")


def test_binding_reports_bad_arguments():
    wl = W.SMALL_DECODE
    announce("binding error path")
    inp = W.generate(wl, DEV)
    batch = dsa.Batch.from_inputs(inp)
    bad_q8 = torch.zeros((inp.num_rows, 64, 64), dtype=torch.uint8, device=DEV)   # d_I = 64: no kernel
    with pytest.raises(dsa.DsaError, match="DSA_ERR_UNSUPPORTED"):
        dsa.indexer(batch, bad_q8, inp.q_scale, inp.w, inp.k8, inp.k_scale)
    with pytest.raises(ValueError):
        dsa.topk(batch, torch.zeros((inp.num_rows, 5000), device=DEV), 5000)   # k > 4096
