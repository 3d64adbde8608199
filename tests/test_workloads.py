"""Seeded input generation (CPU): shapes, determinism, paging, and the tiny workload end to end."""
import numpy as np
import torch

import oracle
import workloads as W
from tests.oracle_io import arrays_of


def test_tiny_workload_shapes_and_determinism():
    a = W.generate(W.TINY_PREFILL, "cpu")
    b = W.generate(W.TINY_PREFILL, "cpu")
    assert a.q8.shape == (256, 4, 32) and a.q8.dtype == torch.uint8
    assert a.k8.shape == (1, 256, 32)
    assert a.q.shape == (256, 8, 64) and a.q.dtype == torch.bfloat16
    assert a.v.shape == (1, 256, 64)
    for x, y in [(a.q8, b.q8), (a.w, b.w), (a.k8, b.k8), (a.q, b.q), (a.kv, b.kv)]:
        assert torch.equal(x, y)
    vals = a.q8.view(torch.float8_e4m3fn).float()
    assert vals.min() >= -3 and vals.max() <= 3 and torch.equal(vals, vals.round())
    assert a.w.min() >= -2 and a.w.max() <= 2


def test_quantize_recipe_roundtrip():
    x = torch.randn(5, 7, 16, generator=torch.Generator().manual_seed(0))
    codes, scale = W.quantize_e4m3fn(x, 2)
    deq = codes.view(torch.float8_e4m3fn).float() * scale[:, None, None]
    assert scale.shape == (5,)
    assert torch.all((deq - x).abs() <= 0.0625 * x.abs() + 1e-6 * scale[:, None, None])
    assert codes.view(torch.float8_e4m3fn).float().abs().amax() == 448.0


def test_paged_lengths_and_table():
    wl = W.SMALL_PAGED
    inp = W.generate(wl, "cpu")
    lens = inp.seq_lens_host
    assert all(wl.min_len <= L <= wl.seq_len for L in lens)
    t = inp.block_table
    nblk = [(L + 63) // 64 for L in lens]
    used = torch.cat([t[b, :n] for b, n in enumerate(nblk)])
    assert sorted(used.tolist()) == list(range(sum(nblk)))
    assert inp.k8.shape[0] == sum(nblk) and inp.k8.shape[1] == 64


def test_tiny_workload_oracle_integer_scores_and_invariants():
    inp = W.generate(W.TINY_PREFILL, "cpu")
    a = arrays_of(inp)
    rows = [0, 1, 63, 64, 65, 200, 255]
    res = oracle.run_rows(a, rows)
    for r, sc, idx in zip(rows, res["scores"], res["idx"]):
        assert len(sc) == r + 1
        assert np.array_equal(sc, np.round(sc))             # integer inputs: exact integer scores
        m = min(64, r + 1)
        sel = idx[:m]
        assert (idx[m:] == -1).all() and (np.diff(sel) > 0).all() and sel.max() <= r
    for o in res["out"]:
        assert np.isfinite(o).all()


def test_sample_rows_include_required():
    wl = W.PREFILL_32K
    rows = W.sample_rows(wl, 32768, 512, always=(0, 1, 2046, 2047, 2048, 2049, 32767))
    assert len(rows) == 512 and len(set(rows)) == 512
    assert {0, 1, 2046, 2047, 2048, 2049, 32767} <= set(rows)
    assert rows == W.sample_rows(wl, 32768, 512, always=(0, 1, 2046, 2047, 2048, 2049, 32767))
