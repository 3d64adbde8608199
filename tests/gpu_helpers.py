"""Shared pieces of the GPU parity tests: running the HIP path and the comparison rules."""
import numpy as np
import torch

import oracle
import sparse_attention_long_06_amd as dsa
from tests.oracle_io import arrays_of  # noqa: F401

DEV = "cuda:0"

# attention outputs (bf16): |gpu - ref| <= ATOL + RTOL * |ref|
ATT_ATOL, ATT_RTOL = 2e-2, 1e-2
# log-sum-exp: the denominators are accumulated in fp32 from the same bf16 inputs
LSE_ATOL = 1e-3
# indexer scores: |gpu - ref| <= SC_RTOL * max(|ref|, sum_j |w_j q_scale k_scale| ReLU(z_j))
SC_RTOL = 1e-4
# top-k on general inputs: any swap must lie within this relative distance of the k-th score
SWAP_RTOL = 1e-5


def announce(*what):
    print("[gpu case]", *what, flush=True)


def gpu_indexer(inp):
    batch = dsa.Batch.from_inputs(inp)
    return batch, dsa.indexer(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale)


def gpu_staged(inp):
    batch, scores = gpu_indexer(inp)
    idx = dsa.topk(batch, scores, inp.wl.k)
    out, lse = dsa.sparse_attn(batch, inp.q, inp.kv, inp.v, inp.wl.scale, idx, D_v=inp.wl.D_v)
    torch.cuda.synchronize()
    return scores, idx, out, lse


def oracle_abs_terms(a, rows):
    """sum_j |w_j| q_scale k_scale ReLU(z_j) per candidate: the scale of the score's rounding error."""
    return oracle.run_rows(a, rows, need=("scores", "abs"))["abs"]


def check_scores(gpu_scores, ref, absterms, rows, exact=False):
    for r, o, A in zip(rows, ref, absterms):
        g = gpu_scores[r, : len(o)].astype(np.float64)
        if exact:
            assert np.array_equal(g, o), f"row {r}: scores not exact"
        else:
            tol = SC_RTOL * np.maximum(np.abs(o), A)
            bad = np.abs(g - o) > tol
            assert not bad.any(), f"row {r}: {bad.sum()} scores off, worst {np.max(np.abs(g - o) - tol)}"


def check_topk_swaps(gpu_idx, ref_idx, ref_scores, k):
    """Same size; every index in the symmetric difference is a near-tie of the k-th score."""
    g = gpu_idx[gpu_idx >= 0]
    o = ref_idx[ref_idx >= 0]
    assert len(g) == len(o), (len(g), len(o))
    assert np.all(np.diff(g) > 0), "gpu indices not ascending"
    diff = np.setxor1d(g, o)
    if len(diff) == 0:
        return True
    tau = np.sort(ref_scores[o])[0]
    assert np.all(np.abs(ref_scores[diff] - tau) <= SWAP_RTOL * abs(tau)), \
        f"non-tie swaps {diff[:8]} around tau={tau}"
    return False


def check_attention(gpu_out, gpu_lse, ref_out, ref_lse, what=""):
    g = gpu_out.astype(np.float64)
    err = np.abs(g - ref_out) - (ATT_ATOL + ATT_RTOL * np.abs(ref_out))
    assert (err <= 0).all(), f"{what}: attention off by {err.max()} beyond tolerance"
    if gpu_lse is not None:
        assert np.allclose(gpu_lse, ref_lse, atol=LSE_ATOL, rtol=0), f"{what}: lse off {np.abs(gpu_lse - ref_lse).max()}"


def to_np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def oracle_rows(a, rows, need=("scores", "abs", "idx", "out"), idx_override=None, workers=16, per_task=8):
    """oracle.run_rows over ``rows``, in tasks of ``per_task`` rows on a thread pool.

    The oracle's heavy steps (matrix products, sorts, elementwise passes over
    large arrays) run inside numpy with the GIL released, so threads overlap;
    BLAS is held to one thread per worker.  The result is the one run_rows
    gives for the same rows in one call (the same function on each task)."""
    from concurrent.futures import ThreadPoolExecutor
    import threadpoolctl

    rows = list(rows)
    tasks = [rows[i: i + per_task] for i in range(0, len(rows), per_task)]
    with threadpoolctl.threadpool_limits(1), ThreadPoolExecutor(max(1, min(workers, len(tasks)))) as ex:
        parts = list(ex.map(lambda rs: oracle.run_rows(a, rs, need=need, idx_override=idx_override), tasks))
    return {key: [x for p in parts for x in p[key]] for key in parts[0]} if parts else \
        {"scores": [], "abs": [], "idx": [], "out": [], "lse": []}


def check_rows(a, rows, g_idx, g_out, g_lse, ref, k, what, min_same=0.9):
    """The selection rule on every row and the attention check on every row.

    g_idx/g_out/g_lse hold the GPU's results for ``rows`` in the same order.
    Where the GPU selected the oracle's set, its attention is compared with the
    oracle's end-to-end output; where a near-tie swap made the sets differ,
    with the oracle's attention over the GPU's own set.  Returns the number of
    rows whose sets agree; at least ``min_same`` of the rows must."""
    same, differ = 0, {}
    for i, r in enumerate(rows):
        if check_topk_swaps(g_idx[i], ref["idx"][i], ref["scores"][i], k):
            same += 1
            check_attention(g_out[i], g_lse[i], ref["out"][i], ref["lse"][i], f"{what} row {r}")
        else:
            differ[r] = i
    if differ:
        own = oracle_rows(a, list(differ), need=("scores", "idx", "out"),
                          idx_override={r: np.asarray(g_idx[i]) for r, i in differ.items()})
        for j, (r, i) in enumerate(differ.items()):
            check_attention(g_out[i], g_lse[i], own["out"][j], own["lse"][j], f"{what} row {r} (GPU's own set)")
    assert same >= min_same * len(rows), f"{what}: only {same}/{len(rows)} rows selected the same set"
    return same
