"""Host-side check of the streaming selection's sampling margins (no GPU, no oracle).

dsa_prefill_streaming thresholds a row on the scores of every 32nd token: the
pair order (score desc, token asc) of the rank-th largest sample, rank =
max(ceil(k/16), 64).  Every token at or above it becomes a candidate.  The
selection stays exact either way (rows outside [k, capacity] are recomputed);
these margins are what keep the recompute rare.  Restates the constants of
csrc/dsa_kernels.h (kStreamStride, stream_rank, stream_cap).
"""
import numpy as np

STRIDE = 32


def rank(k):
    return max((k + 15) // 16, 64)


def cap(k):
    return 56 * rank(k)


def kept_counts(n, k, rows, rng):
    s = rng.standard_normal((rows, n)).astype(np.float32)
    samp = s[:, ::STRIDE]
    r = rank(k)
    # the rank-th largest sampled score (continuous scores: no ties)
    thr = -np.partition(-samp, r - 1, axis=1)[:, r - 1]
    return (s >= thr[:, None]).sum(axis=1)


def test_capacity_and_rank_for_the_budgets():
    assert (rank(2048), cap(2048)) == (128, 7168)
    assert (rank(64), cap(64)) == (64, 3584)
    for k in (1, 64, 512, 1024, 2048):
        # expected kept count STRIDE * rank lies between k and the capacity with room on both sides
        assert k < STRIDE * rank(k) < cap(k)
        # rows that are thresholded (n > cap) have more samples than the rank
        assert (cap(k) + 1 + STRIDE - 1) // STRIDE > rank(k)


def test_kept_counts_stay_inside_the_margins():
    rng = np.random.default_rng(7)
    for n, k in ((cap(2048) + 1, 2048), (32768, 2048), (131072, 2048), (20000, 512)):
        c = kept_counts(n, k, 200 if n < 100000 else 60, rng)
        assert c.min() >= k, (n, k, c.min())
        assert c.max() <= cap(k), (n, k, c.max())
        mean = STRIDE * rank(k)
        assert abs(c.mean() - mean) < 0.05 * mean, (n, k, c.mean())
