"""Plain, slow CPU oracle of the lightning indexer's warm-up objective.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its binding) never touches it, and it shares
no code, table or constant with that path.

What it computes (tenelement.pl article "DeepSeek V3.2-Exp Cuts Long-Context
Costs with DeepSeek Sparse Attention (DSA) While Maintaining Benchmark
Parity", section "Proces Treningu DSA: Od Warm-up do Sparsity"): during a
short warm-up the main model is frozen and the indexer is trained, by a KL
divergence, to reproduce the dense model's attention distribution summed over
its heads.  For one query row t at position p (it sees tokens 0..p):

    target   a[s] = sum_h A[h, s] / sum_{h, s'} A[h, s'],  A[h] = softmax_s(scale * q[h] . K[s])
             (each head's softmax sums to one, so this is the mean over heads)
    model    log P[s] = I[s] - logsumexp_s' I[s']           (softmax of the indexer scores)
    loss     KL(a || P) = sum_s a[s] * (log a[s] - log P[s]),  with 0 * log 0 = 0

I[s] is the indexer score of the main path,
    I[s] = sum_j w[j] * ReLU(qd[j] . kd[s]),  qd = q_scale * q8,  kd = k_scale * k8,
so the trainable inputs are the dequantised indexer query qd, the dequantised
index key kd and the head weights w; the dense side (q, K) is frozen.  The
gradients are those of sum_t loss_t:

    dL/dI[s]    = P[s] - a[s]                                  (softmax + KL, sum a = 1)
    dL/dw[j]    = sum_s dI[s] * ReLU(z[j, s])                  z = qd[j] . kd[s]
    dL/dqd[j,:] = sum_s dI[s] * w[j] * [z[j, s] > 0] * kd[s, :]
    dL/dkd[s,:] = sum_t dI_t[s] * sum_j w_t[j] * [z_t[j, s] > 0] * qd_t[j, :]

ReLU'(0) is taken as 0 (the pages say nothing; a subgradient has to be
picked, and integer inputs hit z = 0 often).  All arithmetic is float64.

Parity status: pinned by tests under tests/ (target against torch.softmax,
KL against scipy.stats.entropy, KL = 0 and zero gradient when the indexer
distribution equals the target, central finite differences of the loss for
every gradient, closed forms for one head and one token).
"""
from __future__ import annotations

import numpy as np

from .dsa_oracle import decode_bf16, decode_e4m3fn, row_geometry


def dense_target(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Mean over heads of each head's softmax attention over the n visible rows.

    q [H, D], K [n, D] (float64) -> a [n], sum 1.
    """
    x = scale * (q @ K.T)                              # [H, n] dense logits
    x = x - x.max(axis=1, keepdims=True)
    e = np.exp(x)
    A = e / e.sum(axis=1, keepdims=True)               # per-head attention probabilities
    s = A.sum(axis=0)                                  # sum over heads
    return s / s.sum()                                 # L1 normalisation


def kl_and_grad(a: np.ndarray, I: np.ndarray):
    """KL(a || softmax(I)) and its gradient with respect to I.

    a [n] target distribution, I [n] scores (float64).
    """
    m = I.max()
    logP = I - (m + np.log(np.exp(I - m).sum()))
    pos = a > 0
    loss = float(np.sum(a[pos] * (np.log(a[pos]) - logP[pos])))
    return loss, np.exp(logP) - a


def indexer_parts(qd: np.ndarray, w: np.ndarray, kd: np.ndarray):
    """z [H_I, n] = qd . kd and the scores I [n] = sum_j w[j] ReLU(z[j])."""
    z = qd @ kd.T
    return z, w @ np.maximum(z, 0.0)


def row_objective(q, K, scale, qd, w, kd):
    """Loss and gradients of one row from dequantised float64 inputs.

    q [H, D], K [n, D], qd [H_I, d_I], w [H_I], kd [n, d_I].
    Returns (loss, dI [n], dw [H_I], dqd [H_I, d_I], dkd [n, d_I]).
    """
    a = dense_target(q, K, scale)
    z, I = indexer_parts(qd, w, kd)
    loss, dI = kl_and_grad(a, I)
    act = (z > 0).astype(np.float64)                   # ReLU'(z), 0 at z = 0
    dw = np.maximum(z, 0.0) @ dI
    coef = w[:, None] * act * dI[None, :]              # [H_I, n]: dI[s] w[j] [z > 0]
    dqd = coef @ kd
    dkd = coef.T @ qd
    return loss, dI, dw, dqd, dkd


def run_warmup(a: dict, rows=None):
    """The objective for the query rows of a batch (contiguous caches only).

    ``a`` holds numpy arrays: q [T,H,D] bf16 bits (or q_f floats), kv
    [B,cap,D] bf16 bits (or kv_f), scale, q8 [T,H_I,d_I] u8, q_scale [T] or
    None, w [T,H_I], k8 [B,cap,d_I] u8, k_scale [B,cap] or None, seq_lens,
    q_start; optional qd_f [T,H_I,d_I] / kd_f [B,cap,d_I] floats replace the
    dequantised FP8 inputs (for finite differences).  Returns per-row loss
    [T] and dI (dict of [n] arrays), and the gradients summed over ``rows``
    (all rows by default): dw [T,H_I], dq [T,H_I,d_I], dk [B,cap,d_I] (zero
    for tokens no listed row sees).
    """
    T = a["q8"].shape[0]
    geo = row_geometry(a["seq_lens"], a["q_start"], T)
    rows = range(T) if rows is None else rows
    B, cap, d_I = a["k8"].shape
    H_I = a["q8"].shape[1]
    loss = np.full(T, np.nan)
    dw = np.zeros((T, H_I))
    dq = np.zeros((T, H_I, d_I))
    dk = np.zeros((B, cap, d_I))
    dI_rows = {}
    for t in rows:
        b, p = geo[t]
        n = p + 1
        qrow = a["q_f"][t].astype(np.float64) if a.get("q_f") is not None else decode_bf16(a["q"][t])
        K = a["kv_f"][b, :n].astype(np.float64) if a.get("kv_f") is not None else decode_bf16(a["kv"][b, :n])
        if a.get("qd_f") is not None:                  # dequantised values given directly
            qd = a["qd_f"][t].astype(np.float64)
            kd = a["kd_f"][b, :n].astype(np.float64)
        else:
            qs = 1.0 if a.get("q_scale") is None else float(a["q_scale"][t])
            ks = np.ones(n) if a.get("k_scale") is None else a["k_scale"][b, :n].astype(np.float64)
            qd = decode_e4m3fn(a["q8"][t]) * qs
            kd = decode_e4m3fn(a["k8"][b, :n]) * ks[:, None]
        l, dI, dwr, dqr, dkr = row_objective(qrow, K, float(a["scale"]), qd,
                                             np.asarray(a["w"][t], dtype=np.float64), kd)
        loss[t] = l
        dI_rows[t] = dI
        dw[t] = dwr
        dq[t] = dqr
        dk[b, :n] += dkr
    return {"loss": loss, "dI": dI_rows, "dw": dw, "dq": dq, "dk": dk}
