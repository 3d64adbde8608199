"""GPU parity of the indexer warm-up objective (dsa_indexer_warmup) against the oracle.

Comparison rules (the arithmetic behind them):
  * loss: the kernels take exp2/log2 of fp32 values and sum in fp32, so
    |loss - ref| <= 1e-4 * sum_s a_s (|log a_s| + |log P_s|) + 1e-6.
  * gradients: dI = P - a is formed in fp32 (error ~1e-5 of P + a), the
    coefficients enter the MFMAs as bf16 hi + lo parts (2^-17 relative) and
    the sums run in fp32, so each gradient entry is checked against
    GRAD_RTOL times its absolute-term sum (the same sum with |dI| replaced
    by P + a and every factor by its magnitude).
  * the ReLU mask [z > 0] is a decision taken on the kernels' fp32 z: where
    |z| is within 1e-6 of sum_d |q_d k_d| (the bf16 MFMA sums to ~3e-8 of
    that) either mask is correct, so such pairs add their whole contribution
    to the tolerance of the entries they touch.  Integer inputs make z exact
    on both sides; they are compared without this allowance.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import warmup_oracle as W
import sparse_attention_long_06_amd as dsa
import workloads
from tests.gpu_helpers import DEV, announce, arrays_of

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-4
GRAD_RTOL = 2e-4
AMBIG = 1e-6


def _run(inp, grads=True, **kw):
    batch = dsa.Batch.from_inputs(inp)
    out = dsa.indexer_warmup(batch, inp.q, inp.kv, inp.wl.scale, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale,
                             grads=grads, **kw)
    torch.cuda.synchronize()
    return [None if x is None else x.cpu().numpy() for x in out]


def _reference(a, rows, allow_ambiguous=True):
    """Oracle outputs for ``rows`` and the tolerance scales of every compared entry."""
    T = a["q8"].shape[0]
    geo = oracle.row_geometry(a["seq_lens"], a["q_start"], T)
    B, cap, d_I = a["k8"].shape
    H_I = a["q8"].shape[1]
    ref = W.run_warmup(a, rows)
    loss_tol = np.zeros(T)
    dw_tol = np.zeros((T, H_I))
    dq_tol = np.zeros((T, H_I, d_I))
    dk_tol = np.zeros((B, cap, d_I))
    for t in rows:
        b, p = geo[t]
        n = p + 1
        q = oracle.decode_bf16(a["q"][t])
        K = oracle.decode_bf16(a["kv"][b, :n])
        qs = 1.0 if a.get("q_scale") is None else float(a["q_scale"][t])
        ks = np.ones(n) if a.get("k_scale") is None else a["k_scale"][b, :n].astype(np.float64)
        q8 = oracle.decode_e4m3fn(a["q8"][t])
        k8 = oracle.decode_e4m3fn(a["k8"][b, :n])
        qd, kd = q8 * qs, k8 * ks[:, None]
        w = a["w"][t].astype(np.float64)
        at = W.dense_target(q, K, float(a["scale"]))
        z, I = W.indexer_parts(qd, w, kd)
        logP = I - (I.max() + np.log(np.exp(I - I.max()).sum()))
        P = np.exp(logP)
        pos = at > 0
        loss_tol[t] = LOSS_RTOL * np.sum(at[pos] * (np.abs(np.log(at[pos])) + np.abs(logP[pos]))) + 1e-6
        mag = P + at                                          # scale of |dI|
        act = (z > 0).astype(np.float64)
        dw_tol[t] = GRAD_RTOL * (np.maximum(z, 0.0) @ mag)
        coef = np.abs(w)[:, None] * act * mag[None, :]        # [H_I, n]
        dq_tol[t] = GRAD_RTOL * (coef @ np.abs(kd))
        dk_tol[b, :n] += GRAD_RTOL * (coef.T @ np.abs(qd))
        if allow_ambiguous:
            zabs = np.abs(q8) @ np.abs(k8).T                   # sum_d |q8_d k8_d|
            amb = (np.abs(q8 @ k8.T) <= AMBIG * zabs).astype(np.float64)
            if amb.any():
                dI = np.abs(P - at)
                c2 = np.abs(w)[:, None] * amb * dI[None, :]
                dq_tol[t] += c2 @ np.abs(kd)
                dk_tol[b, :n] += c2.T @ np.abs(qd)
    return ref, dict(loss=loss_tol, dw=dw_tol, dq=dq_tol, dk=dk_tol)


def _check(name, got, want, tol):
    err = np.abs(got.astype(np.float64) - want)
    bad = err > tol
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} entries off; worst excess "
                           f"{float(np.max(err - tol)):.3e} at {np.unravel_index(np.argmax(err - tol), err.shape)}")


def _compare(inp, rows, allow_ambiguous=True, keys=None):
    a = arrays_of(inp)
    loss, dq, dw, dk = _run(inp)
    ref, tol = _reference(a, rows, allow_ambiguous)
    r = np.array(rows)
    _check("loss", loss[r], ref["loss"][r], tol["loss"][r])
    _check("dw", dw[r], ref["dw"][r], tol["dw"][r])
    _check("dq", dq[r], ref["dq"][r], tol["dq"][r])
    if keys is None:
        _check("dk", dk, ref["dk"][:, : dk.shape[1]], tol["dk"][:, : dk.shape[1]])
    else:
        for b, s_lo, s_hi in keys:
            _check(f"dk[{b}, {s_lo}:{s_hi}]", dk[b, s_lo:s_hi], ref["dk"][b, s_lo:s_hi], tol["dk"][b, s_lo:s_hi])
    assert np.all(np.isfinite(loss[r])) and np.all(loss[r] >= -1e-6)
    return loss, dq, dw, dk


def test_small_prefill_all_rows():
    wl = workloads.SMALL_WARMUP
    announce("warm-up", wl.name)
    inp = workloads.generate(wl, DEV)
    _compare(inp, list(range(inp.num_rows)))


def test_integer_indexer_is_exact_on_the_relu_mask():
    wl = workloads.INT_WARMUP
    announce("warm-up", wl.name)
    inp = workloads.generate(wl, DEV)
    a = arrays_of(inp)
    # the integer draws do put some z exactly on the kink
    z0 = 0
    for t in range(0, inp.num_rows, 17):
        z = oracle.decode_e4m3fn(a["q8"][t]) @ oracle.decode_e4m3fn(a["k8"][0, : t + 1]).T
        z0 += int((z == 0).sum())
    assert z0 > 0
    _compare(inp, list(range(inp.num_rows)), allow_ambiguous=False)


def _ragged(inp, lens, nqs):
    """Two sequences of different lengths whose query rows are their last nq tokens."""
    L = inp.wl.seq_len
    rows = []
    for b, (Lb, nq) in enumerate(zip(lens, nqs)):
        rows.extend(b * L + Lb - nq + i for i in range(nq))
    idx = torch.tensor(rows, device=inp.q.device)
    q_start = [0, nqs[0], nqs[0] + nqs[1]]
    i32 = dict(dtype=torch.int32, device=inp.q.device)
    return workloads.Inputs(
        wl=inp.wl, device=inp.device, seq_lens=torch.tensor(lens, **i32), q_start=torch.tensor(q_start, **i32),
        block_table=None, num_rows=len(rows), max_q=max(nqs), max_len=L, seq_lens_host=list(lens),
        q_start_host=q_start, q8=inp.q8[idx].contiguous(), q_scale=inp.q_scale[idx].contiguous(),
        w=inp.w[idx].contiguous(), k8=inp.k8, k_scale=inp.k_scale, q=inp.q[idx].contiguous(), kv=inp.kv, v=None)


def test_ragged_batch_of_last_rows():
    wl = workloads.RAGGED_WARMUP
    announce("warm-up", wl.name, "lens (260, 190), rows (70, 190)")
    inp = _ragged(workloads.generate(wl, DEV), [260, 190], [70, 190])
    loss, dq, dw, dk = _compare(inp, list(range(inp.num_rows)))
    # tokens no row can see (past the second sequence's length) get exactly zero
    assert np.all(dk[1, 190:] == 0)


def test_other_head_counts():
    """H_I = 32 (one head pair per dk wave, two-wave dq workgroups) and H = 64 dense heads (four waves)."""
    wl = workloads.SHAPES_WARMUP
    announce("warm-up", wl.name)
    inp = workloads.generate(wl, DEV)
    _compare(inp, list(range(inp.num_rows)))


def test_odd_row_counts_and_one_wave():
    """An odd number of rows (the last one has no partner) with H = 16 (one wave per workgroup),
    and a ragged pair of sequences with odd row counts."""
    wl = workloads.ONEWAVE_WARMUP
    announce("warm-up", wl.name)
    inp = workloads.generate(wl, DEV)
    _compare(inp, list(range(inp.num_rows)))
    wl = workloads.RAGGED_WARMUP
    announce("warm-up", wl.name, "lens (260, 191), rows (71, 191)")
    inp = _ragged(workloads.generate(wl, DEV), [260, 191], [71, 191])
    _compare(inp, list(range(inp.num_rows)))


def test_deterministic_and_forward_only():
    wl = workloads.SMALL_WARMUP
    announce("warm-up determinism", wl.name)
    inp = workloads.generate(wl, DEV)
    r1 = _run(inp)
    r2 = _run(inp)
    for x, y in zip(r1, r2):
        assert np.array_equal(x, y)
    loss_only, dq, dw, dk = _run(inp, grads=False)
    assert dq is None and dw is None and dk is None
    assert np.array_equal(loss_only, r1[0])


def test_full_size_sampled_rows():
    """4096-token sequence, every token a query row: sampled rows and the last 16 keys' gradients."""
    wl = workloads.WARMUP_4K
    announce("warm-up", wl.name, "sampled")
    inp = workloads.generate(wl, DEV)
    T = inp.num_rows
    sample = workloads.sample_rows(wl, T, wl.sample_rows, always=(0, 1, 63, 64, 2047, T - 1))
    tail = list(range(T - 16, T))                # every row that sees the last 16 keys
    rows = sorted(set(sample) | set(tail))
    _compare(inp, rows, keys=[(0, T - 16, T)])
