"""The whole oracle path against scalar-loop brute force on sequences of L <= 64 (CPU only).

Every query row of a causal prefill runs through ``oracle.run_rows`` (indexer,
top-k, sparse attention) and is compared with plain Python loops that share
nothing with the oracle:
  * FP8 and bf16 values come from torch's own dtype casts;
  * indexer scores are Python integers (integer workloads) or a correctly
    rounded ``math.fsum`` of the exact e4m3fn products times the scales;
  * the selection is the pairwise rank rule: token s is kept iff fewer than k
    tokens beat it in the order (score desc, index asc);
  * attention is a scalar loop over the kept tokens with ``math.exp``.
Shapes follow the tiny causal prefill (4 indexer heads of 32 FP8 dims, 8
attention heads of 64 dims with a separate V cache), with k below L so the
selection is not the identity, and k above L, where it is.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.oracle_io import arrays_of


def _fp8_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _brute_scores(a, t, n, integer):
    q = _fp8_values(a["q8"][t])                 # [H_I, d_I]
    k = _fp8_values(a["k8"][0, :n])             # [n, d_I]
    H_I, d_I = q.shape
    out = []
    for s in range(n):
        if integer:
            tot = 0
            for j in range(H_I):
                z = sum(int(q[j, d]) * int(k[s, d]) for d in range(d_I))
                tot += int(a["w"][t, j]) * max(z, 0)
            out.append(float(tot))
        else:
            qs = float(a["q_scale"][t])
            ks = float(a["k_scale"][0, s])
            terms = []
            for j in range(H_I):
                z = math.fsum(float(q[j, d]) * float(k[s, d]) for d in range(d_I))   # exact products
                if z > 0:
                    terms.append(float(a["w"][t, j]) * qs * ks * z)
            out.append(math.fsum(terms))
    return out


def _brute_select(scores, k):
    n = len(scores)
    kept = [s for s in range(n)
            if sum(1 for u in range(n) if scores[u] > scores[s] or (scores[u] == scores[s] and u < s)) < k]
    return kept + [-1] * (k - len(kept))


def _brute_attention(a, t, kept, scale):
    q = _bf16_values(a["q"][t])                 # [H, D]
    K = _bf16_values(a["kv"][0])
    V = _bf16_values(a["v"][0])
    H, D = q.shape
    Dv = V.shape[1]
    out = np.zeros((H, Dv))
    lse = np.zeros(H)
    for h in range(H):
        logits = [scale * math.fsum(q[h, d] * K[s, d] for d in range(D)) for s in kept]
        m = max(logits)
        e = [math.exp(x - m) for x in logits]
        den = math.fsum(e)
        lse[h] = m + math.log(den)
        for d in range(Dv):
            out[h, d] = math.fsum(e[i] * V[s, d] for i, s in enumerate(kept)) / den
    return out, lse


@pytest.mark.parametrize("L,k,integer", [(48, 16, True), (48, 64, True), (40, 8, False), (64, 24, False)],
                         ids=["int_L48_k16", "int_L48_k64", "fp8_L40_k8", "fp8_L64_k24"])
def test_whole_path_matches_bruteforce(L, k, integer):
    wl = W.TINY_PREFILL.replace(name=f"bruteforce_L{L}_k{k}", seq_len=L, k=k, integer_indexer=integer,
                                fp32_attention_inputs=False, seed=70 + L + k)
    inp = W.generate(wl, "cpu")
    a = arrays_of(inp)
    res = oracle.run_rows(a, list(range(L)), select_dtype=None)
    for t in range(L):
        n = t + 1
        ref = _brute_scores(a, t, n, integer)
        got = res["scores"][t]
        if integer:
            assert got.tolist() == ref, f"row {t}: scores"
        else:
            assert np.allclose(got, ref, rtol=1e-13, atol=1e-300), f"row {t}: scores"
        kept = _brute_select(ref, k)
        assert res["idx"][t].tolist() == kept, f"row {t}: selection"
        o, l = _brute_attention(a, t, [s for s in kept if s >= 0], wl.scale)
        assert np.allclose(res["out"][t], o, rtol=1e-12, atol=1e-12), f"row {t}: attention output"
        assert np.allclose(res["lse"][t], l, rtol=1e-12, atol=1e-12), f"row {t}: lse"
        if k >= n:
            assert kept[:n] == list(range(n))
