"""Plain, slow CPU oracle of the DeepSeek Sparse Attention (DSA) hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its binding) never touches it, and it shares
no code, table or constant with that path.

What it computes, in the order the pages give it:

1. Lightning indexer.  A light scorer with a few heads, run on FP8 operands,
   scores every cached token for each query; it uses a ReLU (ouchyi.pink post
   on DSA, the DSA paragraph; tenelement.pl article "DeepSeek V3.2-Exp Cuts
   Long-Context Costs with DeepSeek Sparse Attention (DSA) While Maintaining
   Benchmark Parity", section "Architektura DeepSeek V3.2-Exp: Od MoE do DSA").
   The score of cached token s for query t is
       I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s])
   where the FP8 operands carry one fp32 scale per token, so
       I[t,s] = k_scale[s] * sum_j w[t,j] * q_scale[t] * ReLU(q8[t,j] . k8[s]).
2. Top-k selection of k key/value entries per query (k = 2048 on the pages,
   whatever the context length; same two sources, and the digitalreport.com.tr
   article "DeepSeek V3.2-exp: daha ucuz uzun bağlamlı AI" calls it a
   fine-grained token selection).  Order: score descending, then token index
   ascending; -0.0 ties +0.0.  The chosen indices are returned in ascending
   order and padded with -1 up to k.
3. Core attention over only the selected entries, in MQA form: all query heads
   read the same latent KV row (tenelement.pl article, same section: MQA in
   decode; degnora.com "DeepSeekV3, Farkı Ne?", section "MLA — Multi-Latent
   Attention": one shared latent row per token).  K is the whole row, V its
   first D_v dims (or a separate V cache when given).  Softmax runs over the
   selected set only.

Causality: query row at position p sees tokens 0..p (itself included).

All arithmetic is float64.  Where the fp32 kernels take a discrete decision
(the top-k), ``run_rows`` takes it on the fp64 scores rounded to fp32, the
precision the kernels decide in; ``select_dtype`` can switch that off.

Parity status: every function here is pinned by tests under tests/ (decode
tables against torch's dtype casts, brute force on tiny inputs, the dense
causal attention identity for k >= n, closed forms and invariants).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# Storage formats
# --------------------------------------------------------------------------


def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 e4m3fn byte: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    No infinities; S.1111.111 is NaN; exponent 0 is subnormal (2^-6 * m/8).
    The pages say the indexer runs in FP8 (ouchyi.pink post, DSA paragraph).
    """
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3 = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the high half of an IEEE fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):     # signalling-NaN patterns widen quietly
        return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Cache addressing
# --------------------------------------------------------------------------


def token_rows(cache: np.ndarray, seq: int, n: int, block_table=None, block_size: int = 0):
    """Rows of tokens 0..n-1 of sequence ``seq`` in logical order.

    Contiguous caches are indexed [seq, token, ...].  Paged caches are a pool
    [block, slot, ...]: token s of sequence b sits in pool block
    block_table[b, s // block_size] at slot s % block_size.
    """
    if block_table is None:
        return cache[seq, :n]
    s = np.arange(n)
    blocks = np.asarray(block_table)[seq, s // block_size]
    if n and blocks.min() < 0:
        raise ValueError("block table entry -1 inside the sequence")
    return cache[blocks, s % block_size]


# --------------------------------------------------------------------------
# 1. Lightning indexer
# --------------------------------------------------------------------------


def indexer_scores(q8: np.ndarray, q_scale: float, w: np.ndarray, k8: np.ndarray,
                   k_scale, with_abs: bool = False):
    """Scores of n cached tokens for one query row.

    q8 [H_I, d_I] e4m3fn codes, q_scale scalar (None = 1), w [H_I] head weights,
    k8 [n, d_I] e4m3fn codes, k_scale [n] (None = 1).  Returns float64 [n]:
        I[s] = sum_j w[j] * q_scale * k_scale[s] * max(sum_d q[j,d] k[s,d], 0)
    The fp64 dot products are exact: each e4m3fn product is a multiple of
    2^-18 below 2^18, so a 128-term sum needs fewer than 53 bits.
    With ``with_abs`` also returns the absolute-term sum of every score,
        A[s] = sum_j |w[j] * q_scale| * k_scale[s] * max(z[j,s], 0),
    the scale against which a score's rounding error is judged.
    """
    return indexer_scores_values(decode_e4m3fn(q8), q_scale, w, decode_e4m3fn(k8), k_scale, with_abs)


def indexer_scores_values(q: np.ndarray, q_scale, w: np.ndarray, k: np.ndarray, k_scale,
                          with_abs: bool = False):
    """indexer_scores on already decoded FP8 values (q [H_I, d_I], k [n, d_I] float64)."""
    z = q @ k.T                                        # [H_I, n] logits per indexer head
    relu = np.maximum(z, 0.0)
    qs = 1.0 if q_scale is None else float(q_scale)
    ks = np.ones(k.shape[0]) if k_scale is None else np.asarray(k_scale, dtype=np.float64)
    wj = np.asarray(w, dtype=np.float64) * qs          # [H_I]
    scores = (wj @ relu) * ks
    if not with_abs:
        return scores
    return scores, (np.abs(wj) @ relu) * ks


# --------------------------------------------------------------------------
# 2. Top-k selection
# --------------------------------------------------------------------------


def topk_indices(scores: np.ndarray, k: int) -> np.ndarray:
    """First min(k, n) tokens in the order (score desc, index asc); ascending, -1 padded."""
    scores = np.asarray(scores)
    n = scores.shape[0]
    out = np.full(k, -1, dtype=np.int32)
    if n <= k:
        out[:n] = np.arange(n, dtype=np.int32)
        return out
    # lexsort: last key is primary.  -score puts larger scores first; comparing
    # as real numbers makes -0.0 and +0.0 equal, so the index decides.
    order = np.lexsort((np.arange(n), -scores.astype(np.float64)))
    out[:] = np.sort(order[:k]).astype(np.int32)
    return out


# --------------------------------------------------------------------------
# 3. Sparse MQA attention
# --------------------------------------------------------------------------


def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of H heads over m shared rows.

    q [H, D], K [m, D], V [m, D_v] (float64), m >= 1.
    Returns out [H, D_v] and lse [H] (natural log of the softmax denominator
    including the max shift: lse = log sum_i exp(x_i)).
    """
    x = scale * (q @ K.T)                  # [H, m]
    mx = x.max(axis=1, keepdims=True)
    p = np.exp(x - mx)
    den = p.sum(axis=1, keepdims=True)
    out = (p @ V) / den
    lse = mx[:, 0] + np.log(den[:, 0])
    return out, lse


def dense_causal_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Textbook dense causal MQA attention over a whole sequence (reference for k >= L).

    q [L, H, D], K [L, D], V [L, D_v] -> out [L, H, D_v].
    """
    L = K.shape[0]
    x = scale * np.einsum("thd,sd->ths", q, K)
    mask = np.triu(np.ones((L, L), dtype=bool), k=1)      # s > t is in the future
    x = np.where(mask[:, None, :], -np.inf, x)
    x = x - x.max(axis=2, keepdims=True)
    p = np.exp(x)
    p = p / p.sum(axis=2, keepdims=True)
    return np.einsum("ths,sd->thd", p, V)


# --------------------------------------------------------------------------
# The whole path, row by row
# --------------------------------------------------------------------------


def row_geometry(seq_lens, q_start, num_rows: int):
    """(sequence, position) of every query row.

    q_start None: one query per sequence at position len-1 (decode).
    Otherwise the q_start[b+1]-q_start[b] rows of sequence b are its last
    tokens: row i sits at position len_b - nq_b + i.
    """
    seq_lens = [int(x) for x in seq_lens]
    if q_start is None:
        return [(b, L - 1) for b, L in enumerate(seq_lens)]
    q_start = [int(x) for x in q_start]
    out = []
    for b, L in enumerate(seq_lens):
        nq = q_start[b + 1] - q_start[b]
        out.extend((b, L - nq + i) for i in range(nq))
    assert len(out) == num_rows
    return out


def run_rows(a: dict, rows, select_dtype=np.float32, need=("scores", "idx", "out"),
             idx_override=None):
    """Run the path for the given query rows.

    ``a`` holds numpy arrays: q8 [T,H_I,d_I] u8, q_scale [T] or None, w [T,H_I],
    k8 / k_scale / kv / v caches (contiguous [B, cap, ...] or paged pools
    [blocks, block_size, ...]), q / kv / v as bf16 bits (uint16) or as floats
    (keys q_f, kv_f, v_f take precedence when present), seq_lens, q_start,
    block_table, block_size, k, scale.

    Returns a dict of per-row lists: scores (float64 [n]), idx (int32 [k]),
    out (float64 [H, D_v]), lse (float64 [H]), and with "abs" in ``need`` the
    absolute-term sums of the scores (see indexer_scores).  ``idx_override`` maps a row to
    an index set to attend over instead of the oracle's own selection.
    """
    rows = list(rows)
    geo = row_geometry(a["seq_lens"], a.get("q_start"), a["q8"].shape[0])
    table = a.get("block_table")
    bs = int(a.get("block_size") or 0)
    k = int(a["k"])
    res = {"scores": [], "abs": [], "idx": [], "out": [], "lse": []}

    def att_rows(name, b, n, sel):
        """Rows `sel` (logical token indices) of sequence b's cache `name`, as float64."""
        if a.get(name + "_f") is not None:
            return token_rows(a[name + "_f"], b, n, table, bs)[sel].astype(np.float64)
        if a.get(name) is None:
            return None
        return decode_bf16(token_rows(a[name], b, n, table, bs)[sel])

    keys = {}                     # sequence -> decoded index keys of its longest requested prefix

    def key_values(b, n):
        if b not in keys or keys[b].shape[0] < n:
            longest = max(p + 1 for (bb, p) in (geo[r] for r in rows) if bb == b)
            keys[b] = decode_e4m3fn(token_rows(a["k8"], b, longest, table, bs))
        return keys[b][:n]

    for t in rows:
        b, p = geo[t]
        n = p + 1
        ks = None if a.get("k_scale") is None else token_rows(a["k_scale"], b, n, table, bs)
        qs = None if a.get("q_scale") is None else a["q_scale"][t]
        sc = indexer_scores_values(decode_e4m3fn(a["q8"][t]), qs, a["w"][t], key_values(b, n), ks,
                                   with_abs="abs" in need)
        if "abs" in need:
            sc, ab = sc
            res["abs"].append(ab)
        res["scores"].append(sc)
        sel_scores = sc.astype(select_dtype) if select_dtype is not None else sc
        idx = topk_indices(sel_scores, k)
        res["idx"].append(idx)
        if "out" in need:
            use = idx if idx_override is None or t not in idx_override else idx_override[t]
            sel = use[use >= 0]
            K = att_rows("kv", b, n, sel)
            V = att_rows("v", b, n, sel)
            V = K[:, : int(a["D_v"])] if V is None else V
            if a.get("q_f") is not None:
                qrow = a["q_f"][t].astype(np.float64)
            else:
                qrow = decode_bf16(a["q"][t])
            o, l = sparse_attention(qrow, K, V, float(a["scale"]))
            res["out"].append(o)
            res["lse"].append(l)
    return res
