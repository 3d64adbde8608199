"""Seeded synthetic inputs for the DSA hot path.

The tensors are the only thing the HIP path and the CPU oracle share: both
consume exactly these bytes.  Nothing here computes any part of the method;
it draws random numbers, rounds them to the storage formats (OCP e4m3fn for
the indexer, bf16 for attention) and lays them out in memory.

Recipe (per workload, see ``workloads.configs``):

* indexer q/k ~ N(0,1), quantised to e4m3fn with one fp32 scale per token
  (scale = amax/448, the value divided by it, clamped to +-448 and rounded by
  torch's fp32 -> float8_e4m3fn cast); head weights w ~ N(0, 1/64) in fp32.
  Integer workloads instead draw q8/k8 uniformly from the integers [-3,3]
  (exact in e4m3fn), w from the integers [-2,2], and use unit scales.
* attention q and the latent KV rows ~ N(0,1) in bf16 (fp32 draws rounded to
  bf16 when the workload asks for fp32 originals, which are kept alongside).
* decode: one query per sequence at position len-1 (the query token is the
  last cached token); prefill: every position of the sequence is a query row;
  chunked prefill: chunk c holds query rows [c*chunk, (c+1)*chunk) against a
  cache of (c+1)*chunk tokens.
* paged caches: lengths floor(exp(U[ln min_len, ln seq_len])), a pool of
  exactly sum(ceil(len/64)) blocks and a seeded random permutation of the
  pool's block ids as the block table (-1 for unused table entries).

Every tensor is drawn from its own torch generator, seeded from the workload
seed and the tensor's name, so any tensor can be regenerated on its own.
On a GPU device the draws happen on that device (fast at 128K contexts); a
CPU device gives different, equally valid values.
"""
from __future__ import annotations

import dataclasses
import math
import zlib
from dataclasses import dataclass
from typing import Optional

import torch

from .configs import Workload

E4M3_MAX = 448.0


def _gen(device, seed: int, name: str, extra: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + zlib.crc32(name.encode()) * 7919 + extra) % (2**63 - 1))
    return g


def quantize_e4m3fn(x: torch.Tensor, token_dims: int):
    """Per-token e4m3fn quantisation of ``x``; the last ``token_dims`` dims form one token.

    Returns (uint8 codes, fp32 scale per token).  This is input preparation:
    both sides of every comparison consume the returned bytes and scales.
    """
    red = tuple(range(x.dim() - token_dims, x.dim()))
    amax = x.abs().amax(dim=red)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).float()
    shaped = scale.reshape(scale.shape + (1,) * token_dims)
    # clamp first: torch's cast maps out-of-range values to NaN instead of saturating
    codes = (x / shaped).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def _int_e4m3fn(shape, g, device, lo, hi):
    v = torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int32)
    return v.float().to(torch.float8_e4m3fn).view(torch.uint8)


@dataclass
class Inputs:
    wl: Workload
    device: torch.device
    # geometry
    seq_lens: torch.Tensor           # [B] int32
    q_start: Optional[torch.Tensor]  # [B+1] int32, None = one query per sequence (decode)
    block_table: Optional[torch.Tensor]  # [B, max_blocks] int32 or None
    num_rows: int
    max_q: int
    max_len: int
    seq_lens_host: list
    q_start_host: Optional[list]
    # indexer
    q8: torch.Tensor                 # [T, H_I, d_I] uint8 (e4m3fn)
    q_scale: Optional[torch.Tensor]  # [T] fp32 or None (= 1)
    w: torch.Tensor                  # [T, H_I] fp32
    k8: torch.Tensor                 # [B, cap, d_I] or [blocks, bs, d_I] uint8
    k_scale: Optional[torch.Tensor]  # [B, cap] or [blocks, bs] fp32 or None (= 1)
    # attention
    q: torch.Tensor                  # [T, H, D] bf16
    kv: torch.Tensor                 # [B, cap, D] or [blocks, bs, D] bf16
    v: Optional[torch.Tensor]        # separate V cache [.., D_v] bf16, None = kv[..., :D_v]
    q_f32: Optional[torch.Tensor] = None
    kv_f32: Optional[torch.Tensor] = None
    v_f32: Optional[torch.Tensor] = None
    chunk_index: int = 0

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    def to(self, device) -> "Inputs":
        """A copy with every tensor moved to ``device``."""
        moved = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            moved[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        moved["device"] = torch.device(device)
        return Inputs(**moved)

    def row_positions(self):
        """(sequence, position) of every query row, host lists."""
        seqs, poss = [], []
        if self.q_start_host is None:
            for b, L in enumerate(self.seq_lens_host):
                seqs.append(b)
                poss.append(L - 1)
        else:
            for b, L in enumerate(self.seq_lens_host):
                nq = self.q_start_host[b + 1] - self.q_start_host[b]
                for i in range(nq):
                    seqs.append(b)
                    poss.append(L - nq + i)
        return seqs, poss


def decode_lengths(wl: Workload) -> list:
    if wl.min_len <= 0:
        return [wl.seq_len] * wl.seqs
    g = _gen("cpu", wl.seed, "lengths")
    u = torch.rand(wl.seqs, generator=g, dtype=torch.float64)
    lo, hi = math.log(wl.min_len), math.log(wl.seq_len)
    lens = torch.floor(torch.exp(lo + u * (hi - lo))).long().clamp(wl.min_len, wl.seq_len)
    return [int(x) for x in lens]


def _block_table(wl: Workload, lens: list):
    bs = wl.block_size
    nblk = [(L + bs - 1) // bs for L in lens]
    total = sum(nblk)
    g = _gen("cpu", wl.seed, "block_perm")
    perm = torch.randperm(total, generator=g).int()
    max_blocks = max(nblk)
    table = torch.full((len(lens), max_blocks), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, total


def _cache_shape(wl: Workload, lens: list, table_total: int):
    if wl.paged:
        return (table_total, wl.block_size)
    return (wl.seqs, max(lens))


def generate(wl: Workload, device="cpu", chunk_index: int = 0, with_cache: bool = True,
             cache: Optional[dict] = None) -> Inputs:
    """Build the inputs of ``wl`` on ``device``.

    For chunked prefill ``chunk_index`` selects the chunk; the cache (all
    seq_len tokens) is the same for every chunk and may be passed in via
    ``cache`` (a dict returned in a previous Inputs) to avoid redrawing it.
    """
    device = torch.device(device)
    dev = device.type if device.type == "cpu" else device
    s = wl.seed

    # ---- geometry -------------------------------------------------------
    if wl.kind == "decode":
        lens = decode_lengths(wl)
        q_start_host = None
        T = wl.seqs
        max_q = 1
    elif wl.kind == "prefill":
        lens = [wl.seq_len] * wl.seqs
        q_start_host = [i * wl.seq_len for i in range(wl.seqs + 1)]
        T = wl.seqs * wl.seq_len
        max_q = wl.seq_len
    elif wl.kind == "chunked_prefill":
        assert wl.seqs == 1
        nchunks = (wl.seq_len + wl.chunk - 1) // wl.chunk
        assert 0 <= chunk_index < nchunks
        end = min((chunk_index + 1) * wl.chunk, wl.seq_len)
        nq = end - chunk_index * wl.chunk
        lens = [end]
        q_start_host = [0, nq]
        T = nq
        max_q = nq
    else:
        raise ValueError(wl.kind)

    table = None
    total_blocks = 0
    if wl.paged:
        table, total_blocks = _block_table(wl, lens)
    cache_lens = [wl.seq_len] if wl.kind == "chunked_prefill" else lens
    cshape = _cache_shape(wl, cache_lens, total_blocks)

    # ---- query-side tensors (depend on the chunk) -------------------------
    qx = chunk_index
    if wl.integer_indexer:
        q8 = _int_e4m3fn((T, wl.H_I, wl.d_I), _gen(dev, s, "q8", qx), device, -3, 3)
        q_scale = None
        w = torch.randint(-2, 3, (T, wl.H_I), generator=_gen(dev, s, "w", qx), device=device,
                          dtype=torch.int32).float()
    else:
        qf = torch.randn((T, wl.H_I, wl.d_I), generator=_gen(dev, s, "q_idx", qx), device=device)
        q8, q_scale = quantize_e4m3fn(qf, 2)
        del qf
        w = torch.randn((T, wl.H_I), generator=_gen(dev, s, "w", qx), device=device) * (1.0 / 8.0)

    q_f32 = None
    if wl.fp32_attention_inputs:
        q_f32 = torch.randn((T, wl.H, wl.D), generator=_gen(dev, s, "q", qx), device=device)
        q = q_f32.to(torch.bfloat16)
    else:
        q = torch.randn((T, wl.H, wl.D), generator=_gen(dev, s, "q", qx), device=device,
                        dtype=torch.bfloat16)

    # ---- caches ---------------------------------------------------------
    if cache is not None:
        k8, k_scale, kv, v = cache["k8"], cache["k_scale"], cache["kv"], cache["v"]
        kv_f32, v_f32 = cache.get("kv_f32"), cache.get("v_f32")
    elif with_cache:
        if wl.integer_indexer:
            k8 = _int_e4m3fn(cshape + (wl.d_I,), _gen(dev, s, "k8"), device, -3, 3)
            k_scale = None
        else:
            kf = torch.randn(cshape + (wl.d_I,), generator=_gen(dev, s, "k_idx"), device=device)
            k8, k_scale = quantize_e4m3fn(kf, 1)
            del kf
        kv_f32 = v_f32 = None
        if wl.fp32_attention_inputs:
            kv_f32 = torch.randn(cshape + (wl.D,), generator=_gen(dev, s, "kv"), device=device)
            kv = kv_f32.to(torch.bfloat16)
        else:
            kv = torch.randn(cshape + (wl.D,), generator=_gen(dev, s, "kv"), device=device,
                             dtype=torch.bfloat16)
        v = None
        if wl.separate_v:
            if wl.fp32_attention_inputs:
                v_f32 = torch.randn(cshape + (wl.D_v,), generator=_gen(dev, s, "v"), device=device)
                v = v_f32.to(torch.bfloat16)
            else:
                v = torch.randn(cshape + (wl.D_v,), generator=_gen(dev, s, "v"), device=device,
                                dtype=torch.bfloat16)
    else:
        k8 = k_scale = kv = v = kv_f32 = v_f32 = None

    i32 = dict(dtype=torch.int32, device=device)
    return Inputs(
        wl=wl, device=device,
        seq_lens=torch.tensor(lens, **i32),
        q_start=None if q_start_host is None else torch.tensor(q_start_host, **i32),
        block_table=None if table is None else table.to(device),
        num_rows=T, max_q=max_q, max_len=max(lens),
        seq_lens_host=list(lens), q_start_host=q_start_host,
        q8=q8, q_scale=q_scale, w=w, k8=k8, k_scale=k_scale,
        q=q, kv=kv, v=v, q_f32=q_f32, kv_f32=kv_f32, v_f32=v_f32,
        chunk_index=chunk_index)


def cache_of(inp: Inputs) -> dict:
    return dict(k8=inp.k8, k_scale=inp.k_scale, kv=inp.kv, v=inp.v,
                kv_f32=inp.kv_f32, v_f32=inp.v_f32)


def sample_rows(wl: Workload, num_rows: int, count: int, always=()) -> list:
    """Seeded sample of ``count`` query rows (without replacement), always including ``always``."""
    if count <= 0 or count >= num_rows:
        return list(range(num_rows))
    keep = sorted({r for r in always if 0 <= r < num_rows})
    g = _gen("cpu", wl.seed, "sample_rows", num_rows)
    perm = torch.randperm(num_rows, generator=g).tolist()
    out = list(keep)
    seen = set(keep)
    for r in perm:
        if len(out) >= count:
            break
        if r not in seen:
            out.append(r)
            seen.add(r)
    return sorted(out)


def synthetic_scores(rows: int, ld: int, kind: str, seed: int = 0, device="cpu") -> torch.Tensor:
    """Seeded fp32 score matrices [rows, ld] that stress the top-k selection.

    normal: N(0,1); ties: integers in [-3,3]; signed_zeros: +0.0 / -0.0 with a
    few +-1; all_equal: every score 0.5; sparse_ones: zeros with about 1000
    ones per row (the boundary is a huge run of equal zeros).
    """
    dev = torch.device(device)
    gd = dev.type if dev.type == "cpu" else dev
    g = _gen(gd, seed, "scores_" + kind, rows * 7 + ld)
    if kind == "normal":
        return torch.randn((rows, ld), generator=g, device=dev)
    if kind == "ties":
        return torch.randint(-3, 4, (rows, ld), generator=g, device=dev).float()
    if kind == "signed_zeros":
        v = torch.randint(0, 16, (rows, ld), generator=g, device=dev)
        out = torch.zeros((rows, ld), device=dev)
        out = torch.where(v < 7, torch.full_like(out, -0.0), out)
        out = torch.where(v == 14, torch.ones_like(out), out)
        out = torch.where(v == 15, -torch.ones_like(out), out)
        return out
    if kind == "all_equal":
        return torch.full((rows, ld), 0.5, device=dev)
    if kind == "sparse_ones":
        return (torch.rand((rows, ld), generator=g, device=dev) < (1000.0 / ld)).float()
    raise ValueError(kind)
