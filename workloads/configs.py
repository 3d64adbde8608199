"""The five synthetic workloads of the DSA hot path, plus small parity variants.

Each workload fixes the shapes and value distributions of the lightning indexer
(H_I heads of d_I FP8 dims), the top-k budget k, and the MQA core attention
(H query heads sharing one latent KV row of D dims, of which the first D_v are
the value).  The pages describe DSA on a 128K context with k = 2048 selected
tokens per query (ouchyi post, DSA paragraph; tenelement article, section
"Architektura DeepSeek V3.2-Exp: Od MoE do DSA"); every workload below is
synthetic and only stands in for that setting.

This module holds no arithmetic of the method: it only names sizes and seeds.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" | "decode" | "chunked_prefill"
    seqs: int            # sequences in the batch
    seq_len: int         # context length (max for mixed-length decode)
    H_I: int             # indexer heads
    d_I: int             # indexer head dim (FP8 bytes per key)
    k: int               # top-k budget
    H: int               # attention query heads
    D: int               # attention q/k dim (latent + rope)
    D_v: int             # value dim
    seed: int
    integer_indexer: bool = False   # q8/k8 integers in [-3,3], w integers in [-2,2], unit scales
    separate_v: bool = False        # V is its own cache (else the first D_v dims of the KV row)
    fp32_attention_inputs: bool = False  # q/k/v drawn in fp32 (rounded to bf16 for the kernels)
    min_len: int = 0                # mixed decode: lengths log-uniform in [min_len, seq_len]
    paged: bool = False
    block_size: int = 64
    chunk: int = 0                  # chunked prefill: query rows per chunk
    sample_rows: int = 0            # rows the oracle verifies (0 = all)

    @property
    def scale(self) -> float:
        return 1.0 / float(self.D) ** 0.5

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_BIG = dict(H_I=64, d_I=128, k=2048, H=128, D=576, D_v=512)

TINY_PREFILL = Workload(
    name="tiny_prefill_L256", kind="prefill", seqs=1, seq_len=256,
    H_I=4, d_I=32, k=64, H=8, D=64, D_v=64, seed=0,
    integer_indexer=True, separate_v=True, fp32_attention_inputs=True)

DECODE_128K = Workload(
    name="decode_b32_ctx128k", kind="decode", seqs=32, seq_len=131072, seed=1, **_BIG)

PREFILL_32K = Workload(
    name="prefill_L32k", kind="prefill", seqs=1, seq_len=32768, seed=2,
    sample_rows=512, **_BIG)

CHUNKED_128K = Workload(
    name="chunked_prefill_L128k_c4k", kind="chunked_prefill", seqs=1, seq_len=131072,
    chunk=4096, seed=3, sample_rows=256, **_BIG)

PAGED_DECODE_MIXED = Workload(
    name="paged_decode_b128_mixed4k_128k", kind="decode", seqs=128, seq_len=131072,
    min_len=4096, paged=True, block_size=64, seed=4, **_BIG)

ALL = [TINY_PREFILL, DECODE_128K, PREFILL_32K, CHUNKED_128K, PAGED_DECODE_MIXED]
BY_NAME = {w.name: w for w in ALL}

# Reduced-size variants with the production head shapes, small enough for the
# oracle to check every row in seconds while still spanning several key tiles,
# several top-k slices and a ragged tail.
SMALL_DECODE = DECODE_128K.replace(name="decode_b3_ctx5000", seqs=3, seq_len=5000, seed=11)
SMALL_PAGED = PAGED_DECODE_MIXED.replace(
    name="paged_decode_b5_mixed100_6000", seqs=5, seq_len=6000, min_len=100, seed=14)
SMALL_PREFILL = PREFILL_32K.replace(name="prefill_L2500", seq_len=2500, seed=12, sample_rows=0)
SMALL_CHUNKED = CHUNKED_128K.replace(
    name="chunked_prefill_L3000_c1000", seq_len=3000, chunk=1000, seed=13, sample_rows=0)

# Short contexts (every row sees at most k tokens): the selection is every
# prior token and the fused entry points skip the indexer.
DENSE_PREFILL = PREFILL_32K.replace(name="prefill_L1500_dense", seq_len=1500, seed=15, sample_rows=0)
DENSE_DECODE = DECODE_128K.replace(name="decode_b4_ctx2048_dense", seqs=4, seq_len=2048, seed=16)

# Indexer warm-up objective (KL of the head-averaged dense attention against the
# indexer softmax, forward and backward): every token of one sequence is a
# query row, as in training.
WARMUP_4K = PREFILL_32K.replace(name="warmup_L4k", seq_len=4096, seed=17, sample_rows=32)
SMALL_WARMUP = PREFILL_32K.replace(name="warmup_L300", seq_len=300, seed=18, sample_rows=0)
INT_WARMUP = PREFILL_32K.replace(name="warmup_L200_int", seq_len=200, seed=19, sample_rows=0,
                                 integer_indexer=True)
RAGGED_WARMUP = PREFILL_32K.replace(name="warmup_b2_L260", seqs=2, seq_len=260, seed=20, sample_rows=0)

# the warm-up objective's measured workload is selectable by name as well
BY_NAME[WARMUP_4K.name] = WARMUP_4K
SHAPES_WARMUP = PREFILL_32K.replace(name="warmup_L230_hi32_h64", seq_len=230, seed=21, sample_rows=0,
                                    H_I=32, H=64)
ONEWAVE_WARMUP = PREFILL_32K.replace(name="warmup_L151_h16", seq_len=151, seed=22, sample_rows=0, H=16)
