"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

Holds shapes, seeds and random draws only; no part of the method is computed here.
"""
from .configs import (ALL, BY_NAME, CHUNKED_128K, DECODE_128K, DENSE_DECODE, DENSE_PREFILL,  # noqa: F401
                      PAGED_DECODE_MIXED, PREFILL_32K, SMALL_CHUNKED, SMALL_DECODE, SMALL_PAGED,
                      SMALL_PREFILL, TINY_PREFILL, Workload, WARMUP_4K, SMALL_WARMUP, INT_WARMUP,
                      RAGGED_WARMUP, SHAPES_WARMUP, ONEWAVE_WARMUP)
from .gen import Inputs, cache_of, generate, quantize_e4m3fn, sample_rows, synthetic_scores  # noqa: F401
