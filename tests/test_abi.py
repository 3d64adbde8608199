"""C-ABI checks that need no GPU: the library loads, exports every call of
include/dsa.h, sizes workspaces on the host, and rejects bad arguments with
the documented status before anything reaches HIP."""
import ctypes
import os
import re

import pytest

from sparse_attention_long_06_amd import _lib
from sparse_attention_long_06_amd._lib import DsaBatch, DsaCache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_long_06_amd import build
        build.build()
    return _lib.load()


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("dsa_indexer", "dsa_topk", "dsa_sparse_attn", "dsa_decode", "dsa_prefill", "dsa_prefill_streaming",
              "dsa_indexer_warmup", "dsa_workspace_size",
              "dsa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(_lib.SIGNATURES)


FAKE = 0x10000  # never dereferenced: every case below fails validation first


def _batch(**kw):
    d = dict(num_seqs=2, num_rows=2, max_q=1, max_len=1000, seq_lens=FAKE, q_start=None,
             block_table=None, max_blocks=0, block_size=0)
    d.update(kw)
    return DsaBatch(**d)


def _cache(row, seq=1000, data=FAKE):
    return DsaCache(data, row, seq)


def _indexer(lib, b, H_I=64, d_I=128, kidx=None, scores=FAKE, ld=1000, q8=FAKE, w=FAKE):
    kidx = kidx if kidx is not None else _cache(128)
    return lib.dsa_indexer(ctypes.byref(b) if b is not None else None, q8, None, w, ctypes.byref(kidx), None,
                           H_I, d_I, scores, ld, None)


def _err(lib):
    return lib.dsa_last_error().decode()


def test_indexer_validation(lib):
    assert _indexer(lib, None) == _lib.DSA_ERR_NULL
    assert "batch" in _err(lib)
    assert _indexer(lib, _batch(num_seqs=0)) == _lib.DSA_ERR_SHAPE
    assert _indexer(lib, _batch(num_rows=3)) == _lib.DSA_ERR_SHAPE         # decode: rows must equal seqs
    assert _indexer(lib, _batch(seq_lens=None)) == _lib.DSA_ERR_NULL
    assert _indexer(lib, _batch(), H_I=65) == _lib.DSA_ERR_UNSUPPORTED
    assert _indexer(lib, _batch(), H_I=6) == _lib.DSA_ERR_UNSUPPORTED
    assert _indexer(lib, _batch(), d_I=64) == _lib.DSA_ERR_UNSUPPORTED
    assert _indexer(lib, _batch(), q8=None) == _lib.DSA_ERR_NULL
    assert _indexer(lib, _batch(), scores=None) == _lib.DSA_ERR_NULL
    assert _indexer(lib, _batch(), ld=999) == _lib.DSA_ERR_SHAPE
    assert _indexer(lib, _batch(), kidx=_cache(100)) == _lib.DSA_ERR_SHAPE  # row shorter than d_I
    assert _indexer(lib, _batch(), kidx=_cache(136)) == _lib.DSA_ERR_ALIGN  # stride not 16-aligned
    assert _indexer(lib, _batch(), kidx=_cache(128, data=FAKE + 8)) == _lib.DSA_ERR_ALIGN
    assert _indexer(lib, _batch(), kidx=_cache(128, seq=999)) == _lib.DSA_ERR_SHAPE
    assert _indexer(lib, _batch(block_table=FAKE, max_blocks=4, block_size=48)) == _lib.DSA_ERR_SHAPE
    assert _indexer(lib, _batch(block_table=FAKE, max_blocks=4, block_size=64)) == _lib.DSA_ERR_SHAPE  # 256 < 1000


def test_topk_validation(lib):
    b = _batch()
    f = lambda k=2048, ld=1000, scores=FAKE, ws=None, n=0: lib.dsa_topk(ctypes.byref(b), scores, ld, k, FAKE, ws, n, None)
    assert f(k=0) == _lib.DSA_ERR_UNSUPPORTED
    assert f(k=4097) == _lib.DSA_ERR_UNSUPPORTED
    assert f(scores=None) == _lib.DSA_ERR_NULL
    assert f(ld=996) == _lib.DSA_ERR_SHAPE
    assert f(ld=1002) == _lib.DSA_ERR_ALIGN
    # max_len 1000 <= k: no workspace is needed, so the next failure would be HIP itself; use k < max_len
    need = lib.dsa_workspace_size(_lib.DSA_WS_TOPK, ctypes.byref(b), 64, 0, 0)
    assert need > 0
    assert f(k=64, ws=None, n=0) == _lib.DSA_ERR_WORKSPACE
    assert f(k=64, ws=FAKE, n=need - 1) == _lib.DSA_ERR_WORKSPACE
    assert f(k=64, ws=FAKE + 16, n=need) == _lib.DSA_ERR_ALIGN


def test_attention_validation(lib):
    b = _batch()
    kv = _cache(1152)

    def f(H=128, D=576, D_v=512, scale=0.04, k=2048, q=FAKE, kvc=kv, idx=FAKE, out=FAKE):
        return lib.dsa_sparse_attn(ctypes.byref(b), q, ctypes.byref(kvc), None, H, D, D_v, scale, idx, k, out,
                                   None, None, 0, None)
    assert f(D=128, D_v=128) == _lib.DSA_ERR_UNSUPPORTED
    assert f(H=129) == _lib.DSA_ERR_UNSUPPORTED
    assert f(k=5000) == _lib.DSA_ERR_UNSUPPORTED
    assert f(scale=float("nan")) == _lib.DSA_ERR_SHAPE
    assert f(q=None) == _lib.DSA_ERR_NULL
    assert f(q=FAKE + 2) == _lib.DSA_ERR_ALIGN
    assert f(kvc=_cache(1000)) == _lib.DSA_ERR_SHAPE
    assert f(idx=None) == _lib.DSA_ERR_NULL
    # 2 rows < 256: split-K partials need a workspace
    assert f() == _lib.DSA_ERR_WORKSPACE


def test_decode_validation(lib):
    kidx, kv = _cache(128), _cache(1152)

    def f(b, ws=None, n=0, k=2048):
        return lib.dsa_decode(ctypes.byref(b), FAKE, None, FAKE, ctypes.byref(kidx), None, 64, 128, k, FAKE,
                              ctypes.byref(kv), None, 128, 576, 512, 0.04, FAKE, None, None, ws, n, None)
    assert f(_batch(q_start=FAKE, num_rows=4, max_q=2)) == _lib.DSA_ERR_SHAPE
    b = _batch()
    need = lib.dsa_workspace_size(_lib.DSA_WS_DECODE, ctypes.byref(b), 2048, 128, 512)
    assert need > 2 * 1000 * 4
    assert f(b) == _lib.DSA_ERR_WORKSPACE
    assert f(b, FAKE, need - 1) == _lib.DSA_ERR_WORKSPACE


def test_stage_events_validation(lib):
    ev = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, None)
    assert lib.dsa_set_stage_events(ev, 3) == _lib.DSA_ERR_SHAPE
    assert lib.dsa_set_stage_events(ev, 4) == _lib.DSA_ERR_NULL
    assert lib.dsa_set_stage_events(None, 0) == _lib.DSA_OK


def test_indexer_fp8_switch_validation(lib):
    assert lib.dsa_set_indexer_fp8(2) == _lib.DSA_ERR_SHAPE
    assert "0 or 1" in _err(lib)
    assert lib.dsa_set_indexer_fp8(0) == _lib.DSA_OK
    assert lib.dsa_set_indexer_fp8(1) == _lib.DSA_OK


def test_prefill_validation(lib):
    kidx, kv = _cache(128, seq=4096), _cache(1152, seq=4096)

    def f(b, ws=None, n=0, k=2048):
        return lib.dsa_prefill(ctypes.byref(b), FAKE, None, FAKE, ctypes.byref(kidx), None, 64, 128, k, FAKE,
                               ctypes.byref(kv), None, 128, 576, 512, 0.04, FAKE, None, None, ws, n, None)
    assert f(_batch()) == _lib.DSA_ERR_SHAPE                   # q_start NULL: a decode batch
    b = _batch(num_seqs=1, num_rows=3000, max_q=3000, max_len=3000, q_start=FAKE)
    need = lib.dsa_workspace_size(_lib.DSA_WS_PREFILL, ctypes.byref(b), 2048, 128, 512)
    assert need >= 3000 * 3000 * 4                              # the score matrix lives in the workspace
    assert f(b) == _lib.DSA_ERR_WORKSPACE
    assert f(b, FAKE, need - 1) == _lib.DSA_ERR_WORKSPACE
    assert lib.dsa_workspace_size(_lib.DSA_WS_PREFILL, ctypes.byref(_batch()), 2048, 128, 512) == ctypes.c_size_t(-1).value
    assert lib.dsa_workspace_size(_lib.DSA_WS_DECODE, ctypes.byref(b), 2048, 128, 512) == ctypes.c_size_t(-1).value


def test_prefill_streaming_validation(lib):
    kidx, kv = _cache(128, seq=131072), _cache(1152, seq=131072)

    def f(b, ws=None, n=0, k=2048, d_I=128, kidx=kidx):
        return lib.dsa_prefill_streaming(ctypes.byref(b), FAKE, None, FAKE, ctypes.byref(kidx), None, 64, d_I, k,
                                         FAKE, ctypes.byref(kv), None, 128, 576, 512, 0.04, FAKE, None, None, ws, n,
                                         None)
    assert f(_batch()) == _lib.DSA_ERR_SHAPE                   # q_start NULL: a decode batch
    b = _batch(num_seqs=1, num_rows=4096, max_q=4096, max_len=131072, q_start=FAKE)
    assert f(b, d_I=32, kidx=_cache(32, seq=131072)) == _lib.DSA_ERR_UNSUPPORTED
    assert f(b, k=4096) == _lib.DSA_ERR_UNSUPPORTED
    assert f(_batch(num_seqs=1, num_rows=8, max_q=8, max_len=262145, q_start=FAKE)) == _lib.DSA_ERR_UNSUPPORTED
    need = lib.dsa_workspace_size(_lib.DSA_WS_PREFILL_STREAM, ctypes.byref(b), 2048, 128, 512)
    dense = lib.dsa_workspace_size(_lib.DSA_WS_PREFILL, ctypes.byref(b), 2048, 128, 512)
    # no [rows, max_len] score matrix: sampled scores (max_len / 32 per row) and
    # candidate lists (56 * rank pairs per row, rank = 128 for k = 2048) instead
    assert need < dense / 4
    assert need >= 4096 * (131072 // 32) * 4 + 4096 * 56 * 128 * 8
    assert f(b) == _lib.DSA_ERR_WORKSPACE
    assert f(b, FAKE, need - 1) == _lib.DSA_ERR_WORKSPACE
    assert f(b, FAKE + 16, need) == _lib.DSA_ERR_ALIGN
    assert lib.dsa_workspace_size(_lib.DSA_WS_PREFILL_STREAM, ctypes.byref(b), 4096, 128, 512) == \
        ctypes.c_size_t(-1).value
    assert lib.dsa_workspace_size(_lib.DSA_WS_PREFILL_STREAM, ctypes.byref(_batch()), 2048, 128, 512) == \
        ctypes.c_size_t(-1).value


def test_short_context_workspace_has_no_scores(lib):
    """max_len <= k: no scores are computed, so the fused workspace holds no score matrix."""
    short = _batch(num_seqs=1, num_rows=2000, max_q=2000, max_len=2000, q_start=FAKE)
    long_ = _batch(num_seqs=1, num_rows=2000, max_q=2000, max_len=2049, q_start=FAKE)
    ws_s = lib.dsa_workspace_size(_lib.DSA_WS_PREFILL, ctypes.byref(short), 2048, 128, 512)
    ws_l = lib.dsa_workspace_size(_lib.DSA_WS_PREFILL, ctypes.byref(long_), 2048, 128, 512)
    assert ws_l - ws_s >= 2000 * 2049 * 4                     # the long case adds the score matrix


def test_workspace_sizes(lib):
    dec = _batch(num_seqs=32, num_rows=32, max_len=131072)
    ws_topk = lib.dsa_workspace_size(_lib.DSA_WS_TOPK, ctypes.byref(dec), 2048, 0, 0)
    # split mode: histograms + candidate lists for every slice of every row
    assert ws_topk >= 32 * 131072 * 8
    pre = _batch(num_seqs=1, num_rows=32768, max_q=32768, max_len=32768, q_start=FAKE)
    assert lib.dsa_workspace_size(_lib.DSA_WS_TOPK, ctypes.byref(pre), 2048, 0, 0) == 0   # row mode
    assert lib.dsa_workspace_size(_lib.DSA_WS_ATTN, ctypes.byref(pre), 2048, 128, 512) == 0  # no split
    att = lib.dsa_workspace_size(_lib.DSA_WS_ATTN, ctypes.byref(dec), 2048, 128, 512)
    assert att > 0 and att % 256 == 0
    assert lib.dsa_workspace_size(_lib.DSA_WS_DECODE, ctypes.byref(pre), 2048, 128, 512) == ctypes.c_size_t(-1).value
    assert lib.dsa_workspace_size(9, ctypes.byref(dec), 2048, 128, 512) == ctypes.c_size_t(-1).value


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load(str(tmp_path / "libdsa.so"))


def test_warmup_validation(lib):
    kidx, kv = _cache(128, seq=4096), _cache(1152, seq=4096)
    pre = _batch(num_seqs=1, num_rows=3000, max_q=3000, max_len=3000, q_start=FAKE)

    def f(b, ws=None, n=0, H=128, D=576, H_I=64, d_I=128, loss=FAKE, dk=None, kvc=kv):
        return lib.dsa_indexer_warmup(ctypes.byref(b), FAKE, ctypes.byref(kvc), H, D, 0.04, FAKE, None, FAKE,
                                      ctypes.byref(kidx), None, H_I, d_I, loss, None, None, dk, ws, n, None)
    need = lib.dsa_workspace_size(_lib.DSA_WS_WARMUP, ctypes.byref(pre), 0, 128, 0)
    assert need >= 3000 * 3000 * 4 + 3000 * 128 * 4            # scores/dI and the per-head log-sum-exps
    assert f(_batch()) == _lib.DSA_ERR_SHAPE                     # decode batch: no q_start
    assert f(_batch(num_seqs=1, num_rows=4, max_q=4, max_len=64, q_start=FAKE, block_table=FAKE,
                    max_blocks=1, block_size=64)) == _lib.DSA_ERR_UNSUPPORTED   # paged caches
    assert f(pre, FAKE, need, H_I=48) == _lib.DSA_ERR_UNSUPPORTED
    assert f(pre, FAKE, need, d_I=32) == _lib.DSA_ERR_UNSUPPORTED
    assert f(pre, FAKE, need, D=64) == _lib.DSA_ERR_UNSUPPORTED
    assert f(pre, FAKE, need, H=72) == _lib.DSA_ERR_UNSUPPORTED
    assert f(pre, FAKE, need, loss=None) == _lib.DSA_ERR_NULL
    assert f(pre, FAKE, need, dk=FAKE + 4) == _lib.DSA_ERR_ALIGN
    assert f(pre) == _lib.DSA_ERR_WORKSPACE
    assert f(pre, FAKE, need - 1) == _lib.DSA_ERR_WORKSPACE
    assert f(pre, FAKE, need, kvc=_cache(1152, seq=100)) == _lib.DSA_ERR_SHAPE      # kv seq_stride < max_len
    # the workspace size ignores k and needs q_start
    assert lib.dsa_workspace_size(_lib.DSA_WS_WARMUP, ctypes.byref(pre), 99999, 128, 0) == need
    assert lib.dsa_workspace_size(_lib.DSA_WS_WARMUP, ctypes.byref(_batch()), 0, 128, 0) == ctypes.c_size_t(-1).value


# ---------------------------------------------------------------- attainable-peak probes (bench references)

PROBES_HEADER = os.path.join(ROOT, "include", "dsa_probes.h")
PROBES_LIB = os.path.join(ROOT, "sparse_attention_long_06_amd", "libdsa_probes.so")


@pytest.fixture(scope="module")
def probes():
    if not os.path.exists(PROBES_LIB):
        from sparse_attention_long_06_amd import build
        build.build()
    lib = ctypes.CDLL(PROBES_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.dsa_probe_stream_read.argtypes = [vp, i64, vp, i64, vp]
    lib.dsa_probe_stream_read_sink_words.argtypes = [i64]
    lib.dsa_probe_stream_read_sink_words.restype = i64
    lib.dsa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, i64, vp]
    lib.dsa_probe_mfma_sink_words.restype = i64
    lib.dsa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.dsa_probe_mfma_flops.restype = ctypes.c_double
    return lib


def test_probe_library_exports_every_declared_symbol(probes):
    txt = re.sub(r"/\*.*?\*/", "", open(PROBES_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", txt)))
    assert names == ["dsa_probe_mfma", "dsa_probe_mfma_flops", "dsa_probe_mfma_sink_words",
                     "dsa_probe_stream_read", "dsa_probe_stream_read_sink_words"]
    for n in names:
        assert hasattr(probes, n), n


def test_probe_sizes_and_argument_checks(probes):
    # 257 tiles of 2 KiB: two workgroups of 256 threads
    assert probes.dsa_probe_stream_read_sink_words(2048 * 257) == 512
    assert probes.dsa_probe_stream_read_sink_words(1000) == -1
    assert probes.dsa_probe_mfma_flops(0, 3) == 2048 * 4 * 3 * 8 * (2 * 16 * 16 * 32)
    assert probes.dsa_probe_mfma_flops(1, 3) == 2048 * 4 * 3 * 4 * (2 * 32 * 32 * 16)
    assert probes.dsa_probe_mfma_flops(2, 3) == -1
    big = 1 << 30
    # every case fails validation before any launch
    assert probes.dsa_probe_stream_read(None, 2048, FAKE, big, None) == -1
    assert probes.dsa_probe_stream_read(FAKE, 1000, FAKE, big, None) == -1
    assert probes.dsa_probe_stream_read(FAKE + 4, 2048, FAKE, big, None) == -1
    assert probes.dsa_probe_stream_read(FAKE, 2048 * 257, FAKE, 511, None) == -1
    assert probes.dsa_probe_mfma(2, 10, FAKE, big, None) == -1
    assert probes.dsa_probe_mfma(0, 0, FAKE, big, None) == -1
    assert probes.dsa_probe_mfma(1, 10, FAKE, probes.dsa_probe_mfma_sink_words() - 1, None) == -1


def test_noalloc_rejects_batches_beyond_its_scratch(lib):
    # the size check happens on the host before any device call
    assert lib.dsa_noalloc_scratch_bytes() == 256 << 20
    b = _batch(num_seqs=4, num_rows=4, max_len=1 << 24)          # 4 x 16M scores alone exceed 256 MiB
    kidx, kv = _cache(128, seq=1 << 24), _cache(1152, seq=1 << 24)
    st = lib.dsa_decode_noalloc(ctypes.byref(b), FAKE, None, FAKE, ctypes.byref(kidx), None, 64, 128, 2048, FAKE,
                                ctypes.byref(kv), None, 128, 576, 512, 0.04, FAKE, FAKE, None, None)
    assert st == _lib.DSA_ERR_WORKSPACE
    assert "static scratch" in _err(lib)
    st = lib.dsa_decode_noalloc(None, FAKE, None, FAKE, ctypes.byref(kidx), None, 64, 128, 2048, FAKE,
                                ctypes.byref(kv), None, 128, 576, 512, 0.04, FAKE, FAKE, None, None)
    assert st == _lib.DSA_ERR_NULL
