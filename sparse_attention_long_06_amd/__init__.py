"""MI355X (gfx950) DeepSeek Sparse Attention hot path: thin Python binding of libdsa.so.

The binding only marshals torch tensors (device memory) and the current HIP
stream into the C ABI of include/dsa.h; every step of the path runs in the
library's HIP kernels.  If the library is missing, importing works but every
call raises: there is no CPU fallback.

Stages (see include/dsa.h for the full contract):
    indexer(...)      lightning-indexer scores
    topk(...)         per-row top-k token indices
    sparse_attn(...)  MQA attention over the selected tokens
    decode(...)       the three chained for one query per sequence
    prefill(...)      the three chained for query rows per sequence
    indexer_warmup(...)  the indexer's KL warm-up objective and its gradients
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (DSA_WS_ATTN, DSA_WS_DECODE, DSA_WS_PREFILL, DSA_WS_PREFILL_STREAM,  # noqa: F401
                   DSA_WS_TOPK, DSA_WS_WARMUP, DsaBatch, DsaCache)

__all__ = ["Batch", "DsaError", "indexer", "topk", "sparse_attn", "decode", "prefill", "prefill_streaming",
           "indexer_warmup", "workspace_size", "cache_view", "set_attn_splits",
           "set_indexer_fp8"]


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        msg = lib.dsa_last_error().decode()
        super().__init__(f"{where}: {_lib.STATUS_NAMES[status]} ({status}): {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != _lib.DSA_OK:
        raise DsaError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclass
class Batch:
    """Batch geometry: per-sequence cache lengths, query rows and optional page table."""
    seq_lens: torch.Tensor                   # int32 [B] on the device
    num_rows: int
    max_q: int
    max_len: int
    q_start: Optional[torch.Tensor] = None   # int32 [B+1] or None (one query per sequence)
    block_table: Optional[torch.Tensor] = None
    block_size: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    def c(self) -> DsaBatch:
        for name in ("seq_lens", "q_start", "block_table"):
            t = getattr(self, name)
            if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
                raise TypeError(f"{name} must be a contiguous int32 tensor")
        return DsaBatch(self.num_seqs, self.num_rows, self.max_q, self.max_len,
                        self.seq_lens.data_ptr(),
                        None if self.q_start is None else self.q_start.data_ptr(),
                        None if self.block_table is None else self.block_table.data_ptr(),
                        0 if self.block_table is None else int(self.block_table.shape[1]),
                        self.block_size if self.block_table is not None else 0)

    @staticmethod
    def from_inputs(inp) -> "Batch":
        return Batch(seq_lens=inp.seq_lens, num_rows=inp.num_rows, max_q=inp.max_q, max_len=inp.max_len,
                     q_start=inp.q_start, block_table=inp.block_table,
                     block_size=inp.wl.block_size if inp.block_table is not None else 0)


def cache_view(t: Optional[torch.Tensor], batch: Batch) -> Optional[DsaCache]:
    """Describe a cache tensor: [B, cap, ...] (contiguous per sequence) or a paged pool [blocks, block_size, ...]."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise TypeError("cache tensors must be contiguous")
    row_bytes = t[0, 0].numel() * t.element_size() if t.dim() > 2 else t.element_size()
    seq_stride = 0 if batch.paged else int(t.shape[1])
    return DsaCache(t.data_ptr(), row_bytes, seq_stride)


def _ref(c):
    return None if c is None else ctypes.byref(c)


def set_attn_splits(nsplit: int) -> None:
    """dsa_set_attn_splits: force the attention split count of later calls on this thread (0 = automatic)."""
    _check(_lib.load().dsa_set_attn_splits(int(nsplit)), "dsa_set_attn_splits")


def set_indexer_fp8(on: bool) -> None:
    """dsa_set_indexer_fp8: FP8 contraction with exact rescoring (True) or exact scoring only (False, the
    default), for later streaming prefill calls on this thread."""
    _check(_lib.load().dsa_set_indexer_fp8(1 if on else 0), "dsa_set_indexer_fp8")


def workspace_size(entry: int, batch: Batch, k: int, H: int = 0, D_v: int = 0) -> int:
    lib = _lib.load()
    b = batch.c()
    n = lib.dsa_workspace_size(entry, ctypes.byref(b), k, H, D_v)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("dsa_workspace_size: invalid arguments")
    return int(n)


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def indexer(batch: Batch, q8, q_scale, w, k8, k_scale, scores=None, ld=None):
    """Scores [T, ld] fp32 (entries past each row's position are unspecified)."""
    lib = _lib.load()
    H_I, d_I = int(q8.shape[1]), int(q8.shape[2])
    if ld is None:
        ld = (batch.max_len + 3) // 4 * 4
    if scores is None:
        scores = torch.empty((batch.num_rows, ld), dtype=torch.float32, device=q8.device)
    b = batch.c()
    kc, sc = cache_view(k8, batch), cache_view(k_scale, batch)
    _check(lib.dsa_indexer(ctypes.byref(b), _ptr(q8), _ptr(q_scale), _ptr(w), _ref(kc), _ref(sc), H_I, d_I,
                           _ptr(scores), ld, _stream(q8.device)), "dsa_indexer")
    return scores


def topk(batch: Batch, scores, k: int, idx=None):
    lib = _lib.load()
    ld = int(scores.shape[1])
    if idx is None:
        idx = torch.empty((batch.num_rows, k), dtype=torch.int32, device=scores.device)
    ws_n = workspace_size(DSA_WS_TOPK, batch, k)
    ws = _workspace(ws_n, scores.device)
    b = batch.c()
    _check(lib.dsa_topk(ctypes.byref(b), _ptr(scores), ld, k, _ptr(idx), _ptr(ws), ws_n, _stream(scores.device)),
           "dsa_topk")
    return idx


def sparse_attn(batch: Batch, q, kv, v, scale: float, idx, out=None, lse=None, D_v: Optional[int] = None):
    lib = _lib.load()
    T, H, D = (int(x) for x in q.shape)
    k = int(idx.shape[1])
    if D_v is None:
        D_v = int(v.shape[-1]) if v is not None else (512 if D == 576 else D)
    if out is None:
        out = torch.empty((T, H, D_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    ws_n = workspace_size(DSA_WS_ATTN, batch, k, H, D_v)
    ws = _workspace(ws_n, q.device)
    b = batch.c()
    kvc, vc = cache_view(kv, batch), cache_view(v, batch)
    _check(lib.dsa_sparse_attn(ctypes.byref(b), _ptr(q), _ref(kvc), _ref(vc), H, D, D_v, float(scale), _ptr(idx), k,
                               _ptr(out), _ptr(lse), _ptr(ws), ws_n, _stream(q.device)), "dsa_sparse_attn")
    return out, lse


def _fused(entry: str, ws_kind: int, batch: Batch, q8, q_scale, w, k8, k_scale, k: int, q, kv, v, scale: float,
           out=None, lse=None, idx_out=None, workspace=None, D_v: Optional[int] = None):
    lib = _lib.load()
    T, H, D = (int(x) for x in q.shape)
    H_I, d_I = int(q8.shape[1]), int(q8.shape[2])
    if D_v is None:
        D_v = int(v.shape[-1]) if v is not None else (512 if D == 576 else D)
    dev = q.device
    if out is None:
        out = torch.empty((T, H, D_v), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws_n = workspace_size(ws_kind, batch, k, H, D_v)
    if workspace is None:
        workspace = _workspace(ws_n, dev)
    elif workspace.numel() < ws_n:
        raise ValueError(f"workspace too small: {workspace.numel()} < {ws_n}")
    b = batch.c()
    kc, sc = cache_view(k8, batch), cache_view(k_scale, batch)
    kvc, vc = cache_view(kv, batch), cache_view(v, batch)
    _check(getattr(lib, entry)(ctypes.byref(b), _ptr(q8), _ptr(q_scale), _ptr(w), _ref(kc), _ref(sc), H_I, d_I, k,
                               _ptr(q), _ref(kvc), _ref(vc), H, D, D_v, float(scale), _ptr(out), _ptr(lse),
                               _ptr(idx_out), _ptr(workspace), ws_n if workspace is not None else 0, _stream(dev)),
           entry)
    return out, lse, idx_out


def decode(batch: Batch, q8, q_scale, w, k8, k_scale, k: int, q, kv, v, scale: float,
           out=None, lse=None, idx_out=None, workspace=None, D_v: Optional[int] = None):
    """Whole path for one query per sequence (dsa_decode); returns (out, lse, idx_out)."""
    return _fused("dsa_decode", DSA_WS_DECODE, batch, q8, q_scale, w, k8, k_scale, k, q, kv, v, scale,
                  out, lse, idx_out, workspace, D_v)


def prefill(batch: Batch, q8, q_scale, w, k8, k_scale, k: int, q, kv, v, scale: float,
            out=None, lse=None, idx_out=None, workspace=None, D_v: Optional[int] = None):
    """Whole path for query rows per sequence (dsa_prefill); returns (out, lse, idx_out)."""
    return _fused("dsa_prefill", DSA_WS_PREFILL, batch, q8, q_scale, w, k8, k_scale, k, q, kv, v, scale,
                  out, lse, idx_out, workspace, D_v)


def prefill_streaming(batch: Batch, q8, q_scale, w, k8, k_scale, k: int, q, kv, v, scale: float,
                      out=None, lse=None, idx_out=None, workspace=None, D_v: Optional[int] = None):
    """dsa_prefill without the score matrix: the selection streams out of the indexer
    (dsa_prefill_streaming); returns (out, lse, idx_out), equal to prefill's."""
    return _fused("dsa_prefill_streaming", DSA_WS_PREFILL_STREAM, batch, q8, q_scale, w, k8, k_scale, k, q, kv, v,
                  scale, out, lse, idx_out, workspace, D_v)


def indexer_warmup(batch: Batch, q, kv, scale: float, q8, q_scale, w, k8, k_scale, grads: bool = True,
                   loss=None, dq=None, dw=None, dk=None, workspace=None):
    """The indexer's warm-up objective (dsa_indexer_warmup).

    Returns (loss [T], dq [T,H_I,d_I], dw [T,H_I], dk [B,max_len,d_I]); the
    gradients are None when ``grads`` is False and no buffer is passed.
    """
    lib = _lib.load()
    T, H, D = (int(x) for x in q.shape)
    H_I, d_I = int(q8.shape[1]), int(q8.shape[2])
    dev = q.device
    if loss is None:
        loss = torch.empty(T, dtype=torch.float32, device=dev)
    if grads:
        if dq is None:
            dq = torch.empty((T, H_I, d_I), dtype=torch.float32, device=dev)
        if dw is None:
            dw = torch.empty((T, H_I), dtype=torch.float32, device=dev)
        if dk is None:
            dk = torch.empty((batch.num_seqs, batch.max_len, d_I), dtype=torch.float32, device=dev)
    ws_n = workspace_size(DSA_WS_WARMUP, batch, 0, H, 0)
    if workspace is None:
        workspace = _workspace(ws_n, dev)
    elif workspace.numel() < ws_n:
        raise ValueError(f"workspace too small: {workspace.numel()} < {ws_n}")
    b = batch.c()
    kvc = cache_view(kv, batch)
    kc, sc = cache_view(k8, batch), cache_view(k_scale, batch)
    _check(lib.dsa_indexer_warmup(ctypes.byref(b), _ptr(q), _ref(kvc), H, D, float(scale), _ptr(q8), _ptr(q_scale),
                                  _ptr(w), _ref(kc), _ref(sc), H_I, d_I, _ptr(loss), _ptr(dq), _ptr(dw), _ptr(dk),
                                  _ptr(workspace), ws_n, _stream(dev)), "dsa_indexer_warmup")
    return loss, dq, dw, dk
