"""dsa_decode_noalloc (the decode entry point whose workspace is a static device
array) against dsa_decode with a caller workspace, through the C ABI: two calls
in a row, the second on a smaller batch, each bit-identical to dsa_decode.
Collected last on purpose (test_zz_*): the static array stays allocated for
the rest of the process."""
import ctypes

import pytest
import torch

import workloads as W
import sparse_attention_long_06_amd as dsa
from sparse_attention_long_06_amd import _lib
from tests.gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu


def _noalloc(batch, inp, k, out, lse, idx):
    lib = _lib.load()
    wl = inp.wl
    T, H, D = (int(x) for x in inp.q.shape)
    b = batch.c()
    kc, sc = dsa.cache_view(inp.k8, batch), dsa.cache_view(inp.k_scale, batch)
    kvc = dsa.cache_view(inp.kv, batch)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    r = lambda c: None if c is None else ctypes.byref(c)
    st = lib.dsa_decode_noalloc(ctypes.byref(b), p(inp.q8), p(inp.q_scale), p(inp.w), r(kc), r(sc),
                                wl.H_I, wl.d_I, k, p(inp.q), r(kvc), None, H, D, wl.D_v, ctypes.c_float(wl.scale),
                                p(out), p(lse), p(idx), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("first,second", [(W.DECODE_128K.replace(name="decode_b8_ctx64k", seqs=8, seq_len=65536,
                                                                   seed=51),
                                           W.SMALL_PAGED)])
def test_noalloc_decode_matches_decode(first, second):
    lib = _lib.load()
    for wl in (first, second):
        announce("noalloc decode", wl.name)
        inp = W.generate(wl, DEV)
        batch = dsa.Batch.from_inputs(inp)
        idx_r = torch.empty((inp.num_rows, wl.k), dtype=torch.int32, device=DEV)
        out_r, lse_r, _ = dsa.decode(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q, inp.kv,
                                     inp.v, wl.scale, idx_out=idx_r, D_v=wl.D_v)
        out = torch.full_like(out_r, 7.0)
        lse = torch.full_like(lse_r, 7.0)
        idx = torch.full_like(idx_r, 7)
        st = _noalloc(batch, inp, wl.k, out, lse, idx)
        assert st == _lib.DSA_OK, lib.dsa_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_r), wl.name
        assert torch.equal(out.view(torch.int16), out_r.view(torch.int16)), wl.name
        assert torch.equal(lse, lse_r), wl.name
