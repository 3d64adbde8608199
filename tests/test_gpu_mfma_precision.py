"""Measured accuracy of the gfx950 matrix-core dot products the indexer could use.

The indexer's contraction must be accurate to fp32 rounding for the top-k
swap rule (1e-5 of the k-th score) to hold on general inputs.  This test
measures, on per-token e4m3fn-quantised N(0,1) operands (128-dim dots, the
indexer's shape), the error of each MFMA form relative to three scales of the
dot: sum_d |q_d k_d|, ||q||_2 ||k||_2 and max_d |q_d k_d|, and checks:
  * the bf16 form on exactly widened FP8 values (what the library's exact
    scores use) is at fp32 level, below 1e-6 of sum_d |q_d k_d|;
  * the FP8 forms are not: their error reaches 1e-6 of sum_d |q_d k_d| (the
    reason FP8 scores are not used for the selection directly), yet stays
    below 2^-10 of max_d |q_d| * max_d |k_d|.  The streaming indexer's FP8
    filter takes 2^-8 of that product as its margin (four times the pinned
    level), so this pin guards the premise of its exactness.
Besides Gaussian operands the FP8 forms are probed on spiky rows (a few
entries at the e4m3 maximum, the rest tiny) and on pairs built to cancel
(k_d = +-q_d with balanced signs), where the dot is small and the products
are not.  The measured figures are printed one line per form and data set.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu
HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip")


class _Dim3(ctypes.Structure):
    _fields_ = [("x", ctypes.c_uint), ("y", ctypes.c_uint), ("z", ctypes.c_uint)]


def _launch(hip, fn, grid, args, stream):
    argv = (ctypes.c_void_p * len(args))(*[ctypes.cast(ctypes.pointer(a), ctypes.c_void_p) for a in args])
    assert hip.hipLaunchKernel(fn, _Dim3(grid, 1, 1), _Dim3(64, 1, 1), argv, 0, stream) == 0


def _datasets(nrows, g):
    """(name, q, k) float operands of nrows x 128 each, before e4m3fn quantisation."""
    yield "gaussian", torch.randn(nrows, 128, generator=g), torch.randn(nrows, 128, generator=g)
    # spiky: four entries per row 100x the others
    big = torch.zeros(nrows, 128)
    cols = torch.randint(0, 128, (nrows, 4), generator=g)
    big.scatter_(1, cols, 100.0)
    sgn = lambda: torch.randint(0, 2, (nrows, 128), generator=g).float() * 2 - 1
    q = (big + torch.rand(nrows, 128, generator=g)) * sgn()
    k = (big.roll(1, 0) + torch.rand(nrows, 128, generator=g)) * sgn()
    yield "spiky", q, k
    # cancelling: k row i = q row i with half of its signs flipped, so q_i . k_i is near 0
    q = torch.randn(nrows, 128, generator=g) * torch.exp(2 * torch.randn(nrows, 128, generator=g))
    flip = torch.ones(nrows, 128)
    flip[:, torch.randperm(128, generator=g)[:64]] = -1.0
    yield "cancelling", q, q * flip


def test_mfma_forms_accuracy_on_fp8_operands():
    announce("mfma precision probe")
    path = os.path.join(HERE, "libmfma_precision.so")
    if not os.path.exists(path):
        from tests.hip import build_probes
        build_probes.build()
    lib = ctypes.CDLL(path)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipLaunchKernel.argtypes = [ctypes.c_void_p, _Dim3, _Dim3, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    nblk, dev = 800, "cuda:0"
    g = torch.Generator().manual_seed(1)
    for dname, qf, kf in _datasets(nblk * 16, g):
        q8, _ = W.quantize_e4m3fn(qf, 1)
        k8, _ = W.quantize_e4m3fn(kf, 1)
        q16 = q8.view(torch.float8_e4m3fn).to(torch.bfloat16)
        k16 = k8.view(torch.float8_e4m3fn).to(torch.bfloat16)
        bufs = [q8.to(dev), k8.to(dev), q16.to(dev), k16.to(dev)]
        out = torch.zeros(3 * nblk * 256, device=dev)
        out32 = torch.zeros(nblk // 2 * 1024, device=dev)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        args = [ctypes.c_void_p(t.data_ptr()) for t in bufs] + [ctypes.c_void_p(out.data_ptr()), ctypes.c_int(nblk)]
        _launch(hip, ctypes.c_void_p(ctypes.cast(lib.probe, ctypes.c_void_p).value), nblk, args, stream)
        args32 = [ctypes.c_void_p(bufs[0].data_ptr()), ctypes.c_void_p(bufs[1].data_ptr()),
                  ctypes.c_void_p(out32.data_ptr()), ctypes.c_int(nblk // 2)]
        _launch(hip, ctypes.c_void_p(ctypes.cast(lib.probe32, ctypes.c_void_p).value), nblk // 2, args32, stream)
        torch.cuda.synchronize()

        qa = oracle.decode_e4m3fn(q8.numpy())
        ka = oracle.decode_e4m3fn(k8.numpy())
        res = {}

        def stats(name, got, qb, kb):
            exact = np.einsum("bmk,bnk->bmn", qb, kb)
            sabs = np.einsum("bmk,bnk->bmn", np.abs(qb), np.abs(kb))
            norms = np.linalg.norm(qb, axis=2)[:, :, None] * np.linalg.norm(kb, axis=2)[:, None, :]
            pmax = np.max(np.abs(qb[:, :, None, :] * kb[:, None, :, :]), axis=3)
            mm = np.max(np.abs(qb), axis=2)[:, :, None] * np.max(np.abs(kb), axis=2)[:, None, :]
            err = np.abs(got - exact)
            r = dict(sum_abs=(err / sabs).max(), norms=(err / norms).max(), max_prod=(err / pmax).max(),
                     maxes=(err / mm).max(), exact=float(np.mean(err == 0)))
            res[name] = r
            print(f"{dname} {name}: max err / sum|q_d k_d| {r['sum_abs']:.3g}, / (||q|| ||k||) {r['norms']:.3g}, "
                  f"/ max|q_d k_d| {r['max_prod']:.3g}, / (max|q| max|k|) {r['maxes']:.3g}, "
                  f"exact fraction {r['exact']:.3f}", flush=True)

        o = out.cpu().numpy().reshape(3, nblk, 16, 16).astype(np.float64)
        q16b, k16b = qa.reshape(nblk, 16, 128), ka.reshape(nblk, 16, 128)
        for v, name in enumerate(["fp8 16x16x128 (scaled form)", "fp8 4 x 16x16x32", "bf16 4 x 16x16x32"]):
            stats(name, o[v], q16b, k16b)
        o32 = out32.cpu().numpy().reshape(nblk // 2, 32, 32).astype(np.float64)
        stats("fp8 2 x 32x32x64 (scaled form)", o32, qa.reshape(nblk // 2, 32, 128), ka.reshape(nblk // 2, 32, 128))

        assert res["bf16 4 x 16x16x32"]["sum_abs"] < 1e-6, dname   # fp32-level: what the exact scores rely on
        for name in ("fp8 16x16x128 (scaled form)", "fp8 4 x 16x16x32", "fp8 2 x 32x32x64 (scaled form)"):
            if dname == "gaussian":
                assert res[name]["sum_abs"] >= 1e-6, name            # too coarse for the 1e-5 selection rule
            assert res[name]["maxes"] < 2.0 ** -10, (dname, name)    # the filter margin's premise, 4x inside it
