"""Measured accuracy of the gfx950 matrix-core dot products the indexer could use.

The indexer's contraction must be accurate to fp32 rounding for the top-k
swap rule (1e-5 of the k-th score) to hold on general inputs.  This test
measures, on per-token e4m3fn-quantised N(0,1) operands, the error of each
MFMA form relative to sum_d |q_d k_d| and checks that the bf16 form (the one
the library uses, on exactly widened FP8 values) is at fp32 level.  The FP8
forms' error is printed as a measurement, not asserted.
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


def test_bf16_mfma_on_widened_fp8_is_fp32_accurate():
    announce("mfma precision probe")
    path = os.path.join(HERE, "libmfma_precision.so")
    if not os.path.exists(path):
        from tests.hip import build_probes
        build_probes.build()
    lib = ctypes.CDLL(path)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipLaunchKernel.argtypes = [ctypes.c_void_p, _Dim3, _Dim3, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    nblk, dev = 400, "cuda:0"
    g = torch.Generator().manual_seed(1)
    q8, _ = W.quantize_e4m3fn(torch.randn(nblk * 16, 128, generator=g), 1)
    k8, _ = W.quantize_e4m3fn(torch.randn(nblk * 16, 128, generator=g), 1)
    q16 = q8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    k16 = k8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    bufs = [q8.to(dev), k8.to(dev), q16.to(dev), k16.to(dev)]
    out = torch.zeros(3 * nblk * 256, device=dev)
    args = [ctypes.c_void_p(t.data_ptr()) for t in bufs] + [ctypes.c_void_p(out.data_ptr()), ctypes.c_int(nblk)]
    argv = (ctypes.c_void_p * len(args))(*[ctypes.cast(ctypes.pointer(a), ctypes.c_void_p) for a in args])
    fn = ctypes.c_void_p(ctypes.cast(lib.probe, ctypes.c_void_p).value)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert hip.hipLaunchKernel(fn, _Dim3(nblk, 1, 1), _Dim3(64, 1, 1), argv, 0, stream) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(3, nblk, 16, 16).astype(np.float64)
    qa = oracle.decode_e4m3fn(q8.numpy()).reshape(nblk, 16, 128)
    ka = oracle.decode_e4m3fn(k8.numpy()).reshape(nblk, 16, 128)
    exact = np.einsum("bmk,bnk->bmn", qa, ka)
    scale = np.einsum("bmk,bnk->bmn", np.abs(qa), np.abs(ka))
    rel = [np.abs(o[v] - exact) / scale for v in range(3)]
    for v, name in enumerate(["fp8 16x16x128", "fp8 4x16x16x32", "bf16 4x16x16x32"]):
        print(f"{name}: max err/sum|p| {rel[v].max():.3g}, exact fraction {np.mean(rel[v] == 0):.3f}")
    assert rel[2].max() < 1e-6           # fp32-level: what the indexer relies on
    assert rel[0].max() >= rel[2].max()  # the fp8 forms are not more accurate
