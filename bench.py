#!/usr/bin/env python3
"""Benchmark of the DSA hot path on one MI355X: batched decode at 128K context.

One step = one fused dsa_decode call over the whole batch: lightning indexer
over every cached token of every sequence, top-k (k = 2048), sparse MQA
attention over the selected rows, with inputs already resident in HBM.

Prints ONE JSON line (rank 0) with the throughput (queries/s), the roofline
of the dominant kernel (the indexer, HBM-bound) measured with HIP events
inside the timed region, per-stage times, and the CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload decode_b32_ctx128k]
                    [--no-cpu-baseline] [--copy-calibration BYTES]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, vendor figure

# HBM traffic of one decode-indexer launch on this workload, from rocprofv3
# counters (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, averaged over the
# launches of a short bench run), scaled by what the same counters read for a
# 1 GiB device copy: fetch x2.0, write x1.0.  The figures hold only for the
# kernel sources they were taken on; any change to them reports null.
INDEXER_COUNTERS = {
    "workload": "decode_b32_ctx128k",
    "sources": ["sparse_attention_long_06_amd/csrc/indexer.hip", "sparse_attention_long_06_amd/csrc/idx_math.h",
                "sparse_attention_long_06_amd/csrc/dsa_common.h", "sparse_attention_long_06_amd/csrc/dsa_kernels.h",
                "sparse_attention_long_06_amd/csrc/api.hip"],
    "sha256": "bedadf471032f0a17fbb539ae0daf478a6df207d1dd9637e29fb2b9f29085b3c",
    "fetch_kib": 272869.2,
    "write_kib": 16384.0,
    "fetch_scale": 2.0,
    "write_scale": 1.0,
}


def indexer_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in INDEXER_COUNTERS["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def indexer_traffic_bytes(workload="decode_b32_ctx128k"):
    """Counter-measured HBM bytes per indexer launch on the workload the counters
    were taken on, or None (another workload, or the sources changed since)."""
    c = INDEXER_COUNTERS
    if workload != c["workload"] or c["sha256"] is None or c["sha256"] != indexer_sources_sha256():
        return None
    return int(round(c["fetch_kib"] * 1024 * c["fetch_scale"] + c["write_kib"] * 1024 * c["write_scale"]))


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


_ATTAINABLE = None


PROBES_LIB = os.path.join(ROOT, "sparse_attention_long_06_amd", "libdsa_probes.so")


def _probes():
    """ctypes view of libdsa_probes.so (include/dsa_probes.h); raises if it is not built."""
    if not os.path.exists(PROBES_LIB):
        raise RuntimeError(f"{PROBES_LIB} is missing: run `python -m sparse_attention_long_06_amd.build` first")
    lib = ctypes.CDLL(PROBES_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.dsa_probe_stream_read.argtypes = [vp, i64, vp, i64, vp]
    lib.dsa_probe_stream_read.restype = ctypes.c_int
    lib.dsa_probe_stream_read_sink_words.argtypes = [i64]
    lib.dsa_probe_stream_read_sink_words.restype = i64
    lib.dsa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, i64, vp]
    lib.dsa_probe_mfma.restype = ctypes.c_int
    lib.dsa_probe_mfma_sink_words.restype = i64
    lib.dsa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.dsa_probe_mfma_flops.restype = ctypes.c_double
    return lib


def attainable_peaks():
    """Measured reference peaks of this GPU, for fractions beside the vendor ones,
    each the best of 5:
      * HBM: a streaming read of 1 GiB through the DMA-to-LDS path of the decode
        indexer (libdsa_probes.so), a plain 1 GiB device-to-device copy (bytes
        read + written per second) and a 1 GiB torch sum (bytes read per
        second); the HBM reference is the largest of the three;
      * matrix cores: an issue loop of independent bf16 MFMAs in each of the two
        forms the kernels use (v_mfma_f32_16x16x32_bf16, v_mfma_f32_32x32x16_bf16)
        and a bf16 8192^3 GEMM through torch (the vendor BLAS)."""
    global _ATTAINABLE
    if _ATTAINABLE is not None:
        return _ATTAINABLE
    import torch
    probes = _probes()
    n = 1 << 28                                   # 1 GiB of fp32
    src = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda:0")
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda:0")
    nbytes = n * 4
    sink_r = torch.empty(probes.dsa_probe_stream_read_sink_words(nbytes), dtype=torch.int32, device="cuda:0")
    sink_m = torch.empty(probes.dsa_probe_mfma_sink_words(), dtype=torch.float32, device="cuda:0")
    mfma_iters = 4096

    def stream_read():
        st = torch.cuda.current_stream().cuda_stream
        rc = probes.dsa_probe_stream_read(src.data_ptr(), nbytes, sink_r.data_ptr(), sink_r.numel(), st)
        assert rc == 0, f"dsa_probe_stream_read returned {rc}"

    def mfma(form):
        st = torch.cuda.current_stream().cuda_stream
        rc = probes.dsa_probe_mfma(form, mfma_iters, sink_m.data_ptr(), sink_m.numel(), st)
        assert rc == 0, f"dsa_probe_mfma returned {rc}"

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    t_stream = best(stream_read)
    t_copy = best(lambda: dst.copy_(src))
    t_sum = best(lambda: src.sum())
    t_m16 = best(lambda: mfma(0))
    t_m32 = best(lambda: mfma(1))
    t_gemm = best(lambda: torch.mm(a, b))
    stream_gbs = nbytes / (t_stream * 1e-3) / 1e9
    copy_gbs = 2 * nbytes / (t_copy * 1e-3) / 1e9
    read_gbs = nbytes / (t_sum * 1e-3) / 1e9
    m16 = probes.dsa_probe_mfma_flops(0, mfma_iters) / (t_m16 * 1e-3) / 1e12
    m32 = probes.dsa_probe_mfma_flops(1, mfma_iters) / (t_m32 * 1e-3) / 1e12
    _ATTAINABLE = {"stream_read_GB/s": round(stream_gbs, 1), "copy_GB/s": round(copy_gbs, 1),
                   "read_GB/s": round(read_gbs, 1), "hbm_GB/s": round(max(stream_gbs, copy_gbs, read_gbs), 1),
                   "mfma_16x16x32_bf16_TFLOP/s": round(m16, 1), "mfma_32x32x16_bf16_TFLOP/s": round(m32, 1),
                   "gemm_bf16_TFLOP/s": round(2 * 8192 ** 3 / (t_gemm * 1e-3) / 1e12, 1),
                   "how": "1 GiB streaming read by LDS DMA (dsa_probe_stream_read), 1 GiB device copy "
                          "(read + write bytes), 1 GiB torch sum (read bytes); independent bf16 MFMA chains "
                          "(dsa_probe_mfma); bf16 8192^3 torch.mm; best of 5"}
    del src, dst, a, b, sink_r, sink_m
    torch.cuda.empty_cache()
    return _ATTAINABLE


def decode_bytes_per_query(wl, ctx):
    """Algorithmic HBM bytes of one decode query over `ctx` cached tokens.

    index keys + key scales (every token once), the k gathered latent KV rows,
    q, out, and the indexer query (q8, w, q_scale).  Scores and indices are
    intermediate and not counted.
    """
    idx_keys = ctx * (wl.d_I + 4)
    kv = min(wl.k, ctx) * wl.D * 2
    q = wl.H * wl.D * 2
    out = wl.H * wl.D_v * 2
    iq = wl.H_I * wl.d_I + wl.H_I * 4 + 4
    return idx_keys, kv + q + out + iq


def run_bench(args, workload=None, separate_calls=True, attainable=True):
    import torch

    import workloads as W
    import sparse_attention_long_06_amd as dsa
    from sparse_attention_long_06_amd import _lib

    wl = W.BY_NAME[workload or args.workload]
    if wl.kind != "decode":
        raise SystemExit(f"bench.py times the decode path; {wl.name} is a {wl.kind} workload")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # Two copies of the inputs at different addresses, used on alternate
    # steps, so no step finds the previous step's keys in the caches.
    print(f"[bench] generating {wl.name} on {dev} (2 copies)", file=sys.stderr, flush=True)
    sets = [W.generate(wl, dev) for _ in range(2)]
    batches = [dsa.Batch.from_inputs(x) for x in sets]
    inp, batch = sets[0], batches[0]
    B = inp.num_rows
    out = torch.empty((B, wl.H, wl.D_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, wl.H), dtype=torch.float32, device=dev)
    idx = torch.empty((B, wl.k), dtype=torch.int32, device=dev)
    ws_n = dsa.workspace_size(dsa.DSA_WS_DECODE, batch, wl.k, wl.H, wl.D_v)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        x, bt = sets[i % 2], batches[i % 2]
        dsa.decode(bt, x.q8, x.q_scale, x.w, x.k8, x.k_scale, wl.k, x.q, x.kv, x.v,
                   wl.scale, out=out, lse=lse, idx_out=idx, workspace=ws, D_v=wl.D_v)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Four stage events per timed step, recorded by the library on its stream
    # around the indexer (0, 1), after the top-k (2) and at the end (3).
    NEV = 4
    hip = _hip()
    lib = _lib.load()
    events = []
    for _ in range(NEV * args.steps):
        ev = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(ev)) == 0
        events.append(ev.value)
    step_events = [(ctypes.c_void_p * NEV)(*events[NEV * i: NEV * i + NEV]) for i in range(args.steps)]

    # The headline: K steps back to back with nothing else on the stream.
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    # The same K steps again with the stage events armed, for the per-stage
    # times and the indexer's launch duration.  Recording timing events
    # between kernels costs a few microseconds each, so these steps are not
    # the ones the headline is taken from.
    print(f"[bench] timing {args.steps} steps with stage events", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for i in range(args.steps):
        assert lib.dsa_set_stage_events(step_events[i], NEV) == 0
        step(i)
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - te0) * 1e3 / args.steps

    f = ctypes.c_float()

    def ev_ms(e, a, b):
        assert hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(e[a]), ctypes.c_void_p(e[b])) == 0
        return f.value

    stage_ms = {"indexer": 0.0, "topk": 0.0, "attention": 0.0}
    for i in range(args.steps):
        e = events[NEV * i: NEV * i + NEV]
        for name, (a, b) in zip(stage_ms, [(0, 1), (1, 2), (2, 3)]):
            stage_ms[name] += ev_ms(e, a, b) / args.steps
    for ev in events:
        hip.hipEventDestroy(ctypes.c_void_p(ev))

    lens = inp.seq_lens_host
    idx_bytes = sum(decode_bytes_per_query(wl, L)[0] for L in lens)
    other_bytes = sum(decode_bytes_per_query(wl, L)[1] for L in lens)
    idx_gbs = idx_bytes / (stage_ms["indexer"] * 1e-3) / 1e9

    # The three entry points called one by one through the binding (after the
    # timed steps), for reference next to the in-step stage times above.
    st_ix = st_tk = st_at = None
    if separate_calls:
        print("[bench] per-stage calls", file=sys.stderr, flush=True)
        scores = torch.empty((B, (inp.max_len + 3) // 4 * 4), dtype=torch.float32, device=dev)

        def timed(fn, reps=10):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                e1.synchronize()
                ts.append(e0.elapsed_time(e1))
            return sorted(ts)[len(ts) // 2]

        st_ix = timed(lambda: dsa.indexer(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, scores=scores))
        st_tk = timed(lambda: dsa.topk(batch, scores, wl.k, idx=idx))
        st_at = timed(lambda: dsa.sparse_attn(batch, inp.q, inp.kv, inp.v, wl.scale, idx, out=out, lse=lse,
                                              D_v=wl.D_v))
        del scores

    ms = elapsed * 1e3 / args.steps
    qps = B / (elapsed / args.steps)
    ctx_total = sum(lens)
    step_gbs = (idx_bytes + other_bytes) / (ms * 1e-3) / 1e9
    att_bytes = other_bytes - B * (wl.H_I * wl.d_I + wl.H_I * 4 + 4)
    att_gbs = att_bytes / (stage_ms["attention"] * 1e-3) / 1e9
    att_flops = sum(2 * wl.H * min(wl.k, L) * (wl.D + wl.D_v) for L in lens)
    idx_flops = sum(2 * wl.H_I * wl.d_I * L for L in lens)

    res = {
        "metric": "DSA decode queries/s @128K ctx, k=2048; indexer TFLOPS + attn HBM GB/s",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-storage/bf16-mfma",
        "data": "synthetic (seeded N(0,1) draws, per-token e4m3fn quantised indexer q/k; bf16 latent KV; "
                "two input copies used on alternate steps)",
        "config": {"workload": wl.name, "queries": B, "context": wl.seq_len, "k": wl.k, "H_I": wl.H_I,
                   "d_I": wl.d_I, "H": wl.H, "D": wl.D, "D_v": wl.D_v, "paged": wl.paged,
                   "parallelism": "single GPU"},
        "tokens_per_s": round(qps, 1),
        "context_tokens_scanned_per_s": round(ctx_total / (elapsed / args.steps), 1),
        "roofline": {"bound": "hbm", "kernel": "indexer_decode_ring_kernel (decode indexer: FP8 keys, scores)",
                     "achieved": round(idx_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(idx_gbs / HBM_PEAK_GBS, 4), "traffic": indexer_traffic_bytes(wl.name),
                     "bytes_per_launch": idx_bytes, "launch_ms": round(stage_ms["indexer"], 4)},
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "ms_per_step_with_stage_events": round(staged_ms, 4),
        "stages_separate_calls_ms": None if st_ix is None else {
            "indexer": round(st_ix, 4), "topk": round(st_tk, 4), "attention": round(st_at, 4)},
        "step_hbm": {"bytes": idx_bytes + other_bytes, "GB/s": round(step_gbs, 1),
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "indexer_tflops": round(idx_flops / (stage_ms["indexer"] * 1e-3) / 1e12, 2),
        # the decode indexer moves 132 B per 16384 FLOP (124 FLOP/B): at 8 TB/s it
        # can reach at most 0.99 PFLOP/s, about 0.2 of the FP8 matrix-core peak
        "indexer_tflops_frac": {"fp8_peak": round(idx_flops / (stage_ms["indexer"] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                                "hbm_bound_max": round(idx_flops / (stage_ms["indexer"] * 1e-3) / 1e12
                                                       / (HBM_PEAK_GBS * 1e9 * 2 * wl.H_I * wl.d_I
                                                          / (wl.d_I + 4) / 1e12), 4)},
        "attention": {"GB/s": round(att_gbs, 1), "hbm_frac": round(att_gbs / HBM_PEAK_GBS, 4),
                      "TFLOP/s": round(att_flops / (stage_ms["attention"] * 1e-3) / 1e12, 2),
                      "bf16_frac": round(att_flops / (stage_ms["attention"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }
    del ws, out, lse, sets, batches
    torch.cuda.empty_cache()
    if attainable:
        att = attainable_peaks()
        res["attainable"] = att
        res["roofline"]["frac_of_attainable"] = round(idx_gbs / att["hbm_GB/s"], 4)
    return res, inp


def _stream_stage_ms(step, reps):
    """Per-stage times (indexer, selection, attention) of `reps` calls of a fused
    entry point, from the four stage events the library records on its stream."""
    from sparse_attention_long_06_amd import _lib
    hip, lib = _hip(), _lib.load()
    evs = []
    for _ in range(4 * reps):
        ev = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(ev)) == 0
        evs.append(ev.value)
    for i in range(reps):
        assert lib.dsa_set_stage_events((ctypes.c_void_p * 4)(*evs[4 * i: 4 * i + 4]), 4) == 0
        step()
    assert hip.hipDeviceSynchronize() == 0
    f = ctypes.c_float()
    per = {"indexer": [], "topk": [], "attention": []}
    for i in range(reps):
        e = evs[4 * i: 4 * i + 4]
        for name, (a, b) in zip(per, [(0, 1), (1, 2), (2, 3)]):
            assert hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(e[a]), ctypes.c_void_p(e[b])) == 0
            per[name].append(f.value)
    for ev in evs:
        hip.hipEventDestroy(ctypes.c_void_p(ev))
    return {k: sorted(v)[len(v) // 2] for k, v in per.items()}


def _prefill_streaming_call(dsa, wl, inp, batch, out, lse, idx, ws):
    return lambda: dsa.prefill_streaming(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale, wl.k, inp.q,
                                         inp.kv, inp.v, wl.scale, out=out, lse=lse, idx_out=idx, workspace=ws,
                                         D_v=wl.D_v)


def run_prefill(args, attainable=True):
    """One step = indexer, top-k and sparse attention over every row of a causal
    prefill: the three entry points in turn (--select staged, the score matrix
    in HBM between them) or one dsa_prefill_streaming call (--select
    streaming, no score matrix)."""
    import torch

    import workloads as W
    import sparse_attention_long_06_amd as dsa

    wl = W.BY_NAME[args.workload]
    dsa.set_indexer_fp8(bool(getattr(args, "indexer_fp8", False)) and args.select == "streaming")
    if wl.chunk:
        return run_chunked(args, wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {wl.name} on {dev}", file=sys.stderr, flush=True)
    inp = W.generate(wl, dev)
    batch = dsa.Batch.from_inputs(inp)
    T = inp.num_rows
    idx = torch.empty((T, wl.k), dtype=torch.int32, device=dev)
    out = torch.empty((T, wl.H, wl.D_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
    if args.select == "streaming":
        ws_n = dsa.workspace_size(dsa.DSA_WS_PREFILL_STREAM, batch, wl.k, wl.H, wl.D_v)
        ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
        step = _prefill_streaming_call(dsa, wl, inp, batch, out, lse, idx, ws)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        print(f"[bench] timing {args.steps} streaming prefill steps", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        st = _stream_stage_ms(step, max(3, min(args.steps, 10)))
        mem = {"workspace_bytes": ws_n}
    else:
        ld = (inp.max_len + 3) // 4 * 4
        scores = torch.empty((T, ld), dtype=torch.float32, device=dev)
        stages = {"indexer": lambda: dsa.indexer(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale,
                                                 scores=scores),
                  "topk": lambda: dsa.topk(batch, scores, wl.k, idx=idx),
                  "attention": lambda: dsa.sparse_attn(batch, inp.q, inp.kv, inp.v, wl.scale, idx, out=out,
                                                       lse=lse, D_v=wl.D_v)}
        for _ in range(args.warmup):
            for fn in stages.values():
                fn()
        torch.cuda.synchronize()
        print(f"[bench] timing {args.steps} prefill steps", file=sys.stderr, flush=True)
        times = {k: [] for k in stages}
        t0 = time.perf_counter()
        for _ in range(args.steps):
            for name, fn in stages.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                times[name].append((e0, e1))
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        st = {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in times.items()}
        mem = {"score_matrix_bytes": T * ld * 4}
    _, pos = inp.row_positions()
    pairs = sum(p + 1 for p in pos)
    idx_flops = 2 * wl.H_I * wl.d_I * pairs
    att_rows = sum(min(wl.k, p + 1) for p in pos)
    att_flops = 2 * wl.H * (wl.D + wl.D_v) * att_rows
    ms = elapsed * 1e3 / args.steps
    idx_tf = idx_flops / (st["indexer"] * 1e-3) / 1e12
    att_tf = att_flops / (st["attention"] * 1e-3) / 1e12
    return {
        "metric": f"DSA prefill tokens/s (L={wl.seq_len}, k={wl.k}); indexer TFLOPS vs MFMA peak",
        "value": round(T / (elapsed / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8-storage/bf16-mfma",
        "data": "synthetic (seeded N(0,1) draws, per-token e4m3fn quantised indexer q/k; bf16 latent KV)",
        "config": {"workload": wl.name, "rows": T, "context": wl.seq_len, "k": wl.k, "H_I": wl.H_I, "d_I": wl.d_I,
                   "H": wl.H, "D": wl.D, "D_v": wl.D_v, "selection": args.select,
                   "indexer_fp8": bool(getattr(args, "indexer_fp8", False)) and args.select == "streaming",
                   "parallelism": "single GPU"},
        "stages_ms": {k: round(v, 3) for k, v in st.items()},
        "memory": mem,
        "indexer": {"causal_pairs": pairs, "TFLOP/s": round(idx_tf, 1), "fp8_peak_frac": round(idx_tf / 5000.0, 4),
                    "bf16_peak_frac": round(idx_tf / BF16_PEAK_TFLOPS, 4)},
        "attention": {"selected_rows": att_rows, "TFLOP/s": round(att_tf, 1),
                      "bf16_peak_frac": round(att_tf / BF16_PEAK_TFLOPS, 4)},
        "attainable": attainable_peaks() if attainable else None,
        "cpu_baseline": None,
    }


def run_chunked(args, wl):
    """Chunked prefill: every chunk's three stages against the growing cache,
    each chunk's inputs drawn before its stages are timed; one step = all
    chunks."""
    import torch

    import workloads as W
    import sparse_attention_long_06_amd as dsa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nchunks = (wl.seq_len + wl.chunk - 1) // wl.chunk
    print(f"[bench] {wl.name}: {nchunks} chunks", file=sys.stderr, flush=True)
    first = W.generate(wl, dev, chunk_index=0)
    cache = W.cache_of(first)
    st = {"indexer": 0.0, "topk": 0.0, "attention": 0.0}
    pairs = att_rows = rows = 0
    peak_ws = 0
    for c in range(nchunks):
        inp = first if c == 0 else W.generate(wl, dev, chunk_index=c, cache=cache)
        batch = dsa.Batch.from_inputs(inp)
        T = inp.num_rows
        idx = torch.empty((T, wl.k), dtype=torch.int32, device=dev)
        out = torch.empty((T, wl.H, wl.D_v), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
        if args.select == "streaming":
            ws_n = dsa.workspace_size(dsa.DSA_WS_PREFILL_STREAM, batch, wl.k, wl.H, wl.D_v)
            peak_ws = max(peak_ws, ws_n)
            ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
            step = _prefill_streaming_call(dsa, wl, inp, batch, out, lse, idx, ws)
            step()                              # warm-up of this chunk's shapes
            torch.cuda.synchronize()
            for name, v in _stream_stage_ms(step, args.steps).items():
                st[name] += v
            _, pos = inp.row_positions()
            pairs += sum(p + 1 for p in pos)
            att_rows += sum(min(wl.k, p + 1) for p in pos)
            rows += T
            del ws, idx, out, lse
            if c % 8 == 7:
                print(f"[bench] chunk {c + 1}/{nchunks}", file=sys.stderr, flush=True)
            continue
        ld = (inp.max_len + 3) // 4 * 4
        peak_ws = max(peak_ws, T * ld * 4)
        scores = torch.empty((T, ld), dtype=torch.float32, device=dev)
        stages = {"indexer": lambda: dsa.indexer(batch, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale,
                                                 scores=scores),
                  "topk": lambda: dsa.topk(batch, scores, wl.k, idx=idx),
                  "attention": lambda: dsa.sparse_attn(batch, inp.q, inp.kv, inp.v, wl.scale, idx, out=out,
                                                       lse=lse, D_v=wl.D_v)}
        for fn in stages.values():          # warm-up of this chunk's shapes
            fn()
        torch.cuda.synchronize()
        for name, fn in stages.items():
            ts = []
            for _ in range(args.steps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                e1.synchronize()
                ts.append(e0.elapsed_time(e1))
            st[name] += sorted(ts)[len(ts) // 2]
        _, pos = inp.row_positions()
        pairs += sum(p + 1 for p in pos)
        att_rows += sum(min(wl.k, p + 1) for p in pos)
        rows += T
        del scores, idx, out, lse
        if c % 8 == 7:
            print(f"[bench] chunk {c + 1}/{nchunks}", file=sys.stderr, flush=True)
    total = sum(st.values())
    idx_tf = 2 * wl.H_I * wl.d_I * pairs / (st["indexer"] * 1e-3) / 1e12
    att_tf = 2 * wl.H * (wl.D + wl.D_v) * att_rows / (st["attention"] * 1e-3) / 1e12
    return {
        "metric": f"DSA chunked prefill tokens/s (L={wl.seq_len}, chunks of {wl.chunk}, k={wl.k})",
        "value": round(rows / (total * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": 1, "ms_per_step": round(total, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8-storage/bf16-mfma",
        "data": "synthetic (seeded N(0,1) draws, per-token e4m3fn quantised indexer q/k; bf16 latent KV)",
        "config": {"workload": wl.name, "rows": rows, "context": wl.seq_len, "chunk": wl.chunk, "k": wl.k,
                   "selection": args.select,
                   "indexer_fp8": bool(getattr(args, "indexer_fp8", False)) and args.select == "streaming",
                   "parallelism": "single GPU"},
        "stages_ms": {k: round(v, 3) for k, v in st.items()},
        "memory": {("workspace_bytes" if args.select == "streaming" else "score_matrix_bytes"): peak_ws},
        "indexer": {"causal_pairs": pairs, "TFLOP/s": round(idx_tf, 1), "fp8_peak_frac": round(idx_tf / FP8_PEAK_TFLOPS, 4),
                    "bf16_peak_frac": round(idx_tf / BF16_PEAK_TFLOPS, 4)},
        "attention": {"selected_rows": att_rows, "TFLOP/s": round(att_tf, 1),
                      "bf16_peak_frac": round(att_tf / BF16_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    }


def run_warmup(args, att=None):
    """One step = the indexer warm-up objective with all three gradients
    (dsa_indexer_warmup) over every token of the sequence as a query row.
    `att`: attainable-peak measurements already taken in this run (measured
    here when None)."""
    import torch

    import workloads as W
    import sparse_attention_long_06_amd as dsa
    from sparse_attention_long_06_amd import _lib

    wl = W.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {wl.name} on {dev}", file=sys.stderr, flush=True)
    inp = W.generate(wl, dev)
    batch = dsa.Batch.from_inputs(inp)
    T = inp.num_rows
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    dq = torch.empty((T, wl.H_I, wl.d_I), dtype=torch.float32, device=dev)
    dw = torch.empty((T, wl.H_I), dtype=torch.float32, device=dev)
    dk = torch.empty((batch.num_seqs, batch.max_len, wl.d_I), dtype=torch.float32, device=dev)
    ws = torch.empty(dsa.workspace_size(dsa.DSA_WS_WARMUP, batch, 0, wl.H, 0), dtype=torch.uint8, device=dev)

    def step():
        dsa.indexer_warmup(batch, inp.q, inp.kv, wl.scale, inp.q8, inp.q_scale, inp.w, inp.k8, inp.k_scale,
                           loss=loss, dq=dq, dw=dw, dk=dk, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} warm-up objective steps", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps

    # instrumented pass: HIP events recorded by the library between its stages
    hip = _hip()
    names = ["indexer", "dense_lse", "target_kl", "dq_dw", "dk"]
    evs = [ctypes.c_void_p() for _ in range(6)]
    for e in evs:
        hip.hipEventCreate(ctypes.byref(e))
    arr = (ctypes.c_void_p * 6)(*[e.value for e in evs])
    lib = _lib.load()
    acc = [0.0] * 5
    for _ in range(args.steps):
        assert lib.dsa_set_stage_events(arr, 6) == 0
        step()
        torch.cuda.synchronize()
        for i in range(5):
            f = ctypes.c_float()
            hip.hipEventElapsedTime(ctypes.byref(f), evs[i], evs[i + 1])
            acc[i] += f.value
    st = {n: a / args.steps for n, a in zip(names, acc)}
    for e in evs:
        hip.hipEventDestroy(e)

    _, pos = inp.row_positions()
    pairs = sum(p + 1 for p in pos)
    flops = {"indexer": 2 * wl.H_I * wl.d_I * pairs,
             "dense_lse": 2 * wl.H * wl.D * pairs,
             "target_kl": 2 * wl.H * wl.D * pairs,
             "dq_dw": 2 * 2 * wl.H_I * wl.d_I * pairs,      # z recomputed + the dq contraction
             "dk": 2 * 2 * wl.H_I * wl.d_I * pairs}
    tfs = {k: flops[k] / (st[k] * 1e-3) / 1e12 for k in names}
    dom = max(names, key=lambda k: st[k])
    kernel = {"indexer": "indexer_prefill_ring_kernel", "dense_lse": "warm_attn_kernel<0> (dense log-sum-exp pass)",
              "target_kl": "warm_attn_kernel<1> (target, KL, dI)", "dq_dw": "warm_dq_kernel",
              "dk": "warm_dk_kernel + warm_dk_reduce_kernel"}[dom]
    res = {
        "metric": f"DSA indexer warm-up objective tokens/s (KL forward + dq/dw/dk backward, L={wl.seq_len})",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8-storage/bf16-mfma",
        "data": "synthetic (seeded N(0,1) draws, per-token e4m3fn quantised indexer q/k; bf16 q and latent KV)",
        "config": {"workload": wl.name, "rows": T, "context": wl.seq_len, "H_I": wl.H_I, "d_I": wl.d_I,
                   "H": wl.H, "D": wl.D, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": round(tfs[dom], 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tfs[dom] / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "flops_per_launch": flops[dom], "launch_ms": round(st[dom], 4)},
        "stages_ms": {k: round(v, 4) for k, v in st.items()},
        "stages_tflops": {k: round(v, 1) for k, v in tfs.items()},
        "wall_s": round(elapsed, 3),
    }
    if att is None:
        att = attainable_peaks()
        res["attainable"] = att
    # against the fastest measured bf16 matrix-core form (32x32x16); the
    # kernels run the 16x16x32 form, whose own rate gives the second figure
    if att:
        best = max(att["mfma_16x16x32_bf16_TFLOP/s"], att["mfma_32x32x16_bf16_TFLOP/s"])
        res["roofline"]["frac_of_attainable"] = round(tfs[dom] / best, 4)
        res["roofline"]["frac_of_attainable_form_used"] = round(tfs[dom] / att["mfma_16x16x32_bf16_TFLOP/s"], 4)
    if args.no_cpu_baseline:
        res["cpu_baseline"] = None
    else:
        res["cpu_baseline"] = cpu_baseline_warmup(inp, args.cpu_budget)
    return res


def cpu_baseline_warmup(inp, budget_s: float):
    """The warm-up oracle on whole rows, longest first, until ~budget_s of work is done."""
    from oracle import warmup_oracle
    from tests.oracle_io import arrays_of

    a = arrays_of(inp.to("cpu"))
    threads = _oracle_threads()
    T = inp.num_rows
    done = 0
    t0 = time.perf_counter()
    while True:
        warmup_oracle.run_warmup(a, [T - 1 - (done % T)])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    rows = [T - 1 - (i % T) for i in range(done)]
    # the per-row cost grows with the row's position: scale the sampled rate to the whole sequence
    sampled_pairs = sum(r + 1 for r in rows)
    all_pairs = T * (T + 1) // 2
    rate = T / (el * all_pairs / sampled_pairs)
    return {"value": round(rate, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} query rows of {inp.wl.name} from the last backwards (loss, dq, dw, dk of each, "
                      f"{sampled_pairs} causal pairs in {el:.1f} s), fp64 NumPy; rate scaled to all "
                      f"{all_pairs} pairs of the sequence"}


def _oracle_threads():
    try:
        import threadpoolctl
        return max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or os.cpu_count()
    except Exception:  # noqa: BLE001
        return os.cpu_count()


def cpu_baseline(inp, budget_s: float):
    """Time the CPU oracle on whole decode queries until ~budget_s of work is done."""
    import oracle
    from tests.oracle_io import arrays_of

    wl = inp.wl
    B = inp.num_rows
    a = arrays_of(inp.to("cpu"))      # host copies: input preparation, not timed
    threads = _oracle_threads()

    def rate(budget):
        done = 0
        t0 = time.perf_counter()
        while True:                   # cycle over the batch's queries until the budget is spent
            oracle.run_rows(a, [done % B])
            done += 1
            if time.perf_counter() - t0 >= budget:
                break
        return done, time.perf_counter() - t0

    done, el = rate(budget_s)
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    res = {"value": round(done / el, 4), "unit": "queries/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{done} decode queries cycling over the {B} of {wl.name} (each: indexer over "
                     f"{wl.seq_len} tokens, top-{wl.k}, attention), fp64 NumPy, {el:.1f} s",
           "full_step_s": round(B * el / done, 3), "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model}
    try:                              # the same oracle on one thread, over a third of the budget
        import threadpoolctl
        with threadpoolctl.threadpool_limits(1):
            d1, e1 = rate(budget_s / 3)
        res["single_thread_value"] = round(d1 / e1, 4)
        res["single_thread_sample"] = f"{d1} queries, {e1:.1f} s"
    except Exception:  # noqa: BLE001
        res["single_thread_value"] = None
    return res


def copy_calibration(nbytes: int):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_b32_ctx128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="decode headline only: skip the paged-decode, prefill, chunked-prefill and warm-up "
                         "lines of the default run")
    ap.add_argument("--select", choices=("staged", "streaming"), default="streaming",
                    help="prefill workloads: staged entry points with the score matrix, or dsa_prefill_streaming")
    ap.add_argument("--indexer-fp8", action="store_true",
                    help="prefill workloads with --select streaming: the FP8 filter (dsa_set_indexer_fp8(1))")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the DSA path has no multi-GPU mode "
                                   "(sequences or key ranges would be sharded across GPUs); run with --gpus 1"}))
        raise SystemExit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import workloads as W
    if args.workload.startswith("warmup"):
        print(json.dumps(run_warmup(args)), flush=True)
        return
    if W.BY_NAME[args.workload].kind in ("prefill", "chunked_prefill"):
        print(json.dumps(run_prefill(args)), flush=True)
        return
    res, inp = run_bench(args)
    if not args.no_extras and args.workload == "decode_b32_ctx128k":
        res["other_workloads"] = other_workloads(args, res.get("attainable"))
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def other_workloads(args, att=None):
    """The mixed-length paged decode, the 32K prefill (streaming selection,
    then the staged entry points), the 128K chunked prefill and the indexer
    warm-up objective, timed in the same run as the headline (their own
    roofline fractions beside it; `att`: the headline's attainable-peak
    measurements, if taken)."""
    out = {}
    print("[bench] paged_decode_b128_mixed4k_128k", file=sys.stderr, flush=True)
    r, _ = run_bench(args, workload="paged_decode_b128_mixed4k_128k", separate_calls=False, attainable=False)
    out["paged_decode_b128_mixed4k_128k"] = {
        "metric": "queries/s", "value": r["value"], "ms_per_step": r["ms_per_step"], "steps": r["steps"],
        "stages_ms": r["stages_ms"], "step_hbm": r["step_hbm"],
        "indexer": {"GB/s": r["roofline"]["achieved"], "hbm_frac": r["roofline"]["frac"],
                    "bytes_per_launch": r["roofline"]["bytes_per_launch"]},
        "attention": r["attention"]}
    print("[bench] prefill_L32k (streaming selection)", file=sys.stderr, flush=True)
    pargs = argparse.Namespace(**vars(args))
    pargs.workload, pargs.select = "prefill_L32k", "streaming"
    pargs.steps, pargs.warmup = min(args.steps, 5), min(args.warmup, 2)
    p = run_prefill(pargs, attainable=False)
    out["prefill_L32k"] = {k: p[k] for k in ("metric", "value", "unit", "ms_per_step", "steps", "stages_ms",
                                             "indexer", "attention", "memory")}
    if att:
        # the prefill indexer against the fastest measured bf16 matrix-core form
        # (it runs the 16x16x32 form), the attention against the form it runs (32x32x16)
        best = max(att["mfma_16x16x32_bf16_TFLOP/s"], att["mfma_32x32x16_bf16_TFLOP/s"])
        out["prefill_L32k"]["indexer"]["attainable_bf16_frac"] = round(p["indexer"]["TFLOP/s"] / best, 4)
        out["prefill_L32k"]["indexer"]["attainable_form_used_frac"] = round(
            p["indexer"]["TFLOP/s"] / att["mfma_16x16x32_bf16_TFLOP/s"], 4)
        out["prefill_L32k"]["attention"]["attainable_bf16_frac"] = round(
            p["attention"]["TFLOP/s"] / att["mfma_32x32x16_bf16_TFLOP/s"], 4)
    # the same pass through the three staged entry points (score matrix in HBM)
    print("[bench] prefill_L32k (staged selection)", file=sys.stderr, flush=True)
    del p
    sargs = argparse.Namespace(**vars(pargs))
    sargs.select = "staged"
    q = run_prefill(sargs, attainable=False)
    out["prefill_L32k_staged"] = {k: q[k] for k in ("metric", "value", "unit", "ms_per_step", "steps", "stages_ms",
                                                    "memory")}
    del q
    # 128K in 4K-token chunks against the growing cache (streaming selection);
    # each chunk's stages are timed over two passes after one untimed pass
    print("[bench] chunked_prefill_L128k_c4k (streaming selection)", file=sys.stderr, flush=True)
    cargs = argparse.Namespace(**vars(pargs))
    cargs.workload, cargs.select, cargs.steps = "chunked_prefill_L128k_c4k", "streaming", 2
    c = run_prefill(cargs, attainable=False)
    out["chunked_prefill_L128k_c4k"] = {k: c[k] for k in ("metric", "value", "unit", "ms_per_step", "steps",
                                                          "stages_ms", "indexer", "attention", "memory")}
    del c
    print("[bench] warmup_L4k", file=sys.stderr, flush=True)
    wargs = argparse.Namespace(**vars(args))
    wargs.workload, wargs.steps, wargs.warmup, wargs.no_cpu_baseline = "warmup_L4k", 5, 2, True
    w = run_warmup(wargs, att=att or {})
    out["warmup_L4k"] = {k: w[k] for k in ("metric", "value", "unit", "ms_per_step", "steps", "stages_ms",
                                           "stages_tflops", "roofline")}
    return out


if __name__ == "__main__":
    main()
