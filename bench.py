"""Benchmark of the BitLinear W1.58A8 hot path on one MI355X.

Workload (the headline): 7B-class decode, M = 1 token, the three projection shapes
(K, N) = (4096, 4096), (4096, 11008), (11008, 4096).  One step = for each shape,
bitlinear_forward_fused (x fp32 -> y fp32: activation quantization, ternary matmul, dequant in
one kernel), i.e. every per-token step of the path; the weights are quantized once beforehand
(the pages cache them).  The same step through the two-call ABI (bitlinear_quantize_act, then
bitlinear_forward) is reported beside it.  Weights rotate through a pool of distinct
copies (> 1 GiB) so that no step finds its weights in the 256 MiB Infinity Cache or the L2.

The K timed steps are captured into one HIP graph (decode steps are replayed, not re-issued
from Python) and timed with HIP events on the capture stream, bracketed by device syncs.
`value` = packed weight bytes streamed per step * K / elapsed (GB/s).

Extra objects on the same JSON line: `roofline` for the dominant kernel (the decode GEMV on the
(4096, 11008) shape, timed in isolation the same way), `prefill` and `prefill_n4096` (M = 2048, K = 4096, N = 11008 and 4096: int8-MFMA TOPS),
`batched` (M = 2/4/8/16/64), `chain70b` (one decode step of the 70B-class stream) and
`cpu_baseline` (the CPU oracle on a bounded sample of the same workload).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
INT8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, 5.0 POPS
METRIC = "decode GEMV weight GB/s (% HBM peak); prefill int8 TOPS (% MFMA peak)"
DECODE_SHAPES = [(4096, 4096), (4096, 11008), (11008, 4096)]   # (K, N)
POOL_BYTES = 1 << 31


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _graph_time(torch, fn, reps: int, warm_fn=None, warm_replays: int = 1, trials: int = 1):
    """Capture `fn(i)` for i < reps into one graph, replay it `warm_replays` times untimed, then
    time `trials` replays (events on the replaying stream around each); return ms per rep of
    the median replay, and the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(min(reps, 3)):
            (warm_fn or fn)(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    for _ in range(warm_replays):      # untimed replays (first-launch costs, clock ramp)
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    times.sort()
    return times[len(times) // 2], g


def _eager_time(torch, fn, reps: int):
    """Launch `fn(i)` for i < reps eagerly (no graph) back to back on the current stream, after
    three untimed calls; return ms per rep, event to event on that stream."""
    for i in range(min(reps, 3)):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _single_call_us(torch, fn, trials: int = 50):
    """Median over `trials` of one eager call on an idle GPU, events on either side of it."""
    times = []
    for i in range(trials):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(i)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    times.sort()
    return times[len(times) // 2]


def decode_setup(torch, bl, workloads, dev):
    """Quantize the three decode weights once, then fill rotation pools of packed copies."""
    per_step = sum(n * k // 4 for k, n in DECODE_SHAPES)
    copies = max(2, POOL_BYTES // per_step)
    shapes = []
    for idx, (k, n) in enumerate(DECODE_SHAPES):
        w = torch.from_numpy(workloads.weights(2, n, k, index=idx)).to(dev)
        packed, alpha = bl.bitlinear_quantize_weights(w)
        del w
        pool = [packed] + [packed.clone() for _ in range(copies - 1)]
        x = [torch.from_numpy(workloads.activations(2, 1, k, index=100 * idx + j)).to(dev) for j in range(8)]
        xq = torch.empty((1, k), dtype=torch.int8, device=dev)
        beta = torch.empty(1, dtype=torch.float32, device=dev)
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        shapes.append(dict(k=k, n=n, pool=pool, alpha=alpha, x=x, xq=xq, beta=beta, y=y))
    torch.cuda.synchronize()
    return shapes, per_step, copies


def decode_step(bl, shapes, copies, i):
    """One decode step: x fp32 -> y fp32 for each shape, one fused call each
    (activation quantization, ternary matmul and dequantization in one kernel)."""
    for sh in shapes:
        bl.bitlinear_forward_fused(sh["x"][i % 8], sh["pool"][i % copies], sh["alpha"], y=sh["y"])


def decode_step_two_call(bl, shapes, copies, i):
    """The same step through the two-call ABI: quantize_act, then forward."""
    for sh in shapes:
        bl.bitlinear_quantize_act(sh["x"][i % 8], sh["xq"], sh["beta"])
        bl.bitlinear_forward(sh["xq"], sh["beta"], sh["pool"][i % copies], sh["alpha"], y=sh["y"])


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_fused_decode7b_hbm_traffic.md")
KERNEL_SOURCES = ["gemv.hip", "common.hpp"]


def kernel_source_sha():
    """sha256 over the sources of the decode GEMV kernel (the traffic figure is void once they change)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bitlinear_matmul_absmean_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic():
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a copy of known size),
    or None when the summary is missing or the kernel sources have changed since it was taken."""
    try:
        with open(TRAFFIC_PROFILE) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != kernel_source_sha():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


TRACE_PROFILE = os.path.join(ROOT, "profiles", "gemv_fused_decode7b_kernel_trace.md")


def _profile_fields(path):
    """`- key: value` lines of a committed profile summary."""
    vals = {}
    try:
        with open(path) as fh:
            for line in fh:
                if line.startswith("- ") and ": " in line:
                    k, v = line[2:].split(": ", 1)
                    vals[k.strip()] = v.strip().strip("`")
    except OSError:
        pass
    return vals


def committed_kernel_trace(alg_bytes):
    """The roofline kernel's mean duration in the committed rocprofv3 kernel trace (the kernel
    alone, without the dispatch gap, but lengthened by the tracer), with the fraction of the HBM
    peak it gives; None when the summary is missing or the kernel sources changed since."""
    v = _profile_fields(TRACE_PROFILE)
    if v.get("source_sha256") != kernel_source_sha():
        return None
    try:
        mean = float(v["kernel_duration_mean_us"])
    except (KeyError, ValueError):
        return None
    gbs = alg_bytes / (mean * 1e-6) / 1e9
    return {"profile": os.path.relpath(TRACE_PROFILE, ROOT), "kernel": v.get("kernel"),
            "kernel_duration_mean_us": mean, "kernel_duration_median_us": float(v.get("kernel_duration_median_us", "nan")),
            "achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}


def roofline_gemv(torch, bl, sh, copies, reps=480, trials=21):
    """Dominant kernel: the fused decode GEMV on (K, N) = (4096, 11008), back to back in a
    graph on one stream, weights rotating through the pool; per launch = median over `trials`
    replays of the graph of `reps` launches, launch to launch (events on the replaying stream)."""
    k, n = sh["k"], sh["n"]
    ms, _ = _graph_time(torch, lambda i: bl.bitlinear_forward_fused(sh["x"][i % 8], sh["pool"][i % copies],
                                                                    sh["alpha"], y=sh["y"]), reps, trials=trials)
    # algorithmic bytes of one launch: packed weights + x (fp32) + alpha + y (fp32)
    alg = n * k // 4 + 4 * k + 4 + 4 * n
    achieved = alg / (ms * 1e-3) / 1e9
    # the unfused forward kernel alone (x_q in), for reference
    bl.bitlinear_quantize_act(sh["x"][0], sh["xq"], sh["beta"])
    ms_f, _ = _graph_time(torch, lambda i: bl.bitlinear_forward(sh["xq"], sh["beta"], sh["pool"][i % copies],
                                                                sh["alpha"], y=sh["y"]), reps, trials=trials)
    # one call from an idle GPU (weights from the pool, not in cache): launch to completion
    single = _single_call_us(torch, lambda i: bl.bitlinear_forward_fused(sh["x"][i % 8], sh["pool"][(7 * i) % copies],
                                                                         sh["alpha"], y=sh["y"]))
    return dict(kernel=bl.bitlinear_forward_fused_kernel(1, k, n, sh["x"][0], sh["pool"][0]),
                shape=dict(M=1, K=k, N=n), bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=committed_traffic(),
                us_per_launch=round(ms * 1e3, 3), timing=f"launch to launch in a graph of {reps} launches, "
                f"median of {trials} replays (HIP events on the replaying stream); includes the dispatch gap",
                kernel_trace=committed_kernel_trace(alg), graph_launches=reps, graph_trials=trials,
                bytes_per_launch=alg, single_call_us=round(single, 2),
                forward_only=dict(kernel="gemv_dot4", us_per_launch=round(ms_f * 1e3, 3),
                                  gbs=round((n * k // 4 + k + 4 * n) / (ms_f * 1e-3) / 1e9, 1)))


def ceilings(torch, dev, read_sizes):
    """Measured ceilings on this GPU, timed like the path's kernels: a streaming read
    (bitlinear_ceiling_read) at each size in `read_sizes`, rotating through 2 GiB of distinct
    data, and an MFMA-only loop of v_mfma_i32_32x32x32_i8 with random and with constant operands."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "bitlinear_matmul_absmean_amd", "libbitlinear_ceiling.so"))
    lib.bitlinear_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.bitlinear_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p]
    pool_bytes = 2 << 30
    pool = torch.ones(pool_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    out = {"hbm_read_gbs": {}, "mfma_i8_tops": {}}
    for size in read_sizes:
        size = (size + 4095) // 4096 * 4096
        copies = max(1, pool_bytes // size)
        reps = 200 if size < (64 << 20) else 10

        def rd(i, size=size, copies=copies):
            st = torch.cuda.current_stream().cuda_stream
            rc = lib.bitlinear_ceiling_read(ctypes.c_void_p(pool.data_ptr() + (i % copies) * size), size,
                                            ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st))
            if rc != 0:
                raise RuntimeError(f"bitlinear_ceiling_read failed ({rc})")
        ms, _ = _graph_time(torch, rd, reps)
        out["hbm_read_gbs"][str(size)] = round(size / (ms * 1e-3) / 1e9, 1)
    del pool
    g = torch.Generator(device="cpu").manual_seed(1580)
    for kind in ("random", "constant"):
        if kind == "random":
            ops_h = torch.randint(-2**31, 2**31 - 1, (65536,), dtype=torch.int64, generator=g).to(torch.int32)
        else:
            ops_h = torch.full((65536,), 0x03030303, dtype=torch.int32)
        ops_d = ops_h.to(dev)
        nops = ctypes.c_int64(0)
        st = torch.cuda.current_stream().cuda_stream
        blocks, iters = 512, 2000
        for _ in range(2):
            lib.bitlinear_ceiling_mfma(blocks, iters, ctypes.c_void_p(ops_d.data_ptr()), ctypes.c_void_p(sink.data_ptr()),
                                       ctypes.byref(nops), ctypes.c_void_p(st))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            rc = lib.bitlinear_ceiling_mfma(blocks, iters, ctypes.c_void_p(ops_d.data_ptr()), ctypes.c_void_p(sink.data_ptr()),
                                            ctypes.byref(nops), ctypes.c_void_p(st))
            if rc != 0:
                raise RuntimeError(f"bitlinear_ceiling_mfma failed ({rc})")
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        out["mfma_i8_tops"][kind] = round(nops.value / (ms * 1e-3) / 1e12, 1)
    torch.cuda.empty_cache()
    return out


def prefill_bench(torch, bl, workloads, dev, k=4096, n=11008, m=2048, reps=20):
    w = torch.from_numpy(workloads.weights(4, n, k)).to(dev)
    packed, alpha = bl.bitlinear_quantize_weights(w)
    del w
    x = torch.from_numpy(workloads.activations_with_outliers(4, m, k)).to(dev)
    xq, beta = bl.bitlinear_quantize_act(x)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    ms, _ = _graph_time(torch, lambda i: bl.bitlinear_forward(xq, beta, packed, alpha, y=y), reps, warm_replays=3)
    msq, _ = _graph_time(torch, lambda i: bl.bitlinear_quantize_act(x, xq, beta), reps, warm_replays=3)
    tops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    return dict(shape=dict(M=m, K=k, N=n), kernel=bl.bitlinear_forward_kernel(m, k, n, xq, packed),
                us=round(ms * 1e3, 2), tops=round(tops, 1), pct_mfma_peak=round(100 * tops / INT8_MFMA_PEAK_TOPS, 2),
                quantize_act_us=round(msq * 1e3, 2),
                end_to_end_tops=round(2.0 * m * n * k / ((ms + msq) * 1e-3) / 1e12, 1))


def quantize_bench(torch, bl, workloads, dev, reps=20):
    """a1 and a2 against the HBM roofline.  Weight quantization (offline, once per layer) reads W
    twice (absmean first, then the codes) and writes the packed bytes: 8NK + NK/4 bytes for
    W [11008, 4096].  Activation quantization reads x and writes x_q and beta: 5MK + 4M bytes,
    for the prefill batch (M = 2048, K = 4096) and one decode token (M = 1, K = 4096)."""
    n, k = 11008, 4096
    w = torch.from_numpy(workloads.weights(4, n, k)).to(dev)
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device=dev)
    alpha = torch.empty(1, dtype=torch.float32, device=dev)
    alpha_rows = torch.empty(n, dtype=torch.float32, device=dev)
    ws = torch.empty(max(8, bl.lib.bitlinear_quantize_weights_workspace_size(n, k)), dtype=torch.uint8, device=dev)
    ms_w, _ = _graph_time(torch, lambda i: bl.bitlinear_quantize_weights(w, packed, alpha, ws), reps)
    ms_r, _ = _graph_time(torch, lambda i: bl.bitlinear_quantize_weights_rows(w, packed, alpha_rows), reps)
    del w
    bw = 8 * n * k + n * k // 4
    out = {"quantize_weights": {"shape": dict(N=n, K=k), "alg_bytes": bw, "us": round(ms_w * 1e3, 2),
                                "gbs": round(bw / (ms_w * 1e-3) / 1e9, 1),
                                "pct_hbm": round(100 * bw / (ms_w * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                                "per_row_alpha_us": round(ms_r * 1e3, 2)}}
    acts = []
    for m in (2048, 1):
        x = torch.from_numpy(workloads.activations_with_outliers(4, m, k) if m > 1 else
                             workloads.activations(2, 1, k)).to(dev)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        beta = torch.empty(m, dtype=torch.float32, device=dev)
        ms, _ = _graph_time(torch, lambda i: bl.bitlinear_quantize_act(x, xq, beta), 200 if m == 1 else reps)
        ba = 5 * m * k + 4 * m
        acts.append({"M": m, "K": k, "alg_bytes": ba, "us": round(ms * 1e3, 2),
                     "gbs": round(ba / (ms * 1e-3) / 1e9, 1),
                     "pct_hbm": round(100 * ba / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)})
    out["quantize_act"] = acts
    torch.cuda.empty_cache()
    return out


def hadamard_block(k: int) -> int:
    """Largest power of two <= 4096 dividing K: the block of the rotation for that K."""
    b = 1
    while b < 4096 and k % (2 * b) == 0:
        b *= 2
    return b


def hadamard_bench(torch, bl, workloads, dev, ms_plain_step, reps=20):
    """Rotation before absmax [P3 §6.2].  Activations: rotate + per-token absmax int8 in one
    pass reads x and the signs and writes x_q and beta, 5MK + 4M + K bytes.  Weights (offline):
    rotate W [11008, 4096], 8NK + K bytes.  Decode: the 7B-class step with rotated projections,
    one bitlinear_forward_fused_hadamard call each (rotation, quantization and GEMV in one
    launch), beside the two-launch form (hadamard_rows, then the fused GEMV)."""
    out = {}
    acts = []
    for m, k in ((2048, 4096), (2048, 11008), (1, 4096)):
        b = hadamard_block(k)
        x = torch.from_numpy(workloads.activations_with_outliers(4, m, k)).to(dev)
        d = torch.from_numpy(workloads.rotation_signs(4, k)).to(dev)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        beta = torch.empty(m, dtype=torch.float32, device=dev)
        ms, _ = _graph_time(torch, lambda i: bl.bitlinear_quantize_act_hadamard(x, b, d, xq, beta),
                            200 if m == 1 else reps)
        ba = 5 * m * k + 4 * m + k
        acts.append({"M": m, "K": k, "block": b, "alg_bytes": ba, "us": round(ms * 1e3, 2),
                     "gbs": round(ba / (ms * 1e-3) / 1e9, 1),
                     "pct_hbm": round(100 * ba / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)})
    out["quantize_act_hadamard"] = acts
    n, k = 11008, 4096
    w = torch.from_numpy(workloads.weights(4, n, k)).to(dev)
    d = torch.from_numpy(workloads.rotation_signs(4, k)).to(dev)
    wr = torch.empty_like(w)
    ms, _ = _graph_time(torch, lambda i: bl.bitlinear_hadamard_rows(w, 4096, d, wr), reps)
    bw = 8 * n * k + k
    out["hadamard_rows_weights"] = {"N": n, "K": k, "block": 4096, "alg_bytes": bw, "us": round(ms * 1e3, 2),
                                    "gbs": round(bw / (ms * 1e-3) / 1e9, 1),
                                    "pct_hbm": round(100 * bw / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
    del w, wr
    per_step = sum(n * k // 4 for k, n in DECODE_SHAPES)
    copies = max(2, POOL_BYTES // per_step)
    shapes = []
    for idx, (k, n) in enumerate(DECODE_SHAPES):
        b = hadamard_block(k)
        d = torch.from_numpy(workloads.rotation_signs(2, k, index=idx)).to(dev)
        w = torch.from_numpy(workloads.weights(2, n, k, index=idx)).to(dev)
        bl.bitlinear_hadamard_rows(w, b, d, out=w)
        packed, alpha = bl.bitlinear_quantize_weights(w)
        del w
        pool = [packed] + [packed.clone() for _ in range(copies - 1)]
        x = [torch.from_numpy(workloads.activations(2, 1, k, index=100 * idx + j)).to(dev) for j in range(8)]
        shapes.append(dict(k=k, block=b, signs=d, pool=pool, alpha=alpha, x=x,
                           xr=torch.empty((1, k), dtype=torch.float32, device=dev),
                           y=torch.empty((1, n), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()

    def step(i):
        for sh in shapes:
            bl.bitlinear_forward_fused_hadamard(sh["x"][i % 8], sh["block"], sh["signs"], sh["pool"][i % copies],
                                                sh["alpha"], y=sh["y"])

    def step_two_launch(i):
        for sh in shapes:
            bl.bitlinear_hadamard_rows(sh["x"][i % 8], sh["block"], sh["signs"], out=sh["xr"])
            bl.bitlinear_forward_fused(sh["xr"], sh["pool"][i % copies], sh["alpha"], y=sh["y"])

    ms, _ = _graph_time(torch, step, 400)
    ms2, _ = _graph_time(torch, step_two_launch, 400)
    out["decode_rotated"] = {"shapes_KN": DECODE_SHAPES, "blocks": [sh["block"] for sh in shapes],
                             "call": "bitlinear_forward_fused_hadamard",
                             "us_per_step": round(ms * 1e3, 2), "weight_gbs": round(per_step / (ms * 1e-3) / 1e9, 1),
                             "plain_us_per_step": round(ms_plain_step * 1e3, 2),
                             "rotation_overhead_us": round((ms - ms_plain_step) * 1e3, 2),
                             "two_launch_us_per_step": round(ms2 * 1e3, 2)}
    del shapes
    torch.cuda.empty_cache()
    return out


def blocks_bench(torch, bl, workloads, dev, ms_plain_step):
    """Block-scaled weights [P1 §2.3, §4.2] (one alpha per 128 weights): the 7B decode step
    (three GEMVs, M = 1) with block-scaled weights and x_q given, its bytes (NK/4 codes +
    NK/32 scales + K x_q + 4N y per shape), batched M = 4, 16 and 64 on (4096, 11008), and
    prefill M = 2048 on the same shape."""
    per_step = sum(n * k // 4 + n * k // 32 for k, n in DECODE_SHAPES)
    copies = max(2, POOL_BYTES // per_step)
    shapes = []
    for idx, (k, n) in enumerate(DECODE_SHAPES):
        w = torch.from_numpy(workloads.weights(2, n, k, index=idx)).to(dev)
        packed, ab = bl.bitlinear_quantize_weights_blocks(w)
        del w
        pool = [(packed, ab)] + [(packed.clone(), ab.clone()) for _ in range(copies - 1)]
        x = torch.from_numpy(workloads.activations(2, 1, k, index=100 * idx)).to(dev)
        xq, beta = bl.bitlinear_quantize_act(x)
        shapes.append(dict(pool=pool, xq=xq, beta=beta, y=torch.empty((1, n), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()

    def step(i):
        for sh in shapes:
            p, ab = sh["pool"][i % copies]
            bl.bitlinear_forward_blocks(sh["xq"], sh["beta"], p, ab, y=sh["y"])

    ms, _ = _graph_time(torch, step, 400)
    out = {"decode_step": {"shapes_KN": DECODE_SHAPES, "bytes_per_step": per_step, "us_per_step": round(ms * 1e3, 2),
                           "gbs": round(per_step / (ms * 1e-3) / 1e9, 1),
                           "pct_hbm": round(100 * per_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                           "per_tensor_fused_us_per_step": round(ms_plain_step * 1e3, 2)}}
    del shapes
    k, n = 4096, 11008
    w = torch.from_numpy(workloads.weights(3, n, k)).to(dev)
    packed, ab = bl.bitlinear_quantize_weights_blocks(w)
    del w
    copies = max(2, POOL_BYTES // (n * k // 4 + n * k // 32))
    pool = [(packed, ab)] + [(packed.clone(), ab.clone()) for _ in range(copies - 1)]
    out["batched"] = []
    for m in (4, 16, 64):
        x = torch.from_numpy(workloads.activations(3, m, k)).to(dev)
        xq, beta = bl.bitlinear_quantize_act(x)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        ms, _ = _graph_time(torch, lambda i: bl.bitlinear_forward_blocks(xq, beta, *pool[i % copies], y=y), 96, trials=5)
        out["batched"].append({"M": m, "K": k, "N": n, "us": round(ms * 1e3, 2),
                               "kernel": "16x16x64 int8 MFMA tiles, int32 sums per block scaled in fp64" +
                                         (", x_q and codes loaded into LDS" if m >= 3 and k % 256 == 0 else "") +
                                         ("" if m <= 64 else f", {(m + 63) // 64} slices of up to 64 tokens")})
    del pool
    # prefill with block scales: M = 2048 (int8 ops 2MNK) beside the per-tensor GEMM of the same shape
    m = 2048
    x = torch.from_numpy(workloads.activations_with_outliers(4, m, k)).to(dev)
    xq, beta = bl.bitlinear_quantize_act(x)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    ms, _ = _graph_time(torch, lambda i: bl.bitlinear_forward_blocks(xq, beta, packed, ab, y=y), 10, warm_replays=3)
    ops = 2.0 * m * n * k
    out["prefill"] = {"M": m, "K": k, "N": n, "us": round(ms * 1e3, 2), "tops": round(ops / (ms * 1e-3) / 1e12, 1),
                      "pct_mfma_peak": round(100 * ops / (ms * 1e-3) / 1e12 / INT8_MFMA_PEAK_TOPS, 2),
                      "kernel": "block-scaled GEMM, 128 x 128 tiles, fp64 sum per output"}
    torch.cuda.empty_cache()
    return out


def t5_bench(torch, bl, workloads, dev):
    """Five codes per byte (1.6 bits per weight): the 7B decode step (three GEMVs, M = 1,
    x_q given) on 5-trit weights beside the same step on the 2-bit packing, weights rotated
    through pools of copies."""
    out = {"shapes_KN": DECODE_SHAPES}
    for tag in ("2bit", "t5"):
        bytes_step = sum(n * (k // 4 if tag == "2bit" else bl.lib.bitlinear_t5_row_bytes(k)) for k, n in DECODE_SHAPES)
        copies = max(2, POOL_BYTES // bytes_step)
        shapes = []
        for idx, (k, n) in enumerate(DECODE_SHAPES):
            w = torch.from_numpy(workloads.weights(2, n, k, index=idx)).to(dev)
            packed, alpha = bl.bitlinear_quantize_weights(w)
            del w
            p = packed if tag == "2bit" else bl.bitlinear_repack_t5(packed, k)
            pool = [p] + [p.clone() for _ in range(copies - 1)]
            x = torch.from_numpy(workloads.activations(2, 1, k, index=100 * idx)).to(dev)
            xq, beta = bl.bitlinear_quantize_act(x)
            shapes.append(dict(pool=pool, alpha=alpha, xq=xq, beta=beta,
                               y=torch.empty((1, n), dtype=torch.float32, device=dev)))
        torch.cuda.synchronize()
        fwd = bl.bitlinear_forward if tag == "2bit" else bl.bitlinear_forward_t5

        def step(i):
            for sh in shapes:
                fwd(sh["xq"], sh["beta"], sh["pool"][i % copies], sh["alpha"], y=sh["y"])

        ms, _ = _graph_time(torch, step, 400)
        out[tag] = {"bytes_per_step": bytes_step, "us_per_step": round(ms * 1e3, 2),
                    "gbs": round(bytes_step / (ms * 1e-3) / 1e9, 1)}
        del shapes
        torch.cuda.empty_cache()
    return out


def mlp_bench(torch, bl, workloads, dev, d=4096, f=11008):
    """BitMLP [P3 §6.1], y = fc2(GELU(fc1(x))) at 7B-class sizes (d_model 4096, d_ff 11008),
    one bitlinear_mlp_forward call: decode (M = 1, weights rotated through a pool, packed
    bytes 2 d f / 4 per step) and prefill (M = 2048, int8 ops 2 * 2 M d f)."""
    per_step = 2 * d * f // 4
    copies = max(2, POOL_BYTES // per_step)
    w1 = torch.from_numpy(workloads.weights(6, f, d)).to(dev)
    w2 = torch.from_numpy(workloads.weights(6, d, f, index=1)).to(dev)
    p1, a1 = bl.bitlinear_quantize_weights(w1)
    p2, a2 = bl.bitlinear_quantize_weights(w2)
    del w1, w2
    pool = [(p1, p2)] + [(p1.clone(), p2.clone()) for _ in range(copies - 1)]
    x = torch.from_numpy(workloads.activations(6, 1, d)).to(dev)
    y = torch.empty((1, d), dtype=torch.float32, device=dev)
    g = torch.empty((1, f), dtype=torch.float32, device=dev)

    def step(i):
        q1, q2 = pool[i % copies]
        bl.bitlinear_mlp_forward(x, q1, a1, q2, a2, y=y, g=g)

    ms, _ = _graph_time(torch, step, 400)
    out = {"shape": {"d_model": d, "d_ff": f},
           "decode": {"M": 1, "us": round(ms * 1e3, 2), "weight_bytes": per_step,
                      "weight_gbs": round(per_step / (ms * 1e-3) / 1e9, 1),
                      "pct_hbm": round(100 * per_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}}
    del pool
    m = 2048
    xp = torch.from_numpy(workloads.activations(6, m, d)).to(dev)
    yp = torch.empty((m, d), dtype=torch.float32, device=dev)
    gp = torch.empty((m, f), dtype=torch.float32, device=dev)
    xq1 = torch.empty((m, d), dtype=torch.int8, device=dev)
    xq2 = torch.empty((m, f), dtype=torch.int8, device=dev)
    b1 = torch.empty(m, dtype=torch.float32, device=dev)
    b2 = torch.empty(m, dtype=torch.float32, device=dev)
    ms, _ = _graph_time(torch, lambda i: bl.bitlinear_mlp_forward(xp, p1, a1, p2, a2, y=yp, g=gp, x_q1=xq1, beta1=b1,
                                                                   x_q2=xq2, beta2=b2), 10, warm_replays=3)
    ops = 2.0 * 2 * m * d * f
    out["prefill"] = {"M": m, "us": round(ms * 1e3, 2), "tops": round(ops / (ms * 1e-3) / 1e12, 1),
                      "pct_mfma_peak": round(100 * ops / (ms * 1e-3) / 1e12 / INT8_MFMA_PEAK_TOPS, 2)}
    torch.cuda.empty_cache()
    return out


def batched_bench(torch, bl, workloads, dev, reps=96):
    out = []
    for (k, n) in [(4096, 11008), (11008, 4096)]:
        w = torch.from_numpy(workloads.weights(3, n, k)).to(dev)
        packed, alpha = bl.bitlinear_quantize_weights(w)
        del w
        copies = max(2, (1 << 30) // (n * k // 4))
        pool = [packed] + [packed.clone() for _ in range(copies - 1)]
        for m in (2, 4, 8, 16, 64):
            x = torch.from_numpy(workloads.activations(3, m, k)).to(dev)
            xq, beta = bl.bitlinear_quantize_act(x)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            ms, _ = _graph_time(torch, lambda i: bl.bitlinear_forward(xq, beta, pool[i % copies], alpha, y=y), reps,
                                trials=5)
            gbs = n * k / 4 / (ms * 1e-3) / 1e9
            out.append(dict(M=m, K=k, N=n, kernel=bl.bitlinear_forward_kernel(m, k, n, xq, packed),
                            us=round(ms * 1e3, 2), weight_gbs=round(gbs, 1),
                            pct_hbm=round(100 * gbs / HBM_PEAK_GBS, 2)))
        del pool
        torch.cuda.empty_cache()
    return out


def chain70b_bench(torch, bl, workloads, dev, layers=80, reps=3):
    """One decode step of the 70B-class stream: 80 layers x 7 projections, one fused call
    each on x = stream_activation(layer, projection) (the two-call ABI reported beside it),
    weights generated on the device (17.1 GB resident), one stream, in order.  The grouped variant makes 4 calls per layer: q, k and v
    (which read the same x) as one bitlinear_forward_fused_rows call over their stacked rows,
    gate and up likewise, o and down alone -- the same bytes and, bit for bit, the same outputs.
    Each layer's q/k/v and gate/up rows are allocated adjacent, so the grouped calls take views."""
    projs, groups = [], []
    total = 0
    P = workloads.W5_PROJ
    for layer in range(layers):
        alphas = [workloads.stream_alpha(layer, p) for p in range(len(P))]
        bufs = {}
        for members in ((0, 1, 2), (3,), (4, 5), (6,)):
            k = P[members[0]][1]
            rows = sum(P[p][2] for p in members)
            buf = torch.empty((rows, k // 4), dtype=torch.uint8, device=dev)
            r0 = 0
            for p in members:
                n = P[p][2]
                view = buf[r0:r0 + n]
                workloads.device_stream_packed(view, layer, p)
                bufs[p] = view
                r0 += n
            total += buf.numel()
            ar = np.concatenate([np.full(P[p][2], alphas[p], np.float32) for p in members])
            groups.append((k, rows, buf, torch.from_numpy(ar).to(dev)))
        for p, (name, k, n) in enumerate(P):
            projs.append((k, n, bufs[p], torch.tensor([alphas[p]], device=dev)))
    # x per (layer, projection); a grouped call takes the x of its first projection
    xs = [torch.from_numpy(workloads.stream_activation(layer, p, P[p][1])).to(dev)
          for layer in range(layers) for p in range(len(P))]
    gx = [xs[layer * len(P) + first] for layer in range(layers) for first in (0, 3, 4, 6)]
    xq = {k: torch.empty((1, k), dtype=torch.int8, device=dev) for k in (8192, 28672)}
    beta = torch.empty(1, dtype=torch.float32, device=dev)
    ys = {n: torch.empty((1, n), dtype=torch.float32, device=dev) for n in (1024, 8192, 10240, 28672, 57344)}
    torch.cuda.synchronize()

    def step(i):
        for x, (k, n, wp, alpha) in zip(xs, projs):
            bl.bitlinear_forward_fused(x, wp, alpha, y=ys[n])

    def step_two_call(i):
        for x, (k, n, wp, alpha) in zip(xs, projs):
            bl.bitlinear_quantize_act(x, xq[k], beta)
            bl.bitlinear_forward(xq[k], beta, wp, alpha, y=ys[n])

    def step_grouped(i):
        for x, (k, n, wp, alpha_rows) in zip(gx, groups):
            bl.bitlinear_forward_fused_rows(x, wp, alpha_rows, y=ys[n])
    ms, _ = _graph_time(torch, step, reps)
    ms2, _ = _graph_time(torch, step_two_call, reps)
    ms3, _ = _graph_time(torch, step_grouped, reps)
    ms_e = _eager_time(torch, step, 1)
    gbs = total / (ms * 1e-3) / 1e9
    res = dict(layers=layers, weight_bytes=total, ms_per_step=round(ms, 3), weight_gbs=round(gbs, 1),
               pct_hbm=round(100 * gbs / HBM_PEAK_GBS, 2), tokens_per_s=round(1e3 / ms, 1),
               two_call_ms_per_step=round(ms2, 3), eager_ms_per_step=round(ms_e, 3),
               grouped=dict(calls_per_layer=4, ms_per_step=round(ms3, 3),
                            weight_gbs=round(total / (ms3 * 1e-3) / 1e9, 1),
                            pct_hbm=round(100 * total / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                            tokens_per_s=round(1e3 / ms3, 1)))
    del projs, groups
    torch.cuda.empty_cache()
    return res


def host_cpu():
    """nproc (CPUs this process may run on), physical cores among them, and the model name."""
    try:
        cpus = sorted(os.sched_getaffinity(0))
    except AttributeError:
        cpus = list(range(os.cpu_count() or 1))
    cores = set()
    for c in cpus:
        try:
            with open(f"/sys/devices/system/cpu/cpu{c}/topology/core_id") as f:
                core = f.read().strip()
            with open(f"/sys/devices/system/cpu/cpu{c}/topology/physical_package_id") as f:
                pkg = f.read().strip()
            cores.add((pkg, core))
        except OSError:
            cores.add(("?", str(c)))
    model = "unknown"
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    return len(cpus), len(cores), model


def cpu_baseline(workloads, budget_s=3.0, max_threads=16):
    """The CPU oracle (as it stands, never tuned) on bounded samples of the workloads, on this
    host's cores, with 1 thread and with P threads = the physical cores this process may use
    (at most 16, the host share of one GPU), output rows split over the threads:
      * decode: whole 7B decode steps (quantize_act, unpack, integer matmul, dequant for the three
        shapes), weight GB/s -- the headline's metric; `value` is the P-thread figure;
      * batched: M = 64, K = 4096, N = 11008 on a slice of the output rows, scaled to the whole
        matrix (weight GB/s);
      * prefill: M = 2048, K = 4096, N = 11008 on a slice of the output rows, scaled (int8 GOPS);
      * chain70b: one layer of the 70B-class stream (7 projections, the codes generated before
        the timer), scaled by 80 layers (weight GB/s, tokens/s)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    nproc, phys, model = host_cpu()
    P = max(1, min(max_threads, phys))

    def timed(fn, threads, budget):
        pool = ThreadPoolExecutor(threads)
        reps, t0 = 0, time.perf_counter()
        while True:
            fn(pool, threads)
            reps += 1
            if time.perf_counter() - t0 > budget:
                break
        dt = time.perf_counter() - t0
        pool.shutdown()
        return reps, dt

    def forward_rows(pool, threads, xq, beta, packed, k, alpha, n0, n1):
        bounds = np.linspace(n0, n1, threads + 1).astype(int)

        def part(t):
            a, b = bounds[t], bounds[t + 1]
            if b > a:
                oracle.forward(xq, beta, packed[a:b], k, alpha)
        list(pool.map(part, range(threads)))

    log(f"cpu_baseline: {nproc} CPUs, {phys} physical cores ({model}); P = {P} threads")
    out = {"nproc": nproc, "physical_cores": phys, "model_name": model, "threads_p": P, "settings": []}
    # decode steps
    data = []
    for idx, (k, n) in enumerate(DECODE_SHAPES):
        w = workloads.weights(2, n, k, index=idx)
        codes, packed, alpha = oracle.quantize_weights(w)
        data.append((k, n, packed, alpha, workloads.activations(2, 1, k, index=100 * idx)))
    per_step = sum(n * k // 4 for k, n in DECODE_SHAPES)

    def decode(pool, threads):
        for (k, n, packed, alpha, x) in data:
            xq, beta = oracle.quantize_act(x)
            forward_rows(pool, threads, xq, beta, packed, k, alpha, 0, n)
    for th in (1, P):
        reps, dt = timed(decode, th, budget_s)
        out["settings"].append(dict(workload="decode", threads=th, value=round(per_step * reps / dt / 1e9, 4),
                                    unit="GB/s", sample=f"{reps} whole decode steps in {dt:.1f} s"))
    # batched decode and prefill: a slice of the tokens over every output row, scaled to the whole
    # call (a slice of the rows instead would repeat a few rows' code sequence for every token,
    # which the host's branch predictor learns, and overstate the oracle's speed)
    k, n = 4096, 11008
    w = workloads.weights(3, n, k)
    codes, packed, alpha = oracle.quantize_weights(w)
    for name, m, toks in (("batched", 64, 4), ("prefill", 2048, 4)):
        x = workloads.activations_with_outliers(4, m, k) if m >= 512 else workloads.activations(3, m, k)
        xq, beta = oracle.quantize_act(x)
        xs, bs = np.ascontiguousarray(xq[:toks]), np.ascontiguousarray(beta[:toks])
        for th in (1, P):
            reps, dt = timed(lambda pool, t: forward_rows(pool, t, xs, bs, packed, k, alpha, 0, n), th, budget_s)
            per = dt / reps * m / toks                         # seconds per whole call, scaled
            if name == "batched":
                v, unit = n * k / 4 / per / 1e9, "GB/s"
            else:
                v, unit = 2.0 * m * n * k / per / 1e9, "GOPS"
            out["settings"].append(dict(workload=f"{name} M={m} K={k} N={n}", threads=th, value=round(v, 4), unit=unit,
                                        sample=f"{reps} calls on {toks} of {m} tokens (all {n} output rows) in "
                                               f"{dt:.1f} s, scaled by {m / toks:.0f}"))
    # one layer of the 70B-class chain, scaled by its 80 layers
    layer = []
    for p, (_, k, n) in enumerate(workloads.W5_PROJ):
        layer.append((k, workloads.stream_packed_rows(0, p, k, np.arange(n), threads=P),
                      workloads.stream_alpha(0, p), workloads.stream_activation(0, p, k)))
    layer_bytes = sum(pk.nbytes for _, pk, _, _ in layer)

    def chain_layer(pool, threads):
        for (k, pk, alpha, x) in layer:
            xq, beta = oracle.quantize_act(x)
            forward_rows(pool, threads, xq, beta, pk, k, alpha, 0, pk.shape[0])
    reps, dt = timed(chain_layer, P, 0.0)
    per_token = dt / reps * workloads.W5_LAYERS
    out["settings"].append(dict(workload="chain70b (80 layers x 7 projections, M=1)", threads=P,
                                value=round(layer_bytes * workloads.W5_LAYERS / per_token / 1e9, 4), unit="GB/s",
                                tokens_per_s=round(1.0 / per_token, 5),
                                sample=f"{reps} pass of layer 0 ({layer_bytes} B of codes) in {dt:.1f} s, scaled by 80"))
    dec = [st for st in out["settings"] if st["workload"] == "decode" and st["threads"] == P][0]
    out.update(value=dec["value"], unit="GB/s", cores=P, kind="oracle",
               sample=f"whole 7B decode steps (M=1; K,N = 4096x4096, 4096x11008, 11008x4096), {dec['sample']}, "
                      f"output rows split over {P} threads (the physical cores available, at most {max_threads}); "
                      f"the 1-thread figure and the batched, prefill and 70B-chain samples are in settings")
    return out


def kernel_only(kind: str, launches: int, batched_shape=(64, 4096, 11008)):
    """Run only one kernel, `launches` times, for counter collection under rocprofv3:
    gemv_fused = the roofline kernel (decode GEMV, K=4096, N=11008, weights rotating through
    64 copies so every launch reads HBM); copy = a plain 256 MiB device copy (calibrates
    FETCH_SIZE / WRITE_SIZE); gemm = the prefill GEMM (M=2048, K=4096, N=11008); batched =
    the batched decode kernel at `batched_shape` (M, K, N; by default M=64, K=4096, N=11008),
    weights rotating through 32 copies."""
    import torch
    import bitlinear_matmul_absmean_amd as bl
    import workloads
    dev = torch.device("cuda:0")
    if kind == "copy":
        nbytes = 256 << 20
        a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(launches):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy: {launches} x {nbytes} B")
        return
    if kind == "gemv_fused":
        k, n = DECODE_SHAPES[1]
        w = torch.from_numpy(workloads.weights(2, n, k, index=1)).to(dev)
        packed, alpha = bl.bitlinear_quantize_weights(w)
        del w
        pool = [packed] + [packed.clone() for _ in range(63)]
        x = torch.from_numpy(workloads.activations(2, 1, k, index=100)).to(dev)
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for i in range(launches):
            bl.bitlinear_forward_fused(x, pool[i % len(pool)], alpha, y=y)
        torch.cuda.synchronize()
        log(f"gemv_fused: {launches} launches of {bl.bitlinear_forward_fused_kernel(1, k, n, x, packed)}")
        return
    if kind == "gemv_fused_graph":
        # the roofline measurement itself: the same pool and graph as roofline_gemv
        shapes, _, copies = decode_setup(torch, bl, workloads, dev)
        roof = roofline_gemv(torch, bl, shapes[1], copies, reps=launches)
        log(f"gemv_fused_graph: {launches} launches in one graph, {roof['us_per_launch']} us per launch "
            f"(events, launch to launch), {roof['achieved']} GB/s")
        print(json.dumps(roof), flush=True)
        return
    if kind == "batched":
        m, k, n = batched_shape
        w = torch.from_numpy(workloads.weights(3, n, k)).to(dev)
        packed, alpha = bl.bitlinear_quantize_weights(w)
        del w
        pool = [packed] + [packed.clone() for _ in range(31)]
        x = torch.from_numpy(workloads.activations(3, m, k)).to(dev)
        xq, beta = bl.bitlinear_quantize_act(x)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for i in range(launches):
            bl.bitlinear_forward(xq, beta, pool[i % len(pool)], alpha, y=y)
        torch.cuda.synchronize()
        log(f"batched: {launches} launches of {bl.bitlinear_forward_kernel(m, k, n, xq, packed)}")
        return
    if kind == "gemm":
        m, k, n = 2048, 4096, 11008
        w = torch.from_numpy(workloads.weights(4, n, k)).to(dev)
        packed, alpha = bl.bitlinear_quantize_weights(w)
        del w
        x = torch.from_numpy(workloads.activations_with_outliers(4, m, k)).to(dev)
        xq, beta = bl.bitlinear_quantize_act(x)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for _ in range(launches):
            bl.bitlinear_forward(xq, beta, packed, alpha, y=y)
        torch.cuda.synchronize()
        log(f"gemm: {launches} launches")
        return
    raise SystemExit(f"unknown --kernel-only {kind}")


def trace_summary(trace_dir: str, plain_json: str, traced_json: str, commands: str):
    """Markdown summary of `--kernel-only gemv_fused_graph` run without and with
    `rocprofv3 --kernel-trace`: the roofline kernel's launches in the trace are, in order, the
    three eager warm-up calls of the graph timer, the untimed replay, the timed replay (L
    launches each) and the 50 single calls; the timed replay's launch-to-launch time from the
    trace is set against the events of the same traced run."""
    import csv
    import glob
    import statistics
    plain = json.loads(open(plain_json).read().strip().splitlines()[-1])
    traced = json.loads(open(traced_json).read().strip().splitlines()[-1])
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    name = next(r["Kernel_Name"] for r in rows if r["Kernel_Name"].startswith("void bitlinear::k_gemv<")
                and ", true, " in r["Kernel_Name"])
    ts = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows if r["Kernel_Name"] == name)
    # in order: 3 eager warm-up calls, 1 untimed replay and `trials` timed replays of L launches,
    # then the 50 single calls
    L = int(traced["graph_launches"])
    trials = int(traced["graph_trials"])
    assert len(ts) == 3 + L * (1 + trials) + 50, (len(ts), L, trials)
    timed = ts[3 + L:3 + L * (1 + trials)]
    span = (timed[-1][1] - timed[0][0]) / len(timed) / 1e3
    dur = [e - b for b, e in timed]
    out = ["# Roofline kernel: event timing against the kernel trace (fused decode GEMV, M=1, K=4096, N=11008)", "",
           "Commands (repository root, one MI355X):", "", "```"] + [c.strip() for c in commands.split(";")] + [
           "```", "",
           f"Kernel: `{name}`; {L} launches in one graph, replayed {trials} times, weights rotating "
           "through the decode pool.", "",
           "| run | per launch, events (bench.py) | per launch, trace (first start to last end / launches) "
           "| kernel duration in the trace (mean / median / min) |", "|---|---|---|---|",
           f"| without the tracer | {plain['us_per_launch']} us ({plain['achieved']} GB/s) | - | - |",
           f"| with `--kernel-trace` | {traced['us_per_launch']} us | {span:.2f} us "
           f"| {statistics.mean(dur) / 1e3:.2f} / {statistics.median(dur) / 1e3:.2f} / {min(dur) / 1e3:.2f} us |", "",
           "In the traced run the events and the trace agree on the time per launch; the kernel's own",
           "duration is shorter by the dispatch gap between launches.  The tracer itself lengthens every",
           "launch (compare the two event figures), so bench.py's live roofline figure comes from the run",
           "without it; bench.py also reports the fraction of the HBM peak that the trace's mean kernel",
           "duration gives (`roofline.kernel_trace`), read from the fields below while the kernel's",
           "sources still hash to `source_sha256`.", "",
           f"- kernel: `{name}`",
           f"- source_sha256: `{kernel_source_sha()}`",
           f"- launches_timed: {len(timed)} ({trials} replays of {L})",
           f"- kernel_duration_mean_us: {statistics.mean(dur) / 1e3:.3f}",
           f"- kernel_duration_median_us: {statistics.median(dur) / 1e3:.3f}",
           f"- kernel_duration_min_us: {min(dur) / 1e3:.3f}",
           f"- traced_launch_to_launch_us: {span:.3f}",
           f"- untraced_events_us_per_launch: {plain['us_per_launch']}",
           f"- traced_events_us_per_launch: {traced['us_per_launch']}", ""]
    print("\n".join(out))


def _pmc_means(d: str):
    """{kernel name: {counter: mean value per dispatch}} from a rocprofv3 --pmc csv directory."""
    import csv
    import glob
    from collections import defaultdict
    acc = defaultdict(lambda: defaultdict(list))
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} | {"_n": max(len(v) for v in cs.values())}
            for k, cs in acc.items()}


def pmc_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, commands):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, for the roofline kernel and
    for the 256 MiB calibration copy) into the traffic summary kept under profiles/."""
    def pick(means, key, counter):
        cands = [(v["_n"], k, v[counter]) for k, v in means.items() if key in k and counter in v]
        if not cands:
            raise SystemExit(f"no kernel matching {key!r} with {counter} in the counter runs")
        return max(cands)
    nbytes = 256 << 20
    _, gname, fetch_kib = pick(_pmc_means(fetch_dir), "k_gemv", "FETCH_SIZE")
    _, _, write_kib = pick(_pmc_means(write_dir), "k_gemv", "WRITE_SIZE")
    _, cname, cfetch_kib = pick(_pmc_means(cfetch_dir), "copy", "FETCH_SIZE")
    _, _, cwrite_kib = pick(_pmc_means(cwrite_dir), "copy", "WRITE_SIZE")
    ff = nbytes / (cfetch_kib * 1024.0)
    fw = nbytes / (cwrite_kib * 1024.0)
    k, n = DECODE_SHAPES[1]
    alg = n * k // 4 + 4 * k + 4 + 4 * n
    hbm = fetch_kib * 1024.0 * ff + write_kib * 1024.0 * fw
    out = ["# HBM traffic of the decode GEMV (fused, M=1, K=4096, N=11008), from rocprofv3 counters", "",
           "Commands (repository root, one MI355X):", "", "```"] + commands + ["```", "",
           "FETCH_SIZE and WRITE_SIZE are read per dispatch in KiB and scaled by what they read for a "
           f"plain device copy of {nbytes} bytes (`{cname}`): the copy fetches and writes exactly that many "
           "bytes, so factor = bytes / (counter KiB * 1024).", "",
           f"- kernel: `{gname}`",
           f"- source_sha256: `{kernel_source_sha()}`",
           f"- fetch_kib_per_launch: {fetch_kib:.1f}",
           f"- write_kib_per_launch: {write_kib:.1f}",
           f"- copy_fetch_kib: {cfetch_kib:.1f}",
           f"- copy_write_kib: {cwrite_kib:.1f}",
           f"- fetch_factor: {ff:.4f}",
           f"- write_factor: {fw:.4f}",
           f"- hbm_bytes_per_launch: {hbm:.0f}",
           f"- algorithmic_bytes_per_launch: {alg}",
           f"- traffic_over_algorithmic: {hbm / alg:.4f}", ""]
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="headline workload and roofline only")
    ap.add_argument("--no-chain", action="store_true", help="skip the 70B-class chain")
    ap.add_argument("--kernel-only", choices=["gemv_fused", "gemv_fused_graph", "copy", "gemm", "batched"],
                    help="run only this kernel (for rocprofv3 counter runs)")
    ap.add_argument("--launches", type=int, default=50)
    ap.add_argument("--batched-shape", type=int, nargs=3, default=[64, 4096, 11008], metavar=("M", "K", "N"),
                    help="shape of --kernel-only batched")
    ap.add_argument("--trace-summary", nargs=3, metavar=("TRACE_DIR", "PLAIN_JSON", "TRACED_JSON"),
                    help="summarise the roofline kernel's trace against its event timing")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("GEMV_FETCH", "GEMV_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the traffic summary from four rocprofv3 --pmc output directories")
    ap.add_argument("--pmc-commands", default="", help="';'-separated commands recorded in the summary")
    args = ap.parse_args()
    if args.pmc_summary:
        print(pmc_summary(*args.pmc_summary, [c.strip() for c in args.pmc_commands.split(";") if c.strip()]))
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary, args.pmc_commands)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.kernel_only:
        kernel_only(args.kernel_only, args.launches, tuple(args.batched_shape))
        return

    import torch
    import bitlinear_matmul_absmean_amd as bl
    import workloads

    dev = torch.device("cuda:0")
    log(f"device {torch.cuda.get_device_name(0)}; building decode pools")
    shapes, per_step, copies = decode_setup(torch, bl, workloads, dev)
    log(f"pool: {copies} copies x {per_step} B")

    # warmup (untimed), then exactly K steps in one graph
    wms, _ = _graph_time(torch, lambda i: decode_step(bl, shapes, copies, i), max(1, args.warmup))
    torch.cuda.synchronize()
    ms_step, g = _graph_time(torch, lambda i: decode_step(bl, shapes, copies, i), args.steps)
    value = per_step / (ms_step * 1e-3) / 1e9
    log(f"decode step {ms_step * 1e3:.2f} us -> {value:.1f} GB/s")
    ms_two, _ = _graph_time(torch, lambda i: decode_step_two_call(bl, shapes, copies, i), args.steps)
    log(f"decode step, two-call ABI {ms_two * 1e3:.2f} us")
    ms_eager = _eager_time(torch, lambda i: decode_step(bl, shapes, copies, i), args.steps)
    log(f"decode step, eager launches {ms_eager * 1e3:.2f} us")

    roof = roofline_gemv(torch, bl, shapes[1], copies)
    log(f"roofline {roof}")
    del shapes
    torch.cuda.empty_cache()
    extras = {}
    if not args.no_extras:
        extras["prefill"] = prefill_bench(torch, bl, workloads, dev)
        log(f"prefill {extras['prefill']}")
        extras["prefill_n4096"] = prefill_bench(torch, bl, workloads, dev, n=4096)
        log(f"prefill_n4096 {extras['prefill_n4096']}")
        extras["batched"] = batched_bench(torch, bl, workloads, dev)
        log(f"batched {extras['batched']}")
        extras.update(quantize_bench(torch, bl, workloads, dev))
        log(f"quantize_weights {extras['quantize_weights']}")
        log(f"quantize_act {extras['quantize_act']}")
        extras["hadamard"] = hadamard_bench(torch, bl, workloads, dev, ms_step)
        log(f"hadamard {extras['hadamard']}")
        extras["blocks"] = blocks_bench(torch, bl, workloads, dev, ms_step)
        log(f"blocks {extras['blocks']}")
        extras["mlp"] = mlp_bench(torch, bl, workloads, dev)
        log(f"mlp {extras['mlp']}")
        extras["t5"] = t5_bench(torch, bl, workloads, dev)
        log(f"t5 {extras['t5']}")
    if not args.no_extras and not args.no_chain:
        extras["chain70b"] = chain70b_bench(torch, bl, workloads, dev)
        log(f"chain70b {extras['chain70b']}")
    # measured ceilings last: the MFMA loop heats the chip, which would slow what follows it
    ceil = ceilings(torch, dev, [roof["bytes_per_launch"], 1 << 30])
    log(f"ceilings {ceil}")
    read_ceiling = list(ceil["hbm_read_gbs"].values())[0]
    roof["measured_ceiling"] = {"gbs": read_ceiling, "what": "streaming read of the same byte count, same timing",
                                "frac": round(roof["achieved"] / read_ceiling, 4)}
    for key in ("prefill", "prefill_n4096"):
        if key in extras:
            extras[key]["pct_measured_mfma_random"] = round(
                100 * extras[key]["tops"] / ceil["mfma_i8_tops"]["random"], 2)
    cpu = None if args.no_cpu else cpu_baseline(workloads)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "7B-class decode GEMV, M=1: fused quantize_act + forward on (K,N) = "
                               "(4096,4096), (4096,11008), (11008,4096); W ~ N(0,0.02) ternarized, 2-bit packed; "
                               "x ~ N(0,1)", "M": 1, "shapes_KN": DECODE_SHAPES,
                   "weight_bytes_per_step": per_step, "rotation_copies": copies, "timing": "one HIP graph of K steps"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_two_call": {"us_per_step": round(ms_two * 1e3, 2),
                            "weight_gbs": round(per_step / (ms_two * 1e-3) / 1e9, 1)},
        "decode_eager": {"us_per_step": round(ms_eager * 1e3, 2),
                         "weight_gbs": round(per_step / (ms_eager * 1e-3) / 1e9, 1),
                         "what": "the same steps launched without a graph (host launch rate included)"},
        "roofline": roof,
        "ceilings": ceil,
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
