#!/usr/bin/env python3
"""Throughput of the convolution hot path on one MI355X.

A step is one forward convolution through the C ABI (implicit-GEMM kernel:
padded-window gather, LDS staging, fp32 MFMA, split reduction, epilogue,
store) on the 1x512x7x7 -> 512, 3x3, stride 1, pad 1 fp32 layer (the final
ResNet layer of the TVM tutorial's tuning example), with seeded synthetic
inputs already resident in HBM.  In the default mode the K steps are
dispatched once, into a HIP graph, and the timed region is the graph's
replay: the device time of K back-to-back launches, host dispatch excluded.
`eager_ms_per_step` times the same K steps dispatched one by one from the
host through the C ABI (host dispatch included).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--eager]
                    [--tune] [--cache PATH | --no-cache] [--no-cpu-baseline]
                    [--prepared] [--no-per-shape] [--calibrate-copy]

The tile config comes from the tuning log shipped with the package (the
search's recorded winners, loaded with ct_cache_load) unless --no-cache or
--tune is given.  K steps are captured in one HIP graph and replayed
(default) or launched eagerly (--eager); HIP events on the launch stream
bracket the K steps.
With no --workload the line also carries `per_shape`: every other row of
the workload table (the batch-1 fp32 layers, both half-precision layers with
the filter reordered per call and prepared once, the standalone broadcast in
fp16 and fp32, the two matrix products, the three depthwise layers and the
batch-norm chain), each timed the same way.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}  # dense matrix peaks, MI355X
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "tensor_compiler_tiling_amd", "csrc")
DEFAULT_CACHE = os.path.join(ROOT, "tensor_compiler_tiling_amd", "tuned", "gfx950.jsonl")
TRAFFIC_LOG = os.path.join(ROOT, "profiles", "traffic.json")
_SHARED_SRC = ["ct_kernels.hpp", "ct_device.hpp", "igemm_common.hpp"]


def kernel_sources(kernel: str):
    """The source files a kernel (variant name, or "broadcast") is built from."""
    if kernel == "broadcast":
        main = "broadcast.hip"
    elif kernel == "depthwise":
        return ["conv_depthwise.hip", "ct_device.hpp"]
    elif kernel == "chain":
        return ["broadcast_chain.hip", "ct_device.hpp"]
    elif kernel.startswith("f32skc"):
        main = "igemm_f32_skc.hip"
    elif kernel.startswith("f32skt"):
        main = "igemm_f32_skt.hip"
    elif kernel.startswith("f32sk16"):
        main = "igemm_f32_sk16.hip"
    elif kernel.startswith(("f32sk_", "f32skx_")):
        main = "igemm_f32_sk.hip"
    elif kernel.startswith(("hgf16_", "hgbf16_")):
        main = "igemm_f16_gemm.hip"
    elif kernel.startswith("f32g_"):
        main = "igemm_f32_gemm.hip"
    elif kernel.startswith("f32_"):
        main = "igemm_f32.hip"
    elif kernel.startswith(("h2f16_", "h2bf16_")):
        main = "igemm_f16v2.hip"
    elif kernel.startswith(("f16_", "bf16_")):
        main = "igemm_f16.hip"
    else:
        main = "conv_direct.hip"
    return [main] + _SHARED_SRC


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in kernel_sources(kernel):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str, cfg: dict, prepared: bool = False):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE passes
    recorded for this workload, or None when no record matches the kernel
    source, tile config and filter form (reordered per call, or prepared) as
    they are now."""
    try:
        with open(TRAFFIC_LOG) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    digest = source_digest(kernel)
    for r in recs:
        if (r.get("workload") == workload and r.get("kernel") == kernel
                and r.get("source_sha256") == digest and r.get("tile", {}) == cfg
                and (r.get("filter") == "prepared") == prepared):
            return r.get("traffic_bytes_per_launch")
    return None


def calibrate_copy(mib: int = 1024, reps: int = 3) -> None:
    """Plain device-to-device copies of a known size: the reference dispatches
    that scale the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def host_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--eager", action="store_true", help="time eager launches, not a graph")
    ap.add_argument("--tune", action="store_true", help="run the tile-config search first")
    ap.add_argument("--tune-trials", type=int, default=0)
    ap.add_argument("--tune-ms", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prepared", action="store_true",
                    help="half-precision convolution: time the prepared-filter entry point")
    ap.add_argument("--no-per-shape", action="store_true",
                    help="default workload only: leave out the per-shape list of the other rows")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cache", default=DEFAULT_CACHE,
                    help="tuning log (JSON lines) to load before dispatch")
    ap.add_argument("--no-cache", action="store_true", help="do not load a tuning log")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run 1 GiB copies (reference dispatches for the HBM counters)")
    return ap.parse_args()


def _ensure_built():
    from tensor_compiler_tiling_amd import convtile as ct
    if not os.path.exists(ct.LIB_PATH):
        from tensor_compiler_tiling_amd import build
        build.build()


def cpu_baseline(w, seconds: float) -> dict:
    """The fp64 oracle as it stands, on this host's cores, on the same
    workload (whole passes, repeated until about `seconds` have elapsed)."""
    from oracle import oracle as O
    from tensor_compiler_tiling_amd import workloads as wl
    inp = wl.conv_inputs(w)
    x = inp["x"].astype(np.float64)
    k = inp["w"].astype(np.float64)
    cores = host_threads()
    if w.flops > 4e9:
        # a whole pass would take minutes: time the oracle's one-output-at-a-
        # time routine on random outputs instead, doubling the sample until
        # about `seconds` have elapsed
        per_point = 2 * w.CI * w.KH * w.KW
        r = np.random.default_rng(0)
        npts, el = 1024, 0.0
        while True:
            idx = np.stack([r.integers(0, d, npts) for d in (w.N, w.CO, w.OH, w.OW)], axis=1)
            t0 = time.perf_counter()
            O.conv2d_points(x, k, w.stride, w.pad, idx.astype(np.int64))
            el = time.perf_counter() - t0
            if el >= seconds / 2 or npts >= 1 << 26:
                break
            npts *= 2
        return {"value": round(per_point * npts / el / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
                "kind": "oracle",
                "sample": f"{npts} random outputs of {w.name} ({per_point} FLOP each) through the "
                          f"fp64 oracle's per-output routine in {el:.1f} s"}
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.conv2d_nchw(x, k, w.stride, w.pad)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    tflops = w.flops * reps / el / 1e12
    return {"value": round(tflops, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} full passes of the fp64 seven-loop oracle (OpenMP over n, f) "
                      f"on {w.name} in {el:.1f} s"}


def cpu_baseline_gemm(g, seconds: float) -> dict:
    """The fp64 matrix-product oracle on this host's cores, whole products of
    the same workload repeated until about `seconds` have elapsed."""
    from oracle import oracle as O
    from tensor_compiler_tiling_amd import workloads as wl
    inp = wl.gemm_inputs(g)
    A = inp["A"].astype(np.float64)
    B = inp["B"].astype(np.float64)
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.gemm(A, B)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # the oracle also forms sum |A||B| (a second product): count both
    return {"value": round(2 * g.flops * reps / el / 1e12, 5), "unit": "TFLOP/s",
            "cores": host_threads(), "kind": "oracle",
            "sample": f"{reps} full fp64 products (C and its |A||B| scale) of {g.name} in {el:.1f} s"}


def cpu_baseline_broadcast(bw, seconds: float) -> dict:
    """The fp64 oracle broadcast on this host, repeated for about `seconds`;
    reported as bytes of the output dtype written per second."""
    from oracle import oracle as O
    from tensor_compiler_tiling_amd import workloads as wl
    var = wl.broadcast_var(bw)
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.broadcast_exp(var, bw.N, bw.H, bw.W)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(bw.bytes_written() * reps / el / 1e9, 3), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{reps} full [1,{bw.C},1,1]->[{bw.N},{bw.C},{bw.H},{bw.W}] fp64 "
                      f"oracle passes in {el:.1f} s, counted at {bw.out_dtype} output bytes"}


def bench_broadcast(a, name: str) -> dict:
    """[1,C,1,1] -> [N,C,H,W] of exp(var[c]): channel-bound form timed, the
    flat (per-element) form timed beside it.  Outputs rotate over enough
    buffers that the written bytes exceed the 256 MB last-level cache."""
    import torch
    from tensor_compiler_tiling_amd import convtile as ct
    from tensor_compiler_tiling_amd import workloads as wl
    bw = wl.BROADCAST_WORKLOADS[name]
    dev = torch.device("cuda:0")
    dt = torch.float16 if bw.out_dtype == wl.F16 else torch.float32
    var = torch.from_numpy(wl.broadcast_var(bw)).to(dev)
    nbytes = bw.bytes_written()
    nbuf = max(2, -(-300 * 2 ** 20 // nbytes))
    outs = [torch.empty((bw.N, bw.C, bw.H, bw.W), dtype=dt, device=dev) for _ in range(nbuf)]
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    lib = ct.library()
    code = ct.dtype_code(dt)

    def run(mode, i):
        st = lib.ct_broadcast_nchw(var.data_ptr(), outs[i % nbuf].data_ptr(), bw.N, bw.C, bw.H,
                                   bw.W, code, ct.CT_BC_EXP, mode,
                                   torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise ct.ConvTileError(st, "broadcast")

    res = {}
    for mode, label in ((ct.CT_BC_CHANNEL, "channel"), (ct.CT_BC_FLAT, "flat")):
        for i in range(a.warmup):
            run(mode, i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(a.steps):
                run(mode, i)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / a.steps
        res[label] = {"ms_per_step": round(ms, 6), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    gbs = res["channel"]["GB/s"]
    traffic = measured_traffic(name, "broadcast", {"mode": "channel"})
    out = {
        "metric": "per-channel broadcast [1,C,1,1]->[N,C,H,W] of exp(var[c]), HBM GB/s",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": res["channel"]["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": bw.out_dtype,
        "data": "synthetic (seeded var ~ U[0.5, 2])",
        "config": {"workload": name, "N": bw.N, "C": bw.C, "H": bw.H, "W": bw.W,
                   "bytes_written_per_step": nbytes, "rotating_buffers": nbuf,
                   "launch": "hip_graph"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic},
        "flat_form": res["flat"],
        "speedup_channel_vs_flat": round(res["flat"]["ms_per_step"] / res["channel"]["ms_per_step"], 3),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_broadcast(bw, a.cpu_seconds)
    return out


def cpu_baseline_depthwise(d, seconds: float) -> dict:
    """The fp64 oracle depthwise convolution on this host, on a slice of the
    batch repeated for about `seconds`; reported as the layer's algorithmic
    bytes per second, scaled to the slice."""
    from oracle import oracle as O
    from tensor_compiler_tiling_amd import workloads as wl
    inp = wl.depthwise_inputs(d)
    nb = max(1, min(d.N, 8))
    x = inp["x"][:nb].astype(np.float64)
    w = inp["w"].astype(np.float64)
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.conv2d_depthwise(x, w, d.stride, d.pad)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(d.algorithmic_bytes() * nb / d.N * reps / el / 1e9, 3), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{reps} fp64 oracle passes (y and its |x*w| scale) over {nb} of {d.N} images "
                      f"of {d.name} in {el:.1f} s, counted at the layer's algorithmic bytes"}


def bench_depthwise(a, name: str) -> dict:
    """Depthwise convolution: K launches captured in one HIP graph; inputs and
    outputs rotate over enough buffer sets that each step's bytes come from
    HBM, not from the 256 MB last-level cache."""
    import torch
    from tensor_compiler_tiling_amd import convtile as ct
    from tensor_compiler_tiling_amd import workloads as wl
    d = wl.DEPTHWISE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[d.dtype]
    inp = wl.depthwise_inputs(d)
    nbytes = d.algorithmic_bytes()
    nbuf = max(2, -(-300 * 2 ** 20 // nbytes))
    xs = [torch.from_numpy(inp["x"]).to(dev).to(tdt) for _ in range(nbuf)]
    k = torch.from_numpy(inp["w"]).to(dev).to(tdt)
    b = torch.from_numpy(inp["bias"]).to(dev)
    v = torch.from_numpy(inp["var"]).to(dev)
    ys = [torch.empty((d.N, d.C, d.OH, d.OW), dtype=torch.float32, device=dev) for _ in range(nbuf)]
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    lib = ct.library()
    dt = ct.dtype_code(tdt)

    def step(i):
        st = lib.ct_conv2d_nchw_depthwise(xs[i % nbuf].data_ptr(), k.data_ptr(), ys[i % nbuf].data_ptr(),
                                          d.N, d.C, d.H, d.W, d.KH, d.KW, d.stride, d.pad, dt,
                                          d.epilogue, b.data_ptr(), v.data_ptr(), 1e-5,
                                          torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise ct.ConvTileError(st, "depthwise")

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    if a.eager:
        e0.record(stream)
        for i in range(a.steps):
            step(i)
        e1.record(stream)
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(a.steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / a.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "depthwise convolution, HBM GB/s of algorithmic bytes (x, w read once, y written once)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": d.dtype,
        "data": "synthetic (seeded: x ~ U[-1, 1], w He-normal over KH*KW, bias ~ N(0, 0.1))",
        "config": {"workload": name, "N": d.N, "C": d.C, "H": d.H, "W": d.W, "KH": d.KH, "KW": d.KW,
                   "stride": d.stride, "pad": d.pad, "epilogue": d.epilogue,
                   "algorithmic_bytes_per_step": nbytes, "rotating_buffers": nbuf,
                   "launch": "eager" if a.eager else "hip_graph"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(name, "depthwise", {})},
        "gflops": round(d.flops / (ms * 1e-3) / 1e9, 1),
        "wall_s": round(wall, 4),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_depthwise(d, a.cpu_seconds)
    return out


def cpu_baseline_chain(cw, seconds: float) -> dict:
    """The fp64 oracle's chain evaluation on this host, on whole passes of the
    workload for about `seconds`, as algorithmic bytes per second."""
    from oracle import oracle as O
    from tensor_compiler_tiling_amd import workloads as wl
    inp = wl.chain_inputs(cw)
    x = inp["x"].astype(np.float64)
    arrays = [v.astype(np.float64) for v in inp["arrays"]]
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.broadcast_chain(wl.CHAIN_PROGRAMS[cw.program], cw.outer, cw.P, cw.inner, arrays, x)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(cw.algorithmic_bytes() * reps / el / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": f"{reps} full fp64 oracle passes of {cw.name} in {el:.1f} s, counted "
                                        f"at the workload's algorithmic bytes"}


def bench_chain(a, name: str) -> dict:
    """The general per-channel broadcast: the channel-bound form timed (K
    launches in one HIP graph), the flat form timed beside it; inputs and
    outputs rotate over enough buffers to exceed the last-level cache."""
    import torch
    from tensor_compiler_tiling_amd import convtile as ct
    from tensor_compiler_tiling_amd import workloads as wl
    cw = wl.CHAIN_WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = wl.chain_inputs(cw)
    nbytes = cw.algorithmic_bytes()
    nbuf = max(2, -(-300 * 2 ** 20 // nbytes))
    odt = torch.float32 if cw.out_dtype == wl.F32 else torch.float16
    xs = [torch.from_numpy(inp["x"]).to(dev) for _ in range(nbuf)]
    outs = [torch.empty((cw.outer, cw.P, cw.inner), dtype=odt, device=dev) for _ in range(nbuf)]
    arrays = [torch.from_numpy(v).to(dev) for v in inp["arrays"]]
    prog = ct.make_program(*wl.CHAIN_PROGRAMS[cw.program])
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    lib = ct.library()
    code = ct.dtype_code(odt)
    ap = [t.data_ptr() for t in arrays]

    def run(mode, i):
        st = lib.ct_broadcast_chain(ct.ctypes.byref(prog), ap[0], ap[1], ap[2], ap[3], xs[i % nbuf].data_ptr(),
                                    outs[i % nbuf].data_ptr(), code, cw.outer, cw.P, cw.inner, mode,
                                    torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise ct.ConvTileError(st, "broadcast_chain")

    res = {}
    for mode, label in ((ct.CT_BC_CHANNEL, "channel"), (ct.CT_BC_FLAT, "flat")):
        for i in range(a.warmup):
            run(mode, i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(a.steps):
                run(mode, i)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / a.steps
        res[label] = {"ms_per_step": round(ms, 6), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    gbs = res["channel"]["GB/s"]
    out = {
        "metric": "general per-channel broadcast [1,P,1]=>[B,P,B] with a step chain, HBM GB/s of algorithmic bytes",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": res["channel"]["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cw.out_dtype,
        "data": "synthetic (seeded x ~ U[-1, 1]; var, gamma, mean, beta per channel)",
        "config": {"workload": name, "outer": cw.outer, "P": cw.P, "inner": cw.inner, "program": cw.program,
                   "algorithmic_bytes_per_step": nbytes, "rotating_buffers": nbuf, "launch": "hip_graph"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(name, "chain", {})},
        "flat_form": res["flat"],
        "speedup_channel_vs_flat": round(res["flat"]["ms_per_step"] / res["channel"]["ms_per_step"], 3),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_chain(cw, a.cpu_seconds)
    return out


def time_graph(step, stream, steps: int, warmup: int) -> float:
    """Mean ms per step of `steps` calls of step() captured in one HIP graph
    and replayed, timed with HIP events on `stream` (after `warmup` eager
    calls and one untimed replay)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(steps):
            step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / steps


def conv_step(w, prepared: bool = False, stream_handle=None):
    """(step, config) for one convolution of workload w through the C ABI, on
    the stream `stream_handle` (default: the current stream at call time);
    inputs resident on the GPU, their addresses bound once so that a step
    costs the host little beyond the call itself."""
    import torch
    from tensor_compiler_tiling_amd import convtile as ct
    from tensor_compiler_tiling_amd import workloads as wl
    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    inp = wl.conv_inputs(w)
    x = torch.from_numpy(inp["x"]).to(dev).to(tdt)
    k = torch.from_numpy(inp["w"]).to(dev).to(tdt)
    b = torch.from_numpy(inp["bias"]).to(dev)
    v = torch.from_numpy(inp["var"]).to(dev)
    y = torch.empty((w.N, w.CO, w.OH, w.OW), dtype=torch.float32, device=dev)
    dt = ct.dtype_code(tdt)
    args = w.shape_args() + (dt, w.epilogue)
    lib = ct.library()
    if prepared:
        k = ct.prepare_filter(k)
    fn = lib.ct_conv2d_nchw_fwd_prepared if prepared else lib.ct_conv2d_nchw_fwd
    keep = (x, k, b, v, y)  # owners of the bound addresses
    head = (x.data_ptr(), k.data_ptr(), y.data_ptr()) + args
    tail = (b.data_ptr(), v.data_ptr(), 1e-5)

    def step():
        h = stream_handle if stream_handle is not None else torch.cuda.current_stream().cuda_stream
        st = fn(*head, *tail, h)
        if st != 0:
            raise ct.ConvTileError(st, "fwd")
    step.keep = keep

    st, cfg, from_cache = ct.ct_conv2d_query(*args)
    ct.check(st, "query")
    return step, cfg, from_cache


def per_shape(a) -> list:
    """Every other row of the workload table, each timed the way the headline
    is (a HIP graph of back-to-back launches, HIP events on its stream): the
    batch-1 fp32 layers, both half-precision layers (the filter reordered per
    call, and prepared once), the standalone broadcast in fp16 and fp32, the
    matrix products, the depthwise layers and the batch-norm chain."""
    import torch
    from tensor_compiler_tiling_amd import convtile as ct
    from tensor_compiler_tiling_amd import workloads as wl
    steps = max(a.steps, 100)
    out = []
    names = ["resnet_c64_14x14_k3"] + wl.SWEEP + ["f16_n64_c256_14x14_k3", "f16_n128_c128to256_32x32_k3_epi"]
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    for name in names:
        w = wl.CONV_WORKLOADS[name]
        peak = PEAK_TFLOPS[w.dtype]
        for prepared in ((False, True) if w.dtype != "f32" else (False,)):
            step, cfg, _ = conv_step(w, prepared, stream.cuda_stream)
            ms = time_graph(step, stream, steps, a.warmup)
            tf = w.flops / (ms * 1e-3) / 1e12
            vname = ct.variants()[cfg.variant]["name"]
            tile = {"split_k": cfg.split_k, "stages": cfg.stages, "kc": cfg.kc}
            out.append({"workload": name + (" (prepared filter)" if prepared else ""), "dtype": w.dtype,
                        "us": round(ms * 1e3, 3), "TFLOP/s": round(tf, 2), "bound": "mfma",
                        "frac": round(tf / peak, 4), "kernel": vname, "tile": tile,
                        "traffic": measured_traffic(name, vname, tile, prepared)})
    for name in ("bcast_exp_128x256x32x32_f16", "bcast_exp_128x256x32x32_f32"):
        bw = wl.BROADCAST_WORKLOADS[name]
        dt = torch.float16 if bw.out_dtype == wl.F16 else torch.float32
        var = torch.from_numpy(wl.broadcast_var(bw)).to("cuda:0")
        nbytes = bw.bytes_written()
        nbuf = max(2, -(-300 * 2 ** 20 // nbytes))
        outs = [torch.empty((bw.N, bw.C, bw.H, bw.W), dtype=dt, device="cuda:0") for _ in range(nbuf)]
        lib = ct.library()
        code = ct.dtype_code(dt)
        it = [0]

        def bstep():
            i = it[0] = it[0] + 1
            st = lib.ct_broadcast_nchw(var.data_ptr(), outs[i % nbuf].data_ptr(), bw.N, bw.C, bw.H, bw.W, code,
                                       ct.CT_BC_EXP, ct.CT_BC_CHANNEL, torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise ct.ConvTileError(st, "broadcast")

        ms = time_graph(bstep, stream, steps, a.warmup)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out.append({"workload": name, "dtype": bw.out_dtype, "us": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                    "bound": "hbm", "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": "bcast_channel",
                    "rotating_buffers": nbuf,
                    "traffic": measured_traffic(name, "broadcast", {"mode": "channel"})})
        del outs
        torch.cuda.empty_cache()
    # the matrix products, through ct_gemm_fwd with the tuned config (their
    # 1x1 convolution views give the seeded operands)
    dev = torch.device("cuda:0")
    for name, g in wl.GEMM_WORKLOADS.items():
        w = g.conv_view()
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        dt = ct.dtype_code(tdt)
        inp = wl.conv_inputs(w)
        xg = torch.from_numpy(inp["x"]).to(dev).to(tdt)
        kg = torch.from_numpy(inp["w"]).to(dev).to(tdt)
        bg = torch.from_numpy(inp["bias"]).to(dev)
        vg = torch.from_numpy(inp["var"]).to(dev)
        yg = torch.empty((w.N, w.CO, w.OH, w.OW), dtype=torch.float32, device=dev)
        lib = ct.library()
        gargs = (kg.data_ptr(), xg.data_ptr(), yg.data_ptr(), g.M, g.N, g.K, dt, w.epilogue,
                 bg.data_ptr(), vg.data_ptr(), 1e-5, stream.cuda_stream)

        def gstep():
            st = lib.ct_gemm_fwd(*gargs)
            if st != 0:
                raise ct.ConvTileError(st, "gemm")

        st, cfg, _ = ct.ct_gemm_query(g.M, g.N, g.K, dt, w.epilogue)
        ct.check(st, "query")
        ms = time_graph(gstep, stream, max(20, steps // 5), a.warmup)
        tf = w.flops / (ms * 1e-3) / 1e12
        vname = ct.variants()[cfg.variant]["name"]
        tile = {"split_k": cfg.split_k, "stages": cfg.stages, "kc": cfg.kc}
        out.append({"workload": name, "dtype": w.dtype, "us": round(ms * 1e3, 3), "TFLOP/s": round(tf, 2),
                    "bound": "mfma", "frac": round(tf / PEAK_TFLOPS[w.dtype], 4), "kernel": vname,
                    "tile": tile, "traffic": measured_traffic(name, vname, tile)})
        del xg, kg, yg
        torch.cuda.empty_cache()
    # the depthwise layers and the batch-norm chain, timed by their own
    # --workload functions (rotating buffers), summarised
    sub = argparse.Namespace(**vars(a))
    sub.eager, sub.no_cpu_baseline, sub.steps = False, True, steps
    for name, fn, kernel in ([(n, bench_depthwise, "depthwise") for n in wl.DEPTHWISE_WORKLOADS] +
                             [(n, bench_chain, "chain_channel") for n in wl.CHAIN_WORKLOADS]):
        r = fn(sub, name)
        out.append({"workload": name, "dtype": r["dtype"], "us": round(r["ms_per_step"] * 1e3, 3),
                    "GB/s": r["value"], "bound": "hbm", "frac": r["roofline"]["frac"], "kernel": kernel,
                    "rotating_buffers": r["config"]["rotating_buffers"], "traffic": r["roofline"]["traffic"]})
        torch.cuda.empty_cache()
    torch.cuda.set_stream(stream)
    return out


def main():
    a = _parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    _ensure_built()
    import torch
    from tensor_compiler_tiling_amd import convtile as ct
    from tensor_compiler_tiling_amd import workloads as wl

    if a.calibrate_copy:
        calibrate_copy()

    name = a.workload or wl.HEADLINE
    if name in wl.BROADCAST_WORKLOADS:
        print(json.dumps(bench_broadcast(a, name)), flush=True)
        return
    if name in wl.DEPTHWISE_WORKLOADS:
        print(json.dumps(bench_depthwise(a, name)), flush=True)
        return
    if name in wl.CHAIN_WORKLOADS:
        print(json.dumps(bench_chain(a, name)), flush=True)
        return
    gemm = wl.GEMM_WORKLOADS.get(name)
    # a matrix product is timed through ct_gemm_fwd; its 1x1 convolution view
    # gives the seeded operands (A = the view's filter, B = its input) and the
    # CPU baseline
    w = gemm.conv_view() if gemm is not None else wl.CONV_WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ct.check(ct.ct_init(0), "init")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    dt = ct.dtype_code(tdt)
    args = w.shape_args() + (dt, w.epilogue)

    cache_loaded = None
    if not a.no_cache and not a.tune and a.cache and os.path.exists(a.cache):
        ct.check(ct.ct_cache_load(a.cache), "cache load")
        cache_loaded = os.path.relpath(a.cache, ROOT)
    tune_info = None
    if a.tune:
        t0 = time.perf_counter()
        if gemm is not None:
            st, best, recs = ct.ct_gemm_tune(gemm.M, gemm.N, gemm.K, dt, w.epilogue,
                                             max_trials=a.tune_trials, min_repeat_ms=a.tune_ms)
        else:
            st, best, recs = ct.ct_conv2d_tune(*args, max_trials=a.tune_trials,
                                               min_repeat_ms=a.tune_ms)
        ct.check(st, "tune")
        tune_info = {"trials": len(recs), "seconds": round(time.perf_counter() - t0, 2),
                     "best_us": round(best.us, 3)}

    # one side stream for warm-up, capture and replay (the library keys its
    # split workspace by stream, so warm-up on this stream allocates it)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    if gemm is not None:
        inp = wl.conv_inputs(w)
        xg = torch.from_numpy(inp["x"]).to(dev).to(tdt)
        kg = torch.from_numpy(inp["w"]).to(dev).to(tdt)
        bg = torch.from_numpy(inp["bias"]).to(dev)
        vg = torch.from_numpy(inp["var"]).to(dev)
        yg = torch.empty((w.N, w.CO, w.OH, w.OW), dtype=torch.float32, device=dev)
        lib = ct.library()
        gargs = (kg.data_ptr(), xg.data_ptr(), yg.data_ptr(), gemm.M, gemm.N, gemm.K, dt, w.epilogue,
                 bg.data_ptr(), vg.data_ptr(), 1e-5, stream.cuda_stream)

        def step():
            st = lib.ct_gemm_fwd(*gargs)
            if st != 0:
                raise ct.ConvTileError(st, "fwd")

        st, cfg, from_cache = ct.ct_gemm_query(gemm.M, gemm.N, gemm.K, dt, w.epilogue)
        ct.check(st, "query")
    else:
        if a.prepared and w.dtype == "f32":
            print("--prepared applies to half-precision layers only", file=sys.stderr)
            sys.exit(2)
        step, cfg, from_cache = conv_step(w, prepared=a.prepared, stream_handle=stream.cuda_stream)
    vdesc = ct.variants()[cfg.variant]

    t0 = time.perf_counter()
    if a.eager:
        for _ in range(a.warmup):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(a.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_per_step = e0.elapsed_time(e1) / a.steps
    else:
        ms_per_step = time_graph(step, stream, a.steps, a.warmup)
    wall = time.perf_counter() - t0
    tflops = w.flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    # eager launch rate through the C ABI (host dispatch included), for reference
    eager_ms = None
    if not a.eager:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(a.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / a.steps

    if gemm is not None:
        metric = "matrix product TFLOP/s and % of MFMA peak"
    elif w.dtype == "f32":
        metric = "conv2d TFLOP/s per shape (fp32, batch 1) and % of MFMA peak"
    else:
        metric = "conv2d TFLOP/s per shape and % of MFMA peak"
    out = {
        "metric": metric,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded U[-1,1] inputs, He-normal weights)",
        "config": {"workload": name, "N": w.N, "CI": w.CI, "H": w.H, "W": w.W, "CO": w.CO,
                   "KH": w.KH, "KW": w.KW, "stride": w.stride, "pad": w.pad,
                   **({"M": gemm.M, "gemm_N": gemm.N, "K": gemm.K} if gemm is not None else {}),
                   "epilogue": w.epilogue, "flops_per_step": w.flops,
                   "launch": "eager" if a.eager else "hip_graph",
                   **({"filter": "prepared"} if a.prepared else {}),
                   "kernel": vdesc["name"], "split_k": cfg.split_k, "stages": cfg.stages,
                   "kc": cfg.kc, "config_index": cfg.index, "from_cache": bool(from_cache),
                   "tuning_log": cache_loaded},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": measured_traffic(name, vdesc["name"],
                                                 {"split_k": cfg.split_k, "stages": cfg.stages,
                                                  "kc": cfg.kc}, a.prepared)},
        "eager_ms_per_step": round(eager_ms, 6) if eager_ms else None,
        "wall_s": round(wall, 4),
    }
    if tune_info:
        out["tune"] = tune_info
    if a.workload is None and not a.no_per_shape:
        out["per_shape"] = per_shape(a)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline_gemm(gemm, a.cpu_seconds) if gemm is not None
                               else cpu_baseline(w, a.cpu_seconds))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
