"""Run the tile-config search over the named convolution (and matrix-product)
workloads and save the winners as a JSON-lines tuning log.

This is the library's counterpart of the TVM tutorial's tune-then-apply flow
(Tune the Convolution on CUDA, "Start tuning" and the history-best step): the
search times every legal tile config of a shape on the GPU, keeps the fastest
one that matches the on-device direct reference, and the log is later loaded
with ct_cache_load so that ct_conv2d_nchw_fwd dispatches to it.

    python -m tensor_compiler_tiling_amd.tune_all [--out PATH] [--ms MS] [names...]

A matrix-product workload is tuned through ct_gemm_tune, i.e. as its 1x1
convolution view, under which ct_gemm_fwd finds the record.
With no names every workload is tuned and the log is rewritten;
with names, the log's records of the other shapes are kept.  The default
output is the log shipped with the package for gfx950 (tuned/gfx950.jsonl).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

_PKG = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LOG = os.path.join(_PKG, "tuned", "gfx950.jsonl")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("names", nargs="*")
    ap.add_argument("--out", default=DEFAULT_LOG)
    ap.add_argument("--ms", type=float, default=20.0, help="minimum timed milliseconds per repeat")
    ap.add_argument("--trials", type=int, default=0, help="0 = every legal config")
    a = ap.parse_args(argv)

    import torch
    from tensor_compiler_tiling_amd import convtile as ct
    from tensor_compiler_tiling_amd import workloads as wl

    names = a.names or (list(wl.CONV_WORKLOADS) + list(wl.GEMM_WORKLOADS))
    ct.check(ct.ct_cache_clear(), "cache clear")
    if a.names and os.path.exists(a.out):
        # retuning some shapes: keep the log's records of the others
        ct.check(ct.ct_cache_load(a.out), "cache load")
    for name in names:
        g = wl.GEMM_WORKLOADS.get(name)
        w = g if g is not None else wl.CONV_WORKLOADS[name]
        tdt = {wl.F32: torch.float32, wl.F16: torch.float16, wl.BF16: torch.bfloat16}[w.dtype]
        t0 = time.perf_counter()
        if g is not None:
            st, best, recs = ct.ct_gemm_tune(g.M, g.N, g.K, ct.dtype_code(tdt), g.epilogue,
                                             max_trials=a.trials, min_repeat_ms=a.ms)
        else:
            args = w.shape_args() + (ct.dtype_code(tdt), w.epilogue)
            st, best, recs = ct.ct_conv2d_tune(*args, max_trials=a.trials, min_repeat_ms=a.ms)
        ct.check(st, f"tune {name}")
        vname = ct.variants()[best.variant]["name"]
        print(json.dumps({"workload": name, "trials": len(recs),
                          "ok": sum(1 for r in recs if r.error_no == 0),
                          "seconds": round(time.perf_counter() - t0, 2), "variant": vname,
                          "split_k": best.split_k, "stages": best.stages, "kc": best.kc,
                          "us": round(best.us, 3)}), flush=True)
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    tmp = a.out + ".tmp"
    if os.path.exists(tmp):
        os.remove(tmp)
    ct.check(ct.ct_cache_save(tmp), "cache save")  # appends: start from an empty file
    os.replace(tmp, a.out)
    print(f"saved {ct.ct_cache_size()} records to {a.out}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
