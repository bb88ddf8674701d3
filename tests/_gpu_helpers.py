"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the library through its C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import oracle as O
from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl

DEV = "cuda:0"
# max |gpu - ref| <= TOL * S.  Half-precision inputs share the fp32 gate:
# their products are exact in fp32 and accumulation is fp32.
TOL = {wl.F32: 1e-4, wl.F16: 1e-4, wl.BF16: 1e-4}
CT_DT = {wl.F32: ct.CT_F32, wl.F16: ct.CT_F16, wl.BF16: ct.CT_BF16}
TORCH_DT = {wl.F32: torch.float32, wl.F16: torch.float16, wl.BF16: torch.bfloat16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == wl.BF16:
        t = t.to(torch.bfloat16)  # values are already bfloat16-exact
    return t.to(DEV)


def run(w: wl.ConvWorkload, inp: dict, config=None, direct=False, epilogue=None) -> np.ndarray:
    epi = w.epilogue if epilogue is None else epilogue
    x = to_dev(inp["x"], w.dtype)
    k = to_dev(inp["w"], w.dtype)
    b = torch.from_numpy(inp["bias"]).to(DEV) if "bias" in inp else None
    v = torch.from_numpy(inp["var"]).to(DEV) if "var" in inp else None
    y = ct.conv2d(x, k, w.stride, w.pad, epi, b, v, 1e-5, config=config, direct=direct)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def oracle_full(w: wl.ConvWorkload, inp: dict):
    return O.conv2d_nchw(inp["x"].astype(np.float64), inp["w"].astype(np.float64), w.stride, w.pad)


def assert_conv_close(got: np.ndarray, ref: np.ndarray, absacc: np.ndarray, dtype: str, what=""):
    scale = float(absacc.max()) if absacc.size else 0.0
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    tol = TOL[dtype] * scale
    say(f"  {what}: max|gpu-ref| = {err:.3e}  (1e-4*S = {1e-4 * scale:.3e}, gate {tol:.3e})")
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    assert err <= tol, f"{what}: {err} > {tol}"
    return err, scale


def legal_configs(w: wl.ConvWorkload, epilogue=None):
    epi = w.epilogue if epilogue is None else epilogue
    args = w.shape_args() + (CT_DT[w.dtype], epi)
    out = []
    for idx in range(ct.ct_conv2d_space_size(*args)):
        st, cfg, legal = ct.ct_conv2d_space_entity(*args, idx)
        assert st == 0
        if legal:
            out.append(cfg)
    return out


def sample_points(shape, n: int, seed: int) -> np.ndarray:
    """n output coordinates: corners/edges of every dimension plus random ones."""
    r = np.random.default_rng(seed)
    N, C, OH, OW = shape
    pts = [(0, 0, 0, 0), (N - 1, C - 1, OH - 1, OW - 1), (0, C - 1, 0, OW - 1),
           (N - 1, 0, OH - 1, 0)]
    rnd = np.stack([r.integers(0, d, n) for d in shape], axis=1)
    return np.concatenate([np.array(pts), rnd]).astype(np.int64)
