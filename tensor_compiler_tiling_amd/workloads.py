"""Seeded synthetic workloads (shapes and input generators).

This module holds no arithmetic of the convolution or broadcast: only the
shapes of the workloads and the seeded random inputs that both the HIP path
and the fp64 oracle consume.  Generators: numpy PCG64, seed
1000 * cfg_id + {1: x, 2: w, 3: bias, 4: var}.

Distributions: x ~ U[-1, 1]; w ~ N(0, sqrt(2 / (CI*KH*KW))) (He-normal,
fan-in CI*KH*KW); bias ~ N(0, 0.1); var ~ U[0.5, 2].  Half-precision
workloads round x and w to fp16 (numpy astype, round to nearest even) or to
bfloat16 (round to nearest even on the fp32 bit pattern) before anything
sees them.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict, replace
from typing import Dict, Optional

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"
EPI_NONE, EPI_BIAS, EPI_EXP_BIAS_RSQRT = 0, 1, 2


@dataclass(frozen=True)
class ConvWorkload:
    name: str
    cfg_id: int
    N: int
    CI: int
    H: int
    W: int
    CO: int
    KH: int
    KW: int
    stride: int
    pad: int
    dtype: str = F32
    epilogue: int = EPI_NONE

    @property
    def OH(self) -> int:
        return (self.H + 2 * self.pad - self.KH) // self.stride + 1

    @property
    def OW(self) -> int:
        return (self.W + 2 * self.pad - self.KW) // self.stride + 1

    @property
    def flops(self) -> int:
        """2 x multiply-accumulates of the definition (padded taps included)."""
        return 2 * self.N * self.CO * self.OH * self.OW * self.CI * self.KH * self.KW

    def algorithmic_bytes(self) -> int:
        """x, w, (bias, var) read once and y written once."""
        e = 4 if self.dtype == F32 else 2
        b = e * (self.N * self.CI * self.H * self.W + self.CO * self.CI * self.KH * self.KW)
        b += 4 * self.N * self.CO * self.OH * self.OW
        if self.epilogue == EPI_BIAS:
            b += 4 * self.CO
        elif self.epilogue == EPI_EXP_BIAS_RSQRT:
            b += 8 * self.CO
        return b

    def shape_args(self):
        return (self.N, self.CI, self.H, self.W, self.CO, self.KH, self.KW, self.stride, self.pad)

    def as_dict(self) -> dict:
        d = asdict(self)
        d.update(OH=self.OH, OW=self.OW, flops=self.flops)
        return d

    def with_(self, **kw) -> "ConvWorkload":
        return replace(self, **kw)


@dataclass(frozen=True)
class BroadcastWorkload:
    name: str
    cfg_id: int
    N: int
    C: int
    H: int
    W: int
    out_dtype: str = F16

    def bytes_written(self) -> int:
        return self.N * self.C * self.H * self.W * (2 if self.out_dtype == F16 else 4)


# The workloads: ResNet-style layers at batch 1 (fp32), a half-precision
# batched layer, and a half-precision layer with the fused per-channel
# epilogue plus its standalone [1,C,1,1] -> [N,C,H,W] broadcast.
CONV_WORKLOADS: Dict[str, ConvWorkload] = {w.name: w for w in [
    ConvWorkload("resnet_c64_14x14_k3", 1, 1, 64, 14, 14, 64, 3, 3, 1, 1),
    ConvWorkload("resnet_final_c512_7x7_k3", 2, 1, 512, 7, 7, 512, 3, 3, 1, 1),
    ConvWorkload("r18_stem_c3_224x224_k7s2", 30, 1, 3, 224, 224, 64, 7, 7, 2, 3),
    ConvWorkload("r18_c64_56x56_k3", 31, 1, 64, 56, 56, 64, 3, 3, 1, 1),
    ConvWorkload("r18_c64to128_56x56_k3s2", 32, 1, 64, 56, 56, 128, 3, 3, 2, 1),
    ConvWorkload("r18_c128to256_28x28_k3s2", 33, 1, 128, 28, 28, 256, 3, 3, 2, 1),
    ConvWorkload("r18_c256to512_14x14_k3s2", 34, 1, 256, 14, 14, 512, 3, 3, 2, 1),
    ConvWorkload("r18_c256_14x14_k1", 35, 1, 256, 14, 14, 256, 1, 1, 1, 0),
    ConvWorkload("f16_n64_c256_14x14_k3", 4, 64, 256, 14, 14, 256, 3, 3, 1, 1, F16),
    ConvWorkload("f16_n128_c128to256_32x32_k3_epi", 5, 128, 128, 32, 32, 256, 3, 3, 1, 1, F16,
                 EPI_EXP_BIAS_RSQRT),
]}

def gemm_fold(N: int):
    """(H, W) with H * W = N and W the largest divisor of N not above 256: the
    image a row-major [K][N] operand is viewed as (the library's own split)."""
    for w in range(min(N, 256), 0, -1):
        if N % w == 0:
            return N // w, w
    raise ValueError("N must be positive")


@dataclass(frozen=True)
class GemmWorkload:
    """C[M][N] = A[M][K] B[K][N] (row-major), the batch-1 1x1 convolution with
    CO = M, CI = K, H * W = N (A = its filter, B = its input)."""
    name: str
    cfg_id: int
    M: int
    N: int
    K: int
    dtype: str = F32
    epilogue: int = EPI_NONE

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def conv_view(self) -> ConvWorkload:
        H, W = gemm_fold(self.N)
        return ConvWorkload(self.name, self.cfg_id, 1, self.K, H, W, self.M, 1, 1, 1, 0, self.dtype,
                            self.epilogue)


# Matrix products on the same kernels (the 1x1 view): a square fp16 product
# and an fp32 one with the per-row epilogue.
GEMM_WORKLOADS: Dict[str, GemmWorkload] = {g.name: g for g in [
    GemmWorkload("gemm_f16_m4096_n4096_k4096", 60, 4096, 4096, 4096, F16),
    GemmWorkload("gemm_f32_m2048_n2048_k2048_epi", 61, 2048, 2048, 2048, F32, EPI_EXP_BIAS_RSQRT),
]}


def gemm_inputs(g: GemmWorkload) -> dict:
    """A [M, K] (He-normal over K) and B [K, N] (U[-1, 1]), rounded to g.dtype,
    and the per-row bias / var: the 1x1 view's filter, input and epilogue
    parameters, so both views see the same values."""
    c = conv_inputs(g.conv_view())
    return {"A": c["w"].reshape(g.M, g.K), "B": c["x"].reshape(g.K, g.N), "bias": c["bias"],
            "var": c["var"]}


@dataclass(frozen=True)
class DepthwiseWorkload:
    """Depthwise convolution: x [N][C][H][W], w [C][1][KH][KW], every channel
    convolved with its own filter."""
    name: str
    cfg_id: int
    N: int
    C: int
    H: int
    W: int
    KH: int
    KW: int
    stride: int
    pad: int
    dtype: str = F32
    epilogue: int = EPI_NONE

    @property
    def OH(self) -> int:
        return (self.H + 2 * self.pad - self.KH) // self.stride + 1

    @property
    def OW(self) -> int:
        return (self.W + 2 * self.pad - self.KW) // self.stride + 1

    @property
    def flops(self) -> int:
        return 2 * self.N * self.C * self.OH * self.OW * self.KH * self.KW

    def algorithmic_bytes(self) -> int:
        """x and w read once, y (fp32) written once, plus the epilogue's
        per-channel parameters."""
        e = 4 if self.dtype == F32 else 2
        b = e * (self.N * self.C * self.H * self.W + self.C * self.KH * self.KW)
        b += 4 * self.N * self.C * self.OH * self.OW
        if self.epilogue == EPI_BIAS:
            b += 4 * self.C
        elif self.epilogue == EPI_EXP_BIAS_RSQRT:
            b += 8 * self.C
        return b

    def as_dict(self) -> dict:
        d = asdict(self)
        d.update(OH=self.OH, OW=self.OW, flops=self.flops)
        return d


# Depthwise layers of a MobileNet-style network at batch 128: a 3x3 stride-1
# layer on 56x56 planes, a stride-2 layer on 112x112 planes, and an fp16 layer
# on 14x14 planes (several planes a workgroup) with a bias epilogue.
DEPTHWISE_WORKLOADS: Dict[str, DepthwiseWorkload] = {d.name: d for d in [
    DepthwiseWorkload("dw_f32_n128_c128_56x56_k3", 70, 128, 128, 56, 56, 3, 3, 1, 1),
    DepthwiseWorkload("dw_f32_n128_c64_112x112_k3s2", 71, 128, 64, 112, 112, 3, 3, 2, 1),
    DepthwiseWorkload("dw_f16_n128_c512_14x14_k3_bias", 72, 128, 512, 14, 14, 3, 3, 1, 1, F16,
                      EPI_BIAS),
]}


def depthwise_inputs(d: DepthwiseWorkload) -> dict:
    """x ~ U[-1, 1] [N, C, H, W], w He-normal over fan-in KH*KW [C, 1, KH, KW]
    (both rounded to d.dtype), bias ~ N(0, 0.1), var ~ U[0.5, 2] per channel;
    seeds 1000 * cfg_id + {1, 2, 3, 4}."""
    base = 1000 * d.cfg_id
    x = np.random.default_rng(base + 1).uniform(-1.0, 1.0, (d.N, d.C, d.H, d.W))
    w = np.random.default_rng(base + 2).normal(0.0, np.sqrt(2.0 / (d.KH * d.KW)),
                                               (d.C, 1, d.KH, d.KW))
    b = np.random.default_rng(base + 3).normal(0.0, 0.1, d.C).astype(np.float32)
    v = np.random.default_rng(base + 4).uniform(0.5, 2.0, d.C).astype(np.float32)
    return {"x": to_dtype(x, d.dtype), "w": to_dtype(w, d.dtype), "bias": b, "var": v}


@dataclass(frozen=True)
class ChainWorkload:
    """The general per-channel broadcast on [outer][P][inner]: `program` names
    a step-chain recipe (batch-norm inference on a producer's fp32 output)."""
    name: str
    cfg_id: int
    outer: int
    P: int
    inner: int
    program: str
    out_dtype: str = F32

    def algorithmic_bytes(self) -> int:
        """The producer's fp32 elements read once, the output written once, the
        four per-channel arrays read once."""
        n = self.outer * self.P * self.inner
        return 4 * n + (4 if self.out_dtype == F32 else 2) * n + 16 * self.P


# Batch-norm inference applied to a 128x256x32x32 fp32 activation:
# out = (x - mean[c]) * gamma[c] / sqrt(var[c] + eps) + beta[c], as
# c0 = gamma * rsqrt(var + eps), c1 = beta - mean * c0, out = x * c0 + c1.
CHAIN_PROGRAMS = {
    "batchnorm": ([("set", "a0"), ("add", 1e-5), ("rsqrt",), ("mul", "a1")],
                  [("set", "a2"), ("mul", "c0"), ("rsub", "a3")],
                  [("set", "x"), ("mul", "c0"), ("add", "c1")]),
}

CHAIN_WORKLOADS: Dict[str, ChainWorkload] = {c.name: c for c in [
    ChainWorkload("bn_apply_f32_128x256x32x32", 80, 128, 256, 32 * 32, "batchnorm"),
]}


def chain_inputs(cw: ChainWorkload) -> dict:
    """x ~ U[-1, 1] [outer, P, inner] (fp32); arrays a0 = var ~ U[0.5, 2],
    a1 = gamma ~ U[0.5, 1.5], a2 = mean ~ N(0, 0.5), a3 = beta ~ N(0, 0.5);
    seeds 1000 * cfg_id + {1, ..., 5}."""
    base = 1000 * cw.cfg_id
    x = np.random.default_rng(base + 1).uniform(-1.0, 1.0, (cw.outer, cw.P, cw.inner)).astype(np.float32)
    a = [np.random.default_rng(base + 2).uniform(0.5, 2.0, cw.P),
         np.random.default_rng(base + 3).uniform(0.5, 1.5, cw.P),
         np.random.default_rng(base + 4).normal(0.0, 0.5, cw.P),
         np.random.default_rng(base + 5).normal(0.0, 0.5, cw.P)]
    return {"x": x, "arrays": [v.astype(np.float32) for v in a]}


HEADLINE = "resnet_final_c512_7x7_k3"
SWEEP = [n for n, w in CONV_WORKLOADS.items() if w.cfg_id >= 30]

BROADCAST_WORKLOADS: Dict[str, BroadcastWorkload] = {b.name: b for b in [
    BroadcastWorkload("bcast_exp_128x256x32x32_f16", 5, 128, 256, 32, 32, F16),
    BroadcastWorkload("bcast_exp_128x256x32x32_f32", 5, 128, 256, 32, 32, F32),
]}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the workload dtype; returns float32 (f32/bf16 values) or float16."""
    if dtype == F32:
        return a.astype(np.float32)
    if dtype == F16:
        return a.astype(np.float16)
    if dtype == BF16:
        return round_bf16(a.astype(np.float32))
    raise ValueError(dtype)


def conv_inputs(wl: ConvWorkload, seed_base: Optional[int] = None) -> dict:
    """x, w (rounded to wl.dtype), bias, var (float32) for a workload."""
    base = 1000 * (wl.cfg_id if seed_base is None else seed_base)
    rx = np.random.default_rng(base + 1)
    rw = np.random.default_rng(base + 2)
    rb = np.random.default_rng(base + 3)
    rv = np.random.default_rng(base + 4)
    x = rx.uniform(-1.0, 1.0, (wl.N, wl.CI, wl.H, wl.W))
    w = rw.normal(0.0, np.sqrt(2.0 / (wl.CI * wl.KH * wl.KW)), (wl.CO, wl.CI, wl.KH, wl.KW))
    b = rb.normal(0.0, 0.1, wl.CO).astype(np.float32)
    v = rv.uniform(0.5, 2.0, wl.CO).astype(np.float32)
    return {"x": to_dtype(x, wl.dtype), "w": to_dtype(w, wl.dtype), "bias": b, "var": v}


def small_int_inputs(wl: ConvWorkload, seed: int = 7) -> dict:
    """x, w with integer values in [-2, 2]: every partial sum of the conv is an
    integer well below 2^24, so fp32 accumulation in any order is exact."""
    r = np.random.default_rng(seed)
    x = r.integers(-2, 3, (wl.N, wl.CI, wl.H, wl.W)).astype(np.float32)
    w = r.integers(-2, 3, (wl.CO, wl.CI, wl.KH, wl.KW)).astype(np.float32)
    return {"x": to_dtype(x, wl.dtype), "w": to_dtype(w, wl.dtype)}


def broadcast_var(bw: BroadcastWorkload) -> np.ndarray:
    """var[c] ~ U[0.5, 2] (the fused workload's var, seed 1000 * cfg_id + 4)."""
    return np.random.default_rng(1000 * bw.cfg_id + 4).uniform(0.5, 2.0, bw.C).astype(np.float32)
