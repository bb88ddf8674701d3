"""Oracle for the NCHW convolution / per-channel broadcast / tile-space path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
library package (``tensor_compiler_tiling_amd``) never imports this module and
this module never imports the package: the two share no code.

What it holds:

* ctypes bindings to ``conv_oracle.c`` -- the fp64 seven-loop convolution, its
  sampled-point variant, the per-channel epilogue and the broadcast (see that
  file's header for the definitions and the passages they follow);
* plain-Python versions of the search-space arithmetic of the TVM tutorial
  "Tuning High Performance Convolution on NVIDIA GPUs" (Step 1, the
  ``define_split`` / ``define_knob`` space) as printed in the run output of the
  gist that reproduces it: all ordered factorizations ("policy=all"), the
  mixed-radix flat index of a config entity, and the shared-memory footprint
  of the tutorial's schedule template;
* the FLOP count of a convolution (2 x multiply-accumulates, padded taps
  included);
* the matrix product C = A B in fp64 (its definition, with a library matmul
  of fp64 arrays as the one step), which the TVM tutorial's opening names as a
  second use of its template;
* the depthwise convolution in fp64 (the definition written out in numpy: one
  strided slice of the zero-padded input per tap, summed in row-major tap
  order), another operator the tutorial's opening names;
* the ridge regression that the guided tile-config search fits as its cost
  model (the normal equations, one library solve);
* the general per-channel broadcast [1,P,1] => [B,P,B] of the Paddle PR's
  Introduction, with a chain of div / exp / rsqrt-style steps (Performance
  Impact), evaluated step by step in fp64 over numpy broadcasting.

Parity status: every function here is pinned by tests in
``tests/test_oracle_pins.py`` (hand-computed cases, closed forms, invariants,
independent library routines, and the values printed on the pages).
"""
from __future__ import annotations

import ctypes
import itertools
import os
import subprocess
from functools import reduce
from operator import mul
from typing import Dict, List, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build_oracle(force: bool = True) -> str:
    """Compile conv_oracle.c with gcc (fp64, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_oracle(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        L = ctypes.c_long
        lib.oracle_conv2d_nchw.argtypes = [dp, dp, dp, dp] + [L] * 9
        lib.oracle_conv2d_nchw.restype = ctypes.c_int
        lib.oracle_conv2d_points.argtypes = [dp, dp, lp, L, dp, dp] + [L] * 9
        lib.oracle_conv2d_points.restype = ctypes.c_int
        lib.oracle_channel_epilogue.argtypes = [dp, dp, dp, ctypes.c_double, L, L, L,
                                                ctypes.c_int, dp]
        lib.oracle_channel_epilogue.restype = ctypes.c_int
        lib.oracle_broadcast_exp.argtypes = [dp, L, L, L, L, dp]
        lib.oracle_broadcast_exp.restype = ctypes.c_int
        lib.oracle_out_extent_api.argtypes = [L, L, L, L]
        lib.oracle_out_extent_api.restype = L
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _dp(a: np.ndarray):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def out_extent(inp: int, k: int, stride: int, pad: int) -> int:
    """floor((in + 2 pad - k) / stride) + 1 (0 when the kernel does not fit)."""
    return int(_load().oracle_out_extent_api(inp, k, stride, pad))


def conv2d_nchw(x, w, stride: int, pad: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 seven-loop convolution.  Returns (y, absacc) where
    absacc[n,f,oy,ox] = sum |xp * w| over the same taps (tolerance scale)."""
    x = _f64(x)
    w = _f64(w)
    N, CI, H, W = x.shape
    CO, CI2, KH, KW = w.shape
    if CI2 != CI:
        raise ValueError("channel mismatch")
    OH, OW = out_extent(H, KH, stride, pad), out_extent(W, KW, stride, pad)
    if OH <= 0 or OW <= 0:
        raise ValueError("kernel larger than padded input")
    y = np.empty((N, CO, OH, OW), np.float64)
    a = np.empty_like(y)
    rc = _load().oracle_conv2d_nchw(_dp(x), _dp(w), _dp(y), _dp(a), N, CI, H, W, CO, KH, KW,
                                    stride, pad)
    if rc != 0:
        raise ValueError("oracle_conv2d_nchw rejected its arguments")
    return y, a


def conv2d_points(x, w, stride: int, pad: int, idx) -> Tuple[np.ndarray, np.ndarray]:
    """The same sum for selected outputs only; idx is an (npts, 4) array of
    (n, f, oy, ox).  Returns (y, absacc) of length npts."""
    x = _f64(x)
    w = _f64(w)
    N, CI, H, W = x.shape
    CO, _, KH, KW = w.shape
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 4))
    npts = idx.shape[0]
    y = np.empty(npts, np.float64)
    a = np.empty(npts, np.float64)
    rc = _load().oracle_conv2d_points(_dp(x), _dp(w),
                                      idx.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), npts,
                                      _dp(y), _dp(a), N, CI, H, W, CO, KH, KW, stride, pad)
    if rc != 0:
        raise ValueError("oracle_conv2d_points rejected its arguments")
    return y, a


EPI_NONE, EPI_BIAS, EPI_EXP_BIAS_RSQRT = 0, 1, 2


def gemm(A, B) -> Tuple[np.ndarray, np.ndarray]:
    """C[m][n] = sum_k A[m][k] * B[k][n] in fp64, and sum_k |A[m][k] * B[k][n]|
    (the tolerance scale, as conv2d_nchw's absacc).  A [M, K], B [K, N]."""
    a = _f64(A)
    b = _f64(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("gemm: A must be [M, K] and B [K, N]")
    return a @ b, np.abs(a) @ np.abs(b)


def conv2d_depthwise(x, w, stride: int, pad: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 depthwise convolution: x [N, C, H, W], w [C, 1, KH, KW],
    y[n][c][oy][ox] = sum_{ky, kx} xp[n][c][oy*s + ky][ox*s + kx] * w[c][0][ky][kx]
    with xp = x zero-padded by `pad` on each side; the taps are summed in
    row-major (ky, kx) order.  Returns (y, absacc), absacc the same sum of
    |term| (the tolerance scale, as conv2d_nchw's)."""
    x = _f64(x)
    w = _f64(w)
    if x.ndim != 4 or w.ndim != 4 or w.shape[0] != x.shape[1] or w.shape[1] != 1:
        raise ValueError("conv2d_depthwise: x must be [N, C, H, W] and w [C, 1, KH, KW]")
    N, C, H, W = x.shape
    KH, KW = w.shape[2], w.shape[3]
    OH, OW = out_extent(H, KH, stride, pad), out_extent(W, KW, stride, pad)
    if OH <= 0 or OW <= 0:
        raise ValueError("kernel larger than padded input")
    xp = np.zeros((N, C, H + 2 * pad, W + 2 * pad), np.float64)
    xp[:, :, pad:pad + H, pad:pad + W] = x
    y = np.zeros((N, C, OH, OW), np.float64)
    a = np.zeros_like(y)
    for ky in range(KH):
        for kx in range(KW):
            rows = slice(ky, ky + stride * (OH - 1) + 1, stride)
            cols = slice(kx, kx + stride * (OW - 1) + 1, stride)
            t = xp[:, :, rows, cols] * w[:, 0, ky, kx][None, :, None, None]
            y += t
            a += np.abs(t)
    return y, a


def channel_epilogue(y, kind: int, b=None, v=None, eps: float = 1e-5) -> np.ndarray:
    """out = y | y + b[c] | exp(y + b[c]) / sqrt(v[c] + eps), per channel c."""
    y = _f64(y)
    N, C = y.shape[0], y.shape[1]
    HW = int(np.prod(y.shape[2:])) if y.ndim > 2 else 1
    bb = _f64(b) if b is not None else None
    vv = _f64(v) if v is not None else None
    out = np.empty_like(y)
    rc = _load().oracle_channel_epilogue(_dp(y), _dp(bb), _dp(vv), float(eps), N, C, HW,
                                         int(kind), _dp(out))
    if rc != 0:
        raise ValueError("oracle_channel_epilogue rejected its arguments")
    return out


def broadcast_exp(var, N: int, H: int, W: int) -> np.ndarray:
    """[1,C,1,1] => [N,C,H,W] of exp(var[c]) in fp64."""
    var = _f64(var).reshape(-1)
    C = var.shape[0]
    out = np.empty((N, C, H, W), np.float64)
    rc = _load().oracle_broadcast_exp(_dp(var), N, C, H, W, _dp(out))
    if rc != 0:
        raise ValueError("oracle_broadcast_exp rejected its arguments")
    return out


def broadcast_chain(chains, outer: int, P: int, inner: int, arrays=(), x=None) -> np.ndarray:
    """The general per-channel broadcast [1,P,1] => [B,P,B] in fp64, out of
    shape [outer, P, inner].  chains = (c0_steps, c1_steps, v_steps); a step
    is (op,), (op, src) or (op, "imm", value) / (op, value) with op one of
    set add sub mul div rsub rdiv exp rsqrt sqrt and src one of imm x c0 c1
    a0..a3.  Each chain starts from 0 and applies its steps in order:
    c0 from immediates and arrays a_k[p]; c1 may also read c0; v may also
    read c1 and x[o][p][i].  out = v, or c0 when the v chain is empty."""
    arr = [None if a is None else _f64(a).reshape(1, -1, 1) for a in list(arrays) + [None] * 4][:4]
    X = None if x is None else _f64(x).reshape(outer, P, inner)

    def run(steps, regs):
        v = np.zeros((1, 1, 1))
        for st in steps:
            op, rest = st[0], st[1:]
            src, imm = "imm", 0.0
            if len(rest) == 1:
                if isinstance(rest[0], str):
                    src = rest[0]
                else:
                    imm = float(rest[0])
            elif len(rest) == 2:
                src, imm = rest[0], float(rest[1])
            if op in ("exp", "rsqrt", "sqrt"):
                v = {"exp": np.exp, "rsqrt": lambda t: 1.0 / np.sqrt(t), "sqrt": np.sqrt}[op](v)
                continue
            if src == "imm":
                a = np.float64(imm)
            elif src in regs:
                a = regs[src]
            elif src.startswith("a"):
                a = arr[int(src[1])]
            else:
                raise ValueError(f"source {src} not readable here")
            if op == "set":
                v = a + np.zeros((1, 1, 1))
            elif op == "add":
                v = v + a
            elif op == "sub":
                v = v - a
            elif op == "mul":
                v = v * a
            elif op == "div":
                v = v / a
            elif op == "rsub":
                v = a - v
            elif op == "rdiv":
                v = a / v
            else:
                raise ValueError(f"unknown op {op}")
        return v

    c0 = run(chains[0], {})
    c1 = run(chains[1], {"c0": c0})
    v = run(chains[2], {"c0": c0, "c1": c1, "x": X}) if len(chains[2]) else c0
    return np.broadcast_to(v, (outer, P, inner)).astype(np.float64).copy()


def ridge_fit(X, y, lam: float) -> np.ndarray:
    """The ridge regression the guided search fits (its cost model): w
    minimising |X w - y|^2 + lam |w|^2, from the normal equations
    (X^T X + lam I) w = X^T y solved by a library routine."""
    X = _f64(X)
    y = _f64(y)
    return np.linalg.solve(X.T @ X + lam * np.eye(X.shape[1]), X.T @ y)


def conv_flops(N, CI, H, W, CO, KH, KW, stride, pad) -> int:
    """2 x multiply-accumulates of the definition, padded taps included."""
    OH = (H + 2 * pad - KH) // stride + 1
    OW = (W + 2 * pad - KW) // stride + 1
    return 2 * N * CO * OH * OW * CI * KH * KW


# ---------------------------------------------------------------------------
# Search-space arithmetic of the TVM tutorial's template (Step 1) as printed in
# the gist's ConfigSpace dump and tuning log.
# ---------------------------------------------------------------------------

def _divisors(n: int) -> List[int]:
    return [d for d in range(1, n + 1) if n % d == 0]


def ordered_factorizations(n: int, k: int) -> List[List[int]]:
    """All k-tuples of positive integers whose product is n ("policy=all").

    Order: ascending by (x_k, x_{k-1}, ..., x_2), x_1 = n / (x_2 ... x_k).
    Brute force over all divisor tuples; small n only.
    """
    if n <= 0 or k <= 0:
        raise ValueError("n and k must be positive")
    if k == 1:
        return [[n]]
    divs = _divisors(n)
    out = []
    for tail in itertools.product(divs, repeat=k - 1):   # (x_2, ..., x_k)
        p = reduce(mul, tail, 1)
        if n % p == 0:
            out.append([n // p] + list(tail))
    out.sort(key=lambda t: tuple(reversed(t[1:])))
    return out


class OracleSpace:
    """Ordered knobs; each knob is ("split", product, num_outputs) or
    ("option", [values]).  Entities are addressed by a mixed-radix flat index
    with the first declared knob least significant."""

    def __init__(self, knobs: Sequence[Tuple[str, tuple]]):
        self.names = [k[0] for k in knobs]
        self.choices: List[list] = []
        for name, spec in knobs:
            if spec[0] == "split":
                self.choices.append(ordered_factorizations(spec[1], spec[2]))
            elif spec[0] == "option":
                self.choices.append(list(spec[1]))
            else:
                raise ValueError(spec[0])
        self.lens = [len(c) for c in self.choices]

    def __len__(self) -> int:
        return reduce(mul, self.lens, 1)

    def index_of(self, entity: Dict[str, object]) -> int:
        idx, radix = 0, 1
        for name, ch, ln in zip(self.names, self.choices, self.lens):
            idx += ch.index(entity[name]) * radix
            radix *= ln
        return idx

    def entity_at(self, index: int) -> Dict[str, object]:
        if not 0 <= index < len(self):
            raise IndexError(index)
        ent = {}
        for name, ch, ln in zip(self.names, self.choices, self.lens):
            ent[name] = ch[index % ln]
            index //= ln
        return ent


def tvm_tutorial_space(N, H, W, CO, CI, KH, KW, stride, pad) -> OracleSpace:
    """The tutorial template's knobs, in declaration order (Step 1)."""
    OH = (H + 2 * pad - KH) // stride + 1
    OW = (W + 2 * pad - KW) // stride + 1
    return OracleSpace([
        ("tile_f", ("split", CO, 4)),
        ("tile_y", ("split", OH, 4)),
        ("tile_x", ("split", OW, 4)),
        ("tile_rc", ("split", CI, 3)),
        ("tile_ry", ("split", KH, 3)),
        ("tile_rx", ("split", KW, 3)),
        ("auto_unroll_max_step", ("option", [0, 512, 1500])),
        ("unroll_explicit", ("option", [0, 1])),
    ])


def tvm_template_shared_bytes(entity: Dict[str, object], stride: int) -> int:
    """fp32 bytes of the two shared-memory stages of the tutorial's schedule.

    AA (padded data) and WW (kernel) are cached at the rxo loop, so each holds
    one block's output tile against the reduction extents inside rxo:
      AA = RC_s * ((Y_b - 1) * s + RY_s) * ((X_b - 1) * s + RX_s)
      WW = F_b * RC_s * RY_s * RX_s
    where F_b, Y_b, X_b are the products of the vthread/thread/inner factors,
    RC_s = rcm * rci, and -- as the template is printed -- the ry axis is split
    with tile_rx's factors and rx with tile_ry's.
    """
    tf, ty, tx = entity["tile_f"], entity["tile_y"], entity["tile_x"]
    F_b = tf[1] * tf[2] * tf[3]
    Y_b = ty[1] * ty[2] * ty[3]
    X_b = tx[1] * tx[2] * tx[3]
    rc = entity["tile_rc"]
    RC_s = rc[1] * rc[2]
    ry_split = entity["tile_rx"]    # as printed: tile_rx applied to ry
    rx_split = entity["tile_ry"]    # and tile_ry applied to rx
    RY_s = ry_split[1] * ry_split[2]
    RX_s = rx_split[1] * rx_split[2]
    aa = RC_s * ((Y_b - 1) * stride + RY_s) * ((X_b - 1) * stride + RX_s)
    ww = F_b * RC_s * RY_s * RX_s
    return 4 * (aa + ww)


def tvm_template_threads(entity: Dict[str, object]) -> int:
    """Threads per block: product of the thread-level factors."""
    return entity["tile_f"][2] * entity["tile_y"][2] * entity["tile_x"][2]
