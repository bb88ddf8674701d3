"""GPU parity of the depthwise convolution against the fp64 oracle, through
the C ABI.

The kernel converts its inputs to fp32 exactly and accumulates at most 256
products in fp32, so every dtype is held to the fp32 gate: max |gpu - ref| <=
1e-4 * S, S = max over outputs of sum |xp * w| (the oracle's absacc); the
exp-bias-rsqrt epilogue is gated relatively; small-integer inputs bit-exact.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl

from _gpu_helpers import DEV, say, to_dev

pytestmark = pytest.mark.gpu

GATE = 1e-4

# (N, C, H, W, KH, KW, stride, pad): the degenerate 1x1 image, each compiled
# filter size (3x3, 5x5, 7x7 at strides 1 and 2), the generic path (non-square
# filters, 1x1, stride 3, the 16x16 = 256-tap maximum), several row blocks with
# a ragged last one, small planes packed several to a workgroup with a ragged
# last group, rows of 512 or more outputs (one strip row a workgroup), and a
# row so wide that its strip needs more than 64 KB of LDS, and pads wider
# than the filter (row blocks and columns that lie wholly in the padding)
SHAPES = [
    (1, 1, 1, 1, 1, 1, 1, 0),
    (2, 3, 9, 11, 3, 3, 1, 1),
    (2, 5, 8, 8, 3, 3, 2, 1),
    (2, 7, 33, 35, 5, 5, 1, 2),
    (1, 4, 30, 29, 5, 5, 2, 2),
    (1, 3, 13, 13, 7, 7, 2, 3),
    (1, 2, 23, 40, 7, 7, 1, 3),
    (1, 4, 10, 7, 5, 3, 2, 2),
    (3, 2, 6, 6, 1, 1, 1, 0),
    (2, 6, 5, 9, 2, 4, 3, 0),
    (1, 2, 20, 20, 16, 16, 1, 0),
    (1, 3, 70, 130, 3, 3, 1, 1),
    (4, 37, 7, 7, 3, 3, 1, 1),
    (1, 2, 21, 600, 3, 3, 1, 1),
    (1, 1, 5, 300, 7, 7, 2, 3),
    (1, 2, 9, 3000, 3, 3, 1, 1),
    (1, 1, 4, 4, 3, 3, 1, 10),
    (2, 3, 20, 20, 3, 3, 5, 9),
    (3, 2, 7, 9, 2, 2, 3, 4),
    # small-plane form (3x3, stride 1, pad <= 1, rows of at most 32): planes
    # packed 18 a workgroup with a ragged last group, the widest row, pad 0,
    # the tallest output, and a single output pixel per plane
    (3, 37, 14, 14, 3, 3, 1, 1),
    (2, 5, 16, 32, 3, 3, 1, 1),
    (2, 4, 12, 10, 3, 3, 1, 0),
    (1, 3, 34, 6, 3, 3, 1, 0),
    (1, 2, 3, 3, 3, 3, 1, 0),
]
EPIS = [ct.CT_EPI_NONE, ct.CT_EPI_BIAS, ct.CT_EPI_EXP_BIAS_RSQRT]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _inputs(shape, dtype, seed):
    N, C, H, W, KH, KW, s, p = shape
    return wl.depthwise_inputs(wl.DepthwiseWorkload("dw_case", seed, N, C, H, W, KH, KW, s, p, dtype))


def _ref(inp, s, p, epi):
    y, a = O.conv2d_depthwise(inp["x"].astype(np.float64), inp["w"].astype(np.float64), s, p)
    if epi != ct.CT_EPI_NONE:
        y = O.channel_epilogue(y, epi, inp["bias"].astype(np.float64), inp["var"].astype(np.float64),
                               1e-5)
    return y, a


def _run(inp, dtype, s, p, epi, out=None):
    x, w = to_dev(inp["x"], dtype), to_dev(inp["w"], dtype)
    b = torch.from_numpy(inp["bias"]).to(DEV)
    v = torch.from_numpy(inp["var"]).to(DEV)
    y = ct.conv2d_depthwise(x, w, s, p, epi, b, v, 1e-5, out=out)
    torch.cuda.synchronize()
    return y


def _check(got, ref, absacc, epi, what):
    assert got.shape == ref.shape and np.all(np.isfinite(got)), what
    scale = float(absacc.max())
    if epi == ct.CT_EPI_EXP_BIAS_RSQRT:
        rel = float((np.abs(got - ref) / np.abs(ref)).max())
        say(f"  {what}: max rel = {rel:.3e}")
        assert rel <= GATE * scale + 1e-5, (what, rel)
    else:
        err = float(np.abs(got - ref).max())
        say(f"  {what}: max|gpu-ref| = {err:.3e} (gate {GATE * scale:.3e})")
        assert err <= GATE * scale, (what, err)


@pytest.mark.parametrize("epi", EPIS)
@pytest.mark.parametrize("dtype", [wl.F32, wl.F16, wl.BF16])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda t: "x".join(map(str, t)))
def test_depthwise_vs_oracle(shape, dtype, epi):
    inp = _inputs(shape, dtype, 80)
    s, p = shape[6], shape[7]
    ref, absacc = _ref(inp, s, p, epi)
    say(f"[dw] {shape} {dtype} epi={epi}")
    y = _run(inp, dtype, s, p, epi)
    _check(y.cpu().numpy().astype(np.float64), ref, absacc, epi, f"{shape} {dtype} epi={epi}")


@pytest.mark.parametrize("dtype", [wl.F32, wl.F16, wl.BF16])
def test_depthwise_small_integers_bit_exact(dtype):
    """Integer inputs in [-2, 2]: every partial sum is exact in fp32."""
    r = np.random.default_rng(81)
    for shape in [(2, 9, 30, 31, 3, 3, 1, 1), (3, 40, 7, 7, 5, 5, 2, 2), (1, 3, 19, 23, 4, 6, 3, 1)]:
        N, C, H, W, KH, KW, s, p = shape
        x = r.integers(-2, 3, (N, C, H, W)).astype(np.float32)
        w = r.integers(-2, 3, (C, 1, KH, KW)).astype(np.float32)
        say(f"[dw-int] {shape} {dtype}")
        y = ct.conv2d_depthwise(to_dev(wl.to_dtype(x, dtype), dtype), to_dev(wl.to_dtype(w, dtype), dtype),
                                s, p)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().astype(np.float64), O.conv2d_depthwise(x, w, s, p)[0]), shape


def test_depthwise_writes_only_its_output():
    """An output that starts 4 bytes into a buffer (not 16-byte aligned), with
    sentinels on both sides: every output written, nothing outside."""
    shape = (3, 5, 17, 19, 3, 3, 1, 1)
    inp = _inputs(shape, wl.F32, 82)
    ref, absacc = _ref(inp, 1, 1, ct.CT_EPI_NONE)
    n = ref.size
    buf = torch.full((n + 64,), -7.0, dtype=torch.float32, device=DEV)
    y = buf[1:1 + n].view(ref.shape)
    _run(inp, wl.F32, 1, 1, ct.CT_EPI_NONE, out=y)
    host = buf.cpu().numpy()
    assert host[0] == -7.0 and np.all(host[1 + n:] == -7.0)
    _check(host[1:1 + n].reshape(ref.shape).astype(np.float64), ref, absacc, ct.CT_EPI_NONE, "offset output")


def test_depthwise_on_a_stream():
    """The launch goes to the stream given."""
    shape = (2, 8, 40, 40, 3, 3, 1, 1)
    inp = _inputs(shape, wl.F32, 83)
    ref, absacc = _ref(inp, 1, 1, ct.CT_EPI_NONE)
    x, w = to_dev(inp["x"], wl.F32), to_dev(inp["w"], wl.F32)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = ct.conv2d_depthwise(x, w, 1, 1, stream=s)
    s.synchronize()
    _check(y.cpu().numpy().astype(np.float64), ref, absacc, ct.CT_EPI_NONE, "side stream")


@pytest.mark.parametrize("name", list(wl.DEPTHWISE_WORKLOADS))
def test_depthwise_full_size(name):
    """The benchmarked layers at full size, every output against the oracle."""
    d = wl.DEPTHWISE_WORKLOADS[name]
    inp = wl.depthwise_inputs(d)
    say(f"[dw-full] {name}")
    y = _run(inp, d.dtype, d.stride, d.pad, d.epilogue)
    got = y.cpu().numpy().astype(np.float64)
    del y
    ref, absacc = _ref(inp, d.stride, d.pad, d.epilogue)
    _check(got, ref, absacc, d.epilogue, name)


@pytest.mark.parametrize("dtype", [wl.F32, wl.F16])
def test_depthwise_unaligned_input(dtype):
    """An input that starts one element into its buffer (not 16-byte aligned:
    the scalar-load form) gives the same result as the oracle."""
    shape = (2, 6, 18, 24, 3, 3, 1, 1)
    inp = _inputs(shape, dtype, 84)
    ref, absacc = _ref(inp, 1, 1, ct.CT_EPI_NONE)
    x = to_dev(inp["x"], dtype)
    buf = torch.zeros(x.numel() + 16, dtype=x.dtype, device=DEV)
    xu = buf[1:1 + x.numel()].view(x.shape)
    xu.copy_(x)
    assert xu.data_ptr() % 16 != 0
    y = ct.conv2d_depthwise(xu, to_dev(inp["w"], dtype), 1, 1)
    torch.cuda.synchronize()
    _check(y.cpu().numpy().astype(np.float64), ref, absacc, ct.CT_EPI_NONE, f"unaligned x {dtype}")
