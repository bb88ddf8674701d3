"""The no-allocation entry point (ct_conv2d_nchw_fwd_noalloc) against the
allocating one (ct_conv2d_nchw_fwd), both through the C ABI: the same config
and kernel, so the same bits, and both within the oracle's gate.  Two calls
in a row, the second with a smaller input; capture into a HIP graph with no
earlier launch on the stream; the scratch limit."""
import os

import numpy as np
import pytest
import torch

from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl

from _gpu_helpers import CT_DT, DEV, TOL, oracle_full, say, to_dev

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHIPPED_LOG = os.path.join(ROOT, "tensor_compiler_tiling_amd", "tuned", "gfx950.jsonl")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()
    assert ct.ct_init(0) == 0
    assert ct.ct_cache_load(SHIPPED_LOG) == 0
    yield
    torch.cuda.synchronize()


def _tensors(w, inp):
    x = to_dev(inp["x"], w.dtype)
    k = to_dev(inp["w"], w.dtype)
    b = torch.from_numpy(inp["bias"]).to(DEV) if w.epilogue else None
    v = torch.from_numpy(inp["var"]).to(DEV) if w.epilogue else None
    return x, k, b, v


def _call(fn, w, x, k, b, v, y, stream=None):
    return fn(x, k, y, *w.shape_args(), CT_DT[w.dtype], w.epilogue, b, v, 1e-5, stream)


def _check_pair(w):
    inp = wl.conv_inputs(w)
    x, k, b, v = _tensors(w, inp)
    y_alloc = torch.full((w.N, w.CO, w.OH, w.OW), float("nan"), device=DEV)
    y_noalloc = torch.full_like(y_alloc, float("nan"))
    assert _call(ct.ct_conv2d_nchw_fwd, w, x, k, b, v, y_alloc) == 0
    st = _call(ct.ct_conv2d_nchw_fwd_noalloc, w, x, k, b, v, y_noalloc)
    assert st == 0, ct.library().ct_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(y_alloc.view(torch.int32), y_noalloc.view(torch.int32)), w.name
    ref, a = oracle_full(w, inp)
    got = y_noalloc.cpu().numpy().astype(np.float64)
    if w.epilogue == ct.CT_EPI_EXP_BIAS_RSQRT:
        from oracle import oracle as O
        ref = O.channel_epilogue(ref, w.epilogue, inp["bias"].astype(np.float64),
                                 inp["var"].astype(np.float64), 1e-5)
        err = float((np.abs(got - ref) / np.abs(ref)).max())
        gate = TOL[w.dtype] * float(a.max()) + 1e-5
    else:
        err = float(np.abs(got - ref).max())
        gate = TOL[w.dtype] * float(a.max())
    _, cfg, _ = ct.ct_conv2d_query(*w.shape_args(), CT_DT[w.dtype], w.epilogue)
    say(f"  {w.name}: {ct.variants()[cfg.variant]['name']} S={cfg.split_k}: bit-identical to the allocating "
        f"entry point, oracle err {err:.2e} (gate {gate:.2e})")
    assert err <= gate


# first call large, second smaller: fp32 split reduction; the half-precision
# kernel; the half-precision kernel with channel counts that are not a
# multiple of 8, whose reordered filter copy lives in the scratch
PAIRS = [
    ("resnet_final_c512_7x7_k3", "resnet_c64_14x14_k3"),
    ("f16_n64_c256_14x14_k3", wl.ConvWorkload("noalloc_f16_small", 140, 2, 32, 16, 16, 48, 3, 3, 1, 1, wl.F16,
                                               wl.EPI_EXP_BIAS_RSQRT)),
    (wl.ConvWorkload("noalloc_f16_ci36", 141, 8, 36, 20, 20, 96, 3, 3, 1, 1, wl.F16),
     wl.ConvWorkload("noalloc_f16_ci12", 142, 2, 12, 9, 11, 40, 3, 3, 1, 1, wl.F16)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=["fp32_split", "f16", "f16_reordered_filter"])
def test_noalloc_matches_the_allocating_entry_point(pair):
    for item in pair:
        w = wl.CONV_WORKLOADS[item] if isinstance(item, str) else item
        _check_pair(w)


def test_noalloc_captures_without_an_earlier_launch():
    """A fresh stream, no launch on it before capture: the no-allocation
    entry point captures (nothing to grow), and every replay gives the bits of
    the allocating entry point."""
    w = wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"]
    inp = wl.conv_inputs(w)
    x, k, b, v = _tensors(w, inp)
    ref = torch.empty((1, 512, 7, 7), device=DEV)
    assert _call(ct.ct_conv2d_nchw_fwd, w, x, k, b, v, ref) == 0
    torch.cuda.synchronize()
    y = torch.empty_like(ref)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = _call(ct.ct_conv2d_nchw_fwd_noalloc, w, x, k, b, v, y, s)
    assert st == 0, ct.library().ct_last_error().decode()
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), rep
    say("[noalloc] captured with no earlier launch; 3 replays match")


def test_noalloc_rejects_configs_beyond_its_scratch():
    """A half-precision 3x3 layer whose filter the launch reorders into its
    scratch (1024 x 1024 x 9 halves: 18.9 MB, beyond the fixed scratch), so
    the call fails before any launch; a call that fits still works
    afterwards."""
    w = wl.ConvWorkload("noalloc_big_filter", 90, 1, 1024, 16, 16, 1024, 3, 3, 1, 1, wl.F16)
    st, cfg, _ = ct.ct_conv2d_query(*w.shape_args(), ct.CT_F16, w.epilogue)
    assert st == 0
    name = ct.variants()[cfg.variant]["name"]
    assert name.startswith("h2"), name  # the reordering kernel is the one chosen
    assert 2 * 1024 * 1024 * 9 > ct.CT_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((w.N, w.CI, w.H, w.W), dtype=torch.float16, device=DEV)
    k = torch.zeros((w.CO, w.CI, w.KH, w.KW), dtype=torch.float16, device=DEV)
    b = torch.zeros(w.CO, device=DEV)
    v = torch.ones(w.CO, device=DEV)
    y = torch.empty((w.N, w.CO, w.OH, w.OW), device=DEV)
    st = _call(ct.ct_conv2d_nchw_fwd_noalloc, w, x, k, b, v, y)
    msg = ct.library().ct_last_error().decode()
    say(f"  {w.name} ({name}): status {st}: {msg}")
    assert st == ct.CT_ERR_UNSUPPORTED and "above the" in msg
    _check_pair(wl.CONV_WORKLOADS["resnet_c64_14x14_k3"])
