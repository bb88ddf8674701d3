"""GPU parity of the per-channel broadcast [1,C,1,1] -> [N,C,H,W] of exp(var[c])
against the fp64 oracle, through the C ABI, in every binding mode."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl

from _gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

MODES = [ct.CT_BC_AUTO, ct.CT_BC_CHANNEL, ct.CT_BC_FLAT]


def _ulp16(v: np.ndarray) -> np.ndarray:
    """Spacing of fp16 values around |v| (normal range)."""
    e = np.floor(np.log2(np.abs(v)))
    return np.exp2(e - 10)


def _check(var: np.ndarray, out: torch.Tensor, N, H, W, dtype):
    ref = O.broadcast_exp(var.astype(np.float64), N, H, W)
    got = out.float().cpu().numpy().astype(np.float64)
    # every element of a channel is bitwise the same value
    assert torch.equal(out, out[:1, :, :1, :1].expand_as(out))
    if dtype == torch.float16:
        # nearest-even rounding of an exp that is good to ~1e-6: within 1 fp16 ulp
        err_ulp = float((np.abs(got - ref) / _ulp16(ref)).max())
        say(f"  max error {err_ulp:.3f} fp16 ulp")
        assert err_ulp <= 1.0
    else:
        rel = float((np.abs(got - ref) / ref).max())
        say(f"  max rel error {rel:.3e}")
        assert rel <= 4e-6  # a few fp32 ulps from 2^(x log2 e)


@pytest.mark.parametrize("name", list(wl.BROADCAST_WORKLOADS))
@pytest.mark.parametrize("mode", MODES)
def test_broadcast_workload(name, mode):
    bw = wl.BROADCAST_WORKLOADS[name]
    say(f"[bcast] {name} mode={mode}")
    var = wl.broadcast_var(bw)
    dt = torch.float16 if bw.out_dtype == wl.F16 else torch.float32
    v = torch.from_numpy(var).to(DEV)
    out = torch.full((bw.N, bw.C, bw.H, bw.W), float("nan"), dtype=dt, device=DEV)
    ct.broadcast(v, bw.N, bw.H, bw.W, out=out, mode=mode)
    torch.cuda.synchronize()
    _check(var, out, bw.N, bw.H, bw.W, dt)


@pytest.mark.parametrize("shape", [(1, 3, 1, 1), (2, 5, 3, 7), (3, 64, 8, 4), (1, 300, 16, 2),
                                   (70000, 2, 4, 8), (5, 1, 33, 33)])
@pytest.mark.parametrize("dt", [torch.float16, torch.float32])
def test_broadcast_odd_shapes(shape, dt):
    N, C, H, W = shape
    var = np.random.default_rng(C).uniform(-3.0, 3.0, C).astype(np.float32)
    v = torch.from_numpy(var).to(DEV)
    for mode in MODES:
        out = torch.full(shape, float("nan"), dtype=dt, device=DEV)
        chan_ok = (H * W) % 32 == 0
        st = ct.ct_broadcast_nchw(v, out, N, C, H, W, ct.dtype_code(dt), ct.CT_BC_EXP, mode)
        if mode == ct.CT_BC_CHANNEL and not chan_ok:
            assert st == ct.CT_ERR_UNSUPPORTED
            continue
        assert st == 0, ct.ct_last_error()
        torch.cuda.synchronize()
        _check(var, out, N, H, W, dt)


def test_broadcast_misaligned_output_falls_back():
    var = np.linspace(0.5, 2.0, 8).astype(np.float32)
    v = torch.from_numpy(var).to(DEV)
    buf = torch.zeros(2 * 8 * 32 + 1, dtype=torch.float16, device=DEV)
    view = buf[1:]  # 2-byte offset: not 16-byte aligned
    st = ct.ct_broadcast_nchw(v, view.data_ptr(), 2, 8, 4, 8, ct.CT_F16, ct.CT_BC_EXP,
                              ct.CT_BC_CHANNEL)
    assert st == ct.CT_ERR_UNSUPPORTED
    st = ct.ct_broadcast_nchw(v, view.data_ptr(), 2, 8, 4, 8, ct.CT_F16, ct.CT_BC_EXP,
                              ct.CT_BC_AUTO)
    assert st == 0
    torch.cuda.synchronize()
    assert buf[0].item() == 0.0
    _check(var, view.view(2, 8, 4, 8), 2, 4, 8, torch.float16)
