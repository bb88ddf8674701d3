"""Determinism and HIP-graph replay of the entry points added beside the
convolution: the depthwise convolution, the general per-channel broadcast
and the matrix product.  Two eager runs must give the same bits; a captured
graph is replayed several times, with eager work and synchronisations in
between, and every replay must give the eager run's bits."""
import numpy as np
import pytest
import torch

from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl

from _gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _cases():
    d = wl.DepthwiseWorkload("replay_dw", 110, 4, 24, 30, 31, 3, 3, 1, 1, wl.F16, wl.EPI_BIAS)
    dinp = wl.depthwise_inputs(d)
    dx = torch.from_numpy(dinp["x"]).to(DEV)
    dw_ = torch.from_numpy(dinp["w"]).to(DEV)
    db = torch.from_numpy(dinp["bias"]).to(DEV)
    dv = torch.from_numpy(dinp["var"]).to(DEV)
    dy = torch.empty((d.N, d.C, d.OH, d.OW), dtype=torch.float32, device=DEV)

    cw = wl.ChainWorkload("replay_chain", 111, 8, 48, 256, "batchnorm")
    cinp = wl.chain_inputs(cw)
    cx = torch.from_numpy(cinp["x"]).to(DEV)
    ca = [torch.from_numpy(v).to(DEV) for v in cinp["arrays"]]
    co = torch.empty((cw.outer, cw.P, cw.inner), dtype=torch.float32, device=DEV)
    prog = ct.make_program(*wl.CHAIN_PROGRAMS[cw.program])

    g = wl.GemmWorkload("replay_gemm", 112, 200, 600, 300, wl.F16)
    ginp = wl.gemm_inputs(g)
    gA = torch.from_numpy(ginp["A"]).to(DEV)
    gB = torch.from_numpy(ginp["B"]).to(DEV)
    gC = torch.empty((g.M, g.N), dtype=torch.float32, device=DEV)
    return {
        "depthwise": (lambda s=None: ct.conv2d_depthwise(dx, dw_, 1, 1, wl.EPI_BIAS, db, dv, out=dy, stream=s), dy),
        "chain": (lambda s=None: ct.broadcast_chain(prog, cw.outer, cw.P, cw.inner, ca, cx, out=co, stream=s), co),
        "gemm": (lambda s=None: ct.gemm(gA, gB, out=gC, stream=s), gC),
    }


@pytest.mark.parametrize("name", ["depthwise", "chain", "gemm"])
def test_two_eager_runs_give_the_same_bits(name):
    run, out = _cases()[name]
    run()
    torch.cuda.synchronize()
    first = out.clone()
    out.fill_(float("nan"))
    run()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int32), out.view(torch.int32)), name


@pytest.mark.parametrize("name", ["depthwise", "chain", "gemm"])
def test_graph_replays_match_the_eager_run(name):
    run, out = _cases()[name]
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    # one eager run on the capture stream first: the library's per-stream
    # workspaces exist before capture (they cannot grow while capturing)
    with torch.cuda.stream(s):
        run(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(s)
    for rep in range(4):
        out.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int32), out.view(torch.int32)), (name, rep)
    say(f"[replay] {name}: 4 graph replays match the eager run")
