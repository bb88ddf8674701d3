"""GPU parity of the general per-channel broadcast (ct_broadcast_chain)
against the fp64 oracle, through the C ABI.

Gates: |gpu - ref| / max(|ref|, 1) within 1e-5 for fp32 output (chains of
at most 8 steps, each about 1 ulp in fp32, operands of order one; the floor of
1 covers outputs that cross zero) and within 1e-3 for fp16 output (one
rounding to fp16 on top).  The channel-bound and flat
forms must agree bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl

from _gpu_helpers import DEV, say, to_dev

pytestmark = pytest.mark.gpu

# named programs: (c0, c1, v) step lists; what each reads
PROGRAMS = {
    # the [1,C,1,1] => [N,C,H,W] of exp(var[c])
    "exp": ([("set", "a0"), ("exp",)], [], []),
    # batch-norm inference on a producer's output
    "bn": ([("set", "a0"), ("add", 1e-5), ("rsqrt",), ("mul", "a1")],
           [("set", "a2"), ("mul", "c0"), ("rsub", "a3")],
           [("set", "x"), ("mul", "c0"), ("add", "c1")]),
    # the fused convolution epilogue as a separate pass: exp(y + b) * rsqrt(v + eps)
    "epi": ([("set", "a1"), ("add", 1e-5), ("rsqrt",)], [],
            [("set", "x"), ("add", "a0"), ("exp",), ("mul", "c0")]),
    # every step kind once
    "mix": ([("set", "a0"), ("sqrt",), ("rdiv", 2.0)], [("set", "c0"), ("div", "a1"), ("sub", 0.25)],
            [("set", "x"), ("rsub", "c1"), ("mul", "a2"), ("div", 3.0), ("add", "c0")]),
}
READS_X = {"exp": False, "bn": True, "epi": True, "mix": True}

# (outer, P, inner): the degenerate 1x1x1, shapes only the flat form takes
# (inner < 32, rows not whole vectors), channel-bound shapes, P above 65535
SHAPES = [(1, 1, 1), (2, 3, 5), (3, 7, 33), (4, 16, 32), (3, 5, 100), (8, 256, 1024), (2, 3, 4096),
          (1, 70000, 32)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _arrays(P, seed):
    r = np.random.default_rng(seed)
    return [r.uniform(0.5, 2.0, P).astype(np.float32), r.uniform(0.5, 2.0, P).astype(np.float32),
            r.normal(0.0, 0.5, P).astype(np.float32), r.normal(0.0, 0.5, P).astype(np.float32)]


def _x(outer, P, inner, seed):
    return np.random.default_rng(seed).uniform(-1.0, 1.0, (outer, P, inner)).astype(np.float32)


def _run(prog_name, outer, P, inner, arrays, x, odt, mode):
    prog = ct.make_program(*PROGRAMS[prog_name])
    ta = [torch.from_numpy(a).to(DEV) for a in arrays]
    tx = torch.from_numpy(x).to(DEV) if x is not None else None
    out = ct.broadcast_chain(prog, outer, P, inner, ta, tx, out_dtype=odt, mode=mode)
    torch.cuda.synchronize()
    return out


def _gate(got, ref, odt, what):
    # relative to max(|ref|, 1): operands are of order one, and outputs that
    # cross zero (x * c0 + c1) lose relative accuracy to cancellation
    rel = float((np.abs(got - ref) / np.maximum(np.abs(ref), 1.0)).max())
    tol = 1e-5 if odt == torch.float32 else 1e-3
    say(f"  {what}: max rel = {rel:.3e} (gate {tol:.0e})")
    assert rel <= tol, (what, rel)


@pytest.mark.parametrize("odt", [torch.float32, torch.float16], ids=["f32", "f16"])
@pytest.mark.parametrize("name", list(PROGRAMS))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda t: "x".join(map(str, t)))
def test_chain_vs_oracle_and_forms_agree(shape, name, odt):
    outer, P, inner = shape
    arrays = _arrays(P, 95)
    x = _x(outer, P, inner, 96) if READS_X[name] else None
    say(f"[chain] {name} {shape} {odt}")
    auto = _run(name, outer, P, inner, arrays, x, odt, ct.CT_BC_AUTO)
    flat = _run(name, outer, P, inner, arrays, x, odt, ct.CT_BC_FLAT)
    assert torch.equal(auto.view(torch.int16 if odt == torch.float16 else torch.int32),
                       flat.view(torch.int16 if odt == torch.float16 else torch.int32)), "forms differ"
    vec = 8 if odt == torch.float16 else 4
    if inner >= 32 and inner % vec == 0:
        chan = _run(name, outer, P, inner, arrays, x, odt, ct.CT_BC_CHANNEL)
        assert torch.equal(chan.view(torch.int16 if odt == torch.float16 else torch.int32),
                           flat.view(torch.int16 if odt == torch.float16 else torch.int32)), "forms differ"
    ref = O.broadcast_chain(PROGRAMS[name], outer, P, inner, [a.astype(np.float64) for a in arrays],
                            None if x is None else x.astype(np.float64))
    _gate(auto.float().cpu().numpy().astype(np.float64), ref, odt, f"{name} {shape}")


@pytest.mark.parametrize("odt", [torch.float32, torch.float16], ids=["f32", "f16"])
def test_chain_exp_equals_the_nchw_broadcast(odt):
    """The chain set(a0), exp is the [1,C,1,1] => [N,C,H,W] broadcast: the
    same bits as ct_broadcast_nchw in both of its forms."""
    bw = wl.BROADCAST_WORKLOADS["bcast_exp_128x256x32x32_f16"]
    var = torch.from_numpy(wl.broadcast_var(bw)).to(DEV)
    N, C, H, W = 16, bw.C, 8, 12
    prog = ct.make_program([("set", "a0"), ("exp",)])
    for mode in (ct.CT_BC_CHANNEL, ct.CT_BC_FLAT):
        a = ct.broadcast_chain(prog, N, C, H * W, [var], out_dtype=odt, mode=mode)
        b = ct.broadcast(var, N, H, W, out_dtype=odt, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(a.reshape(N, C, H, W), b), mode


def test_chain_in_place_after_a_convolution():
    """The epilogue chain applied in place to a convolution's output equals
    the oracle's convolution followed by its epilogue."""
    w = wl.ConvWorkload("chain_after_conv", 97, 2, 16, 9, 9, 24, 3, 3, 1, 1, wl.F32)
    inp = wl.conv_inputs(w)
    y = ct.conv2d(to_dev(inp["x"], wl.F32), to_dev(inp["w"], wl.F32), 1, 1)
    b = torch.from_numpy(inp["bias"]).to(DEV)
    v = torch.from_numpy(inp["var"]).to(DEV)
    prog = ct.make_program(*PROGRAMS["epi"])
    out = ct.broadcast_chain(prog, w.N, w.CO, w.OH * w.OW, [b, v], x=y, out=y)
    torch.cuda.synchronize()
    assert out.data_ptr() == y.data_ptr()
    yr, _ = O.conv2d_nchw(inp["x"].astype(np.float64), inp["w"].astype(np.float64), 1, 1)
    ref = O.channel_epilogue(yr, 2, inp["bias"].astype(np.float64), inp["var"].astype(np.float64), 1e-5)
    got = y.cpu().numpy().astype(np.float64)
    rel = float((np.abs(got - ref) / np.abs(ref)).max())
    say(f"  conv + chain in place: max rel = {rel:.3e}")
    # the convolution's own fp32 error (1e-4 of the tap sum) passes through exp
    _, absacc = O.conv2d_nchw(inp["x"].astype(np.float64), inp["w"].astype(np.float64), 1, 1)
    assert rel <= 1e-4 * float(absacc.max()) + 1e-5


def test_chain_unaligned_output_takes_the_flat_form():
    """An output 4 bytes into its buffer: AUTO falls back to the flat form and
    writes exactly the output, nothing around it."""
    outer, P, inner = 3, 5, 64
    arrays = _arrays(P, 98)
    prog = ct.make_program(*PROGRAMS["exp"])
    n = outer * P * inner
    buf = torch.full((n + 8,), -3.0, dtype=torch.float32, device=DEV)
    o = buf[1:1 + n].view(outer, P, inner)
    ct.broadcast_chain(prog, outer, P, inner, [torch.from_numpy(arrays[0]).to(DEV)], out=o)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert host[0] == -3.0 and np.all(host[1 + n:] == -3.0)
    ref = O.broadcast_chain(PROGRAMS["exp"], outer, P, inner, [arrays[0].astype(np.float64)])
    _gate(host[1:1 + n].reshape(outer, P, inner).astype(np.float64), ref, torch.float32, "unaligned")


def test_chain_swapped_grid():
    """More than 65535 row blocks: the channel-bound grid puts the row blocks
    on its first axis (a block takes 32 KiB = 512 rows of 32 fp16 outputs;
    33.6 M rows, 2 channels: a 4.3 GB output)."""
    outer, P, inner = 65536 * 512 + 3, 2, 32
    arrays = _arrays(P, 99)
    prog = ct.make_program(*PROGRAMS["exp"])
    out = ct.broadcast_chain(prog, outer, P, inner, [torch.from_numpy(arrays[0]).to(DEV)],
                             out_dtype=torch.float16, mode=ct.CT_BC_CHANNEL)
    torch.cuda.synchronize()
    ref = np.exp(arrays[0].astype(np.float64))
    for p in range(P):
        col = out[:, p, :]
        assert bool((col == col[0, 0]).all()), p
        _gate(np.array([float(col[0, 0])]), ref[p:p + 1], torch.float16, f"swapped p={p}")
    del out


@pytest.mark.parametrize("name", list(wl.CHAIN_WORKLOADS))
def test_chain_full_size(name):
    """The benchmarked workload at full size in the launch bench.py times
    (channel-bound), every element against the oracle."""
    cw = wl.CHAIN_WORKLOADS[name]
    inp = wl.chain_inputs(cw)
    prog = ct.make_program(*wl.CHAIN_PROGRAMS[cw.program])
    say(f"[chain-full] {name}")
    out = ct.broadcast_chain(prog, cw.outer, cw.P, cw.inner, [torch.from_numpy(v).to(DEV) for v in inp["arrays"]],
                             torch.from_numpy(inp["x"]).to(DEV), mode=ct.CT_BC_CHANNEL)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    del out
    ref = O.broadcast_chain(wl.CHAIN_PROGRAMS[cw.program], cw.outer, cw.P, cw.inner,
                            [v.astype(np.float64) for v in inp["arrays"]], inp["x"].astype(np.float64))
    # batch-norm output crosses zero: gate relative to the larger of |ref| and the operands' scale
    err = float((np.abs(got - ref) / np.maximum(np.abs(ref), 1.0)).max())
    say(f"  {name}: max err = {err:.3e}")
    assert err <= 1e-5, err
