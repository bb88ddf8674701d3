"""GPU parity of the convolution path against the fp64 oracle, through the C ABI.

Gates: max |gpu - ref| <= 1e-4 * S for every input dtype, S = max over
outputs of sum |xp * w| (the oracle's absacc).  fp16 / bf16 inputs get the
fp32 gate because their products are exact in fp32 (11- or 8-bit
significands) and the kernels accumulate in fp32, so the only error is the
same fp32 summation error; the oracle consumes the same rounded values.
Also: bit-exact output for small-integer inputs, whose partial sums are exact in
fp32 in any order; bit-identical repeat runs.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl

from _gpu_helpers import (CT_DT, DEV, TOL, assert_conv_close, legal_configs, oracle_full, run, say,
                          to_dev)

pytestmark = pytest.mark.gpu

FP32_FULL = ["resnet_c64_14x14_k3", "resnet_final_c512_7x7_k3"] + wl.SWEEP
ODD = [
    wl.ConvWorkload("odd_h13_co48", 101, 1, 16, 13, 13, 48, 3, 3, 1, 1),
    wl.ConvWorkload("odd_ci3_s2", 102, 1, 3, 17, 19, 40, 3, 3, 2, 1),
    wl.ConvWorkload("odd_batch3_cross", 103, 3, 5, 5, 6, 8, 3, 3, 1, 1),
    wl.ConvWorkload("odd_k7_s3_p2", 104, 2, 6, 23, 21, 20, 7, 7, 3, 2),
    wl.ConvWorkload("odd_k1_s2_p0", 105, 2, 24, 9, 11, 33, 1, 1, 2, 0),
    wl.ConvWorkload("odd_k5x3_p0", 106, 1, 9, 12, 10, 70, 5, 3, 1, 0),
    wl.ConvWorkload("odd_k2_s2", 107, 4, 12, 8, 8, 130, 2, 2, 2, 0),
    wl.ConvWorkload("odd_tiny", 108, 1, 1, 1, 1, 1, 1, 1, 1, 0),
    wl.ConvWorkload("odd_pad_bigger_than_input", 109, 1, 2, 2, 3, 3, 3, 3, 1, 2),
    wl.ConvWorkload("odd_n130_1x1", 110, 130, 7, 3, 3, 9, 3, 3, 1, 1),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    torch.cuda.init()
    ct.ct_cache_clear()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", FP32_FULL)
def test_default_config_full_workload(name):
    w = wl.CONV_WORKLOADS[name]
    say(f"[conv] {name} default config")
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    got = run(w, inp)
    assert_conv_close(got, y, a, w.dtype, name)
    st, cfg, _ = ct.ct_conv2d_query(*w.shape_args(), CT_DT[w.dtype], w.epilogue)
    say(f"  config: {ct.variants()[cfg.variant]['name']} S={cfg.split_k} stages={cfg.stages} "
        f"kc={cfg.kc}")


@pytest.mark.parametrize("name", FP32_FULL)
def test_direct_kernel_full_workload(name):
    w = wl.CONV_WORKLOADS[name]
    say(f"[conv-direct] {name}")
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    assert_conv_close(run(w, inp, direct=True), y, a, w.dtype, name + " direct")


@pytest.mark.parametrize("name", ["resnet_final_c512_7x7_k3", "resnet_c64_14x14_k3",
                                  "r18_c256to512_14x14_k3s2", "r18_c256_14x14_k1"])
def test_every_legal_config(name):
    """Each point of the space that passes the legality check computes the
    same convolution (variants x split_k x stages x kc)."""
    w = wl.CONV_WORKLOADS[name]
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    cfgs = legal_configs(w)
    say(f"[conv-space] {name}: {len(cfgs)} legal configs")
    assert cfgs
    x = to_dev(inp["x"], w.dtype)
    k = to_dev(inp["w"], w.dtype)
    scale = float(a.max())
    worst = 0.0
    for cfg in cfgs:
        out = torch.full((w.N, w.CO, w.OH, w.OW), float("nan"), device=DEV)
        ct.conv2d(x, k, w.stride, w.pad, config=cfg, out=out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        err = float(np.abs(got - y).max())
        worst = max(worst, err)
        assert np.all(np.isfinite(got)) and err <= 1e-4 * scale, (
            ct.variants()[cfg.variant]["name"], cfg.split_k, cfg.stages, cfg.kc, err)
    say(f"  worst max|gpu-ref| over configs = {worst:.3e} (gate {1e-4 * scale:.3e})")


@pytest.mark.parametrize("w", ODD, ids=lambda w: w.name)
def test_odd_shapes_every_config(w):
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    cfgs = legal_configs(w)
    say(f"[conv-odd] {w.name}: {len(cfgs)} legal configs")
    assert_conv_close(run(w, inp), y, a, w.dtype, w.name + " default")
    assert_conv_close(run(w, inp, direct=True), y, a, w.dtype, w.name + " direct")
    for cfg in cfgs:
        got = run(w, inp, config=cfg)
        err = float(np.abs(got - y).max())
        assert err <= 1e-4 * float(a.max()), (ct.variants()[cfg.variant]["name"], cfg.split_k,
                                              cfg.stages, cfg.kc, err)


@pytest.mark.parametrize("name", FP32_FULL)
def test_small_integers_bit_exact(name):
    """Integer inputs in [-2, 2]: exact in fp32 whatever the summation order,
    so every config must reproduce the oracle bit for bit (padding included)."""
    w = wl.CONV_WORKLOADS[name]
    inp = wl.small_int_inputs(w)
    y, _ = O.conv2d_nchw(inp["x"].astype(np.float64), inp["w"].astype(np.float64), w.stride, w.pad)
    assert np.abs(y).max() < 2 ** 24
    say(f"[conv-int] {name}")
    assert np.array_equal(run(w, inp), y)
    assert np.array_equal(run(w, inp, direct=True), y)
    cfgs = legal_configs(w)
    step = max(1, len(cfgs) // 12)
    for cfg in cfgs[::step]:
        got = run(w, inp, config=cfg)
        assert np.array_equal(got, y), (ct.variants()[cfg.variant]["name"], cfg.split_k,
                                        cfg.stages, cfg.kc)


def test_ones_count_valid_taps():
    w = wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"]
    inp = {"x": np.ones((1, 512, 7, 7), np.float32), "w": np.ones((512, 512, 3, 3), np.float32)}
    got = run(w, inp)
    assert got[0, 0, 0, 0] == 2048 and got[0, 5, 0, 3] == 3072 and got[0, 511, 3, 3] == 4608
    exp = np.full((7, 7), 9.0)
    exp[0, :] -= 3; exp[-1, :] -= 3; exp[:, 0] -= 3; exp[:, -1] -= 3
    exp[0, 0] = exp[0, -1] = exp[-1, 0] = exp[-1, -1] = 4
    assert np.array_equal(got[0], np.broadcast_to(512 * exp, (512, 7, 7)))


# Layers with the compiled geometries of the shape-specialised kernels
# ("f32skc*": 3x3 pad 1 at 7x7 stride 1, 14x14 stride 2 and 14x14 stride 1
# in 7x7 quadrants; 1x1 at 14x14 and 3x3 stride 2 at 28x28 in quadrants;
# 3x3 at 56x56, stride 1 and 2, in tile windows; "f32skt*": the 3-channel
# 7x7 stride-2 layer at 224x224), at output-channel counts that leave a
# partial 16-row tile, and the full first layer.
SKC_LAYERS = [
    wl.ConvWorkload("skc_7x7_ci64_co40", 111, 1, 64, 7, 7, 40, 3, 3, 1, 1),
    wl.ConvWorkload("skc_14x14s2_ci64_co24", 112, 1, 64, 14, 14, 24, 3, 3, 2, 1),
    # 14x14 stride 1: four 7x7 quadrant column tiles
    wl.ConvWorkload("skc_14x14q_ci64_co40", 113, 1, 64, 14, 14, 40, 3, 3, 1, 1),
    # 1x1 filter, 14x14, quadrants
    wl.ConvWorkload("skc_14x14q_1x1_ci64_co40", 114, 1, 64, 14, 14, 40, 1, 1, 1, 0),
    # 28x28 stride 2: a 14x14 output in quadrants
    wl.ConvWorkload("skc_28x28s2q_ci32_co24", 115, 1, 32, 28, 28, 24, 3, 3, 2, 1),
    # 56x56, stride 1 and 2: 7x7 tiles, each staging only its receptive field
    wl.ConvWorkload("skc_56x56w_ci64_co24", 116, 1, 64, 56, 56, 24, 3, 3, 1, 1),
    wl.ConvWorkload("skc_56x56s2w_ci64_co40", 117, 1, 64, 56, 56, 40, 3, 3, 2, 1),
    # 3-channel 7x7 stride-2 first layer: lane groups split the filter rows;
    # 40 output channels leave a partial channel tile
    wl.ConvWorkload("skt_stem_c3_224x224_k7s2_co40", 118, 1, 3, 224, 224, 40, 7, 7, 2, 3),
    wl.CONV_WORKLOADS["r18_stem_c3_224x224_k7s2"],
]


def _skc_configs(w):
    return [c for c in legal_configs(w)
            if ct.variants()[c.variant]["name"].startswith(("f32skc", "f32skt"))]


@pytest.mark.parametrize("misaligned", ["none", "x", "w", "y"],
                         ids=["aligned", "x_offset_4B", "w_offset_4B", "y_offset_4B"])
@pytest.mark.parametrize("epi", [ct.CT_EPI_NONE, ct.CT_EPI_BIAS, ct.CT_EPI_EXP_BIAS_RSQRT])
@pytest.mark.parametrize("w", SKC_LAYERS, ids=lambda w: w.name)
def test_shape_specialised_split_k(w, epi, misaligned):
    """Every legal config of the shape-specialised kernels against the oracle:
    conv gate, epilogue gates, an input that is not 16-byte aligned (the
    kernels then load the window word by word), a filter that is not, and an
    output that is not (16-byte stores fall back to words)."""
    w = w.with_(epilogue=epi)
    cfgs = _skc_configs(w)
    say(f"[conv-skc] {w.name} epi={epi} misaligned={misaligned}: {len(cfgs)} configs")
    assert cfgs
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    ref = y if epi == ct.CT_EPI_NONE else O.channel_epilogue(
        y, epi, inp["bias"].astype(np.float64), inp["var"].astype(np.float64), 1e-5)
    S = float(a.max())
    xd = to_dev(inp["x"], w.dtype)
    if misaligned == "x":
        buf = torch.empty(xd.numel() + 1, dtype=xd.dtype, device=DEV)
        buf[1:].copy_(xd.reshape(-1))
        xd = buf[1:].view(xd.shape)
        assert xd.data_ptr() % 16 != 0
    k = to_dev(inp["w"], w.dtype)
    if misaligned == "w":
        buf = torch.empty(k.numel() + 1, dtype=k.dtype, device=DEV)
        buf[1:].copy_(k.reshape(-1))
        k = buf[1:].view(k.shape)
        assert k.data_ptr() % 16 != 0
    b = torch.from_numpy(inp["bias"]).to(DEV)
    v = torch.from_numpy(inp["var"]).to(DEV)
    for cfg in cfgs:
        out = None
        if misaligned == "y":
            ybuf = torch.full((w.N * w.CO * w.OH * w.OW + 1,), float("nan"), device=DEV)
            out = ybuf[1:].view(w.N, w.CO, w.OH, w.OW)
            assert out.data_ptr() % 16 != 0
        got = ct.conv2d(xd, k, w.stride, w.pad, epi, b, v, 1e-5, config=cfg, out=out)
        torch.cuda.synchronize()
        if out is not None:
            assert got.data_ptr() == out.data_ptr()
            assert torch.isnan(ybuf[:1]).all(), "a store landed before the output"
        got = got.cpu().numpy().astype(np.float64)
        what = (ct.variants()[cfg.variant]["name"], cfg.split_k, cfg.stages, cfg.kc)
        assert np.all(np.isfinite(got)), what
        if epi == ct.CT_EPI_EXP_BIAS_RSQRT:
            rel = float((np.abs(got - ref) / np.abs(ref)).max())
            assert rel <= 1e-4 * S + 1e-5, (what, rel)
        else:
            assert float(np.abs(got - ref).max()) <= 1e-4 * S, what


@pytest.mark.parametrize("w", SKC_LAYERS + [wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"],
                                            wl.CONV_WORKLOADS["r18_c256to512_14x14_k3s2"],
                                            wl.CONV_WORKLOADS["resnet_c64_14x14_k3"]],
                         ids=lambda w: w.name)
def test_shape_specialised_integers_bit_exact(w):
    inp = wl.small_int_inputs(w)
    y, _ = O.conv2d_nchw(inp["x"].astype(np.float64), inp["w"].astype(np.float64), w.stride, w.pad)
    cfgs = _skc_configs(w)
    say(f"[conv-skc-int] {w.name}: {len(cfgs)} configs")
    assert cfgs
    for cfg in cfgs:
        assert np.array_equal(run(w, inp, config=cfg), y), (ct.variants()[cfg.variant]["name"],
                                                            cfg.split_k, cfg.stages, cfg.kc)


def test_xcd_local_variants_enabled():
    """The XCD-local split-K variants are legal on this device only if the
    runtime's placement probe saw workgroup b run on XCD b % 8."""
    w = wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"]
    names = {ct.variants()[c.variant]["name"] for c in legal_configs(w)}
    xl = sorted(n for n in names if n.startswith("f32skc7x_"))
    say(f"[conv-xcd-local] legal XCD-local variants: {xl}")
    assert xl, "placement probe did not observe round-robin XCD placement"


def test_split_reduction_interleaved_configs():
    """Back-to-back launches on one stream of the shape-specialised split-K
    kernels with split counts that change from launch to launch, interleaved
    with the other split-K kernels that share the stream's tickets and
    workspace: each result is bit-identical to the first run of its config,
    and the first runs match the oracle."""
    w = wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"]
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    x = to_dev(inp["x"], w.dtype)
    k = to_dev(inp["w"], w.dtype)
    cfgs = [c for c in legal_configs(w) if c.split_k > 1]
    skc = [c for c in cfgs if ct.variants()[c.variant]["name"].startswith("f32skc")]
    other = [c for c in cfgs if not ct.variants()[c.variant]["name"].startswith("f32skc")][:4]
    assert len({c.split_k for c in skc}) > 1 and other
    order = []
    for rep in range(3):
        for i, c in enumerate(skc):
            order.append(c)
            if i % 2 == rep % 2:
                order.append(other[(i + rep) % len(other)])
    first = {}
    outs = []
    for c in order:
        outs.append((c, ct.conv2d(x, k, 1, 1, config=c)))
    torch.cuda.synchronize()
    for c, out in outs:
        key = (c.variant, c.split_k, c.stages, c.kc)
        if key not in first:
            first[key] = out
            err = float(np.abs(out.cpu().numpy().astype(np.float64) - y).max())
            assert err <= 1e-4 * float(a.max()), (ct.variants()[c.variant]["name"], key, err)
        else:
            assert torch.equal(out, first[key]), (ct.variants()[c.variant]["name"], key)
    say(f"[conv-split-interleaved] {len(order)} launches, {len(first)} configs")


def test_split_reduction_is_deterministic():
    w = wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"]
    inp = wl.conv_inputs(w)
    x = to_dev(inp["x"], w.dtype)
    k = to_dev(inp["w"], w.dtype)
    for cfg in [c for c in legal_configs(w) if c.split_k > 1][:8]:
        y1 = ct.conv2d(x, k, 1, 1, config=cfg)
        y2 = ct.conv2d(x, k, 1, 1, config=cfg)
        for _ in range(5):  # back-to-back launches reuse the tickets
            y3 = ct.conv2d(x, k, 1, 1, config=cfg)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(y1, y3)


@pytest.mark.parametrize("epi", [ct.CT_EPI_BIAS, ct.CT_EPI_EXP_BIAS_RSQRT])
@pytest.mark.parametrize("name", ["resnet_final_c512_7x7_k3", "r18_c64_56x56_k3"])
def test_fused_epilogue_fp32(name, epi):
    w = wl.CONV_WORKLOADS[name].with_(epilogue=epi)
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    ref = O.channel_epilogue(y, epi, inp["bias"].astype(np.float64), inp["var"].astype(np.float64),
                             1e-5)
    S = float(a.max())
    for cfg in [None] + legal_configs(w)[::7]:
        got = run(w, inp, config=cfg)
        if epi == ct.CT_EPI_BIAS:
            err = float(np.abs(got - ref).max())
            assert err <= 1e-4 * S
        else:
            # exp turns an absolute error e of the pre-activation into a
            # relative error of about e; rsqrt adds about 1e-7
            rel = float((np.abs(got - ref) / np.abs(ref)).max())
            assert rel <= 1e-4 * S + 1e-5, rel
    say(f"[epi] {name} epi={epi} ok")


def test_epilogue_closed_form_zero_weights():
    w = wl.ConvWorkload("zero_w", 120, 2, 8, 6, 6, 40, 3, 3, 1, 1, wl.F32, ct.CT_EPI_EXP_BIAS_RSQRT)
    inp = wl.conv_inputs(w)
    inp["w"] = np.zeros_like(inp["w"])
    got = run(w, inp)
    b = inp["bias"].astype(np.float64)
    v = inp["var"].astype(np.float64)
    want = np.exp(b) / np.sqrt(v + 1e-5)
    rel = np.abs(got - want[None, :, None, None]) / want[None, :, None, None]
    assert rel.max() < 2e-6
    # every element of a channel is bitwise the same value
    assert np.all(got == got[:, :, :1, :1])


HALF_SMALL = [
    # N, CI, H, W, CO, KH, KW, stride, pad: odd width (1-pixel window runs),
    # a partial channel stage and windows that cross images
    ("half_small", 130, 3, 24, 11, 9, 40, 3, 3, 1, 1),
    # width 16: 8-pixel runs; 32 channels: whole stages
    ("half_w16", 131, 2, 32, 16, 16, 48, 3, 3, 1, 1),
    # width 14: 2-pixel runs, 40 channels (a partial stage), 70 filters
    ("half_w14", 132, 2, 40, 10, 14, 70, 3, 3, 1, 1),
    # width 12, stride 2: 4-pixel runs
    ("half_w12_s2", 133, 1, 16, 12, 12, 32, 3, 3, 2, 1),
    # 12 channels, not a multiple of 8: the filter goes through the reordered
    # copy instead of being staged from the caller's layout
    ("half_ci12", 136, 2, 12, 9, 11, 40, 3, 3, 1, 1),
    # batch 1 with a last stage that starts within 8 channels of CI: the
    # window loads of its channels past CI come from descriptors placed past
    # the whole tensor (an empty range: zeros)
    ("half_n1_ci20", 137, 1, 20, 10, 10, 40, 3, 3, 1, 1),
]


@pytest.mark.parametrize("shape", HALF_SMALL, ids=lambda t: t[0])
@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_half_precision_small(dtype, shape):
    w = wl.ConvWorkload(*shape, dtype)
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    assert_conv_close(run(w, inp), y, a, dtype, f"{dtype} default")
    assert_conv_close(run(w, inp, direct=True), y, a, dtype, f"{dtype} direct")
    for cfg in legal_configs(w):
        assert_conv_close(run(w, inp, config=cfg), y, a, dtype,
                          f"{dtype} {ct.variants()[cfg.variant]['name']} S={cfg.split_k}")
    ints = wl.small_int_inputs(w)
    yi, _ = O.conv2d_nchw(ints["x"].astype(np.float64), ints["w"].astype(np.float64), w.stride,
                          w.pad)
    assert np.array_equal(run(w, ints), yi)
    for cfg in legal_configs(w):
        assert np.array_equal(run(w, ints, config=cfg), yi), ct.variants()[cfg.variant]["name"]
    # a filter that is not 16-byte aligned (staged with 2-byte loads)
    x = to_dev(ints["x"], dtype)
    k = to_dev(ints["w"], dtype)
    buf = torch.empty(k.numel() + 1, dtype=k.dtype, device=DEV)
    buf[1:].copy_(k.reshape(-1))
    k1 = buf[1:].view(k.shape)
    assert k1.data_ptr() % 16 != 0
    for cfg in [None] + legal_configs(w):
        got = ct.conv2d(x, k1, w.stride, w.pad, config=cfg)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().astype(np.float64), yi), ("misaligned w", cfg)
    # an output that is not 16-byte aligned (stored element by element)
    ybuf = torch.empty(yi.size + 1, device=DEV)
    y1 = ybuf[1:].view(yi.shape)
    assert y1.data_ptr() % 16 != 0
    for cfg in [None] + legal_configs(w):
        y1.fill_(float("nan"))
        ct.conv2d(x, k, w.stride, w.pad, config=cfg, out=y1)
        torch.cuda.synchronize()
        assert np.array_equal(y1.cpu().numpy().astype(np.float64), yi), ("misaligned y", cfg)


HALF_FULL = ["f16_n64_c256_14x14_k3", "f16_n128_c128to256_32x32_k3_epi"]
_FULL_REF = {}


def _half_full_reference(name):
    """The whole fp64 oracle pass of a full-size half-precision workload
    (y and its sum |xp*w| scale), computed once per module."""
    if name not in _FULL_REF:
        w = wl.CONV_WORKLOADS[name]
        inp = wl.conv_inputs(w)
        say(f"  oracle: full fp64 pass of {name} ({w.flops / 1e9:.1f} GFLOP)")
        y, a = oracle_full(w, inp)
        _FULL_REF[name] = (inp, y, a)
    return _FULL_REF[name]


@pytest.mark.parametrize("name", HALF_FULL)
def test_half_precision_full_size(name):
    """Full-size half-precision workloads in the default launch config, every
    output against the full oracle pass: the convolution alone (epilogue off)
    under the conv gate, then the fused run under the relative gate."""
    w = wl.CONV_WORKLOADS[name]
    say(f"[conv-f16-full] {name}")
    inp, y, a = _half_full_reference(name)
    got = run(w, inp, epilogue=ct.CT_EPI_NONE)
    assert_conv_close(got, y, a, w.dtype, name + " conv-only")
    if w.epilogue != ct.CT_EPI_NONE:
        S = float(a.max())
        ref = O.channel_epilogue(y, w.epilogue, inp["bias"].astype(np.float64),
                                 inp["var"].astype(np.float64), 1e-5)
        fused = run(w, inp)
        assert np.all(np.isfinite(fused))
        rel = float((np.abs(fused - ref) / np.abs(ref)).max())
        say(f"  fused: max rel err = {rel:.3e} (gate {TOL[w.dtype] * S + 1e-5:.3e})")
        assert rel <= TOL[w.dtype] * S + 1e-5


@pytest.mark.parametrize("name", HALF_FULL)
def test_half_precision_full_size_every_variant(name):
    """Full-size half-precision workloads through every variant (one split
    factor each: the smallest legal one), every output against the oracle."""
    w = wl.CONV_WORKLOADS[name]
    inp, y, a = _half_full_reference(name)
    chosen = {}
    for cfg in legal_configs(w, epilogue=ct.CT_EPI_NONE):
        v = cfg.variant
        if v not in chosen or (cfg.split_k, cfg.stages) < (chosen[v].split_k, chosen[v].stages):
            chosen[v] = cfg
    say(f"[conv-f16-variants] {name}: {len(chosen)} variants")
    assert chosen
    for cfg in chosen.values():
        got = run(w, inp, config=cfg, epilogue=ct.CT_EPI_NONE)
        assert_conv_close(got, y, a, w.dtype,
                          f"{ct.variants()[cfg.variant]['name']} S={cfg.split_k} stages={cfg.stages}")


@pytest.mark.parametrize("name", HALF_FULL)
def test_half_precision_full_size_staging_waves_split(name):
    """Full-size half-precision workloads through every variant with
    window-staging waves at a two-way split (the last arriving workgroup of
    a tile sums both partials), every output against the oracle."""
    w = wl.CONV_WORKLOADS[name]
    inp, y, a = _half_full_reference(name)
    cfgs = [cfg for cfg in legal_configs(w, epilogue=ct.CT_EPI_NONE)
            if cfg.split_k == 2 and ct.variants()[cfg.variant]["name"].rsplit("_", 1)[-1] in ("x1", "x2")]
    say(f"[conv-f16-staging-split] {name}: {len(cfgs)} configs")
    assert cfgs
    for cfg in cfgs:
        got = run(w, inp, config=cfg, epilogue=ct.CT_EPI_NONE)
        assert_conv_close(got, y, a, w.dtype, f"{ct.variants()[cfg.variant]['name']} S=2 stages={cfg.stages}")


def test_bf16_full_size_staging_waves():
    """The 64x256x14x14 layer in bf16 (inputs rounded to bf16, the same
    seeded draw) through every bf16 variant with window-staging waves, at
    one and two splits, every output against the oracle."""
    w = wl.ConvWorkload("bf16_n64_c256_14x14_k3", 4, 64, 256, 14, 14, 256, 3, 3, 1, 1, wl.BF16)
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    cfgs = [cfg for cfg in legal_configs(w, epilogue=ct.CT_EPI_NONE)
            if cfg.split_k <= 2 and ct.variants()[cfg.variant]["name"].rsplit("_", 1)[-1] in ("x1", "x2")]
    say(f"[conv-bf16-staging] {len(cfgs)} configs")
    assert cfgs
    for cfg in cfgs:
        got = run(w, inp, config=cfg, epilogue=ct.CT_EPI_NONE)
        assert_conv_close(got, y, a, w.dtype, f"{ct.variants()[cfg.variant]['name']} S={cfg.split_k}")


@pytest.mark.parametrize("name", HALF_FULL)
def test_half_precision_full_size_integers_bit_exact(name):
    """Full-size half-precision workloads on integer inputs in [-2, 2] (exact
    in fp16): every partial sum is an integer of at most 4*CI*KH*KW (9,216 for
    64x256x14x14, 4,608 for 128x128x32x32), exact in fp32 in any order, so
    the default config must reproduce the oracle bit for bit."""
    w = wl.CONV_WORKLOADS[name]
    ints = wl.small_int_inputs(w)
    say(f"[conv-f16-int-full] {name}")
    yi, _ = oracle_full(w, ints)
    assert np.abs(yi).max() <= 4 * w.CI * w.KH * w.KW < 2 ** 24
    assert np.array_equal(run(w, ints, epilogue=ct.CT_EPI_NONE), yi)


HALF_EPI = [
    # 3x3 layers of the stage-major half-precision kernel, with partial
    # channel stages and output-channel tiles, under both epilogues
    ("half_epi_w16", 134, 2, 32, 16, 16, 48, 3, 3, 1, 1),
    ("half_epi_w14", 135, 3, 40, 10, 14, 70, 3, 3, 1, 1),
]


@pytest.mark.parametrize("epi", [ct.CT_EPI_BIAS, ct.CT_EPI_EXP_BIAS_RSQRT])
@pytest.mark.parametrize("shape", HALF_EPI, ids=lambda t: t[0])
@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_half_precision_epilogue_every_config(dtype, shape, epi):
    """The fused epilogue of every legal half-precision config, every output
    against the oracle's epilogue (relative gate for exp, conv gate for the
    bias)."""
    w = wl.ConvWorkload(*shape, dtype, epi)
    inp = wl.conv_inputs(w)
    y, a = oracle_full(w, inp)
    S = float(a.max())
    ref = O.channel_epilogue(y, epi, inp["bias"].astype(np.float64), inp["var"].astype(np.float64),
                             1e-5)
    cfgs = legal_configs(w)
    say(f"[conv-f16-epi] {w.name} {dtype} epi={epi}: {len(cfgs)} configs")
    assert cfgs
    for cfg in [None] + cfgs:
        got = run(w, inp, config=cfg)
        what = "default" if cfg is None else (ct.variants()[cfg.variant]["name"], cfg.split_k, cfg.stages,
                                              cfg.kc)
        assert np.all(np.isfinite(got)), what
        if epi == ct.CT_EPI_EXP_BIAS_RSQRT:
            rel = float((np.abs(got - ref) / np.abs(ref)).max())
            assert rel <= TOL[dtype] * S + 1e-5, (what, rel)
        else:
            assert float(np.abs(got - ref).max()) <= TOL[dtype] * S, what


def _regroup(w: np.ndarray) -> np.ndarray:
    """The documented prepared layout: wp[co][g][t][j] = w[co][8g+j][t],
    zeros past CI (t = ky*KW + kx), rows of CI rounded up to 64 channels."""
    CO, CI, KH, KW = w.shape
    G = (CI + 63) // 64 * 8
    wpad = np.zeros((CO, 8 * G, KH * KW), w.dtype)
    wpad[:, :CI] = w.reshape(CO, CI, KH * KW)
    return wpad.reshape(CO, G, 8, KH * KW).transpose(0, 1, 3, 2).copy()


def _bits16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("misaligned", [False, True], ids=["aligned", "w_offset_2B"])
@pytest.mark.parametrize("shape", HALF_SMALL, ids=lambda t: t[0])
@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_prepared_filter(dtype, shape, misaligned):
    """ct_conv2d_prepare_filter writes exactly the documented layout, and the
    prepared entry point gives the bits of ct_conv2d_nchw_fwd (same kernel and
    config), within the oracle's gate -- or, for a shape where no tile config
    reads a prepared filter (a channel count with no 16- or 32-channel
    stage), refuses it."""
    w = wl.ConvWorkload(*shape, dtype)
    inp = wl.conv_inputs(w)
    x = to_dev(inp["x"], dtype)
    k = to_dev(inp["w"], dtype)
    if misaligned:
        buf = torch.empty(k.numel() + 1, dtype=k.dtype, device=DEV)
        buf[1:].copy_(k.reshape(-1))
        k = buf[1:].view(k.shape)
        assert k.data_ptr() % 16 != 0
    wp = ct.prepare_filter(k)
    torch.cuda.synchronize()
    want = _regroup(_bits16(k.contiguous()).reshape(k.shape))
    assert np.array_equal(_bits16(wp).reshape(want.shape), want)
    y_fwd = ct.conv2d(x, k, w.stride, w.pad)
    if not any(ct.variants()[c.variant]["name"].startswith("h2") for c in legal_configs(w)):
        y_pre = torch.empty_like(y_fwd)
        st = ct.ct_conv2d_nchw_fwd_prepared(x, wp, y_pre, *w.shape_args(), CT_DT[dtype], w.epilogue)
        assert st == ct.CT_ERR_UNSUPPORTED
        return
    y_pre = ct.conv2d_prepared(x, wp, tuple(k.shape), w.stride, w.pad)
    torch.cuda.synchronize()
    _, cfg, _ = ct.ct_conv2d_query(*w.shape_args(), CT_DT[dtype], w.epilogue)
    if ct.variants()[cfg.variant]["name"].startswith("h2"):
        assert torch.equal(y_fwd.view(torch.int32), y_pre.view(torch.int32))
    y, a = oracle_full(w, inp)
    assert_conv_close(y_pre.cpu().numpy().astype(np.float64), y, a, dtype, f"{w.name} prepared")


@pytest.mark.parametrize("name", HALF_FULL)
def test_prepared_filter_full_size(name):
    """Both full-size half-precision workloads: the prepared entry point gives
    the bits of ct_conv2d_nchw_fwd, the fused epilogue included."""
    w = wl.CONV_WORKLOADS[name]
    inp, y, a = _half_full_reference(name)
    x = to_dev(inp["x"], w.dtype)
    k = to_dev(inp["w"], w.dtype)
    b = torch.from_numpy(inp["bias"]).to(DEV)
    v = torch.from_numpy(inp["var"]).to(DEV)
    wp = ct.prepare_filter(k)
    y_fwd = ct.conv2d(x, k, w.stride, w.pad, w.epilogue, b, v)
    y_pre = ct.conv2d_prepared(x, wp, tuple(k.shape), w.stride, w.pad, w.epilogue, b, v)
    torch.cuda.synchronize()
    assert torch.equal(y_fwd.view(torch.int32), y_pre.view(torch.int32))
    say(f"[conv-f16-prepared] {name}: bit-identical to the raw-filter entry point")


def test_prepared_filter_rejects_fp32():
    k = torch.zeros((8, 8, 3, 3), device=DEV)
    wp = torch.zeros(8 * 8 * 9, device=DEV)
    assert ct.ct_conv2d_prepare_filter(k, wp, 8, 8, 3, 3, ct.CT_F32) == ct.CT_ERR_INVALID_ARG
