"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes part of the oracle with something independent of it: values
hand-computed from the definition, values printed on the pages (the gist's run
output of the TVM tutorial), closed forms, invariants, and independent library
routines (numpy matmul, torch CPU conv2d in fp64).  A dropped term, a wrong
sign or index, a flipped kernel or a transposed operand in the oracle fails at
least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, lo=-1.0, hi=1.0):
    return np.random.default_rng(seed).uniform(lo, hi, size=shape)


# --------------------------------------------------------------------------
# convolution
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_hand_cases(case):
    x = np.array(case["x"], np.float64)[None, None]
    w = np.array(case["w"], np.float64)[None, None]
    y, a = O.conv2d_nchw(x, w, case["stride"], case["pad"])
    assert y.shape[2:] == np.array(case["y"]).shape
    assert np.array_equal(y[0, 0], np.array(case["y"], np.float64))


def test_against_torch_fp64_conv():
    # independent library routine (ATen CPU conv2d in fp64), several shapes
    shapes = [(1, 3, 9, 11, 4, 3, 3, 1, 1), (2, 5, 8, 8, 3, 3, 3, 2, 1),
              (1, 4, 10, 7, 6, 5, 3, 2, 2), (3, 2, 6, 6, 5, 1, 1, 1, 0),
              (1, 3, 13, 13, 2, 7, 7, 2, 3), (2, 6, 5, 9, 7, 2, 4, 3, 0)]
    for i, (N, CI, H, W, CO, KH, KW, s, p) in enumerate(shapes):
        x = _rand((N, CI, H, W), 10 + i)
        w = _rand((CO, CI, KH, KW), 50 + i)
        y, _ = O.conv2d_nchw(x, w, s, p)
        ref = torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(w),
                                         stride=s, padding=p).numpy()
        assert y.shape == ref.shape
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_im2col_matmul_brute_force():
    # explicit padded copy + window gather + numpy matmul (a different route)
    rng = np.random.default_rng(7)
    for trial in range(6):
        N, CI, CO = rng.integers(1, 3), rng.integers(1, 5), rng.integers(1, 5)
        KH, KW = rng.integers(1, 4), rng.integers(1, 4)
        s, p = rng.integers(1, 3), rng.integers(0, 3)
        H, W = rng.integers(KH, 9), rng.integers(KW, 9)
        x = rng.uniform(-1, 1, (N, CI, H, W))
        w = rng.uniform(-1, 1, (CO, CI, KH, KW))
        xp = np.zeros((N, CI, H + 2 * p, W + 2 * p))
        xp[:, :, p:p + H, p:p + W] = x
        OH = (H + 2 * p - KH) // s + 1
        OW = (W + 2 * p - KW) // s + 1
        cols = np.empty((N, CI * KH * KW, OH * OW))
        for oy in range(OH):
            for ox in range(OW):
                win = xp[:, :, oy * s:oy * s + KH, ox * s:ox * s + KW]
                cols[:, :, oy * OW + ox] = win.reshape(N, -1)
        ref = np.stack([w.reshape(CO, -1) @ cols[n] for n in range(N)]).reshape(N, CO, OH, OW)
        y, _ = O.conv2d_nchw(x, w, int(s), int(p))
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_one_by_one_kernel_is_matmul():
    x = _rand((2, 7, 5, 6), 1)
    w = _rand((9, 7, 1, 1), 2)
    y, _ = O.conv2d_nchw(x, w, 1, 0)
    for n in range(2):
        ref = w[:, :, 0, 0] @ x[n].reshape(7, -1)
        np.testing.assert_allclose(y[n].reshape(9, -1), ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("K", [1, 3, 5, 7])
def test_centred_delta_is_identity(K):
    C = 3
    x = _rand((2, C, 8, 9), 3)
    w = np.zeros((C, C, K, K))
    for c in range(C):
        w[c, c, K // 2, K // 2] = 1.0
    y, _ = O.conv2d_nchw(x, w, 1, (K - 1) // 2)
    assert np.array_equal(y, x)


def test_linearity():
    x1, x2 = _rand((1, 4, 6, 6), 4), _rand((1, 4, 6, 6), 5)
    w1, w2 = _rand((3, 4, 3, 3), 6), _rand((3, 4, 3, 3), 7)
    a, b = 0.75, -1.5
    ya, _ = O.conv2d_nchw(a * x1 + b * x2, w1, 1, 1)
    y1, _ = O.conv2d_nchw(x1, w1, 1, 1)
    y2, _ = O.conv2d_nchw(x2, w1, 1, 1)
    np.testing.assert_allclose(ya, a * y1 + b * y2, rtol=1e-12, atol=1e-12)
    yb, _ = O.conv2d_nchw(x1, a * w1 + b * w2, 1, 1)
    y3, _ = O.conv2d_nchw(x1, w2, 1, 1)
    np.testing.assert_allclose(yb, a * y1 + b * y3, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s", [2, 3])
def test_stride_is_subsampled_stride_one(s):
    x = _rand((1, 3, 11, 10), 8)
    w = _rand((2, 3, 3, 3), 9)
    y1, _ = O.conv2d_nchw(x, w, 1, 1)
    ys, _ = O.conv2d_nchw(x, w, s, 1)
    assert np.array_equal(ys, y1[:, :, ::s, ::s])


def test_all_ones_counts_valid_taps_final_resnet_layer():
    # x = w = 1 on the 1x512x7x7 -> 512, 3x3, s1 p1 layer: y = CI * (#taps inside)
    x = np.ones((1, 512, 7, 7))
    w = np.ones((4, 512, 3, 3))          # 4 output channels are enough
    y, a = O.conv2d_nchw(x, w, 1, 1)
    assert y[0, 0, 0, 0] == 512 * 4 and y[0, 0, 0, 3] == 512 * 6 and y[0, 0, 3, 3] == 512 * 9
    assert y[0, 3, 6, 6] == 2048 and y[0, 1, 6, 2] == 3072
    assert np.array_equal(a, y)


def test_absacc_scale():
    x = _rand((1, 3, 7, 7), 11)
    w = _rand((4, 3, 3, 3), 12)
    y, a = O.conv2d_nchw(x, w, 1, 1)
    assert np.all(a >= np.abs(y) - 1e-15)
    ya, _ = O.conv2d_nchw(np.abs(x), np.abs(w), 1, 1)   # sum |x w| = conv(|x|, |w|)
    np.testing.assert_allclose(a, ya, rtol=1e-13)
    _, a2 = O.conv2d_nchw(-x, w, 1, 1)
    assert np.array_equal(a, a2)


def test_points_match_full():
    x = _rand((2, 5, 9, 8), 13)
    w = _rand((6, 5, 3, 3), 14)
    y, a = O.conv2d_nchw(x, w, 2, 1)
    rng = np.random.default_rng(15)
    idx = np.stack([rng.integers(0, d, 40) for d in y.shape], axis=1)
    yp, ap = O.conv2d_points(x, w, 2, 1, idx)
    for t, (n, f, oy, ox) in enumerate(idx):
        assert yp[t] == y[n, f, oy, ox] and ap[t] == a[n, f, oy, ox]


def test_output_extents_of_the_workloads():
    cases = [((14, 3, 1, 1), 14), ((7, 3, 1, 1), 7), ((224, 7, 2, 3), 112), ((56, 3, 1, 1), 56),
             ((56, 3, 2, 1), 28), ((28, 3, 2, 1), 14), ((14, 3, 2, 1), 7), ((14, 1, 1, 0), 14),
             ((32, 3, 1, 1), 32), ((5, 7, 1, 0), 0)]
    for args, want in cases:
        assert O.out_extent(*args) == want


def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.conv2d_nchw(np.ones((1, 1, 2, 2)), np.ones((1, 1, 3, 3)), 1, 0)
    with pytest.raises(ValueError):
        O.conv2d_nchw(np.ones((1, 1, 4, 4)), np.ones((1, 1, 3, 3)), 0, 0)


# --------------------------------------------------------------------------
# epilogue and broadcast
# --------------------------------------------------------------------------

def test_epilogue_closed_forms():
    rng = np.random.default_rng(16)
    C = 5
    b = rng.normal(0, 0.1, C)
    v = rng.uniform(0.5, 2.0, C)
    eps = 1e-5
    # w = 0  =>  conv = 0  =>  out = exp(b[c]) / sqrt(v[c] + eps)
    y, _ = O.conv2d_nchw(_rand((2, 3, 4, 4), 17), np.zeros((C, 3, 3, 3)), 1, 1)
    out = O.channel_epilogue(y, O.EPI_EXP_BIAS_RSQRT, b, v, eps)
    for c in range(C):
        want = math.exp(b[c]) / math.sqrt(v[c] + eps)
        assert np.all(np.abs(out[:, c] - want) <= 1e-15 * want)
    # b = 0, v = 1 - eps  =>  out = exp(y)
    y2 = rng.normal(0, 1, (2, C, 3, 3))
    out2 = O.channel_epilogue(y2, O.EPI_EXP_BIAS_RSQRT, np.zeros(C), np.full(C, 1 - eps), eps)
    np.testing.assert_allclose(out2, np.exp(y2), rtol=1e-15)
    # bias only, and none
    out3 = O.channel_epilogue(y2, O.EPI_BIAS, b)
    np.testing.assert_array_equal(out3, y2 + b[None, :, None, None])
    np.testing.assert_array_equal(O.channel_epilogue(y2, O.EPI_NONE), y2)


def test_broadcast_exp():
    var = np.random.default_rng(18).uniform(0.5, 2.0, 6)
    out = O.broadcast_exp(var, 3, 4, 5)
    assert out.shape == (3, 6, 4, 5)
    for c in range(6):
        assert np.all(out[:, c] == math.exp(var[c]))


# --------------------------------------------------------------------------
# search space of the tutorial's template, against the gist's printed output
# --------------------------------------------------------------------------

def _count_closed_form(n, k):
    # number of ordered k-factorizations: prod over prime powers p^e || n of C(e+k-1, k-1)
    total, m, p = 1, n, 2
    while p * p <= m:
        e = 0
        while m % p == 0:
            m //= p
            e += 1
        total *= math.comb(e + k - 1, k - 1)
        p += 1
    if m > 1:
        total *= k
    return total


@pytest.mark.parametrize("n", [1, 3, 7, 12, 36, 49, 64, 96, 360, 512])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_factorization_count_closed_form(n, k):
    fs = O.ordered_factorizations(n, k)
    assert len(fs) == _count_closed_form(n, k)
    assert len({tuple(f) for f in fs}) == len(fs)
    assert all(math.prod(f) == n and len(f) == k for f in fs)


def test_space_dump_matches_gist():
    g = _load("tvm_tuning_log.json")
    wl = g["workload"]
    sp = O.tvm_tutorial_space(wl["N"], wl["H"], wl["W"], wl["CO"], wl["CI"], wl["KH"], wl["KW"],
                              wl["stride"], wl["pad"])
    assert sp.lens == [k["len"] for k in g["space"]["knobs"]]
    assert len(sp) == g["space"]["total"] == 10454400


def test_flat_indices_match_gist():
    g = _load("tvm_tuning_log.json")
    sp = O.tvm_tutorial_space(1, 7, 7, 512, 512, 3, 3, 1, 1)
    pairs = [(t["config"], t["index"]) for t in g["trials"]] + [(g["best"]["config"], g["best"]["index"])]
    assert len(pairs) == 21
    for cfg, idx in pairs:
        assert sp.index_of(cfg) == idx
        assert sp.entity_at(idx) == cfg


def test_shared_memory_rule_reproduces_gist_outcomes():
    # Reading: the template's verify pass rejects a kernel whose shared stages
    # exceed 48 KiB (error_no 1); every other trial was built and launched.
    g = _load("tvm_tuning_log.json")
    limit = 48 * 1024
    for t in g["trials"]:
        rejected = O.tvm_template_shared_bytes(t["config"], 1) > limit
        assert rejected == (t["error_no"] == 1), t["no"]
        assert O.tvm_template_threads(t["config"]) <= 1024
    best = O.tvm_template_shared_bytes(g["best"]["config"], 1)
    assert best == 4 * (8 * 9 * 9 + 64 * 8 * 3 * 3)


def test_flop_count_reproduces_gist_gflops():
    g = _load("tvm_tuning_log.json")
    flops = O.conv_flops(1, 512, 7, 7, 512, 3, 3, 1, 1)
    assert flops == 231211008
    ok = [t for t in g["trials"] if t["error_no"] == 0]
    assert len(ok) == 5
    for t in ok:
        gf = flops / t["cost"] / 1e9
        # printed to 2 decimals; the tool's own count sits ~0.12% above 2*MAC
        assert abs(gf - t["gflops"]) <= 0.005 + 1.5e-3 * t["gflops"], (t["no"], gf)


# ---- matrix product ---------------------------------------------------------
def test_gemm_textbook_case():
    """[[1,2,3],[4,5,6]] x [[7,8],[9,10],[11,12]] = [[58,64],[139,154]] (worked by
    hand: 1*7+2*9+3*11 = 58, 1*8+2*10+3*12 = 64, 4*7+5*9+6*11 = 139,
    4*8+5*10+6*12 = 154).  A transposed operand or swapped product fails it."""
    A = np.array([[1, 2, 3], [4, 5, 6]], dtype=np.float64)
    B = np.array([[7, 8], [9, 10], [11, 12]], dtype=np.float64)
    C, absacc = O.gemm(A, B)
    assert C.tolist() == [[58, 64], [139, 154]]
    assert absacc.tolist() == [[58, 64], [139, 154]]
    C, absacc = O.gemm(-A, B)
    assert C.tolist() == [[-58, -64], [-139, -154]] and absacc.tolist() == [[58, 64], [139, 154]]


def test_gemm_brute_force_loops():
    r = np.random.default_rng(11)
    for M, N, K in [(1, 1, 1), (3, 5, 4), (7, 2, 9)]:
        A, B = r.normal(size=(M, K)), r.normal(size=(K, N))
        C, _ = O.gemm(A, B)
        for m in range(M):
            for n in range(N):
                s = 0.0
                for k in range(K):
                    s += A[m, k] * B[k, n]
                assert abs(C[m, n] - s) <= 1e-12 * (1 + abs(s))


def test_gemm_identity():
    A = np.random.default_rng(12).normal(size=(6, 6))
    assert np.array_equal(O.gemm(A, np.eye(6))[0], A)
    assert np.array_equal(O.gemm(np.eye(6), A)[0], A)


@pytest.mark.parametrize("fold", [(1, 20), (4, 5), (20, 1)])
def test_gemm_is_the_seven_loop_1x1_convolution(fold):
    """The library's view of a matrix product: w = A as [M][K][1][1], x = B as
    [1][K][H][W] with H*W = N, y = C.  The seven-loop convolution (independent
    C code) gives the same numbers for every split of N; integer inputs make
    both sums exact."""
    r = np.random.default_rng(13)
    M, K, N = 6, 7, 20
    A = r.integers(-3, 4, (M, K)).astype(np.float64)
    B = r.integers(-3, 4, (K, N)).astype(np.float64)
    H, W = fold
    y, _ = O.conv2d_nchw(B.reshape(1, K, H, W), A.reshape(M, K, 1, 1), 1, 0)
    assert np.array_equal(y.reshape(M, N), O.gemm(A, B)[0])


# ---- depthwise convolution --------------------------------------------------
def test_depthwise_hand_case():
    """Two channels worked by hand.  Channel 0: filter [[1, 0], [0, -1]], so
    y = x[oy][ox] - x[oy+1][ox+1] (-4 everywhere on 1..9); with pad 1 and
    stride 2 the taps fall on xp[2oy][2ox] - xp[2oy+1][2ox+1] = (0 - 1, 0 - 3,
    0 - 7, 5 - 9).  Channel 1: filter [[2, 1], [0, 1]] on [[1, 0, -1],
    [2, 0, -2], [0, 1, 0]] gives [[2, -3], [5, -2]] (e.g. top right:
    2*0 + 1*(-1) + 0*0 + 1*(-2) = -3).  A flipped filter, a channel mix-up or
    a wrong padding offset fails it."""
    x = np.array([[[[1, 2, 3], [4, 5, 6], [7, 8, 9]],
                   [[1, 0, -1], [2, 0, -2], [0, 1, 0]]]], np.float64)
    w = np.array([[[[1, 0], [0, -1]]], [[[2, 1], [0, 1]]]], np.float64)
    y, a = O.conv2d_depthwise(x, w, 1, 0)
    assert y.tolist() == [[[[-4, -4], [-4, -4]], [[2, -3], [5, -2]]]]
    assert a[0, 0].tolist() == [[6, 8], [12, 14]]
    y, _ = O.conv2d_depthwise(x[:, :1], w[:1], 2, 1)
    assert y.tolist() == [[[[-1, -3], [-7, -4]]]]


def test_depthwise_against_torch_grouped_conv():
    """ATen's CPU conv2d with groups = C (fp64) is an independent routine."""
    shapes = [(1, 3, 9, 11, 3, 3, 1, 1), (2, 5, 8, 8, 3, 3, 2, 1), (1, 4, 10, 7, 5, 3, 2, 2),
              (3, 2, 6, 6, 1, 1, 1, 0), (1, 3, 13, 13, 7, 7, 2, 3), (2, 6, 5, 9, 2, 4, 3, 0)]
    for i, (N, C, H, W, KH, KW, s, p) in enumerate(shapes):
        x = _rand((N, C, H, W), 400 + i)
        w = _rand((C, 1, KH, KW), 450 + i)
        y, _ = O.conv2d_depthwise(x, w, s, p)
        ref = torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(w), stride=s,
                                         padding=p, groups=C).numpy()
        assert y.shape == ref.shape
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("ints", [True, False])
def test_depthwise_is_block_diagonal_seven_loop_convolution(ints):
    """The seven-loop convolution (independent C code) with the filter
    w_full[c][c'] = w[c] if c == c' else 0 gives the depthwise result: exactly
    for integer inputs, to rounding for random ones."""
    r = np.random.default_rng(460)
    N, C, H, W, KH, KW, s, p = 2, 5, 11, 9, 3, 3, 2, 1
    if ints:
        x = r.integers(-3, 4, (N, C, H, W)).astype(np.float64)
        w = r.integers(-3, 4, (C, 1, KH, KW)).astype(np.float64)
    else:
        x, w = r.normal(size=(N, C, H, W)), r.normal(size=(C, 1, KH, KW))
    wf = np.zeros((C, C, KH, KW))
    for c in range(C):
        wf[c, c] = w[c, 0]
    y, a = O.conv2d_depthwise(x, w, s, p)
    yf, af = O.conv2d_nchw(x, wf, s, p)
    if ints:
        assert np.array_equal(y, yf) and np.array_equal(a, af)
    else:
        np.testing.assert_allclose(y, yf, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(a, af, rtol=1e-13, atol=1e-13)


def test_depthwise_closed_forms():
    r = np.random.default_rng(470)
    x = r.normal(size=(2, 4, 7, 6))
    # a 1x1 filter scales each channel
    w1 = r.normal(size=(4, 1, 1, 1))
    assert np.array_equal(O.conv2d_depthwise(x, w1, 1, 0)[0], x * w1[:, 0, 0, 0][None, :, None, None])
    # a delta filter at (1, 2) of a 3x4 filter with pad 1 reads xp[oy + 1][ox + 2]
    wd = np.zeros((4, 1, 3, 4))
    wd[:, 0, 1, 2] = 1.0
    y, _ = O.conv2d_depthwise(x, wd, 1, 1)
    xp = np.pad(x, ((0, 0), (0, 0), (1, 1), (1, 1)))
    assert np.array_equal(y, xp[:, :, 1:1 + y.shape[2], 2:2 + y.shape[3]])
    # stride s samples the stride-1 output at multiples of s
    w = r.normal(size=(4, 1, 3, 3))
    y1, _ = O.conv2d_depthwise(x, w, 1, 1)
    for s in (2, 3):
        ys, _ = O.conv2d_depthwise(x, w, s, 1)
        assert np.array_equal(ys, y1[:, :, ::s, ::s][:, :, :ys.shape[2], :ys.shape[3]])
    # all ones: every output counts the taps that land inside the image
    y, a = O.conv2d_depthwise(np.ones((1, 1, 4, 4)), np.ones((1, 1, 3, 3)), 1, 1)
    assert y[0, 0].tolist() == [[4, 6, 6, 4], [6, 9, 9, 6], [6, 9, 9, 6], [4, 6, 6, 4]]
    assert np.array_equal(a, y)


def test_depthwise_channels_are_independent():
    r = np.random.default_rng(480)
    x = r.normal(size=(2, 5, 8, 8))
    w = r.normal(size=(5, 1, 3, 3))
    y0, _ = O.conv2d_depthwise(x, w, 1, 1)
    x2 = x.copy()
    x2[:, 3] += 1.0
    y2, _ = O.conv2d_depthwise(x2, w, 1, 1)
    changed = np.any(y0 != y2, axis=(0, 2, 3))
    assert changed.tolist() == [False, False, False, True, False]


def test_depthwise_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.conv2d_depthwise(np.ones((1, 2, 4, 4)), np.ones((3, 1, 3, 3)), 1, 0)
    with pytest.raises(ValueError):
        O.conv2d_depthwise(np.ones((1, 2, 4, 4)), np.ones((2, 2, 3, 3)), 1, 0)
    with pytest.raises(ValueError):
        O.conv2d_depthwise(np.ones((1, 2, 2, 2)), np.ones((2, 1, 3, 3)), 1, 0)


# ---- general per-channel broadcast ------------------------------------------
def test_chain_hand_case_batchnorm_form():
    """c0 = rsqrt(a0 + 1) with a0 = [3, 8]: [1/2, 1/3]; v = (x - a1) * c0 *
    a2 + a3 with x = 5, a1 = [1, 2], a2 = [3, 6], a3 = [-1, 0]:
    (5-1)/2*3 - 1 = 5 and (5-2)/3*6 + 0 = 6, worked by hand."""
    chains = ([("set", "a0"), ("add", 1.0), ("rsqrt",)], [],
              [("set", "x"), ("sub", "a1"), ("mul", "c0"), ("mul", "a2"), ("add", "a3")])
    arrays = [np.array([3.0, 8.0]), np.array([1.0, 2.0]), np.array([3.0, 6.0]), np.array([-1.0, 0.0])]
    x = np.full((2, 2, 3), 5.0)
    out = O.broadcast_chain(chains, 2, 2, 3, arrays, x)
    np.testing.assert_allclose(out[:, 0], 5.0, rtol=1e-15)
    np.testing.assert_allclose(out[:, 1], 6.0, rtol=1e-15)
    # with no v chain the output is c0
    c0 = O.broadcast_chain((chains[0], [], []), 1, 2, 1, arrays)
    np.testing.assert_allclose(c0.reshape(-1), [0.5, 1.0 / 3.0], rtol=1e-15)


def test_chain_exp_matches_the_c_broadcast():
    """[1,C,1,1] => [N,C,H,W] of exp(var[c]) is the chain set(a0), exp with
    outer = N, inner = H*W; the C oracle's broadcast is separate code."""
    var = np.random.default_rng(490).uniform(0.5, 2.0, 6)
    out = O.broadcast_chain(([("set", "a0"), ("exp",)], [], []), 3, 6, 20, [var])
    ref = O.broadcast_exp(var, 3, 4, 5).reshape(3, 6, 20)
    np.testing.assert_allclose(out, ref, rtol=1e-15)


def test_chain_step_orientation_and_identities():
    one = lambda steps: float(O.broadcast_chain((steps, [], []), 1, 1, 1)[0, 0, 0])
    assert one([("set", 3.0), ("rsub", 10.0)]) == 7.0      # 10 - 3
    assert one([("set", 3.0), ("rdiv", 12.0)]) == 4.0      # 12 / 3
    assert one([("set", 3.0), ("sub", 10.0)]) == -7.0
    assert one([("set", 12.0), ("div", 3.0)]) == 4.0
    assert one([("set", 4.0), ("sqrt",)]) == 2.0
    assert one([("set", 4.0), ("rsqrt",)]) == 0.5
    assert one([("exp",)]) == 1.0                           # a chain starts from 0
    assert one([("add", 2.0), ("mul", 3.0)]) == 6.0
    assert one([]) == 0.0


def test_chain_layout_brute_force():
    """out[o][p][i] = a0[p] * 10 + x[o][p][i] over explicit loops: a wrong
    axis order or a transposed broadcast fails it."""
    outer, P, inner = 3, 4, 5
    a0 = np.arange(P, dtype=np.float64) + 1.0
    x = np.random.default_rng(491).normal(size=(outer, P, inner))
    out = O.broadcast_chain(([("set", "a0"), ("mul", 10.0)], [], [("set", "x"), ("add", "c0")]),
                            outer, P, inner, [a0], x)
    for o in range(outer):
        for p in range(P):
            for i in range(inner):
                assert out[o, p, i] == x[o, p, i] + a0[p] * 10.0
    # without x the value depends on p only
    out = O.broadcast_chain(([("set", "a0"), ("exp",)], [], []), outer, P, inner, [a0])
    for p in range(P):
        assert np.all(out[:, p, :] == out[0, p, 0])
    assert len(set(out[0, :, 0].tolist())) == P


def test_chain_identity_and_c1():
    x = np.random.default_rng(492).normal(size=(2, 3, 4))
    assert np.array_equal(O.broadcast_chain(([], [], [("set", "x")]), 2, 3, 4, x=x), x)
    # c1 reads c0: c1 = c0 * 2, v = x * c1
    a0 = np.array([1.0, 2.0, 3.0])
    out = O.broadcast_chain(([("set", "a0")], [("set", "c0"), ("mul", 2.0)], [("set", "x"), ("mul", "c1")]),
                            2, 3, 4, [a0], x)
    assert np.array_equal(out, x * (a0 * 2.0)[None, :, None])


# ---- the guided search's cost model -----------------------------------------
def test_ridge_recovers_an_exact_linear_model():
    """y = X w exactly and lam = 0: the fit returns w (a closed form)."""
    r = np.random.default_rng(500)
    X = np.column_stack([np.ones(30), r.normal(size=(30, 4))])
    w = np.array([0.5, -1.0, 2.0, 0.25, 3.0])
    np.testing.assert_allclose(O.ridge_fit(X, X @ w, 0.0), w, rtol=1e-10, atol=1e-12)


def test_ridge_hand_case_and_shrinkage():
    """One feature x = (1, 2), y = (2, 4): w = sum(xy) / (sum(x^2) + lam) =
    10 / (5 + lam), worked by hand; a huge lam shrinks w to 0."""
    X = np.array([[1.0], [2.0]])
    y = np.array([2.0, 4.0])
    assert abs(O.ridge_fit(X, y, 0.0)[0] - 2.0) < 1e-15
    assert abs(O.ridge_fit(X, y, 5.0)[0] - 1.0) < 1e-15
    assert abs(O.ridge_fit(X, y, 1e12)[0]) < 1e-10
