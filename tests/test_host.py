"""Host-side checks that need no GPU: the C-ABI library loads and exports what
include/convtile.h declares, argument checking, the tile-config space (against
the oracle's plain enumerator and the gist's printed space), the legality
check, the default config, and the JSON-lines cache."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from oracle import oracle as O
from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(ct.LIB_PATH):
        from tensor_compiler_tiling_amd import build
        build.build()


def _declared():
    src = open(os.path.join(ROOT, "include", "convtile.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ct_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ct.library()
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(ct.exported_names()) == names
    assert "gfx950" in ct.ct_version()


def test_status_strings():
    assert ct.ct_status_string(0) == "ok"
    assert ct.ct_status_string(ct.CT_ERR_INVALID_ARG) == "invalid argument"


# ------------------------------------------------------------ argument checks
BAD_SHAPES = [
    dict(N=0), dict(CI=0), dict(H=-1), dict(CO=0), dict(KH=0), dict(stride=0), dict(pad=-1),
    dict(H=2, W=2, KH=5, KW=5, pad=0), dict(dtype=7), dict(epilogue=9),
]


@pytest.mark.parametrize("bad", BAD_SHAPES)
def test_invalid_shapes_rejected_before_any_hip_call(bad):
    a = dict(N=1, CI=4, H=8, W=8, CO=4, KH=3, KW=3, stride=1, pad=1, dtype=0, epilogue=0)
    a.update(bad)
    args = [a[k] for k in ("N", "CI", "H", "W", "CO", "KH", "KW", "stride", "pad", "dtype",
                           "epilogue")]
    # fake non-null pointers: the call must fail on the shape before touching them
    st = ct.library().ct_conv2d_nchw_fwd(16, 16, 16, *args, 16, 16, 1e-5, None)
    assert st == ct.CT_ERR_INVALID_ARG
    assert ct.ct_last_error()
    assert ct.ct_conv2d_space_size(*args) == ct.CT_ERR_INVALID_ARG


@pytest.mark.parametrize("mnk", [(0, 4, 4), (4, 0, 4), (4, 4, 0), (-1, 4, 4)])
def test_gemm_invalid_sizes_rejected_before_any_hip_call(mnk):
    M, N, K = mnk
    # fake non-null pointers: the call must fail on the sizes before touching them
    st = ct.library().ct_gemm_fwd(16, 16, 16, M, N, K, 0, 0, 16, 16, 1e-5, None)
    assert st == ct.CT_ERR_INVALID_ARG
    assert "M, N and K" in ct.ct_last_error()
    st, _, _ = ct.ct_gemm_query(M, N, K, 0, 0)
    assert st == ct.CT_ERR_INVALID_ARG


def test_gemm_null_and_dtype_errors():
    assert ct.library().ct_gemm_fwd(None, 16, 16, 4, 4, 4, 0, 0, None, None, 1e-5, None) == ct.CT_ERR_INVALID_ARG
    assert ct.library().ct_gemm_fwd(16, 16, 16, 4, 4, 4, 7, 0, None, None, 1e-5, None) == ct.CT_ERR_INVALID_ARG


def test_gemm_query_uses_the_folded_convolution_shape():
    """The matrix product's cached config is the 1x1 convolution's with N split as
    H*W (W the largest divisor of N not above 256)."""
    for M, N, K, dt in [(64, 4096, 128, ct.CT_F16), (37, 53, 29, ct.CT_F32), (8, 1000, 16, ct.CT_BF16)]:
        H, W = wl.gemm_fold(N)
        assert H * W == N and W <= 256
        st, c1, fc1 = ct.ct_gemm_query(M, N, K, dt, 0)
        st2, c2, fc2 = ct.ct_conv2d_query(1, K, H, W, M, 1, 1, 1, 0, dt, 0)
        assert st == 0 and st2 == 0
        assert (c1.variant, c1.split_k, c1.stages, c1.kc) == (c2.variant, c2.split_k, c2.stages, c2.kc)
        assert ct.variants()[c1.variant]["kind"] == 1, "a tiled kernel, not the direct reference"


def test_null_pointers_rejected():
    lib = ct.library()
    shape = (1, 4, 8, 8, 4, 3, 3, 1, 1, 0)
    assert lib.ct_conv2d_nchw_fwd(None, 16, 16, *shape, 0, None, None, 1e-5, None) == -1
    assert lib.ct_conv2d_nchw_fwd(16, 16, None, *shape, 0, None, None, 1e-5, None) == -1
    # the epilogue reads bias / var
    assert lib.ct_conv2d_nchw_fwd(16, 16, 16, *shape, 1, None, None, 1e-5, None) == -1
    assert lib.ct_conv2d_nchw_fwd(16, 16, 16, *shape, 2, 16, None, 1e-5, None) == -1
    assert lib.ct_broadcast_nchw(None, 16, 1, 4, 8, 8, 0, 0, 0, None) == -1
    assert lib.ct_broadcast_nchw(16, 16, 1, 4, 8, 8, 5, 0, 0, None) == -1
    assert lib.ct_broadcast_nchw(16, 16, 1, 4, 8, 8, 0, 3, 0, None) == -1
    assert lib.ct_broadcast_nchw(16, 16, 1, 4, 8, 8, 0, 0, 9, None) == -1


# ------------------------------------------------------------ split enumerator
@pytest.mark.parametrize("n", [1, 2, 3, 7, 12, 49, 64, 96, 128, 256, 360, 512])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_split_enumerator_matches_oracle(n, k):
    want = O.ordered_factorizations(n, k)
    assert ct.ct_split_count(n, k) == len(want)
    for i, f in enumerate(want):
        st, got = ct.ct_split_entity(n, k, i)
        assert st == 0 and got == f


def test_split_counts_of_the_gist_space():
    # ConfigSpace lens printed for the 1x512x7x7 -> 512 3x3 workload
    assert [ct.ct_split_count(512, 4), ct.ct_split_count(7, 4), ct.ct_split_count(512, 3),
            ct.ct_split_count(3, 3)] == [220, 4, 55, 3]
    assert ct.ct_split_count(0, 3) < 0 and ct.ct_split_count(8, 9) < 0


# ------------------------------------------------------------ tile-config space
def _dt(w):
    return {wl.F32: ct.CT_F32, wl.F16: ct.CT_F16, wl.BF16: ct.CT_BF16}[w.dtype]


def _args(w):
    return w.shape_args() + (_dt(w), w.epilogue)


@pytest.mark.parametrize("name", list(wl.CONV_WORKLOADS))
def test_space_is_split_times_variants(name):
    w = wl.CONV_WORKLOADS[name]
    n_var = sum(1 for v in ct.variants() if v["kind"] == 1 and v["dtype"] == _dt(w))
    size = ct.ct_conv2d_space_size(*_args(w))
    assert size == len(O.ordered_factorizations(w.CI, 3)) * n_var
    splits = O.ordered_factorizations(w.CI, 3)
    seen_legal = 0
    for idx in range(size):
        st, cfg, legal = ct.ct_conv2d_space_entity(*_args(w), idx)
        assert st == 0 and cfg.index == idx
        # mixed radix, first knob (tile_ci) least significant
        assert [cfg.split_k, cfg.stages, cfg.kc] == splits[idx % len(splits)]
        seen_legal += legal
    if n_var:
        assert seen_legal > 0, "no legal tile config"
    st, _, _ = ct.ct_conv2d_space_entity(*_args(w), size)
    assert st == ct.CT_ERR_INVALID_ARG


def test_legality_rejects_oversized_stage():
    w = wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"]
    by_name = {v["name"]: v for v in ct.variants()}
    big = by_name["f32_m128n128_w2x2x1_r2x2"]
    size = ct.ct_conv2d_space_size(*_args(w))
    for idx in range(size):
        st, cfg, legal = ct.ct_conv2d_space_entity(*_args(w), idx)
        if cfg.variant == big["id"] and cfg.kc == 64:
            # a 128-row W tile of 64 channels x 9 taps alone is 295 KB
            assert legal == 0
        if legal:
            v = ct.variants()[cfg.variant]
            assert cfg.kc <= v["kc_max"]
            if v["name"].startswith(("f32sk_", "f32sk16_")):
                # the split-K kernels hold a stage's kc * KH * KW k values in lanes
                assert cfg.kc * 9 <= v["kc_max"]


def test_staging_wave_variants_describe_their_workgroup():
    """The fp16 variants with window-staging waves (names ending _x1, _x2)
    report the whole workgroup: the matrix waves' threads plus 64 a staging
    wave; every other tiled variant reports its matrix waves alone."""
    seen = 0
    for v in ct.variants():
        if v["kind"] != 1:
            continue
        matrix = v["waves_m"] * v["waves_n"] * v["waves_k"] * 64
        tail = v["name"].rsplit("_", 1)[-1]
        if v["name"].startswith(("h2f16_", "h2bf16_")) and tail in ("x1", "x2"):
            assert v["threads"] == matrix + 64 * int(tail[1]), v
            seen += 1
        else:
            assert v["threads"] == matrix, v
    assert seen >= 3
    # the shipped tuning log picks one of them for the 64x256x14x14 fp16 layer,
    # and it is legal there
    w = wl.CONV_WORKLOADS["f16_n64_c256_14x14_k3"]
    by_name = {v["name"]: v for v in ct.variants()}
    x2 = by_name["h2f16_m128n128_w2x2_r2x2_kc16_x2"]
    legal = [cfg for i in range(ct.ct_conv2d_space_size(*_args(w)))
             for st, cfg, ok in [ct.ct_conv2d_space_entity(*_args(w), i)] if ok and cfg.variant == x2["id"]]
    assert legal


def test_query_default_without_gpu():
    ct.ct_cache_clear()
    for w in wl.CONV_WORKLOADS.values():
        st, cfg, from_cache = ct.ct_conv2d_query(*_args(w))
        assert st == 0 and from_cache == 0
        info = ct.variants()[cfg.variant]
        assert info["dtype"] == _dt(w)
        if info["kind"] == 1:
            st2, cfg2, legal = ct.ct_conv2d_space_entity(*_args(w), cfg.index)
            assert legal == 1 and cfg2.variant == cfg.variant


# ------------------------------------------------------------ cache file
def test_cache_roundtrip_and_corrupt_lines(tmp_path):
    w = wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"]
    size = ct.ct_conv2d_space_size(*_args(w))
    legal_idx = [i for i in range(size) if ct.ct_conv2d_space_entity(*_args(w), i)[2]]
    st, cfg, _ = ct.ct_conv2d_space_entity(*_args(w), legal_idx[3])
    vname = ct.variants()[cfg.variant]["name"]
    rec = {"key": "x", "N": 1, "CI": 512, "H": 7, "W": 7, "CO": 512, "KH": 3, "KW": 3,
           "stride": 1, "pad": 1, "dtype": 0, "epilogue": 0, "arch": "gfx950", "variant": vname,
           "split_k": cfg.split_k, "stages": cfg.stages, "kc": cfg.kc, "index": 0, "us": 4.25,
           "error_no": 0, "costs_us": [4.2, 4.3, 4.25], "all_cost": 0.5, "timestamp": 1.0}
    p = tmp_path / "cache.jsonl"
    bad_variant = dict(rec, variant="no_such_kernel")
    failed = dict(rec, error_no=4)
    p.write_text("not json\n" + json.dumps(bad_variant) + "\n{\"N\": 1,\n" +
                 json.dumps(failed) + "\n" + json.dumps(rec) + "\n")
    ct.ct_cache_clear()
    assert ct.ct_cache_load(str(p)) == 0
    assert ct.ct_cache_size() == 1
    st, got, from_cache = ct.ct_conv2d_query(*_args(w))
    assert st == 0 and from_cache == 1
    assert (got.variant, got.split_k, got.stages, got.kc) == (cfg.variant, cfg.split_k,
                                                              cfg.stages, cfg.kc)
    assert got.index == legal_idx[3]
    assert abs(got.us - 4.25) < 1e-6
    # save appends; loading the saved file reproduces the same entry
    p2 = tmp_path / "saved.jsonl"
    assert ct.ct_cache_save(str(p2)) == 0
    ct.ct_cache_clear()
    assert ct.ct_cache_size() == 0
    assert ct.ct_cache_load(str(p2)) == 0
    st, got2, fc = ct.ct_conv2d_query(*_args(w))
    assert fc == 1 and got2.index == got.index
    ct.ct_cache_clear()
    assert ct.ct_cache_load(str(tmp_path / "missing.jsonl")) == ct.CT_ERR_IO


def test_workload_shapes():
    ohs = [w.OH for w in wl.CONV_WORKLOADS.values()]
    assert ohs == [14, 7, 112, 56, 28, 14, 7, 14, 14, 32]
    assert wl.CONV_WORKLOADS[wl.HEADLINE].flops == 231211008
    assert wl.CONV_WORKLOADS["f16_n128_c128to256_32x32_k3_epi"].flops == 77309411328


def test_shipped_tuning_log_is_legal():
    """Every record of the package's gfx950 tuning log parses, names a compiled
    variant and is legal for its shape (the loader drops anything else)."""
    log = os.path.join(ROOT, "tensor_compiler_tiling_amd", "tuned", "gfx950.jsonl")
    lines = [l for l in open(log).read().splitlines() if l.strip()]
    keys = {json.loads(l)["key"] for l in lines}
    ct.ct_cache_clear()
    try:
        assert ct.ct_cache_load(log) == 0
        assert ct.ct_cache_size() == len(keys)
        for name, w in wl.CONV_WORKLOADS.items():
            st, cfg, from_cache = ct.ct_conv2d_query(*_args(w))
            assert st == 0 and from_cache == 1, name
    finally:
        ct.ct_cache_clear()


def test_traffic_lookup_matches_the_filter_form(tmp_path, monkeypatch):
    """bench.py reports a traffic record only for the kernel source, tile and
    filter form (reordered per call or prepared) it was measured with."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    kern = "h2f16_m128n128_w2x2_r2x2_kc16"
    tile = {"split_k": 1, "stages": 16, "kc": 16}
    dig = bench.source_digest(kern)
    recs = [{"workload": "w", "kernel": kern, "tile": tile, "source_sha256": dig, "traffic_bytes_per_launch": 11},
            {"workload": "w", "kernel": kern, "tile": tile, "source_sha256": dig, "traffic_bytes_per_launch": 22,
             "filter": "prepared"},
            {"workload": "v", "kernel": kern, "tile": tile, "source_sha256": "0" * 64, "traffic_bytes_per_launch": 33}]
    log = tmp_path / "traffic.json"
    log.write_text(json.dumps(recs))
    monkeypatch.setattr(bench, "TRAFFIC_LOG", str(log))
    assert bench.measured_traffic("w", kern, tile) == 11
    assert bench.measured_traffic("w", kern, tile, prepared=True) == 22
    assert bench.measured_traffic("w", kern, {"split_k": 2, "stages": 16, "kc": 16}) is None
    assert bench.measured_traffic("v", kern, tile) is None  # taken with another kernel source


def test_traffic_records_point_at_summaries():
    recs = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for r in recs:
        assert os.path.exists(os.path.join(ROOT, r["summary"])), r["summary"]
        assert r["traffic_bytes_per_launch"] > 0
        assert len(r["source_sha256"]) == 64


# ------------------------------------------------------- depthwise convolution
@pytest.mark.parametrize("bad", [
    dict(N=0), dict(C=0), dict(H=0), dict(KW=0), dict(stride=0), dict(pad=-1),
    dict(KH=12),  # larger than the padded input (8 + 2)
])
def test_depthwise_invalid_shapes_rejected_before_any_hip_call(bad):
    a = dict(N=1, C=4, H=8, W=8, KH=3, KW=3, stride=1, pad=1)
    a.update(bad)
    st = ct.library().ct_conv2d_nchw_depthwise(16, 16, 16, a["N"], a["C"], a["H"], a["W"], a["KH"],
                                               a["KW"], a["stride"], a["pad"], 0, 0, None, None, 1e-5,
                                               None)
    assert st == ct.CT_ERR_INVALID_ARG, ct.ct_last_error()


def test_depthwise_null_and_unsupported():
    lib = ct.library()
    shape = (1, 4, 8, 8, 3, 3, 1, 1)
    assert lib.ct_conv2d_nchw_depthwise(None, 16, 16, *shape, 0, 0, None, None, 1e-5, None) == -1
    assert lib.ct_conv2d_nchw_depthwise(16, 16, 16, *shape, 7, 0, None, None, 1e-5, None) == -1
    assert lib.ct_conv2d_nchw_depthwise(16, 16, 16, *shape, 0, 1, None, None, 1e-5, None) == -1
    assert lib.ct_conv2d_nchw_depthwise(16, 16, 16, *shape, 0, 2, 16, None, 1e-5, None) == -1
    # more than 256 taps
    st = lib.ct_conv2d_nchw_depthwise(16, 16, 16, 1, 2, 40, 40, 17, 17, 1, 0, 0, 0, None, None, 1e-5, None)
    assert st == ct.CT_ERR_UNSUPPORTED and "256 taps" in ct.ct_last_error()
    # an output row wider than one workgroup's LDS window
    st = lib.ct_conv2d_nchw_depthwise(16, 16, 16, 1, 2, 4, 60000, 3, 3, 1, 1, 0, 0, None, None, 1e-5, None)
    assert st == ct.CT_ERR_UNSUPPORTED and "LDS" in ct.ct_last_error()


# ------------------------------------------------------ general broadcast chain
def test_chain_program_layout_matches_the_header():
    """ct_bcast_program as ctypes sees it: 3 ints, then 3 x 8 steps of
    (int, int, float)."""
    assert ctypes.sizeof(ct.ct_chain_op) == 12
    assert ctypes.sizeof(ct.ct_bcast_program) == 12 + 3 * 8 * 12
    p = ct.make_program([("set", "a0"), ("add", 1e-5), ("rsqrt",)], [], [("set", "x"), ("mul", "c0")])
    assert list(p.n_ops) == [3, 0, 2]
    assert (p.ops[0][1].op, p.ops[0][1].src) == (ct.CHAIN_OPS["add"], ct.CHAIN_SRCS["imm"])
    assert abs(p.ops[0][1].imm - 1e-5) < 1e-12
    assert (p.ops[2][1].op, p.ops[2][1].src) == (ct.CHAIN_OPS["mul"], ct.CHAIN_SRCS["c0"])


@pytest.mark.parametrize("case", [
    "null_prog", "null_out", "zero_outer", "zero_P", "zero_inner", "dtype", "mode", "too_many_steps",
    "bad_op", "bad_src", "c0_reads_x", "c0_reads_c1", "c1_reads_c1", "array_null", "x_null", "inplace_f16",
])
def test_chain_invalid_arguments_rejected_before_any_hip_call(case):
    lib = ct.library()
    prog = ct.make_program([("set", "a0")], [], [("set", "x"), ("mul", "c0")])
    a = dict(prog=ctypes.byref(prog), a0=16, x=32, out=64, dt=ct.CT_F32, outer=2, P=3, inner=64, mode=0)
    if case == "null_prog":
        a["prog"] = None
    elif case == "null_out":
        a["out"] = None
    elif case == "zero_outer":
        a["outer"] = 0
    elif case == "zero_P":
        a["P"] = 0
    elif case == "zero_inner":
        a["inner"] = 0
    elif case == "dtype":
        a["dt"] = ct.CT_BF16
    elif case == "mode":
        a["mode"] = 7
    elif case == "too_many_steps":
        prog.n_ops[1] = 9
    elif case == "bad_op":
        prog.ops[0][0].op = 42
    elif case == "bad_src":
        prog.ops[0][0].src = 8
    elif case == "c0_reads_x":
        prog.ops[0][0].src = ct.CHAIN_SRCS["x"]
    elif case == "c0_reads_c1":
        prog.ops[0][0].src = ct.CHAIN_SRCS["c1"]
    elif case == "c1_reads_c1":
        prog.n_ops[1] = 1
        prog.ops[1][0].op, prog.ops[1][0].src = ct.CHAIN_OPS["set"], ct.CHAIN_SRCS["c1"]
    elif case == "array_null":
        a["a0"] = None
    elif case == "x_null":
        a["x"] = None
    elif case == "inplace_f16":
        a["dt"], a["out"] = ct.CT_F16, a["x"]
    st = lib.ct_broadcast_chain(a["prog"], a["a0"], None, None, None, a["x"], a["out"], a["dt"], a["outer"],
                                a["P"], a["inner"], a["mode"], None)
    assert st == ct.CT_ERR_INVALID_ARG, (case, ct.ct_last_error())


def test_chain_channel_mode_unsupported_shapes():
    """CT_BC_CHANNEL where the channel-bound conditions fail: an error before
    any launch (inner < 32, rows not whole 16-byte vectors, misaligned out)."""
    lib = ct.library()
    prog = ct.make_program([("set", 1.0)], [], [])
    for inner, out, dt in [(16, 256, ct.CT_F32), (34, 256, ct.CT_F32), (36, 256, ct.CT_F16), (64, 260, ct.CT_F32)]:
        st = lib.ct_broadcast_chain(ctypes.byref(prog), None, None, None, None, None, out, dt, 4, 3, inner,
                                    ct.CT_BC_CHANNEL, None)
        assert st == ct.CT_ERR_UNSUPPORTED, (inner, out, dt, ct.ct_last_error())


# ------------------------------------------------------------- guided search
@pytest.mark.parametrize("lam", [0.0, 1e-3, 2.5])
def test_ridge_fit_matches_the_oracle(lam):
    r = np.random.default_rng(510)
    X = np.column_stack([np.ones(40), r.normal(size=(40, 7))])
    y = r.normal(size=40)
    st, w = ct.ct_ridge_fit(X, y, lam)
    assert st == ct.CT_OK
    np.testing.assert_allclose(w, O.ridge_fit(X, y, lam), rtol=1e-9, atol=1e-12)


def test_ridge_fit_errors():
    X = np.ones((3, 2))  # rank 1: singular without shrinkage
    assert ct.ct_ridge_fit(X, np.ones(3), 0.0)[0] == ct.CT_ERR_INVALID_ARG
    assert ct.ct_ridge_fit(X, np.ones(3), 1e-3)[0] == ct.CT_OK
    assert ct.ct_ridge_fit(X, np.ones(3), -1.0)[0] == ct.CT_ERR_INVALID_ARG


def _landscape(n, d, seed):
    """Features with an intercept and costs exactly exp(features . w_true)."""
    r = np.random.default_rng(seed)
    F = np.column_stack([np.ones(n), r.normal(size=(n, d - 1))])
    w = r.normal(size=d)
    return F, np.exp(F @ w)


def test_guided_search_order_is_a_deterministic_prefix_without_repeats():
    F, c = _landscape(300, 6, 520)
    st, a = ct.ct_guided_search_table(F, c, 40, 8, 2, seed=7)
    st2, b = ct.ct_guided_search_table(F, c, 40, 8, 2, seed=7)
    st3, e = ct.ct_guided_search_table(F, c, 40, 8, 2, seed=8)
    assert st == st2 == st3 == ct.CT_OK
    assert a == b and len(a) == 40 and len(set(a)) == 40 and all(0 <= i < 300 for i in a)
    assert a[:8] != e[:8]  # the first batch is the seed's draw


def test_guided_search_times_everything_when_the_budget_allows():
    F, c = _landscape(50, 4, 521)
    st, order = ct.ct_guided_search_table(F, c, 1000, 8, 2)
    assert st == ct.CT_OK and sorted(order) == list(range(50))


def test_guided_search_finds_the_optimum_of_a_log_linear_landscape():
    """Costs exactly log-linear in the features: once the first batch has
    more points than features, the fit is exact and the next batch's model
    picks are the true best untimed points, so the optimum is timed in the
    second batch -- where uniform draws of the same budget would miss it."""
    F, c = _landscape(2000, 6, 522)
    st, order = ct.ct_guided_search_table(F, c, 16, 8, 2, seed=3)
    assert st == ct.CT_OK
    assert int(np.argmin(c)) in order[8:16]
    best_found = min(c[i] for i in order)
    assert best_found == c.min()


def test_guided_search_skips_failed_trials_in_the_fit():
    """Points whose trial fails (cost <= 0) are timed once and never refit; the
    search still reaches the optimum among the rest."""
    F, c = _landscape(500, 5, 523)
    c = c.copy()
    worst = np.argsort(c)[-100:]
    c[worst] = -1.0
    st, order = ct.ct_guided_search_table(F, c, 24, 8, 2, seed=4)
    assert st == ct.CT_OK and len(set(order)) == 24
    ok = c > 0
    assert min(c[i] for i in order if ok[i]) == c[ok].min()


def test_guided_search_errors():
    F, c = _landscape(10, 3, 524)
    for kw in [dict(max_trials=0, batch=4, n_explore=1), dict(max_trials=5, batch=0, n_explore=0),
               dict(max_trials=5, batch=4, n_explore=5)]:
        assert ct.ct_guided_search_table(F, c, kw["max_trials"], kw["batch"], kw["n_explore"])[0] == \
            ct.CT_ERR_INVALID_ARG
    best = ct.ct_tile_config()
    # batch < 1 is refused before any HIP call
    st = ct.library().ct_conv2d_tune_guided(1, 8, 8, 8, 8, 3, 3, 1, 1, 0, 0, 4, 0, 0, 1.0, None,
                                            ctypes.byref(best), None, 0, None)
    assert st == ct.CT_ERR_INVALID_ARG and "batch" in ct.ct_last_error()


def test_tensor_helpers_reject_host_and_strided_tensors():
    """The helpers hand raw pointers to the C ABI: a CPU tensor (or a
    non-contiguous view) is refused before any call."""
    import torch
    x = torch.ones(1, 2, 6, 6)
    with pytest.raises(ValueError, match="GPU"):
        ct.conv2d(x, torch.ones(3, 2, 3, 3))
    with pytest.raises(ValueError, match="GPU"):
        ct.conv2d_depthwise(x, torch.ones(2, 1, 3, 3))
    with pytest.raises(ValueError, match="GPU"):
        ct.gemm(torch.ones(4, 5), torch.ones(5, 6))
    with pytest.raises(ValueError, match="GPU"):
        ct.broadcast(torch.ones(4), 2, 3, 3)
    with pytest.raises(ValueError, match="GPU"):
        ct.broadcast_chain(ct.make_program([("set", 1.0)]), 2, 3, 4, arrays=[torch.ones(3)])


def test_prepared_filter_bytes():
    # [CO][CI64/8][KH*KW][8] halves, CI64 = CI rounded up to 64
    assert ct.ct_conv2d_filter_prepared_bytes(256, 256, 3, 3, ct.CT_F16) == 2 * 256 * 256 * 9
    assert ct.ct_conv2d_filter_prepared_bytes(40, 12, 3, 3, ct.CT_BF16) == 2 * 40 * 64 * 9
    assert ct.ct_conv2d_filter_prepared_bytes(40, 72, 3, 3, ct.CT_F16) == 2 * 40 * 128 * 9
    assert ct.ct_conv2d_filter_prepared_bytes(4096, 4096, 1, 1, ct.CT_F16) == 2 * 4096 * 4096
    assert ct.ct_conv2d_filter_prepared_bytes(8, 8, 3, 3, ct.CT_F32) == ct.CT_ERR_INVALID_ARG
    assert ct.ct_conv2d_filter_prepared_bytes(0, 8, 3, 3, ct.CT_F16) == ct.CT_ERR_INVALID_ARG


def _log_line(shape, variant_name, split, stages, kc, error_no=0, us=5.0):
    N, CI, H, W, CO, KH, KW, s, p, dt, epi = shape
    key = f"{N},{CI},{H},{W},{CO},{KH},{KW},{s},{p},{dt},{epi},gfx950,v1"
    return json.dumps({"key": key, "N": N, "CI": CI, "H": H, "W": W, "CO": CO, "KH": KH, "KW": KW,
                       "stride": s, "pad": p, "dtype": dt, "epilogue": epi, "arch": "gfx950",
                       "variant": variant_name, "split_k": split, "stages": stages, "kc": kc, "index": -1,
                       "us": us, "error_no": error_no, "costs_us": [us, us, us], "all_cost": 0.1,
                       "timestamp": 1.0})


def test_tuning_log_resume_skips_logged_points(tmp_path, monkeypatch):
    """The exhaustive search's trial order, then the same order with a log that
    already holds some of the shape's points (successful, failed and illegal
    outcomes, as the tutorial's log does): the logged points are left out and
    the rest keep their order; lines of other shapes and malformed lines are
    ignored."""
    shape = (1, 512, 7, 7, 512, 3, 3, 1, 1, ct.CT_F32, ct.CT_EPI_NONE)
    monkeypatch.delenv("CT_CACHE_PATH", raising=False)
    st, full = ct.ct_conv2d_tune_order(*shape)
    assert st == 0 and len(full) == ct.ct_conv2d_space_size(*shape)
    assert len(set(full)) == len(full)
    logged = full[:5] + full[-2:]  # the first legal points and two illegal ones
    lines = []
    for i, idx in enumerate(logged):
        st, cfg, _ = ct.ct_conv2d_space_entity(*shape, idx)
        assert st == 0
        name = ct.variants()[cfg.variant]["name"]
        lines.append(_log_line(shape, name, cfg.split_k, cfg.stages, cfg.kc, error_no=(0, 4, 6, 1)[i % 4]))
    other = (1, 64, 14, 14, 64, 3, 3, 1, 1, ct.CT_F32, ct.CT_EPI_NONE)
    st, cfg0, _ = ct.ct_conv2d_space_entity(*shape, full[5])
    lines.append(_log_line(other, ct.variants()[cfg0.variant]["name"], cfg0.split_k, cfg0.stages, cfg0.kc))
    lines.append("{not json")
    log = tmp_path / "tune.jsonl"
    log.write_text("\n".join(lines) + "\n")
    monkeypatch.setenv("CT_CACHE_PATH", str(log))
    st, resumed = ct.ct_conv2d_tune_order(*shape)
    assert st == 0
    assert resumed == [i for i in full if i not in set(logged)]
    st, first3 = ct.ct_conv2d_tune_order(*shape, max_trials=3)
    assert st == 0 and first3 == resumed[:3]


def test_tuning_log_loads_the_fastest_successful_record(tmp_path):
    """A log holding every trial of a search (failed ones included) loads as
    one cache record per shape: the fastest successful one."""
    shape = (1, 512, 7, 7, 512, 3, 3, 1, 1, ct.CT_F32, ct.CT_EPI_NONE)
    st, full = ct.ct_conv2d_tune_order(*shape)
    pts = []
    for idx in full[:6]:
        st, cfg, legal = ct.ct_conv2d_space_entity(*shape, idx)
        assert legal
        pts.append(cfg)
    lines = [_log_line(shape, ct.variants()[c.variant]["name"], c.split_k, c.stages, c.kc,
                       error_no=e, us=u) for c, e, u in zip(pts, (0, 0, 6, 0, 4, 0), (9.0, 7.5, 1.0, 8.0, 0.5, 7.75))]
    log = tmp_path / "all.jsonl"
    log.write_text("\n".join(lines) + "\n")
    ct.ct_cache_clear()
    assert ct.ct_cache_load(str(log)) == 0 and ct.ct_cache_size() == 1
    st, cfg, from_cache = ct.ct_conv2d_query(*shape)
    assert from_cache == 1 and (cfg.variant, cfg.split_k, cfg.stages, cfg.kc) == (
        pts[1].variant, pts[1].split_k, pts[1].stages, pts[1].kc)
    ct.ct_cache_clear()


# ---- the tutorial template's space and resource check in the runtime ------

def _gist():
    with open(os.path.join(os.path.dirname(__file__), "golden", "tvm_tuning_log.json")) as f:
        return json.load(f)


_GIST_SHAPE = (1, 512, 7, 7, 512, 3, 3, 1, 1)  # N, CI, H, W, CO, KH, KW, stride, pad


def test_tvm_space_size_matches_the_gist_dump():
    g = _gist()
    assert ct.ct_tvm_space_size(*_GIST_SHAPE) == g["space"]["total"] == 10454400


def test_tvm_space_indices_match_the_gist_log():
    g = _gist()
    pairs = [(t["config"], t["index"]) for t in g["trials"]] + [(g["best"]["config"], g["best"]["index"])]
    assert len(pairs) == 21
    for cfg, idx in pairs:
        assert ct.ct_tvm_space_index(*_GIST_SHAPE, cfg) == idx
        st, got = ct.ct_tvm_space_entity(*_GIST_SHAPE, idx)
        assert st == 0 and got == cfg


def test_tvm_page_limits_reproduce_the_gist_rejections():
    """Page-1 mode: exactly the trials the tutorial's run rejected before
    timing them (error_no 1) exceed the 48 KiB shared-memory limit."""
    g = _gist()
    for t in g["trials"]:
        fits, nbytes, threads = ct.ct_tvm_config_check(t["config"], 1, ct.CT_TVM_LIMITS_PAGE)
        assert fits == (0 if t["error_no"] == 1 else 1), (t["no"], nbytes)
        assert threads <= 1024
    fits, nbytes, threads = ct.ct_tvm_config_check(g["best"]["config"], 1, ct.CT_TVM_LIMITS_PAGE)
    # Y_b = X_b = 7, RC_s = 8, RY_s = RX_s = 3, F_b = 64 (threads 64)
    assert (fits, nbytes, threads) == (1, 4 * (8 * 9 * 9 + 64 * 8 * 3 * 3), 64)
    # gfx950's 160 KiB admits every config the page mode admits
    for t in g["trials"]:
        if ct.ct_tvm_config_check(t["config"], 1, ct.CT_TVM_LIMITS_PAGE)[0] == 1:
            assert ct.ct_tvm_config_check(t["config"], 1, ct.CT_TVM_LIMITS_GFX950)[0] == 1


def test_tvm_space_agrees_with_the_oracle_on_random_points():
    sp = O.tvm_tutorial_space(*(_GIST_SHAPE[:1] + _GIST_SHAPE[2:4] + (_GIST_SHAPE[4], _GIST_SHAPE[1])
                                + _GIST_SHAPE[5:]))
    rng = np.random.default_rng(77)
    for idx in rng.integers(0, 10454400, 300):
        st, got = ct.ct_tvm_space_entity(*_GIST_SHAPE, int(idx))
        assert st == 0 and got == sp.entity_at(int(idx))
        for stride in (1, 2):
            fits, nbytes, _ = ct.ct_tvm_config_check(got, stride, ct.CT_TVM_LIMITS_GFX950)
            assert nbytes == O.tvm_template_shared_bytes(got, stride)
            assert fits == int(nbytes <= 160 * 1024 and O.tvm_template_threads(got) <= 1024)
    # a strided, non-square shape: the space is the product of its knob lengths
    shape = (2, 48, 13, 9, 40, 3, 1, 2, 1)
    N, CI, H, W, CO, KH, KW, s, p = shape
    OH, OW = (H + 2 * p - KH) // s + 1, (W + 2 * p - KW) // s + 1
    want = (ct.ct_split_count(CO, 4) * ct.ct_split_count(OH, 4) * ct.ct_split_count(OW, 4)
            * ct.ct_split_count(CI, 3) * ct.ct_split_count(KH, 3) * ct.ct_split_count(KW, 3) * 3 * 2)
    assert ct.ct_tvm_space_size(*shape) == want
    for idx in (0, 1, want // 3, want - 1):
        st, cfg = ct.ct_tvm_space_entity(*shape, idx)
        assert st == 0 and ct.ct_tvm_space_index(*shape, cfg) == idx


def test_tvm_space_argument_errors():
    assert ct.ct_tvm_space_size(0, 512, 7, 7, 512, 3, 3, 1, 1) == ct.CT_ERR_INVALID_ARG
    st, _ = ct.ct_tvm_space_entity(*_GIST_SHAPE, 10454400)
    assert st == ct.CT_ERR_INVALID_ARG
    st, _ = ct.ct_tvm_space_entity(*_GIST_SHAPE, -1)
    assert st == ct.CT_ERR_INVALID_ARG
    g = _gist()
    cfg = dict(g["best"]["config"])
    cfg["tile_f"] = [8, 1, 64, 2]  # product 1024, not a split of 512
    assert ct.ct_tvm_space_index(*_GIST_SHAPE, cfg) == -1
    cfg = dict(g["best"]["config"], auto_unroll_max_step=7)
    assert ct.ct_tvm_space_index(*_GIST_SHAPE, cfg) == -1
    cfg = dict(g["best"]["config"], tile_rc=[64, 0, 8])
    assert ct.ct_tvm_config_check(cfg, 1)[0] == ct.CT_ERR_INVALID_ARG
    assert ct.ct_tvm_config_check(g["best"]["config"], 1, 5)[0] == ct.CT_ERR_INVALID_ARG
    assert ct.ct_tvm_config_check(g["best"]["config"], 0)[0] == ct.CT_ERR_INVALID_ARG
