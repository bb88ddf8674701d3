"""ctypes binding of libconvtile.so (include/convtile.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  The functions named like the C entry points take device pointers
(ints) or torch tensors and return the C status; the short helpers
(``conv2d``, ``broadcast``, ``tune``, ``query``) allocate outputs with torch
and raise ``ConvTileError`` on a non-zero status.  There is no fallback: if
the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libconvtile.so")

CT_OK = 0
CT_ERR_INVALID_ARG = -1
CT_ERR_UNSUPPORTED = -2
CT_ERR_HIP = -3
CT_ERR_NO_MEMORY = -4
CT_ERR_IO = -5
CT_ERR_TUNE_FAILED = -6

CT_F32, CT_F16, CT_BF16 = 0, 1, 2
# bytes of the no-allocation entry point's fixed scratch (partials and filter copy)
CT_NOALLOC_SCRATCH_BYTES = 16 << 20
CT_EPI_NONE, CT_EPI_BIAS, CT_EPI_EXP_BIAS_RSQRT = 0, 1, 2
CT_BC_EXP = 0
CT_BC_AUTO, CT_BC_CHANNEL, CT_BC_FLAT = 0, 1, 2
CT_CHAIN_MAX_OPS = 8
CHAIN_OPS = {"set": 0, "add": 1, "sub": 2, "mul": 3, "div": 4, "rsub": 5, "rdiv": 6, "exp": 7, "rsqrt": 8,
             "sqrt": 9}
CHAIN_SRCS = {"imm": 0, "x": 1, "c0": 2, "c1": 3, "a0": 4, "a1": 5, "a2": 6, "a3": 7}
CT_TRIAL_OK, CT_TRIAL_ILLEGAL, CT_TRIAL_RUNTIME, CT_TRIAL_TIMEOUT = 0, 1, 4, 6


class ct_tile_config(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("split_k", ctypes.c_int), ("stages", ctypes.c_int),
                ("kc", ctypes.c_int), ("index", ctypes.c_longlong), ("us", ctypes.c_float),
                ("error_no", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class ct_chain_op(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int), ("src", ctypes.c_int), ("imm", ctypes.c_float)]


class ct_bcast_program(ctypes.Structure):
    _fields_ = [("n_ops", ctypes.c_int * 3), ("ops", (ct_chain_op * CT_CHAIN_MAX_OPS) * 3)]


class ct_tvm_config(ctypes.Structure):
    _fields_ = [("tile_f", ctypes.c_int * 4), ("tile_y", ctypes.c_int * 4), ("tile_x", ctypes.c_int * 4),
                ("tile_rc", ctypes.c_int * 3), ("tile_ry", ctypes.c_int * 3), ("tile_rx", ctypes.c_int * 3),
                ("auto_unroll_max_step", ctypes.c_int), ("unroll_explicit", ctypes.c_int)]

    def as_dict(self):
        return {f: (list(getattr(self, f)) if f.startswith("tile_") else getattr(self, f))
                for f, _ in self._fields_}

    @classmethod
    def from_dict(cls, d):
        c = cls()
        for f, _ in cls._fields_:
            if f.startswith("tile_"):
                arr = getattr(c, f)
                for i, v in enumerate(d[f]):
                    arr[i] = v
            else:
                setattr(c, f, d[f])
        return c


CT_TVM_LIMITS_PAGE = 0
CT_TVM_LIMITS_GFX950 = 1


class ct_variant_desc(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("dtype", ctypes.c_int), ("kind", ctypes.c_int),
                ("mfma_m", ctypes.c_int), ("mfma_n", ctypes.c_int), ("mfma_k", ctypes.c_int),
                ("waves_m", ctypes.c_int), ("waves_n", ctypes.c_int), ("waves_k", ctypes.c_int),
                ("reps_m", ctypes.c_int), ("reps_n", ctypes.c_int), ("tile_m", ctypes.c_int),
                ("tile_n", ctypes.c_int), ("kc_max", ctypes.c_int), ("threads", ctypes.c_int)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["name"] = self.name.decode()
        return d


class ct_tune_record(ctypes.Structure):
    _fields_ = [("cfg", ct_tile_config), ("costs_us", ctypes.c_float * 3), ("n_costs", ctypes.c_int),
                ("error_no", ctypes.c_int), ("all_cost_s", ctypes.c_double),
                ("timestamp", ctypes.c_double)]


class ConvTileError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        lib = _load()
        msg = lib.ct_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.ct_status_string(status).decode()} ({status}): {msg}")


_I, _LL, _F, _P = ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_void_p
_SHAPE = [_I] * 11  # N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue

_SIGS = {
    "ct_conv2d_nchw_fwd": (_I, [_P, _P, _P] + [_I] * 11 + [_P, _P, _F, _P]),
    "ct_conv2d_nchw_fwd_noalloc": (_I, [_P, _P, _P] + [_I] * 11 + [_P, _P, _F, _P]),
    "ct_conv2d_nchw_fwd_prepared": (_I, [_P, _P, _P] + [_I] * 11 + [_P, _P, _F, _P]),
    "ct_conv2d_filter_prepared_bytes": (_LL, [_I] * 5),
    "ct_conv2d_prepare_filter": (_I, [_P, _P] + [_I] * 5 + [_P]),
    "ct_conv2d_nchw_fwd_config": (_I, [_P, _P, _P] + [_I] * 11 +
                                  [_P, _P, _F, ctypes.POINTER(ct_tile_config), _P]),
    "ct_conv2d_nchw_direct": (_I, [_P, _P, _P] + [_I] * 11 + [_P, _P, _F, _P]),
    "ct_conv2d_space_size": (_LL, _SHAPE),
    "ct_conv2d_space_entity": (_I, _SHAPE + [_LL, ctypes.POINTER(ct_tile_config),
                                             ctypes.POINTER(_I)]),
    "ct_conv2d_tune": (_I, _SHAPE + [_I, _F, _P, ctypes.POINTER(ct_tile_config),
                                     ctypes.POINTER(ct_tune_record), _I, ctypes.POINTER(_I)]),
    "ct_conv2d_query": (_I, _SHAPE + [ctypes.POINTER(ct_tile_config), ctypes.POINTER(_I)]),
    "ct_conv2d_tune_order": (_I, _SHAPE + [_I, ctypes.POINTER(_LL), _I, ctypes.POINTER(_I)]),
    "ct_conv2d_tune_guided": (_I, _SHAPE + [_I, _I, ctypes.c_ulonglong, _F, _P, ctypes.POINTER(ct_tile_config),
                                            ctypes.POINTER(ct_tune_record), _I, ctypes.POINTER(_I)]),
    "ct_ridge_fit": (_I, [_P, _P, _I, _I, ctypes.c_double, _P]),
    "ct_guided_search_table": (_I, [_P, _P, _I, _I, _I, _I, _I, ctypes.c_ulonglong, ctypes.c_double, _P, _P]),
    "ct_gemm_fwd": (_I, [_P, _P, _P] + [_I] * 5 + [_P, _P, _F, _P]),
    "ct_gemm_tune": (_I, [_I] * 5 + [_I, _F, _P, ctypes.POINTER(ct_tile_config),
                                   ctypes.POINTER(ct_tune_record), _I, ctypes.POINTER(_I)]),
    "ct_gemm_query": (_I, [_I] * 5 + [ctypes.POINTER(ct_tile_config), ctypes.POINTER(_I)]),
    "ct_conv2d_nchw_depthwise": (_I, [_P, _P, _P] + [_I] * 10 + [_P, _P, _F, _P]),
    "ct_broadcast_chain": (_I, [ctypes.POINTER(ct_bcast_program)] + [_P] * 6 + [_I, _LL, _I, _LL, _I, _P]),
    "ct_variant_count": (_I, []),
    "ct_variant_info": (_I, [_I, ctypes.POINTER(ct_variant_desc)]),
    "ct_split_count": (_LL, [_LL, _I]),
    "ct_split_entity": (_I, [_LL, _I, _LL, ctypes.POINTER(_LL)]),
    "ct_tvm_space_size": (_LL, [_I] * 9),
    "ct_tvm_space_entity": (_I, [_I] * 9 + [_LL, ctypes.POINTER(ct_tvm_config)]),
    "ct_tvm_space_index": (_LL, [_I] * 9 + [ctypes.POINTER(ct_tvm_config)]),
    "ct_tvm_config_check": (_I, [ctypes.POINTER(ct_tvm_config), _I, _I, ctypes.POINTER(_LL),
                                 ctypes.POINTER(_I)]),
    "ct_broadcast_nchw": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "ct_cache_load": (_I, [ctypes.c_char_p]),
    "ct_cache_save": (_I, [ctypes.c_char_p]),
    "ct_cache_clear": (_I, []),
    "ct_cache_size": (_I, []),
    "ct_release": (_I, []),
    "ct_init": (_I, [_I]),
    "ct_plan_misses": (_LL, []),
    "ct_status_string": (ctypes.c_char_p, [_I]),
    "ct_last_error": (ctypes.c_char_p, []),
    "ct_version": (ctypes.c_char_p, []),
}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m tensor_compiler_tiling_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def exported_names() -> List[str]:
    return list(_SIGS)


# ---------------------------------------------------------------- marshal --
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch tensor or a device pointer, got {type(t)}")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def dtype_code(torch_dtype) -> int:
    import torch
    m = {torch.float32: CT_F32, torch.float16: CT_F16, torch.bfloat16: CT_BF16}
    if torch_dtype not in m:
        raise ValueError(f"unsupported dtype {torch_dtype}")
    return m[torch_dtype]


def out_extent(inp: int, k: int, stride: int, pad: int) -> int:
    return (inp + 2 * pad - k) // stride + 1


# ------------------------------------------------- entry points (same names) --
def ct_conv2d_nchw_fwd(x, w, y, N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue,
                       bias=None, var=None, eps=1e-5, stream=None) -> int:
    return _load().ct_conv2d_nchw_fwd(_ptr(x), _ptr(w), _ptr(y), N, CI, H, W, CO, KH, KW, stride,
                                      pad, dtype, epilogue, _ptr(bias), _ptr(var), eps,
                                      _stream(stream))


def ct_conv2d_nchw_fwd_noalloc(x, w, y, N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue,
                               bias=None, var=None, eps=1e-5, stream=None) -> int:
    return _load().ct_conv2d_nchw_fwd_noalloc(_ptr(x), _ptr(w), _ptr(y), N, CI, H, W, CO, KH, KW, stride,
                                              pad, dtype, epilogue, _ptr(bias), _ptr(var), eps,
                                              _stream(stream))


def ct_conv2d_nchw_fwd_prepared(x, wp, y, N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue,
                                bias=None, var=None, eps=1e-5, stream=None) -> int:
    return _load().ct_conv2d_nchw_fwd_prepared(_ptr(x), _ptr(wp), _ptr(y), N, CI, H, W, CO, KH, KW, stride,
                                               pad, dtype, epilogue, _ptr(bias), _ptr(var), eps,
                                               _stream(stream))


def ct_conv2d_filter_prepared_bytes(CO, CI, KH, KW, dtype) -> int:
    return _load().ct_conv2d_filter_prepared_bytes(CO, CI, KH, KW, dtype)


def ct_conv2d_prepare_filter(w, wp, CO, CI, KH, KW, dtype, stream=None) -> int:
    return _load().ct_conv2d_prepare_filter(_ptr(w), _ptr(wp), CO, CI, KH, KW, dtype, _stream(stream))


def prepare_filter(w, stream=None):
    """The prepared (regrouped) copy of a half-precision filter w [CO, CI, KH, KW]
    as a flat torch tensor of the same dtype."""
    import torch
    _on_gpu(w=w)
    CO, CI, KH, KW = w.shape
    dt = dtype_code(w.dtype)
    nbytes = ct_conv2d_filter_prepared_bytes(CO, CI, KH, KW, dt)
    check(nbytes if nbytes < 0 else 0, "prepare_filter")
    wp = torch.empty(nbytes // 2, dtype=w.dtype, device=w.device)
    check(ct_conv2d_prepare_filter(w, wp, CO, CI, KH, KW, dt, stream), "prepare_filter")
    return wp


def ct_conv2d_nchw_fwd_config(x, w, y, N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue,
                              bias, var, eps, cfg: ct_tile_config, stream=None) -> int:
    return _load().ct_conv2d_nchw_fwd_config(_ptr(x), _ptr(w), _ptr(y), N, CI, H, W, CO, KH, KW,
                                             stride, pad, dtype, epilogue, _ptr(bias), _ptr(var),
                                             eps, ctypes.byref(cfg), _stream(stream))


def ct_conv2d_nchw_direct(x, w, y, N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue,
                          bias=None, var=None, eps=1e-5, stream=None) -> int:
    return _load().ct_conv2d_nchw_direct(_ptr(x), _ptr(w), _ptr(y), N, CI, H, W, CO, KH, KW,
                                         stride, pad, dtype, epilogue, _ptr(bias), _ptr(var), eps,
                                         _stream(stream))


def ct_conv2d_space_size(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue) -> int:
    return _load().ct_conv2d_space_size(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue)


def ct_conv2d_space_entity(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue,
                           index) -> Tuple[int, ct_tile_config, int]:
    cfg = ct_tile_config()
    legal = _I(0)
    st = _load().ct_conv2d_space_entity(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue,
                                        index, ctypes.byref(cfg), ctypes.byref(legal))
    return st, cfg, legal.value


def ct_conv2d_tune(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials=0,
                   min_repeat_ms=100.0, stream=None, max_records=4096):
    best = ct_tile_config()
    recs = (ct_tune_record * max(max_records, 1))()
    n = _I(0)
    st = _load().ct_conv2d_tune(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials,
                                min_repeat_ms, _stream(stream), ctypes.byref(best), recs,
                                max_records, ctypes.byref(n))
    return st, best, [recs[i] for i in range(n.value)]


def ct_conv2d_query(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue):
    cfg = ct_tile_config()
    fc = _I(0)
    st = _load().ct_conv2d_query(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue,
                                 ctypes.byref(cfg), ctypes.byref(fc))
    return st, cfg, fc.value


def ct_gemm_fwd(A, B, C, M, N, K, dtype, epilogue, bias=None, var=None, eps=1e-5, stream=None) -> int:
    return _load().ct_gemm_fwd(_ptr(A), _ptr(B), _ptr(C), M, N, K, dtype, epilogue, _ptr(bias),
                               _ptr(var), eps, _stream(stream))


def ct_conv2d_nchw_depthwise(x, w, y, N, C, H, W, KH, KW, stride, pad, dtype, epilogue, bias=None,
                             var=None, eps=1e-5, stream=None) -> int:
    return _load().ct_conv2d_nchw_depthwise(_ptr(x), _ptr(w), _ptr(y), N, C, H, W, KH, KW, stride, pad,
                                            dtype, epilogue, _ptr(bias), _ptr(var), eps,
                                            _stream(stream))


def ct_broadcast_chain(prog, a0, a1, a2, a3, x, out, out_dtype, outer, P, inner, mode=CT_BC_AUTO,
                       stream=None) -> int:
    return _load().ct_broadcast_chain(ctypes.byref(prog), _ptr(a0), _ptr(a1), _ptr(a2), _ptr(a3), _ptr(x),
                                      _ptr(out), out_dtype, outer, P, inner, mode, _stream(stream))


def ct_conv2d_tune_guided(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials=64, batch=8,
                          seed=0, min_repeat_ms=100.0, stream=None, max_records=4096):
    best = ct_tile_config()
    recs = (ct_tune_record * max(max_records, 1))()
    n = _I(0)
    st = _load().ct_conv2d_tune_guided(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials, batch,
                                       seed, min_repeat_ms, _stream(stream), ctypes.byref(best), recs, max_records,
                                       ctypes.byref(n))
    return st, best, [recs[i] for i in range(n.value)]


def ct_ridge_fit(X, y, lam=0.0):
    """numpy in, numpy out: (status, w)."""
    import numpy as np
    X = np.ascontiguousarray(X, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    n, d = X.shape
    w = np.zeros(d, np.float64)
    st = _load().ct_ridge_fit(X.ctypes.data, y.ctypes.data, n, d, float(lam), w.ctypes.data)
    return st, w


def ct_guided_search_table(feats, costs, max_trials, batch, n_explore, seed=0, lam=1e-3):
    """numpy in: (status, order of the points the search would time)."""
    import numpy as np
    F = np.ascontiguousarray(feats, dtype=np.float64)
    c = np.ascontiguousarray(costs, dtype=np.float64)
    n, d = F.shape
    order = np.zeros(max(max_trials, 1), np.int32)
    cnt = _I(0)
    st = _load().ct_guided_search_table(F.ctypes.data, c.ctypes.data, n, d, max_trials, batch, n_explore, seed,
                                        float(lam), order.ctypes.data, ctypes.addressof(cnt))
    return st, order[:cnt.value].tolist()


def ct_gemm_tune(M, N, K, dtype, epilogue, max_trials=0, min_repeat_ms=100.0, stream=None,
                 max_records=4096):
    best = ct_tile_config()
    recs = (ct_tune_record * max(max_records, 1))()
    n = _I(0)
    st = _load().ct_gemm_tune(M, N, K, dtype, epilogue, max_trials, min_repeat_ms, _stream(stream),
                              ctypes.byref(best), recs, max_records, ctypes.byref(n))
    return st, best, [recs[i] for i in range(n.value)]


def ct_gemm_query(M, N, K, dtype, epilogue):
    cfg = ct_tile_config()
    fc = _I(0)
    st = _load().ct_gemm_query(M, N, K, dtype, epilogue, ctypes.byref(cfg), ctypes.byref(fc))
    return st, cfg, fc.value


def ct_variant_count() -> int:
    return _load().ct_variant_count()


def ct_variant_info(v: int):
    d = ct_variant_desc()
    st = _load().ct_variant_info(v, ctypes.byref(d))
    return st, d


def ct_split_count(n: int, k: int) -> int:
    return _load().ct_split_count(n, k)


def ct_split_entity(n: int, k: int, i: int):
    out = (_LL * k)()
    st = _load().ct_split_entity(n, k, i, out)
    return st, list(out)


def ct_tvm_space_size(N, CI, H, W, CO, KH, KW, stride, pad) -> int:
    return _load().ct_tvm_space_size(N, CI, H, W, CO, KH, KW, stride, pad)


def ct_tvm_space_entity(N, CI, H, W, CO, KH, KW, stride, pad, index):
    """(status, config dict) of flat index `index` of the template's space."""
    out = ct_tvm_config()
    st = _load().ct_tvm_space_entity(N, CI, H, W, CO, KH, KW, stride, pad, index, ctypes.byref(out))
    return st, out.as_dict()


def ct_tvm_space_index(N, CI, H, W, CO, KH, KW, stride, pad, cfg: dict) -> int:
    c = ct_tvm_config.from_dict(cfg)
    return _load().ct_tvm_space_index(N, CI, H, W, CO, KH, KW, stride, pad, ctypes.byref(c))


def ct_tvm_config_check(cfg: dict, stride: int, mode: int = CT_TVM_LIMITS_PAGE):
    """(fits 1/0 or status < 0, shared bytes, threads per block)."""
    c = ct_tvm_config.from_dict(cfg)
    nb, nt = _LL(0), _I(0)
    r = _load().ct_tvm_config_check(ctypes.byref(c), stride, mode, ctypes.byref(nb), ctypes.byref(nt))
    return r, nb.value, nt.value


def ct_broadcast_nchw(var, out, N, C, H, W, out_dtype, op=CT_BC_EXP, mode=CT_BC_AUTO,
                      stream=None) -> int:
    return _load().ct_broadcast_nchw(_ptr(var), _ptr(out), N, C, H, W, out_dtype, op, mode,
                                     _stream(stream))


def ct_cache_load(path: str) -> int:
    return _load().ct_cache_load(path.encode())


def ct_cache_save(path: str) -> int:
    return _load().ct_cache_save(path.encode())


def ct_cache_clear() -> int:
    return _load().ct_cache_clear()


def ct_cache_size() -> int:
    return _load().ct_cache_size()


def ct_release() -> int:
    return _load().ct_release()


def ct_status_string(st: int) -> str:
    return _load().ct_status_string(st).decode()


def ct_last_error() -> str:
    return _load().ct_last_error().decode(errors="replace")


def ct_init(device: int = 0) -> int:
    return _load().ct_init(device)


def ct_plan_misses() -> int:
    return _load().ct_plan_misses()


def ct_conv2d_tune_order(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials=0):
    """(status, [flat indices]) the exhaustive search would time, in order,
    skipping points already in the CT_CACHE_PATH log."""
    n = _I(0)
    st = _load().ct_conv2d_tune_order(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials,
                                      None, 0, ctypes.byref(n))
    if st != 0:
        return st, []
    buf = (_LL * max(1, n.value))()
    st = _load().ct_conv2d_tune_order(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials,
                                      buf, n.value, ctypes.byref(n))
    return st, list(buf[:n.value])


def ct_version() -> str:
    return _load().ct_version().decode()


def check(status: int, where: str = "convtile") -> None:
    if status != CT_OK:
        raise ConvTileError(status, where)


# ------------------------------------------------------------ helpers --------
def variants() -> List[dict]:
    out = []
    for v in range(ct_variant_count()):
        st, d = ct_variant_info(v)
        check(st, "ct_variant_info")
        out.append(dict(d.as_dict(), id=v))
    return out


def variant_id(name: str) -> int:
    for d in variants():
        if d["name"] == name:
            return d["id"]
    raise KeyError(name)


def _on_gpu(**tensors) -> None:
    """The C ABI takes raw device pointers: every tensor handed to it must live
    on a GPU and be contiguous (None is skipped)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def conv2d(x, w, stride: int = 1, pad: int = 0, epilogue: int = CT_EPI_NONE, bias=None, var=None,
           eps: float = 1e-5, config: Optional[ct_tile_config] = None, out=None, stream=None,
           direct: bool = False):
    """y = conv2d_nchw(x, w) (+ epilogue), fp32 output allocated with torch."""
    import torch
    _on_gpu(x=x, w=w, bias=bias, var=var, out=out)
    N, CI, H, W = x.shape
    CO, CI2, KH, KW = w.shape
    if CI2 != CI or w.dtype != x.dtype:
        raise ValueError("x and w disagree in channels or dtype")
    OH, OW = out_extent(H, KH, stride, pad), out_extent(W, KW, stride, pad)
    y = out if out is not None else torch.empty((N, CO, OH, OW), dtype=torch.float32,
                                                device=x.device)
    dt = dtype_code(x.dtype)
    if direct:
        st = ct_conv2d_nchw_direct(x, w, y, N, CI, H, W, CO, KH, KW, stride, pad, dt, epilogue,
                                   bias, var, eps, stream)
    elif config is not None:
        st = ct_conv2d_nchw_fwd_config(x, w, y, N, CI, H, W, CO, KH, KW, stride, pad, dt,
                                       epilogue, bias, var, eps, config, stream)
    else:
        st = ct_conv2d_nchw_fwd(x, w, y, N, CI, H, W, CO, KH, KW, stride, pad, dt, epilogue, bias,
                                var, eps, stream)
    check(st, "conv2d")
    return y


def conv2d_prepared(x, wp, filter_shape, stride: int = 1, pad: int = 0, epilogue: int = CT_EPI_NONE,
                    bias=None, var=None, eps: float = 1e-5, out=None, stream=None):
    """conv2d with a half-precision filter already prepared by prepare_filter;
    filter_shape = (CO, CI, KH, KW) of the original filter."""
    import torch
    _on_gpu(x=x, wp=wp, bias=bias, var=var, out=out)
    N, CI, H, W = x.shape
    CO, CI2, KH, KW = filter_shape
    if CI2 != CI or wp.dtype != x.dtype:
        raise ValueError("x and the prepared filter disagree in channels or dtype")
    OH, OW = out_extent(H, KH, stride, pad), out_extent(W, KW, stride, pad)
    y = out if out is not None else torch.empty((N, CO, OH, OW), dtype=torch.float32, device=x.device)
    st = ct_conv2d_nchw_fwd_prepared(x, wp, y, N, CI, H, W, CO, KH, KW, stride, pad, dtype_code(x.dtype),
                                     epilogue, bias, var, eps, stream)
    check(st, "conv2d_prepared")
    return y


def gemm(A, B, epilogue: int = CT_EPI_NONE, bias=None, var=None, eps: float = 1e-5, out=None,
         stream=None):
    """C = A @ B (+ per-row epilogue), fp32 output allocated with torch: A [M, K], B [K, N],
    same dtype, contiguous."""
    import torch
    _on_gpu(A=A, B=B, bias=bias, var=var, out=out)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or A.dtype != B.dtype:
        raise ValueError("A and B disagree in the inner dimension or dtype")
    C = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=A.device)
    check(ct_gemm_fwd(A, B, C, M, N, K, dtype_code(A.dtype), epilogue, bias, var, eps, stream), "gemm")
    return C


def conv2d_depthwise(x, w, stride: int = 1, pad: int = 0, epilogue: int = CT_EPI_NONE, bias=None,
                     var=None, eps: float = 1e-5, out=None, stream=None):
    """Depthwise y[n][c] = conv2d(x[n][c], w[c][0]) (+ epilogue), fp32 output allocated with
    torch: x [N, C, H, W], w [C, 1, KH, KW], same dtype, contiguous."""
    import torch
    _on_gpu(x=x, w=w, bias=bias, var=var, out=out)
    N, C, H, W = x.shape
    C2, one, KH, KW = w.shape
    if C2 != C or one != 1 or w.dtype != x.dtype:
        raise ValueError("w must be [C, 1, KH, KW] of x's channels and dtype")
    OH, OW = out_extent(H, KH, stride, pad), out_extent(W, KW, stride, pad)
    y = out if out is not None else torch.empty((N, C, OH, OW), dtype=torch.float32,
                                                device=x.device)
    st = ct_conv2d_nchw_depthwise(x, w, y, N, C, H, W, KH, KW, stride, pad, dtype_code(x.dtype),
                                  epilogue, bias, var, eps, stream)
    check(st, "conv2d_depthwise")
    return y


def broadcast(var, N: int, H: int, W: int, out_dtype=None, mode: int = CT_BC_AUTO, out=None,
              stream=None):
    """[1,C,1,1] -> [N,C,H,W] of exp(var[c])."""
    import torch
    _on_gpu(var=var, out=out)
    out_dtype = out_dtype or torch.float16
    C = var.numel()
    o = out if out is not None else torch.empty((N, C, H, W), dtype=out_dtype, device=var.device)
    st = ct_broadcast_nchw(var, o, N, C, H, W, dtype_code(o.dtype), CT_BC_EXP, mode, stream)
    check(st, "broadcast")
    return o


def make_program(c0=(), c1=(), v=()) -> ct_bcast_program:
    """A broadcast program from three step lists.  A step is (op,), (op, src)
    or (op, "imm", value) / (op, value): op a CHAIN_OPS name, src a
    CHAIN_SRCS name, a bare number meaning an immediate."""
    prog = ct_bcast_program()
    for c, steps in enumerate((c0, c1, v)):
        steps = list(steps)
        if len(steps) > CT_CHAIN_MAX_OPS:
            raise ValueError(f"chain {c} has {len(steps)} steps (at most {CT_CHAIN_MAX_OPS})")
        prog.n_ops[c] = len(steps)
        for k, st in enumerate(steps):
            op, rest = st[0], st[1:]
            src, imm = "imm", 0.0
            if len(rest) == 1:
                if isinstance(rest[0], str):
                    src = rest[0]
                else:
                    imm = float(rest[0])
            elif len(rest) == 2:
                src, imm = rest[0], float(rest[1])
            prog.ops[c][k].op = CHAIN_OPS[op]
            prog.ops[c][k].src = CHAIN_SRCS[src]
            prog.ops[c][k].imm = imm
    return prog


def broadcast_chain(prog: ct_bcast_program, outer: int, P: int, inner: int, arrays=(), x=None,
                    out_dtype=None, mode: int = CT_BC_AUTO, out=None, stream=None):
    """out[o][p][i] = the program's value ([outer][P][inner], torch-allocated
    unless `out` is given); arrays: up to four per-channel fp32 tensors of P
    floats; x: the producer's fp32 tensor of the output's size, or None."""
    import torch
    arrays = list(arrays) + [None] * (4 - len(arrays))
    _on_gpu(a0=arrays[0], a1=arrays[1], a2=arrays[2], a3=arrays[3], x=x, out=out)
    dev = next((t.device for t in arrays + [x, out] if t is not None), None)
    if dev is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.empty((outer, P, inner), dtype=out_dtype or torch.float32, device=dev)
    st = ct_broadcast_chain(prog, arrays[0], arrays[1], arrays[2], arrays[3], x, out,
                            dtype_code(out.dtype), outer, P, inner, mode, stream)
    check(st, "broadcast_chain")
    return out


def make_config(variant, split_k: int, stages: int, kc: int) -> ct_tile_config:
    c = ct_tile_config()
    c.variant = variant if isinstance(variant, int) else variant_id(variant)
    c.split_k, c.stages, c.kc, c.index = split_k, stages, kc, -1
    return c
