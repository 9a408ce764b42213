"""CPU oracle of the block-scaled low-bit MoE layer (double precision).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
bench's CPU-baseline leg, never by the GPU library.  Thin numpy/ctypes wrapper
over oracle.c, which holds every step of the arithmetic.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None

FMT_E2M1 = 1          # e2m1 + e4m3 per 16
FMT_E2M3 = 2          # e2m3 + UE8M0 per 128
FMT_MXFP4 = 3         # e2m1 + UE8M0 per 32
FMT_INT4_F16 = 4      # int4 + fp16 per 64
FMT_E2M3_E4M3 = 5     # e2m3 + e4m3 per 16
FORMATS = (FMT_E2M1, FMT_E2M3, FMT_MXFP4, FMT_INT4_F16, FMT_E2M3_E4M3)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_init.restype = i32
    lib.oracle_tables.argtypes = [vp, vp, vp, vp]
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_decode.argtypes = [i32, i64, i64, vp, vp, vp]
    lib.oracle_gemv.argtypes = [i32, i64, i64, vp, vp, vp, i64, vp, i64, vp]
    lib.oracle_route.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.oracle_route.restype = i32
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_ffn.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, vp, i64, vp, vp]
    lib.oracle_layer.argtypes = [i32, i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                 i64, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp]
    lib.oracle_layer.restype = i32
    lib.oracle_bf16_round.argtypes = [ctypes.c_double]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_bf16_round_array.argtypes = [vp, i64, vp]
    lib.oracle_fp16_value.argtypes = [ctypes.c_uint]
    lib.oracle_fp16_value.restype = ctypes.c_double
    lib.oracle_int4_table.argtypes = [vp]
    lib.oracle_code_row_bytes.argtypes = [i32, i64]
    lib.oracle_code_row_bytes.restype = i64
    lib.oracle_scale_row_bytes.argtypes = [i32, i64]
    lib.oracle_scale_row_bytes.restype = i64
    lib.oracle_rmsnorm.argtypes = [i64, i64, vp, vp, ctypes.c_double, vp]
    lib.oracle_router_logits.argtypes = [i64, i64, i64, vp, vp, vp]
    lib.oracle_residual_add.argtypes = [i64, vp, vp, vp]
    lib.oracle_quantize_mx_e4m3.argtypes = [i64, i64, vp, vp, vp]
    lib.oracle_threads.argtypes = [i32]
    lib.oracle_threads.restype = i32
    lib.oracle_init()
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def code_row_bytes(fmt, cols):
    return int(_load().oracle_code_row_bytes(fmt, cols))


def scale_row_bytes(fmt, cols):
    return int(_load().oracle_scale_row_bytes(fmt, cols))


def tables():
    """The decode tables: e2m1[16], e2m3[64], e4m3[256], ue8m0[256], int4[16]."""
    lib = _load()
    t = [np.empty(n, np.float64) for n in (16, 64, 256, 256, 16)]
    lib.oracle_tables(*[a.ctypes.data for a in t[:4]])
    lib.oracle_int4_table(t[4].ctypes.data)
    return {"e2m1": t[0], "e2m3": t[1], "e4m3": t[2], "ue8m0": t[3], "int4": t[4]}


def fp16_value(bits: int) -> float:
    """The IEEE binary16 value of a 16-bit pattern (the int4 format's group scale)."""
    return float(_load().oracle_fp16_value(int(bits)))


def bf16_value(bits: int) -> float:
    return float(_load().oracle_bf16_value(int(bits)))


def bf16_round(v) -> np.ndarray:
    v, pv = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_bf16_round_array(pv, v.size, out.ctypes.data)
    return out


def decode(fmt, rows, cols, codes, scales) -> np.ndarray:
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint8)
    assert codes.size == rows * code_row_bytes(fmt, cols) and scales.size == rows * scale_row_bytes(fmt, cols)
    out = np.empty((rows, cols), np.float64)
    _load().oracle_decode(fmt, rows, cols, pc, ps, out.ctypes.data)
    return out


def gemv(fmt, rows, cols, codes, scales, x_bf16, row_list=None) -> np.ndarray:
    """y[b][i] = W[row_list[i]] . x[b] (all rows when row_list is None)."""
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint8)
    x, px = _c(np.atleast_2d(x_bf16), np.uint16)
    B = x.shape[0]
    assert x.shape[1] == cols
    if row_list is None:
        n, pr = rows, None
    else:
        rl, pr = _c(row_list, np.int64)
        n = rl.size
        assert rl.min() >= 0 and rl.max() < rows
    y = np.empty((B, n), np.float64)
    _load().oracle_gemv(fmt, rows, cols, pc, ps, px, B, pr, n, y.ctypes.data)
    return y


def route(logits, k):
    """(idx int32 [T][k], w float64 [T][k]) in rank order."""
    l, pl = _c(np.atleast_2d(logits), np.float32)
    T, E = l.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = _load().oracle_route(pl, T, E, k, idx.ctypes.data, w.ctypes.data)
    if rc:
        raise ValueError("oracle_route: invalid k=%d for E=%d" % (k, E))
    return idx, w


def set_threads(n: int) -> int:
    """Threads of the oracle's parallel loops (n <= 0: unchanged); returns the
    count in force.  Results do not depend on it."""
    return int(_load().oracle_threads(int(n)))


def silu(z: float) -> float:
    return float(_load().oracle_silu(float(z)))


def ffn(fmt, H, I, ew, x_bf16, out_rows=None, return_h=False):
    """One SwiGLU expert on one token; ew has w13_codes/w13_scales/w2_codes/w2_scales."""
    arrs = [_c(ew[k], np.uint8) for k in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")]
    assert arrs[0][0].size == 2 * I * code_row_bytes(fmt, H)
    assert arrs[2][0].size == H * code_row_bytes(fmt, I)
    x, px = _c(x_bf16, np.uint16)
    assert x.size == H
    if out_rows is None:
        n, pr = H, None
    else:
        rl, pr = _c(out_rows, np.int64)
        n = rl.size
    y = np.empty(n, np.float64)
    h = np.empty(I, np.float64)
    _load().oracle_ffn(fmt, H, I, *[p for _, p in arrs], px, pr, n, h.ctypes.data, y.ctypes.data)
    return (y, h) if return_h else y


def layer(fmt, H, I, E, k, experts, x_bf16, logits, shared=None, shared_inter=0, out_rows=None):
    """The MoE layer for T tokens.

    experts: dict expert index -> dict of its four uint8 arrays (only the
    experts the tokens select are needed).  shared: the shared expert's arrays
    (with shared_inter > 0).  Returns (idx, w, out[T][n_out] float64)."""
    lib = _load()
    x, px = _c(np.atleast_2d(x_bf16), np.uint16)
    l, pl = _c(np.atleast_2d(logits), np.float32)
    T = x.shape[0]
    assert x.shape[1] == H and l.shape == (T, E)
    keep = []
    ptrs = {}
    for name in ("w13_codes", "w13_scales", "w2_codes", "w2_scales"):
        arr = (ctypes.c_void_p * E)()
        for e, ew in experts.items():
            a, p = _c(ew[name], np.uint8)
            keep.append(a)
            arr[e] = p
        ptrs[name] = arr
    sh = [None] * 4
    if shared_inter:
        for i, name in enumerate(("w13_codes", "w13_scales", "w2_codes", "w2_scales")):
            a, p = _c(shared[name], np.uint8)
            keep.append(a)
            sh[i] = p
    if out_rows is None:
        n, pr = H, None
    else:
        rl, pr = _c(out_rows, np.int64)
        n = rl.size
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    out = np.empty((T, n), np.float64)
    rc = lib.oracle_layer(fmt, T, H, I, E, k, ptrs["w13_codes"], ptrs["w13_scales"], ptrs["w2_codes"],
                          ptrs["w2_scales"], shared_inter, sh[0], sh[1], sh[2], sh[3], px, pl, pr, n,
                          idx.ctypes.data, w.ctypes.data, out.ctypes.data)
    if rc == -3:
        raise KeyError("oracle.layer: a selected expert's weights were not supplied")
    if rc:
        raise ValueError("oracle.layer failed: %d" % rc)
    return idx, w, out


def rmsnorm(x_bf16, gamma_bf16, eps):
    """y = x * g / sqrt(mean(x^2) + eps) per token, in double (x [T][H], g [H] bf16 bits)."""
    x, px = _c(np.atleast_2d(x_bf16), np.uint16)
    g, pg = _c(gamma_bf16, np.uint16)
    T, H = x.shape
    assert g.size == H
    y = np.empty((T, H), np.float64)
    _load().oracle_rmsnorm(T, H, px, pg, float(eps), y.ctypes.data)
    return y


def router_logits(x_bf16, wr_bf16):
    """Router scores in double: logits[t][e] = Wr[e] . x[t] (Wr [E][H], x [T][H] bf16 bits)."""
    x, px = _c(np.atleast_2d(x_bf16), np.uint16)
    wr, pw = _c(np.atleast_2d(wr_bf16), np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    assert wr.shape[1] == H
    out = np.empty((T, E), np.float64)
    _load().oracle_router_logits(T, H, E, px, pw, out.ctypes.data)
    return out


def residual_add(r_bf16, y):
    r, pr = _c(r_bf16, np.uint16)
    y, py = _c(y, np.float64)
    assert r.shape == y.shape
    out = np.empty(y.shape, np.float64)
    _load().oracle_residual_add(y.size, pr, py, out.ctypes.data)
    return out


def block(fmt, H, I, E, k, experts, x_bf16, gamma_bf16, wr_bf16, eps, shared=None, shared_inter=0,
          out_rows=None):
    """The whole MoE block for T tokens of the residual stream x:
        xn = bf16(RMSNorm(x))              the activation the experts take
        logits = Wr xn, rounded to fp32    the scores routing ranks
        out = x + MoE(xn, logits)          the residual add
    Returns (idx, w, out double, xn bf16 bits, logits double)."""
    x = np.atleast_2d(np.asarray(x_bf16, np.uint16))
    xn = bf16_round(rmsnorm(x, gamma_bf16, eps))
    lg = router_logits(xn, wr_bf16)
    idx, w, y = layer(fmt, H, I, E, k, experts, xn, lg.astype(np.float32), shared=shared,
                      shared_inter=shared_inter, out_rows=out_rows)
    r = x if out_rows is None else x[:, np.asarray(out_rows)]
    return idx, w, residual_add(np.ascontiguousarray(r), y), xn, lg


def quantize_mx_e4m3(x_bf16):
    """Activations [T][H] (bf16 bits) -> (e4m3 codes uint8 [T][H], UE8M0 scales uint8 [T][H/32])."""
    x, px = _c(np.atleast_2d(x_bf16), np.uint16)
    T, H = x.shape
    assert H % 32 == 0
    codes = np.empty((T, H), np.uint8)
    scales = np.empty((T, H // 32), np.uint8)
    _load().oracle_quantize_mx_e4m3(T, H, px, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def dequantize_mx_e4m3(codes, scales):
    """value(code) * 2^(scale - 127) in double."""
    t = tables()
    c = np.asarray(codes)
    s = np.repeat(np.asarray(scales).astype(np.float64) - 127.0, 32, axis=-1)
    return t["e4m3"][c] * np.exp2(s)


def use_library(path=None):
    """Point this module at another build of oracle.c (the mutation tests build
    deliberately broken copies); None restores the normal build."""
    global _lib, _LIB_PATH
    _lib = None
    _LIB_PATH = path or os.path.join(_HERE, "_build", "liboracle.so")
    return _load()
