"""Seeded synthetic inputs shared by the GPU library's tests/bench and the oracle.

Holds no part of the method's arithmetic (see gen.c).  Every tensor is drawn
from its own counter-based stream (seed, stream id), so one expert, one row or
one call's logits can be regenerated alone.

Layouts produced (row-major, each row contiguous, planar codes and scales):
  e2m1  codes [rows][cols/2]   (element j in byte j>>1, low nibble first)
        scales [rows][cols/16] (fp8 e4m3, one per 16 consecutive weights)
  e2m3  codes [rows][3*cols/4] (element j in bits [6j, 6j+6) of the row's
        little-endian bit string)
        scales [rows][cols/128] (UE8M0, one per 128 consecutive weights)
  MXFP4 (e2m1 + UE8M0/32) and int4 (+ fp16/64) codes as e2m1; e2m3 + e4m3/16
        codes as e2m3; scales [rows][cols/32] (one byte), [rows][cols/64][2]
        (fp16, low byte first), [rows][cols/16] (e4m3).
Uniform random code bytes make every 4-bit or 6-bit code uniform.
"""
import ctypes
import os

import numpy as np

from . import configs
from .configs import FMT_E2M1, FMT_E2M3, FMT_E2M3_E4M3, FMT_INT4_F16, FMT_MXFP4, FORMATS, GemvConfig, MoEConfig

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "libsynth.so")
_lib = None

# stream kinds
K_W13_CODES, K_W13_SCALES, K_W2_CODES, K_W2_SCALES = 1, 2, 3, 4
K_X, K_LOGITS = 5, 6
K_W_CODES, K_W_SCALES = 7, 8
K_GAMMA, K_ROUTER = 9, 10


def stream_id(kind: int, sub: int) -> int:
    return (kind << 32) | int(sub)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, vp, d = ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double
    lib.synth_word.argtypes = [u64, u64, u64]
    lib.synth_word.restype = u64
    lib.synth_bytes.argtypes = [u64, u64, u64, u64, vp]
    lib.synth_e4m3_loguniform.argtypes = [u64, u64, u64, u64, d, d, vp]
    lib.synth_ue8m0_uniform.argtypes = [u64, u64, u64, u64, ctypes.c_int, ctypes.c_int, vp]
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, d, vp]
    lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, d, vp]
    lib.synth_normal_bf16_mean.argtypes = [u64, u64, u64, u64, d, d, vp]
    lib.synth_bf16_from_double.argtypes = [d]
    lib.synth_bf16_from_double.restype = ctypes.c_uint16
    lib.synth_fp16_loguniform.argtypes = [u64, u64, u64, u64, d, d, vp]
    lib.synth_fp16_encode.argtypes = [d]
    lib.synth_fp16_encode.restype = ctypes.c_uint16
    lib.synth_e4m3_encode.argtypes = [d]
    lib.synth_e4m3_encode.restype = ctypes.c_uint8
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- primitives
def random_bytes(seed, stream, n, offset=0, out=None):
    out = np.empty(n, np.uint8) if out is None else out
    _load().synth_bytes(seed, stream, offset, n, _ptr(out))
    return out


def e4m3_loguniform(seed, stream, n, lo, hi, offset=0, out=None):
    out = np.empty(n, np.uint8) if out is None else out
    _load().synth_e4m3_loguniform(seed, stream, offset, n, lo, hi, _ptr(out))
    return out


def ue8m0_uniform(seed, stream, n, lo, hi, offset=0, out=None):
    out = np.empty(n, np.uint8) if out is None else out
    _load().synth_ue8m0_uniform(seed, stream, offset, n, lo, hi, _ptr(out))
    return out


def fp16_loguniform(seed, stream, n, lo, hi, offset=0, out=None):
    """n fp16 scales (2n bytes, low byte first) of values 2^U[lo, hi)."""
    out = np.empty(2 * n, np.uint8) if out is None else out
    _load().synth_fp16_loguniform(seed, stream, offset, n, lo, hi, _ptr(out))
    return out


def fp16_encode(v: float) -> int:
    return int(_load().synth_fp16_encode(float(v)))


def normal_bf16(seed, stream, n, sigma=1.0, offset=0, out=None):
    out = np.empty(n, np.uint16) if out is None else out
    _load().synth_normal_bf16(seed, stream, offset, n, sigma, _ptr(out))
    return out


def normal_f32(seed, stream, n, sigma=1.0, offset=0, out=None):
    out = np.empty(n, np.float32) if out is None else out
    _load().synth_normal_f32(seed, stream, offset, n, sigma, _ptr(out))
    return out


def bf16_from_double(v: float) -> int:
    return int(_load().synth_bf16_from_double(float(v)))


def e4m3_encode(v: float) -> int:
    return int(_load().synth_e4m3_encode(float(v)))


# ---------------------------------------------------------------- layouts
def code_row_bytes(fmt: int, cols: int) -> int:
    return cols // 2 if fmt in (FMT_E2M1, FMT_MXFP4, FMT_INT4_F16) else cols * 3 // 4


def scale_row_bytes(fmt: int, cols: int) -> int:
    return {FMT_E2M1: cols // 16, FMT_E2M3: cols // 128, FMT_MXFP4: cols // 32, FMT_INT4_F16: cols // 32,
            FMT_E2M3_E4M3: cols // 16}[fmt]


def fill_matrix(fmt, rows, cols, seed, codes_stream, scales_stream, codes_out, scales_out,
                scale_log2=(-6.0, -2.0), ue8m0_exp=(-8, -3), fp16_log2=(-8.0, -4.0)):
    """Draw one block-scaled matrix [rows][cols] into flat uint8 views."""
    nc = rows * code_row_bytes(fmt, cols)
    ns = rows * scale_row_bytes(fmt, cols)
    assert codes_out.size == nc and scales_out.size == ns
    random_bytes(seed, codes_stream, nc, out=codes_out)
    if fmt in (FMT_E2M1, FMT_E2M3_E4M3):
        e4m3_loguniform(seed, scales_stream, ns, scale_log2[0], scale_log2[1], out=scales_out)
    elif fmt == FMT_INT4_F16:
        fp16_loguniform(seed, scales_stream, ns // 2, fp16_log2[0], fp16_log2[1], out=scales_out)
    else:
        ue8m0_uniform(seed, scales_stream, ns, ue8m0_exp[0], ue8m0_exp[1], out=scales_out)


def matrix(fmt, rows, cols, seed, codes_stream, scales_stream, **kw):
    c = np.empty((rows, code_row_bytes(fmt, cols)), np.uint8)
    s = np.empty((rows, scale_row_bytes(fmt, cols)), np.uint8)
    fill_matrix(fmt, rows, cols, seed, codes_stream, scales_stream, c.reshape(-1), s.reshape(-1), **kw)
    return c, s


# ---------------------------------------------------------------- MoE layers
def expert_shapes(cfg: MoEConfig, inter=None):
    I = cfg.inter if inter is None else inter
    H, f = cfg.hidden, cfg.fmt
    return {
        "w13_codes": (2 * I, code_row_bytes(f, H)), "w13_scales": (2 * I, scale_row_bytes(f, H)),
        "w2_codes": (H, code_row_bytes(f, I)), "w2_scales": (H, scale_row_bytes(f, I)),
    }


def fill_expert(cfg: MoEConfig, e: int, out: dict):
    """Expert e's four arrays (e == cfg.experts is the shared expert) into `out`
    (dict of flat or shaped uint8 arrays with the sizes of expert_shapes)."""
    I = cfg.shared_inter if e == cfg.experts else cfg.inter
    kw = dict(scale_log2=cfg.scale_log2, ue8m0_exp=cfg.ue8m0_exp, fp16_log2=cfg.fp16_log2)
    fill_matrix(cfg.fmt, 2 * I, cfg.hidden, cfg.seed, stream_id(K_W13_CODES, e), stream_id(K_W13_SCALES, e),
                out["w13_codes"].reshape(-1), out["w13_scales"].reshape(-1), **kw)
    fill_matrix(cfg.fmt, cfg.hidden, I, cfg.seed, stream_id(K_W2_CODES, e), stream_id(K_W2_SCALES, e),
                out["w2_codes"].reshape(-1), out["w2_scales"].reshape(-1), **kw)


def expert_weights(cfg: MoEConfig, e: int) -> dict:
    I = cfg.shared_inter if e == cfg.experts else cfg.inter
    out = {k: np.empty(s, np.uint8) for k, s in expert_shapes(cfg, I).items()}
    fill_expert(cfg, e, out)
    return out


def layer_weights(cfg: MoEConfig) -> dict:
    """Whole layer on the host: routed arrays [E][...] plus the shared expert's."""
    shp = expert_shapes(cfg)
    out = {k: np.empty((cfg.experts,) + s, np.uint8) for k, s in shp.items()}
    for e in range(cfg.experts):
        fill_expert(cfg, e, {k: out[k][e] for k in shp})
    if cfg.shared_inter:
        sh = expert_weights(cfg, cfg.experts)
        for k in shp:
            out["shared_" + k] = sh[k]
    return out


def hidden_states(cfg, tokens=None, sub=0) -> np.ndarray:
    T = cfg.tokens if tokens is None else tokens
    return normal_bf16(cfg.seed, stream_id(K_X, sub), T * cfg.hidden, cfg.x_sigma).reshape(T, cfg.hidden)


def router_logits(cfg, tokens=None, sub=0) -> np.ndarray:
    T = cfg.tokens if tokens is None else tokens
    return normal_f32(cfg.seed, stream_id(K_LOGITS, sub), T * cfg.experts, cfg.logit_sigma).reshape(T, cfg.experts)


def norm_gamma(cfg) -> np.ndarray:
    """RMSNorm gains, bf16 bits [H]: 1 + N(0, gamma_sigma)."""
    out = np.empty(cfg.hidden, np.uint16)
    _load().synth_normal_bf16_mean(cfg.seed, stream_id(K_GAMMA, 0), 0, cfg.hidden, 1.0, cfg.gamma_sigma, _ptr(out))
    return out


def router_weights(cfg) -> np.ndarray:
    """Router weights, bf16 bits [E][H]: N(0, logit_sigma / sqrt(H))."""
    sigma = cfg.logit_sigma / float(np.sqrt(cfg.hidden))
    return normal_bf16(cfg.seed, stream_id(K_ROUTER, 0), cfg.experts * cfg.hidden, sigma).reshape(cfg.experts, cfg.hidden)


# ---------------------------------------------------------------- dense GEMV
def gemv_weights(cfg: GemvConfig):
    return matrix(cfg.fmt, cfg.rows, cfg.cols, cfg.seed, stream_id(K_W_CODES, 0), stream_id(K_W_SCALES, 0),
                  scale_log2=cfg.scale_log2, ue8m0_exp=cfg.ue8m0_exp, fp16_log2=cfg.fp16_log2)


def gemv_x(cfg: GemvConfig, batch: int, sub=0) -> np.ndarray:
    return normal_bf16(cfg.seed, stream_id(K_X, sub), batch * cfg.cols, cfg.x_sigma).reshape(batch, cfg.cols)


__all__ = ["configs", "FMT_E2M1", "FMT_E2M3", "FMT_MXFP4", "FMT_INT4_F16", "FMT_E2M3_E4M3", "FORMATS", "MoEConfig",
           "GemvConfig"]
