"""Python binding of the block-scaled low-bit MoE library (include/moeq.h).

Argument marshalling only: torch tensors become device pointers and the
current HIP stream; every step of the computation runs in the HIP kernels of
libmoeq.so.  There is no fallback: if the library is not built, or a tensor is
not on the GPU, the call raises.

Functions carry the C names: moe_route_topk, moe_layer_workspace_bytes,
moe_expert_ffn_q, moe_layer_decode, moe_layer_decode_noalloc, dense_gemv_q,
moe_rmsnorm, moe_router_topk_scores, moe_block_workspace_bytes, moe_block_decode,
moe_quantize_mx_e4m3,
moe_workspace_status, moe_last_error, moe_version.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libmoeq.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_EKERNEL = 0, -1, -2, -3, -4, -5
MOE_FMT_E2M1_E4M3_B16, MOE_FMT_E2M3_UE8M0_B128 = 1, 2
MOE_FMT_E2M1_UE8M0_B32, MOE_FMT_INT4_F16_B64, MOE_FMT_E2M3_E4M3_B16 = 3, 4, 5
FORMATS = (1, 2, 3, 4, 5)
MOE_OUT_F32 = 1
MOE_ACT_MXFP8 = 1 << 27
MOE_DECODER_LUT = 1 << 28
MOE_DECODER_HW = 1 << 29
MOE_DEBUG_SPIN_LIMIT = 1 << 30
MAX_DECODE_TOKENS = 16

_lib = None


class MoeError(RuntimeError):
    def __init__(self, code, message):
        super().__init__("moeq error %d: %s" % (code, message))
        self.code = code


class moe_qmat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class moe_layer(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("w13_codes", ctypes.c_void_p), ("w13_scales", ctypes.c_void_p),
                ("w2_codes", ctypes.c_void_p), ("w2_scales", ctypes.c_void_p),
                ("sh13_codes", ctypes.c_void_p), ("sh13_scales", ctypes.c_void_p),
                ("sh2_codes", ctypes.c_void_p), ("sh2_scales", ctypes.c_void_p)]


class moe_block(ctypes.Structure):
    _fields_ = [("layer", moe_layer), ("norm_gamma", ctypes.c_void_p), ("router_w", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("reserved", ctypes.c_int32)]


def load_library(path=None):
    """Load libmoeq.so (built in-tree by build.py).  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError("libmoeq.so is not built (%s); run __graft_entry__.build()" % p)
    lib = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moe_route_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.moe_layer_workspace_bytes.argtypes = [ctypes.POINTER(moe_layer), i32]
    lib.moe_layer_workspace_bytes.restype = sz
    lib.moe_expert_ffn_q.argtypes = [ctypes.POINTER(moe_layer), i32, vp, i32, vp, i32, vp, sz, vp]
    lib.moe_layer_decode.argtypes = [ctypes.POINTER(moe_layer), vp, vp, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.moe_layer_decode_noalloc.argtypes = [ctypes.POINTER(moe_layer), vp, vp, i32, vp, vp, vp, i32, vp]
    lib.dense_gemv_q.argtypes = [ctypes.POINTER(moe_qmat), vp, i32, vp, i32, vp]
    lib.moe_rmsnorm.argtypes = [vp, vp, i32, i32, ctypes.c_float, vp, i32, vp]
    lib.moe_quantize_mx_e4m3.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.moe_router_topk_scores.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_block_workspace_bytes.argtypes = [ctypes.POINTER(moe_block), i32]
    lib.moe_block_workspace_bytes.restype = sz
    lib.moe_block_decode.argtypes = [ctypes.POINTER(moe_block), vp, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.moe_workspace_status.argtypes = [vp, sz, vp]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_version.restype = i32
    for f in ("moe_route_topk", "moe_expert_ffn_q", "moe_layer_decode", "moe_layer_decode_noalloc", "dense_gemv_q",
              "moe_workspace_status", "moe_rmsnorm", "moe_router_topk_scores", "moe_block_decode",
              "moe_quantize_mx_e4m3"):
        getattr(lib, f).restype = i32
    if path is None:
        _lib = lib
    return lib


def moe_last_error():
    return load_library().moe_last_error().decode()


def moe_version():
    return load_library().moe_version()


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, moe_last_error())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtypes):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU (the library has no CPU path)" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)


def _shape(t, name, shape):
    """Refuse a tensor whose shape is not `shape` (the kernels would read or
    write past its allocation)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _numel(t, name, n):
    if t.numel() != n:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), n))


def code_row_bytes(fmt, cols):
    """Bytes of one row of codes of `cols` weights (four- or six-bit codes)."""
    return cols * 3 // 4 if fmt in (MOE_FMT_E2M3_UE8M0_B128, MOE_FMT_E2M3_E4M3_B16) else cols // 2


def scale_row_bytes(fmt, cols):
    """Scale bytes of one row of `cols` weights."""
    return {1: cols // 16, 2: cols // 128, 3: cols // 32, 4: 2 * (cols // 64), 5: cols // 16}[fmt]


class QMat:
    """A block-scaled matrix [rows][cols] on the GPU (codes and scales uint8)."""

    def __init__(self, fmt, rows, cols, codes, scales):
        self.fmt, self.rows, self.cols = fmt, rows, cols
        self.codes, self.scales = codes, scales
        _numel(codes, "codes", rows * code_row_bytes(fmt, cols))
        _numel(scales, "scales", rows * scale_row_bytes(fmt, cols))
        self.c = moe_qmat(fmt, rows, cols, 0, _dev(codes, "codes", _U8).value, _dev(scales, "scales", _U8).value)


class Layer:
    """One MoE layer's weights on the GPU, as the moe_layer descriptor sees them.

    w13_codes [E][2I][H*bits/8], w13_scales [E][2I][H/block], w2_codes [E][H][I*bits/8],
    w2_scales [E][H][I/block]; optional shared_* arrays of the shared expert."""

    def __init__(self, fmt, hidden, inter, n_experts, top_k, w13_codes, w13_scales, w2_codes, w2_scales,
                 shared_inter=0, shared=None):
        self.fmt, self.hidden, self.inter, self.n_experts, self.top_k = fmt, hidden, inter, n_experts, top_k
        self.shared_inter = shared_inter
        self.tensors = [w13_codes, w13_scales, w2_codes, w2_scales]
        H, I, E = hidden, inter, n_experts
        _numel(w13_codes, "w13_codes", E * 2 * I * code_row_bytes(fmt, H))
        _numel(w13_scales, "w13_scales", E * 2 * I * scale_row_bytes(fmt, H))
        _numel(w2_codes, "w2_codes", E * H * code_row_bytes(fmt, I))
        _numel(w2_scales, "w2_scales", E * H * scale_row_bytes(fmt, I))
        sh = [None] * 4
        if shared_inter:
            names = ("w13_codes", "w13_scales", "w2_codes", "w2_scales")
            Is = shared_inter
            _numel(shared["w13_codes"], "shared w13_codes", 2 * Is * code_row_bytes(fmt, H))
            _numel(shared["w13_scales"], "shared w13_scales", 2 * Is * scale_row_bytes(fmt, H))
            _numel(shared["w2_codes"], "shared w2_codes", H * code_row_bytes(fmt, Is))
            _numel(shared["w2_scales"], "shared w2_scales", H * scale_row_bytes(fmt, Is))
            sh = [_dev(shared[n], "shared " + n, _U8).value for n in names]
            self.tensors += [shared[n] for n in names]
        self.c = moe_layer(fmt, hidden, inter, n_experts, top_k, shared_inter,
                           _dev(w13_codes, "w13_codes", _U8).value, _dev(w13_scales, "w13_scales", _U8).value,
                           _dev(w2_codes, "w2_codes", _U8).value, _dev(w2_scales, "w2_scales", _U8).value,
                           *sh)

    def with_top_k(self, k):
        """A descriptor of the same weights with another top-k."""
        other = object.__new__(Layer)
        other.__dict__.update(self.__dict__)
        c = moe_layer()
        ctypes.pointer(c)[0] = self.c
        c.top_k = k
        other.c, other.top_k = c, k
        return other


def moe_route_topk(logits, k, idx=None, w=None):
    """logits fp32 [T][E] -> (idx int32 [T][k], w fp32 [T][k])."""
    T, E = logits.shape
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _shape(idx, "idx", (T, k))
    _shape(w, "w", (T, k))
    _check(load_library().moe_route_topk(_dev(logits, "logits", (torch.float32,)), T, E, k,
                                         _dev(idx, "idx", (torch.int32,)), _dev(w, "w", (torch.float32,)),
                                         _stream()))
    return idx, w


def moe_layer_workspace_bytes(layer, T):
    n = load_library().moe_layer_workspace_bytes(ctypes.byref(layer.c), T)
    if not n:
        raise MoeError(MOE_EINVAL, moe_last_error())
    return n


def workspace(layer, T, device=None):
    """A zeroed workspace of the size the call needs (torch memory)."""
    return torch.zeros(moe_layer_workspace_bytes(layer, T), dtype=torch.uint8, device=device or "cuda")


def _out(x, rows, cols, flags, out):
    if out is not None:
        return out
    dt = torch.float32 if flags & MOE_OUT_F32 else torch.bfloat16
    return torch.empty((rows, cols), dtype=dt, device=x.device)


def moe_expert_ffn_q(layer, expert, x, y=None, flags=0, ws=None):
    """One expert's SwiGLU FFN on the M rows of x (bf16 [M][H]); expert -1 = shared."""
    M = x.shape[0]
    _shape(x, "x", (M, layer.hidden))
    y = _out(x, M, layer.hidden, flags, y)
    _shape(y, "y", (M, layer.hidden))
    ws = workspace(layer, M, x.device) if ws is None else ws
    _check(load_library().moe_expert_ffn_q(ctypes.byref(layer.c), expert, _dev(x, "x", _BF16), M,
                                           _dev(y, "y", (torch.bfloat16, torch.float32)), flags,
                                           _dev(ws, "ws", _U8), ws.numel(), _stream()))
    return y


def moe_layer_decode(layer, x, logits, out=None, idx_out=None, w_out=None, flags=0, ws=None):
    """The MoE layer for the T rows of x: returns out [T][H] (bf16, or fp32 with MOE_OUT_F32)."""
    T = x.shape[0]
    _shape(x, "x", (T, layer.hidden))
    _shape(logits, "logits", (T, layer.n_experts))
    out = _out(x, T, layer.hidden, flags, out)
    _shape(out, "out", (T, layer.hidden))
    if idx_out is not None:
        _shape(idx_out, "idx_out", (T, layer.top_k))
    if w_out is not None:
        _shape(w_out, "w_out", (T, layer.top_k))
    ws = workspace(layer, T, x.device) if ws is None else ws
    pi = _dev(idx_out, "idx_out", (torch.int32,)) if idx_out is not None else None
    pw = _dev(w_out, "w_out", (torch.float32,)) if w_out is not None else None
    _check(load_library().moe_layer_decode(ctypes.byref(layer.c), _dev(x, "x", _BF16),
                                           _dev(logits, "logits", (torch.float32,)), T,
                                           _dev(out, "out", (torch.bfloat16, torch.float32)), pi, pw, flags,
                                           _dev(ws, "ws", _U8), ws.numel(), _stream()))
    return out


def moe_layer_decode_noalloc(layer, x, logits, out, idx_out=None, w_out=None, flags=0):
    """moe_layer_decode on the library's static workspace (T <= 16): the caller
    passes every output, nothing is allocated."""
    T = x.shape[0]
    _shape(x, "x", (T, layer.hidden))
    _shape(logits, "logits", (T, layer.n_experts))
    _shape(out, "out", (T, layer.hidden))
    if idx_out is not None:
        _shape(idx_out, "idx_out", (T, layer.top_k))
    if w_out is not None:
        _shape(w_out, "w_out", (T, layer.top_k))
    pi = _dev(idx_out, "idx_out", (torch.int32,)) if idx_out is not None else None
    pw = _dev(w_out, "w_out", (torch.float32,)) if w_out is not None else None
    _check(load_library().moe_layer_decode_noalloc(ctypes.byref(layer.c), _dev(x, "x", _BF16),
                                                   _dev(logits, "logits", (torch.float32,)), T,
                                                   _dev(out, "out", (torch.bfloat16, torch.float32)), pi, pw, flags,
                                                   _stream()))
    return out


def dense_gemv_q(W, x, y=None, flags=0):
    """y [B][rows] = W x[b] for x bf16 [B][cols]."""
    B = x.shape[0]
    _shape(x, "x", (B, W.cols))
    y = _out(x, B, W.rows, flags, y)
    _shape(y, "y", (B, W.rows))
    _check(load_library().dense_gemv_q(ctypes.byref(W.c), _dev(x, "x", _BF16), B,
                                       _dev(y, "y", (torch.bfloat16, torch.float32)), flags, _stream()))
    return y


def moe_rmsnorm(x, gamma, eps, y=None, flags=0):
    """RMSNorm of the T rows of x (bf16 [T][H]) with gains gamma (bf16 [H])."""
    T, H = x.shape
    _shape(gamma, "gamma", (H,))
    y = _out(x, T, H, flags, y)
    _shape(y, "y", (T, H))
    _check(load_library().moe_rmsnorm(_dev(x, "x", _BF16), _dev(gamma, "gamma", _BF16), T, H, float(eps),
                                      _dev(y, "y", (torch.bfloat16, torch.float32)), flags, _stream()))
    return y


def moe_quantize_mx_e4m3(x, codes=None, scales=None):
    """x bf16 [T][H] -> (MX e4m3 codes uint8 [T][H], UE8M0 scales uint8 [T][H/32])."""
    T, H = x.shape
    codes = torch.empty((T, H), dtype=torch.uint8, device=x.device) if codes is None else codes
    scales = torch.empty((T, H // 32), dtype=torch.uint8, device=x.device) if scales is None else scales
    _shape(codes, "codes", (T, H))
    _shape(scales, "scales", (T, H // 32))
    _check(load_library().moe_quantize_mx_e4m3(_dev(x, "x", _BF16), T, H, _dev(codes, "codes", _U8),
                                               _dev(scales, "scales", _U8), _stream()))
    return codes, scales


def moe_router_topk_scores(x, router_w, k, logits=None, idx=None, w=None, ws=None):
    """Router scores (fp32 [T][E]) of x (bf16 [T][H]) with router_w (bf16 [E][H]) and their top-k."""
    T, H = x.shape
    E = router_w.shape[0]
    _shape(router_w, "router_w", (E, H))
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if logits is None else logits
    idx = torch.empty((T, k), dtype=torch.int32, device=dev) if idx is None else idx
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    ws = torch.zeros(256, dtype=torch.uint8, device=dev) if ws is None else ws
    _shape(logits, "logits", (T, E))
    _shape(idx, "idx", (T, k))
    _shape(w, "w", (T, k))
    _check(load_library().moe_router_topk_scores(_dev(x, "x", _BF16), _dev(router_w, "router_w", _BF16), T, H, E, k,
                                                 _dev(logits, "logits", (torch.float32,)),
                                                 _dev(idx, "idx", (torch.int32,)), _dev(w, "w", (torch.float32,)),
                                                 _dev(ws, "ws", _U8), ws.numel(), _stream()))
    return logits, idx, w


class Block:
    """A MoE block on the GPU: a Layer plus RMSNorm gains (bf16 [H]) and router
    weights (bf16 [E][H])."""

    def __init__(self, layer, norm_gamma, router_w, norm_eps=1e-6):
        _shape(norm_gamma, "norm_gamma", (layer.hidden,))
        _shape(router_w, "router_w", (layer.n_experts, layer.hidden))
        self.layer, self.norm_gamma, self.router_w, self.norm_eps = layer, norm_gamma, router_w, norm_eps
        self.hidden, self.n_experts, self.top_k = layer.hidden, layer.n_experts, layer.top_k
        self.c = moe_block(layer.c, _dev(norm_gamma, "norm_gamma", _BF16).value,
                           _dev(router_w, "router_w", _BF16).value, float(norm_eps), 0)


def moe_block_workspace_bytes(block, T):
    n = load_library().moe_block_workspace_bytes(ctypes.byref(block.c), T)
    if not n:
        raise MoeError(MOE_EINVAL, moe_last_error())
    return n


def block_workspace(block, T, device=None):
    return torch.zeros(moe_block_workspace_bytes(block, T), dtype=torch.uint8, device=device or "cuda")


def moe_block_decode(block, x, out=None, idx_out=None, w_out=None, flags=0, ws=None):
    """The MoE block on the residual stream x (bf16 [T][H]): x + layer(RMSNorm(x))."""
    T = x.shape[0]
    _shape(x, "x", (T, block.hidden))
    out = _out(x, T, block.hidden, flags, out)
    _shape(out, "out", (T, block.hidden))
    if idx_out is not None:
        _shape(idx_out, "idx_out", (T, block.top_k))
    if w_out is not None:
        _shape(w_out, "w_out", (T, block.top_k))
    ws = block_workspace(block, T, x.device) if ws is None else ws
    pi = _dev(idx_out, "idx_out", (torch.int32,)) if idx_out is not None else None
    pw = _dev(w_out, "w_out", (torch.float32,)) if w_out is not None else None
    _check(load_library().moe_block_decode(ctypes.byref(block.c), _dev(x, "x", _BF16), T,
                                           _dev(out, "out", (torch.bfloat16, torch.float32)), pi, pw, flags,
                                           _dev(ws, "ws", _U8), ws.numel(), _stream()))
    return out


def moe_workspace_status(ws):
    """MOE_OK, or raises MoeError(MOE_EKERNEL) when a kernel's bounded wait expired."""
    _check(load_library().moe_workspace_status(_dev(ws, "ws", _U8), ws.numel(), _stream()))
    return MOE_OK
