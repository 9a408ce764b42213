"""The C-ABI library on the CPU: it loads, exports every entry point the header
declares, and rejects bad arguments before touching the GPU (every call here
fails validation, so no HIP work is attempted)."""
import ctypes
import os
import re

import pytest

import block_scaled_bit_moe_amd as moeq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moeq.h")
FAKE = 0x10000          # an aligned non-null address; never dereferenced by validation
FAKE2 = 0x20000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+|dense_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return moeq.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) >= {"moe_route_topk", "moe_layer_workspace_bytes", "moe_expert_ffn_q", "moe_layer_decode",
                          "dense_gemv_q", "moe_last_error", "moe_version", "moe_workspace_status",
                          "moe_layer_decode_noalloc", "moe_rmsnorm", "moe_router_topk_scores",
                          "moe_block_workspace_bytes", "moe_block_decode", "moe_quantize_mx_e4m3"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.moe_version() >= 100


def _err(lib):
    return lib.moe_last_error().decode()


def _ws_bytes(lib, L, T):
    """moe_layer_workspace_bytes: the size, or 0 when the arguments break a rule."""
    return lib.moe_layer_workspace_bytes(ctypes.byref(L), T)


def _layer(**kw):
    d = dict(fmt=1, hidden=256, inter=512, n_experts=8, top_k=2, shared_inter=0,
             w13_codes=FAKE, w13_scales=FAKE, w2_codes=FAKE, w2_scales=FAKE)
    d.update(kw)
    L = moeq.moe_layer()
    for k, v in d.items():
        setattr(L, k, v)
    return L


def test_route_validation(lib):
    assert lib.moe_route_topk(None, 1, 8, 2, FAKE, FAKE, None) == moeq.MOE_EINVAL
    assert "logits" in _err(lib)
    assert lib.moe_route_topk(FAKE + 4, 1, 8, 2, FAKE, FAKE, None) == moeq.MOE_EINVAL
    assert "aligned" in _err(lib)
    assert lib.moe_route_topk(FAKE, 0, 8, 2, FAKE, FAKE, None) == moeq.MOE_EINVAL
    assert lib.moe_route_topk(FAKE, 1, 8, 9, FAKE, FAKE, None) == moeq.MOE_EINVAL
    assert "k=9" in _err(lib)
    assert lib.moe_route_topk(FAKE, 1, 1025, 2, FAKE, FAKE, None) == moeq.MOE_EINVAL
    assert lib.moe_route_topk(FAKE, 1, 64, 33, FAKE, FAKE, None) == moeq.MOE_EINVAL


@pytest.mark.parametrize("field,value,needle", [
    ("fmt", 6, "fmt"), ("fmt", 0, "fmt"), ("hidden", 48, "hidden"), ("inter", 0, "inter"), ("n_experts", 0, "n_experts"),
    ("top_k", 9, "top_k"), ("top_k", 0, "top_k"), ("shared_inter", -32, "shared_inter"),
    ("w13_codes", 0, "w13_codes"), ("w2_scales", FAKE + 8, "w2_scales"), ("shared_inter", 48, "shared_inter"),
])
def test_layer_validation(lib, field, value, needle):
    L = _layer(**{field: value})
    assert _ws_bytes(lib, L, 1) == 0 and needle in _err(lib)


def test_e2m3_dims_must_be_whole_blocks(lib):
    L = _layer(fmt=2, hidden=256, inter=512 + 32)
    assert _ws_bytes(lib, L, 1) == 0
    assert "multiple of 128" in _err(lib)


def test_shared_pointers_required(lib):
    L = _layer(shared_inter=512)
    assert _ws_bytes(lib, L, 1) == 0
    assert "sh13_codes" in _err(lib)


def test_workspace_bytes_and_checks(lib):
    L = _layer()
    need = _ws_bytes(lib, L, 1)
    assert need > 16384 and _err(lib) == ""
    assert _ws_bytes(lib, L, 0) == 0 and "T=0" in _err(lib)
    assert _ws_bytes(lib, L, 65537) == 0
    assert lib.moe_layer_workspace_bytes(None, 1) == 0 and "NULL" in _err(lib)
    # too small, misaligned, NULL: workspace errors, nothing launched
    assert lib.moe_layer_decode(ctypes.byref(L), FAKE, FAKE, 1, FAKE, None, None, 0, FAKE2, need - 1,
                                None) == moeq.MOE_EWORKSPACE
    assert lib.moe_layer_decode(ctypes.byref(L), FAKE, FAKE, 1, FAKE, None, None, 0, FAKE2 + 16, need,
                                None) == moeq.MOE_EWORKSPACE
    assert lib.moe_layer_decode(ctypes.byref(L), FAKE, FAKE, 1, FAKE, None, None, 0, None, need,
                                None) == moeq.MOE_EWORKSPACE
    assert lib.moe_layer_decode(ctypes.byref(L), FAKE, None, 1, FAKE, None, None, 0, FAKE2, need,
                                None) == moeq.MOE_EINVAL
    assert lib.moe_layer_decode(ctypes.byref(L), FAKE, FAKE, 1, FAKE, FAKE + 4, None, 0, FAKE2, need,
                                None) == moeq.MOE_EINVAL
    assert lib.moe_layer_decode(ctypes.byref(L), FAKE, FAKE, 0, FAKE, None, None, 0, FAKE2, need,
                                None) == moeq.MOE_EINVAL


def test_many_token_workspace(lib):
    """T > 16 takes the many-token path: its workspace grows with the chunk
    (at most 2,048 tokens) and a smaller workspace is refused."""
    L = _layer()
    sizes = {}
    for T in (16, 17, 2048, 2049, 65536):
        sizes[T] = _ws_bytes(lib, L, T)
        assert sizes[T] > 0
    assert sizes[17] < sizes[2048] == sizes[2049] == sizes[65536]
    H, I, k = L.hidden, max(L.inter, L.shared_inter), L.top_k
    assert sizes[2048] >= 2048 * (k + 1) * (H * 4 + I * 4)      # fp32 partials + h pair per (token, expert)
    assert lib.moe_layer_decode(ctypes.byref(L), FAKE, FAKE, 17, FAKE, None, None, 0, FAKE2, sizes[17] - 1,
                                None) == moeq.MOE_EWORKSPACE
    assert "needs" in _err(lib)


def test_expert_ffn_validation(lib):
    L = _layer()
    n = _ws_bytes(lib, L, 1)
    assert lib.moe_expert_ffn_q(ctypes.byref(L), 8, FAKE, 1, FAKE, 0, FAKE2, n, None) == moeq.MOE_EINVAL
    assert lib.moe_expert_ffn_q(ctypes.byref(L), -1, FAKE, 1, FAKE, 0, FAKE2, n, None) == moeq.MOE_EINVAL
    assert "shared" in _err(lib)
    assert lib.moe_expert_ffn_q(ctypes.byref(L), 0, FAKE, 0, FAKE, 0, FAKE2, n, None) == moeq.MOE_EINVAL


def test_gemv_validation(lib):
    W = moeq.moe_qmat(2, 100, 5120, 0, FAKE, FAKE)
    assert lib.dense_gemv_q(ctypes.byref(W), FAKE, 0, FAKE, 0, None) == moeq.MOE_EINVAL
    assert lib.dense_gemv_q(ctypes.byref(W), FAKE, 9, FAKE, 0, None) == moeq.MOE_EINVAL
    W.cols = 5000
    assert lib.dense_gemv_q(ctypes.byref(W), FAKE, 1, FAKE, 0, None) == moeq.MOE_EINVAL
    W.cols, W.reserved = 5120, 1
    assert lib.dense_gemv_q(ctypes.byref(W), FAKE, 1, FAKE, 0, None) == moeq.MOE_EINVAL
    W.reserved, W.fmt = 0, 0
    assert lib.dense_gemv_q(ctypes.byref(W), FAKE, 1, FAKE, 0, None) == moeq.MOE_EINVAL
    W.fmt, W.codes = 2, 0
    assert lib.dense_gemv_q(ctypes.byref(W), FAKE, 1, FAKE, 0, None) == moeq.MOE_EINVAL
    assert lib.dense_gemv_q(None, FAKE, 1, FAKE, 0, None) == moeq.MOE_EINVAL


def test_status_validation(lib):
    assert lib.moe_workspace_status(None, 1 << 20, None) == moeq.MOE_EWORKSPACE
    assert lib.moe_workspace_status(FAKE, 100, None) == moeq.MOE_EWORKSPACE


def test_binding_refuses_cpu_tensors():
    import torch
    logits = torch.zeros(1, 8)
    with pytest.raises(ValueError, match="GPU"):
        moeq.moe_route_topk(logits, 2)


def test_block_steps_validation(lib):
    """RMSNorm, router scores + top-k and the block refuse bad arguments before
    anything is enqueued."""
    assert lib.moe_rmsnorm(FAKE, FAKE, 1, 48, ctypes.c_float(1e-6), FAKE, 0, None) == moeq.MOE_EINVAL
    assert "H=48" in _err(lib)
    assert lib.moe_rmsnorm(FAKE, FAKE, 0, 64, ctypes.c_float(1e-6), FAKE, 0, None) == moeq.MOE_EINVAL
    assert lib.moe_rmsnorm(FAKE, FAKE, 1, 64, ctypes.c_float(-1.0), FAKE, 0, None) == moeq.MOE_EINVAL
    assert lib.moe_rmsnorm(FAKE, None, 1, 64, ctypes.c_float(1e-6), FAKE, 0, None) == moeq.MOE_EINVAL
    ok = (FAKE, FAKE, 2, 64, 8, 2, FAKE, FAKE, FAKE)
    assert lib.moe_router_topk_scores(*ok, None, 256, None) == moeq.MOE_EWORKSPACE
    assert lib.moe_router_topk_scores(*ok, FAKE2, 255, None) == moeq.MOE_EWORKSPACE
    assert lib.moe_router_topk_scores(FAKE, FAKE, 2, 64, 8, 9, FAKE, FAKE, FAKE, FAKE2, 256, None) == moeq.MOE_EINVAL
    assert lib.moe_router_topk_scores(FAKE, FAKE, 2, 64, 1025, 2, FAKE, FAKE, FAKE, FAKE2, 256, None) == moeq.MOE_EINVAL
    B = moeq.moe_block(_layer(), FAKE, FAKE, 1e-6, 0)
    need = lib.moe_block_workspace_bytes(ctypes.byref(B), 4)
    assert need > _ws_bytes(lib, _layer(), 4)
    B.reserved = 1
    assert lib.moe_block_workspace_bytes(ctypes.byref(B), 4) == 0 and "reserved" in _err(lib)
    B.reserved, B.router_w = 0, None
    assert lib.moe_block_workspace_bytes(ctypes.byref(B), 4) == 0 and "router_w" in _err(lib)
    B.router_w = FAKE
    assert lib.moe_block_decode(ctypes.byref(B), FAKE, 4, FAKE, None, None, 0, FAKE2, need - 1,
                                None) == moeq.MOE_EWORKSPACE
    assert lib.moe_block_decode(ctypes.byref(B), None, 4, FAKE, None, None, 0, FAKE2, need, None) == moeq.MOE_EINVAL


def test_quantiser_validation(lib):
    """The MX e4m3 activation quantiser refuses bad shapes and NULL buffers
    before anything is enqueued."""
    assert lib.moe_quantize_mx_e4m3(FAKE, 2, 48, FAKE, FAKE, None) == moeq.MOE_EINVAL
    assert "H=48" in _err(lib)
    assert lib.moe_quantize_mx_e4m3(FAKE, 0, 64, FAKE, FAKE, None) == moeq.MOE_EINVAL
    assert lib.moe_quantize_mx_e4m3(None, 2, 64, FAKE, FAKE, None) == moeq.MOE_EINVAL
    assert lib.moe_quantize_mx_e4m3(FAKE, 2, 64, FAKE, None, None) == moeq.MOE_EINVAL
    assert "scales" in _err(lib)
