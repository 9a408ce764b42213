"""The Python binding refuses tensors whose shapes do not match the layer or
matrix they go with, before anything reaches the C library (a mismatched
tensor would let the kernels read or write past its allocation).  Every check
here runs on CPU tensors and raises before the first GPU touch."""
import ctypes

import pytest
import torch

import block_scaled_bit_moe_amd as moeq

H, I, E, K = 256, 512, 8, 2


def _fake_layer(fmt=1, shared_inter=0):
    """A Layer with its shape fields only (no GPU tensors): enough for the
    binding's shape checks, which come before any device pointer is taken."""
    L = object.__new__(moeq.Layer)
    L.fmt, L.hidden, L.inter, L.n_experts, L.top_k, L.shared_inter = fmt, H, I, E, K, shared_inter
    L.c = moeq.moe_layer()
    return L


def _u8(n):
    return torch.zeros(n, dtype=torch.uint8)


def _weights(fmt=1, e=E, h=H, i=I):
    crb, srb = moeq.code_row_bytes, moeq.scale_row_bytes
    return [_u8(e * 2 * i * crb(fmt, h)), _u8(e * 2 * i * srb(fmt, h)), _u8(e * h * crb(fmt, i)),
            _u8(e * h * srb(fmt, i))]


@pytest.mark.parametrize("which", range(4))
def test_layer_refuses_wrong_weight_sizes(which):
    w = _weights()
    w[which] = _u8(w[which].numel() - 16)
    with pytest.raises(ValueError, match="elements, expected"):
        moeq.Layer(1, H, I, E, K, *w)


def test_layer_refuses_wrong_shared_sizes():
    w = _weights()
    sh = dict(zip(("w13_codes", "w13_scales", "w2_codes", "w2_scales"), _weights(e=1, i=128)))
    sh["w2_codes"] = _u8(sh["w2_codes"].numel() + 16)
    with pytest.raises(ValueError, match="shared w2_codes"):
        moeq.Layer(1, H, I, E, K, *w, shared_inter=128, shared=sh)


def test_layer_with_right_sizes_reaches_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        moeq.Layer(1, H, I, E, K, *_weights())
    with pytest.raises(ValueError, match="GPU"):
        moeq.Layer(2, H, I, E, K, *_weights(fmt=2))


def test_qmat_refuses_wrong_sizes():
    with pytest.raises(ValueError, match="codes"):
        moeq.QMat(2, 100, 1280, _u8(100 * 960 - 1), _u8(100 * 10))
    with pytest.raises(ValueError, match="scales"):
        moeq.QMat(2, 100, 1280, _u8(100 * 960), _u8(100 * 10 + 1))
    with pytest.raises(ValueError, match="GPU"):
        moeq.QMat(2, 100, 1280, _u8(100 * 960), _u8(100 * 10))


@pytest.mark.parametrize("case", ["x_cols", "x_rows", "logits_cols", "logits_rows", "out", "idx", "w"])
def test_layer_decode_refuses_wrong_shapes(case):
    L = _fake_layer()
    T = 3
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    lg = torch.zeros(T, E)
    out = torch.zeros(T, H, dtype=torch.bfloat16)
    idx = torch.zeros(T, K, dtype=torch.int32)
    w = torch.zeros(T, K)
    if case == "x_cols":
        x = torch.zeros(T, H + 32, dtype=torch.bfloat16)
    elif case == "x_rows":
        lg = torch.zeros(T + 1, E)
    elif case == "logits_cols":
        lg = torch.zeros(T, E + 1)
    elif case == "logits_rows":
        lg = torch.zeros(T - 1, E)
    elif case == "out":
        out = torch.zeros(T, H - 32, dtype=torch.bfloat16)
    elif case == "idx":
        idx = torch.zeros(T, K + 1, dtype=torch.int32)
    else:
        w = torch.zeros(T + 1, K)
    with pytest.raises(ValueError, match="shape"):
        moeq.moe_layer_decode(L, x, lg, out=out, idx_out=idx, w_out=w)


def test_expert_ffn_refuses_wrong_shapes():
    L = _fake_layer()
    with pytest.raises(ValueError, match="x has shape"):
        moeq.moe_expert_ffn_q(L, 0, torch.zeros(2, H + 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="y has shape"):
        moeq.moe_expert_ffn_q(L, 0, torch.zeros(2, H, dtype=torch.bfloat16),
                              y=torch.zeros(3, H, dtype=torch.bfloat16))


def test_route_refuses_wrong_output_shapes():
    lg = torch.zeros(4, E)
    with pytest.raises(ValueError, match="idx has shape"):
        moeq.moe_route_topk(lg, K, idx=torch.zeros(4, K + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="w has shape"):
        moeq.moe_route_topk(lg, K, w=torch.zeros(3, K))


def test_gemv_refuses_wrong_shapes():
    W = object.__new__(moeq.QMat)
    W.fmt, W.rows, W.cols, W.c = 2, 100, 1280, moeq.moe_qmat()
    with pytest.raises(ValueError, match="x has shape"):
        moeq.dense_gemv_q(W, torch.zeros(2, 1280 + 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="y has shape"):
        moeq.dense_gemv_q(W, torch.zeros(2, 1280, dtype=torch.bfloat16), y=torch.zeros(2, 99, dtype=torch.bfloat16))
