"""Every code of every format through the GPU decoders (LDS tables and the
hardware conversions), read back through one-hot activations: the result
must be the code's value exactly."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import oracle
from gpu_util import dev_bf16, dev_u8, require_gpu

pytestmark = pytest.mark.gpu
DECODERS = [moeq.MOE_DECODER_LUT, moeq.MOE_DECODER_HW]
BF16_ONE = 0x3F80


def _one_hots(cols, js):
    x = np.zeros((len(js), cols), np.uint16)
    for i, j in enumerate(js):
        x[i, j] = BF16_ONE
    return x


@pytest.mark.parametrize("dec", DECODERS, ids=["lut", "hw"])
def test_e2m1_every_code_every_position(dec):
    require_gpu()
    cols, rows = 64, 16
    codes = np.array([[r | (r << 4)] * (cols // 2) for r in range(rows)], np.uint8)   # row r: all code r
    scales = np.full((rows, cols // 16), 0x38, np.uint8)                            # 1.0
    W = moeq.QMat(1, rows, cols, dev_u8(codes), dev_u8(scales))
    tab = oracle.tables()["e2m1"]
    for j0 in range(0, cols, 8):
        x = dev_bf16(_one_hots(cols, range(j0, j0 + 8)))
        y = moeq.dense_gemv_q(W, x, flags=moeq.MOE_OUT_F32 | dec).cpu().numpy()
        assert np.array_equal(y, np.tile(tab[:rows], (8, 1))), j0


@pytest.mark.parametrize("dec", DECODERS, ids=["lut", "hw"])
def test_e2m3_every_code_every_position(dec):
    require_gpu()
    cols, rows = 128, 64
    codes = np.zeros((rows, cols * 3 // 4), np.uint8)
    for r in range(rows):                 # row r: every element code r
        w = 0
        for q in range(4):
            w |= r << (6 * q)
        codes[r] = np.tile(np.array([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], np.uint8), cols // 4)
    scales = np.full((rows, 1), 127, np.uint8)
    W = moeq.QMat(2, rows, cols, dev_u8(codes), dev_u8(scales))
    tab = oracle.tables()["e2m3"]
    for j0 in range(0, cols, 8):
        x = dev_bf16(_one_hots(cols, range(j0, j0 + 8)))
        y = moeq.dense_gemv_q(W, x, flags=moeq.MOE_OUT_F32 | dec).cpu().numpy()
        assert np.array_equal(y, np.tile(tab, (8, 1))), j0


@pytest.mark.parametrize("dec", DECODERS, ids=["lut", "hw"])
def test_e4m3_every_finite_scale(dec):
    require_gpu()
    bytes_ = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)      # 254 finite codes
    rows, cols = len(bytes_), 32
    codes = np.full((rows, cols // 2), 0x22, np.uint8)                            # every weight 1.0
    scales = np.stack([bytes_, bytes_], axis=1)
    W = moeq.QMat(1, rows, cols, dev_u8(codes), dev_u8(scales))
    x = dev_bf16(_one_hots(cols, [0, 31]))
    y = moeq.dense_gemv_q(W, x, flags=moeq.MOE_OUT_F32 | dec).cpu().numpy()
    want = oracle.tables()["e4m3"][bytes_].astype(np.float32)
    assert np.array_equal(y[0], want) and np.array_equal(y[1], want)
    # 64 columns (two units per row): the several-token kernel takes it, scale folded into the weights
    W2 = moeq.QMat(1, rows, 64, dev_u8(np.full((rows, 32), 0x22, np.uint8)),
                   dev_u8(np.ascontiguousarray(np.stack([bytes_] * 4, axis=1))))
    y2 = moeq.dense_gemv_q(W2, dev_bf16(_one_hots(64, [0, 63])), flags=moeq.MOE_OUT_F32 | dec).cpu().numpy()
    assert np.array_equal(y2[0], want) and np.array_equal(y2[1], want)


@pytest.mark.parametrize("dec", DECODERS, ids=["lut", "hw"])
def test_ue8m0_scales(dec):
    require_gpu()
    bytes_ = np.arange(1, 255, dtype=np.uint8)          # 2^-126 .. 2^127 (fp32 normal)
    rows, cols = len(bytes_), 128
    w = 8 | (8 << 6) | (8 << 12) | (8 << 18)             # code 8 = 1.0
    codes = np.tile(np.array([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], np.uint8), (rows, cols // 4))
    scales = bytes_.reshape(rows, 1)
    W = moeq.QMat(2, rows, cols, dev_u8(codes), dev_u8(scales))
    x = dev_bf16(_one_hots(cols, [5, cols - 1]))     # two tokens: the several-token kernel too
    y = moeq.dense_gemv_q(W, x, flags=moeq.MOE_OUT_F32 | dec).cpu().numpy()
    want = oracle.tables()["ue8m0"][bytes_].astype(np.float32)
    assert np.array_equal(y[0], want) and np.array_equal(y[1], want)
    y1 = moeq.dense_gemv_q(W, x[:1], flags=moeq.MOE_OUT_F32 | dec).cpu().numpy()
    assert np.array_equal(y1[0], want)
