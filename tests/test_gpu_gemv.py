"""dense_gemv_q against the oracle: several shapes (ragged row counts, several
row tiles), batch sizes 1..8, both formats and both decoders."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import oracle
import synth
from gpu_util import bf16_rne_of_f32, dev_bf16, dev_u8, host_bf16, require_gpu
from helpers import PARITY_TOL, max_rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dec", [moeq.MOE_DECODER_LUT, moeq.MOE_DECODER_HW], ids=["lut", "hw"])
@pytest.mark.parametrize("fmt,rows,cols", [(1, 1, 32), (1, 37, 256), (1, 1000, 2048), (1, 515, 6144),
                                           (2, 3, 128), (2, 301, 1280), (2, 777, 5120), (2, 64, 8192)])
@pytest.mark.parametrize("B", [1, 3, 4, 8])
def test_gemv_parity(fmt, rows, cols, B, dec):
    require_gpu()
    c, s = synth.matrix(fmt, rows, cols, 11, synth.stream_id(synth.K_W_CODES, rows), synth.stream_id(synth.K_W_SCALES, rows))
    x = synth.normal_bf16(11, synth.stream_id(synth.K_X, cols), B * cols).reshape(B, cols)
    W = moeq.QMat(fmt, rows, cols, dev_u8(c), dev_u8(s))
    xd = dev_bf16(x)
    y32 = moeq.dense_gemv_q(W, xd, flags=moeq.MOE_OUT_F32 | dec)
    y16 = moeq.dense_gemv_q(W, xd, flags=dec)
    ref = oracle.gemv(fmt, rows, cols, c, s, x)
    assert max_rel_err(y32.cpu().numpy(), ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(y16), bf16_rne_of_f32(y32))


def test_gemv_full_size_sampled():
    """25600 x 5120 e2m3 at B = 1 and 4: sampled rows against the oracle."""
    require_gpu()
    cfg = synth.configs.GEMV
    c, s = synth.gemv_weights(cfg)
    W = moeq.QMat(cfg.fmt, cfg.rows, cfg.cols, dev_u8(c), dev_u8(s))
    rows = np.unique(np.concatenate([np.arange(0, cfg.rows, 397), [cfg.rows - 1]]))
    for B in cfg.batches:
        x = synth.gemv_x(cfg, B)
        y32 = moeq.dense_gemv_q(W, dev_bf16(x), flags=moeq.MOE_OUT_F32).cpu().numpy()
        ref = oracle.gemv(cfg.fmt, cfg.rows, cfg.cols, c, s, x, row_list=rows)
        assert max_rel_err(y32[:, rows], ref) <= PARITY_TOL


@pytest.mark.parametrize("fmt,rows,cols,B", [(1, 33000, 256, 3), (2, 1000, 384, 5), (1, 17, 64, 2), (2, 2070, 1152, 8)])
def test_gemv_matrix_core_tiling(fmt, rows, cols, B):
    """The several-token kernel's tiling edge cases: more 16-row tiles than a
    workgroup holds partial sums for (33000 rows: two tile groups on some
    workgroups), fewer K steps than waves (one or two), a ragged last tile, and
    fewer tiles than CUs; sampled rows against the oracle."""
    require_gpu()
    c, s = synth.matrix(fmt, rows, cols, 13, synth.stream_id(synth.K_W_CODES, rows), synth.stream_id(synth.K_W_SCALES, rows))
    x = synth.normal_bf16(13, synth.stream_id(synth.K_X, cols), B * cols).reshape(B, cols)
    W = moeq.QMat(fmt, rows, cols, dev_u8(c), dev_u8(s))
    y32 = moeq.dense_gemv_q(W, dev_bf16(x), flags=moeq.MOE_OUT_F32).cpu().numpy()
    sample = np.unique(np.concatenate([np.arange(0, rows, max(1, rows // 300)), np.arange(rows - 40, rows)]))
    sample = sample[sample >= 0]
    ref = oracle.gemv(fmt, rows, cols, c, s, x, row_list=sample)
    assert max_rel_err(y32[:, sample], ref) <= PARITY_TOL
