"""Pins of the oracle's GEMV: closed forms, exact invariants, one-hot columns
and a library matmul over the (separately pinned) decoded matrix."""
import numpy as np
import pytest

import oracle
import synth

E2M1, E2M3 = oracle.FMT_E2M1, oracle.FMT_E2M3
BF16_ONE = 0x3F80


def _rand_matrix(fmt, rows, cols, seed=3):
    return synth.matrix(fmt, rows, cols, seed, synth.stream_id(synth.K_W_CODES, 9), synth.stream_id(synth.K_W_SCALES, 9))


def _x(cols, B, seed=4):
    return synth.normal_bf16(seed, synth.stream_id(synth.K_X, 77), B * cols).reshape(B, cols)


@pytest.mark.parametrize("fmt,code,val,scale_byte,scale", [
    (E2M1, 3, 1.5, 0x30, 0.5), (E2M1, 0xD, -3.0, 0x4C, 6.0),
    (E2M3, 13, 1.625, 120, 2.0 ** -7), (E2M3, 63, -7.5, 130, 8.0)])
def test_constant_matrix_times_ones(fmt, code, val, scale_byte, scale):
    rows, cols = 5, 384
    if fmt == E2M1:
        codes = np.full((rows, cols // 2), code | (code << 4), np.uint8)
    else:
        w = 0
        for q in range(4):
            w |= code << (6 * q)
        grp = np.array([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], np.uint8)
        codes = np.tile(grp, (rows, cols // 4))
    scales = np.full((rows, oracle.scale_row_bytes(fmt, cols)), scale_byte, np.uint8)
    x = np.full((2, cols), BF16_ONE, np.uint16)
    y = oracle.gemv(fmt, rows, cols, codes, scales, x)
    assert (y == cols * val * scale).all()


@pytest.mark.parametrize("fmt", [E2M1, E2M3])
def test_sign_flip_and_power_of_two_scaling(fmt):
    rows, cols = 33, 512
    c, s = _rand_matrix(fmt, rows, cols)
    x = _x(cols, 3)
    y = oracle.gemv(fmt, rows, cols, c, s, x)
    # flip every code's sign bit
    if fmt == E2M1:
        cf = c ^ 0x88
    else:
        cf = c.copy()
        bits = np.unpackbits(cf, axis=1, bitorder="little")
        bits[:, 5::6] ^= 1
        cf = np.packbits(bits, axis=1, bitorder="little")
    yf = oracle.gemv(fmt, rows, cols, cf, s, x)
    assert (yf == -y).all()
    # x * 4: add 2 to every bf16 exponent (values stay normal)
    x4 = x + np.uint16(2 << 7)
    y4 = oracle.gemv(fmt, rows, cols, c, s, x4)
    assert (y4 == 4 * y).all()


@pytest.mark.parametrize("fmt", [E2M1, E2M3])
def test_one_hot_x_returns_a_column(fmt):
    rows, cols = 40, 256
    c, s = _rand_matrix(fmt, rows, cols)
    W = oracle.decode(fmt, rows, cols, c, s)
    for j in (0, 1, 15, 16, 127, 128, 255):
        x = np.zeros((1, cols), np.uint16)
        x[0, j] = BF16_ONE
        y = oracle.gemv(fmt, rows, cols, c, s, x)[0]
        assert np.array_equal(y, W[:, j])


@pytest.mark.parametrize("fmt,rows,cols", [(E2M1, 48, 320), (E2M3, 21, 640)])
def test_random_against_library_matmul(fmt, rows, cols):
    """Non-square so a transposed operand cannot pass."""
    c, s = _rand_matrix(fmt, rows, cols)
    x = _x(cols, 4)
    W = oracle.decode(fmt, rows, cols, c, s)
    xf = np.array([[oracle.bf16_value(int(b)) for b in r] for r in x])
    ref = xf @ W.T
    y = oracle.gemv(fmt, rows, cols, c, s, x)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    sub = np.array([5, 0, rows - 1, 7])
    ys = oracle.gemv(fmt, rows, cols, c, s, x, row_list=sub)
    assert np.array_equal(ys, y[:, sub])
