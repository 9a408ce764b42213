"""Pins of the oracle's three further formats: e2m1 with a UE8M0 scale per 32
(MXFP4), two's-complement int4 with an fp16 scale per 64, and e2m3 with an
e4m3 scale per 16.  Each is pinned against something other than the oracle:
library decoders (numpy's float16, sign extension of int8), hand-worked rows,
one-hot placement, per-block scale placement, closed-form GEMVs and a numpy
matmul of the decoded matrix."""
import numpy as np
import pytest

import oracle
import synth
from helpers import read_format_variants

MX, I4, E3 = oracle.FMT_MXFP4, oracle.FMT_INT4_F16, oracle.FMT_E2M3_E4M3
NEW = [MX, I4, E3]
BF16_ONE = 0x3F80
NAMES = {"mxfp4": MX, "int4": I4, "e2m3_e4m3": E3}
ONE_SCALE = {MX: b"\x7f", I4: b"\x00\x3c", E3: b"\x38"}   # 1.0 in UE8M0, fp16, e4m3
BLOCK = {MX: 32, I4: 64, E3: 16}


def test_int4_table_is_twos_complement():
    c = np.arange(16, dtype=np.uint8)
    ref = ((c << 4).astype(np.int8) >> 4).astype(np.float64)     # sign extension by arithmetic shift
    assert np.array_equal(oracle.tables()["int4"], ref)


def test_fp16_decoder_matches_numpy_on_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_value(int(b)) for b in bits])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    assert np.array_equal(np.signbit(got[m]), np.signbit(ref[m]))


def test_row_and_scale_sizes():
    for fmt, cb, sb in ((MX, 64, 4), (I4, 64, 4), (E3, 96, 8)):
        assert oracle.code_row_bytes(fmt, 128) == cb and oracle.scale_row_bytes(fmt, 128) == sb
        assert synth.code_row_bytes(fmt, 128) == cb and synth.scale_row_bytes(fmt, 128) == sb


@pytest.mark.parametrize("case", read_format_variants(), ids=lambda c: c[0] + ":" + c[1].hex())
def test_hand_worked_rows(case):
    name, row, srow, vals = case
    fmt = NAMES[name]
    cols = 64 if fmt != E3 else 128
    codes = np.zeros(oracle.code_row_bytes(fmt, cols), np.uint8)
    codes[: len(row)] = np.frombuffer(row, np.uint8)
    scales = np.frombuffer(srow * (oracle.scale_row_bytes(fmt, cols) // len(srow)), np.uint8).copy()
    w = oracle.decode(fmt, 1, cols, codes, scales)[0]
    got = w[: len(vals)]
    assert list(got) == vals
    assert list(np.signbit(got)) == list(np.signbit(vals))
    assert not w[len(vals):].any()


def _put_code(fmt, row, j, c):
    if fmt in (MX, I4):
        b = j >> 1
        row[b] = (row[b] & 0xF0) | c if j % 2 == 0 else (row[b] & 0x0F) | (c << 4)
    else:
        for t in range(6):
            bit = 6 * j + t
            if (c >> t) & 1:
                row[bit >> 3] |= 1 << (bit & 7)


@pytest.mark.parametrize("fmt", NEW)
def test_one_hot_positions(fmt):
    """A single nonzero code at column j decodes at column j only."""
    cols = 256
    code, val = {MX: (7, 6.0), I4: (8, -8.0), E3: (31, 7.5)}[fmt]
    rows = []
    for j in range(cols):
        r = np.zeros(oracle.code_row_bytes(fmt, cols), np.uint8)
        _put_code(fmt, r, j, code)
        rows.append(r)
    scales = np.tile(np.frombuffer(ONE_SCALE[fmt], np.uint8), (cols, cols // BLOCK[fmt]))
    W = oracle.decode(fmt, cols, cols, np.stack(rows), scales)
    assert np.array_equal(W, val * np.eye(cols))


@pytest.mark.parametrize("fmt", NEW)
def test_scale_blocks(fmt):
    """Scale b of a row applies to columns [b*block, (b+1)*block) of that row."""
    cols, rows = 512, 3
    block, nb = BLOCK[fmt], 512 // BLOCK[fmt]
    one = {MX: 2, I4: 1, E3: 8}[fmt]                  # code of value 1.0
    codes = np.zeros((rows, oracle.code_row_bytes(fmt, cols)), np.uint8)
    for r in range(rows):
        for j in range(cols):
            _put_code(fmt, codes[r], j, one)
    if fmt == I4:
        h = (0x2C00 + 37 * (np.arange(rows)[:, None] * nb + np.arange(nb)[None, :])).astype(np.uint16)
        scales = h.astype("<u2").view(np.uint8).reshape(rows, 2 * nb)
        expect = h.view(np.float16).astype(np.float64)
    elif fmt == MX:
        scales = (110 + np.arange(rows)[:, None] * 3 + np.arange(nb)[None, :]).astype(np.uint8)
        expect = 2.0 ** (scales.astype(np.float64) - 127)
    else:
        scales = (0x20 + (np.arange(rows)[:, None] * 5 + np.arange(nb)[None, :]) % 0x50).astype(np.uint8)
        import torch
        expect = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    W = oracle.decode(fmt, rows, cols, codes, scales)
    assert np.array_equal(W, expect[:, np.arange(cols) // block])


@pytest.mark.parametrize("fmt,code,val,scale,sval", [
    (MX, 0x3, 1.5, b"\x7c", 0.125), (MX, 0xD, -3.0, b"\x83", 16.0),
    (I4, 0x5, 5.0, b"\x00\x3a", 0.75), (I4, 0x9, -7.0, b"\x01\x30", 0.125 * (1 + 2.0 ** -10)),
    (E3, 13, 1.625, b"\x30", 0.5), (E3, 63, -7.5, b"\x4c", 6.0)])
def test_constant_matrix_times_ones(fmt, code, val, scale, sval):
    rows, cols = 5, 384
    if fmt in (MX, I4):
        codes = np.full((rows, cols // 2), code | (code << 4), np.uint8)
    else:
        w = 0
        for q in range(4):
            w |= code << (6 * q)
        codes = np.tile(np.array([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], np.uint8), (rows, cols // 4))
    scales = np.tile(np.frombuffer(scale, np.uint8), (rows, cols // BLOCK[fmt]))
    x = np.full((2, cols), BF16_ONE, np.uint16)
    y = oracle.gemv(fmt, rows, cols, codes, scales, x)
    assert (y == cols * val * sval).all()


def _rand(fmt, rows, cols):
    return synth.matrix(fmt, rows, cols, 3, synth.stream_id(synth.K_W_CODES, 19), synth.stream_id(synth.K_W_SCALES, 19))


@pytest.mark.parametrize("fmt,rows,cols", [(MX, 40, 320), (I4, 24, 640), (E3, 30, 448)])
def test_random_against_library_matmul(fmt, rows, cols):
    c, s = _rand(fmt, rows, cols)
    x = synth.normal_bf16(4, synth.stream_id(synth.K_X, 78), 3 * cols).reshape(3, cols)
    W = oracle.decode(fmt, rows, cols, c, s)
    xf = np.array([[oracle.bf16_value(int(b)) for b in r] for r in x])
    ref = xf @ W.T
    y = oracle.gemv(fmt, rows, cols, c, s, x)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def test_int4_negation_and_power_of_two_scaling():
    """Negating every code (two's complement, codes other than -8) negates y
    exactly; multiplying x by 4 multiplies y by 4 exactly."""
    rows, cols = 17, 512
    c, s = _rand(I4, rows, cols)
    lo, hi = c & 0x0F, c >> 4
    lo[lo == 8] = 7
    hi[hi == 8] = 7
    c = (lo | (hi << 4)).astype(np.uint8)
    neg = (((16 - lo) & 0xF) | (((16 - hi) & 0xF) << 4)).astype(np.uint8)
    x = synth.normal_bf16(5, synth.stream_id(synth.K_X, 79), 2 * cols).reshape(2, cols)
    y = oracle.gemv(I4, rows, cols, c, s, x)
    assert (oracle.gemv(I4, rows, cols, neg, s, x) == -y).all()
    assert (oracle.gemv(I4, rows, cols, c, s, x + np.uint16(2 << 7)) == 4 * y).all()


@pytest.mark.parametrize("fmt", NEW)
def test_generator_scales_decode_to_their_distribution(fmt):
    """The generator's scales for each format decode (by the oracle) to values
    in the configured range."""
    c, s = _rand(fmt, 64, 512)
    W = oracle.decode(fmt, 64, 512, c, s)
    one = {MX: 2, I4: 1, E3: 8}[fmt]
    codes = np.zeros_like(c)
    for j in range(512):
        _put_code(fmt, codes[0], j, one)
    codes[:] = codes[0]
    S = oracle.decode(fmt, 64, 512, codes, s)     # every weight = its scale
    lo, hi = {MX: (2.0 ** -8, 2.0 ** -3), I4: (2.0 ** -8, 2.0 ** -4), E3: (2.0 ** -6, 2.0 ** -2)}[fmt]
    assert (S >= lo * (1 - 2 ** -10)).all() and (S <= hi * (1 + 2 ** -3)).all()
    assert np.isfinite(W).all()
