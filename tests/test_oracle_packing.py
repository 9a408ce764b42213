"""Pins of the oracle's unpacking: hand-worked rows, per-position one-hot
codes and per-block scale placement."""
import numpy as np
import pytest

import oracle
from helpers import read_packing_examples

E2M1, E2M3 = oracle.FMT_E2M1, oracle.FMT_E2M3
ONE_E4M3 = 0x38     # 1.0
ONE_UE8M0 = 127     # 1.0


@pytest.mark.parametrize("case", read_packing_examples(), ids=lambda c: c[0] + ":" + c[1].hex())
def test_hand_worked_rows(case):
    fmt_name, row, vals = case
    fmt = E2M1 if fmt_name == "e2m1" else E2M3
    cols = 32 if fmt == E2M1 else 128
    codes = np.zeros(oracle.code_row_bytes(fmt, cols), np.uint8)
    codes[: len(row)] = np.frombuffer(row, np.uint8)
    scales = np.full(oracle.scale_row_bytes(fmt, cols), ONE_E4M3 if fmt == E2M1 else ONE_UE8M0, np.uint8)
    w = oracle.decode(fmt, 1, cols, codes, scales)[0]
    got = w[: len(vals)]
    assert list(got) == vals
    assert list(np.signbit(got)) == list(np.signbit(vals))
    assert not w[len(vals):].any()


def _put_code(fmt, row, j, c):
    if fmt == E2M1:
        b = j >> 1
        row[b] = (row[b] & 0xF0) | c if j % 2 == 0 else (row[b] & 0x0F) | (c << 4)
    else:
        for t in range(6):
            bit = 6 * j + t
            if (c >> t) & 1:
                row[bit >> 3] |= 1 << (bit & 7)


@pytest.mark.parametrize("fmt", [E2M1, E2M3])
def test_one_hot_positions(fmt):
    """A single nonzero code at column j decodes at column j only, for every j."""
    cols = 256
    tmax = 7 if fmt == E2M1 else 31            # the largest positive code
    vmax = 6.0 if fmt == E2M1 else 7.5
    rows = []
    for j in range(cols):
        r = np.zeros(oracle.code_row_bytes(fmt, cols), np.uint8)
        _put_code(fmt, r, j, tmax)
        rows.append(r)
    codes = np.stack(rows)
    scales = np.full((cols, oracle.scale_row_bytes(fmt, cols)), ONE_E4M3 if fmt == E2M1 else ONE_UE8M0, np.uint8)
    W = oracle.decode(fmt, cols, cols, codes, scales)
    assert np.array_equal(W, vmax * np.eye(cols))


@pytest.mark.parametrize("fmt", [E2M1, E2M3])
def test_scale_blocks(fmt):
    """Scale byte b applies to columns [b*block, (b+1)*block) of its own row."""
    cols, block = (512, 16) if fmt == E2M1 else (1024, 128)
    nb = cols // block
    rows = 3
    one_code = 2 if fmt == E2M1 else 8           # value 1.0 in both formats
    codes = np.zeros((rows, oracle.code_row_bytes(fmt, cols)), np.uint8)
    for r in range(rows):
        for j in range(cols):
            _put_code(fmt, codes[r], j, one_code)
    if fmt == E2M1:
        # distinct e4m3 scales: bytes 0x20 .. (normal values 2^-3 .. )
        scales = (0x20 + (np.arange(rows)[:, None] * 3 + np.arange(nb)[None, :]) % 0x40).astype(np.uint8)
    else:
        scales = (100 + np.arange(rows)[:, None] * 5 + np.arange(nb)[None, :]).astype(np.uint8)
    W = oracle.decode(fmt, rows, cols, codes, scales)
    tab = oracle.tables()["e4m3" if fmt == E2M1 else "ue8m0"]
    expect = tab[scales][:, np.arange(cols) // block]
    assert np.array_equal(W, expect)
