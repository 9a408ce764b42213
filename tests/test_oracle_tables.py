"""Pins of the oracle's decode tables against the format definitions and
independent library decoders (torch's float8 dtypes)."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import read_table


def _same(a, b):
    """Equal as IEEE values, including the sign of zero and NaN positions."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape
    na, nb = np.isnan(a), np.isnan(b)
    assert (na == nb).all(), np.nonzero(na != nb)
    m = ~na
    assert (a[m] == b[m]).all(), np.nonzero(a[m] != b[m])
    assert (np.signbit(a[m]) == np.signbit(b[m])).all()


def test_e2m1_table_matches_published_values():
    t = oracle.tables()["e2m1"]
    g = read_table("e2m1_values.txt")
    _same(t, [g[c] for c in range(16)])


def test_e2m3_table_matches_published_values():
    t = oracle.tables()["e2m3"]
    g = read_table("e2m3_values.txt")
    pos = np.array([g[c] for c in range(32)])
    _same(t[:32], pos)
    _same(t[32:], -pos)            # sign bit 5; code 32 is -0


def test_e2m3_structure():
    t = oracle.tables()["e2m3"][:32]
    assert (np.diff(t) > 0).all()                      # strictly increasing over the positive codes
    assert t[31] == 7.5 and t[1] == 0.125
    assert np.allclose(np.diff(t[:9]), 0.125)          # subnormals and the first binade share unit 1/8
    for e in (1, 2, 3):                                 # 8 evenly spaced values per binade
        b = t[8 * e: 8 * e + 8]
        assert np.allclose(np.diff(b), 2.0 ** (e - 1) / 8)


def test_e4m3_table_matches_torch_float8_e4m3fn():
    t = oracle.tables()["e4m3"]
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    _same(t, ref)
    assert t[0x7E] == 448.0 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x01] == 2.0 ** -9 and t[0x38] == 1.0


def test_ue8m0_table_matches_torch_float8_e8m0fnu():
    t = oracle.tables()["ue8m0"]
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    # torch's decoder may flush 2^-127 (a binary32 subnormal) -- compare where it does not
    ok = ~((np.arange(256) == 0) & (ref == 0))
    _same(t[ok], ref[ok])
    for b in range(255):
        assert t[b] == math.ldexp(1.0, b - 127)
    assert np.isnan(t[255])


def test_bf16_widening_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.int64).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    _same(got, ref)


def test_bf16_round_matches_torch_for_float32_inputs():
    rng = np.random.default_rng(1)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),          # subnormal range
        # exact ties: bf16 value plus half an ulp
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 3.3895314e38, -3.3895314e38], np.float32),
    ])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(f.astype(np.float64))
    assert (got == ref).all(), np.nonzero(got != ref)[0][:10]
