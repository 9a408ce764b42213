"""Pins of the oracle's activation quantiser (MX: e4m3 elements, a UE8M0
scale per 32): closed-form blocks, the scale exponent against numpy's log2,
the element rounding against torch's float8_e4m3fn conversion, saturation,
zero and signed-zero blocks, and the round-trip error bound."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import MoEConfig


def _bf(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _f(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("p", [-20, -3, 0, 5, 30])
def test_power_of_two_block(p):
    x = _bf(np.full((1, 32), 2.0 ** p))
    c, s = oracle.quantize_mx_e4m3(x)
    assert s[0, 0] == 127 + p - 8
    assert (c == 0x78).all()                       # 256 = 2^8 in e4m3
    assert (oracle.dequantize_mx_e4m3(c, s) == 2.0 ** p).all()


def test_zero_and_signed_zero():
    x = np.zeros((1, 64), np.uint16)
    x[0, 40] = 0x8000                              # -0 in the second block (all zeros)
    x[0, 3] = _bf([1.0])[0]
    x[0, 5] = 0x8000                               # -0 beside a nonzero
    c, s = oracle.quantize_mx_e4m3(x)
    assert s[0, 1] == 0 and c[0, 40] == 0x80 and (np.delete(c[0, 32:], 8) == 0).all()
    assert c[0, 5] == 0x80 and s[0, 0] == 127 - 8


def test_saturation_at_448():
    """amax = 1.9375 * 2^k scales to 496 > 448: it saturates to 448 (0x7E)."""
    x = _bf(np.concatenate([[1.9375 * 4, -1.9375 * 4], np.full(30, 0.5)])[None, :])
    c, s = oracle.quantize_mx_e4m3(x)
    assert s[0, 0] == 127 + 2 - 8
    assert c[0, 0] == 0x7E and c[0, 1] == 0xFE


def test_scale_rule_and_rounding_against_libraries():
    cfg = MoEConfig("q", tokens=7, hidden=512, experts=2, top_k=1, inter=32, x_sigma=3.0)
    x = synth.hidden_states(cfg)
    x[2, 64:96] = _bf(np.linspace(-1e-30, 1e-30, 32))      # tiny block
    x[3, :32] = _bf(2.0 ** np.arange(-20, 12, dtype=np.float64))   # wide range
    c, s = oracle.quantize_mx_e4m3(x)
    xf = _f(x)
    blocks = xf.reshape(7, -1, 32)
    amax = np.abs(blocks).max(axis=2)
    X = np.floor(np.log2(amax)) - 8
    assert np.array_equal(s.astype(np.float64) - 127, np.clip(X, -127, 127))
    scaled = blocks / np.exp2(s.astype(np.float64) - 127)[..., None]
    ok = np.abs(scaled) <= 448
    ref = torch.from_numpy(scaled[ok]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(c.reshape(7, -1, 32)[ok], ref)
    assert (c.reshape(7, -1, 32)[~ok] & 0x7F == 0x7E).all()


def test_round_trip_bound():
    cfg = MoEConfig("q2", tokens=9, hidden=1024, experts=2, top_k=1, inter=32)
    x = synth.hidden_states(cfg, sub=3)
    c, s = oracle.quantize_mx_e4m3(x)
    d = oracle.dequantize_mx_e4m3(c, s)
    xf = _f(x)
    X = np.repeat(s.astype(np.float64) - 127, 32, axis=1)
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** (X - 10))   # half an e4m3 unit, normal or subnormal
    sat = np.abs(xf) > 448 * 2.0 ** X      # the block's top binade above 448: the rule saturates these
    assert (np.abs(d - xf)[~sat] <= bound[~sat]).all()
    assert np.array_equal(d[sat], np.sign(xf[sat]) * 448 * 2.0 ** X[sat])
