"""The seeded generator: determinism, independence of streams, random access
by offset, and the value distributions the workloads ask for."""
import numpy as np
import pytest
import torch

import synth
from synth import configs


def test_deterministic_and_random_access():
    a = synth.random_bytes(0, synth.stream_id(1, 3), 10000)
    b = synth.random_bytes(0, synth.stream_id(1, 3), 10000)
    assert np.array_equal(a, b)
    c = synth.random_bytes(0, synth.stream_id(1, 3), 5003, offset=4997)
    assert np.array_equal(a[4997:], c)
    d = synth.random_bytes(0, synth.stream_id(1, 4), 10000)
    e = synth.random_bytes(1, synth.stream_id(1, 3), 10000)
    assert (a != d).mean() > 0.99 and (a != e).mean() > 0.99
    x = synth.normal_bf16(0, 5, 1000)
    assert np.array_equal(x[100:], synth.normal_bf16(0, 5, 900, offset=100))


def test_code_bytes_uniform():
    a = synth.random_bytes(0, synth.stream_id(synth.K_W13_CODES, 0), 1 << 20)
    lo, hi = np.bincount(a & 15, minlength=16), np.bincount(a >> 4, minlength=16)
    exp = a.size / 16
    for cnt in (lo, hi):
        chi2 = ((cnt - exp) ** 2 / exp).sum()
        assert chi2 < 60            # 15 dof; p ~ 1e-7
    # 6-bit codes from the same uniform bytes are uniform too
    bits = np.unpackbits(a[: 3 * 65536], bitorder="little").reshape(-1, 6)
    codes = (bits * (1 << np.arange(6))).sum(1)
    cnt = np.bincount(codes, minlength=64)
    assert ((cnt - cnt.mean()) ** 2 / cnt.mean()).sum() < 150


def test_e4m3_scales_log_uniform():
    s = synth.e4m3_loguniform(0, 7, 200000, -6.0, -2.0)
    v = torch.from_numpy(s).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert v.min() >= 2.0 ** -6 and v.max() <= 2.0 ** -2
    lg = np.log2(v)
    assert abs(lg.mean() - (-4.0)) < 0.02
    # 2^u with u ~ U[-6, -2) rounds into binade e when u lies in
    # [e - 1 + log2(1.9375), e + log2(1.9375)) (RNE at 4 significant bits)
    c = np.log2(1.9375)
    for e in (-6, -5, -4, -3, -2):
        lo, hi = max(-6.0, e - 1 + c), min(-2.0, e + c)
        frac = ((lg >= e) & (lg < e + 1)).mean()
        assert abs(frac - (hi - lo) / 4.0) < 0.005, e


def test_e4m3_encoder_is_round_to_nearest_even():
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(1, 0x7E):
        assert synth.e4m3_encode(vals[b]) == b
        mid = (vals[b] + vals[b + 1]) / 2          # a tie goes to the even code
        want = b if b % 2 == 0 else b + 1
        assert synth.e4m3_encode(mid) == want, b


def test_ue8m0_exponents_uniform():
    s = synth.ue8m0_uniform(0, 9, 60000, -8, -3)
    assert s.min() == 119 and s.max() == 124
    cnt = np.bincount(s - 119, minlength=6)
    assert np.abs(cnt / cnt.sum() - 1 / 6).max() < 0.01


def test_normals_and_bf16_rounding():
    x = synth.normal_bf16(0, 11, 400000, sigma=1.0)
    v = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    l = synth.normal_f32(0, 12, 400000, sigma=1.5)
    assert abs(l.std() - 1.5) < 0.01
    rng = np.random.default_rng(0)
    f = rng.standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([synth.bf16_from_double(float(t)) for t in f], np.uint16)
    assert np.array_equal(got, ref)


def test_layer_shapes():
    cfg = configs.TOY
    L = synth.layer_weights(cfg)
    assert L["w13_codes"].shape == (8, 1024, 128) and L["w13_scales"].shape == (8, 1024, 16)
    assert L["w2_codes"].shape == (8, 256, 256) and L["w2_scales"].shape == (8, 256, 32)
    e3 = synth.expert_weights(cfg, 3)
    assert np.array_equal(e3["w2_codes"], L["w2_codes"][3])


def test_fp16_encoder_matches_numpy():
    """The int4 format's fp16 scales: round to nearest even over normal values."""
    rng = np.random.default_rng(5)
    vals = np.concatenate([2.0 ** rng.uniform(-14, 15, 4000), [1.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504.0,
                                                              2.0 ** -14]])
    for v in vals:
        assert synth.fp16_encode(float(v)) == int(np.float16(v).view(np.uint16)), v
    b = synth.fp16_loguniform(0, 9, 5000, -8.0, -4.0)
    h = b.view("<u2").view(np.float16).astype(np.float64)
    assert (h >= 2.0 ** -8 * (1 - 2 ** -11)).all() and (h <= 2.0 ** -4 * (1 + 2 ** -11)).all()
    assert abs(np.log2(h).mean() + 6.0) < 0.1
