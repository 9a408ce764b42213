"""Planted mistakes in copies of the oracle's source must each fail a pin.

Each mutant is the oracle with one plausible slip (a wrong bias, nibble or bit
order, scale index, tie-break, dropped term, swapped operand ...).  The copy
is compiled on the CPU into a temporary library and run through a battery of
the pins; the test passes when at least one pin rejects every mutant."""
import os
import subprocess
import tempfile

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth
from helpers import read_format_variants, read_packing_examples, read_table
from synth.configs import MoEConfig

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

MUTANTS = {
    "e2m1_bias": ("minifloat(c, 2, 1, 1)", "minifloat(c, 2, 1, 2)"),
    "e2m3_fields": ("minifloat(c, 2, 3, 1)", "minifloat(c, 3, 2, 1)"),
    "e4m3_bias": ("minifloat(b, 4, 3, 7)", "minifloat(b, 4, 3, 8)"),
    "e4m3_nan": ("(b & 0x7F) == 0x7F", "(b & 0x7F) == 0x7E"),
    "subnormal_exp": ("ldexp((double)m / (double)(1u << mbits), 1 - bias)",
                      "ldexp((double)m / (double)(1u << mbits), -bias)"),
    "nibble_order": ("(j & 1) ? (b >> 4) : (b & 0x0F)", "(j & 1) ? (b & 0x0F) : (b >> 4)"),
    "e2m3_bit_order": ("& 1) << t;", "& 1) << (5 - t);"),
    "scale_block": ("case ORACLE_FMT_E2M1: return T_E2M1[c] * T_E4M3[srow[j / 16]];",
                    "case ORACLE_FMT_E2M1: return T_E2M1[c] * T_E4M3[srow[j / 32]];"),
    "mxfp4_block": ("T_E2M1[c] * T_UE8M0[srow[j / 32]]", "T_E2M1[c] * T_UE8M0[srow[j / 16]]"),
    "mxfp4_scale_kind": ("T_E2M1[c] * T_UE8M0[srow[j / 32]]", "T_E2M1[c] * T_E4M3[srow[j / 32]]"),
    "mxfp4_six_bit": ("fmt == ORACLE_FMT_MXFP4 || ", ""),
    "int4_unsigned": ("T_INT4[c] = (double)(c & 7u) - ((c & 8u) ? 8.0 : 0.0);", "T_INT4[c] = (double)c;"),
    "int4_offset_binary": ("T_INT4[c] = (double)(c & 7u) - ((c & 8u) ? 8.0 : 0.0);", "T_INT4[c] = (double)c - 8.0;"),
    "int4_group": ("srow + 2 * (j / 64)", "srow + 2 * (j / 32)"),
    "fp16_byte_order": ("(unsigned)g[0] | ((unsigned)g[1] << 8)", "(unsigned)g[1] | ((unsigned)g[0] << 8)"),
    "fp16_bias": ("ldexp(1.0 + (double)m / 1024.0, (int)e - 15)", "ldexp(1.0 + (double)m / 1024.0, (int)e - 16)"),
    "fp16_subnormal": ("ldexp((double)m / 1024.0, -14)", "ldexp((double)m / 1024.0, -15)"),
    "rmsnorm_no_eps": ("sqrt(ss / (double)H + eps)", "sqrt(ss / (double)H)"),
    "rmsnorm_sum_not_mean": ("sqrt(ss / (double)H + eps)", "sqrt(ss + eps)"),
    "rmsnorm_no_gain": ("y[t * H + i] = bf16_value(xt[i]) * bf16_value(g[i]) * r;", "y[t * H + i] = bf16_value(xt[i]) * r;"),
    "router_transposed": ("bf16_value(wr[e * H + j])", "bf16_value(wr[j * E + e])"),
    "residual_dropped": ("out[i] = bf16_value(r[i]) + y[i];", "out[i] = y[i];"),
    "quant_emax": ("X = (e - 1) - 8;", "X = (e - 1) - 7;"),
    "quant_ceil": ("X = (e - 1) - 8;", "X = e - 8;"),
    "quant_ties_odd": ("(d == bd && (c & 1u) == 0)", "(d == bd && (c & 1u) == 1)"),
    "quant_block16": ("const uint16_t *xb = x + t * H + 32 * b;", "const uint16_t *xb = x + t * H + 16 * b;"),
    "quant_sign_dropped": ("const uint8_t s = signbit(v) ? 0x80 : 0x00;", "const uint8_t s = 0x00;"),
    "e2m3_e4m3_block": ("T_E2M3[c] * T_E4M3[srow[j / 16]]", "T_E2M3[c] * T_E4M3[srow[j / 128]]"),
    "e2m3_e4m3_scale_kind": ("T_E2M3[c] * T_E4M3[srow[j / 16]]", "T_E2M3[c] * T_UE8M0[srow[j / 16]]"),
    "ue8m0_bias": ("ldexp(1.0, (int)b - 127)", "ldexp(1.0, (int)b - 126)"),
    "bf16_widen": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    "gemv_last_col": ("for (int64_t j = 0; j < cols; ++j) acc += weight_at(fmt, crow, srow, j) * bf16_value(x[j]);",
                      "for (int64_t j = 0; j < cols - 1; ++j) acc += weight_at(fmt, crow, srow, j) * bf16_value(x[j]);"),
    "tie_break": ("    if (la < lb) return 0;\n    return a < b;", "    if (la < lb) return 0;\n    return a > b;"),
    "nan_order": ("return nb;", "return na;"),
    "softmax_no_norm": ("w[t * k + r] = exp((double)l[idx[t * k + r]] - l0) / z;",
                        "w[t * k + r] = exp((double)l[idx[t * k + r]] - l0);"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "gate_up_swap": ("h[i] = oracle_silu(g) * u;", "h[i] = oracle_silu(u) * g;"),
    "up_rows": ("w13c + (I + i) * cbH, w13s + (I + i) * sbH", "w13c + i * cbH, w13s + i * sbH"),
    "shared_weight": ("for (int64_t q = 0; q < n_out; ++q) o[q] += y[q];",
                      "for (int64_t q = 0; q < n_out; ++q) o[q] += 0.5 * y[q];"),
    "drop_rank0": ("for (int64_t r = 0; r < k; ++r) {\n            int32_t e",
                   "for (int64_t r = 1; r < k; ++r) {\n            int32_t e"),
}

CFG = MoEConfig("mut", tokens=2, hidden=128, experts=4, top_k=2, inter=64, shared_inter=64)


def _pin_tables():
    t = oracle.tables()
    g1, g3 = read_table("e2m1_values.txt"), read_table("e2m3_values.txt")
    assert list(t["e2m1"]) == [g1[c] for c in range(16)]
    assert list(t["e2m3"][:32]) == [g3[c] for c in range(32)]
    import torch
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t["e4m3"]), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(t["e4m3"][m], ref[m])
    assert all(t["ue8m0"][b] == 2.0 ** (b - 127) for b in range(255))
    assert oracle.bf16_value(0x3F80) == 1.0


def _pin_packing():
    for fmt_name, row, vals in read_packing_examples():
        fmt = 1 if fmt_name == "e2m1" else 2
        cols = 32 if fmt == 1 else 128
        codes = np.zeros(oracle.code_row_bytes(fmt, cols), np.uint8)
        codes[: len(row)] = np.frombuffer(row, np.uint8)
        scales = np.full(oracle.scale_row_bytes(fmt, cols), 0x38 if fmt == 1 else 127, np.uint8)
        assert list(oracle.decode(fmt, 1, cols, codes, scales)[0][: len(vals)]) == vals


def _pin_scale_blocks():
    cols = 64
    codes = np.full((1, 32), 0x22, np.uint8)               # every weight 1.0
    scales = np.array([[0x30, 0x38, 0x40, 0x48]], np.uint8)
    W = oracle.decode(1, 1, cols, codes, scales)[0]
    tab = oracle.tables()["e4m3"]
    assert np.array_equal(W, np.repeat(tab[scales[0]], 16))


def _pin_gemv():
    rows, cols = 3, 256
    codes = np.full((rows, cols // 2), 0x33, np.uint8)      # 1.5 everywhere
    scales = np.full((rows, cols // 16), 0x30, np.uint8)    # 0.5
    x = np.full((1, cols), 0x3F80, np.uint16)
    assert (oracle.gemv(1, rows, cols, codes, scales, x) == cols * 0.75).all()


def _rule(l, k):
    key = lambda i: (1, 0.0, i) if np.isnan(l[i]) else (0, -float(l[i]), i)
    return sorted(range(len(l)), key=key)[:k]


def _pin_route():
    import itertools
    for pattern in itertools.product([0.0, 1.0], repeat=4):
        l = np.array(pattern, np.float32)
        for k in range(1, 5):
            idx, w = oracle.route(l, k)
            assert list(idx[0]) == _rule(l, k)
            assert abs(w.sum() - 1) < 1e-15
    l = np.array([np.nan, 1.0, np.nan, 1.0], np.float32)
    assert list(oracle.route(l, 4)[0][0]) == [1, 3, 0, 2]
    l = synth.router_logits(CFG)
    idx, w = oracle.route(l, 3)
    sel = np.take_along_axis(l.astype(np.float64), idx.astype(np.int64), axis=1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-14, atol=0)


def _pin_silu():
    assert oracle.silu(0.0) == 0.0
    for z in (-3.0, 0.7, 2.0):
        assert abs(oracle.silu(z) - z * expit(z)) < 1e-15


def _pin_ffn_and_layer():
    H, I = CFG.hidden, CFG.inter
    x = synth.hidden_states(CFG)
    ex = {e: synth.expert_weights(CFG, e) for e in range(CFG.experts)}
    sh = synth.expert_weights(CFG, CFG.experts)
    l = synth.router_logits(CFG)
    ys = {}
    for e, ew in ex.items():
        W13 = oracle.decode(1, 2 * I, H, ew["w13_codes"], ew["w13_scales"])
        W2 = oracle.decode(1, H, I, ew["w2_codes"], ew["w2_scales"])
        xf = np.array([oracle.bf16_value(int(b)) for b in x[0]])
        g, u = W13[:I] @ xf, W13[I:] @ xf
        ref = W2 @ (g * expit(g) * u)
        y = oracle.ffn(1, H, I, ew, x[0])
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        ys[e] = y
    _, _, out = oracle.layer(1, H, I, 4, 4, ex, x[:1], l[:1])
    p = softmax(l[0].astype(np.float64))
    ref = sum(p[e] * ys[e] for e in range(4))
    assert np.allclose(out[0], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    _, _, a = oracle.layer(1, H, I, 4, 2, ex, x[:1], l[:1])
    _, _, b = oracle.layer(1, H, I, 4, 2, ex, x[:1], l[:1], shared=sh, shared_inter=CFG.shared_inter)
    ysh = oracle.ffn(1, H, CFG.shared_inter, sh, x[0])
    assert np.allclose(b[0] - a[0], ysh, rtol=1e-12, atol=1e-12 * np.abs(ysh).max())


def _pin_formats():
    """The further formats: int4 by sign extension, fp16 by numpy on a spread of
    patterns, the hand-worked rows, and one block placement each."""
    c = np.arange(16, dtype=np.uint8)
    assert np.array_equal(oracle.tables()["int4"], ((c << 4).astype(np.int8) >> 4).astype(np.float64))
    for b in list(range(0, 1 << 16, 97)) + [0x0001, 0x03FF, 0x0400, 0x3C00, 0x3555, 0x7BFF, 0x8001]:
        ref = float(np.array([b], np.uint16).view(np.float16)[0])
        got = oracle.fp16_value(b)
        assert (np.isnan(ref) and np.isnan(got)) or got == ref
    names = {"mxfp4": 3, "int4": 4, "e2m3_e4m3": 5}
    for name, row, srow, vals in read_format_variants():
        fmt = names[name]
        cols = 128
        codes = np.zeros(oracle.code_row_bytes(fmt, cols), np.uint8)
        codes[: len(row)] = np.frombuffer(row, np.uint8)
        scales = np.frombuffer(srow * (oracle.scale_row_bytes(fmt, cols) // len(srow)), np.uint8).copy()
        assert list(oracle.decode(fmt, 1, cols, codes, scales)[0][: len(vals)]) == vals
    # block placement: value 1.0 everywhere, a distinct scale per block
    for fmt, one_byte, block, sc in ((3, 0x22, 32, [120, 121, 122, 123]), (5, None, 16, list(range(0x30, 0x38))),
                                     (4, 0x11, 64, [0x00, 0x3C, 0x00, 0x40])):
        cols = 128
        if one_byte is not None:
            codes = np.full((1, cols // 2), one_byte, np.uint8)
        else:   # e2m3 code 8 (1.0) in every 6-bit slot
            w = sum(8 << (6 * q) for q in range(4))
            codes = np.tile(np.array([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], np.uint8), (1, cols // 4))
        scales = np.array([sc], np.uint8)
        W = oracle.decode(fmt, 1, cols, codes, scales)[0]
        if fmt == 3:
            expect = np.repeat(2.0 ** (np.array(sc, np.float64) - 127), block)
        elif fmt == 4:
            expect = np.repeat(np.array(sc, np.uint8).view("<u2").view(np.float16).astype(np.float64), block)
        else:
            import torch
            expect = np.repeat(torch.tensor(sc, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy(), block)
        assert np.array_equal(W, expect)


def _pin_block():
    """RMSNorm one-hot and constant rows, router scores against a numpy matmul
    (E != H), residual add of known values."""
    H = 256
    g = np.full(H, 0x3F80, np.uint16)
    x = np.zeros((1, H), np.uint16)
    x[0, 3] = 0x4080                                         # 4.0
    y = oracle.rmsnorm(x, g, 0.0)[0]
    assert y[3] == 16.0 and not np.delete(y, 3).any()
    xc = np.full((1, H), 0x4040, np.uint16)                   # 3.0
    assert np.allclose(oracle.rmsnorm(xc, g, 0.5)[0], 3.0 / np.sqrt(9.5), rtol=1e-15, atol=0)
    g2 = np.full(H, 0x4000, np.uint16)                        # gain 2
    assert oracle.rmsnorm(x, g2, 0.0)[0][3] == 32.0
    cfg = MoEConfig("r", tokens=2, hidden=96, experts=40, top_k=3, inter=32)
    xr, wr = synth.hidden_states(cfg), synth.router_weights(cfg)
    f = lambda a: np.array([[oracle.bf16_value(int(b)) for b in r] for r in a])
    ref = f(xr) @ f(wr).T
    assert np.allclose(oracle.router_logits(xr, wr), ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    assert list(oracle.residual_add(np.array([0x3FC0, 0xC000], np.uint16), np.array([0.25, 0.5]))) == [1.75, -1.5]


def _pin_quant():
    """Quantiser: a power-of-two block, saturation, -0, and torch's e4m3
    rounding of a scaled random block."""
    x = np.full((1, 32), 0x4080, np.uint16)                       # 4.0
    c, s = oracle.quantize_mx_e4m3(x)
    assert s[0, 0] == 127 + 2 - 8 and (c == 0x78).all()
    xs = np.full((1, 32), 0x3F00, np.uint16)                      # 0.5
    xs[0, 0], xs[0, 1], xs[0, 2] = 0x40F8, 0xC0F8, 0x8000         # 7.75, -7.75, -0
    c, s = oracle.quantize_mx_e4m3(xs)
    assert s[0, 0] == 127 + 2 - 8 and c[0, 0] == 0x7E and c[0, 1] == 0xFE and c[0, 2] == 0x80
    import torch
    cfg = MoEConfig("q", tokens=2, hidden=64, experts=2, top_k=1, inter=32, x_sigma=3.0)
    xr = synth.hidden_states(cfg)
    c, s = oracle.quantize_mx_e4m3(xr)
    xf = (xr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sc = xf / np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    ok = np.abs(sc) <= 448
    assert np.array_equal(c[ok], torch.from_numpy(sc[ok]).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert np.array_equal(s.astype(np.float64) - 127, np.floor(np.log2(np.abs(xf).reshape(2, 2, 32).max(axis=2))) - 8)


PINS = [_pin_tables, _pin_packing, _pin_scale_blocks, _pin_gemv, _pin_route, _pin_silu, _pin_ffn_and_layer,
        _pin_formats, _pin_block, _pin_quant]


def _failures():
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, KeyError) as exc:
            failed.append(pin.__name__)
    return failed


def test_unmutated_oracle_passes_the_battery():
    oracle.use_library(None)
    assert _failures() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site must be unique: %s" % name
    path = tmp_path / "oracle_mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("liboracle_%s.so" % name))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                    "-ffp-contract=off", str(path), "-o", lib, "-lm"], check=True)
    try:
        oracle.use_library(lib)
        failed = _failures()
    finally:
        oracle.use_library(None)
    assert failed, "mutant %s passed every pin" % name
