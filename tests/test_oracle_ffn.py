"""Pins of the oracle's SwiGLU expert and layer: closed forms, zero matrices,
library matmuls, one-hot routing, k = E dense mixture, 4-expert brute force
and the shared expert's weight."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth
from synth import configs
from synth.configs import MoEConfig

E2M1, E2M3 = oracle.FMT_E2M1, oracle.FMT_E2M3
SMALL = MoEConfig("small", tokens=3, hidden=128, experts=4, top_k=2, inter=64, shared_inter=64)
SMALL6 = MoEConfig("small6", tokens=2, hidden=256, experts=4, top_k=2, inter=128, fmt=E2M3)


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(40.0) == 40.0 / (1 + math.exp(-40.0))
    assert abs(oracle.silu(40.0) - 40.0) < 1e-15
    s = oracle.silu(-800.0)
    assert s == 0.0 and math.copysign(1, s) == -1.0   # -800 / inf -> -0
    for z in (-3.0, -0.5, 0.7, 2.0):
        assert abs(oracle.silu(z) - z * expit(z)) < 1e-15


def _decoded_expert(cfg, ew, I):
    H, f = cfg.hidden, cfg.fmt
    W13 = oracle.decode(f, 2 * I, H, ew["w13_codes"], ew["w13_scales"])
    W2 = oracle.decode(f, H, I, ew["w2_codes"], ew["w2_scales"])
    return W13[:I], W13[I:], W2


@pytest.mark.parametrize("cfg", [SMALL, SMALL6], ids=lambda c: c.name)
def test_ffn_against_library_matmul(cfg):
    H, I = cfg.hidden, cfg.inter
    x = synth.hidden_states(cfg)
    for e in range(cfg.experts):
        ew = synth.expert_weights(cfg, e)
        Wg, Wu, Wd = _decoded_expert(cfg, ew, I)
        xf = np.array([oracle.bf16_value(int(b)) for b in x[0]])
        g, u = Wg @ xf, Wu @ xf
        h_ref = g * expit(g) * u
        y_ref = Wd @ h_ref
        y, h = oracle.ffn(cfg.fmt, H, I, ew, x[0], return_h=True)
        assert np.allclose(h, h_ref, rtol=1e-12, atol=1e-12 * np.abs(h_ref).max())
        assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-12 * np.abs(y_ref).max())
        rows = np.array([3, 0, H - 1])
        ys = oracle.ffn(cfg.fmt, H, I, ew, x[0], out_rows=rows)
        assert np.array_equal(ys, y[rows])


def test_zero_gate_or_zero_up_gives_exact_zero():
    cfg = SMALL
    H, I = cfg.hidden, cfg.inter
    x = synth.hidden_states(cfg)[0]
    ew = synth.expert_weights(cfg, 1)
    for half in (0, 1):                      # gate rows, then up rows
        z = {k: v.copy() for k, v in ew.items()}
        z["w13_codes"][half * I:(half + 1) * I] = 0
        y = oracle.ffn(cfg.fmt, H, I, z, x)
        assert (y == 0).all()


def _all_ffn(cfg, x_row):
    return {e: oracle.ffn(cfg.fmt, cfg.hidden, cfg.inter, synth.expert_weights(cfg, e), x_row)
            for e in range(cfg.experts)}


def test_layer_k1_is_the_selected_expert():
    cfg = SMALL
    ex = {e: synth.expert_weights(cfg, e) for e in range(cfg.experts)}
    x = synth.hidden_states(cfg)
    l = synth.router_logits(cfg)
    idx, w, out = oracle.layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, 1, ex, x, l)
    for t in range(cfg.tokens):
        assert w[t, 0] == 1.0
        y = oracle.ffn(cfg.fmt, cfg.hidden, cfg.inter, ex[idx[t, 0]], x[t])
        assert np.array_equal(out[t], y)


@pytest.mark.parametrize("cfg", [SMALL, SMALL6], ids=lambda c: c.name)
def test_layer_k_equals_E_is_the_dense_softmax_mixture(cfg):
    ex = {e: synth.expert_weights(cfg, e) for e in range(cfg.experts)}
    x = synth.hidden_states(cfg)
    l = synth.router_logits(cfg)
    _, _, out = oracle.layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.experts, ex, x, l)
    for t in range(cfg.tokens):
        p = softmax(l[t].astype(np.float64))
        ys = _all_ffn(cfg, x[t])
        ref = sum(p[e] * ys[e] for e in range(cfg.experts))
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_four_expert_brute_force_over_subsets():
    cfg = MoEConfig("four", tokens=4, hidden=128, experts=4, top_k=2, inter=64, logit_sigma=2.0)
    ex = {e: synth.expert_weights(cfg, e) for e in range(4)}
    x = synth.hidden_states(cfg)
    l = synth.router_logits(cfg)
    for t in range(cfg.tokens):
        ys = _all_ffn(cfg, x[t])
        for k in range(1, 5):
            mixes = {}
            for S in itertools.combinations(range(4), k):
                p = softmax(l[t, list(S)].astype(np.float64))
                mixes[S] = sum(pi * ys[e] for pi, e in zip(p, S))
            _, _, out = oracle.layer(cfg.fmt, 128, 64, 4, k, ex, x[t:t + 1], l[t:t + 1])
            chosen = tuple(sorted(np.argsort(-l[t].astype(np.float64), kind="stable")[:k]))
            matches = [S for S, m in mixes.items() if np.allclose(out[0], m, rtol=1e-12, atol=1e-12)]
            assert matches == [chosen]


def test_shared_expert_enters_with_weight_one():
    cfg = SMALL
    ex = {e: synth.expert_weights(cfg, e) for e in range(cfg.experts)}
    sh = synth.expert_weights(cfg, cfg.experts)
    x = synth.hidden_states(cfg)
    l = synth.router_logits(cfg)
    _, _, a = oracle.layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, 2, ex, x, l)
    _, _, b = oracle.layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, 2, ex, x, l,
                           shared=sh, shared_inter=cfg.shared_inter)
    for t in range(cfg.tokens):
        ysh = oracle.ffn(cfg.fmt, cfg.hidden, cfg.shared_inter, sh, x[t])
        assert np.allclose(b[t] - a[t], ysh, rtol=1e-12, atol=1e-12 * np.abs(ysh).max())


def test_missing_selected_expert_is_an_error():
    cfg = SMALL
    x = synth.hidden_states(cfg)
    l = synth.router_logits(cfg)
    with pytest.raises(KeyError):
        oracle.layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, 2, {}, x, l)
