"""Pins of the oracle's steps either side of the MoE layer: RMSNorm, the
router scores and the residual add, and their composition into the block.
Closed forms (one-hot rows, constant rows), exact invariants (scaling by
powers of two, unit mean square), a numpy matmul for the scores, and special
cases of the composition (all-zero experts leave the residual stream exactly;
the block minus its input is the layer on the normalised input)."""
import numpy as np
import pytest

import oracle
import synth
from synth.configs import MoEConfig

ONE = 0x3F80


def _bf(vals):
    """bf16 bits of values exactly representable in bf16."""
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_rmsnorm_one_hot_closed_form():
    """x = c e_k, eps = 0: mean square c^2/H, so y_k = sign(c) sqrt(H) g_k, the rest 0."""
    H = 256
    g = _bf(np.linspace(0.5, 2.0, H).astype(np.float32).astype(np.float64).round(3))
    gv = np.array([oracle.bf16_value(int(b)) for b in g])
    for c, k in ((4.0, 0), (-0.25, 17), (2.0 ** -10, H - 1)):
        x = np.zeros((1, H), np.uint16)
        x[0, k] = _bf([c])[0]
        y = oracle.rmsnorm(x, g, 0.0)[0]
        assert y[k] == np.sign(c) * 16.0 * gv[k]
        assert not np.delete(y, k).any()


def test_rmsnorm_constant_row_with_eps():
    H = 128
    g = np.full(H, ONE, np.uint16)
    for c, eps in ((3.0, 1e-6), (0.125, 0.5), (-2.0, 4.0)):
        x = np.full((1, H), _bf([c])[0], np.uint16)
        y = oracle.rmsnorm(x, g, eps)[0]
        assert np.allclose(y, c / np.sqrt(c * c + eps), rtol=1e-15, atol=0)


def test_rmsnorm_invariants():
    """eps = 0: scaling x by 2^p leaves y unchanged exactly; with g = 1 the mean
    square of y is 1."""
    cfg = MoEConfig("n", tokens=3, hidden=384, experts=4, top_k=2, inter=32)
    x = synth.hidden_states(cfg)
    g = np.full(cfg.hidden, ONE, np.uint16)
    y = oracle.rmsnorm(x, g, 0.0)
    assert np.allclose((y * y).mean(axis=1), 1.0, rtol=1e-14, atol=0)
    y8 = oracle.rmsnorm(x + np.uint16(3 << 7), g, 0.0)     # x * 8
    assert np.array_equal(y, y8)
    gs = synth.norm_gamma(cfg)
    yg = oracle.rmsnorm(x, gs, 0.0)
    gv = np.array([oracle.bf16_value(int(b)) for b in gs])
    assert np.allclose(yg, y * gv, rtol=1e-15, atol=0)


def test_router_scores_against_library_matmul():
    """Non-square (E != H) so a transposed operand cannot pass."""
    cfg = MoEConfig("r", tokens=5, hidden=192, experts=40, top_k=3, inter=32, logit_sigma=1.5)
    x = synth.hidden_states(cfg)
    wr = synth.router_weights(cfg)
    f = lambda a: np.array([[oracle.bf16_value(int(b)) for b in r] for r in a])
    ref = f(x) @ f(wr).T
    got = oracle.router_logits(x, wr)
    assert got.shape == (5, 40)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    oh = np.zeros((1, cfg.hidden), np.uint16)
    oh[0, 7] = ONE
    assert np.array_equal(oracle.router_logits(oh, wr)[0], f(wr)[:, 7])


def test_residual_add():
    r = _bf([1.5, -2.0, 0.0, 3.0])
    y = np.array([0.25, 0.5, -1.0, 0.0])
    assert list(oracle.residual_add(r, y)) == [1.75, -1.5, -1.0, 3.0]


BLK = MoEConfig("blk", tokens=3, hidden=256, experts=6, top_k=2, inter=64, shared_inter=64, logit_sigma=1.5)


def _experts(cfg):
    return {e: synth.expert_weights(cfg, e) for e in range(cfg.experts)}, synth.expert_weights(cfg, cfg.experts)


def test_block_with_zero_experts_is_the_residual():
    cfg = BLK
    ex, sh = _experts(cfg)
    zero = lambda w: {k: (np.zeros_like(v) if k.endswith("codes") else v) for k, v in w.items()}
    ex = {e: zero(w) for e, w in ex.items()}
    x = synth.hidden_states(cfg)
    _, _, out, _, _ = oracle.block(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, ex, x,
                                   synth.norm_gamma(cfg), synth.router_weights(cfg), cfg.norm_eps, shared=zero(sh),
                                   shared_inter=cfg.shared_inter)
    assert np.array_equal(out, np.array([[oracle.bf16_value(int(b)) for b in r] for r in x]))


def test_block_is_norm_then_scores_then_layer_then_residual():
    cfg = BLK
    ex, sh = _experts(cfg)
    x = synth.hidden_states(cfg)
    g, wr = synth.norm_gamma(cfg), synth.router_weights(cfg)
    idx, w, out, xn, lg = oracle.block(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, ex, x, g, wr,
                                       cfg.norm_eps, shared=sh, shared_inter=cfg.shared_inter)
    # the normalised input is the bf16 rounding of the norm; the scores a numpy matmul of it
    assert np.array_equal(xn, oracle.bf16_round(oracle.rmsnorm(x, g, cfg.norm_eps)))
    f = lambda a: np.array([[oracle.bf16_value(int(b)) for b in r] for r in a])
    assert np.allclose(lg, f(xn) @ f(wr).T, rtol=1e-13, atol=1e-13 * np.abs(lg).max())
    # k = E: the layer is the dense softmax mixture, plus the shared expert and the residual
    ide, we, oute, _, _ = oracle.block(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.experts, ex, x, g, wr,
                                       cfg.norm_eps, shared=sh, shared_inter=cfg.shared_inter)
    lg32 = lg.astype(np.float32).astype(np.float64)
    for t in range(cfg.tokens):
        p = np.exp(lg32[t] - lg32[t].max())
        p /= p.sum()
        dense = sum(p[e] * oracle.ffn(cfg.fmt, cfg.hidden, cfg.inter, ex[e], xn[t]) for e in range(cfg.experts))
        dense += oracle.ffn(cfg.fmt, cfg.hidden, cfg.shared_inter, sh, xn[t])
        ref = f(x[t:t + 1])[0] + dense
        assert np.allclose(oute[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
