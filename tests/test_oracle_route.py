"""Pins of the oracle's routing: brute force over tie patterns, +-0, NaN,
and the gate weights against a library softmax."""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth
from synth import configs


def _rule(l, k):
    """Reference order: larger logit first, equal logits by lower index, NaN last."""
    key = lambda i: (1, 0.0, i) if np.isnan(l[i]) else (0, -float(l[i]), i)
    return sorted(range(len(l)), key=key)[:k]


@pytest.mark.parametrize("E", [1, 2, 3, 4, 5, 6])
def test_every_tie_pattern(E):
    for pattern in itertools.product([0.0, 1.0, 2.0], repeat=E):
        l = np.array(pattern, np.float32)
        for k in range(1, E + 1):
            idx, w = oracle.route(l, k)
            assert list(idx[0]) == _rule(l, k), (pattern, k)
            assert abs(w.sum() - 1.0) < 1e-15
            assert len(set(idx[0])) == k


def test_signed_zero_ties_and_nan_last():
    l = np.array([-0.0, 0.0, np.nan, -np.inf, -0.0], np.float32)
    idx, _ = oracle.route(l, 5)
    assert list(idx[0]) == [0, 1, 4, 3, 2]
    l = np.array([np.nan, 1.0, np.nan, 1.0], np.float32)
    idx, _ = oracle.route(l, 4)
    assert list(idx[0]) == [1, 3, 0, 2]


def test_weights_closed_forms():
    l = synth.router_logits(configs.WIDE)
    idx, w = oracle.route(l, 1)
    assert w[0, 0] == 1.0
    idx, w = oracle.route(np.full((1, 16), 0.25, np.float32), 4)
    assert list(idx[0]) == [0, 1, 2, 3] and np.allclose(w, 0.25, rtol=0, atol=1e-16)


@pytest.mark.parametrize("cfg", [configs.TOY, configs.WIDE, configs.BATCHED, configs.PREFILL],
                         ids=lambda c: c.name)
def test_random_logits_against_stable_argsort_and_softmax(cfg):
    l = synth.router_logits(cfg)
    T = min(cfg.tokens, 64)
    l = l[:T]
    idx, w = oracle.route(l, cfg.top_k)
    ref = np.argsort(-l.astype(np.float64), axis=1, kind="stable")[:, : cfg.top_k]
    assert np.array_equal(idx, ref)
    sel = np.take_along_axis(l.astype(np.float64), ref, axis=1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-14, atol=0)
    # softmax over all E, kept and renormalised, is the same thing
    full = softmax(l.astype(np.float64), axis=1)
    kept = np.take_along_axis(full, ref, axis=1)
    assert np.allclose(w, kept / kept.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)
