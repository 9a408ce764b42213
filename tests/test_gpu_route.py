"""moe_route_topk against the oracle: indices bit-exact (ties to the lower
index, +-0 equal, NaN last), weights within 1e-6 relative and summing to 1."""
import itertools

import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import oracle
import synth
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def _check(l, k):
    idx, w = moeq.moe_route_topk(torch.from_numpy(np.ascontiguousarray(l)).cuda(), k)
    ridx, rw = oracle.route(l, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    wg = w.cpu().numpy().astype(np.float64)
    assert np.allclose(wg, rw, rtol=1e-6, atol=0)
    assert np.all(np.abs(wg.sum(1) - 1.0) <= 4 * 2.0 ** -24 * k)


@pytest.mark.parametrize("T,E,k,sigma", [(1, 8, 2, 1.0), (1, 512, 10, 1.5), (16, 288, 8, 1.0), (2048, 512, 10, 1.0),
                                         (7, 1000, 32, 1.0), (5, 64, 1, 1.0), (3, 33, 33 - 1, 1.0), (4, 1024, 17, 3.0)])
def test_route_random(T, E, k, sigma):
    require_gpu()
    l = synth.normal_f32(5, synth.stream_id(synth.K_LOGITS, E * 1000 + T), T * E, sigma).reshape(T, E)
    _check(l, k)


def test_route_every_tie_pattern_small():
    require_gpu()
    E = 6
    pats = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=E)), np.float32)
    for k in range(1, E + 1):
        _check(pats, k)


def test_route_signed_zero_nan_and_coarse_ties():
    require_gpu()
    l = np.array([[-0.0, 0.0, np.nan, -np.inf, -0.0, 1.0, np.nan, 0.5]], np.float32)
    idx, _ = moeq.moe_route_topk(torch.from_numpy(l).cuda(), 8)
    assert list(idx.cpu().numpy()[0]) == [5, 7, 0, 1, 4, 3, 2, 6]
    # many exact ties among 512 logits rounded to a coarse grid
    l = np.round(synth.normal_f32(1, 99, 64 * 512).reshape(64, 512) * 2) / 2
    _check(l.astype(np.float32), 10)
