"""The steps either side of the layer on the GPU: RMSNorm, the router scores
with their fused top-k, and the whole block (norm -> scores -> layer ->
residual add), against the oracle, also with the activations quantised to MX
e4m3 on MXFP4 experts.

Where floating point decides an integer -- the bf16 rounding of the
normalised activation, and which experts the scores select -- the GPU decides
in fp32 and the oracle in double.  So: the fp32 values are compared within a
tolerance; the GPU's bf16 rounding is checked bit for bit against its own fp32
value, and against the oracle's rounding up to one bf16 unit where the two
sides fall on either side of a rounding boundary; the GPU's top-k is checked
bit for bit against the oracle's ranking of the GPU's own scores; and the
oracle's selection is required to agree wherever the gap between the k-th and
(k+1)-th score is larger than the scores' error bound."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import oracle
import synth
import synth.device
from gpu_util import bf16_rne_of_f32, dev_bf16, host_bf16, oracle_layer, require_gpu, upload_layer
from helpers import PARITY_TOL, max_rel_err
from synth import configs
from synth.configs import MoEConfig

pytestmark = pytest.mark.gpu
F32 = moeq.MOE_OUT_F32


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("T,H", [(1, 32), (5, 2048), (16, 6144), (100, 1056), (3, 8192)])
def test_rmsnorm(T, H):
    require_gpu()
    cfg = MoEConfig("rn", tokens=T, hidden=H, experts=4, top_k=2, inter=32)
    x = synth.hidden_states(cfg, sub=H)
    g = synth.norm_gamma(cfg)
    xd, gd = dev_bf16(x), dev_bf16(g)
    y32 = moeq.moe_rmsnorm(xd, gd, 1e-6, flags=F32).cpu().numpy()
    y16 = moeq.moe_rmsnorm(xd, gd, 1e-6)
    ref = oracle.rmsnorm(x, g, 1e-6)
    assert np.max(np.abs(y32 - ref) / np.maximum(np.abs(ref), 1e-30)) <= 2e-6
    bits = host_bf16(y16)
    assert np.array_equal(bits, bf16_rne_of_f32(torch.from_numpy(y32)))
    rb = oracle.bf16_round(ref)
    diff = bits.astype(np.int64) - rb.astype(np.int64)
    assert np.abs(diff).max() <= 1 and (diff != 0).mean() < 1e-3


def _route_margin_ok(lg, k, tol):
    """Whether every token's k-th and (k+1)-th scores are further apart than tol."""
    if k >= lg.shape[1]:
        return True
    s = -np.sort(-lg, axis=1)
    return bool(np.all(s[:, k - 1] - s[:, k] > tol))


@pytest.mark.parametrize("T,H,E,k", [(1, 2048, 512, 10), (3, 256, 8, 2), (16, 6144, 288, 8), (16, 1024, 1000, 32),
                                     (40, 512, 64, 6)])
def test_router_scores_and_topk(T, H, E, k):
    require_gpu()
    cfg = MoEConfig("rt", tokens=T, hidden=H, experts=E, top_k=k, inter=32, logit_sigma=1.5)
    x = synth.hidden_states(cfg, sub=E)
    wr = synth.router_weights(cfg)
    lg, idx, w = moeq.moe_router_topk_scores(dev_bf16(x), dev_bf16(wr), k)
    lg, idx, w = lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    ref = oracle.router_logits(x, wr)
    tol = 1e-5 * np.abs(ref).max()
    assert np.max(np.abs(lg - ref)) <= tol
    # the top-k of the GPU's own scores, bit for bit
    gi, gw = oracle.route(lg, k)
    assert np.array_equal(idx, gi)
    assert np.allclose(w, gw, rtol=1e-6, atol=0)
    # and the oracle's selection wherever the scores leave no doubt
    if _route_margin_ok(ref, k, 2 * tol):
        assert np.array_equal(idx, oracle.route(ref.astype(np.float32), k)[0])


BLK = {
    "small": MoEConfig("blk_small", tokens=16, hidden=1024, experts=48, top_k=6, inter=256, shared_inter=256,
                       logit_sigma=1.5),
    "e2m3": MoEConfig("blk_e2m3", tokens=16, hidden=768, experts=20, top_k=4, inter=384, shared_inter=128, fmt=2,
                      logit_sigma=1.5),
}
_blocks = {}


def _block(cfg):
    if cfg.name not in _blocks:
        L = upload_layer(cfg)
        _blocks[cfg.name] = moeq.Block(L, dev_bf16(synth.norm_gamma(cfg)), dev_bf16(synth.router_weights(cfg)),
                                       cfg.norm_eps)
    return _blocks[cfg.name]


def _oracle_block(cfg, x, out_rows=None):
    xn = oracle.bf16_round(oracle.rmsnorm(x, synth.norm_gamma(cfg), cfg.norm_eps))
    lg = oracle.router_logits(xn, synth.router_weights(cfg))
    idx, _ = oracle.route(lg.astype(np.float32), cfg.top_k)
    ex = {int(e): synth.expert_weights(cfg, int(e)) for e in np.unique(idx)}
    sh = synth.expert_weights(cfg, cfg.experts) if cfg.shared_inter else None
    return oracle.block(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, ex, x, synth.norm_gamma(cfg),
                        synth.router_weights(cfg), cfg.norm_eps, shared=sh, shared_inter=cfg.shared_inter,
                        out_rows=out_rows)


def _check_block(cfg, B, x, out_rows=None, ws=None):
    T = x.shape[0]
    xd = dev_bf16(x)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    ws = moeq.block_workspace(B, T) if ws is None else ws
    out32 = moeq.moe_block_decode(B, xd, idx_out=idx, flags=F32, ws=ws)
    out16 = moeq.moe_block_decode(B, xd, ws=ws)
    moeq.moe_workspace_status(ws)
    ridx, _, ref, _, rlg = _oracle_block(cfg, x, out_rows)
    assert _route_margin_ok(rlg, cfg.top_k, 1e-5 * np.abs(rlg).max()), "seeded scores too close to call"
    assert np.array_equal(idx.cpu().numpy(), ridx)
    got = out32.cpu().numpy()
    got = got if out_rows is None else got[:, out_rows]
    assert max_rel_err(got, ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))
    return out32


@pytest.mark.parametrize("name", sorted(BLK))
@pytest.mark.parametrize("T", [1, 2, 7, 16, 40])
def test_block_parity(name, T):
    """T = 40 takes the many-token path for the layer."""
    require_gpu()
    cfg = BLK[name]
    _check_block(cfg, _block(cfg), synth.hidden_states(cfg, tokens=T, sub=50 + T))


def test_block_with_zero_experts_returns_the_residual_stream():
    require_gpu()
    cfg = MoEConfig("blk_zero", tokens=4, hidden=512, experts=8, top_k=2, inter=128, shared_inter=64)
    devs, shared = synth.device.upload_layer_tensors(cfg)
    for d in (devs, shared):
        d["w13_codes"].zero_()
        d["w2_codes"].zero_()
    L = moeq.Layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, devs["w13_codes"], devs["w13_scales"],
                   devs["w2_codes"], devs["w2_scales"], shared_inter=cfg.shared_inter, shared=shared)
    B = moeq.Block(L, dev_bf16(synth.norm_gamma(cfg)), dev_bf16(synth.router_weights(cfg)), cfg.norm_eps)
    for T in (1, 4, 33):
        x = synth.hidden_states(cfg, tokens=T, sub=T)
        out = moeq.moe_block_decode(B, dev_bf16(x))
        assert np.array_equal(host_bf16(out), x)


@pytest.mark.parametrize("cfg", [configs.WIDE_BLOCK, configs.BATCHED_BLOCK], ids=lambda c: c.name)
def test_full_size_block(cfg):
    """The full-size blocks (sampled output rows for the 16-token one), eagerly
    and replayed from a graph."""
    require_gpu()
    L = upload_layer(cfg)
    B = moeq.Block(L, dev_bf16(synth.norm_gamma(cfg)), dev_bf16(synth.router_weights(cfg)), cfg.norm_eps)
    rows = None if cfg.tokens == 1 else np.unique(np.concatenate([np.arange(0, cfg.hidden, 61), [cfg.hidden - 1]]))
    x = synth.hidden_states(cfg)
    ws = moeq.block_workspace(B, cfg.tokens)
    eager = _check_block(cfg, B, x, out_rows=rows, ws=ws)
    xd = dev_bf16(x)
    o = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            moeq.moe_block_decode(B, xd, out=o, flags=F32, ws=ws)
    torch.cuda.synchronize()
    for _ in range(2):
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager)


# MXFP4 experts with quantised activations through the block call (the
# quantiser takes the normalised rows; the residual is the raw stream)
BLK_MX = MoEConfig("blk_mx", tokens=16, hidden=1024, experts=24, top_k=4, inter=256, shared_inter=128, fmt=3,
                   ue8m0_exp=(-6, -2), logit_sigma=1.5)


@pytest.mark.parametrize("T", [1, 16, 40])
def test_block_with_quantised_activations(T):
    """moe_block_decode with MOE_ACT_MXFP8 against the oracle: the norm's output
    taken from moe_rmsnorm (the kernel the block runs, so bitwise its rows),
    the scores and ranking in double from those rows, the experts on the
    activations quantised to MX e4m3 and dequantised, plus the residual."""
    require_gpu()
    cfg = BLK_MX
    B = _block(cfg)
    x = synth.hidden_states(cfg, tokens=T, sub=60 + T)
    xd = dev_bf16(x)
    ws = moeq.block_workspace(B, T)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    mx = moeq.MOE_ACT_MXFP8
    out32 = moeq.moe_block_decode(B, xd, idx_out=idx, flags=F32 | mx, ws=ws)
    out16 = moeq.moe_block_decode(B, xd, flags=mx, ws=ws)
    moeq.moe_workspace_status(ws)
    xn = host_bf16(moeq.moe_rmsnorm(xd, dev_bf16(synth.norm_gamma(cfg)), cfg.norm_eps))
    lg = oracle.router_logits(xn, synth.router_weights(cfg))
    assert _route_margin_ok(lg, cfg.top_k, 1e-5 * np.abs(lg).max()), "seeded scores too close to call"
    c, s = oracle.quantize_mx_e4m3(xn)
    xq = oracle.bf16_round(oracle.dequantize_mx_e4m3(c, s))
    ridx, _, ref = oracle_layer(cfg, xq, lg.astype(np.float32))
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ref = ref + _bf16_to_f64(x)
    assert max_rel_err(out32.cpu().numpy(), ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))
