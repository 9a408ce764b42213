"""moe_expert_ffn_q and moe_layer_decode against the oracle, plus the
exactness invariants: a token alone equals the same token inside a batch,
two runs are bitwise equal, both decoders agree bitwise, top-1 routing equals
the picked expert's FFN bitwise, bf16 output is the RNE of the fp32 output,
and the bounded-wait expiry path reports MOE_EKERNEL."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import oracle
import synth
from gpu_util import bf16_rne_of_f32, dev_bf16, host_bf16, oracle_layer, require_gpu, upload_layer
from helpers import PARITY_TOL, max_rel_err
from synth import configs
from synth.configs import MoEConfig

pytestmark = pytest.mark.gpu
F32 = moeq.MOE_OUT_F32
DECS = [moeq.MOE_DECODER_LUT, moeq.MOE_DECODER_HW]

SMALL = MoEConfig("gpu_small", tokens=16, hidden=512, experts=64, top_k=6, inter=256, shared_inter=256)
SMALL6 = MoEConfig("gpu_small6", tokens=5, hidden=1024, experts=16, top_k=4, inter=384, shared_inter=128, fmt=2)
RAGGED = MoEConfig("gpu_ragged", tokens=9, hidden=1056, experts=40, top_k=3, inter=96, shared_inter=160)
CFGS = [configs.TOY, SMALL, SMALL6, RAGGED]
_layers = {}


def _layer(cfg):
    if cfg.name not in _layers:
        _layers[cfg.name] = upload_layer(cfg)
    return _layers[cfg.name]


def _inputs(cfg, T, sub=0):
    x = synth.hidden_states(cfg, tokens=T, sub=sub)
    l = synth.router_logits(cfg, tokens=T, sub=sub)
    return x, l


@pytest.mark.parametrize("dec", DECS, ids=["lut", "hw"])
@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
@pytest.mark.parametrize("M", [1, 3, 16])
def test_expert_ffn_parity(cfg, M, dec):
    require_gpu()
    L = _layer(cfg)
    x = synth.hidden_states(cfg, tokens=M, sub=7)
    xd = dev_bf16(x)
    experts = [0, cfg.experts - 1] + ([-1] if cfg.shared_inter else [])
    for e in experts:
        y32 = moeq.moe_expert_ffn_q(L, e, xd, flags=F32 | dec).cpu().numpy()
        y16 = moeq.moe_expert_ffn_q(L, e, xd, flags=dec)
        ee = cfg.experts if e < 0 else e
        I = cfg.shared_inter if e < 0 else cfg.inter
        ew = synth.expert_weights(cfg, ee)
        ref = np.stack([oracle.ffn(cfg.fmt, cfg.hidden, I, ew, x[m]) for m in range(M)])
        assert max_rel_err(y32, ref) <= PARITY_TOL, (e, max_rel_err(y32, ref))
        y32t = moeq.moe_expert_ffn_q(L, e, xd, flags=F32 | dec)
        assert np.array_equal(host_bf16(y16), bf16_rne_of_f32(y32t))


@pytest.mark.parametrize("dec", DECS, ids=["lut", "hw"])
@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
@pytest.mark.parametrize("T", [1, 2, 7, 16])
def test_layer_parity(cfg, T, dec):
    require_gpu()
    L = _layer(cfg)
    x, l = _inputs(cfg, T, sub=T)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    ws = moeq.workspace(L, T)
    out32 = moeq.moe_layer_decode(L, xd, ld, idx_out=idx, w_out=w, flags=F32 | dec, ws=ws)
    out16 = moeq.moe_layer_decode(L, xd, ld, flags=dec, ws=ws)
    ridx, rw, ref = oracle_layer(cfg, x, l)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)
    err = max_rel_err(out32.cpu().numpy(), ref)
    assert err <= PARITY_TOL, err
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))
    moeq.moe_workspace_status(ws)


@pytest.mark.parametrize("cfg", [SMALL, RAGGED], ids=lambda c: c.name)
def test_batch_invariance_and_determinism(cfg):
    """Each row of a 16-token call equals the same row decoded alone, bit for
    bit; repeated calls and the two decoders agree bit for bit."""
    require_gpu()
    L = _layer(cfg)
    x, l = _inputs(cfg, 16, sub=3)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    ws = moeq.workspace(L, 16)
    full = moeq.moe_layer_decode(L, xd, ld, flags=F32 | moeq.MOE_DECODER_LUT, ws=ws)
    again = moeq.moe_layer_decode(L, xd, ld, flags=F32 | moeq.MOE_DECODER_LUT, ws=ws)
    hw = moeq.moe_layer_decode(L, xd, ld, flags=F32 | moeq.MOE_DECODER_HW, ws=ws)
    assert torch.equal(full, again) and torch.equal(full, hw)
    for t in range(16):
        one = moeq.moe_layer_decode(L, xd[t:t + 1].contiguous(), ld[t:t + 1].contiguous(), flags=F32, ws=ws)
        assert torch.equal(one[0], full[t]), t
    for T in (3, 8):
        part = moeq.moe_layer_decode(L, xd[:T].contiguous(), ld[:T].contiguous(), flags=F32, ws=ws)
        assert torch.equal(part, full[:T])


def test_top1_equals_expert_ffn_bitwise():
    require_gpu()
    cfg = SMALL
    L1 = _layer(cfg).with_top_k(1)
    x, l = _inputs(cfg, 16, sub=4)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    idx = torch.empty((16, 1), dtype=torch.int32, device="cuda")
    # no shared expert in this comparison: build a descriptor without it
    L1.c.shared_inter = 0
    out = moeq.moe_layer_decode(L1, xd, ld, idx_out=idx, flags=F32)
    for t, e in enumerate(idx.cpu().numpy()[:, 0]):
        y = moeq.moe_expert_ffn_q(L1, int(e), xd[t:t + 1].contiguous(), flags=F32)
        assert torch.equal(y[0], out[t]), t


def test_k_equals_E_is_the_dense_mixture():
    require_gpu()
    cfg = MoEConfig("gpu_dense_mix", tokens=4, hidden=256, experts=8, top_k=8, inter=128)
    L = _layer(cfg)
    x, l = _inputs(cfg, 4)
    out = moeq.moe_layer_decode(L, dev_bf16(x), torch.from_numpy(l).cuda(), flags=F32).cpu().numpy()
    from scipy.special import softmax
    ys = {e: np.stack([oracle.ffn(cfg.fmt, 256, 128, synth.expert_weights(cfg, e), x[t]) for t in range(4)])
          for e in range(8)}
    ref = np.stack([sum(softmax(l[t].astype(np.float64))[e] * ys[e][t] for e in range(8)) for t in range(4)])
    assert max_rel_err(out, ref) <= PARITY_TOL


def test_four_experts_every_k():
    require_gpu()
    cfg = MoEConfig("gpu_four", tokens=8, hidden=256, experts=4, top_k=4, inter=64, logit_sigma=2.0)
    base = _layer(cfg)
    x, l = _inputs(cfg, 8)
    for k in range(1, 5):
        L = base.with_top_k(k)
        out = moeq.moe_layer_decode(L, dev_bf16(x), torch.from_numpy(l).cuda(), flags=F32).cpu().numpy()
        _, _, ref = oracle_layer(cfg, x, l, k=k)
        assert max_rel_err(out, ref) <= PARITY_TOL, k


def test_one_expert_takes_every_token():
    """Identical logits for all 16 tokens: every selected expert serves 16 rows."""
    require_gpu()
    cfg = SMALL
    L = _layer(cfg)
    x, l = _inputs(cfg, 16, sub=5)
    l[:] = l[0]
    out = moeq.moe_layer_decode(L, dev_bf16(x), torch.from_numpy(l).cuda(), flags=F32).cpu().numpy()
    _, _, ref = oracle_layer(cfg, x, l)
    assert max_rel_err(out, ref) <= PARITY_TOL


def test_bounded_wait_expiry_is_reported_then_recovers():
    require_gpu()
    cfg = SMALL
    L = _layer(cfg)
    x, l = _inputs(cfg, 4, sub=6)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    ws = moeq.workspace(L, 4)
    moeq.moe_layer_decode(L, xd, ld, flags=F32 | moeq.MOE_DEBUG_SPIN_LIMIT, ws=ws)
    with pytest.raises(moeq.MoeError) as ei:
        moeq.moe_workspace_status(ws)
    assert ei.value.code == moeq.MOE_EKERNEL
    assert moeq.moe_workspace_status(ws) == moeq.MOE_OK            # the read cleared it
    hdr = ws[:16384].view(torch.int32).cpu().numpy()
    hdr[3] = 0                                                    # the call counter keeps counting
    assert not hdr.any()                                          # counters back at zero
    out = moeq.moe_layer_decode(L, xd, ld, flags=F32, ws=ws).cpu().numpy()
    _, _, ref = oracle_layer(cfg, x, l)
    assert max_rel_err(out, ref) <= PARITY_TOL
    assert moeq.moe_workspace_status(ws) == moeq.MOE_OK


def test_single_token_wait_expiry_is_reported_then_recovers():
    """The one-token kernel's bounded wait (its exchange of h between
    workgroups), forced to expire by the test hook: the status call reports
    it once, and the following calls on the same workspace match the oracle."""
    require_gpu()
    cfg = SMALL
    L = _layer(cfg)
    x, l = _inputs(cfg, 1, sub=7)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    ws = moeq.workspace(L, 1)
    moeq.moe_layer_decode(L, xd, ld, flags=F32 | moeq.MOE_DEBUG_SPIN_LIMIT, ws=ws)
    with pytest.raises(moeq.MoeError) as ei:
        moeq.moe_workspace_status(ws)
    assert ei.value.code == moeq.MOE_EKERNEL
    assert moeq.moe_workspace_status(ws) == moeq.MOE_OK
    _, _, ref = oracle_layer(cfg, x, l)
    for _ in range(3):
        out = moeq.moe_layer_decode(L, xd, ld, flags=F32, ws=ws).cpu().numpy()
        assert max_rel_err(out, ref) <= PARITY_TOL
        assert moeq.moe_workspace_status(ws) == moeq.MOE_OK


ONE_TOKEN_SHAPES = [
    # e2m3, two activation units per lane (H = 384) and two h units per lane on the down side
    MoEConfig("one_e2m3", tokens=2, hidden=384, experts=12, top_k=3, inter=256, shared_inter=128, fmt=2),
    # H = 2080: 65 units per row, the last one on a second unit slot of lane 0
    MoEConfig("one_h2080", tokens=2, hidden=2080, experts=32, top_k=8, inter=256),
    # eight experts of eight: one output row per workgroup
    MoEConfig("one_k8", tokens=2, hidden=256, experts=8, top_k=8, inter=512),
    # 4,864 pairs over 256 workgroups: pair ranges straddle two experts
    MoEConfig("one_straddle", tokens=2, hidden=256, experts=16, top_k=9, inter=512, shared_inter=256),
]


@pytest.mark.parametrize("cfg", ONE_TOKEN_SHAPES, ids=lambda c: c.name)
def test_single_token_kernel_shapes(cfg):
    """Shapes that take the one-token kernel's less common paths: against the
    oracle, and bitwise equal to the same token inside a two-token call (the
    general kernel)."""
    require_gpu()
    L = _layer(cfg)
    x, l = _inputs(cfg, 2, sub=8)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    ws = moeq.workspace(L, 2)
    idx = torch.empty((1, cfg.top_k), dtype=torch.int32, device="cuda")
    one = moeq.moe_layer_decode(L, xd[:1], ld[:1], idx_out=idx, flags=F32, ws=ws)
    two = moeq.moe_layer_decode(L, xd, ld, flags=F32, ws=ws)
    moeq.moe_workspace_status(ws)
    ridx, _, ref = oracle_layer(cfg, x[:1], l[:1])
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_rel_err(one.cpu().numpy(), ref) <= PARITY_TOL
    assert torch.equal(one[0], two[0])


def test_single_token_routing_ties():
    """The one-token kernel routes by ranks of unique keys: logits on a coarse
    grid (many exact ties, and a tie across the k-th place) must still give the
    oracle's picks, ties to the lower index."""
    require_gpu()
    cfg = SMALL
    L = _layer(cfg)
    for sub in range(4):
        x, l = _inputs(cfg, 1, sub=30 + sub)
        l = (np.round(l * 2.0) / 2.0).astype(np.float32)
        xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
        idx = torch.empty((1, cfg.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((1, cfg.top_k), dtype=torch.float32, device="cuda")
        out = moeq.moe_layer_decode(L, xd, ld, idx_out=idx, w_out=w, flags=F32)
        ridx, rw, ref = oracle_layer(cfg, x, l)
        assert np.array_equal(idx.cpu().numpy(), ridx), sub
        assert np.allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)
        assert max_rel_err(out.cpu().numpy(), ref) <= PARITY_TOL


FEW_TOKEN_SHAPES = [
    # H = 8192: four activation units per lane, at most six tokens of x in LDS per batch
    MoEConfig("few_h8192", tokens=7, hidden=8192, experts=16, top_k=2, inter=256),
    # shared expert twice as wide as the routed ones: two h units per lane on the down side
    MoEConfig("few_wide_shared", tokens=5, hidden=512, experts=16, top_k=4, inter=256, shared_inter=512),
    # e2m3 on a 1536-wide layer
    MoEConfig("few_e2m3", tokens=4, hidden=1536, experts=32, top_k=4, inter=512, shared_inter=256, fmt=2),
    # top-32 of 64 with 16 tokens and a shared expert: all 528 pair positions in use
    MoEConfig("few_k32", tokens=16, hidden=256, experts=64, top_k=32, inter=128, shared_inter=128),
    # the largest expert count: sixteen logits per lane in the routing wave
    MoEConfig("few_e1024", tokens=6, hidden=256, experts=1024, top_k=10, inter=128, shared_inter=128),
]


@pytest.mark.parametrize("same_logits", [False, True], ids=["own_logits", "same_logits"])
@pytest.mark.parametrize("cfg", FEW_TOKEN_SHAPES, ids=lambda c: c.name)
def test_few_token_kernel_shapes(cfg, same_logits):
    """Shapes that take the 2-16 token kernel's less common paths (several
    token batches per group when every token picks the same experts, wide
    rows, a wide shared expert, the largest pair count): routing bit-exact and
    outputs within tolerance of the oracle, and every token bitwise equal to
    the same token decoded alone."""
    require_gpu()
    L = _layer(cfg)
    T = cfg.tokens
    x, l = _inputs(cfg, T, sub=9)
    if same_logits:
        l[:] = l[0]
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    ws = moeq.workspace(L, T)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    out = moeq.moe_layer_decode(L, xd, ld, idx_out=idx, flags=F32, ws=ws)
    ridx, _, ref = oracle_layer(cfg, x, l)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_rel_err(out.cpu().numpy(), ref) <= PARITY_TOL
    for t in (0, T - 1):
        one = moeq.moe_layer_decode(L, xd[t:t + 1], ld[t:t + 1], flags=F32, ws=ws)
        assert torch.equal(one[0], out[t]), t
    assert moeq.moe_workspace_status(ws) == moeq.MOE_OK


def test_calls_of_every_kernel_share_one_workspace():
    """Calls of 1, 3 and 16 tokens (the single-token, few-token kernels) in a
    mixed order on one workspace: every output bitwise equal to the same call
    on a fresh workspace, so the call tag one kernel leaves behind never lets
    another take a stale word as current."""
    require_gpu()
    cfg = SMALL
    L = _layer(cfg)
    x, l = _inputs(cfg, 16, sub=11)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    fresh = {}
    for T in (1, 3, 16):
        fresh[T] = moeq.moe_layer_decode(L, xd[:T], ld[:T], flags=F32, ws=moeq.workspace(L, 16))
    ws = moeq.workspace(L, 16)
    for T in (3, 1, 3, 16, 1, 16, 3, 1):
        out = moeq.moe_layer_decode(L, xd[:T], ld[:T], flags=F32, ws=ws)
        assert torch.equal(out, fresh[T]), T
    assert moeq.moe_workspace_status(ws) == moeq.MOE_OK
