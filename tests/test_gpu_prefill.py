"""The many-token path (T > 16: route, group, MFMA gate/up and down, combine)
against the oracle: several tiles with ragged tails in H, I and the shared
expert's width, both formats, experts with no tokens and with more tokens
than one block holds, fixed-expert calls, chunking past 2,048 tokens, and the
full-size 2,048-token workload on sampled tokens; the down projection with
the block's h resident in LDS for every weight format, and its persistent
grid over runs of passes; the widest routing (1,024 experts + shared, top-32);
top-1 (bitwise the expert's FFN) and top-E (the dense mixture)."""
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

# H = 512: 4 K steps; I = 256: 4 gate/up tiles
PF_SMALL = MoEConfig("pf_small", tokens=100, hidden=512, experts=16, top_k=4, inter=256)
# H = 256 (2 down tiles), I = 96 (ragged K step and gate/up tile), Ish = 160 > I
PF_SHARED = MoEConfig("pf_shared", tokens=77, hidden=256, experts=24, top_k=5, inter=96, shared_inter=160)
# e2m3 with UE8M0/128; Ish < I
PF_E2M3 = MoEConfig("pf_e2m3", tokens=90, hidden=384, experts=12, top_k=3, inter=256, shared_inter=128, fmt=2)
# more than one chunk of 2,048 tokens
PF_CHUNKED = MoEConfig("pf_chunked", tokens=2085, hidden=256, experts=8, top_k=2, inter=128, shared_inter=64)
CFGS = [PF_SMALL, PF_SHARED, PF_E2M3]
# down with the block's h resident in LDS: I = 512 (four K steps a pass, routed
# experts) and Ish = 384 (three), H = 768 (three passes of 256 rows), experts
# with two blocks (up to 64 tokens and a ragged rest), every weight format
PF_RES = [MoEConfig("pf_res_f%d" % f, tokens=150, hidden=768, experts=6, top_k=2, inter=512, shared_inter=384,
                    fmt=f) for f in (1, 2, 3, 4, 5)]
# the resident down projection's persistent grid: more passes (blocks x
# ceil(H / 256)) than CUs, so workgroups take runs of passes that start inside
# a block and cross into the next; H = 1152 ends in a half-empty pass
PF_RES_WIDE = MoEConfig("pf_res_wide", tokens=1024, hidden=1152, experts=8, top_k=4, inter=256, shared_inter=256)
# the largest routing the C ABI takes: 1,024 experts plus the shared one (1,025
# slots, so the plan builder's threads take two slots each) and top-32
PF_WIDEST = MoEConfig("pf_widest", tokens=96, hidden=256, experts=1024, top_k=32, inter=256, shared_inter=256)
# the degenerate routings on the many-token path: top-1 and top-E
PF_DEG = MoEConfig("pf_deg", tokens=40, hidden=256, experts=8, top_k=8, inter=256)
_layers = {}


def _layer(cfg):
    if cfg.name not in _layers:
        _layers[cfg.name] = upload_layer(cfg)
    return _layers[cfg.name]


def _run(cfg, x, l, flags=0, ws=None):
    L = _layer(cfg)
    T = x.shape[0]
    ws = ws if ws is not None else moeq.workspace(L, T)
    xd, ld = dev_bf16(x), torch.from_numpy(np.ascontiguousarray(l)).cuda()
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    out32 = moeq.moe_layer_decode(L, xd, ld, idx_out=idx, w_out=w, flags=F32 | flags, ws=ws)
    out16 = moeq.moe_layer_decode(L, xd, ld, flags=flags, ws=ws)
    moeq.moe_workspace_status(ws)
    return idx.cpu().numpy(), w.cpu().numpy(), out32, out16


def _check(cfg, x, l, idx, w, out32, out16):
    ridx, rw, ref = oracle_layer(cfg, x, l)
    assert np.array_equal(idx, ridx)
    assert np.allclose(w, rw, rtol=1e-6, atol=0)
    err = max_rel_err(out32.cpu().numpy(), ref)
    assert err <= PARITY_TOL, err
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_prefill_parity(cfg):
    require_gpu()
    print("prefill parity", cfg.name, flush=True)
    x, l = synth.hidden_states(cfg), synth.router_logits(cfg)
    _check(cfg, x, l, *_run(cfg, x, l))


@pytest.mark.parametrize("cfg", PF_RES, ids=lambda c: c.name)
def test_prefill_resident_down(cfg):
    require_gpu()
    print("prefill resident down", cfg.name, flush=True)
    x, l = synth.hidden_states(cfg), synth.router_logits(cfg)
    _check(cfg, x, l, *_run(cfg, x, l))


def test_prefill_resident_down_runs_of_passes():
    """About 85 blocks of 5 passes each, shared out over the CUs: every
    token's output against the oracle on 128 tokens spread over the call
    (each block holds tokens among them), the bf16 output bit for bit."""
    require_gpu()
    cfg = PF_RES_WIDE
    print("prefill resident down, runs of passes", flush=True)
    x, l = synth.hidden_states(cfg, sub=41), synth.router_logits(cfg, sub=41)
    idx, w, out32, out16 = _run(cfg, x, l)
    rows = np.arange(3, cfg.tokens, 8)
    ridx, rw, ref = oracle_layer(cfg, x[rows], l[rows])
    assert np.array_equal(idx[rows], ridx)
    assert np.allclose(w[rows], rw, rtol=1e-6, atol=0)
    assert max_rel_err(out32.cpu().numpy()[rows], ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))


def test_prefill_widest_routing():
    """1,024 routed experts, most of them with a few tokens or none, top-32,
    and the shared expert: every token against the oracle."""
    require_gpu()
    cfg = PF_WIDEST
    print("prefill widest routing", flush=True)
    x, l = synth.hidden_states(cfg, sub=43), synth.router_logits(cfg, sub=43)
    _check(cfg, x, l, *_run(cfg, x, l))


def test_prefill_top1_equals_expert_ffn_bitwise():
    """k = 1: each token's output is its expert's FFN (weight exactly 1), the
    same bits as that expert run over all 40 tokens on the same path (a
    token's row is multiplied the same way whatever block it sits in)."""
    require_gpu()
    cfg = PF_DEG
    L1 = _layer(cfg).with_top_k(1)
    x, l = synth.hidden_states(cfg, sub=45), synth.router_logits(cfg, sub=45)
    xd, ld = dev_bf16(x), torch.from_numpy(np.ascontiguousarray(l)).cuda()
    idx = torch.empty((cfg.tokens, 1), dtype=torch.int32, device="cuda")
    out = moeq.moe_layer_decode(L1, xd, ld, idx_out=idx, flags=F32)
    ie = idx.cpu().numpy()[:, 0]
    assert np.array_equal(ie, oracle.route(l, 1)[0][:, 0])
    for e in np.unique(ie):
        y = moeq.moe_expert_ffn_q(L1, int(e), xd, flags=F32)
        rows = torch.from_numpy(np.nonzero(ie == e)[0]).cuda()
        assert torch.equal(y[rows], out[rows]), int(e)


def test_prefill_top_e_is_the_dense_mixture():
    """k = E: every expert serves every token, weights the softmax over all."""
    require_gpu()
    cfg = PF_DEG
    x, l = synth.hidden_states(cfg, sub=46), synth.router_logits(cfg, sub=46)
    _check(cfg, x, l, *_run(cfg, x, l))


@pytest.mark.parametrize("E", [100, 200])
def test_prefill_expert_counts(E):
    """Expert counts that take the routing's two- and four-logits-per-lane
    instances (65..128 and 129..256 experts) in the route+group launch."""
    require_gpu()
    cfg = MoEConfig("pf_e%d" % E, tokens=70, hidden=256, experts=E, top_k=6, inter=128, shared_inter=64)
    x, l = synth.hidden_states(cfg, sub=47), synth.router_logits(cfg, sub=47)
    _check(cfg, x, l, *_run(cfg, x, l))


@pytest.mark.parametrize("T", [17, 64, 65, 130])
def test_prefill_token_counts(T):
    require_gpu()
    cfg = PF_SHARED
    print("prefill T", T, flush=True)
    x, l = synth.hidden_states(cfg, tokens=T, sub=T), synth.router_logits(cfg, tokens=T, sub=T)
    _check(cfg, x, l, *_run(cfg, x, l))


def test_prefill_skewed_routing():
    """Every token picks expert 3 (3 full blocks + a partial one) and expert
    5 gets nothing: blocks of one expert and empty experts."""
    require_gpu()
    cfg = PF_SMALL
    T = 200
    x = synth.hidden_states(cfg, tokens=T, sub=3)
    l = synth.router_logits(cfg, tokens=T, sub=3).copy()
    l[:, 3] += 8.0
    l[:, 5] -= 8.0
    idx, w, out32, out16 = _run(cfg, x, l)
    assert (idx[:, 0] == 3).all() and not (idx == 5).any()
    _check(cfg, x, l, idx, w, out32, out16)


def test_prefill_deterministic_and_token_independent():
    """Two calls agree bitwise, and a token's output does not depend on which
    other tokens share its call (the first 40 tokens alone vs inside 100)."""
    require_gpu()
    cfg = PF_SMALL
    x, l = synth.hidden_states(cfg, tokens=100, sub=9), synth.router_logits(cfg, tokens=100, sub=9)
    _, _, a32, _ = _run(cfg, x, l)
    _, _, b32, _ = _run(cfg, x, l)
    assert torch.equal(a32, b32)
    _, _, c32, _ = _run(cfg, x[:40], l[:40])
    assert torch.equal(a32[:40], c32)


@pytest.mark.parametrize("cfg", [PF_SHARED, PF_E2M3], ids=lambda c: c.name)
def test_prefill_expert_ffn(cfg):
    """moe_expert_ffn_q with M > 16: one expert (or the shared one) on every row."""
    require_gpu()
    L = _layer(cfg)
    M = 70
    x = synth.hidden_states(cfg, tokens=M, sub=11)
    xd = dev_bf16(x)
    for e in [0, cfg.experts - 1, -1]:
        y32 = moeq.moe_expert_ffn_q(L, e, xd, flags=F32)
        y16 = moeq.moe_expert_ffn_q(L, e, xd)
        ee = cfg.experts if e < 0 else e
        I = cfg.shared_inter if e < 0 else cfg.inter
        ew = synth.expert_weights(cfg, ee)
        ref = np.stack([oracle.ffn(cfg.fmt, cfg.hidden, I, ew, x[m]) for m in range(M)])
        assert max_rel_err(y32.cpu().numpy(), ref) <= PARITY_TOL, e
        assert np.array_equal(host_bf16(y16), bf16_rne_of_f32(y32))


def test_prefill_chunked():
    """2,085 tokens: one chunk of 2,048 and a tail of 37, on one workspace."""
    require_gpu()
    cfg = PF_CHUNKED
    x, l = synth.hidden_states(cfg), synth.router_logits(cfg)
    _check(cfg, x, l, *_run(cfg, x, l))


def test_prefill_full_size_sampled():
    """The 2,048-token, 512-expert top-10 layer in the bench's launch
    configuration; the oracle checks 12 tokens spread over the chunk."""
    require_gpu()
    cfg = configs.PREFILL
    print("prefill full size", flush=True)
    L = upload_layer(cfg)
    x, l = synth.hidden_states(cfg), synth.router_logits(cfg)
    ws = moeq.workspace(L, cfg.tokens)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    idx = torch.empty((cfg.tokens, cfg.top_k), dtype=torch.int32, device="cuda")
    out32 = moeq.moe_layer_decode(L, xd, ld, idx_out=idx, flags=F32, ws=ws)
    out16 = moeq.moe_layer_decode(L, xd, ld, ws=ws)
    moeq.moe_workspace_status(ws)
    rows = np.array([0, 1, 63, 64, 500, 1023, 1024, 1500, 2000, 2045, 2046, 2047])
    ridx, _, ref = oracle_layer(cfg, x[rows], l[rows])
    assert np.array_equal(idx.cpu().numpy()[rows], ridx)
    assert max_rel_err(out32.cpu().numpy()[rows], ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))
    # every token was routed exactly as the oracle routes it
    full_idx, _ = oracle.route(l, cfg.top_k)
    assert np.array_equal(idx.cpu().numpy(), full_idx)


def test_one_workspace_for_both_paths():
    """Many-token and decode calls alternate on one workspace (sized for the
    many-token call) and each still matches the oracle."""
    require_gpu()
    cfg = PF_SHARED
    L = _layer(cfg)
    ws = moeq.workspace(L, 100)
    for T, sub in [(100, 21), (1, 22), (4, 23), (100, 24), (1, 25)]:
        print("mixed workspace T", T, flush=True)
        x, l = synth.hidden_states(cfg, tokens=T, sub=sub), synth.router_logits(cfg, tokens=T, sub=sub)
        _check(cfg, x, l, *_run(cfg, x, l, ws=ws))


@pytest.mark.parametrize("cfg", [PF_SHARED, PF_CHUNKED], ids=lambda c: c.name)
def test_prefill_claim_words_back_at_zero(cfg):
    """Routed calls group their tokens through per-slot claim words in the
    workspace header (places in the expert lists follow the order the claims
    arrive in); after every call, single chunk or several, the last workgroup
    has reset them and the arrival counter, so consecutive calls on one
    workspace agree bitwise and the status stays clean."""
    require_gpu()
    L = _layer(cfg)
    T = cfg.tokens
    ws = moeq.workspace(L, T)
    x, l = synth.hidden_states(cfg, tokens=T, sub=31), synth.router_logits(cfg, tokens=T, sub=31)
    outs = []
    for _ in range(3):
        _, _, o32, _ = _run(cfg, x, l, ws=ws)
        hdr = ws[:16384].view(torch.int32).cpu().numpy()
        ns = cfg.experts + (1 if cfg.shared_inter else 0)
        assert not hdr[2048:2048 + ns].any() and hdr[4] == 0
        assert moeq.moe_workspace_status(ws) == moeq.MOE_OK
        outs.append(o32)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
