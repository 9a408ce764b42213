"""Quantised activations: the MX e4m3 quantiser bit for bit against the
oracle, and the layer with MOE_ACT_MXFP8 -- on the scaled low-precision
matrix cores for the MX weight formats (many-token path), on the dequantised
values elsewhere -- against the oracle's layer on the oracle's dequantised
activations (exact in bf16 here)."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import oracle
import synth
from gpu_util import bf16_rne_of_f32, dev_bf16, host_bf16, oracle_layer, require_gpu, upload_layer
from helpers import PARITY_TOL, max_rel_err
from synth.configs import MoEConfig

pytestmark = pytest.mark.gpu
F32 = moeq.MOE_OUT_F32
MX = moeq.MOE_ACT_MXFP8


def _bf(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("T,H,sigma", [(1, 32, 1.0), (7, 2048, 1.0), (16, 6144, 3.0), (300, 512, 0.01)])
def test_quantiser_bit_exact(T, H, sigma):
    require_gpu()
    cfg = MoEConfig("aq", tokens=T, hidden=H, experts=2, top_k=1, inter=32, x_sigma=sigma)
    x = synth.hidden_states(cfg, sub=H)
    c, s = moeq.moe_quantize_mx_e4m3(dev_bf16(x))
    rc, rs = oracle.quantize_mx_e4m3(x)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(c.cpu().numpy(), rc)


def test_quantiser_edge_blocks():
    """Zero blocks, -0, saturation, subnormal and huge inputs, exact ties."""
    require_gpu()
    rows = []
    rows.append(np.zeros(32))
    r = np.full(32, 0.5); r[0], r[1] = 7.75, -7.75; rows.append(r)                 # saturating top binade
    rows.append(2.0 ** np.arange(-20, 12, dtype=np.float64))                       # wide range in one block
    rows.append(np.linspace(-1e-38, 1e-38, 32))                                    # bf16 subnormals
    rows.append(np.full(32, 3.0e38) * np.where(np.arange(32) % 2, 1, -1))          # near bf16's maximum
    t = np.full(32, 1.0); t[1:] = 1.0 + 2.0 ** -4 * np.arange(1, 32) / 31; rows.append(t)
    x = _bf(np.stack(rows))
    x[0, 7] = 0x8000
    x[1, 9] = 0x8000
    # exact ties between e4m3 neighbours after scaling: 256 * (1 + odd/16) with amax 256 -> X = 0
    tie = np.full(32, 1.0 + 1.0 / 16) * 256.0
    tie[0] = 256.0
    x = np.vstack([x, _bf(tie[None, :])])
    c, s = moeq.moe_quantize_mx_e4m3(dev_bf16(x))
    rc, rs = oracle.quantize_mx_e4m3(x)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(c.cpu().numpy(), rc)


def _deq_bits(x):
    c, s = oracle.quantize_mx_e4m3(x)
    d = oracle.dequantize_mx_e4m3(c, s)
    b = oracle.bf16_round(d)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32).astype(np.float64), d)   # exact in bf16
    return b


CFGS = {
    3: MoEConfig("aq_mxfp4", tokens=16, hidden=1024, experts=24, top_k=4, inter=256, shared_inter=128, fmt=3,
                 ue8m0_exp=(-6, -2)),
    2: MoEConfig("aq_e2m3", tokens=16, hidden=768, experts=16, top_k=3, inter=384, shared_inter=256, fmt=2),
    1: MoEConfig("aq_e2m1", tokens=16, hidden=512, experts=12, top_k=2, inter=256, fmt=1),
}
_layers = {}


def _layer(cfg):
    if cfg.name not in _layers:
        _layers[cfg.name] = upload_layer(cfg)
    return _layers[cfg.name]


@pytest.mark.parametrize("fmt", sorted(CFGS))
@pytest.mark.parametrize("T", [1, 5, 16, 70, 300])
def test_layer_with_quantised_activations(fmt, T):
    require_gpu()
    cfg = CFGS[fmt]
    L = _layer(cfg)
    x = synth.hidden_states(cfg, tokens=T, sub=90 + T)
    l = synth.router_logits(cfg, tokens=T, sub=90 + T)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    ws = moeq.workspace(L, T)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    out32 = moeq.moe_layer_decode(L, xd, ld, idx_out=idx, flags=F32 | MX, ws=ws)
    out16 = moeq.moe_layer_decode(L, xd, ld, flags=MX, ws=ws)
    moeq.moe_workspace_status(ws)
    ridx, _, ref = oracle_layer(cfg, _deq_bits(x), l)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_rel_err(out32.cpu().numpy(), ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))
    # and the quantisation is really there: the unquantised call differs
    plain = moeq.moe_layer_decode(L, xd, ld, flags=F32, ws=ws)
    assert not torch.equal(plain, out32)
