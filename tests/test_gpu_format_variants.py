"""The three further formats (MXFP4 = e2m1 + UE8M0/32, int4 + fp16/64,
e2m3 + e4m3/16) on every call: the code and scale tables through one-hot
activations (exact), the dense GEMV, one expert's FFN, and the whole layer on
the decode kernels (1, 2..16 tokens) and the many-token matrix-core path,
each against the oracle with both decoders."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import oracle
import synth
from gpu_util import bf16_rne_of_f32, dev_bf16, dev_u8, host_bf16, oracle_layer, require_gpu, upload_layer
from helpers import PARITY_TOL, max_rel_err
from synth.configs import MoEConfig

pytestmark = pytest.mark.gpu
F32 = moeq.MOE_OUT_F32
DECS = [moeq.MOE_DECODER_LUT, moeq.MOE_DECODER_HW]
MX, I4, E3 = 3, 4, 5
NEW = [MX, I4, E3]
BF16_ONE = 0x3F80
ONE_SCALE = {MX: b"\x7f", I4: b"\x00\x3c", E3: b"\x38"}
BLOCK = {MX: 32, I4: 64, E3: 16}


def _one_hots(cols, js):
    x = np.zeros((len(js), cols), np.uint16)
    for i, j in enumerate(js):
        x[i, j] = BF16_ONE
    return x


def _fill_code(fmt, cols, code):
    if fmt in (MX, I4):
        return np.full(cols // 2, code | (code << 4), np.uint8)
    w = 0
    for q in range(4):
        w |= code << (6 * q)
    return np.tile(np.array([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], np.uint8), cols // 4)


@pytest.mark.parametrize("dec", DECS, ids=["lut", "hw"])
@pytest.mark.parametrize("fmt", NEW)
def test_every_code_every_position(fmt, dec):
    require_gpu()
    ncodes = 64 if fmt == E3 else 16
    cols = 128
    codes = np.stack([_fill_code(fmt, cols, r) for r in range(ncodes)])
    scales = np.tile(np.frombuffer(ONE_SCALE[fmt], np.uint8), (ncodes, cols // BLOCK[fmt]))
    W = moeq.QMat(fmt, ncodes, cols, dev_u8(codes), dev_u8(scales))
    tab = oracle.tables()["e2m3" if fmt == E3 else ("int4" if fmt == I4 else "e2m1")]
    for j0 in range(0, cols, 8):
        x = dev_bf16(_one_hots(cols, range(j0, j0 + 8)))
        y = moeq.dense_gemv_q(W, x, flags=F32 | dec).cpu().numpy()
        assert np.array_equal(y, np.tile(tab[:ncodes], (8, 1))), j0


@pytest.mark.parametrize("dec", DECS, ids=["lut", "hw"])
@pytest.mark.parametrize("fmt", NEW)
def test_every_scale(fmt, dec):
    """Every UE8M0 byte in fp32 range (MXFP4), every finite e4m3 byte (e2m3 +
    e4m3/16), and fp16 patterns across the whole range incl. subnormals."""
    require_gpu()
    cols = 128
    if fmt == MX:
        vals = np.arange(1, 255, dtype=np.uint8)
        scale_rows = np.repeat(vals[:, None], cols // 32, axis=1)
        want = 2.0 ** (vals.astype(np.float64) - 127)
    elif fmt == E3:
        vals = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
        scale_rows = np.repeat(vals[:, None], cols // 16, axis=1)
        want = oracle.tables()["e4m3"][vals]
    else:
        bits = np.array(sorted(set(list(range(1, 0x7C00, 61)) + [0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF]) |
                               set(b | 0x8000 for b in range(1, 0x7C00, 211))), np.uint16)
        scale_rows = np.repeat(bits.astype("<u2").view(np.uint8).reshape(-1, 2), cols // 64, axis=0).reshape(len(bits), -1)
        want = np.array([oracle.fp16_value(int(b)) for b in bits])
    rows = len(want)
    one = {MX: 2, I4: 1, E3: 8}[fmt]
    codes = np.tile(_fill_code(fmt, cols, one), (rows, 1))
    W = moeq.QMat(fmt, rows, cols, dev_u8(codes), dev_u8(np.ascontiguousarray(scale_rows)))
    x = dev_bf16(_one_hots(cols, [0, cols - 1]))
    y = moeq.dense_gemv_q(W, x, flags=F32 | dec).cpu().numpy()
    assert np.array_equal(y[0], want.astype(np.float32)) and np.array_equal(y[1], want.astype(np.float32))


@pytest.mark.parametrize("dec", DECS, ids=["lut", "hw"])
@pytest.mark.parametrize("fmt,rows,cols", [(MX, 37, 256), (MX, 515, 2048), (I4, 3, 64), (I4, 777, 5120),
                                           (E3, 301, 1280), (E3, 64, 8192)])
@pytest.mark.parametrize("B", [1, 4, 8])
def test_gemv_parity(fmt, rows, cols, B, dec):
    require_gpu()
    c, s = synth.matrix(fmt, rows, cols, 12, synth.stream_id(synth.K_W_CODES, rows), synth.stream_id(synth.K_W_SCALES, rows))
    x = synth.normal_bf16(12, synth.stream_id(synth.K_X, cols), B * cols).reshape(B, cols)
    W = moeq.QMat(fmt, rows, cols, dev_u8(c), dev_u8(s))
    xd = dev_bf16(x)
    y32 = moeq.dense_gemv_q(W, xd, flags=F32 | dec)
    y16 = moeq.dense_gemv_q(W, xd, flags=dec)
    ref = oracle.gemv(fmt, rows, cols, c, s, x)
    assert max_rel_err(y32.cpu().numpy(), ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(y16), bf16_rne_of_f32(y32))


CFGS = {
    MX: MoEConfig("v_mxfp4", tokens=16, hidden=1024, experts=40, top_k=6, inter=256, shared_inter=320, fmt=MX,
                  ue8m0_exp=(-6, -2)),
    I4: MoEConfig("v_int4", tokens=16, hidden=768, experts=24, top_k=4, inter=384, shared_inter=128, fmt=I4),
    E3: MoEConfig("v_e2m3s", tokens=16, hidden=1280, experts=33, top_k=5, inter=192, shared_inter=256, fmt=E3),
}
_layers = {}


def _layer(cfg):
    if cfg.name not in _layers:
        _layers[cfg.name] = upload_layer(cfg)
    return _layers[cfg.name]


@pytest.mark.parametrize("dec", DECS, ids=["lut", "hw"])
@pytest.mark.parametrize("fmt", NEW)
def test_expert_ffn_parity(fmt, dec):
    require_gpu()
    cfg = CFGS[fmt]
    L = _layer(cfg)
    x = synth.hidden_states(cfg, tokens=3, sub=7)
    xd = dev_bf16(x)
    for e in (0, cfg.experts - 1, -1):
        y32 = moeq.moe_expert_ffn_q(L, e, xd, flags=F32 | dec).cpu().numpy()
        ee = cfg.experts if e < 0 else e
        I = cfg.shared_inter if e < 0 else cfg.inter
        ew = synth.expert_weights(cfg, ee)
        ref = np.stack([oracle.ffn(fmt, cfg.hidden, I, ew, x[m]) for m in range(3)])
        assert max_rel_err(y32, ref) <= PARITY_TOL, (e, max_rel_err(y32, ref))


@pytest.mark.parametrize("dec", DECS, ids=["lut", "hw"])
@pytest.mark.parametrize("fmt", NEW)
@pytest.mark.parametrize("T", [1, 2, 7, 16])
def test_layer_parity(fmt, T, dec):
    require_gpu()
    cfg = CFGS[fmt]
    L = _layer(cfg)
    x = synth.hidden_states(cfg, tokens=T, sub=T)
    l = synth.router_logits(cfg, tokens=T, sub=T)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    ws = moeq.workspace(L, T)
    out32 = moeq.moe_layer_decode(L, xd, ld, idx_out=idx, flags=F32 | dec, ws=ws)
    out16 = moeq.moe_layer_decode(L, xd, ld, flags=dec, ws=ws)
    ridx, _, ref = oracle_layer(cfg, x, l)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_rel_err(out32.cpu().numpy(), ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))
    moeq.moe_workspace_status(ws)


@pytest.mark.parametrize("fmt", NEW)
def test_decoders_agree_and_batch_invariance(fmt):
    require_gpu()
    cfg = CFGS[fmt]
    L = _layer(cfg)
    x = synth.hidden_states(cfg, tokens=16, sub=21)
    l = synth.router_logits(cfg, tokens=16, sub=21)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    ws = moeq.workspace(L, 16)
    a = moeq.moe_layer_decode(L, xd, ld, flags=F32 | moeq.MOE_DECODER_LUT, ws=ws)
    b = moeq.moe_layer_decode(L, xd, ld, flags=F32 | moeq.MOE_DECODER_HW, ws=ws)
    assert torch.equal(a, b)
    for t in (0, 5, 15):
        one = moeq.moe_layer_decode(L, xd[t:t + 1].clone(), ld[t:t + 1].clone(), flags=F32, ws=ws)
        assert torch.equal(one[0], a[t]), t


@pytest.mark.parametrize("fmt", NEW)
def test_many_token_path(fmt):
    """T = 70 > 16: the matrix-core path (route, group, MFMA GEMMs, combine)."""
    require_gpu()
    cfg = CFGS[fmt]
    L = _layer(cfg)
    T = 70
    x = synth.hidden_states(cfg, tokens=T, sub=33)
    l = synth.router_logits(cfg, tokens=T, sub=33)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    ws = moeq.workspace(L, T)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    out32 = moeq.moe_layer_decode(L, xd, ld, idx_out=idx, flags=F32, ws=ws)
    out16 = moeq.moe_layer_decode(L, xd, ld, ws=ws)
    ridx, _, ref = oracle_layer(cfg, x, l)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_rel_err(out32.cpu().numpy(), ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))
    moeq.moe_workspace_status(ws)
