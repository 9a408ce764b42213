"""moe_layer_decode_noalloc (the library's static workspace) against
moe_layer_decode (a caller workspace) through the C ABI: two calls in a row,
the second with fewer tokens, each bitwise equal to the caller-workspace call
on the same inputs and within the parity bar of the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import synth
from gpu_util import dev_bf16, oracle_layer, require_gpu, upload_layer
from helpers import PARITY_TOL, max_rel_err
from synth import configs
from synth.configs import MoEConfig

pytestmark = pytest.mark.gpu
F32 = moeq.MOE_OUT_F32
SMALL = MoEConfig("noalloc_small", tokens=16, hidden=1024, experts=48, top_k=6, inter=256, shared_inter=256)


@pytest.mark.parametrize("cfg", [SMALL, configs.WIDE], ids=lambda c: c.name)
def test_noalloc_matches_workspace_call(cfg):
    require_gpu()
    L = upload_layer(cfg)
    ws = moeq.workspace(L, 16)
    for T, sub in ((16, 1), (3, 2), (1, 3)):
        x = synth.hidden_states(cfg, tokens=T, sub=sub)
        l = synth.router_logits(cfg, tokens=T, sub=sub)
        xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
        ref_out = moeq.moe_layer_decode(L, xd, ld, flags=F32, ws=ws)
        out = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
        moeq.moe_layer_decode_noalloc(L, xd, ld, out, idx_out=idx, flags=F32)
        out16 = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
        moeq.moe_layer_decode_noalloc(L, xd, ld, out16)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), T
        assert torch.equal(out16, ref_out.to(torch.bfloat16)), T
        rows = None if T * cfg.hidden <= 4096 else np.arange(0, cfg.hidden, 7)
        ridx, _, ref = oracle_layer(cfg, x, l, out_rows=rows)
        got = out.cpu().numpy() if rows is None else out.cpu().numpy()[:, rows]
        assert np.array_equal(idx.cpu().numpy(), ridx)
        assert max_rel_err(got, ref) <= PARITY_TOL


def test_noalloc_refuses_what_does_not_fit():
    require_gpu()
    L = upload_layer(SMALL)
    x = torch.zeros((17, SMALL.hidden), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((17, SMALL.experts), dtype=torch.float32, device="cuda")
    out = torch.empty((17, SMALL.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moeq.MoeError, match="static workspace"):
        moeq.moe_layer_decode_noalloc(L, x, lg, out)
