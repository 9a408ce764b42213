"""The full-size MoE workloads against the oracle (sampled output rows where
the oracle would be slow), in the launch configuration the bench times."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import synth
from gpu_util import bf16_rne_of_f32, dev_bf16, host_bf16, oracle_layer, require_gpu, upload_layer
from helpers import PARITY_TOL, max_rel_err
from synth import configs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [configs.WIDE, configs.BATCHED], ids=lambda c: c.name)
def test_full_size_decode(cfg):
    require_gpu()
    L = upload_layer(cfg)
    x, l = synth.hidden_states(cfg), synth.router_logits(cfg)
    xd, ld = dev_bf16(x), torch.from_numpy(l).cuda()
    ws = moeq.workspace(L, cfg.tokens)
    idx = torch.empty((cfg.tokens, cfg.top_k), dtype=torch.int32, device="cuda")
    out32 = moeq.moe_layer_decode(L, xd, ld, idx_out=idx, flags=moeq.MOE_OUT_F32, ws=ws)
    out16 = moeq.moe_layer_decode(L, xd, ld, ws=ws)
    rows = None if cfg.tokens == 1 else np.unique(np.concatenate([np.arange(0, cfg.hidden, 61), [cfg.hidden - 1]]))
    ridx, _, ref = oracle_layer(cfg, x, l, out_rows=rows)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    got = out32.cpu().numpy()
    got = got if rows is None else got[:, rows]
    assert max_rel_err(got, ref) <= PARITY_TOL
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))
    moeq.moe_workspace_status(ws)
