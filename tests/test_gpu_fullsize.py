"""The full-size MoE decode workloads against the oracle (sampled output rows
where the oracle would be slow), eagerly and in the launch mode the bench
times: calls with fresh logits captured in a HIP graph on one workspace and
replayed."""
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
    x = synth.hidden_states(cfg)
    xd = dev_bf16(x)
    ws = moeq.workspace(L, cfg.tokens)
    rows = None if cfg.tokens == 1 else np.unique(np.concatenate([np.arange(0, cfg.hidden, 61), [cfg.hidden - 1]]))

    def check(out32, l, idx=None):
        ridx, _, ref = oracle_layer(cfg, x, l, out_rows=rows)
        if idx is not None:
            assert np.array_equal(idx.cpu().numpy(), ridx)
        got = out32.cpu().numpy()
        got = got if rows is None else got[:, rows]
        assert max_rel_err(got, ref) <= PARITY_TOL

    # eager, with the routing written out
    l0 = synth.router_logits(cfg)
    ld0 = torch.from_numpy(l0).cuda()
    idx = torch.empty((cfg.tokens, cfg.top_k), dtype=torch.int32, device="cuda")
    out32 = moeq.moe_layer_decode(L, xd, ld0, idx_out=idx, flags=moeq.MOE_OUT_F32, ws=ws)
    out16 = moeq.moe_layer_decode(L, xd, ld0, ws=ws)
    check(out32, l0, idx)
    assert np.array_equal(host_bf16(out16), bf16_rne_of_f32(out32))
    moeq.moe_workspace_status(ws)

    # three calls with fresh logits, captured and replayed twice
    ls = [synth.router_logits(cfg, sub=s) for s in (1, 2, 3)]
    lds = [torch.from_numpy(l).cuda() for l in ls]
    eager = [moeq.moe_layer_decode(L, xd, ld, flags=moeq.MOE_OUT_F32, ws=ws) for ld in lds]
    outs = [torch.empty_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for ld, o in zip(lds, outs):
                moeq.moe_layer_decode(L, xd, ld, out=o, flags=moeq.MOE_OUT_F32, ws=ws)
    torch.cuda.synchronize()
    for rep in range(2):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        moeq.moe_workspace_status(ws)
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), rep
    for o, l in zip(outs, ls):
        check(o, l)
