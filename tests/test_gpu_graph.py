"""Calls captured in a HIP graph and replayed: the launch mode the bench times.

Ten moe_layer_decode calls on ONE workspace are captured into one graph: a
one-token layer shaped like the wide decode layer (shared expert, top-10) and
a 16-token layer shaped like the batched one, each with two weight replicas,
every call with its own logits and its own output.  The graph is replayed
twice, with eager calls on the same workspace in between.  Every replayed
output must equal the eager output of the same call bit for bit and match the
oracle element-wise to the parity bar.  This exercises the workspace's call
counter (read on entry, raised on exit) across graph replays, which bake in
the kernels' arguments but not the counter's value."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import synth
from gpu_util import dev_bf16, oracle_layer, require_gpu, upload_layer
from helpers import PARITY_TOL, max_rel_err
from synth.configs import MoEConfig

pytestmark = pytest.mark.gpu
F32 = moeq.MOE_OUT_F32

WIDE_S = MoEConfig("graph_wide", tokens=1, hidden=2048, experts=64, top_k=10, inter=512, shared_inter=512,
                   logit_sigma=1.5)
BATCH_S = MoEConfig("graph_batched", tokens=16, hidden=1536, experts=48, top_k=8, inter=512)


def _replica(L, cfg):
    """The same weights in fresh memory (a second replica of the layer)."""
    t = [x.clone() for x in L.tensors[:4]]
    sh = None
    if cfg.shared_inter:
        sh = dict(zip(("w13_codes", "w13_scales", "w2_codes", "w2_scales"), [x.clone() for x in L.tensors[4:]]))
    return moeq.Layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, *t, shared_inter=cfg.shared_inter,
                      shared=sh)


def test_graph_replay_matches_eager_and_oracle():
    require_gpu()
    plan = []
    layers = {}
    for cfg in (WIDE_S, BATCH_S):
        L0 = upload_layer(cfg)
        layers[cfg.name] = [L0, _replica(L0, cfg)]
    ws_bytes = max(moeq.moe_layer_workspace_bytes(layers[c.name][0], c.tokens) for c in (WIDE_S, BATCH_S))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    for i in range(10):
        cfg = WIDE_S if i % 2 == 0 else BATCH_S
        T = cfg.tokens
        x = synth.hidden_states(cfg, tokens=T, sub=100 + i)
        l = synth.router_logits(cfg, tokens=T, sub=100 + i)
        plan.append(dict(cfg=cfg, L=layers[cfg.name][(i // 2) % 2], x=x, l=l, xd=dev_bf16(x),
                         ld=torch.from_numpy(l).cuda(),
                         out=torch.full((T, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")))

    def run(outs):
        for p, o in zip(plan, outs):
            moeq.moe_layer_decode(p["L"], p["xd"], p["ld"], out=o, flags=F32, ws=ws)

    eager = [torch.empty_like(p["out"]) for p in plan]
    run(eager)
    torch.cuda.synchronize()
    moeq.moe_workspace_status(ws)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run([p["out"] for p in plan])
    torch.cuda.synchronize()

    refs = [oracle_layer(p["cfg"], p["x"], p["l"])[2] for p in plan]
    for rep in range(2):
        for p in plan:
            p["out"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        moeq.moe_workspace_status(ws)
        for i, (p, e, ref) in enumerate(zip(plan, eager, refs)):
            got = p["out"]
            assert torch.equal(got, e), (rep, i, p["cfg"].name)
            err = max_rel_err(got.cpu().numpy(), ref)
            assert err <= PARITY_TOL, (rep, i, p["cfg"].name, err)
        # eager calls on the same workspace between the replays
        again = [torch.empty_like(p["out"]) for p in plan]
        run(again)
        torch.cuda.synchronize()
        for a, e in zip(again, eager):
            assert torch.equal(a, e)
