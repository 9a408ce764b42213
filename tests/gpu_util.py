"""Helpers for the GPU tests: move seeded inputs to the device, run the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import synth

NAMES = ("w13_codes", "w13_scales", "w2_codes", "w2_scales")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moeq.load_library()      # raises if the HIP library is not built


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bf16(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_rne_of_f32(t):
    """Bits of RNE_bf16(t) for a float32 tensor (torch's conversion is RNE)."""
    return host_bf16(t.to(torch.bfloat16))


def upload_layer(cfg, top_k=None, chunk=16):
    """The whole layer on the GPU, generated expert by expert on the host."""
    shp = synth.expert_shapes(cfg)
    devs = {n: torch.empty((cfg.experts,) + shp[n], dtype=torch.uint8, device="cuda") for n in NAMES}
    for e0 in range(0, cfg.experts, chunk):
        e1 = min(cfg.experts, e0 + chunk)
        host = {n: np.empty((e1 - e0,) + shp[n], np.uint8) for n in NAMES}
        for e in range(e0, e1):
            synth.fill_expert(cfg, e, {n: host[n][e - e0] for n in NAMES})
        for n in NAMES:
            devs[n][e0:e1].copy_(torch.from_numpy(host[n]))
    shared = None
    if cfg.shared_inter:
        sh = synth.expert_weights(cfg, cfg.experts)
        shared = {n: dev_u8(sh[n]) for n in NAMES}
    layer = moeq.Layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, top_k or cfg.top_k,
                       devs["w13_codes"], devs["w13_scales"], devs["w2_codes"], devs["w2_scales"],
                       shared_inter=cfg.shared_inter, shared=shared)
    return layer


def oracle_layer(cfg, x_bits, logits, k=None, out_rows=None):
    """Oracle output for the tokens, regenerating only the selected experts."""
    import oracle
    k = k or cfg.top_k
    idx, _ = oracle.route(logits, k)
    experts = {int(e): synth.expert_weights(cfg, int(e)) for e in np.unique(idx)}
    shared = synth.expert_weights(cfg, cfg.experts) if cfg.shared_inter else None
    return oracle.layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, k, experts, x_bits, logits,
                        shared=shared, shared_inter=cfg.shared_inter, out_rows=out_rows)
