"""Helpers for the GPU tests: move seeded inputs to the device, run the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_bit_moe_amd as moeq
import synth

def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moeq.load_library()      # raises if the HIP library is not built


from synth.device import dev_bf16, dev_u8, upload_layer_tensors  # noqa: F401


def host_bf16(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_rne_of_f32(t):
    """Bits of RNE_bf16(t) for a float32 tensor (torch's conversion is RNE)."""
    return host_bf16(t.to(torch.bfloat16))


def upload_layer(cfg, top_k=None):
    """The whole layer on the GPU as a moeq.Layer."""
    devs, shared = upload_layer_tensors(cfg)
    return moeq.Layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, top_k or cfg.top_k,
                      devs["w13_codes"], devs["w13_scales"], devs["w2_codes"], devs["w2_scales"],
                      shared_inter=cfg.shared_inter, shared=shared)


def oracle_layer(cfg, x_bits, logits, k=None, out_rows=None):
    """Oracle output for the tokens, regenerating only the selected experts."""
    import oracle
    k = k or cfg.top_k
    idx, _ = oracle.route(logits, k)
    experts = {int(e): synth.expert_weights(cfg, int(e)) for e in np.unique(idx)}
    shared = synth.expert_weights(cfg, cfg.experts) if cfg.shared_inter else None
    return oracle.layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, k, experts, x_bits, logits,
                        shared=shared, shared_inter=cfg.shared_inter, out_rows=out_rows)
