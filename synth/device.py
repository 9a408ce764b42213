"""Moving seeded inputs to the GPU (torch memory as plumbing; no arithmetic)."""
import numpy as np
import torch

from . import expert_shapes, expert_weights, fill_expert

NAMES = ("w13_codes", "w13_scales", "w2_codes", "w2_scales")


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    """uint16 bit patterns -> a bf16 CUDA tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def upload_layer_tensors(cfg, chunk=16):
    """The whole layer's arrays on the GPU, generated expert by expert on the
    host.  Returns (dict of [E][...] uint8 tensors, shared dict or None)."""
    shp = expert_shapes(cfg)
    devs = {n: torch.empty((cfg.experts,) + shp[n], dtype=torch.uint8, device="cuda") for n in NAMES}
    for e0 in range(0, cfg.experts, chunk):
        e1 = min(cfg.experts, e0 + chunk)
        host = {n: np.empty((e1 - e0,) + shp[n], np.uint8) for n in NAMES}
        for e in range(e0, e1):
            fill_expert(cfg, e, {n: host[n][e - e0] for n in NAMES})
        for n in NAMES:
            devs[n][e0:e1].copy_(torch.from_numpy(host[n]))
    shared = None
    if cfg.shared_inter:
        sh = expert_weights(cfg, cfg.experts)
        shared = {n: dev_u8(sh[n]) for n in NAMES}
    return devs, shared
