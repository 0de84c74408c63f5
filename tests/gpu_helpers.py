"""Shared helpers of the GPU parity tests (inputs from the seeded generators,
expected values from the CPU oracle only)."""

from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
from mixture_experts_expert_mm_amd import moe
from mixture_experts_expert_mm_amd import workloads as wl

TOL = {"bf16": 1e-2, "fp8": 5e-2, "int8": 5e-2, "mxfp8": 5e-2, "mxfp4": 5e-2}


def log(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=4)
def cpu_inputs(cfg: wl.Config) -> wl.Inputs:
    return wl.make_inputs(cfg)


def expert_fn(inp: wl.Inputs):
    """Oracle view of the generated weights (formula layout, raw codes)."""
    w = inp.weights
    uc = inp.cfg.usecase

    def expert(e):
        w1, w2 = w.w1[e], w.w2[e]
        if uc in wl.MX_USECASES:
            return wl.unpack_codes(w1, inp.cfg), wl.unpack_codes(w2, inp.cfg), w.s1[e].numpy(), w.s2[e].numpy()
        if uc == "fp8":
            w1, w2 = w1.view(torch.uint8), w2.view(torch.uint8)
        elif uc == "bf16":
            w1, w2 = w1.float(), w2.float()
        s1 = None if w.s1 is None else w.s1[e].numpy()
        s2 = None if w.s2 is None else w.s2[e].numpy()
        return w1.numpy(), w2.numpy(), s1, s2

    return expert


def make_layer(inp: wl.Inputs, y_dtype="f32", activation_clamp=None):
    c = inp.cfg
    layer = moe.ExpertLayer(c.T, c.H, c.I, c.E, c.K, c.usecase, y_dtype, "cuda", activation_clamp=activation_clamp,
                            num_shared_experts=c.shared)
    layer.load_weights(inp.weights.w1, inp.weights.w2, inp.weights.s1, inp.weights.s2)
    return layer


def device_inputs(inp: wl.Inputs):
    return inp.x.cuda(), inp.topk_ids.cuda(), inp.topk_weights.cuda()


def device_active(inp: wl.Inputs):
    return None if inp.active is None else inp.active.cuda()


def oracle_y(inp: wl.Inputs, tokens=None, activation_clamp=None):
    c = inp.cfg
    y, _ = oracle.moe_forward(inp.x.float().numpy(), inp.topk_ids.numpy(), inp.topk_weights.numpy(),
                              expert_fn(inp), c.usecase, tokens=tokens, activation_clamp=activation_clamp,
                              shared_expert=c.E if c.shared else None,
                              active=None if inp.active is None else inp.active.numpy())
    return y


def oracle_routes(inp: wl.Inputs) -> np.ndarray:
    """Route table [T, K+S] (shared slot, inactive tokens -1) from the oracle."""
    c = inp.cfg
    ids, _ = oracle.route_table(inp.topk_ids.numpy(), inp.topk_weights.numpy(), c.E if c.shared else None,
                                None if inp.active is None else inp.active.numpy())
    return ids


def check_layout(inp: wl.Inputs, block_m: int, counts, offs, psrc, r2p):
    """Bit-exact dispatch metadata against the oracle: counts, padded offsets,
    per-expert (token, slot) multisets, -1 padding, inverse map, skipped
    routes.  Returns the valid pool rows."""
    c = inp.cfg
    ids = oracle_routes(inp)
    Et = c.E + c.shared
    d = oracle.dispatch_layout(ids, Et, block_m)
    np.testing.assert_array_equal(np.asarray(counts), d["counts"][:len(counts)])
    np.testing.assert_array_equal(offs, d["offsets"])
    for e in range(Et):
        o, n, o1 = offs[e], d["counts"][e], offs[e + 1]
        np.testing.assert_array_equal(np.sort(psrc[o:o + n]), d["routes"][e])
        assert np.all(psrc[o + n:o1] == -1)
    flat = ids.reshape(-1)
    valid = flat >= 0
    assert np.all(r2p[~valid] == -1)
    rv = np.nonzero(valid)[0]
    np.testing.assert_array_equal(psrc[r2p[rv]], rv)
    return np.concatenate([np.arange(offs[e], offs[e] + d["counts"][e]) for e in range(Et)])


def rel_err(y_gpu: np.ndarray, y_or: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(y_or ** 2)))
    return float(np.abs(y_gpu - y_or).max() / rms)


def bf16_bits_of_f32(y32: torch.Tensor) -> torch.Tensor:
    """torch's own RNE cast of the float32 result, as int16 bit patterns."""
    return y32.to(torch.bfloat16).view(torch.int16)
