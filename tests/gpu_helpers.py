"""Shared helpers of the GPU parity tests (inputs from the seeded generators,
expected values from the CPU oracle only)."""

from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
from mixture_experts_expert_mm_amd import moe
from mixture_experts_expert_mm_amd import workloads as wl

TOL = {"bf16": 1e-2, "fp8": 5e-2, "int8": 5e-2}


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
    layer = moe.ExpertLayer(c.T, c.H, c.I, c.E, c.K, c.usecase, y_dtype, "cuda", activation_clamp=activation_clamp)
    layer.load_weights(inp.weights.w1, inp.weights.w2, inp.weights.s1, inp.weights.s2)
    return layer


def device_inputs(inp: wl.Inputs):
    return inp.x.cuda(), inp.topk_ids.cuda(), inp.topk_weights.cuda()


def oracle_y(inp: wl.Inputs, tokens=None, activation_clamp=None):
    y, _ = oracle.moe_forward(inp.x.float().numpy(), inp.topk_ids.numpy(), inp.topk_weights.numpy(),
                              expert_fn(inp), inp.cfg.usecase, tokens=tokens, activation_clamp=activation_clamp)
    return y


def rel_err(y_gpu: np.ndarray, y_or: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(y_or ** 2)))
    return float(np.abs(y_gpu - y_or).max() / rms)


def bf16_bits_of_f32(y32: torch.Tensor) -> torch.Tensor:
    """torch's own RNE cast of the float32 result, as int16 bit patterns."""
    return y32.to(torch.bfloat16).view(torch.int16)
