"""mega_moe_noalloc: the entry point for callers that cannot allocate runs
on the library's static per-GPU scratch and must give what mega_moe gives
on a caller workspace, bit for bit, call after call (the scratch keeps the
previous call's contents; the second call here is smaller)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from mixture_experts_expert_mm_amd import binding as B
from mixture_experts_expert_mm_amd import workloads as wl

from gpu_helpers import TOL, check_layout, device_active, device_inputs, log, make_layer, oracle_y, rel_err

pytestmark = pytest.mark.gpu


def _run_both(cfg):
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    act = device_active(inp)
    y_ref, c_ref = layer.forward(x, ids, wts, active=act)
    y = torch.full_like(y_ref, float("nan"))
    c = torch.full_like(c_ref, -7)
    log(f"[noalloc] {cfg.name}: T={cfg.T} fused workspace {layer.plan.fused_workspace_bytes / 2**20:.1f} MiB")
    B.mega_moe_noalloc(layer.plan, x, ids, wts, act, layer.w1, layer.s1, layer.w2, layer.s2, y, c)
    torch.cuda.synchronize()
    assert B.mm_read_device_error(layer.plan, None) == 0
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    assert torch.equal(c, c_ref)
    # the metadata it built in the static scratch is the oracle's too
    i32 = dict(dtype=torch.int32, device="cuda")
    off = torch.empty(layer.Et + 1, **i32)
    psrc = torch.empty(layer.plan.pool_rows, **i32)
    r2p = torch.empty(cfg.T * layer.Ks, **i32)
    B.mm_debug_fused_layout(layer.plan, None, off, psrc, r2p)
    torch.cuda.synchronize()
    check_layout(inp, layer.plan.block_m, c.cpu().numpy(), off.cpu().numpy(), psrc.cpu().numpy(), r2p.cpu().numpy())
    err = rel_err(y.cpu().double().numpy(), oracle_y(inp))
    log(f"    max|dY|/rms = {err:.3e}")
    assert err <= TOL[cfg.usecase], err


@pytest.mark.parametrize("usecase", ["bf16", "fp8", "int8"])
def test_noalloc_equals_mega_moe_two_calls_second_smaller(usecase):
    big = wl.Config(f"noalloc_big_{usecase}", usecase, 300, 1024, 512, 16, 4, 0.5, 41, masked_ratio=0.1,
                    shared=1, inactive_ratio=0.2)
    small = wl.Config(f"noalloc_small_{usecase}", usecase, 37, 512, 256, 8, 2, 0.5, 42)
    _run_both(big)
    _run_both(small)


def test_noalloc_at_the_largest_documented_size():
    """The 128-token layer of hidden 7168, intermediate 2048, 32 experts,
    top-8 (fp8: the largest workspace of the three use cases) fits."""
    _run_both(wl.CONFIGS["dsv3_fp8_t128"])


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    plan = B.mm_plan_create(4096, 7168, 2048, 32, 8, "fp8")
    assert plan.fused_workspace_bytes > 96 << 20
    good = 1 << 20
    lib = B.load()
    import ctypes
    st = lib.mega_moe_noalloc(ctypes.byref(plan), good, good, good, None, good, good, good, good, good, good, None)
    assert st == 3   # MM_ERR_WORKSPACE, before any HIP call
