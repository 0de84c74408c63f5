"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: dispatch metadata bit-exact (counts, padded offsets, per-expert
(token, slot) multisets, inverse map); quantised activation codes and
scales bit-exact (both sides decide them in IEEE float32); int8 GEMM
accumulators exact; Y within max|dY|/rms(Y_oracle) <= 1e-2 (bf16) or
5e-2 (fp8 / int8), evaluated on the float32 output of the kernel, with the
bf16 output equal bit for bit to the round-to-nearest-even of that float32
output; fused == three-call bit for bit; run-to-run bit-identical.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_expert_mm_amd import binding as B
from mixture_experts_expert_mm_amd import moe
from mixture_experts_expert_mm_amd import workloads as wl

from gpu_helpers import (TOL, bf16_bits_of_f32, check_layout, cpu_inputs, device_active, device_inputs, expert_fn,
                         log, make_layer, oracle_routes, oracle_y, rel_err)

pytestmark = pytest.mark.gpu

# shapes that span several tiles and a ragged tail in every GEMM dimension;
# bm64 has 17 rows per expert on average (BLOCK_M 64) and, from a strong
# router bias, two experts of more than one M-block and seven empty ones
SMALL = {
    "bm32": dict(T=20, H=256, I=128, E=16, K=2, bias=0.5),
    "bm64": dict(T=200, H=512, I=256, E=24, K=2, bias=2.0),
    "bm128": dict(T=333, H=768, I=384, E=6, K=3, bias=0.5),
    # BLOCK_M 256 (forced): ~300 rows per expert, one full and one ragged
    # M-block each, 3 x 2 and 3 x 3 tiles of 256 x 256
    "bm256": dict(T=600, H=768, I=384, E=4, K=2, bias=0.5),
}
FORCED_TILE = {"bm256": "2"}   # MM_FORCE_TILE of shapes whose tile the plan would not choose


def small_cfg(shape: str, usecase: str, **kw) -> wl.Config:
    """A SMALL shape with the use case's dtype (extra Config fields in kw)."""
    s = SMALL[shape]
    return wl.Config(f"{shape}_{usecase}", usecase, s["T"], s["H"], s["I"], s["E"], s["K"], s["bias"], 2024, **kw)


def check_dispatch(layer: moe.ExpertLayer, inp: wl.Inputs, im, sample_rows=None):
    """Bit-exact dispatch metadata and pool rows against the oracle."""
    c = inp.cfg
    counts = im.expert_counts.cpu().numpy()
    rows = check_layout(inp, layer.plan.block_m, counts, im.expert_offsets.cpu().numpy(), im.pool_src.cpu().numpy(),
                        im.route_to_pool.cpu().numpy())
    psrc = im.pool_src.cpu().numpy()
    # pool rows: x_i itself (bf16) or its quantised codes and scale
    if sample_rows is not None and rows.size > sample_rows:
        rows = np.random.default_rng(0).choice(rows, sample_rows, replace=False)
    tok = psrc[rows] // (c.K + c.shared)
    rows_t = torch.from_numpy(rows).cuda()
    if c.usecase in wl.MX_USECASES:
        codes, e8 = oracle.mx_quantize(inp.x.float().numpy()[tok].astype(np.float64), "e4m3")
        xp = im.x_pool.view(-1, c.H)[rows_t].cpu().numpy()
        np.testing.assert_array_equal(xp, codes)
        np.testing.assert_array_equal(im.x_pool_scale.view(-1, c.H // 32)[rows_t].cpu().numpy(), e8)
    elif c.usecase == "bf16":
        xp = im.x_pool.view(torch.int16).view(-1, c.H)[rows_t].cpu()
        np.testing.assert_array_equal(xp.numpy(), inp.x.view(torch.int16)[torch.from_numpy(tok)].numpy())
    else:
        codes, s, _ = oracle.quantize_tokens(inp.x.float().numpy()[tok], c.usecase)
        xp = im.x_pool.view(-1, c.H)[rows_t].cpu().numpy()
        np.testing.assert_array_equal(xp.view(np.uint8), codes.view(np.uint8))
        np.testing.assert_array_equal(im.x_pool_scale[rows_t].cpu().numpy(), s)


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_dispatch_metadata_full_configs(name):
    cfg = wl.CONFIGS[name]
    log(f"[dispatch] {name}")
    inp = cpu_inputs(cfg)
    layer = moe.ExpertLayer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.usecase, "f32", "cuda")
    im = layer.new_intermediates()
    x, ids, _ = device_inputs(inp)
    layer.dispatch(x, ids, im)
    torch.cuda.synchronize()
    check_dispatch(layer, inp, im, sample_rows=4096)


@pytest.mark.parametrize("shape", list(SMALL))
@pytest.mark.parametrize("usecase", ["bf16", "fp8", "int8"])
def test_dispatch_small_masked(shape, usecase, monkeypatch):
    if shape in FORCED_TILE:
        monkeypatch.setenv("MM_FORCE_TILE", FORCED_TILE[shape])
    cfg = small_cfg(shape, usecase, masked_ratio=0.2)
    log(f"[dispatch masked] {cfg.name}")
    inp = wl.make_inputs(cfg)
    layer = moe.ExpertLayer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.usecase, "f32", "cuda")
    im = layer.new_intermediates()
    x, ids, _ = device_inputs(inp)
    layer.dispatch(x, ids, im)
    torch.cuda.synchronize()
    check_dispatch(layer, inp, im)


@pytest.mark.parametrize("usecase", ["fp8", "int8"])
def test_activation_quantiser_all_bf16_patterns(usecase):
    """Every finite bf16 bit pattern goes through the dispatch quantiser once."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    finite = bits[np.isfinite(f)]
    rng = np.random.default_rng(5)
    H = 256
    n = (finite.size + H - 1) // H * H
    pat = np.concatenate([finite, rng.choice(finite, n - finite.size)])
    rng.shuffle(pat)
    x = torch.from_numpy(pat.astype(np.uint16).view(np.int16).reshape(-1, H)).view(torch.bfloat16)
    T = x.shape[0]
    log(f"[quantiser] {usecase} T={T}")
    layer = moe.ExpertLayer(T, H, 128, 1, 1, usecase, "f32", "cuda")
    im = layer.new_intermediates()
    ids = torch.zeros((T, 1), dtype=torch.int32)
    layer.dispatch(x.cuda(), ids.cuda(), im)
    torch.cuda.synchronize()
    codes, s, _ = oracle.quantize_tokens(x.float().numpy(), usecase)
    psrc = im.pool_src.cpu().numpy()[:T]
    xp = im.x_pool.view(-1, H)[:T].cpu().numpy().view(np.uint8)
    np.testing.assert_array_equal(xp, codes.view(np.uint8)[psrc])
    np.testing.assert_array_equal(im.x_pool_scale[:T].cpu().numpy(), s[psrc])


# ---------------------------------------------------------------------------
# Y parity, small shapes (every element compared)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", list(SMALL))
@pytest.mark.parametrize("usecase", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("masked", [0.0, 0.25])
def test_y_parity_small(shape, usecase, masked, monkeypatch):
    if shape in FORCED_TILE:
        monkeypatch.setenv("MM_FORCE_TILE", FORCED_TILE[shape])
    cfg = small_cfg(shape, usecase, masked_ratio=masked)
    log(f"[y small] {cfg.name} masked={masked}")
    inp = wl.make_inputs(cfg)
    x, ids, wts = device_inputs(inp)
    layer32 = make_layer(inp, "f32")
    y32, counts = layer32.forward(x, ids, wts)
    layer16 = make_layer(inp, "bf16")
    y16, _ = layer16.forward(x, ids, wts)
    torch.cuda.synchronize()
    y_or = oracle_y(inp)
    err = rel_err(y32.cpu().double().numpy(), y_or)
    log(f"    max|dY|/rms = {err:.3e}")
    assert err <= TOL[usecase], err
    assert torch.equal(y16.view(torch.int16).cpu(), bf16_bits_of_f32(y32).cpu())
    ids_np = inp.topk_ids.numpy()
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(ids_np[ids_np >= 0], minlength=cfg.E))


def test_tiny_config_all_elements():
    cfg = wl.CONFIGS["tiny_bf16"]
    inp = cpu_inputs(cfg)
    x, ids, wts = device_inputs(inp)
    y32, _ = make_layer(inp, "f32").forward(x, ids, wts)
    torch.cuda.synchronize()
    err = rel_err(y32.cpu().double().numpy(), oracle_y(inp))
    log(f"[tiny] max|dY|/rms = {err:.3e}")
    assert err <= TOL["bf16"]


# ---------------------------------------------------------------------------
# exact integer accumulators (A8W8-INT)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", ["bm64", "bm256", "split128", "split64"])
def test_int8_accumulators_exact(shape, monkeypatch):
    """int32 accumulators before any scaling equal numpy's int64 products on
    every valid row.  bm64: the 64 x 128 tile, no split; bm256: the 256 x 256
    tile (forced).  split128 / split64: 256 routes per expert, so the tail
    tiles of both GEMMs are split along K (BLOCK_M 128: Linear1 in up to 4
    pieces, Linear2 in 2; BLOCK_M 64 forced: more pieces) and piece 0 adds
    the others' partial sums."""
    if shape in ("bm64", "bm256"):
        if shape in FORCED_TILE:
            monkeypatch.setenv("MM_FORCE_TILE", FORCED_TILE[shape])
        cfg = small_cfg(shape, "int8")
    else:
        cfg = wl.Config(f"{shape}_int8", "int8", 512, 2048, 1024, 8, 4, 0.3, 61)
        if shape == "split64":
            monkeypatch.setenv("MM_FORCE_TILE", "0")
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    log(f"[int8 exact] {shape}: BLOCK_M {layer.plan.block_m}")
    x, ids, wts = device_inputs(inp)
    im = layer.new_intermediates()
    layer.dispatch(x, ids, im)
    layer.linear1(im)
    P = layer.plan.pool_rows
    ws = layer.workspace(False)
    c1 = torch.empty((P, 2 * cfg.I), dtype=torch.int32, device="cuda")
    c2 = torch.empty((P, cfg.H), dtype=torch.int32, device="cuda")
    B.mm_debug_raw_accumulators(layer.plan, 1, im.expert_offsets, im.expert_counts, im.x_pool, layer.w1, c1, ws)
    B.mm_debug_raw_accumulators(layer.plan, 2, im.expert_offsets, im.expert_counts, im.a_pool, layer.w2, c2, ws)
    torch.cuda.synchronize()
    assert layer.device_error(fused=False) == 0
    offs = im.expert_offsets.cpu().numpy()
    counts = im.expert_counts.cpu().numpy()
    psrc = im.pool_src.cpu().numpy()
    q, _, _ = oracle.quantize_tokens(inp.x.float().numpy(), "int8")
    a_codes = im.a_pool.view(torch.int8).view(P, cfg.I).cpu().numpy().astype(np.int64)
    c1 = c1.cpu().numpy()
    c2 = c2.cpu().numpy()
    for e in range(cfg.E):
        rows = np.arange(offs[e], offs[e] + counts[e])
        if rows.size == 0:
            continue
        w1 = inp.weights.w1[e].numpy().astype(np.int64)
        w2 = inp.weights.w2[e].numpy().astype(np.int64)
        np.testing.assert_array_equal(c1[rows], q[psrc[rows] // cfg.K].astype(np.int64) @ w1)
        np.testing.assert_array_equal(c2[rows], a_codes[rows] @ w2)
        assert np.all(np.abs(a_codes[rows]) <= 127)


def test_gemm_entry_points_on_a_dirty_workspace():
    """The GEMM entry points clear the split-tile flags themselves: Linear1
    and Linear2 run on a separate workspace filled with 0xFF (as a fresh
    allocation may be) give Y bit-equal to a clean run, on an int8 shape
    whose tail tiles are split along K."""
    cfg = wl.Config("dirty_ws_int8", "int8", 512, 2048, 1024, 8, 4, 0.3, 62)
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    y_ref, _ = layer.forward_3call(x, ids, wts)
    im = layer.new_intermediates()
    layer.dispatch(x, ids, im)
    dirty = torch.full((layer.plan.workspace_bytes,), 255, dtype=torch.uint8, device="cuda")
    y = layer.new_y()
    log("[dirty workspace] int8 L1 + L2 on a 0xFF workspace")
    B.mm_grouped_l1_swiglu(layer.plan, im.expert_offsets, im.expert_counts, im.x_pool, im.x_pool_scale, layer.w1,
                           layer.s1, im.a_pool, im.a_pool_scale, dirty)
    B.mm_grouped_l2_combine(layer.plan, im.expert_offsets, im.expert_counts, im.pool_src, im.route_to_pool, im.a_pool,
                            im.a_pool_scale, layer.w2, layer.s2, wts, y, dirty)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))


# ---------------------------------------------------------------------------
# shared expert and x_active_mask
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", ["bm64", "bm128"])
@pytest.mark.parametrize("usecase", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("variant", ["shared", "active", "shared_active"])
def test_shared_expert_and_active_mask(shape, usecase, variant):
    """A shared expert (one more slot per token, weight 1) and/or an
    x_active_mask with about a third of the tokens inactive: Y within the
    oracle tolerance, inactive rows exactly 0, fused == three-call bit for
    bit, the dispatch metadata of both paths bit-exact, expert_token_nums
    the routed experts' counts."""
    cfg = small_cfg(shape, usecase, masked_ratio=0.1, shared=int("shared" in variant),
                    inactive_ratio=0.35 if "active" in variant else 0.0)
    inp = wl.make_inputs(cfg)
    log(f"[{variant}] {cfg.name}")
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    act = device_active(inp)
    y_f, c_f = layer.forward(x, ids, wts, active=act)
    y_f = y_f.clone()
    off, psrc, r2p = (t.cpu().numpy() for t in layer.fused_layout())
    y_3, im = layer.forward_3call(x, ids, wts, active=act)
    torch.cuda.synchronize()
    assert layer.device_error(fused=True) == 0 and layer.device_error(fused=False) == 0
    assert torch.equal(y_f.view(torch.int32), y_3.view(torch.int32))
    check_dispatch(layer, inp, im)
    check_layout(inp, layer.plan.block_m, c_f.cpu().numpy(), off, psrc, r2p)
    np.testing.assert_array_equal(c_f.cpu().numpy(), im.expert_counts.cpu().numpy()[:cfg.E])
    y_or = oracle_y(inp)
    err = rel_err(y_f.cpu().double().numpy(), y_or)
    log(f"    max|dY|/rms = {err:.3e}")
    assert err <= TOL[usecase], err
    if inp.active is not None:
        off_rows = (inp.active.numpy() == 0)
        assert off_rows.any() and not y_f.cpu().numpy()[off_rows].any()


# ---------------------------------------------------------------------------
# fused vs three-call, determinism, edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("usecase", ["bf16", "fp8", "int8"])
def test_fused_equals_three_call_and_is_deterministic(usecase):
    cfg = small_cfg("bm128", usecase)
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    y_f, c_f = layer.forward(x, ids, wts)
    y_f2, _ = layer.forward(x, ids, wts)
    y_3, im = layer.forward_3call(x, ids, wts)
    torch.cuda.synchronize()
    assert torch.equal(y_f.view(torch.int32), y_f2.view(torch.int32))
    assert torch.equal(y_f.view(torch.int32), y_3.view(torch.int32))
    assert torch.equal(c_f, im.expert_counts)
    assert layer.device_error(fused=True) == 0 and layer.device_error(fused=False) == 0


@pytest.mark.parametrize("shape,usecase", [("bm128", "bf16"), ("bm128", "fp8"), ("bm256", "int8")])
def test_cooperative_launch_equals_ordinary(shape, usecase, monkeypatch):
    """A plan made with MM_COOPERATIVE=1 launches the fused kernel
    cooperatively; the results are those of the ordinary launch, bit for bit."""
    if shape in FORCED_TILE:
        monkeypatch.setenv("MM_FORCE_TILE", FORCED_TILE[shape])
    cfg = small_cfg(shape, usecase)
    inp = wl.make_inputs(cfg)
    x, ids, wts = device_inputs(inp)
    ordinary = make_layer(inp, "f32")
    y0, c0 = ordinary.forward(x, ids, wts)
    monkeypatch.setenv("MM_COOPERATIVE", "1")
    coop = make_layer(inp, "f32")
    assert coop.plan.reserved[2] == 1 and ordinary.plan.reserved[2] == 0
    y1, c1 = coop.forward(x, ids, wts)
    torch.cuda.synchronize()
    assert coop.device_error() == 0
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
    assert torch.equal(c0, c1)


@pytest.mark.parametrize("case", ["bm256_bf16", "bm256_fp8", "bm256_int8", "bm128_fp8", "bm128_mxfp8"])
def test_tile_claiming_equals_static_tiles(case, monkeypatch):
    """The fused kernel's tiles claimed from per-XCD counters, other XCDs'
    tiles taken once a slice is done (the default at 256 x 256, and with at
    least 8 tiles per workgroup at 128 x 256), give the results of the static
    round robin (a plan made with MM_STATIC_TILES=1) and of the three-call
    path, bit for bit."""
    shape, usecase = case.split("_")
    if shape == "bm256":
        monkeypatch.setenv("MM_FORCE_TILE", "2")
        cfg = small_cfg("bm256", usecase, masked_ratio=0.1)
    else:   # 32 M-blocks per XCD slice x 8 Linear1 tiles: claimed at 128 x 256 too
        monkeypatch.setenv("MM_FORCE_TILE", "1")
        cfg = wl.Config(f"claim_{usecase}", usecase, 8192, 256, 1024, 8, 4, 0.5, 5, masked_ratio=0.1)
    inp = wl.make_inputs(cfg)
    x, ids, wts = device_inputs(inp)
    log(f"[tile claiming] {cfg.name}")
    dyn = make_layer(inp, "f32")
    y_dyn, c_dyn = dyn.forward(x, ids, wts)
    y_dyn = y_dyn.clone()
    y_3, _ = dyn.forward_3call(x, ids, wts)
    monkeypatch.setenv("MM_STATIC_TILES", "1")
    sta = make_layer(inp, "f32")
    assert sta.plan.reserved[4] == 1 and dyn.plan.reserved[4] == 0
    y_sta, c_sta = sta.forward(x, ids, wts)
    torch.cuda.synchronize()
    assert dyn.device_error(fused=True) == 0 and sta.device_error(fused=True) == 0
    assert torch.equal(y_dyn.view(torch.int32), y_sta.view(torch.int32))
    assert torch.equal(y_dyn.view(torch.int32), y_3.view(torch.int32))
    assert torch.equal(c_dyn, c_sta)


@pytest.mark.parametrize("shape,usecase", [("bm64", "fp8"), ("bm128", "bf16"), ("bm128", "fp8"), ("bm128", "int8"),
                                           ("bm128", "mxfp8"), ("bm256", "bf16"), ("bm256", "fp8"), ("bm256", "int8")])
def test_dependency_schedule_equals_barriers(shape, usecase, monkeypatch):
    """The fused kernel's per-M-block dependency schedule (Linear1, the
    requantisation and Linear2 without grid barriers between them) gives
    the results of the barrier schedule (the default) and of the three-call
    path, bit for bit; masked routes and a shared expert."""
    if shape in FORCED_TILE:
        monkeypatch.setenv("MM_FORCE_TILE", FORCED_TILE[shape])
    cfg = small_cfg(shape, usecase, masked_ratio=0.1, shared=1)
    inp = wl.make_inputs(cfg)
    x, ids, wts = device_inputs(inp)
    log(f"[dependency schedule] {cfg.name}")
    bar = make_layer(inp, "f32")
    monkeypatch.setenv("MM_DEP", "1")
    dep = make_layer(inp, "f32")
    assert dep.plan.reserved[3] == 1 and bar.plan.reserved[3] == 0
    y_dep, c_dep = dep.forward(x, ids, wts)
    y_dep = y_dep.clone()
    y_3, _ = dep.forward_3call(x, ids, wts)
    y_bar, c_bar = bar.forward(x, ids, wts)
    torch.cuda.synchronize()
    assert dep.device_error(fused=True) == 0 and bar.device_error(fused=True) == 0
    assert torch.equal(y_dep.view(torch.int32), y_bar.view(torch.int32))
    assert torch.equal(y_dep.view(torch.int32), y_3.view(torch.int32))
    assert torch.equal(c_dep, c_bar)


@pytest.mark.parametrize("usecase", ["bf16", "fp8"])
@pytest.mark.parametrize("T,E,block_m", [(1024, 32, 128), (1025, 32, 128), (512, 256, 64), (513, 256, 64)])
def test_fused_one_block_dispatch_boundary(T, E, block_m, usecase):
    """The fused kernel dispatches a batch of at most 16 routes per thread
    of a block (8192 with BLOCK_M 128, 4096 with BLOCK_M 64) in one block,
    a larger one over the grid: at and just past each limit, with masked
    routes, the fused result equals the three-call one bit for bit, the
    counts match, and Y is within the oracle tolerance."""
    cfg = wl.Config(f"dispatch_boundary_{usecase}", usecase, T, 512, 256, E, 8, 0.5, 91, masked_ratio=0.1)
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    assert layer.plan.block_m == block_m
    x, ids, wts = device_inputs(inp)
    log(f"[one-block dispatch] {usecase}: {T * 8} routes over {E} experts, BLOCK_M {block_m}")
    y_f, c_f = layer.forward(x, ids, wts)
    y_3, im = layer.forward_3call(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error(fused=True) == 0 and layer.device_error(fused=False) == 0
    assert torch.equal(y_f.view(torch.int32), y_3.view(torch.int32))
    assert torch.equal(c_f, im.expert_counts)
    err = rel_err(y_f.cpu().double().numpy(), oracle_y(inp))
    log(f"    max|dY|/rms = {err:.3e}")
    assert err <= TOL[usecase], err


@pytest.mark.parametrize("usecase", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("shape", ["bm64", "bm128"])
def test_activation_clamp(shape, usecase):
    """The operator's activation_clamp: H (both halves, after dequantisation)
    clamped to [-c, c] before SwiGLU.  With c small enough to clip most of H
    (|H| is about 1 here), Y matches the oracle with the same clamp, differs
    from the unclamped Y by far more than the tolerance, and fused ==
    three-call."""
    cfg = small_cfg(shape, usecase)
    inp = wl.make_inputs(cfg)
    x, ids, wts = device_inputs(inp)
    c = 0.3
    layer = make_layer(inp, "f32", activation_clamp=c)
    log(f"[clamp] {cfg.name}: c = {c}")
    y_f, _ = layer.forward(x, ids, wts)
    y_3, _ = layer.forward_3call(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error(fused=True) == 0 and layer.device_error(fused=False) == 0
    assert torch.equal(y_f.view(torch.int32), y_3.view(torch.int32))
    y_or = oracle_y(inp, activation_clamp=c)
    err = rel_err(y_f.cpu().double().numpy(), y_or)
    log(f"    max|dY|/rms = {err:.3e}")
    assert err <= TOL[usecase], err
    assert rel_err(oracle_y(inp), y_or) > 10 * TOL[usecase]


@pytest.mark.parametrize("usecase", ["bf16", "fp8", "int8"])
def test_fused_deterministic_with_experts_of_several_m_blocks(usecase):
    """Experts of about 500 routes (four M-blocks each, tail tiles in every
    GEMM): the dispatch's atomics place a route in any M-block of its expert,
    and the result must not depend on where: two fused calls and the
    three-call path agree bit for bit."""
    cfg = wl.Config(f"placement_{usecase}", usecase, 2000, 512, 256, 32, 8, 0.5, 93)
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    log(f"[placement] {usecase}")
    y_a, _ = layer.forward(x, ids, wts)
    y_a = y_a.clone()
    y_b, _ = layer.forward(x, ids, wts)
    y_3, _ = layer.forward_3call(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error(fused=True) == 0 and layer.device_error(fused=False) == 0
    assert torch.equal(y_a.view(torch.int32), y_b.view(torch.int32))
    assert torch.equal(y_a.view(torch.int32), y_3.view(torch.int32))


@pytest.mark.parametrize("usecase", ["bf16", "fp8", "int8", "mxfp8"])
@pytest.mark.parametrize("y_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K,shared", [(8, 0), (7, 1), (8, 1)])
@pytest.mark.parametrize("T", [40, 300])
def test_fused_combine_slot_counts(usecase, y_dtype, K, shared, T):
    """The fused kernel's Token Combine takes up to 8 slots a token through
    LDS and more (top-8 plus a shared expert) through registers.  Masked
    routes, a hidden size that ends inside a column segment, 64-row and
    128-row tiles (T = 40 and 300): fused == three-call bit for bit, and
    the float32 Y within the oracle tolerance (the bar is set on float32
    output; bf16 output adds its own rounding)."""
    cfg = wl.Config(f"combine_{usecase}", usecase, T, 1280, 256, 16, K, 0.5, 77, masked_ratio=0.2, shared=shared)
    inp = wl.make_inputs(cfg)
    log(f"[combine] {usecase} y={y_dtype} T={T} K={K} shared={shared}")
    layer = make_layer(inp, y_dtype)
    x, ids, wts = device_inputs(inp)
    y_f, _ = layer.forward(x, ids, wts)
    y_f = y_f.clone()
    y_3, _ = layer.forward_3call(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error(fused=True) == 0 and layer.device_error(fused=False) == 0
    assert torch.equal(y_f.view(torch.int16), y_3.view(torch.int16))
    if y_dtype == "f32":
        err = rel_err(y_f.cpu().double().numpy(), oracle_y(inp))
        assert err <= TOL[usecase], err


@pytest.mark.parametrize("usecase", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("shape", ["max_hidden", "max_intermediate"])
def test_largest_hidden_and_intermediate(shape, usecase):
    """The largest hidden size (16384: the fused kernel quantises a token row
    in two passes, the combine spans 2048 column groups) and the largest
    intermediate size (16384: requantisation rows read twice, 128 Linear1
    column tiles per M-block): oracle tolerance, fused == three-call."""
    T, E, K = 24, 3, 2
    H, I = (16384, 256) if shape == "max_hidden" else (256, 16384)
    cfg = wl.Config(f"{shape}_{usecase}", usecase, T, H, I, E, K, 0.5, 91)
    inp = wl.make_inputs(cfg)
    log(f"[max] {shape} {usecase}")
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    y_f, _ = layer.forward(x, ids, wts)
    y_3, _ = layer.forward_3call(x, ids, wts)
    torch.cuda.synchronize()
    err = rel_err(y_f.cpu().double().numpy(), oracle_y(inp))
    log(f"    max|dY|/rms = {err:.3e}")
    assert err <= TOL[usecase], err
    assert torch.equal(y_f.view(torch.int32), y_3.view(torch.int32))
    assert layer.device_error(fused=True) == 0 and layer.device_error(fused=False) == 0


@pytest.mark.parametrize("tile", ["0", "1"])
@pytest.mark.parametrize("usecase", ["int8", "bf16", "fp8"])
def test_split_tail_tiles(usecase, tile, monkeypatch):
    """Few tiles on many workgroups: the tail tiles are split along K (with
    BLOCK_M 64: eight pieces in Linear1, two in Linear2; with BLOCK_M 128:
    eight and four) and piece 0 adds the others' partial sums in piece order.
    About 32 routes per expert, so every tile has padding rows, whose partial
    sums are not exchanged.  int8 accumulators are exact, so the split result
    equals the unsplit one bit for bit; every use case stays within the
    oracle tolerance, and fused == three-call (each expert has one M-block
    here, so where a route lands does not change how its sums round; float
    use cases split only when asked to)."""
    cfg = wl.Config(f"split_{usecase}", usecase, 64, 4096, 1024, 4, 2, 0.5, 77)
    inp = wl.make_inputs(cfg)
    x, ids, wts = device_inputs(inp)
    monkeypatch.setenv("MM_FORCE_TILE", tile)   # the piece counts above
    monkeypatch.setenv("MM_MAX_SPLIT", "1")     # read when the plan is made
    y_one, _ = make_layer(inp, "f32").forward(x, ids, wts)
    y_one = y_one.clone()
    monkeypatch.setenv("MM_MAX_SPLIT", "8")
    layer = make_layer(inp, "f32")
    assert layer.plan.workspace_bytes > 0
    log(f"[split] {usecase}, BLOCK_M {64 << int(tile)}: unsplit vs split tail tiles")
    y_f, _ = layer.forward(x, ids, wts)
    y_3, _ = layer.forward_3call(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error(fused=True) == 0 and layer.device_error(fused=False) == 0
    assert torch.equal(y_f.view(torch.int32), y_3.view(torch.int32))
    if usecase == "int8":
        assert torch.equal(y_f.view(torch.int32), y_one.view(torch.int32))
    y_or = oracle_y(inp)
    for y in (y_one, y_f):
        err = rel_err(y.cpu().double().numpy(), y_or)
        log(f"    max|dY|/rms = {err:.3e}")
        assert err <= TOL[usecase], err


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_fp8_linear1_modes(mode, monkeypatch):
    """e4m3 Linear1 on the e4m3 MFMA (fast, the default for I >= 1024) or on
    the bf16 MFMA after exact widening (exact, the default below): both stay
    within the fp8 bar at I = 1024, and fused == three-call in each mode."""
    cfg = wl.Config(f"fp8_l1_{mode}", "fp8", 256, 1024, 1024, 8, 4, 0.5, 31)
    inp = wl.make_inputs(cfg)
    x, ids, wts = device_inputs(inp)
    layer = make_layer(inp, "f32")
    monkeypatch.setenv("MM_FP8_L1", mode)
    log(f"[fp8 Linear1] {mode}")
    y_f, _ = layer.forward(x, ids, wts)
    y_3, _ = layer.forward_3call(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error(fused=True) == 0
    assert torch.equal(y_f.view(torch.int32), y_3.view(torch.int32))
    err = rel_err(y_f.cpu().double().numpy(), oracle_y(inp))
    log(f"    max|dY|/rms = {err:.3e}")
    assert err <= TOL["fp8"], err


def test_fused_barrier_timeout_is_reported_and_recovers(monkeypatch):
    """A grid barrier that gives up (forced from the host with a one-poll
    limit) sets its error bit and every block still leaves the kernel; the
    next call with the normal limit is exact again."""
    cfg = small_cfg("bm64", "bf16")
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    y_ok, _ = layer.forward(x, ids, wts)
    y_ok = y_ok.clone()
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    monkeypatch.setenv("MM_BARRIER_SPIN", "1")
    log("[timeout] mega_moe with a one-poll barrier limit")
    layer.forward(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error() & B.MM_DEVERR_BARRIER_TIMEOUT
    monkeypatch.delenv("MM_BARRIER_SPIN")
    y2, _ = layer.forward(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    assert torch.equal(y_ok.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("corrupt", ["past_pool", "unaligned", "count_overflow"])
def test_gemm_rejects_offsets_outside_the_pool(corrupt):
    """Offsets a caller hands to the GEMM entry points that do not describe a
    padded pool of at most P rows run no tile and raise
    MM_DEVERR_BAD_OFFSETS (the kernel never addresses outside the pool)."""
    cfg = small_cfg("bm64", "bf16")
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    im = layer.new_intermediates()
    layer.dispatch(x, ids, im)
    torch.cuda.synchronize()
    assert layer.device_error(fused=False) == 0
    bm = layer.plan.block_m
    off = im.expert_offsets.clone()
    if corrupt == "past_pool":
        off[-1] = layer.plan.pool_rows + bm
    elif corrupt == "unaligned":
        off[1:] += 1
    else:
        im.expert_counts[0] = int(off[1] - off[0]) + 1
    im.expert_offsets.copy_(off)
    log(f"[bad offsets] {corrupt}")
    layer.linear1(im)
    torch.cuda.synchronize()
    assert layer.device_error(fused=False) & B.MM_DEVERR_BAD_OFFSETS


def _edge_inputs(T, H, I, E, K, ids_np, usecase="bf16", seed=77):
    cfg = wl.Config("edge", usecase, T, H, I, E, K, 0.0, seed)
    ids = torch.from_numpy(ids_np.astype(np.int32))
    wts = torch.from_numpy(np.random.default_rng(seed).random((T, K)).astype(np.float32))
    wts[ids < 0] = 0.0
    return wl.Inputs(cfg, wl.tokens(cfg), ids, wts, wl.all_weights(cfg))


@pytest.mark.parametrize("case", ["one_expert", "empty_expert", "single_token", "topk1", "odd_tokens", "ids_out_of_range",
                                  "many_experts", "topk64", "all_masked"])
def test_edge_cases(case):
    H, I = 256, 128
    rng = np.random.default_rng(3)
    if case == "many_experts":   # the largest expert count, almost all of them empty
        T, E, K = 64, 1024, 8
        ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    elif case == "topk64":       # the largest top-k
        T, E, K = 20, 64, 64
        ids = np.stack([rng.permutation(E) for _ in range(T)])
    elif case == "all_masked":   # no route at all: y = 0, no tile runs
        T, E, K = 33, 4, 2
        ids = np.full((T, K), -1)
    elif case == "one_expert":
        T, E, K = 150, 4, 1
        ids = np.full((T, 1), 2)
    elif case == "empty_expert":
        T, E, K = 90, 6, 2
        ids = np.stack([rng.choice([0, 1, 2, 4, 5], 2, replace=False) for _ in range(T)])
    elif case == "single_token":
        T, E, K = 1, 8, 4
        ids = np.array([[7, 0, 3, 5]])
    elif case == "topk1":
        T, E, K = 77, 5, 1
        ids = rng.integers(0, E, (T, 1))
    elif case == "odd_tokens":
        T, E, K = 67, 9, 3
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    else:   # ids >= E are skipped like masked routes
        T, E, K = 40, 4, 2
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
        ids[::5, 1] = E + 3
    inp = _edge_inputs(T, H, I, E, K, ids)
    log(f"[edge] {case}")
    layer = make_layer(inp, "f32")
    x, idt, wts = device_inputs(inp)
    y, counts = layer.forward(x, idt, wts)
    torch.cuda.synchronize()
    ids_or = ids.copy()
    ids_or[ids_or >= E] = -1
    y_or, _ = oracle.moe_forward(inp.x.float().numpy(), ids_or, inp.topk_weights.numpy(), expert_fn(inp), "bf16")
    if case == "all_masked":
        assert not y_or.any() and not y.cpu().numpy().any()
    else:
        assert rel_err(y.cpu().double().numpy(), y_or) <= TOL["bf16"]
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(ids_or[ids_or >= 0], minlength=E))
    assert layer.device_error() == (B.MM_DEVERR_BAD_EXPERT if case == "ids_out_of_range" else 0)


@pytest.mark.parametrize("usecase", ["bf16", "fp8"])
def test_prepare_weights_layout(usecase):
    cfg = small_cfg("bm64", usecase)
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    torch.cuda.synchronize()
    g = layer.plan.gate_up_group
    n = np.arange(2 * cfg.I)
    q, m = n // (2 * g), n % (2 * g)
    col = np.where(m < g, q * g + m, cfg.I + q * g + (m - g))
    view = torch.int16 if usecase == "bf16" else torch.uint8
    w1 = inp.weights.w1.view(view)
    exp1 = w1[:, :, torch.from_numpy(col)].transpose(1, 2).contiguous()
    assert torch.equal(layer.w1.view(view).cpu(), exp1)
    assert torch.equal(layer.w2.view(view).cpu(), inp.weights.w2.view(view).transpose(1, 2).contiguous())


# ---------------------------------------------------------------------------
# MX use cases (MX-FP8 weights; FP8 x FP4)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("order", ["shuffled", "sorted"])
def test_mx_quantiser_all_bf16_patterns(order):
    """Every finite bf16 bit pattern goes through the MX dispatch quantiser
    (groups of 32 along hidden) once: shuffled, a pattern meets groups of any
    spread; sorted by magnitude, every pattern sits next to its group's
    largest.  Codes and E8M0 scales equal the oracle's bit for bit."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    finite = bits[np.isfinite(f)]
    rng = np.random.default_rng(6)
    H = 256
    n = (finite.size + H - 1) // H * H
    pat = np.concatenate([finite, rng.choice(finite, n - finite.size)])
    if order == "shuffled":
        rng.shuffle(pat)
    else:
        pat = pat[np.argsort(np.abs((pat << 16).view(np.float32)), kind="stable")]
    x = torch.from_numpy(pat.astype(np.uint16).view(np.int16).reshape(-1, H)).view(torch.bfloat16)
    T = x.shape[0]
    log(f"[mx quantiser] {order} T={T}")
    layer = moe.ExpertLayer(T, H, 128, 1, 1, "mxfp8", "f32", "cuda")
    im = layer.new_intermediates()
    ids = torch.zeros((T, 1), dtype=torch.int32)
    layer.dispatch(x.cuda(), ids.cuda(), im)
    torch.cuda.synchronize()
    codes, e8 = oracle.mx_quantize(x.float().numpy().astype(np.float64), "e4m3")
    psrc = im.pool_src.cpu().numpy()[:T]
    np.testing.assert_array_equal(im.x_pool.view(-1, H)[:T].cpu().numpy(), codes[psrc])
    np.testing.assert_array_equal(im.x_pool_scale.view(-1, H // 32)[:T].cpu().numpy(), e8[psrc])


MX_SHAPES = {
    "mx_bm128": dict(T=256, H=1024, I=1024, E=8, K=4, bias=0.5),    # 128 rows per expert
    "mx_bm64": dict(T=96, H=1024, I=512, E=16, K=2, bias=1.0),      # 12 rows per expert: BLOCK_M 64
}


@pytest.mark.parametrize("shape", list(MX_SHAPES))
@pytest.mark.parametrize("usecase", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("variant", ["plain", "masked", "shared_active"])
def test_mx_y_parity(shape, usecase, variant):
    """MX-FP8 and FP8 x FP4: Y within the fp8 bar against the oracle (which
    quantises X and the SwiGLU output with Q_MX and multiplies the
    dequantised values), fused == three-call bit for bit, run-to-run
    identical, the dispatch metadata and the MX pool rows (codes and E8M0
    scales) bit-exact; also with masked routes, a shared expert and inactive
    tokens."""
    sh = MX_SHAPES[shape]
    cfg = wl.Config(f"{shape}_{usecase}_{variant}", usecase, sh["T"], sh["H"], sh["I"], sh["E"], sh["K"], sh["bias"],
                    2025, masked_ratio=0.15 if variant != "plain" else 0.0,
                    shared=int(variant == "shared_active"), inactive_ratio=0.3 if variant == "shared_active" else 0.0)
    inp = wl.make_inputs(cfg)
    log(f"[mx y] {cfg.name}")
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    act = device_active(inp)
    y_f, c_f = layer.forward(x, ids, wts, active=act)
    y_f = y_f.clone()
    off, psrc, r2p = (t.cpu().numpy() for t in layer.fused_layout())
    y_f2, _ = layer.forward(x, ids, wts, active=act)
    y_3, im = layer.forward_3call(x, ids, wts, active=act)
    torch.cuda.synchronize()
    assert layer.device_error(fused=True) == 0 and layer.device_error(fused=False) == 0
    assert torch.equal(y_f.view(torch.int32), y_f2.view(torch.int32))
    assert torch.equal(y_f.view(torch.int32), y_3.view(torch.int32))
    check_dispatch(layer, inp, im)
    check_layout(inp, layer.plan.block_m, c_f.cpu().numpy(), off, psrc, r2p)
    err = rel_err(y_f.cpu().double().numpy(), oracle_y(inp))
    log(f"    max|dY|/rms = {err:.3e}")
    assert err <= TOL[usecase], err


def test_mx_swiglu_quantisation_in_the_linear1_epilogue():
    """The three-call Linear1 writes A = Q_MX(SwiGLU(H)) per row: its E8M0
    scales equal the oracle's Q_MX of the SwiGLU of the exact Linear1
    product for all but a few groups (the MFMA's float32 sums can move an
    amax across a power of two); in the groups whose scale agrees, at least
    99 % of the codes agree and no decoded value is more than one e4m3 step
    (of the group's top binade) from the oracle's."""
    cfg = wl.Config("mx_a_pool", "mxfp8", 64, 1024, 1024, 4, 2, 0.3, 77)
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    im = layer.new_intermediates()
    layer.dispatch(x, ids, im)
    layer.linear1(im)
    torch.cuda.synchronize()
    off = im.expert_offsets.cpu().numpy()
    cnt = im.expert_counts.cpu().numpy()
    psrc = im.pool_src.cpu().numpy()
    xc, xe = oracle.mx_quantize(inp.x.float().numpy().astype(np.float64), "e4m3")
    xin = oracle.mx_dequantize(xc, xe, "e4m3")
    a_codes = im.a_pool.view(-1, cfg.I).cpu().numpy()
    a_e8 = im.a_pool_scale.view(-1, cfg.I // 32).cpu().numpy()
    expert = expert_fn(inp)
    n_groups = n_same = n_codes = n_codes_same = 0
    for e in range(cfg.E):
        rows = np.arange(off[e], off[e] + cnt[e])
        if rows.size == 0:
            continue
        w1 = oracle.mx_dequantize(expert(e)[0].T, expert(e)[2], "e4m3").T
        u = oracle.swiglu(xin[psrc[rows] // cfg.K] @ w1)
        uc, ue = oracle.mx_quantize(u, "e4m3")
        same = ue == a_e8[rows]                                          # [rows, groups]
        n_groups += ue.size
        n_same += int(same.sum())
        gc = a_codes[rows].reshape(rows.size, -1, 32)[same]
        oc = uc.reshape(rows.size, -1, 32)[same]
        n_codes += gc.size
        n_codes_same += int((gc == oc).sum())
        step = np.ldexp(1.0, ue[same].astype(int) - 127 + 8 - 3)[:, None]   # e4m3 step of the top binade
        assert np.all(np.abs(oracle.e4m3_decode(gc) - oracle.e4m3_decode(oc)) * np.ldexp(1.0, ue[same].astype(int) - 127)[:, None]
                      <= step * (1 + 1e-9))
    log(f"[mx a_pool] E8M0 equal on {n_same} of {n_groups} groups, codes {n_codes_same} of {n_codes}")
    assert n_same >= 0.99 * n_groups and n_codes_same >= 0.99 * n_codes


# ---------------------------------------------------------------------------
# full-size configurations, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

def _tokens_covering_every_m_block(inp, offs, psrc, block_m, extra, seed=11):
    """One token of the first and of the last valid row of every M-block of
    every expert (so every tile row-block and every ragged tail is compared),
    plus `extra` random tokens."""
    c = inp.cfg
    Ks = c.K + c.shared
    ids = oracle_routes(inp)
    counts = np.bincount(ids[ids >= 0].ravel(), minlength=c.E + c.shared)
    toks = set()
    for e in range(c.E + c.shared):
        for j in range(0, counts[e], block_m):
            for r in (j, min(counts[e], j + block_m) - 1):
                toks.add(int(psrc[offs[e] + r]) // Ks)
    rng = np.random.default_rng(seed)
    toks.update(rng.choice(c.T, min(c.T, extra), replace=False).tolist())
    return np.array(sorted(toks))


FULL = ["tiny_bf16", "mid_bf16", "dsv3_bf16", "dsv3_fp8_t128", "dsv3_bf16_t128", "dsv3_fp8_t16384", "dsv3_int8",
        "dsv3_bf16_t16384", "dsv3_mxfp8_t128", "dsv3_mxfp4_t128", "dsv3_mxfp8_t16384", "dsv3_mxfp4_t16384"]


@pytest.mark.parametrize("name", FULL)
def test_full_config(name):
    """Every workload at its full size, through mega_moe as the benchmark
    times it: the fused kernel's own dispatch metadata (offsets, pool rows,
    inverse map) bit-exact against the oracle; two fused calls and the
    three-call path agree bit for bit; the three-call dispatch bit-exact too
    (pool rows sampled); Y within the oracle tolerance on every token up to
    4096 tokens, else on a token of the first and last row of every M-block
    of every expert plus 512 random ones."""
    cfg = wl.CONFIGS[name]
    log(f"[full] {name}: generating inputs")
    inp = cpu_inputs(cfg)
    x, ids, wts = device_inputs(inp)
    layer = make_layer(inp, "f32")
    y32, counts = layer.forward(x, ids, wts)
    y32 = y32.clone()
    off, psrc, r2p = (t.cpu().numpy() for t in layer.fused_layout())
    y_again, _ = layer.forward(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error(fused=True) == 0
    assert torch.equal(y32.view(torch.int32), y_again.view(torch.int32)), "two calls differ"
    del y_again
    log(f"[full] {name}: fused metadata")
    check_layout(inp, layer.plan.block_m, counts.cpu().numpy(), off, psrc, r2p)
    y3, im = layer.forward_3call(x, ids, wts)
    torch.cuda.synchronize()
    assert layer.device_error(fused=False) == 0
    assert torch.equal(y32.view(torch.int32), y3.view(torch.int32)), "fused != three-call"
    log(f"[full] {name}: three-call metadata")
    check_dispatch(layer, inp, im, sample_rows=4096)
    del y3, im
    layer._ws = None
    if cfg.T <= 4096:
        tokens = np.arange(cfg.T)
    else:
        tokens = _tokens_covering_every_m_block(inp, off, psrc, layer.plan.block_m, extra=512)
    log(f"[full] {name}: oracle on {tokens.size} tokens")
    y_or = oracle_y(inp, tokens=tokens)
    err = rel_err(y32[torch.from_numpy(tokens).cuda()].cpu().double().numpy(), y_or)
    log(f"[full] {name}: max|dY|/rms = {err:.3e}")
    assert err <= TOL[cfg.usecase], err
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode,bound", [("exact", 1e-6), ("fast", 2e-4)])
def test_fp8_linear1_accumulator_deviation(mode, bound, monkeypatch):
    """How far Linear1's float32 sums of e4m3 code products are from the
    exact sums (numpy float64 of the same codes): the exact mode (bf16 MFMA
    on exactly widened codes) is float32 rounding only; the e4m3 MFMA rounds
    inside each instruction, about 4e-5 of the result's RMS (the reason MX
    and small-I Linear1 default to the exact mode)."""
    cfg = wl.Config(f"fp8_dev_{mode}", "fp8", 128, 1024, 512, 4, 2, 0.3, 88)
    inp = wl.make_inputs(cfg)
    layer = make_layer(inp, "f32")
    x, ids, wts = device_inputs(inp)
    im = layer.new_intermediates()
    layer.dispatch(x, ids, im)
    monkeypatch.setenv("MM_FP8_L1", mode)
    P = layer.plan.pool_rows
    c1 = torch.empty((P, 2 * cfg.I), dtype=torch.int32, device="cuda")
    B.mm_debug_raw_accumulators(layer.plan, 1, im.expert_offsets, im.expert_counts, im.x_pool, layer.w1, c1,
                                layer.workspace(False))
    torch.cuda.synchronize()
    c1 = c1.view(torch.float32).cpu().numpy().astype(np.float64)
    offs = im.expert_offsets.cpu().numpy()
    counts = im.expert_counts.cpu().numpy()
    xq = oracle.e4m3_decode(im.x_pool.view(-1, cfg.H).cpu().numpy())
    se = sr = 0.0
    for e in range(cfg.E):
        rows = np.arange(offs[e], offs[e] + counts[e])
        if rows.size == 0:
            continue
        ref = xq[rows] @ oracle.e4m3_decode(inp.weights.w1[e].view(torch.uint8).numpy())
        se += float(((c1[rows] - ref) ** 2).sum())
        sr += float((ref ** 2).sum())
    dev = np.sqrt(se / sr)
    log(f"[fp8 accumulators] {mode}: rms(sum - exact) / rms(exact) = {dev:.3e}")
    assert dev <= bound, dev
