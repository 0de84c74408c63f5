"""The C-ABI library on the host (no GPU): it loads, exports every symbol the
header declares, and its host-side planning and argument validation return
the documented status codes before any HIP call."""

import ctypes
import os
import re

import pytest

from mixture_experts_expert_mm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "megamoe.h")


def _lib():
    if not os.path.exists(B.lib_path()):
        from mixture_experts_expert_mm_amd import _build
        _build.build()
    return B.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mm_plan_create", "mm_prepare_weights", "mm_dispatch_layout", "mm_grouped_l1_swiglu",
              "mm_grouped_l2_combine", "mega_moe", "mm_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(B.EXPORTS)


def test_struct_sizes_match_header():
    # mm_problem: 5 int64 + 3 int32 + float + 2 int32; mm_plan: problem + 4 int32 + 9 int64 + u64 + 8 int64
    assert ctypes.sizeof(B.MMProblem) == 64
    assert ctypes.sizeof(B.MMPlan) == 64 + 16 + 72 + 8 + 64


def test_plan_sizes_and_block_m():
    _lib()
    p = B.mm_plan_create(4096, 7168, 2048, 32, 8, "bf16")   # 1024 rows per expert: 256 x 256
    assert p.block_m == 256
    assert B.mm_plan_create(2048, 7168, 2048, 32, 8, "bf16").block_m == 128   # 512 rows per expert
    R = 4096 * 8
    assert p.pool_rows % p.block_m == 0
    assert p.pool_rows >= R + 32 * (p.block_m - 1)
    assert p.x_pool_bytes == p.pool_rows * 7168 * 2
    assert p.w1_bytes == 32 * 7168 * 4096 * 2
    assert p.fused_workspace_bytes > p.workspace_bytes > 0
    t128 = B.mm_plan_create(128, 7168, 2048, 32, 8, "fp8")   # 32 rows per expert
    assert t128.block_m == 128
    small = B.mm_plan_create(64, 7168, 2048, 32, 8, "fp8")    # 16 rows per expert
    assert small.block_m == 64 and small.x_pool_bytes == small.pool_rows * 7168
    tiny = B.mm_plan_create(20, 256, 128, 16, 2, "int8")
    assert tiny.block_m == 64


@pytest.mark.parametrize("dims", [
    (0, 256, 128, 8, 2), (64, 100, 128, 8, 2), (64, 256, 100, 8, 2), (64, 256, 128, 0, 1),
    (64, 256, 128, 8, 9), (64, 256, 128, 2000, 2), (64, 256, 128, 128, 65),
])
def test_plan_rejects_bad_dimensions(dims):
    _lib()
    with pytest.raises(B.MMError) as ei:
        B.mm_plan_create(*dims, "bf16")
    assert ei.value.status == 1


def test_plan_with_shared_expert():
    _lib()
    p0 = B.mm_plan_create(4096, 7168, 2048, 32, 8, "fp8")
    p1 = B.mm_plan_create(4096, 7168, 2048, 32, 8, "fp8", num_shared_experts=1)
    assert p1.prob.num_shared_experts == 1
    R1 = 4096 * 9                        # one shared slot per token
    assert p1.pool_rows % p1.block_m == 0 and p1.pool_rows >= R1 + 33 * (p1.block_m - 1)
    assert p1.w1_bytes == 33 * 7168 * 4096 and p1.w2_bytes == 33 * 2048 * 7168
    assert p1.fused_workspace_bytes > p0.fused_workspace_bytes
    B.mm_plan_create(64, 256, 128, 64, 63, "bf16", num_shared_experts=1)      # 64 slots: the limit


@pytest.mark.parametrize("dims,shared", [((64, 256, 128, 8, 2), 2), ((64, 256, 128, 8, 2), -1),
                                         ((64, 256, 128, 64, 64), 1), ((64, 256, 128, 1024, 2), 1)])
def test_plan_rejects_bad_shared_experts(dims, shared):
    _lib()
    with pytest.raises(B.MMError) as ei:
        B.mm_plan_create(*dims, "bf16", num_shared_experts=shared)
    assert ei.value.status == 1


def test_plan_rejects_nonzero_reserved():
    lib = _lib()
    prob = B.MMProblem(64, 256, 128, 8, 2, B.MM_A16W16, B.MM_OUT_BF16, 0, 0.0, 0, 5)
    assert lib.mm_plan_create(ctypes.byref(prob), ctypes.byref(B.MMPlan())) == 1


@pytest.mark.parametrize("flag,clamp", [(1, -0.5), (1, float("nan")), (2, 1.0)])
def test_plan_rejects_bad_activation_clamp(flag, clamp):
    lib = _lib()
    prob = B.MMProblem(64, 256, 128, 8, 2, B.MM_A16W16, B.MM_OUT_BF16, flag, clamp)
    plan = B.MMPlan()
    assert lib.mm_plan_create(ctypes.byref(prob), ctypes.byref(plan)) == 1   # MM_ERR_INVALID_ARG


def test_plan_accepts_activation_clamp():
    _lib()
    for c in (None, 0.0, 2.5):
        plan = B.mm_plan_create(64, 256, 128, 8, 2, "bf16", activation_clamp=c)
        assert plan.prob.clamp_activation == (0 if c is None else 1)


def test_plan_mx_sizes():
    _lib()
    for uc, wdiv in (("mxfp8", 1), ("mxfp4", 2)):
        p = B.mm_plan_create(4096, 7168, 2048, 32, 8, uc)
        assert p.x_pool_scale_bytes == p.pool_rows * 7168 // 32
        assert p.a_pool_scale_bytes == p.pool_rows * 2048 // 32
        assert p.w1_bytes == 32 * 7168 * 4096 // wdiv and p.w2_bytes == 32 * 2048 * 7168 // wdiv
    q = B.mm_plan_create(64, 256, 128, 8, 2, "int8")
    assert q.x_pool_scale_bytes == q.pool_rows * 4 == q.a_pool_scale_bytes
    assert B.mm_plan_create(64, 256, 128, 8, 2, "bf16").x_pool_scale_bytes == 0
    with pytest.raises(B.MMError):                         # MX holds at most 512 experts
        B.mm_plan_create(64, 256, 128, 600, 2, "mxfp8")


def test_plan_rejects_unknown_usecase():
    _lib()
    with pytest.raises(B.MMError) as ei:
        B.mm_plan_create(64, 256, 128, 8, 2, 7)
    assert ei.value.status == 2


def test_entry_points_validate_before_any_hip_call():
    lib = _lib()
    plan = B.mm_plan_create(64, 256, 128, 8, 2, "bf16")
    good = 1 << 20          # an aligned fake address; never dereferenced on these paths
    P = ctypes.byref(plan)
    # NULL pointer (x_active_mask, the fifth argument, may be NULL)
    assert lib.mega_moe(P, None, good, good, None, good, None, good, None, good, good, good, 1 << 40, None) == 1
    # misaligned pointer
    assert lib.mega_moe(P, good + 2, good, good, None, good, None, good, None, good, good, good, 1 << 40, None) == 1
    # workspace too small
    assert lib.mega_moe(P, good, good, good, None, good, None, good, None, good, good, good, 16, None) == 3
    assert lib.mm_dispatch_layout(P, good, None, good, good, good, good, good, good, None, good, 16, None) == 3
    # a modified plan is rejected
    bad = B.MMPlan.from_buffer_copy(plan)
    bad.pool_rows += 1
    assert lib.mega_moe(ctypes.byref(bad), good, good, good, None, good, None, good, None, good, good, good,
                        1 << 40, None) == 1
    # quantised plans need the scales
    q = B.mm_plan_create(64, 256, 128, 8, 2, "int8")
    assert lib.mega_moe(ctypes.byref(q), good, good, good, None, good, None, good, None, good, good, good,
                        1 << 40, None) == 1
    # the error word needs a host destination
    assert lib.mm_read_device_error(P, good, None, None) == 1
    # raw accumulators exist for int8 and fp8 only, and need a large enough workspace
    assert lib.mm_debug_raw_accumulators(P, 1, good, good, good, good, good, good, 1 << 40, None) == 2
    assert lib.mm_debug_raw_accumulators(ctypes.byref(q), 3, good, good, good, good, good, good, 1 << 40, None) == 1
    assert lib.mm_debug_raw_accumulators(ctypes.byref(q), 1, good, good, good, good, good, good, 16, None) == 3
    # the fused-layout reader needs its three destinations
    assert lib.mm_debug_fused_layout(P, good, good, None, good, None) == 1


def test_names():
    _lib()
    assert B.status_string(3) == "workspace too small"
    assert B.mm_kernel_name(4) == "l1_swiglu"
    assert B.mm_kernel_name(9) == "mega"
