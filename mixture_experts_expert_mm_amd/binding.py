"""ctypes binding of include/megamoe.h: argument marshalling only.

Every function takes torch tensors (device memory) or plain integers and
forwards raw pointers to the C ABI of libmegamoe.so; all work happens in the
HIP kernels.  If the library is missing this module raises -- there is no
fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

from . import _build

MM_A16W16, MM_A8W8_FP8, MM_A8W8_INT8, MM_MXFP8, MM_MXFP4 = 0, 1, 2, 3, 4
MM_OUT_BF16, MM_OUT_F32 = 0, 1
USECASE = {"bf16": MM_A16W16, "fp8": MM_A8W8_FP8, "int8": MM_A8W8_INT8, "mxfp8": MM_MXFP8, "mxfp4": MM_MXFP4}
KERNEL_IDS = 10
MM_DEVERR_BAD_EXPERT, MM_DEVERR_BARRIER_TIMEOUT, MM_DEVERR_BAD_OFFSETS = 1, 2, 4


class MMProblem(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("intermediate_hidden", ctypes.c_int64),
        ("num_experts", ctypes.c_int64),
        ("num_topk", ctypes.c_int64),
        ("usecase", ctypes.c_int32),
        ("y_dtype", ctypes.c_int32),
        ("clamp_activation", ctypes.c_int32),
        ("activation_clamp", ctypes.c_float),
        ("num_shared_experts", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
    ]


class MMPlan(ctypes.Structure):
    _fields_ = [
        ("prob", MMProblem),
        ("block_m", ctypes.c_int32),
        ("tile_l1", ctypes.c_int32),
        ("tile_l2", ctypes.c_int32),
        ("gate_up_group", ctypes.c_int32),
        ("pool_rows", ctypes.c_int64),
        ("x_pool_bytes", ctypes.c_int64),
        ("a_pool_bytes", ctypes.c_int64),
        ("x_pool_scale_bytes", ctypes.c_int64),
        ("a_pool_scale_bytes", ctypes.c_int64),
        ("w1_bytes", ctypes.c_int64),
        ("w2_bytes", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("fused_workspace_bytes", ctypes.c_int64),
        ("checksum", ctypes.c_uint64),
        ("reserved", ctypes.c_int64 * 8),
    ]


EXPORTS = [
    "mm_plan_create", "mm_prepare_weights", "mm_dispatch_layout", "mm_grouped_l1_swiglu",
    "mm_grouped_l2_combine", "mega_moe", "mega_moe_noalloc", "mm_read_device_error", "mm_debug_raw_accumulators",
    "mm_debug_fused_layout", "mm_read_kernel_clock", "mm_trace_enable", "mm_trace_collect", "mm_kernel_name", "mm_status_string",
]

_lib = None


class MMError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def lib_path() -> str:
    return _build.LIB


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32p, f32p, u64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64
    P = ctypes.POINTER(MMPlan)
    lib.mm_plan_create.argtypes = [ctypes.POINTER(MMProblem), P]
    lib.mm_prepare_weights.argtypes = [P, vp, vp, vp, vp, vp]
    lib.mm_dispatch_layout.argtypes = [P, i32p, vp, vp, i32p, i32p, i32p, i32p, vp, f32p, vp, u64, vp]
    lib.mm_grouped_l1_swiglu.argtypes = [P, i32p, i32p, vp, f32p, vp, f32p, vp, f32p, vp, u64, vp]
    lib.mm_grouped_l2_combine.argtypes = [P, i32p, i32p, i32p, i32p, vp, f32p, vp, f32p, f32p, vp, vp, u64, vp]
    lib.mega_moe.argtypes = [P, vp, i32p, f32p, vp, vp, f32p, vp, f32p, vp, i32p, vp, u64, vp]
    lib.mega_moe_noalloc.argtypes = [P, vp, i32p, f32p, vp, vp, f32p, vp, f32p, vp, i32p, vp]
    lib.mm_read_device_error.argtypes = [P, vp, ctypes.POINTER(ctypes.c_int32), vp]
    lib.mm_debug_raw_accumulators.argtypes = [P, ctypes.c_int, i32p, i32p, vp, vp, i32p, vp, u64, vp]
    lib.mm_debug_fused_layout.argtypes = [P, vp, i32p, i32p, i32p, vp]
    lib.mm_read_kernel_clock.argtypes = [P, vp, ctypes.POINTER(ctypes.c_uint64), vp]
    lib.mm_trace_enable.argtypes = [ctypes.c_int]
    lib.mm_trace_collect.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]
    lib.mm_kernel_name.argtypes = [ctypes.c_int]
    lib.mm_kernel_name.restype = ctypes.c_char_p
    lib.mm_status_string.argtypes = [ctypes.c_int]
    lib.mm_status_string.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("mm_kernel_name", "mm_status_string"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mm_status_string(status).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, st):
    if st != 0:
        raise MMError(fn, st)


# ------------------------------------------------------------------ entries

def mm_plan_create(T, H, I, E, K, usecase="bf16", y_dtype="bf16", activation_clamp=None,
                   num_shared_experts=0) -> MMPlan:
    """activation_clamp: None (no clamp) or c >= 0 (H clamped to [-c, c] before SwiGLU);
    num_shared_experts: 0 or 1 (expert index E of the weight arrays)."""
    prob = MMProblem(T, H, I, E, K, USECASE.get(usecase, usecase) if isinstance(usecase, str) else usecase,
                     MM_OUT_F32 if y_dtype in ("f32", "fp32", MM_OUT_F32) else MM_OUT_BF16,
                     0 if activation_clamp is None else 1, 0.0 if activation_clamp is None else float(activation_clamp),
                     int(num_shared_experts), 0)
    plan = MMPlan()
    _check("mm_plan_create", load().mm_plan_create(ctypes.byref(prob), ctypes.byref(plan)))
    return plan


def mm_prepare_weights(plan, w1, w2, w1_out, w2_out, stream=None):
    _check("mm_prepare_weights", load().mm_prepare_weights(
        ctypes.byref(plan), _ptr(w1), _ptr(w2), _ptr(w1_out), _ptr(w2_out), _stream(stream)))


def mm_dispatch_layout(plan, topk_ids, x_active_mask, x, expert_counts, expert_offsets, pool_src, route_to_pool,
                       x_pool, x_pool_scale, workspace, stream=None):
    _check("mm_dispatch_layout", load().mm_dispatch_layout(
        ctypes.byref(plan), _ptr(topk_ids), _ptr(x_active_mask), _ptr(x), _ptr(expert_counts), _ptr(expert_offsets),
        _ptr(pool_src), _ptr(route_to_pool), _ptr(x_pool), _ptr(x_pool_scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mm_grouped_l1_swiglu(plan, expert_offsets, expert_counts, x_pool, x_pool_scale, w1, w1_scale,
                         a_pool, a_pool_scale, workspace, stream=None):
    _check("mm_grouped_l1_swiglu", load().mm_grouped_l1_swiglu(
        ctypes.byref(plan), _ptr(expert_offsets), _ptr(expert_counts), _ptr(x_pool), _ptr(x_pool_scale),
        _ptr(w1), _ptr(w1_scale), _ptr(a_pool), _ptr(a_pool_scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mm_grouped_l2_combine(plan, expert_offsets, expert_counts, pool_src, route_to_pool, a_pool,
                          a_pool_scale, w2, w2_scale, topk_weights, y, workspace, stream=None):
    _check("mm_grouped_l2_combine", load().mm_grouped_l2_combine(
        ctypes.byref(plan), _ptr(expert_offsets), _ptr(expert_counts), _ptr(pool_src), _ptr(route_to_pool),
        _ptr(a_pool), _ptr(a_pool_scale), _ptr(w2), _ptr(w2_scale), _ptr(topk_weights), _ptr(y),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def mega_moe(plan, x, topk_ids, topk_weights, x_active_mask, w1, w1_scale, w2, w2_scale, y, expert_token_nums,
             workspace, stream=None):
    _check("mega_moe", load().mega_moe(
        ctypes.byref(plan), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(x_active_mask), _ptr(w1), _ptr(w1_scale),
        _ptr(w2), _ptr(w2_scale), _ptr(y), _ptr(expert_token_nums), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mega_moe_noalloc(plan, x, topk_ids, topk_weights, x_active_mask, w1, w1_scale, w2, w2_scale, y,
                     expert_token_nums, stream=None):
    _check("mega_moe_noalloc", load().mega_moe_noalloc(
        ctypes.byref(plan), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(x_active_mask), _ptr(w1),
        _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(y), _ptr(expert_token_nums), _stream(stream)))


def mm_read_device_error(plan, workspace, stream=None) -> int:
    """The device error word (mm_device_error bits) of the last call on `workspace`."""
    out = ctypes.c_int32(0)
    _check("mm_read_device_error", load().mm_read_device_error(
        ctypes.byref(plan), _ptr(workspace), ctypes.byref(out), _stream(stream)))
    torch.cuda.synchronize()
    return out.value


def mm_read_kernel_clock(plan, workspace, stream=None):
    """(shader clocks, 100 MHz ticks) spanned by workgroup 0 of the last mega_moe call; waits for the device."""
    out = (ctypes.c_uint64 * 4)()
    _check("mm_read_kernel_clock", load().mm_read_kernel_clock(ctypes.byref(plan), _ptr(workspace), out,
                                                                _stream(stream)))
    torch.cuda.synchronize()
    return out[1] - out[0], out[3] - out[2]


def mm_debug_raw_accumulators(plan, which, expert_offsets, expert_counts, act_pool, w_prepared, c_out,
                              workspace, stream=None):
    _check("mm_debug_raw_accumulators", load().mm_debug_raw_accumulators(
        ctypes.byref(plan), which, _ptr(expert_offsets), _ptr(expert_counts), _ptr(act_pool),
        _ptr(w_prepared), _ptr(c_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def mm_debug_fused_layout(plan, workspace, offsets_out, pool_src_out, route_to_pool_out, stream=None):
    _check("mm_debug_fused_layout", load().mm_debug_fused_layout(
        ctypes.byref(plan), _ptr(workspace), _ptr(offsets_out), _ptr(pool_src_out), _ptr(route_to_pool_out),
        _stream(stream)))


def mm_trace_enable(on: bool):
    _check("mm_trace_enable", load().mm_trace_enable(1 if on else 0))


def mm_trace_collect():
    """Returns {kernel name: (launches, total ms)} and clears the record."""
    n = (ctypes.c_int32 * KERNEL_IDS)()
    ms = (ctypes.c_double * KERNEL_IDS)()
    _check("mm_trace_collect", load().mm_trace_collect(n, ms))
    return {load().mm_kernel_name(i).decode(): (n[i], ms[i]) for i in range(KERNEL_IDS)}


def mm_kernel_name(i: int) -> str:
    return load().mm_kernel_name(i).decode()
