"""Device-memory plumbing around the C ABI (torch allocates, the library computes).

``ExpertLayer`` holds one plan, the prepared expert weights and a
workspace, and calls the C-ABI entry points through ``binding``.  Nothing
here computes any part of the expert path.
"""

from __future__ import annotations

import dataclasses

import torch

from . import binding as B

_DT = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "int8": torch.int8, "mxfp8": torch.uint8,
       "mxfp4": torch.uint8}
MX = ("mxfp8", "mxfp4")


@dataclasses.dataclass
class Intermediates:
    expert_counts: torch.Tensor
    expert_offsets: torch.Tensor
    pool_src: torch.Tensor
    route_to_pool: torch.Tensor
    x_pool: torch.Tensor
    x_pool_scale: torch.Tensor | None
    a_pool: torch.Tensor
    a_pool_scale: torch.Tensor | None


class ExpertLayer:
    def __init__(self, T, H, I, E, K, usecase="bf16", y_dtype="bf16", device="cuda", activation_clamp=None,
                 num_shared_experts=0):
        self.T, self.H, self.I, self.E, self.K = T, H, I, E, K
        self.S = int(num_shared_experts)
        self.Et, self.Ks = E + self.S, K + self.S      # experts with weights; slots per token
        self.usecase = usecase
        self.y_dtype = y_dtype
        self.device = torch.device(device)
        self.plan = B.mm_plan_create(T, H, I, E, K, usecase, y_dtype, activation_clamp, self.S)
        self.w1 = self.w2 = self.s1 = self.s2 = None
        self._ws = None
        self._fused_ws = None

    # ---------------------------------------------------------------- weights
    def load_weights(self, w1, w2, s1=None, s2=None, stream=None):
        """Upload formula-layout weights ([E+S,H,2I], [E+S,I,H]; a shared expert last; e2m1 packed two per
        byte along the last dimension) and relayout them once.  Scales: float32 per output channel (A8W8)
        or E8M0 bytes [E+S][N][K_in/32] (MX)."""
        dt = _DT[self.usecase]
        w1d = w1.to(self.device).contiguous()
        w2d = w2.to(self.device).contiguous()
        assert w1d.dtype == dt and w2d.dtype == dt
        Et = self.Et
        half = 2 if self.usecase == "mxfp4" else 1
        assert tuple(w1d.shape) == (Et, self.H, 2 * self.I // half) and tuple(w2d.shape) == (Et, self.I, self.H // half)
        self.w1 = torch.empty((Et, 2 * self.I, self.H // half), dtype=dt, device=self.device)
        self.w2 = torch.empty((Et, self.H, self.I // half), dtype=dt, device=self.device)
        B.mm_prepare_weights(self.plan, w1d, w2d, self.w1, self.w2, stream)
        if self.usecase in MX:
            assert tuple(s1.shape) == (Et, 2 * self.I, self.H // 32) and tuple(s2.shape) == (Et, self.H, self.I // 32)
            self.s1 = s1.to(self.device, torch.uint8).contiguous()
            self.s2 = s2.to(self.device, torch.uint8).contiguous()
        elif self.usecase != "bf16":
            self.s1 = s1.to(self.device, torch.float32).contiguous()
            self.s2 = s2.to(self.device, torch.float32).contiguous()
        torch.cuda.current_stream(self.device).synchronize() if stream is None else None
        del w1d, w2d

    # -------------------------------------------------------------- buffers
    def workspace(self, fused: bool) -> torch.Tensor:
        n = self.plan.fused_workspace_bytes if fused else self.plan.workspace_bytes
        attr = "_fused_ws" if fused else "_ws"
        ws = getattr(self, attr)
        if ws is None or ws.numel() < n:
            ws = torch.empty(n, dtype=torch.uint8, device=self.device)
            setattr(self, attr, ws)
        return ws

    def new_intermediates(self) -> Intermediates:
        P, dev = self.plan.pool_rows, self.device
        q = self.usecase != "bf16"
        es = 2 if self.usecase == "bf16" else 1
        i32 = dict(dtype=torch.int32, device=dev)
        return Intermediates(
            expert_counts=torch.empty(self.Et, **i32),
            expert_offsets=torch.empty(self.Et + 1, **i32),
            pool_src=torch.empty(P, **i32),
            route_to_pool=torch.empty(self.T * self.Ks, **i32),
            x_pool=torch.empty(P * self.H * es, dtype=torch.uint8, device=dev),
            x_pool_scale=self._scale_buf(self.plan.x_pool_scale_bytes) if q else None,
            a_pool=torch.empty(P * self.I * es, dtype=torch.uint8, device=dev),
            a_pool_scale=self._scale_buf(self.plan.a_pool_scale_bytes) if q else None,
        )

    def _scale_buf(self, nbytes):
        """float32 [P] (A8W8) or E8M0 bytes [P][K_in/32] (MX) of a pool."""
        if self.usecase in MX:
            return torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return torch.empty(nbytes // 4, dtype=torch.float32, device=self.device)

    def new_y(self):
        dt = torch.float32 if self.y_dtype in ("f32", "fp32") else torch.bfloat16
        return torch.empty((self.T, self.H), dtype=dt, device=self.device)

    # -------------------------------------------------------------- entries
    def forward(self, x, topk_ids, topk_weights, y=None, counts=None, stream=None, active=None):
        """mega_moe: returns (y, expert_token_nums).  active: int8 [T] x_active_mask or None."""
        y = self.new_y() if y is None else y
        counts = torch.empty(self.E, dtype=torch.int32, device=self.device) if counts is None else counts
        B.mega_moe(self.plan, x, topk_ids, topk_weights, active, self.w1, self.s1, self.w2, self.s2, y, counts,
                   self.workspace(True), stream)
        return y, counts

    def fused_layout(self):
        """Dispatch metadata the last forward() built in its workspace: (offsets, pool_src, route_to_pool)."""
        i32 = dict(dtype=torch.int32, device=self.device)
        off = torch.empty(self.Et + 1, **i32)
        psrc = torch.empty(self.plan.pool_rows, **i32)
        r2p = torch.empty(self.T * self.Ks, **i32)
        B.mm_debug_fused_layout(self.plan, self.workspace(True), off, psrc, r2p)
        return off, psrc, r2p

    def device_error(self, fused: bool = True) -> int:
        """The device error word of the last call on this layer's workspace
        (mm_device_error bits; waits for the device)."""
        return B.mm_read_device_error(self.plan, self.workspace(fused))

    def dispatch(self, x, topk_ids, im: Intermediates, stream=None, active=None):
        B.mm_dispatch_layout(self.plan, topk_ids, active, x, im.expert_counts, im.expert_offsets, im.pool_src,
                             im.route_to_pool, im.x_pool, im.x_pool_scale, self.workspace(False), stream)

    def linear1(self, im: Intermediates, stream=None):
        B.mm_grouped_l1_swiglu(self.plan, im.expert_offsets, im.expert_counts, im.x_pool, im.x_pool_scale,
                               self.w1, self.s1, im.a_pool, im.a_pool_scale, self.workspace(False), stream)

    def linear2_combine(self, im: Intermediates, topk_weights, y, stream=None):
        B.mm_grouped_l2_combine(self.plan, im.expert_offsets, im.expert_counts, im.pool_src, im.route_to_pool,
                                im.a_pool, im.a_pool_scale, self.w2, self.s2, topk_weights, y,
                                self.workspace(False), stream)

    def forward_3call(self, x, topk_ids, topk_weights, stream=None, active=None):
        im = self.new_intermediates()
        y = self.new_y()
        self.dispatch(x, topk_ids, im, stream, active)
        self.linear1(im, stream)
        self.linear2_combine(im, topk_weights, y, stream)
        return y, im
