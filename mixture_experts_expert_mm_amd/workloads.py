"""Seeded synthetic inputs for the routed-expert path.

This module only draws and stores inputs; it holds none of the expert path's
arithmetic (no dispatch, no GEMM, no SwiGLU, no activation quantisation, no
combine).  Both the CPU oracle and the GPU path are fed from here.

Recipe (all draws are numpy PCG64, float32):

* Expert weights, one stream per expert ``default_rng([seed, 0, e])``:
  ``W1[e] ~ N(0,1)/sqrt(hidden)`` of shape ``[hidden, 2*intermediate]`` then
  ``W2[e] ~ N(0,1)/sqrt(intermediate)`` of shape ``[intermediate, hidden]``,
  both rounded to bf16 (the model weights).  The layout is the one of the
  Formula paragraph of the Ascend ``mega_moe`` operator page
  (``W1 in R^{E x hidden x 2I}``, ``W2 in R^{E x I x hidden}``).
* Per-expert routing bias ``default_rng([seed, 2]) ~ N(0,1) * bias_std``
  (``bias_std = 0.5`` for the skewed DeepSeek-V3-like shapes, 0 otherwise).
* Router scores ``default_rng([seed, 1, T]) ~ N(0,1)`` of shape ``[T, E]``
  plus the bias; ``topk_ids`` are the K largest (descending, ties to the
  lower expert id), ``topk_weights`` the float32 softmax over the K selected
  scores.  The pages' own examples draw top-k of randn scores the same way
  (Ascend page, Example; DeepEP metadata notes, section 4.1).
* Tokens ``X ~ N(0,1)`` rounded to bf16, drawn in row chunks of 1024 with
  stream ``default_rng([seed, 3, T, chunk])``.
* Optional masked routes (DeepEP metadata notes, section 5.2): each route is
  set to id -1 with probability ``masked_ratio`` (stream
  ``default_rng([seed, 4, T])``) and its weight to 0.
* Optional shared expert (DeepGEMM MegaMoE page, section 6): ``shared = 1``
  adds expert index ``E`` to the weight arrays, drawn like a routed expert
  (stream ``default_rng([seed, 0, E])``).
* Optional x_active_mask (Ascend page, Parameters): each token is inactive
  with probability ``inactive_ratio`` (stream ``default_rng([seed, 5, T])``);
  ``active_mask`` returns int8 [T] (1 active, 0 inactive) or None.

Quantised use cases take the weights offline to the use case's dtype, as the
Ascend page's A2/A3 example does before calling the operator: per output
channel (amax over the input dimension), ``scale = max(amax / Qmax, 1e-8)``
in float32, ``q = w / scale`` in float32, then round-half-even and clamp to
+-127 (int8, Qmax 127) or saturate to +-448 and round to OCP e4m3fn (fp8,
Qmax 448).  This is input preparation outside the operator, not part of the
path under test.

The MX use cases (Ascend page, A8W8-FP: element codes with one FLOAT8_E8M0
scale per output channel and group of 32 along the input dimension; the
DeepGEMM page's FP8 x FP4 path: FP4 e2m1 weights) draw the weights directly
as (element code, scale) pairs, stream ``default_rng([seed, 6, e])``:

* ``mxfp8``: codes = torch's float8_e4m3fn cast of N(0,1) * 64 (clipped to
  +-448, the largest finite e4m3fn value); E8M0 =
  127 - round(log2(64 * sqrt(fan_in))) + a uniform jitter in {-1, 0, 1};
* ``mxfp4``: e2m1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 drawn with fixed
  probabilities (``FP4_MAGNITUDE_P``), random sign; E8M0 =
  127 - round(log2(1.7 * sqrt(fan_in))) + jitter; two codes per byte along
  the output dimension (even column in the low nibble).

so every weight is about N(0, 1/fan_in) in value.  Shapes: W1 codes
[E][H][2I] (fp4: [E][H][I] bytes), W2 [E][I][H] (fp4: [E][I][H/2] bytes),
scales S1 [E][2I][H/32], S2 [E][H][I/32] uint8.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

USECASES = ("bf16", "fp8", "int8", "mxfp8", "mxfp4")
QMAX = {"fp8": 448.0, "int8": 127.0}
MX_USECASES = ("mxfp8", "mxfp4")
# probabilities of the e2m1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 in drawn FP4 weights
FP4_MAGNITUDE_P = (0.16, 0.26, 0.20, 0.13, 0.09, 0.09, 0.05, 0.02)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    usecase: str
    T: int
    H: int
    I: int
    E: int
    K: int
    bias_std: float
    seed: int
    masked_ratio: float = 0.0
    shared: int = 0
    inactive_ratio: float = 0.0

    @property
    def routes(self) -> int:
        return self.T * self.K

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads (names say what they are).  The fp8 shape is swept over
# two token counts that share one weight set (same seed).
CONFIGS = {
    "tiny_bf16": Config("tiny_bf16", "bf16", 64, 256, 128, 8, 2, 0.0, 1000),
    "mid_bf16": Config("mid_bf16", "bf16", 2048, 4096, 1408, 16, 4, 0.0, 1001),
    "dsv3_bf16": Config("dsv3_bf16", "bf16", 4096, 7168, 2048, 32, 8, 0.5, 1002),
    "dsv3_fp8_t128": Config("dsv3_fp8_t128", "fp8", 128, 7168, 2048, 32, 8, 0.5, 1003),
    "dsv3_fp8_t16384": Config("dsv3_fp8_t16384", "fp8", 16384, 7168, 2048, 32, 8, 0.5, 1003),
    "dsv3_int8": Config("dsv3_int8", "int8", 8192, 7168, 2048, 32, 8, 0.0, 1004),
    # the bf16 layer at the two token counts the throughput targets name
    # (16K tokens: MFMA-bound; 128 tokens: weight streaming); same weights
    # as dsv3_bf16
    "dsv3_bf16_t16384": Config("dsv3_bf16_t16384", "bf16", 16384, 7168, 2048, 32, 8, 0.5, 1002),
    "dsv3_bf16_t128": Config("dsv3_bf16_t128", "bf16", 128, 7168, 2048, 32, 8, 0.5, 1002),
    # the MX use cases (MX-FP8 weights; FP4 weights) on the same layer shape
    # and routing, at the two token counts
    "dsv3_mxfp8_t16384": Config("dsv3_mxfp8_t16384", "mxfp8", 16384, 7168, 2048, 32, 8, 0.5, 1005),
    "dsv3_mxfp8_t128": Config("dsv3_mxfp8_t128", "mxfp8", 128, 7168, 2048, 32, 8, 0.5, 1005),
    "dsv3_mxfp4_t16384": Config("dsv3_mxfp4_t16384", "mxfp4", 16384, 7168, 2048, 32, 8, 0.5, 1006),
    "dsv3_mxfp4_t128": Config("dsv3_mxfp4_t128", "mxfp4", 128, 7168, 2048, 32, 8, 0.5, 1006),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# --------------------------------------------------------------------------
# routing + tokens
# --------------------------------------------------------------------------

def routing(cfg: Config):
    """Return ``(topk_ids int32 [T,K], topk_weights float32 [T,K])`` as torch CPU tensors."""
    rng = np.random.default_rng([cfg.seed, 1, cfg.T])
    scores = rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.bias_std > 0:
        bias = np.random.default_rng([cfg.seed, 2]).standard_normal(cfg.E, dtype=np.float32)
        scores = scores + (bias * np.float32(cfg.bias_std))[None, :]
    order = np.argsort(-scores, axis=1, kind="stable")[:, : cfg.K]
    sel = np.take_along_axis(scores, order, axis=1).astype(np.float64)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    wts = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    ids = order.astype(np.int32)
    if cfg.masked_ratio > 0:
        m = np.random.default_rng([cfg.seed, 4, cfg.T]).random((cfg.T, cfg.K)) < cfg.masked_ratio
        ids = np.where(m, np.int32(-1), ids)
        wts = np.where(m, np.float32(0.0), wts)
    return torch.from_numpy(np.ascontiguousarray(ids)), torch.from_numpy(np.ascontiguousarray(wts))


def active_mask(cfg: Config):
    """x_active_mask as an int8 torch CPU tensor ``[T]``, or None when every token is active."""
    if cfg.inactive_ratio <= 0:
        return None
    off = np.random.default_rng([cfg.seed, 5, cfg.T]).random(cfg.T) < cfg.inactive_ratio
    return torch.from_numpy((~off).astype(np.int8))


def tokens(cfg: Config) -> torch.Tensor:
    """Return X as a bf16 torch CPU tensor ``[T, H]``."""
    chunk = 1024
    n_chunks = (cfg.T + chunk - 1) // chunk
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16)

    def one(c):
        r0, r1 = c * chunk, min(cfg.T, (c + 1) * chunk)
        a = np.random.default_rng([cfg.seed, 3, cfg.T, c]).standard_normal((r1 - r0, cfg.H), dtype=np.float32)
        out[r0:r1] = torch.from_numpy(a).to(torch.bfloat16)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(n_chunks)))
    return out


# --------------------------------------------------------------------------
# expert weights
# --------------------------------------------------------------------------

def expert_weights_f32(cfg: Config, e: int):
    """bf16-rounded model weights of expert ``e`` as float32 ``(W1[H,2I], W2[I,H])``."""
    rng = np.random.default_rng([cfg.seed, 0, e])
    w1 = rng.standard_normal((cfg.H, 2 * cfg.I), dtype=np.float32)
    w1 *= np.float32(1.0 / np.sqrt(cfg.H))
    w2 = rng.standard_normal((cfg.I, cfg.H), dtype=np.float32)
    w2 *= np.float32(1.0 / np.sqrt(cfg.I))
    w1 = torch.from_numpy(w1).to(torch.bfloat16).float()
    w2 = torch.from_numpy(w2).to(torch.bfloat16).float()
    return w1, w2


def quantize_weight_per_channel(w: torch.Tensor, usecase: str):
    """Offline per-output-channel weight quantisation (input preparation).

    ``w`` is float32 ``[K_in, N]``; returns ``(q, scale[N] float32)`` with ``q``
    int8 or float8_e4m3fn.  Follows the per-channel recipe of the Ascend
    page's A2/A3 example (amax over dim 0, clamp 1e-8, round, clamp).
    """
    qmax = QMAX[usecase]
    amax = w.abs().amax(dim=0)
    sf = torch.clamp(amax / qmax, min=1e-8).to(torch.float32)
    v = w / sf[None, :]
    if usecase == "int8":
        q = torch.round(v).clamp_(-127, 127).to(torch.int8)
    else:
        q = v.clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q, sf


def mx_expert_weights(cfg: Config, e: int):
    """Expert ``e`` of an MX use case: ``(w1, w2, s1, s2)`` as uint8 tensors
    (codes in the formula layout, fp4 packed two per byte along the output
    dimension; E8M0 scales per output channel and group of 32)."""
    rng = np.random.default_rng([cfg.seed, 6, e])

    def codes(k_in, n):
        if cfg.usecase == "mxfp8":
            v = np.clip(rng.standard_normal((k_in, n), dtype=np.float32) * np.float32(64.0), -448.0, 448.0)
            v = torch.from_numpy(v)
            return v.to(torch.float8_e4m3fn).view(torch.uint8), 64.0
        mag = rng.choice(8, size=(k_in, n), p=FP4_MAGNITUDE_P).astype(np.uint8)
        sign = (rng.random((k_in, n)) < 0.5).astype(np.uint8) << 3
        c = mag | sign
        packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
        return torch.from_numpy(np.ascontiguousarray(packed)), 1.7

    def scales(n, k_in, unit):
        base = 127 - int(round(np.log2(unit * np.sqrt(k_in))))
        return torch.from_numpy((base + rng.integers(-1, 2, (n, k_in // 32))).astype(np.uint8))

    w1, u1 = codes(cfg.H, 2 * cfg.I)
    s1 = scales(2 * cfg.I, cfg.H, u1)
    w2, u2 = codes(cfg.I, cfg.H)
    s2 = scales(cfg.H, cfg.I, u2)
    return w1, w2, s1, s2


def unpack_codes(w: torch.Tensor, cfg: Config) -> np.ndarray:
    """Element codes of MX weights, one per uint8, in the formula layout
    ``[K_in][N]`` (fp4 nibbles unpacked: even column from the low nibble)."""
    b = w.view(torch.uint8).numpy()
    if cfg.usecase != "mxfp4":
        return b
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def expert_weights(cfg: Config, e: int):
    """Weights of expert ``e`` in the use case's dtype.

    Returns ``(w1, w2, s1, s2)``: ``w1 [H,2I]``, ``w2 [I,H]`` in bf16 / fp8 /
    int8; ``s1 [2I]``, ``s2 [H]`` float32 per-channel scales (``None`` for bf16).
    """
    if cfg.usecase in MX_USECASES:
        return mx_expert_weights(cfg, e)
    w1, w2 = expert_weights_f32(cfg, e)
    if cfg.usecase == "bf16":
        return w1.to(torch.bfloat16), w2.to(torch.bfloat16), None, None
    q1, s1 = quantize_weight_per_channel(w1, cfg.usecase)
    q2, s2 = quantize_weight_per_channel(w2, cfg.usecase)
    return q1, q2, s1, s2


@dataclasses.dataclass
class Weights:
    w1: torch.Tensor            # [E+S, H, 2I] (a shared expert last)
    w2: torch.Tensor            # [E+S, I, H]
    s1: torch.Tensor | None     # [E+S, 2I] float32
    s2: torch.Tensor | None     # [E+S, H] float32


def all_weights(cfg: Config) -> Weights:
    n = cfg.E + cfg.shared
    q = cfg.usecase != "bf16"
    if cfg.usecase in MX_USECASES:
        half = 2 if cfg.usecase == "mxfp4" else 1
        w1 = torch.empty((n, cfg.H, 2 * cfg.I // half), dtype=torch.uint8)
        w2 = torch.empty((n, cfg.I, cfg.H // half), dtype=torch.uint8)
        s1 = torch.empty((n, 2 * cfg.I, cfg.H // 32), dtype=torch.uint8)
        s2 = torch.empty((n, cfg.H, cfg.I // 32), dtype=torch.uint8)
    else:
        dt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "int8": torch.int8}[cfg.usecase]
        w1 = torch.empty((n, cfg.H, 2 * cfg.I), dtype=dt)
        w2 = torch.empty((n, cfg.I, cfg.H), dtype=dt)
        s1 = torch.empty((n, 2 * cfg.I), dtype=torch.float32) if q else None
        s2 = torch.empty((n, cfg.H), dtype=torch.float32) if q else None

    def one(e):
        a, b, c, d = expert_weights(cfg, e)
        w1[e] = a
        w2[e] = b
        if q:
            s1[e] = c
            s2[e] = d

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(n)))
    return Weights(w1, w2, s1, s2)


@dataclasses.dataclass
class Inputs:
    cfg: Config
    x: torch.Tensor
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    weights: Weights
    active: torch.Tensor | None = None   # x_active_mask int8 [T], None: every token active


def make_inputs(cfg: Config) -> Inputs:
    ids, wts = routing(cfg)
    return Inputs(cfg, tokens(cfg), ids, wts, all_weights(cfg), active_mask(cfg))
