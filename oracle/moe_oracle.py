"""Plain float64 oracle of the routed-expert path (test infrastructure only).

Sources, cited by page title and section:

* [ASC] "mega_moe" -- Ascend CANN ops-transformer operator page.
  Formula, Conventions, Computation Process (A16W16 non-quantized use case;
  A8W8-INT Quantization Use Case; A8W8-FP Quantization Use Case with MX
  per-group quantisation), Parameters table, Deterministic Computation.
* [MD]  "05_05 Metadata System" -- DeepEP-v2 notes on DeepGEMM Mega MoE.
  Section 1 (Count -> Prefix Sum -> Scatter), section 3.5 (pool block
  offset), section 5.2 (masked routes).
* [DG]  "DeepGEMM MegaMoE: Fused Communication and Expert Compute".
  Section 1 (FP8 activations x FP4 weights), section 2 (token identities),
  section 3.3 (the (1, 1, 32) scale recipe), section 4 steps 5-6 (UE8M0
  block scales, FP8 re-quantisation of the L1 output), section 6 (optional
  shared experts).

Readings taken where the pages are silent or ambiguous (each one is listed
with its reason in the design notes of the repository):

* rounding ``round-to-nearest`` of [ASC] Conventions is ties-to-even;
* a zero row gets the 1e-8 scale floor the page's weight example uses, so
  its codes are 0;
* the fp8 (OCP e4m3fn) variant of the A8W8 formulas uses Qmax = 448 and
  saturates to +-448 before rounding, per-row scales over the full row;
* the activation quantisation before Dispatch is evaluated in IEEE float32
  (the precision the kernels use), so the integer / e4m3 codes it decides
  are the same on both sides;
* the Linear2 operand A is rounded to the Linear's activation dtype of the
  use case table (bf16 for A16W16);
* route ids < 0 are masked: skipped, counted nowhere, contribute 0 ([MD] 5.2);
* a token whose x_active_mask entry is 0 ([ASC] Parameters: the token does
  not take part in the communication) sends nothing to any expert, routed or
  shared, so its output row is 0;
* a shared expert ([DG] section 6: an always-local MLP on every token, its
  output in the extra combine slot num_topk, summed with the routed slots)
  enters with weight 1, after the routed slots;
* MX per-group quantisation ([ASC] A8W8-FP: groups of 32 along the
  contraction dimension, a shared exponent stored as FLOAT8_E8M0, elements in
  the fp8 format) follows the OCP Microscaling definition: shared exponent
  floor(log2(max|v|)) minus the largest exponent of the element format
  (8 for e4m3, 2 for e2m1), clamped to the E8M0 range [-127, 127] (an
  all-zero group takes -127); elements round to nearest even and saturate;
* the FP8 x FP4 use case ([DG] sections 1 and 4) is the same computation with
  MX-FP4 (e2m1) weights and MX-FP8 activations.
"""

from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_E4M3_MAX = 448.0


def _round_to_significand(a: np.ndarray, sig_bits: int, min_exp: int) -> np.ndarray:
    """Round float64 ``a`` to ``sig_bits`` significant bits, ties to even.

    Numbers below ``2**min_exp`` (the smallest normal) share the subnormal
    quantum ``2**(min_exp - sig_bits + 1)``.  Division by a power of two is
    exact in float64, so the only rounding is the one ``np.rint`` does.
    """
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(a)                      # a = m * 2**ex, 0.5 <= |m| < 1
    e = np.maximum(ex - 1, min_exp)          # |a| in [2**e, 2**(e+1))
    quantum = np.ldexp(1.0, e - (sig_bits - 1))
    return np.rint(a / quantum) * quantum


def bf16_round(a) -> np.ndarray:
    """Value of ``a`` rounded to bfloat16 (8 significant bits, ties to even)."""
    r = _round_to_significand(a, 8, -126)
    return np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)


def e4m3_round(a) -> np.ndarray:
    """Value of ``a`` in OCP float8 e4m3fn: saturate to +-448, round half-even.

    e4m3fn has 4 significant bits, exponent bias 7, smallest normal 2**-6,
    subnormal quantum 2**-9, no infinity, largest finite 448.
    """
    a = np.clip(np.asarray(a, dtype=np.float64), -_E4M3_MAX, _E4M3_MAX)
    return _round_to_significand(a, 4, -6)


def e4m3_encode(a) -> np.ndarray:
    """Bit pattern (uint8) of ``e4m3_round(a)``; sign bit kept for -0."""
    a = np.asarray(a, dtype=np.float64)
    r = e4m3_round(a)
    sign = np.signbit(a).astype(np.uint8) << 7
    mag = np.abs(r)
    _, ex = np.frexp(mag)
    e = ex - 1
    normal = mag >= 2.0 ** -6
    ebits = np.where(normal, e + 7, 0)
    mant = np.where(normal, mag / np.ldexp(1.0, e) - 1.0, mag / 2.0 ** -9) * np.where(normal, 8.0, 1.0)
    mant = np.rint(mant).astype(np.int64)
    code = (ebits.astype(np.int64) << 3) | mant
    code = np.where(mag == 0, 0, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of e4m3fn bit patterns (0x7f / 0xff are NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    eb = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(eb == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, eb - 7))
    val = np.where((eb == 0xF) & (m == 0x7), np.nan, val)
    return s * val


_E2M1_MAX = 6.0


def e2m1_round(a) -> np.ndarray:
    """Value of ``a`` in OCP FP4 e2m1: saturate to +-6, round half-even.

    e2m1 has 2 significant bits, exponent bias 1, smallest normal 1,
    subnormal quantum 0.5: the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    """
    a = np.clip(np.asarray(a, dtype=np.float64), -_E2M1_MAX, _E2M1_MAX)
    return _round_to_significand(a, 2, 0)


def e2m1_decode(codes) -> np.ndarray:
    """float64 value of 4-bit e2m1 codes (held one per uint8): bit 3 sign,
    bits 2-1 exponent, bit 0 mantissa."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    eb = (c >> 1) & 0x3
    m = c & 0x1
    return s * np.where(eb == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, eb - 1))


def e2m1_encode(a) -> np.ndarray:
    """4-bit code (one per uint8) of ``e2m1_round(a)``; sign bit kept for -0."""
    a = np.asarray(a, dtype=np.float64)
    mag = np.abs(e2m1_round(a))
    table = e2m1_decode(np.arange(8, dtype=np.uint8))          # the 8 magnitudes, ascending
    code = np.searchsorted(table, mag).astype(np.uint8)        # exact: mag is one of them
    return (code | (np.signbit(a).astype(np.uint8) << 3)).astype(np.uint8)


# --------------------------------------------------------------------------
# MX per-group quantisation ([ASC] A8W8-FP Quantization Use Case: Q_MX and
# DQ_MX, group size 32, FLOAT8_E8M0 scales)
# --------------------------------------------------------------------------

MX_GROUP = 32
# the exponent of the largest power of two of each element format
MX_EMAX = {"e4m3": 8, "e2m1": 2}


def _elem_encode(v, fmt):
    return e4m3_encode(v) if fmt == "e4m3" else e2m1_encode(v)


def elem_decode(codes, fmt) -> np.ndarray:
    """float64 values of element codes of format ``fmt`` ("e4m3" or "e2m1")."""
    return e4m3_decode(codes) if fmt == "e4m3" else e2m1_decode(codes)


def mx_quantize(v, fmt: str):
    """Q_MX along the last axis (a multiple of 32): ``(codes, e8m0)``.

    Per group of 32 values: shared exponent ``X = floor(log2(max|v|)) -
    MX_EMAX[fmt]`` clamped to [-127, 127] (-127 for an all-zero group), E8M0
    code ``X + 127``, element codes = ``fmt`` encoding of ``v / 2**X`` (round
    half-even, saturating).  Division by a power of two is exact.
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    assert n % MX_GROUP == 0
    g = v.reshape(*v.shape[:-1], n // MX_GROUP, MX_GROUP)
    amax = np.max(np.abs(g), axis=-1)
    _, ex = np.frexp(amax)                                   # amax = m * 2**ex, 0.5 <= m < 1
    x = np.where(amax > 0, ex - 1 - MX_EMAX[fmt], -127)
    x = np.clip(x, -127, 127).astype(np.int64)
    codes = _elem_encode(g / np.ldexp(1.0, x)[..., None], fmt)
    return codes.reshape(v.shape), (x + 127).astype(np.uint8)


def mx_dequantize(codes, e8m0, fmt: str) -> np.ndarray:
    """DQ_MX along the last axis: element value times 2**(e8m0 - 127) of its group."""
    vals = elem_decode(codes, fmt)
    n = vals.shape[-1]
    scale = np.ldexp(1.0, np.asarray(e8m0).astype(np.int64) - 127)
    return (vals.reshape(*vals.shape[:-1], n // MX_GROUP, MX_GROUP) * scale[..., None]).reshape(vals.shape)


# --------------------------------------------------------------------------
# activation
# --------------------------------------------------------------------------

def silu(z):
    """SiLU(z) = z / (1 + e^{-z})  ([ASC] Conventions)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(h: np.ndarray) -> np.ndarray:
    """[ASC] Computation Process, Expert Compute step 2 (SwiGLU activation).

    The first ``intermediate_hidden`` columns of the Linear1 output are the
    gate part, the last ``intermediate_hidden`` the up part;
    ``A = SiLU(H_gate) * H_up``.
    """
    n2 = h.shape[-1]
    assert n2 % 2 == 0
    inter = n2 // 2
    return silu(h[..., :inter]) * h[..., inter:]


# --------------------------------------------------------------------------
# quantisation ([ASC] A8W8-INT use case; fp8 variant by the same formulas)
# --------------------------------------------------------------------------

QMAX = {"int8": 127, "fp8": 448}


def quantize_tokens(x_f32: np.ndarray, usecase: str):
    """Per-token activation quantisation done before Dispatch.

    [ASC] A8W8-INT Quantization Use Case, EP Dispatch: ``s_i = max|X[i,:]|/Qmax``,
    ``q_i = round(X[i,:] / s_i)`` in the symmetric range.  Evaluated in IEEE
    float32 (amax exact, one correctly rounded division for the scale, one per
    element for the quotient); scale floored at 1e-8.

    Returns ``(codes, scale float32 [T], values float64)`` where ``codes`` is
    int8 (int8 use case) or the uint8 e4m3 bit patterns (fp8), and ``values``
    are the integer / e4m3 values the codes stand for.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    qmax = np.float32(QMAX[usecase])
    amax = np.max(np.abs(x), axis=1)
    s = np.maximum(amax / qmax, np.float32(1e-8)).astype(np.float32)
    v = (x / s[:, None]).astype(np.float32)
    if usecase == "int8":
        q = np.clip(np.rint(v), -127, 127).astype(np.int8)
        return q, s, q.astype(np.float64)
    codes = e4m3_encode(v)
    return codes, s, e4m3_decode(codes)


def requantize_rows(a: np.ndarray, usecase: str, emulate_fp32: bool = False):
    """Per-row requantisation of the SwiGLU output before Linear2.

    [ASC] A8W8-INT use case, Expert Compute step 3: ``s^A_i = max|A[i,:]|/Qmax``,
    ``A^q[i,:] = round(A[i,:] / s^A_i)``.  float64 by default; with
    ``emulate_fp32`` the row is first rounded to float32 and the scale and
    quotients are float32 operations.  Returns ``(values float64, scale float64)``.
    """
    qmax = QMAX[usecase]
    if emulate_fp32:
        af = np.asarray(a, dtype=np.float32)
        s = np.maximum(np.max(np.abs(af), axis=1) / np.float32(qmax), np.float32(1e-8)).astype(np.float32)
        v = (af / s[:, None]).astype(np.float32).astype(np.float64)
        s = s.astype(np.float64)
    else:
        a = np.asarray(a, dtype=np.float64)
        s = np.maximum(np.max(np.abs(a), axis=1) / qmax, 1e-8)
        v = a / s[:, None]
    if usecase == "int8":
        q = np.clip(np.rint(v), -127, 127)
    else:
        q = e4m3_round(v)
    return q, s


# --------------------------------------------------------------------------
# dispatch layout ([MD] sections 1, 3.5; [ASC] EP Dispatch)
# --------------------------------------------------------------------------

def dispatch_layout(topk_ids: np.ndarray, num_experts: int, block_m: int):
    """Count -> Prefix Sum -> Scatter, with a BLOCK_M-padded pool.

    * ``counts[e] = N_e`` = number of valid routes with id ``e`` ([ASC] EP
      Dispatch defines ``N_e = |I_e|``; ids are distinct per token, so this is
      also the route count).  Masked routes (id < 0) are not counted.
    * ``offsets[e+1] = offsets[e] + BLOCK_M * ceil(N_e / BLOCK_M)`` -- each
      expert owns a contiguous, block-aligned pool range ([MD] 3.5).
    * ``routes[e]`` = the sorted flat route ids ``i*K + k`` with
      ``E[i,k] == e`` -- the (token, top-k slot) identity multiset of the
      expert ([DG] section 2; [MD] 4.2).  Their order inside the pool is any
      fixed order ([ASC] EP Dispatch), so only the multiset is defined.
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    if np.any(ids >= num_experts):
        raise ValueError("expert id out of range")
    valid = ids >= 0
    counts = np.bincount(ids[valid], minlength=num_experts).astype(np.int64)
    blocks = (counts + block_m - 1) // block_m
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(blocks * block_m)
    routes = [np.nonzero(ids == e)[0] for e in range(num_experts)]
    return {"counts": counts, "offsets": offsets, "routes": routes}


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------

def _e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 e4m3fn codes (``e4m3_decode`` itself)."""
    return e4m3_decode(np.arange(256, dtype=np.uint8))


# MX use cases: activations MX-FP8 (e4m3 elements) in both Linears; the
# weights' element format
MX_WEIGHT_FORMAT = {"mxfp8": "e4m3", "mxfp4": "e2m1"}


def _expert_f64(expert, e, usecase):
    """Decode expert ``e`` to float64 ``(W1 [H,2I], W2 [I,H], s1, s2)``.

    e4m3 weights are decoded by looking each code up in the 256 values
    ``e4m3_decode`` gives for the 256 codes: the same values, without
    re-deriving the format for every one of the H*3I weights.
    """
    w1, w2, s1, s2 = expert(e)
    w1 = np.asarray(w1)
    w2 = np.asarray(w2)
    if usecase in MX_WEIGHT_FORMAT:
        # codes [K_in, N] (one per uint8) with E8M0 scales [N][K_in / 32]:
        # per output column, per group of 32 along the contraction dimension
        fmt = MX_WEIGHT_FORMAT[usecase]
        w1 = mx_dequantize(w1.view(np.uint8).T, np.asarray(s1), fmt).T
        w2 = mx_dequantize(w2.view(np.uint8).T, np.asarray(s2), fmt).T
        return w1, w2, None, None
    if usecase == "fp8":
        table = _e4m3_table()
        w1 = table[w1.view(np.uint8)]
        w2 = table[w2.view(np.uint8)]
    else:
        w1 = w1.astype(np.float64)
        w2 = w2.astype(np.float64)
    if usecase != "bf16":
        s1 = np.asarray(s1, dtype=np.float64)
        s2 = np.asarray(s2, dtype=np.float64)
    return w1, w2, s1, s2


def route_table(topk_ids, topk_weights, shared_expert=None, active=None):
    """Routes of every token as ``(ids [T, K+S], weights [T, K+S])``.

    The K routed slots come first; with ``shared_expert`` (an expert index)
    every token gets one more slot on that expert with weight 1 ([DG]
    section 6).  Tokens with ``active[i] == 0`` get id -1 in every slot
    ([ASC] Parameters, x_active_mask).
    """
    ids = np.asarray(topk_ids).astype(np.int64)
    g = np.asarray(topk_weights, dtype=np.float64)
    T = ids.shape[0]
    if shared_expert is not None:
        ids = np.concatenate([ids, np.full((T, 1), int(shared_expert), dtype=np.int64)], axis=1)
        g = np.concatenate([g, np.ones((T, 1))], axis=1)
    if active is not None:
        on = np.asarray(active).reshape(-1) != 0
        ids = np.where(on[:, None], ids, -1)
    return ids, g


def moe_forward(x_f32, topk_ids, topk_weights, expert, usecase: str,
                tokens=None, requant_fp32: bool = False, activation_clamp=None,
                shared_expert=None, active=None):
    """y_i = sum_k G[i,k] * SwiGLU-FFN_{E[i,k]}(x_i), float64.

    [ASC] Computation Process: EP Dispatch groups the tokens per expert,
    Linear1 ``H_e = X_e W1[e]``, SwiGLU, Linear2 ``Y_e = A_e W2[e]``, Token
    Combine ``y_i = sum_k w_k Y_{e_ik}[row(i,k)]``.  For A8W8 the Linear1
    result is dequantised ``(C * s^W1) * s^X``, A is requantised per row, and
    the Linear2 result is dequantised ``(D * s^W2) * s^A``.

    Inputs: ``x_f32`` [T,H] float32 holding the bf16 token values; ``topk_ids``
    [T,K] int; ``topk_weights`` [T,K] float32; ``expert(e)`` returns expert
    ``e``'s weights (bf16 values as float32, int8, or e4m3 bit patterns as
    uint8) and per-channel scales.  The MX use cases ([ASC] A8W8-FP; "mxfp8":
    e4m3 weights, "mxfp4": e2m1 weights, [DG] section 1) take the weights as
    element codes (one per uint8) with E8M0 scales [N][K_in/32], quantise X
    per token and the SwiGLU output per row with Q_MX in groups of 32 along
    the contraction dimension (e4m3 elements), and multiply the dequantised
    values: ``Z = DQ(X^) DQ(W1)``, ``U = SwiGLU(Z)``, ``O = DQ(Q_MX(U)) DQ(W2)``.  ``tokens`` optionally restricts the
    result to those token indices (rows are independent, so each is the same
    as in the full computation).  Returns ``(y float64 [T or len(tokens), H],
    counts)``.  ``activation_clamp`` (None or c >= 0): [ASC] Parameters,
    activation_clamp — the activation function's input, the whole Linear1
    output H (gate and up halves, after dequantisation), is clamped to
    [-c, c] before SwiGLU.

    ``shared_expert`` (None or an expert index): every token also goes
    through that expert with weight 1 ([DG] section 6).  ``active`` (None or
    [T]): tokens whose entry is 0 contribute nothing, their rows of y are 0
    ([ASC] Parameters, x_active_mask).  The returned counts cover every
    expert index used, the shared expert's included.

    Rows are grouped per expert and multiplied with float64 BLAS, which
    changes no definition: every GEMM row is independent of the others.
    The float64 sum over the top-k slots is independent of order at the
    tolerances used.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    ids, g = route_table(topk_ids, topk_weights, shared_expert, active)
    T, K = ids.shape
    if tokens is None:
        tok = np.arange(T)
    else:
        tok = np.asarray(tokens, dtype=np.int64)
    pos = np.full(T, -1, dtype=np.int64)
    pos[tok] = np.arange(len(tok))

    mx = usecase in MX_WEIGHT_FORMAT
    if mx:
        xc, xe = mx_quantize(x[tok].astype(np.float64), "e4m3")
        xin_sub = mx_dequantize(xc, xe, "e4m3")
    elif usecase != "bf16":
        _, sx_sub, xin_sub = quantize_tokens(x[tok], usecase)

    H = x.shape[1]
    y = np.zeros((len(tok), H), dtype=np.float64)
    flat = ids.reshape(-1)
    sub_mask = np.zeros(T, dtype=bool)
    sub_mask[tok] = True
    e_max = int(flat.max()) if flat.size else -1
    counts = np.bincount(flat[flat >= 0], minlength=max(e_max + 1, 0))
    for e in range(e_max + 1):
        r = np.nonzero(flat == e)[0]
        r = r[sub_mask[r // K]]
        if r.size == 0:
            continue
        i = r // K
        rows = pos[i]
        w1, w2, s1, s2 = _expert_f64(expert, e, usecase)
        if usecase == "bf16":
            xe = x[i].astype(np.float64)
            h = xe @ w1
            if activation_clamp is not None:
                h = np.clip(h, -activation_clamp, activation_clamp)
            a = bf16_round(swiglu(h))
            o = a @ w2
        elif mx:
            h = xin_sub[rows] @ w1
            if activation_clamp is not None:
                h = np.clip(h, -activation_clamp, activation_clamp)
            uc, ue = mx_quantize(swiglu(h), "e4m3")
            o = mx_dequantize(uc, ue, "e4m3") @ w2
        else:
            c = xin_sub[rows] @ w1
            h = (c * s1[None, :]) * sx_sub[rows].astype(np.float64)[:, None]
            if activation_clamp is not None:
                h = np.clip(h, -activation_clamp, activation_clamp)
            a = swiglu(h)
            aq, sa = requantize_rows(a, usecase, emulate_fp32=requant_fp32)
            d = aq @ w2
            o = (d * s2[None, :]) * sa[:, None]
        np.add.at(y, rows, g.reshape(-1)[r][:, None] * o)
    return y, counts


def moe_forward_bruteforce(x_f32, topk_ids, topk_weights, expert, usecase: str, activation_clamp=None,
                           shared_expert=None, active=None):
    """Literal per-token, per-slot scalar loops (tiny inputs only).

    Follows [ASC] Computation Process one scalar at a time: for token i and
    slot k with e = E[i,k] >= 0, h_c = sum_j x_ij W1[e][j,c]; a_c =
    SiLU(h_c) * h_{I+c}; o_n = sum_c a_c W2[e][c,n]; y_in += G[i,k] o_n.
    Quantised use cases take the quantised tokens, dequantise h per element,
    requantise a per route with its own amax, and dequantise o per element.
    An inactive token (active[i] == 0) is skipped whole; a shared expert is
    one more slot after the routed ones, with weight 1.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    ids = np.asarray(topk_ids).astype(np.int64)
    g = np.asarray(topk_weights, dtype=np.float64)
    T, K = ids.shape
    H = x.shape[1]
    mx = usecase in MX_WEIGHT_FORMAT
    if mx:
        xc, xe = mx_quantize(x.astype(np.float64), "e4m3")
        xq = mx_dequantize(xc, xe, "e4m3")
    elif usecase != "bf16":
        _, sx, xq = quantize_tokens(x, usecase)
    y = [[0.0] * H for _ in range(T)]
    cache = {}
    for i in range(T):
        if active is not None and int(np.asarray(active).reshape(-1)[i]) == 0:
            continue
        slots = [(int(ids[i, k]), float(g[i, k])) for k in range(K)]
        if shared_expert is not None:
            slots.append((int(shared_expert), 1.0))
        for e, gw in slots:
            if e < 0:
                continue
            if e not in cache:
                cache[e] = _expert_f64(expert, e, usecase)
            w1, w2, s1, s2 = cache[e]
            n2 = w1.shape[1]
            inter = n2 // 2
            h = []
            for c in range(n2):
                acc = 0.0
                for j in range(H):
                    xv = float(x[i, j]) if usecase == "bf16" else float(xq[i, j])
                    acc += xv * float(w1[j, c])
                if usecase != "bf16" and not mx:
                    acc = acc * float(s1[c]) * float(sx[i])
                if activation_clamp is not None:
                    acc = min(float(activation_clamp), max(-float(activation_clamp), acc))
                h.append(acc)
            a = []
            for c in range(inter):
                z = h[c]
                a.append((z / (1.0 + math.exp(-z))) * h[inter + c])
            if usecase == "bf16":
                a = [float(bf16_round(v)) for v in a]
                sa = 1.0
            elif mx:
                # Q_MX of the row: one E8M0 exponent per group of 32
                a_new = []
                for g0 in range(0, inter, MX_GROUP):
                    grp = a[g0:g0 + MX_GROUP]
                    amax = max(abs(v) for v in grp)
                    xexp = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - MX_EMAX["e4m3"]))
                    a_new += [float(e4m3_round(v / 2.0 ** xexp)) * 2.0 ** xexp for v in grp]
                a = a_new
                sa = 1.0
            else:
                qmax = QMAX[usecase]
                sa = max(max(abs(v) for v in a) / qmax, 1e-8)
                if usecase == "int8":
                    a = [float(min(127.0, max(-127.0, round(v / sa)))) for v in a]
                else:
                    a = [float(e4m3_round(v / sa)) for v in a]
            for n in range(H):
                acc = 0.0
                for c in range(inter):
                    acc += a[c] * float(w2[c, n])
                if usecase != "bf16" and not mx:
                    acc = acc * float(s2[n]) * sa
                y[i][n] += gw * acc
    return np.array(y, dtype=np.float64)
