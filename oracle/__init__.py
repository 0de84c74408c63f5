"""CPU oracle for the fused Mega-MoE routed-expert path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything under ``oracle/``; only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP kernels or the C-ABI library.

What it computes is the definition on the Ascend ``mega_moe`` operator page
(section "Computation Process": EP Dispatch, Linear1, SwiGLU, Linear2, Token
Combine, for the A16W16 and A8W8-INT use cases) in float64, on the
dtype-rounded inputs, plus the layout metadata of the DeepEP "Metadata
System" notes (Count -> Prefix Sum -> Scatter, BLOCK_M-padded pool).

Every function is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py``; there is no "parity unpinned" function.
"""

from .moe_oracle import (  # noqa: F401
    bf16_round,
    e4m3_decode,
    e4m3_encode,
    e4m3_round,
    e2m1_decode,
    e2m1_encode,
    e2m1_round,
    elem_decode,
    mx_quantize,
    mx_dequantize,
    MX_WEIGHT_FORMAT,
    silu,
    swiglu,
    quantize_tokens,
    requantize_rows,
    dispatch_layout,
    route_table,
    moe_forward,
    moe_forward_bruteforce,
)
