"""CPU oracle for blockwise FP8 linear layers -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
path is checked against.  Only the test suite, the smoke check and the
benchmark's ``cpu_baseline`` leg may import it; the product path never does,
and it shares no code, tables or constants with the HIP sources.

What it computes follows these passages:

* Puro-2B paper (zh-TW translation, papers.lianghsun.dev), section 3.2
  "FP8 mixed-precision training": E4M3 operands; scales computed online per
  local group; activations and activation gradients in 1-D groups of 128
  consecutive values along the GEMM reduction dimension; weights in 128x128
  2-D blocks.
* Puro-2B tutorial (bloombook.cn), section on FP8 and MuonH, MXFP format
  figure: a block shares one scale X and each element decodes as
  V_i = Q_i * X.
* FP8 Formats for Deep Learning (Micikevicius et al., 2022; cited in the
  translation's reference list), E4M3 definition: bias 7, no infinities,
  S.1111.111 is NaN, largest finite 448.

* Puro-2B translation, section 3.2, again: on SM120 every logical block
  scale was a power of two on the native MXFP8 path (``mx.py``: E8M0 scales,
  1x128 / 128x128 groups and the MXFP8 1x32 groups of the tutorial's MXFP
  figure).

Readings where the pages are silent:
scale = fl32(amax / 448); element map fl32(x * fl32(448 / amax)); saturating
round-to-nearest-even; an all-zero group gets scale 1.0; signed zeros are
kept; fp32 accumulation is promoted once per 128-deep K block.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (library casts, brute force, exact integer or
rational arithmetic, closed-form invariants).  No function is parity
unpinned.
"""

from .e4m3 import e4m3_decode, e4m3_encode, E4M3_MAX
from .quant import (
    quantize_group,
    quantize_act,
    quantize_act_transposed,
    quantize_weight,
    GROUP,
)
from .gemm import dequantize_operand, gemm_ref, logical_operand, normwise_error, o6_error
from .mx import (
    E8M0_BIAS,
    dequantize_mx_operand,
    e8m0_decode,
    logical_mx_operand,
    gemm_mx_ref,
    pow2_exponent,
    quantize_mx_act,
    quantize_mx_act_transposed,
    quantize_mx_group,
    quantize_mx_weight,
)

__all__ = [
    "e4m3_decode",
    "e4m3_encode",
    "E4M3_MAX",
    "quantize_group",
    "quantize_act",
    "quantize_act_transposed",
    "quantize_weight",
    "GROUP",
    "dequantize_operand",
    "gemm_ref",
    "o6_error",
    "logical_operand",
    "normwise_error",
    "E8M0_BIAS",
    "pow2_exponent",
    "e8m0_decode",
    "quantize_mx_group",
    "quantize_mx_act",
    "quantize_mx_act_transposed",
    "quantize_mx_weight",
    "dequantize_mx_operand",
    "logical_mx_operand",
    "gemm_mx_ref",
]
