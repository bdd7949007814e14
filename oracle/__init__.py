"""Plain CPU oracle for fine-grained E4M3 quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the entry point's smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers); the only thing both sides
share is the seeded input generator package ``synth``, which holds none of the
method's arithmetic.

Sources, cited by page title and section (the pages are the method's only
description; no code was taken from anywhere):

* "How does the unified E4M3 format contribute to the efficiency of
  DeepSeek-V3" (codingmall.com), sections "Fine-Grained Quantization Strategy"
  (1x128 activation tiles, 128x128 weight blocks, one E4M3 format everywhere),
  "Dynamic Scaling and Online Quantization" (a scale computed from each group's
  current values) and "Enhanced Numerical Stability" (partial results promoted
  to FP32 at intervals).
* The innerforce.co.kr excerpt of the DeepSeek-V3 report, paragraph on
  Figure 7 (a): the max-abs of a group is mapped to the largest FP8 value;
  activations are grouped per token per 128 channels, weights per 128 input x
  128 output channels.  The following paragraph: FP32 accumulation of the FP8
  GEMM, with dequantization folded into it.
* "DeepSeek FP8 Training" (arcalunar.github.io), the Fprop pipeline list, the
  weight-gradient list and the input-gradient list: which operands are
  quantized, and that the outputs are BF16 (Fprop, Dgrad) and FP32 (Wgrad).
* "FP8 Mixed-Precision Training: Hardware Acceleration Beyond NVIDIA's
  Paradigm" (intl.cloud.baidu.com), section 1.1: E4M3 has a 4-bit exponent and
  a 3-bit mantissa.  The remaining facts of the format (bias 7, the single NaN
  pattern, no infinities, largest value 448) are those of the OCP FP8 E4M3FN
  encoding.

Readings taken where the pages are silent:

* scale s = fl32(amax'/448) is stored; values are multiplied by
  inv = fl32(448/amax'), amax' = max(amax, 2^-100).  The pages do not say
  whether a value is divided by s or multiplied by 1/s; the two conventions
  give different codes for some values, and the tests pin the one chosen here
  (an exact rational re-derivation of every code, and a planted switch to the
  other convention that the tests must catch).
* round-to-nearest-even, saturation to +-448, the sign of zero kept.
* Wgrad operands are grouped 1x128 along the token (contraction) axis.
* the GEMM result is defined as the exact contraction of the dequantized
  operands; the FP32 promotion every 128 K is how a kernel approaches it.
* Microscaling variant (``mx``): OCP MXFP8 E4M3, 1x32 blocks along the
  contraction axis with E8M0 power-of-two scales; a comparison variant, not
  the method.
* MoE backward (``grouped``): an expert's tokens are quantized on their own
  for the weight gradient (no 128-token group mixes two experts), placed in
  a token-padded layout whose chunks each belong to one expert.
"""

from . import e4m3, quant, gemm, grouped, mx  # noqa: F401
from .e4m3 import decode, encode  # noqa: F401
from .quant import (quant_act_1x128, quant_weight_128x128,  # noqa: F401
                    quant_transpose)
from .gemm import (fprop_ref, dgrad_ref, wgrad_ref, grouped_ref,  # noqa: F401
                   exact_outputs)
from .grouped import (quant_transpose_grouped, grouped_dgrad_ref,  # noqa: F401
                      grouped_wgrad_ref, padded_starts, token_capacity)
