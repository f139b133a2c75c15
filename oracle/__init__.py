"""CPU oracle for the block-scaled quantized linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
numpy implementation of what the GPU library computes.  Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it; the
product path (the HIP library and its Python binding) never does, and shares
no code, tables or helpers with it.

Arithmetic is carried out in float64 (exact wherever the rounding rules below
depend on it, which each function states), on the exact real values the
format definitions describe.

Sources, cited by page title and section (the pages do not give bit layouts,
block sizes or rounding rules; those readings are listed in each module):

* "Chameleon" format-selection article (rit.work blog, Russian), sections
  "the format is chosen by the value distribution" (per-output-channel weight
  format by least reconstruction error; activation format table per timestep
  interval, ten intervals; concat convolutions forced to MXFP8) and "plans
  should add calibration" (routing is a table read).
* Nunchaku / SVDQuant article (jiti.kz, Kazakh), section "main explanation"
  (16-bit low-rank branch next to the 4-bit residual GEMM).
* "Bridging the Gap Between Promise and Performance for Microscaling FP4
  Quantization" summary (maximeter.ru), the two reasons FP4 fails (NVFP4's
  small groups, MXFP4's power-of-two scales), modification 1 (least-MSE grid:
  block and tensor scales optimised in turn) and modification 3
  (block-diagonal Hadamard rotation of activations at inference).

Module map:
  formats   E2M1 / E4M3 / E8M0 element and scale codes, round-to-nearest-even
  quantize  MXFP4, MXFP8, NVFP4, INT4 block quantizers and their dequantizers
  hadamard  Sylvester block-diagonal Hadamard rotation
  gemm      dequantized fp64 linear layer (+ low-rank branch) and its tolerance
  select    per-output-channel format choice by minimum reconstruction error
  mse_scales  least-squared-error block (and NVFP4 tensor) scales for weights
  lowrank   offline SVDQuant split W ~= (L1 L2)^T + R (truncated SVD)
  route     timestep-bucket activation-format lookup

Parity unpinned (no independent pin possible): the GPU's MFMA-internal
summation order (bounded only by the stated tolerance) and near-tie format
choices whose errors agree to 1e-12 relative.
"""

from . import formats, quantize, hadamard, gemm, select, route, mse_scales, lowrank  # noqa: F401
