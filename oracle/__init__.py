"""CPU oracle for the NVFP4 token-wise MoE hot path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP kernels are checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``nvfp4_quantized_moe_token_amd``) never imports, calls or links anything in
here, and nothing in here imports the product path.

Sources.  The pages this work follows are three news reports on the miniTE
technical report:

* "miniTE ускоряет RL в NVFP4 на B300: 1,39× к BF16 на Qwen3-30B-A3B"
  (hamidun.com, Russian) and its Arabic twin "miniTE يسرّع RL بصيغة NVFP4 على
  B300" -- native NVFP4 W4A4 (4-bit weights and activations); the NVFP4
  kernels, the scaling scheme and the grouped GEMMs for MoE experts are where
  the time goes (section "Диагностика, выравнивание и быстрые ядра").
* "miniTE報告、NVFP4強化学習の安定性を検証" (aib.vote, Japanese), fourth
  paragraph -- the token-wise NVFP4 path gets a contiguous data layout,
  device-side metadata, amax reuse, grouped GEMM and op fusion; first
  paragraph -- the backward pass runs in BF16.

The pages name NVFP4 but never define it.  The definition used here is the
library's own: 1x16 blocks along K, an E4M3 (OCP E4M3FN) block scale derived
from each block's amax, one FP32 global (decode) scale per tensor, and E2M1
codes rounded to nearest, ties to even.  Every further reading where the
pages are silent (op order of the block scale, sign of zero, nibble order,
permutation order, accumulation order of the combine) is stated in the
docstring of the function that takes it.

Modules:
  nvfp4   -- scalar codecs, quantize, dequantize           (fp32 as defined)
  moe     -- permutation metadata, gather, unpermute, SiLU gate (fp64)
  mx      -- MX formats (MXFP8 / MXFP4, E8M0 per 32) of the W4A8 variant
  gemm    -- grouped W4A4, W4A8 and BF16 GEMMs (fp64 on exact operands)
  layer   -- the MoE layer forward / BF16 backward composed from the above

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against hand-worked values (``tests/golden/``), brute force on tiny inputs,
library routines and invariants -- never against itself.
"""

from . import nvfp4, mx, moe, gemm, layer  # noqa: F401
