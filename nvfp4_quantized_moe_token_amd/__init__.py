"""nvfp4_quantized_moe_token_amd -- NVFP4 token-wise quantization and the
W4A4 MoE grouped GEMM hot path on one AMD MI355X (gfx950).

The compute lives in the HIP library ``libnvfp4moe.so`` (C ABI declared in
``include/nvfp4moe.h``); ``ops`` binds it with the same entry-point names and
``moe_layer`` chains the entry points into one MoE layer forward (W4A4) and
backward (BF16).  Importing this package does not load the library; the
first op call does, and fails loudly if it has not been built.
"""

__all__ = ["ops", "moe_layer", "build"]
