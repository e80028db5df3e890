"""ctypes view of the nvfp4moe C ABI (include/nvfp4moe.h).

Loading fails loudly when the HIP library has not been built: there is no
CPU fallback anywhere in this package.
"""

import ctypes
import os

from .build import LIB_PATH

c_int, c_i64, c_size, c_vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
c_char_p = ctypes.c_char_p

# name -> (restype, argtypes), in header order.
SIGNATURES = {
    "nvfp4moe_abi_version": (c_int, []),
    "nvfp4moe_status_string": (c_char_p, [c_int]),
    "nvfp4_quantize": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "nvfp4_quantize_onepass_workspace_size": (c_size, [c_i64, c_i64, c_i64]),
    "nvfp4_quantize_onepass": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_size,
                                       c_vp]),
    "moe_permute_workspace_size": (c_size, [c_i64, c_int, c_int]),
    "moe_permute": (c_int, [c_vp, c_i64, c_int, c_int, c_vp, c_int, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                            c_vp, c_size, c_vp, c_vp]),
    "moe_permute_nvfp4": (c_int, [c_vp, c_i64, c_int, c_int, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                  c_vp, c_vp, c_vp, c_vp, c_size, c_vp, c_vp]),
    "moe_permute_nvfp4_noalloc": (c_int, [c_vp, c_i64, c_int, c_int, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_permute_mx": (c_int, [c_vp, c_i64, c_int, c_int, c_vp, c_int, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                               c_size, c_vp, c_vp]),
    "moe_gather": (c_int, [c_vp, c_int, c_i64, c_vp, c_vp, c_int, c_i64, c_vp, c_int, c_vp]),
    "moe_scatter": (c_int, [c_vp, c_int, c_i64, c_vp, c_vp, c_vp, c_int, c_i64, c_int, c_vp, c_int, c_vp, c_vp]),
    "moe_unpermute": (c_int, [c_vp, c_int, c_vp, c_vp, c_i64, c_int, c_i64, c_vp, c_int, c_vp]),
    "grouped_gemm_w4a4": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64,
                                  c_vp, c_int, c_int, c_vp, c_vp, c_size, c_vp]),
    "grouped_gemm_w4a4_silu_gate": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64,
                                            c_vp, c_vp, c_vp, c_vp]),
    "grouped_gemm_w4a4_silu_gate_nvfp4": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64,
                                                  c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "nvfp4_quantize_colwise": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_int, c_vp, c_vp, c_vp, c_vp, c_i64,
                                       c_vp]),
    "nvfp4_quantize_transposed": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "grouped_gemm_w4a4_wgrad": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_i64,
                                        c_vp, c_int, c_vp]),
    "grouped_gemm_w4a4_scaled_mfma": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64,
                                              c_vp, c_int, c_vp]),
    "mx_quantize": (c_int, [c_vp, c_int, c_i64, c_i64, c_int, c_vp, c_vp, c_vp]),
    "grouped_gemm_w4a8": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_int, c_vp]),
    "grouped_gemm_w4a8_silu_gate": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp,
                                            c_vp, c_vp]),
    "grouped_gemm_w4a8_silu_gate_mx": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp,
                                               c_vp, c_vp, c_vp, c_vp]),
    "grouped_gemm_bf16": (c_int, [c_int, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_int, c_int,
                                  c_vp, c_size, c_vp]),
    "grouped_gemm_bf16_tn_gather": (c_int, [c_vp, c_vp, c_vp, c_int, c_i64, c_vp, c_int, c_i64, c_i64, c_i64,
                                            c_vp, c_int, c_int, c_vp]),
    "silu_gate_fwd": (c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "silu_gate_bwd": (c_int, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]),
}

# Constants mirrored from the header.
OK, EINVAL, ESHAPE, EARCH, ELAUNCH, EWORKSPACE = 0, -1, -2, -3, -4, -5
F32, BF16, U8 = 0, 1, 2
NT, NN, TN = 0, 1, 2
EPI_NONE, EPI_SILU_GATE = 0, 1
MX_E4M3, MX_E2M1 = 0, 1
ABI_VERSION = 2
NOALLOC_SCRATCH_BYTES = 2 << 20
STATUS_BAD_EXPERT = 1

_LIB = None


class LibraryNotBuilt(RuntimeError):
    pass


def load(path=LIB_PATH):
    """Load (once) and return the ctypes library with typed entry points."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            "nvfp4moe HIP library not found at %s; build it with "
            "`python -m nvfp4_quantized_moe_token_amd.build`" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.nvfp4moe_abi_version() != ABI_VERSION:
        raise RuntimeError("nvfp4moe ABI version mismatch")
    _LIB = lib
    return lib


def status_string(rc):
    return load().nvfp4moe_status_string(rc).decode()
