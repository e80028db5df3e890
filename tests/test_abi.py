"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    from nvfp4_quantized_moe_token_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_entry_points():
    names = _declared_functions()
    for n in ["nvfp4_quantize", "nvfp4_quantize_onepass", "nvfp4_quantize_onepass_workspace_size", "moe_permute", "moe_permute_workspace_size", "moe_gather", "moe_unpermute",
              "grouped_gemm_w4a4", "grouped_gemm_w4a4_silu_gate", "grouped_gemm_bf16", "moe_scatter",
              "grouped_gemm_bf16_tn_gather", "silu_gate_fwd",
              "silu_gate_bwd", "moe_permute_nvfp4", "moe_permute_nvfp4_noalloc", "moe_permute_mx",
              "grouped_gemm_w4a4_silu_gate_nvfp4", "grouped_gemm_w4a4_scaled_mfma", "nvfp4_quantize_colwise",
              "nvfp4_quantize_transposed", "grouped_gemm_w4a4_wgrad", "mx_quantize", "grouped_gemm_w4a8",
              "grouped_gemm_w4a8_silu_gate", "grouped_gemm_w4a8_silu_gate_mx",
              "nvfp4moe_abi_version", "nvfp4moe_status_string"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from nvfp4_quantized_moe_token_amd import _lib
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_version_and_status_strings(lib):
    from nvfp4_quantized_moe_token_amd import _lib
    macro = int(re.search(r"#define NVFP4MOE_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.nvfp4moe_abi_version() == macro == _lib.ABI_VERSION
    for rc in (0, -1, -2, -3, -4, -5):
        assert lib.nvfp4moe_status_string(rc)
    assert lib.nvfp4moe_status_string(12345) == b"unknown status"


def test_header_constants_match_binding():
    from nvfp4_quantized_moe_token_amd import _lib
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define NVFP4MOE_(\w+) \(?(-?\d+)\)?", text))
    assert int(consts["OK"]) == _lib.OK and int(consts["EINVAL"]) == _lib.EINVAL
    assert int(consts["ESHAPE"]) == _lib.ESHAPE and int(consts["EWORKSPACE"]) == _lib.EWORKSPACE
    assert int(consts["F32"]) == _lib.F32 and int(consts["BF16"]) == _lib.BF16 and int(consts["U8"]) == _lib.U8
    assert int(consts["NT"]) == _lib.NT and int(consts["NN"]) == _lib.NN and int(consts["TN"]) == _lib.TN


FAKE = 0x10000  # a 64 KiB-aligned fake device address: never dereferenced


def test_quantize_validation(lib):
    q = lib.nvfp4_quantize
    # NULL x with work to do
    assert q(None, 1, 4, 32, 1, None, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    # bad dtype
    assert q(FAKE, 7, 4, 32, 1, None, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    # negative sizes, groups < 1
    assert q(FAKE, 1, -1, 32, 1, None, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert q(FAKE, 1, 4, 32, 0, None, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    # both amax_in and amax_out NULL
    assert q(FAKE, 1, 4, 32, 1, None, None, FAKE, FAKE, FAKE, None, None) == -1
    # K % 16, rows % groups
    assert q(FAKE, 1, 4, 24, 1, None, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    assert q(FAKE, 1, 5, 32, 2, None, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    # misaligned x
    assert q(FAKE + 4, 1, 4, 32, 1, None, FAKE, FAKE, FAKE, FAKE, None, None) == -2



def test_quantize_onepass_validation(lib):
    q = lib.nvfp4_quantize_onepass
    ws = lib.nvfp4_quantize_onepass_workspace_size
    # one 4-byte slot per group and slice of 1024 blocks of 16
    assert ws(4, 32, 1) == 4
    assert ws(128 * 1536, 2048, 128) == 128 * 192 * 4
    assert ws(3 * 1000, 4096, 3) == 3 * 250 * 4
    assert ws(0, 32, 4) == 0
    assert ws(5, 32, 2) == 0 and ws(4, 24, 1) == 0 and ws(4, 32, 0) == 0
    # NULL x with work to do; bad dtype; groups < 1; amax_out NULL
    assert q(None, 1, 4, 32, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == -1
    assert q(FAKE, 7, 4, 32, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == -1
    assert q(FAKE, 1, 4, 32, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == -1
    assert q(FAKE, 1, 4, 32, 1, None, FAKE, FAKE, FAKE, FAKE, 4, None) == -1
    # K % 16, rows % groups, misaligned x
    assert q(FAKE, 1, 4, 24, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == -2
    assert q(FAKE, 1, 5, 32, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == -2
    assert q(FAKE + 4, 1, 4, 32, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == -2
    # workspace missing or too small
    assert q(FAKE, 1, 4, 32, 1, FAKE, FAKE, FAKE, FAKE, None, 4, None) == -5
    assert q(FAKE, 1, 4, 32, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 3, None) == -5
    assert q(FAKE, 1, 128 * 1536, 2048, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 128 * 192 * 4 - 1, None) == -5

def test_permute_validation(lib):
    p = lib.moe_permute
    ws = lib.moe_permute_workspace_size(100, 8, 128)
    assert ws >= 128 * 4
    assert lib.moe_permute_workspace_size(-1, 8, 128) == 0
    # histograms (one per 1024 assignments) plus the fused call's amax parts
    # (one per histogram workgroup, at least 256)
    for T, k, E in [(100, 8, 128), (8192, 8, 128), (131072, 8, 128), (1, 1, 4096)]:
        chunks = -(-T * k // 1024)
        assert lib.moe_permute_workspace_size(T, k, E) >= chunks * E * 4 + max(chunks, 256) * 4
    assert p(FAKE, 100, 0, 128, None, 1, 0, None, FAKE, FAKE, FAKE, None, FAKE, ws, None, None) == -1  # k = 0
    assert p(FAKE, 100, 8, 5000, None, 1, 0, None, FAKE, FAKE, FAKE, None, FAKE, 10 ** 9, None, None) == -2  # E too big
    assert p(FAKE, 100, 8, 128, None, 1, 0, None, None, FAKE, FAKE, None, FAKE, ws, None, None) == -1  # offsets NULL
    assert p(FAKE, 100, 8, 128, None, 1, 0, None, FAKE, FAKE, FAKE, None, FAKE, ws - 1, None, None) == -5
    assert p(FAKE, 100, 8, 128, FAKE, 1, 12, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None, None) == -2  # 24 B rows
    assert p(FAKE, 100, 8, 128, FAKE, 2, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None, None) == -1  # amax of u8


def test_permute_nvfp4_validation(lib):
    f = lib.moe_permute_nvfp4
    ws = lib.moe_permute_workspace_size(100, 8, 128)
    ok = [FAKE, 100, 8, 128, FAKE, 2048, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None, None]
    bad = list(ok); bad[2] = 0
    assert f(*bad) == -1                       # k = 0
    bad = list(ok); bad[7] = None; bad[8] = None
    assert f(*bad) == -1                       # neither amax_in nor amax_out
    bad = list(ok); bad[11] = None
    assert f(*bad) == -1                       # gscale NULL
    bad = list(ok); bad[5] = 2040
    assert f(*bad) == -2                       # D % 16
    bad = list(ok); bad[4] = FAKE + 8
    assert f(*bad) == -2                       # x alignment
    bad = list(ok); bad[3] = 5000
    assert f(*bad) == -2                       # E too big
    bad = list(ok); bad[16] = ws - 1
    assert f(*bad) == -5                       # workspace too small



def test_permute_mx_validation(lib):
    p = lib.moe_permute_mx
    ws = lib.moe_permute_workspace_size(10, 8, 4)
    args = [FAKE, 10, 8, 4, FAKE, 1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None, None]
    bad = list(args); bad[5] = 2
    assert p(*bad) == -1                       # u8 payload: not quantizable
    bad = list(args); bad[4] = None
    assert p(*bad) == -1                       # x NULL with rows
    bad = list(args); bad[8] = None
    assert p(*bad) == -1                       # scales NULL
    bad = list(args); bad[6] = 48
    assert p(*bad) == -2                       # D % 32
    bad = list(args); bad[7] = FAKE + 8
    assert p(*bad) == -2                       # q alignment
    bad = list(args); bad[3] = 5000
    assert p(*bad) == -2                       # E > 4096
    bad = list(args); bad[13] = ws - 1
    assert p(*bad) == -5                       # workspace too small

def test_gather_unpermute_validation(lib):
    assert lib.moe_gather(FAKE, 1, 64, FAKE, None, 0, 10, FAKE, 1, None) == -1
    assert lib.moe_gather(FAKE, 2, 64, FAKE, FAKE, 8, 10, FAKE, 2, None) == -1  # weighted bytes
    assert lib.moe_gather(FAKE, 1, 12, FAKE, FAKE, 8, 10, FAKE, 1, None) == -2
    sc = lib.moe_scatter
    assert sc(FAKE, 1, 64, FAKE, None, FAKE, 4, 10, 0, FAKE, 1, None, None) == -1       # k = 0
    assert sc(FAKE, 2, 64, FAKE, None, FAKE, 4, 10, 8, FAKE, 1, None, None) == -1       # u8 payload
    assert sc(FAKE, 1, 64, FAKE, None, None, 4, 10, 8, FAKE, 1, None, None) == -1       # offsets NULL
    assert sc(FAKE, 1, 12, FAKE, None, FAKE, 4, 10, 8, FAKE, 1, None, None) == -2       # row_elems % 8
    assert sc(FAKE, 1, 64, FAKE, None, FAKE, 4, 10, 8, FAKE, 1, FAKE + 2, None) == -2   # misaligned amax
    assert lib.moe_unpermute(FAKE, 2, FAKE, None, 4, 8, 64, FAKE, 1, None) == -1
    assert lib.moe_unpermute(FAKE, 1, FAKE, None, 4, 8, 60, FAKE, 1, None) == -2
    assert lib.moe_unpermute(None, 1, FAKE, None, 4, 8, 64, FAKE, 1, None) == -1


def test_gemm_validation(lib):
    g = lib.grouped_gemm_w4a4
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 64, 64, FAKE, 0, 0, None, None, 0, None]
    bad = list(args); bad[12] = 9
    assert g(*bad) == -1                       # dtype
    bad = list(args); bad[13] = 2
    assert g(*bad) == -1                       # unknown epilogue
    bad = list(args); bad[13] = 1
    assert g(*bad) == -1                       # SiLU-gate epilogue needs a bf16 H
    bad = list(args); bad[13] = 1; bad[12] = 1
    assert g(*bad) == -2                       # SiLU-gate epilogue: N % 256
    bad = list(args); bad[10] = 48
    assert g(*bad) == -2                       # K % 64
    bad = list(args); bad[10] = 96
    assert g(*bad) == -2                       # K % 64 (a multiple of 32 is not enough)
    bad = list(args); bad[9] = 40
    assert g(*bad) == -2                       # N % 32
    bad = list(args); bad[6] = None
    assert g(*bad) == -1                       # offsets
    b = lib.grouped_gemm_bf16
    assert b(3, FAKE, FAKE, FAKE, 4, 64, 64, 64, FAKE, 0, 0, None, 0, None) == -1
    assert b(0, FAKE, FAKE, FAKE, 4, 64, 64, 64, FAKE, 1, 1, None, 0, None) == -1  # accumulate bf16
    assert b(1, FAKE, FAKE, FAKE, 4, 64, 64, 48, FAKE, 0, 0, None, 0, None) == -2
    assert b(2, FAKE + 8, FAKE, FAKE, 4, 64, 64, 64, FAKE, 0, 0, None, 0, None) == -2


def test_gemm_silu_gate_validation(lib):
    g = lib.grouped_gemm_w4a4_silu_gate
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 64, FAKE, FAKE, None, None]
    bad = list(args); bad[12] = None
    assert g(*bad) == -1                       # H is required
    bad = list(args); bad[9] = -1
    assert g(*bad) == -1                       # F < 0
    bad = list(args); bad[9] = 96
    assert g(*bad) == -2                       # F % 128
    bad = list(args); bad[10] = 96
    assert g(*bad) == -2                       # K % 64
    bad = list(args); bad[11] = FAKE + 8
    assert g(*bad) == -2                       # Y1 alignment
    bad = list(args); bad[12] = FAKE + 2
    assert g(*bad) == -2                       # H alignment


def test_gemm_tn_gather_validation(lib):
    g = lib.grouped_gemm_bf16_tn_gather
    args = [FAKE, FAKE, FAKE, 8, 100, FAKE, 4, 64, 64, 64, FAKE, 0, 0, None]
    bad = list(args); bad[3] = 0
    assert g(*bad) == -1                       # k < 1
    bad = list(args); bad[2] = None
    assert g(*bad) == -1                       # b_src NULL with rows to reduce
    bad = list(args); bad[4] = -1
    assert g(*bad) == -1                       # negative b_rows
    bad = list(args); bad[11] = 1; bad[12] = 1
    assert g(*bad) == -1                       # accumulate into bf16
    bad = list(args); bad[9] = 48
    assert g(*bad) == -2                       # K % 32
    bad = list(args); bad[2] = FAKE + 2
    assert g(*bad) == -2                       # b_src alignment
    bad = list(args); bad[4] = 1 << 25
    assert g(*bad) == -2                       # b_rows * N * 2 >= 2^31


def test_scaled_mfma_and_silu_nvfp4_validation(lib):
    g = lib.grouped_gemm_w4a4_scaled_mfma
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 64, 64, FAKE, 0, None]
    bad = list(args); bad[12] = 9
    assert g(*bad) == -1                       # dtype
    bad = list(args); bad[10] = 96
    assert g(*bad) == -2                       # K % 64
    bad = list(args); bad[7] = 0
    assert g(*bad) == -1                       # E < 1
    f = lib.grouped_gemm_w4a4_silu_gate_nvfp4
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 64, None, None, None, FAKE, FAKE, FAKE, FAKE,
            None]
    bad = list(args); bad[15] = None
    assert f(*bad) == -1                       # q_h NULL
    bad = list(args); bad[14] = None
    assert f(*bad) == -1                       # amax_h_in NULL
    bad = list(args); bad[17] = None
    assert f(*bad) == -1                       # g_h NULL
    bad = list(args); bad[13] = FAKE
    assert f(*bad) == -1                       # amax_out aliases amax_h_in
    bad = list(args); bad[9] = 96
    assert f(*bad) == -2                       # F % 128
    bad = list(args); bad[15] = FAKE + 2
    assert f(*bad) == -2                       # q_h alignment


def test_colwise_and_transposed_validation(lib):
    c = lib.nvfp4_quantize_colwise
    Kp = 64 * (100 // 64 + 4)
    args = [FAKE, 1, 100, 64, FAKE, 4, FAKE, FAKE, FAKE, FAKE, Kp, None]
    bad = list(args); bad[1] = 0
    assert c(*bad) == -1                       # only bf16 input
    bad = list(args); bad[6] = None
    assert c(*bad) == -1                       # amax_in NULL
    bad = list(args); bad[5] = 0
    assert c(*bad) == -1                       # E < 1
    bad = list(args); bad[3] = 60
    assert c(*bad) == -2                       # N % 8
    bad = list(args); bad[10] = Kp - 64
    assert c(*bad) == -2                       # Kp below 64 * (M/64 + E)
    bad = list(args); bad[10] = Kp + 32
    assert c(*bad) == -2                       # Kp % 64
    bad = list(args); bad[7] = FAKE + 4
    assert c(*bad) == -2                       # q_t alignment
    bad = list(args); bad[3] = 1 << 20; bad[10] = 1 << 13
    assert c(*bad) == -2                       # codes of 2^20 x 2^12 bytes: past 2 GiB
    t = lib.nvfp4_quantize_transposed
    args = [FAKE, 1, 4, 128, 64, FAKE, None, FAKE, FAKE, FAKE, None]
    bad = list(args); bad[5] = None
    assert t(*bad) == -1                       # neither amax_in nor amax_out
    bad = list(args); bad[0] = None
    assert t(*bad) == -1                       # x NULL with elements
    bad = list(args); bad[3] = 96
    assert t(*bad) == -2                       # L % 64
    bad = list(args); bad[4] = 12
    assert t(*bad) == -2                       # N % 8
    bad = list(args); bad[2] = 0
    assert t(*bad) == -1                       # groups < 1
    bad = list(args); bad[2] = 1 << 10; bad[3] = 1 << 12; bad[4] = 1 << 11
    assert t(*bad) == -2                       # codes of 2^10 x 2^12 x 2^10 bytes: past 2 GiB


def test_wgrad_validation(lib):
    w = lib.grouped_gemm_w4a4_wgrad
    Kp = 64 * (100 // 64 + 4)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 100, Kp, 64, 64, FAKE, 0, None]
    bad = list(args); bad[13] = 9
    assert w(*bad) == -1                       # dtype
    bad = list(args); bad[12] = None
    assert w(*bad) == -1                       # c NULL
    bad = list(args); bad[2] = None
    assert w(*bad) == -1                       # a_g NULL
    bad = list(args); bad[9] = Kp - 64
    assert w(*bad) == -2                       # Kp too small for the padded segments
    bad = list(args); bad[10] = 48
    assert w(*bad) == -2                       # N1 % 32
    bad = list(args); bad[11] = 40
    assert w(*bad) == -2                       # N2 % 32
    bad = list(args); bad[10] = 1 << 20; bad[9] = 1 << 12
    assert w(*bad) == -2                       # N1 * Kp / 2 >= 2^31


def test_mx_validation(lib):
    from nvfp4_quantized_moe_token_amd import _lib
    m = lib.mx_quantize
    assert m(FAKE, 1, 4, 64, 7, FAKE, FAKE, None) == -1                # unknown element format
    assert m(FAKE, 2, 4, 64, _lib.MX_E4M3, FAKE, FAKE, None) == -1     # u8 input
    assert m(FAKE, 1, 4, 48, _lib.MX_E4M3, FAKE, FAKE, None) == -2     # K % 32
    assert m(FAKE, 1, 4, 64, _lib.MX_E4M3, FAKE + 8, FAKE, None) == -2  # fp8 codes need 16-byte alignment
    assert m(FAKE, 1, 4, 64, _lib.MX_E2M1, FAKE, None, None) == -1     # scales NULL
    assert m(FAKE, 1, -1, 64, _lib.MX_E2M1, FAKE, FAKE, None) == -1    # negative rows
    g = lib.grouped_gemm_w4a8
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 64, 128, FAKE, 0, None]
    bad = list(args); bad[8] = 64
    assert g(*bad) == -2                       # K % 128
    bad = list(args); bad[7] = 48
    assert g(*bad) == -2                       # N % 32
    bad = list(args); bad[4] = None
    assert g(*bad) == -1                       # offsets NULL
    bad = list(args); bad[10] = 2
    assert g(*bad) == -1                       # u8 output
    s = lib.grouped_gemm_w4a8_silu_gate
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 128, None, FAKE, None, None]
    bad = list(args); bad[10] = None
    assert s(*bad) == -1                       # H is required
    bad = list(args); bad[7] = 64
    assert s(*bad) == -2                       # F % 128
    bad = list(args); bad[7] = -128
    assert s(*bad) == -1                       # F < 0
    m = lib.grouped_gemm_w4a8_silu_gate_mx
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 128, None, None, None, FAKE, FAKE, None]
    bad = list(args); bad[12] = None
    assert m(*bad) == -1                       # q_h is required
    bad = list(args); bad[13] = None
    assert m(*bad) == -1                       # s_h is required
    bad = list(args); bad[12] = FAKE + 4
    assert m(*bad) == -2                       # q_h alignment
    bad = list(args); bad[7] = 64
    assert m(*bad) == -2                       # F % 128


def test_silu_validation(lib):
    assert lib.silu_gate_fwd(None, 4, 64, FAKE, None, None) == -1
    assert lib.silu_gate_fwd(FAKE, 4, 60, FAKE, None, None) == -2
    assert lib.silu_gate_bwd(FAKE, FAKE, -1, 64, FAKE, None, None) == -1
    assert lib.silu_gate_bwd(FAKE, FAKE, 4, 64, FAKE, FAKE + 2, None) == -2


def test_ops_refuse_cpu_tensors():
    import torch
    from nvfp4_quantized_moe_token_amd import ops
    with pytest.raises(ValueError):
        ops.nvfp4_quantize(torch.zeros(4, 32))


def test_ctypes_pointer_width():
    assert ctypes.sizeof(ctypes.c_void_p) == 8


def test_noalloc_rejects_sizes_beyond_scratch(lib):
    # The allocation-free permute-quantize refuses a call whose histograms
    # would not fit its scratch array, before any HIP call.
    from nvfp4_quantized_moe_token_amd import _lib
    T, k, E = 1 << 20, 8, 4096
    assert lib.moe_permute_workspace_size(T, k, E) > _lib.NOALLOC_SCRATCH_BYTES
    rc = lib.moe_permute_nvfp4_noalloc(FAKE, T, k, E, FAKE, 64, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, None, None)
    assert rc == _lib.EWORKSPACE
    # within the limit the same call passes validation and stops at the
    # architecture check (no GPU here) or at a NULL pointer
    assert lib.moe_permute_nvfp4_noalloc(None, 64, 8, 128, FAKE, 64, None, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, None, None) == _lib.EINVAL
    text = open(HEADER).read()
    assert int(re.search(r"#define NVFP4MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text).group(1)) << 20 \
        == _lib.NOALLOC_SCRATCH_BYTES
