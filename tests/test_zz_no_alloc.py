"""The allocation-free fused permute-quantize (library-owned scratch array)
against the entry point with a caller workspace, through the C ABI: bit-
identical outputs on two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents).  The size limit is checked
on the CPU (tests/test_abi.py)."""

import numpy as np
import torch

import workloads
from _helpers import gpu, require_gpu, to_gpu, to_np

pytestmark = gpu

KEYS = ("offsets", "dest", "src", "x_perm", "q", "scales", "gscale", "amax")


def _inputs(seed, T, k, E, D, bad=0):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    if bad:
        ids.reshape(-1)[rng.choice(T * k, bad, replace=False)] = E + 1
    x = workloads._bf16(rng.standard_normal((T, D)).astype(np.float32) * 2)
    return to_gpu(ids, torch.int32), to_gpu(x, torch.bfloat16)


def test_noalloc_matches_workspace_entry_point_twice():
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    for seed, (T, k, E, D, bad) in enumerate([(3000, 8, 128, 2048, 5), (333, 4, 40, 256, 0)]):
        ids, x = _inputs(seed, T, k, E, D, bad)
        st_a = torch.zeros(1, dtype=torch.int32, device="cuda")
        st_b = torch.zeros(1, dtype=torch.int32, device="cuda")
        a = ops.moe_permute_nvfp4(ids, E, x, status=st_a)
        b = ops.moe_permute_nvfp4_noalloc(ids, E, x, status=st_b)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(a[key].view(torch.uint8), b[key].view(torch.uint8)), (T, key)
        assert to_np(st_a)[0] == to_np(st_b)[0] == (1 if bad else 0)
        # with the amax handed in (amax reuse)
        amax = (x.float().abs().amax() * 1.25).reshape(1)
        a = ops.moe_permute_nvfp4(ids, E, x, amax_in=amax, want_x_perm=False)
        b = ops.moe_permute_nvfp4_noalloc(ids, E, x, amax_in=amax, want_x_perm=False)
        torch.cuda.synchronize()
        for key in ("offsets", "dest", "src", "q", "scales", "gscale"):
            assert torch.equal(a[key].view(torch.uint8), b[key].view(torch.uint8)), (T, key)
