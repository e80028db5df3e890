"""Shared helpers for the GPU parity tests (no method arithmetic here)."""

import numpy as np
import pytest
import torch

gpu = pytest.mark.gpu


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from nvfp4_quantized_moe_token_amd import _lib
    _lib.load()  # raises loudly if the HIP library is missing


def dev():
    return torch.device("cuda:0")


def to_gpu(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev()).to(dtype)


def to_np(t):
    if t.dtype in (torch.uint8, torch.int32, torch.int64):
        return t.cpu().numpy()
    return t.detach().float().cpu().numpy()


def assert_gemm_close(got, ref, absbound, bf16_out=False, what="gemm"):
    """|got - ref| <= 1e-3 * sum|a*b| per element (+ bf16 output rounding)."""
    got = np.asarray(got, np.float64)
    tol = 1e-3 * absbound + 1e-30
    if bf16_out:
        tol = tol + 2.0 ** -8 * (np.abs(ref) + 1e-3 * absbound)
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d/%d elements out of tolerance, e.g. %s: got %s ref %s tol %s" % (
            what, int(bad.sum()), bad.size, idx.tolist(), got[tuple(idx[0])], ref[tuple(idx[0])], tol[tuple(idx[0])]))


def assert_bf16_close(got, ref, scale=None, what="bf16"):
    """bf16-stored fp32 computation: rounding of the result plus a little fp32
    slack proportional to ``scale`` (defaults to |ref|)."""
    got = np.asarray(got, np.float64)
    s = np.abs(ref) if scale is None else scale
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * s + 1e-30
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d/%d out of tolerance, e.g. %s got %s ref %s" % (
            what, int(bad.sum()), bad.size, idx.tolist(), got[tuple(idx[0])], ref[tuple(idx[0])]))
