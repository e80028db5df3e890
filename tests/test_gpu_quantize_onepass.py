"""GPU parity of nvfp4_quantize_onepass (the amax of each row-group and the
NVFP4 encoding from one read of the input): every output must equal the
oracle's, and the two-pass nvfp4_quantize's, bit for bit.

The cases cover groups of one slice and of many (a slice is 1024 blocks of
16), a ragged last slice, more than 256 slices per group (the wait loop's
stride), teams of one workgroup (many tiny groups), a group too large to be
held in flight (the two-pass path inside the call), empty input, all-zero
groups, fp32 input, a workspace reused without clearing, the expert
weights at the MoE gate+up shape, and the path a workgroup takes when its
group's other slices are not published in time (forced from the host)."""

import os

import numpy as np
import torch

from _helpers import gpu, require_gpu, to_gpu, to_np
from oracle import nvfp4
from oracle.layer import bf16_round

pytestmark = gpu


def _onepass(x, groups, workspace=None):
    from nvfp4_quantized_moe_token_amd import ops
    q, s, g, a = ops.nvfp4_quantize_onepass(x, groups=groups, workspace=workspace)
    torch.cuda.synchronize()
    return q, s, g, a


def _twopass(x, groups):
    from nvfp4_quantized_moe_token_amd import ops
    out = ops.nvfp4_quantize(x, groups=groups)
    torch.cuda.synchronize()
    return out


def _assert_same_gpu(got, want, what):
    for name, u, v in zip(("q", "scales", "gscale", "amax"), got, want):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), (what, name)


def _assert_oracle(x_np, dtype, groups):
    x = to_gpu(x_np, dtype)
    q, s, g, a = (to_np(t) for t in _onepass(x, groups))
    xv = x_np if dtype == torch.float32 else bf16_round(x_np)
    rq, rs, rg, ra = nvfp4.quantize(xv, groups=groups)
    np.testing.assert_array_equal(a.view(np.uint32), ra.view(np.uint32))
    np.testing.assert_array_equal(g.view(np.uint32), rg.view(np.uint32))
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)


def test_small_groups_against_oracle():
    require_gpu()
    rng = np.random.default_rng(21)
    E, N, K = 6, 40, 96                  # 240 blocks per group: one ragged slice
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    w[2] *= 100.0
    w[4] = 0.0                           # an all-zero group: amax 0, g = 1
    w[5, N - 1, K - 1] = -3.0            # the amax in the group's last element
    _assert_oracle(w.reshape(E * N, K), torch.bfloat16, E)
    _assert_oracle(w.reshape(E * N, K), torch.float32, E)


def test_multi_slice_groups_against_oracle():
    """Groups of 3 slices and a ragged fourth (3 * 1024 + 208 blocks), with
    each group's amax planted in a different slice."""
    require_gpu()
    rng = np.random.default_rng(22)
    G, K = 4, 16 * 8
    rows = 410                           # 410 * 8 = 3 * 1024 + 208 blocks per group
    x = rng.standard_normal((G * rows, K)).astype(np.float32)
    for gi in range(G):
        r = gi * rows + (gi * 131) % rows
        x[r, (gi * 37) % K] = 50.0 * (gi + 1) * (-1) ** gi
    _assert_oracle(x, torch.bfloat16, G)
    _assert_oracle(x, torch.float32, G)


def test_many_tiny_groups_and_empty():
    require_gpu()
    rng = np.random.default_rng(23)
    G, N, K = 300, 2, 32                 # one workgroup per group
    w = (rng.standard_normal((G * N, K)) * 0.5).astype(np.float32)
    w[rng.integers(0, G * N, 40), rng.integers(0, K, 40)] *= 300.0
    _assert_oracle(w, torch.bfloat16, G)
    _assert_oracle(w, torch.float32, G)
    _assert_oracle(np.zeros((0, 64), np.float32), torch.bfloat16, 1)
    _assert_oracle(np.zeros((0, 64), np.float32), torch.bfloat16, 3)
    _assert_oracle(np.array([[1.5] + [0.0] * 15], np.float32), torch.bfloat16, 1)


def test_more_than_256_slices_per_group():
    """2 groups of 600 x 8192 (300 slices each): each thread of the wait
    loop reads two slots.  Whole outputs against the two-pass quantizer,
    sampled rows (the first, the last, and around the planted amax)
    against the oracle."""
    require_gpu()
    G, rows, K = 2, 600, 8192
    gen = torch.Generator(device="cuda")
    gen.manual_seed(24)
    x = torch.randn(G * rows, K, device="cuda", generator=gen, dtype=torch.bfloat16)
    x[rows + 599, 8191] = 900.0          # group 1's amax in its last element
    x[17, 4000] = -250.0
    got = _onepass(x, G)
    _assert_same_gpu(got, _twopass(x, G), "300 slices")
    q, s, g, a = got
    for gi in range(G):
        assert float(a[gi]) == float(x[gi * rows:(gi + 1) * rows].float().abs().max())
        for r in (0, 17, rows - 1):
            row = gi * rows + r
            rq, rs, rg, _ = nvfp4.quantize(to_np(x[row:row + 1].float()), amax=[np.float32(a[gi].item())])
            np.testing.assert_array_equal(to_np(q[row:row + 1]), rq)
            np.testing.assert_array_equal(to_np(s[row:row + 1]), rs)
            assert to_np(g[gi:gi + 1]).view(np.uint32)[0] == rg.view(np.uint32)[0]


def test_group_too_large_for_one_team():
    """One group of 8192 x 4096 (2048 slices, more than the device holds in
    flight): the call takes the two-pass path, same bits."""
    require_gpu()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(25)
    x = torch.randn(8192, 4096, device="cuda", generator=gen, dtype=torch.bfloat16)
    x[8191, 4095] = 77.0
    _assert_same_gpu(_onepass(x, 1), _twopass(x, 1), "one large group")


def test_workspace_reused_without_clearing():
    """Two calls sharing one workspace, the second on a smaller input whose
    slots overlap the first call's (now stale) ones."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    gen = torch.Generator(device="cuda")
    gen.manual_seed(26)
    a = torch.randn(16 * 1536, 2048, device="cuda", generator=gen, dtype=torch.bfloat16) * 0.02
    b = torch.randn(8 * 512, 2048, device="cuda", generator=gen, dtype=torch.bfloat16) * 0.05
    b[3 * 512 + 9, 100] = 12.0
    ws = torch.empty(ops._lib.load().nvfp4_quantize_onepass_workspace_size(16 * 1536, 2048, 16),
                     dtype=torch.uint8, device="cuda")
    _assert_same_gpu(_onepass(a, 16, ws), _twopass(a, 16), "first call")
    _assert_same_gpu(_onepass(b, 8, ws), _twopass(b, 8), "second call, smaller")
    _assert_same_gpu(_onepass(b, 8, ws), _twopass(b, 8), "third call, repeat")


def test_expert_weights_gate_up_full_size():
    """Expert weights at the MoE gate+up shape [128, 1536, 2048] (805 MB of
    bf16, 192 slices per expert), an outlier expert and an all-zero one:
    every output equals the two-pass quantizer's, the amax equals torch's,
    and each expert's first and last rows equal the oracle's."""
    require_gpu()
    E, N, K = 128, 1536, 2048
    gen = torch.Generator(device="cuda")
    gen.manual_seed(27)
    w = (torch.randn(E, N, K, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    w[9] *= 64.0
    w[100] = 0.0
    got = _onepass(w.view(E * N, K), E)
    _assert_same_gpu(got, _twopass(w.view(E * N, K), E), "gate+up weights")
    q, s, g, a = got
    assert torch.equal(a, w.float().abs().amax(dim=(1, 2)))
    q3, s3 = q.view(E, N, K // 2), s.view(E, N, K // 16)
    for e in range(0, E, 9):
        idx = torch.tensor([0, N - 1], device="cuda")
        rq, rs, rg, _ = nvfp4.quantize(to_np(w[e, idx].float()), amax=[np.float32(a[e].item())])
        np.testing.assert_array_equal(to_np(q3[e, idx]), rq)
        np.testing.assert_array_equal(to_np(s3[e, idx]), rs)
        assert to_np(g[e:e + 1]).view(np.uint32)[0] == rg.view(np.uint32)[0], e


def test_wait_bound_fallback_reads_the_group():
    """With the wait's bound forced to 0 every workgroup takes the amax of its
    group by reading the whole group: the same bits."""
    require_gpu()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(28)
    w = (torch.randn(12 * 1536, 2048, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    w[5 * 1536 + 1535, 2047] = -40.0
    x = torch.randn(4 * 410, 128, device="cuda", generator=gen)
    os.environ["NVFP4MOE_ONEPASS_POLL_LIMIT"] = "0"
    try:
        got_w = _onepass(w, 12)
        got_x = _onepass(x, 4)
    finally:
        del os.environ["NVFP4MOE_ONEPASS_POLL_LIMIT"]
    _assert_same_gpu(got_w, _twopass(w, 12), "fallback, bf16")
    _assert_same_gpu(got_x, _twopass(x, 4), "fallback, fp32")


def test_two_calls_overlapping_on_two_streams():
    """Two one-pass calls issued on two streams at once, each sized to fill
    the device with its own teams: whatever share of the device each gets,
    every workgroup either sees its group's slices or reads the group
    itself, so both results equal the two-pass quantizer's bit for bit."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    gen = torch.Generator(device="cuda")
    gen.manual_seed(29)
    a = (torch.randn(64 * 1536, 2048, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    b = (torch.randn(96 * 1024, 2048, device="cuda", generator=gen) * 0.05).to(torch.bfloat16)
    b[77 * 1024 + 5, 9] = -31.0
    want_a, want_b = _twopass(a, 64), _twopass(b, 96)
    lib = ops._lib.load()
    ws_a = torch.empty(lib.nvfp4_quantize_onepass_workspace_size(a.shape[0], 2048, 64), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(lib.nvfp4_quantize_onepass_workspace_size(b.shape[0], 2048, 96), dtype=torch.uint8,
                       device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            got_a = ops.nvfp4_quantize_onepass(a, groups=64, workspace=ws_a)
        with torch.cuda.stream(s2):
            got_b = ops.nvfp4_quantize_onepass(b, groups=96, workspace=ws_b)
        torch.cuda.synchronize()
        _assert_same_gpu(got_a, want_a, "stream 1")
        _assert_same_gpu(got_b, want_b, "stream 2")
