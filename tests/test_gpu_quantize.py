"""GPU parity of nvfp4_quantize: packed codes, scale bytes and global scales
must equal the oracle's bit for bit."""

import os

import numpy as np
import torch

import workloads
from _helpers import gpu, require_gpu, to_gpu, to_np
from conftest import GOLDEN
from oracle import nvfp4
from oracle.layer import bf16_round

pytestmark = gpu


def _gpu_quant(x_np, dtype, groups=1, amax=None):
    from nvfp4_quantized_moe_token_amd import ops
    x = to_gpu(x_np, dtype)
    amax_t = None if amax is None else to_gpu(np.asarray(amax, np.float32).reshape(groups), torch.float32)
    q, s, g, a = ops.nvfp4_quantize(x, groups=groups, amax_in=amax_t)
    torch.cuda.synchronize()
    return to_np(q), to_np(s), to_np(g), to_np(a)


def _assert_same(x_np, dtype, groups=1, amax=None):
    q, s, g, a = _gpu_quant(x_np, dtype, groups, amax)
    xv = x_np if dtype == torch.float32 else bf16_round(x_np)
    rq, rs, rg, ra = nvfp4.quantize(xv, groups=groups, amax=amax)
    np.testing.assert_array_equal(a.view(np.uint32), ra.view(np.uint32))
    np.testing.assert_array_equal(g.view(np.uint32), rg.view(np.uint32))
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)


def test_golden_blocks_gpu():
    require_gpu()
    path = os.path.join(GOLDEN, "quant_blocks.txt")
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, amax, xs, ss, qs = [p.strip() for p in line.split(";")]
        vals = [float.fromhex(t) if t.strip().lower().startswith(("0x", "-0x")) else float(t) for t in xs.split(",")]
        x = np.array(vals, np.float32)[None, :]
        q, s, g, _ = _gpu_quant(x, torch.float32, amax=None if amax == "-" else [float(amax)])
        assert s.tobytes() == bytes.fromhex(ss.replace(" ", "")), name
        assert q.tobytes() == bytes.fromhex(qs.replace(" ", "")), name


def test_threshold_sweep_unit_scale():
    # g = 1 and block amax 6 give d = 1, so every element ratio is the
    # element itself: sweep every E2M1 threshold +-3 ulps, both signs.
    require_gpu()
    pts = [0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6]
    vals = []
    for p in pts:
        p = np.float32(p)
        lo = hi = p
        vals.append(p)
        for _ in range(3):
            lo = np.nextafter(lo, np.float32(-1))
            hi = np.nextafter(hi, np.float32(7))
            vals += [lo, hi]
    v = np.array([x for x in vals if 0 <= x <= 6], np.float32)
    v = np.concatenate([v, -v])
    n = (v.size + 14) // 15
    v = np.concatenate([v, np.zeros(n * 15 - v.size, np.float32)]).reshape(n, 15)
    x = np.concatenate([np.full((n, 1), 6.0, np.float32), v], axis=1)
    _assert_same(x, torch.float32, amax=[2688.0])


def test_all_bf16_values_several_scales():
    # Every finite bf16 value, in blocks, under several global amax values
    # (including stale ones that saturate) -> every code path.
    require_gpu()
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    f = f[: (f.size // 64) * 64].reshape(-1, 64)
    for amax in [float(np.abs(f).max()), 1.0, 2688.0, 3.0e-30, 7.5e20]:
        _assert_same(f, torch.bfloat16, amax=[amax])


def test_random_fp32_outliers_and_tiny():
    require_gpu()
    rng = np.random.default_rng(0)
    for scale in [1.0, 1e-3, 1e-35, 1e30]:
        x = (rng.standard_normal((96, 512)) * scale).astype(np.float32)
        m = rng.random(x.shape) < 0.01
        x[m] *= 64
        x[rng.random(x.shape) < 0.05] = 0.0
        x[rng.random(x.shape) < 0.01] = -0.0
        _assert_same(x, torch.float32)
        _assert_same(x, torch.float32, amax=[float(np.abs(x).max()) * 0.3])   # stale, saturating


def test_dense_small_fp32():
    require_gpu()
    d = workloads.dense_small()
    _assert_same(d["x"], torch.float32)
    _assert_same(d["w"], torch.float32)


def test_qwen3_4b_up_activation_full():
    require_gpu()
    d = workloads.qwen3_4b_up()
    _assert_same(d["x"], torch.bfloat16)


def test_qwen3_4b_up_weight_sampled_rows():
    # Full-size launch; rows are independent once the amax is known, so the
    # oracle checks a seeded sample of rows with the same global amax.
    require_gpu()
    d = workloads.qwen3_4b_up()
    w = d["w"]
    q, s, g, a = _gpu_quant(w, torch.bfloat16)
    amax = np.float32(np.abs(w).max())
    assert a[0] == amax
    rows = np.sort(np.random.default_rng(1).choice(w.shape[0], 512, replace=False))
    rq, rs, rg, _ = nvfp4.quantize(w[rows], amax=[amax])
    np.testing.assert_array_equal(q[rows], rq)
    np.testing.assert_array_equal(s[rows], rs)
    assert g[0] == rg[0]


def test_grouped_expert_weights():
    require_gpu()
    rng = np.random.default_rng(2)
    E, N, K = 6, 40, 96
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    w[2] *= 100.0
    w[4] = 0.0                       # an all-zero expert: g = 1
    _assert_same(w.reshape(E * N, K), torch.bfloat16, groups=E)


def test_many_groups_and_group_grid_limits():
    """Amax reduction at its grid limits: more groups than the reduction's
    workgroup budget (one workgroup per group), a group smaller than one
    workgroup's first loads, and fp32 input with a per-group outlier."""
    require_gpu()
    rng = np.random.default_rng(12)
    G, N, K = 300, 2, 32                  # 300 groups of 2 rows
    w = (rng.standard_normal((G * N, K)) * 0.5).astype(np.float32)
    w[rng.integers(0, G * N, 40), rng.integers(0, K, 40)] *= 300.0
    _assert_same(w, torch.bfloat16, groups=G)
    _assert_same(w, torch.float32, groups=G)
    _assert_same(w[:3], torch.bfloat16, groups=1)   # 3 rows: 12 words, far below one pass
    big = rng.standard_normal((4096 + 3, 48)).astype(np.float32)
    big[4098, 17] = -7000.0                          # the amax sits in the last, ragged pass
    _assert_same(big, torch.bfloat16, groups=1)


def test_expert_weights_full_size_sampled():
    # Expert weights at the MoE down-projection shape [128, 2048, 768] (403 MB
    # of bf16), one global scale per expert, amax computed by the library.
    # Every expert's first and last rows and a seeded sample of others are
    # checked against the oracle with that expert's amax.
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    E, N, K = 128, 2048, 768
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    w = (torch.randn(E, N, K, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    w[7] *= 64.0
    w[70] = 0.0
    q, s, g, a = ops.nvfp4_quantize(w.view(E * N, K), groups=E)
    torch.cuda.synchronize()
    want_amax = w.float().abs().amax(dim=(1, 2))
    assert torch.equal(a, want_amax)
    rng = np.random.default_rng(6)
    q3, s3 = q.view(E, N, K // 2), s.view(E, N, K // 16)
    for e in range(E):
        rows = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 2)]))
        xe = to_np(w[e, torch.as_tensor(rows, device="cuda")].float())
        rq, rs, rg, _ = nvfp4.quantize(xe, amax=[np.float32(want_amax[e].item())])
        idx = torch.as_tensor(rows, device="cuda")
        np.testing.assert_array_equal(to_np(q3[e, idx]), rq)
        np.testing.assert_array_equal(to_np(s3[e, idx]), rs)
        assert to_np(g[e:e + 1]).view(np.uint32)[0] == rg.view(np.uint32)[0], e


def test_empty_and_single_block():
    require_gpu()
    _assert_same(np.zeros((0, 64), np.float32), torch.float32)
    _assert_same(np.array([[1.5] + [0.0] * 15], np.float32), torch.bfloat16)


def test_deterministic_repeat():
    require_gpu()
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1000, 256)).astype(np.float32)
    a = _gpu_quant(x, torch.bfloat16)
    b = _gpu_quant(x, torch.bfloat16)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_beyond_2_31_elements():
    """A bf16 tensor of 262 147 x 8192 = 2 147 508 224 elements (4.3 GB),
    just past 2^31: the amax pass and the quantizer address it with 64-bit
    offsets.  The computed amax is checked against a host max streamed over
    the whole tensor (its largest value planted in the last 16-byte word),
    and rows on both sides of element 2^31, the first and the last rows,
    against the oracle with that amax."""
    require_gpu()
    from nvfp4_quantized_moe_token_amd import ops
    rows, K = 262147, 8192
    assert rows * K > 2 ** 31
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    x = torch.randn(rows, K, device="cuda", generator=gen, dtype=torch.bfloat16)
    x[rows - 1, K - 5] = -300.0
    q, s, g, a = ops.nvfp4_quantize(x)
    torch.cuda.synchronize()
    m = np.float32(0.0)
    for r0 in range(0, rows, 16384):
        m = max(m, np.float32(np.abs(to_np(x[r0:r0 + 16384].float())).max()))
    assert to_np(a)[0] == m == np.float32(300.0)
    cross = 2 ** 31 // K                      # the row that holds element 2^31
    sel = np.array([0, 1, cross - 1, cross, cross + 1, rows - 2, rows - 1])
    idx = torch.as_tensor(sel, device="cuda")
    rq, rs, rg, _ = nvfp4.quantize(to_np(x[idx].float()), amax=[m])
    np.testing.assert_array_equal(to_np(q[idx]), rq)
    np.testing.assert_array_equal(to_np(s[idx]), rs)
    assert to_np(g).view(np.uint32)[0] == rg.view(np.uint32)[0]
