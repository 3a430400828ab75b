"""Kernel-level parity: each C-ABI kernel entry against the oracle (or the
plain definition) on identical seeded inputs, including ragged tails and
degenerate sizes."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import rel_err
from tests.gpu_helpers import dev, host, TORCH_DT
from workloads import round_to

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- RoPE
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n,h,dh,delta", [(1, 1, 64, 5), (37, 4, 64, 640), (300, 32, 128, 3840),
                                          (129, 8, 128, 8191), (50, 2, 128, -700),
                                          (0, 2, 64, 3)])
def test_rope_rerotate_vs_oracle(lib, dt, n, h, dh, delta):
    rng = np.random.default_rng(n + dh)
    k = round_to(rng.standard_normal((n, h, dh)), dt)
    v = round_to(rng.standard_normal((n, h, dh)), dt)
    kd, vd = dev(k, dt), dev(v, dt)
    ko, vo = torch.empty_like(kd), torch.empty_like(vd)
    lib.cb_rope_rerotate(kd, ko, vd, vo, n, h, dh, delta)
    torch.cuda.synchronize()
    if n == 0:
        return
    ref = oracle.rope_rotate(k, delta, 1e4)
    np.testing.assert_array_equal(host(vo), v)
    if dt == "f32":
        assert rel_err(host(ko), ref) < 2e-6
    else:   # within one bf16 rounding of the exact rotation
        assert np.max(np.abs(host(ko) - ref) / np.maximum(np.abs(ref), 1e-3)) < 2 ** -7


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rope_rerotate_closed_form_and_identity(lib, dt):
    """Rotating a key encoded at j by delta equals encoding it at j + delta
    (Prompt Cache explainer, RoPE position adjustment); delta 0 is exact."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 4, 128))
    j = 100
    enc = round_to(oracle.rope_rotate(x, j, 1e4), dt)
    kd = dev(enc, dt)
    ko = torch.empty_like(kd)
    lib.cb_rope_rerotate(kd, ko, None, None, 64, 4, 128, 2000)
    torch.cuda.synchronize()
    tol = 2e-6 if dt == "f32" else 1e-2
    assert rel_err(host(ko), oracle.rope_rotate(enc, 2000, 1e4)) < tol
    assert rel_err(host(ko), oracle.rope_rotate(x, j + 2000, 1e4)) < (1e-5 if dt == "f32" else 2e-2)
    moved = ko.clone()
    lib.cb_rope_rerotate(kd, ko, None, None, 64, 4, 128, 0)
    torch.cuda.synchronize()
    assert torch.equal(ko, kd)
    k2 = kd.clone()                                     # in place
    lib.cb_rope_rerotate(k2, k2, None, None, 64, 4, 128, 2000)
    torch.cuda.synchronize()
    assert torch.equal(k2, moved)


# ---------------------------------------------------------------- deviation
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("mode,name", [(0, "KV"), (1, "K"), (2, "V")])
@pytest.mark.parametrize("n,row", [(1, 8), (77, 256), (3840, 4096), (5, 1024), (145, 4096),
                                   (1023, 1024), (1024, 1024)])
def test_deviation_vs_oracle(lib, dt, mode, name, n, row):
    rng = np.random.default_rng(row + n)
    a = [round_to(rng.standard_normal((n, row)), dt) for _ in range(4)]
    t = [dev(x, dt) for x in a]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    lib.cb_deviation(t[0], t[1], t[2], t[3], n, row, mode, out)
    torch.cuda.synchronize()
    ref = oracle.kv_deviation(a[0], a[1], a[2], a[3], name)
    assert np.max(np.abs(host(out) - ref) / ref) < 1e-5


# ---------------------------------------------------------------- top-k (bit-exact)
def _topk_case(lib, d, k):
    dd = torch.from_numpy(np.asarray(d, dtype=np.float32)).cuda()
    out = torch.full((max(k, 1),), -1, dtype=torch.int32, device="cuda")
    lib.cb_topk_select(dd, len(d), k, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[:k]
    ref = oracle.topk_select(np.asarray(d, dtype=np.float32).astype(np.float64), k)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("n", [1, 2, 7, 64, 1000, 1025, 3840, 8192, 20000])
def test_topk_random_bit_exact(lib, n):
    rng = np.random.default_rng(n)
    d = rng.standard_normal(n).astype(np.float32) ** 2
    for k in sorted({1, max(1, n // 7), max(1, (n * 15) // 100), n - 1 if n > 1 else 1, n}):
        _topk_case(lib, d, k)


def test_topk_ties_nan_inf_signed_zero(lib):
    rng = np.random.default_rng(1)
    pool = np.array([0.0, -0.0, 1.0, 2.5, np.inf, -np.inf, np.nan, -1.0, 1e-30, 3.0],
                    dtype=np.float32)
    for n in (1, 5, 16, 333, 4096):
        d = rng.choice(pool, size=n)
        for k in sorted({1, n // 3 or 1, n // 2 or 1, n}):
            _topk_case(lib, d, k)
    # all equal: position order decides
    _topk_case(lib, np.full(1000, 0.5, np.float32), 150)
    # values that differ only in the last mantissa bit
    base = np.float32(1.2345)
    d = np.array([np.nextafter(base, np.float32(2)) if i % 3 else base for i in range(999)],
                 dtype=np.float32)
    _topk_case(lib, d, 400)


# ---------------------------------------------------------------- rows
def test_gather_scatter_bit_exact(lib):
    rng = np.random.default_rng(2)
    src = torch.from_numpy(rng.standard_normal((500, 96)).astype(np.float32)).cuda()
    idx = torch.from_numpy(rng.permutation(500)[:123].astype(np.int32)).cuda()
    dst = torch.empty((123, 96), device="cuda")
    lib.cb_gather_rows(src, dst, idx, 123, 96 * 4)
    torch.cuda.synchronize()
    assert torch.equal(dst, src[idx.long()])
    back = torch.zeros_like(src)
    lib.cb_scatter_rows(dst, back, idx, 123, 96 * 4)
    torch.cuda.synchronize()
    assert torch.equal(back[idx.long()], dst)
    odd = torch.from_numpy(rng.standard_normal((40, 5)).astype(np.float32)).cuda()  # 20-byte rows
    d2 = torch.empty((3, 5), device="cuda")
    i2 = torch.tensor([39, 0, 7], dtype=torch.int32, device="cuda")
    lib.cb_gather_rows(odd, d2, i2, 3, 20)
    torch.cuda.synchronize()
    assert torch.equal(d2, odd[i2.long()])


# ---------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("rows,d", [(1, 256), (77, 4096), (5, 5120), (3, 100)])
def test_rmsnorm_vs_oracle(lib, dt, rows, d):
    rng = np.random.default_rng(d)
    x = round_to(rng.standard_normal((rows, d)) * 3, dt)
    g = round_to(rng.standard_normal(d), dt)
    xd, gd = dev(x, dt), dev(g, dt)
    y = torch.empty_like(xd)
    lib.cb_rmsnorm(xd, gd, y, rows, d, 1e-5)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x, g, 1e-5)
    assert rel_err(host(y), ref) < (1e-6 if dt == "f32" else 8e-3)


# ---------------------------------------------------------------- GEMM
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("m,n,k", [(1, 16, 64), (7, 130, 64), (130, 128, 256), (832, 384, 4096),
                                   (257, 1000, 1024), (128, 11008, 512), (3, 4096, 11008),
                                   (1600, 520, 384), (2048, 256, 128), (1537, 2000, 1152),
                                   (832, 4096, 4096), (1000, 1536, 2048), (640, 2816, 1536),
                                   (832, 22016, 1024), (700, 10000, 512), (947, 6000, 256),
                                   (600, 20000, 320), (520, 30000, 192),
                                   # 224x192 tiles (ragged rows and columns, M = 224, K = 64)
                                   (832, 12288, 4096), (833, 12288, 192), (650, 12000, 320),
                                   (224, 40000, 64),
                                   # 224x192 register-staged tiles (K a multiple of 128,
                                   # down to two K stages; ragged rows and columns)
                                   (833, 12000, 128), (650, 12100, 384), (1300, 7000, 256),
                                   (833, 12100, 1280),
                                   # 256x256 tiles (ragged rows and columns; the last one
                                   # takes more than four rounds: the 4-stage kernel)
                                   (2048, 8192, 256), (2000, 8000, 320), (4096, 4096, 1024),
                                   (4000, 20000, 256),
                                   # rows split: 896 on 224x192 tiles, the last 51 on 128x128
                                   (947, 22016, 1024)])
def test_gemm_vs_definition(lib, dt, m, n, k):
    rng = np.random.default_rng(m * 7 + n)
    a = round_to(rng.standard_normal((m, k)), dt)
    b = round_to(rng.standard_normal((n, k)) * 0.02, dt)
    c = torch.full((m, n), float("nan"), device="cuda")
    lib.cb_gemm(dev(a, dt), dev(b, dt), c, m, n, k)
    torch.cuda.synchronize()
    ref = a @ b.T
    assert rel_err(host(c), ref) < (1e-5 if dt == "f32" else 1e-5)


# ---------------------------------------------------------------- attention
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("nq,nkv,hq,hkv,dh", [(1, 1, 1, 1, 64), (23, 90, 4, 4, 64),
                                              (70, 416, 4, 2, 64), (200, 1000, 8, 1, 128),
                                              (832, 4096, 4, 4, 128), (129, 129, 2, 2, 128),
                                              (1, 3000, 2, 1, 128), (300, 2500, 4, 2, 64),
                                              (64, 1025, 3, 3, 128), (640, 4096, 64, 8, 64)])
def test_attention_vs_oracle(lib, dt, nq, nkv, hq, hkv, dh):
    rng = np.random.default_rng(nq + nkv)
    qpos = np.sort(rng.choice(nkv, size=nq, replace=False))
    if nq == nkv:
        qpos = np.arange(nkv)
    q = round_to(rng.standard_normal((nq, hq, dh)), dt)
    k = round_to(rng.standard_normal((nkv, hkv, dh)), dt)
    v = round_to(rng.standard_normal((nkv, hkv, dh)), dt)
    out = torch.full((nq, hq, dh), float("nan"), dtype=TORCH_DT[dt], device="cuda")
    qp = torch.from_numpy(qpos.astype(np.int32)).cuda()
    lib.cb_attention(dev(q, dt), qp, nq, dev(k, dt), dev(v, dt), nkv, hq, hkv, dh, out)
    torch.cuda.synchronize()
    ref = oracle.attention(q, qpos, k, v, np.arange(nkv))
    assert rel_err(host(out), ref) < (1e-5 if dt == "f32" else 2e-2)
