"""First token and one decode step on a fused cache, against the oracle.
Inputs (the fused cache, the new token's embedding, the LM head) are seeded
and come from the oracle or the generators, never from the library.
Tolerances as for the fusion: fp32 1e-4, bf16 2e-2 normwise; the argmax is
an integer decided from float32 logits, so it is checked bit for bit
against numpy on the library's own logits, and against the oracle's logits
within the tolerance."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import make_case, rel_err
from tests.gpu_helpers import make_model, dev, host, TORCH_DT
from workloads import TINY, ModelShape, round_to

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def decode_inputs(shape, n_ctx, dt, seed, pad=0):
    """A fused cache of n_ctx rows (the oracle's full prefill of a seeded
    prompt, rounded to dt), laid out with layer_rows = n_ctx + pad, and the
    next token's embedding."""
    case = make_case(shape, (n_ctx,) if n_ctx else (), 1, seed=seed, dtype=dt)
    L = shape.n_layers
    if n_ctx:
        k, v, _ = oracle.prefill(case.weights, shape, case.x0[:n_ctx])
        k, v = round_to(k, dt), round_to(v, dt)
    else:
        k = v = np.zeros((L, 0, shape.n_kv_heads, shape.head_dim))
    buf_k = np.zeros((L, n_ctx + pad, shape.n_kv_heads, shape.head_dim))
    buf_v = np.zeros_like(buf_k)
    buf_k[:, :n_ctx], buf_v[:, :n_ctx] = k, v
    return case, k, v, buf_k, buf_v, case.x0[n_ctx]


_DECODE_SHAPES = {
    "gqa": ModelShape(2, 256, 14, 2, 128, 512, vocab=512),      # 7 query heads per KV head
    "gqa8": ModelShape(2, 256, 16, 2, 128, 512, vocab=512),     # 8
    "gqa64": ModelShape(2, 256, 8, 2, 64, 512, vocab=512),      # 4, head dim 64
}


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape_name,n_ctx,pad", [("tiny", 416, 0), ("tiny", 0, 3),
                                                  ("tiny", 255, 7), ("gqa", 600, 0),
                                                  ("gqa", 1, 0), ("gqa", 0, 0), ("gqa", 63, 2),
                                                  ("gqa", 64, 0), ("gqa8", 300, 5),
                                                  ("gqa64", 130, 1)])
def test_decode_step_vs_oracle(lib, dt, shape_name, n_ctx, pad):
    print(f"[decode] dt={dt} {shape_name} n_ctx={n_ctx} pad={pad}", flush=True)
    shape = TINY if shape_name == "tiny" else _DECODE_SHAPES[shape_name]
    case, k, v, bk, bv, x_new = decode_inputs(shape, n_ctx, dt, seed=7 + n_ctx, pad=pad)
    model = make_model(lib, case, dt)
    L = shape.n_layers
    fk, fv = dev(bk, dt), dev(bv, dt)
    kn = torch.full((L, shape.n_kv_heads, shape.head_dim), float("nan"), dtype=TORCH_DT[dt],
                    device="cuda")
    vn = torch.full_like(kn, float("nan"))
    hid = torch.full((shape.d_model,), float("nan"), device="cuda")
    lib.cb_decode_step(model, dev(x_new, dt), n_ctx, fk, fv, n_ctx + pad, kn, vn, hid)
    torch.cuda.synchronize()
    h_ref, k_ref, v_ref = oracle.decode_step(case.weights, shape, x_new, k, v, n_ctx)
    assert rel_err(host(hid), h_ref) < TOL[dt]
    assert rel_err(host(kn), k_ref) < TOL[dt]
    assert rel_err(host(vn), v_ref) < TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_lm_head_and_argmax(lib, dt):
    rng = np.random.default_rng(61)
    case = make_case(TINY, (40,), 1, seed=3, dtype=dt)
    model = make_model(lib, case, dt)
    d, V, rows = TINY.d_model, 1003, 3
    x = rng.standard_normal((rows, d))
    g = round_to(rng.uniform(0.5, 1.5, d), dt)
    w = round_to(rng.standard_normal((V, d)) * 0.05, dt)
    # exact ties: rows 17 and 9 of the head are equal, and made the largest for row 1
    w[9] = w[17] = round_to(np.sign(x[1]) * 0.2, dt)
    logits = torch.full((rows, V), float("nan"), device="cuda")
    am = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    xt = torch.from_numpy(x.astype(np.float32)).cuda()
    lib.cb_lm_head(model, xt, rows, dev(g, dt), dev(w, dt), V, logits, am)
    torch.cuda.synchronize()
    ref = oracle.lm_head(x.astype(np.float32), g, w, TINY.rms_eps)
    got = logits.cpu().numpy().astype(np.float64)
    assert rel_err(got, ref) < TOL[dt]
    for r in range(rows):
        # the integer decision on the library's own float32 logits: exact
        assert am[r].item() == oracle.argmax_first(logits[r].cpu().numpy())
        # and a maximum of the oracle's logits within the tolerance
        assert ref[r].max() - ref[r][am[r].item()] <= TOL[dt] * np.abs(ref[r]).max()
    assert am[1].item() == 9


def test_decode_consistency_with_gpu_prefill(lib):
    """On the GPU: decoding token N over the library's prefill cache of N
    tokens agrees with the library's prefill of N+1 tokens (fp32)."""
    dt = "f32"
    shape = TINY
    case = make_case(shape, (300,), 1, seed=11, dtype=dt)
    model = make_model(lib, case, dt)
    L, n = shape.n_layers, 300
    x = dev(case.x0[:n + 1], dt)
    k = torch.empty((L, n + 1, shape.n_kv_heads, shape.head_dim), device="cuda")
    v = torch.empty_like(k)
    hid = torch.empty((n + 1, shape.d_model), device="cuda")
    lib.cb_prefill(model, x, n + 1, 0, k, v, hid)
    k2 = torch.empty((L, n, shape.n_kv_heads, shape.head_dim), device="cuda")
    v2 = torch.empty_like(k2)
    lib.cb_prefill(model, x[:n].contiguous(), n, 0, k2, v2, None)
    kn = torch.empty((L, shape.n_kv_heads, shape.head_dim), device="cuda")
    vn = torch.empty_like(kn)
    h1 = torch.empty((shape.d_model,), device="cuda")
    lib.cb_decode_step(model, x[n].contiguous(), n, k2, v2, n, kn, vn, h1)
    torch.cuda.synchronize()
    assert rel_err(host(h1), host(hid[n])) < 1e-4
    assert rel_err(host(kn), host(k[:, n])) < 1e-4


def test_decode_validation(lib):
    case = make_case(TINY, (40,), 1, seed=3, dtype="f32")
    model = make_model(lib, case, "f32")
    t = torch.zeros(4096, device="cuda")
    with pytest.raises(lib.CBError) as e:
        lib.cb_decode_step(model, t, 5, t, t, 4, t, t, t)       # layer_rows < n_ctx
    assert e.value.status == lib.CB_E_INVALID
    with pytest.raises(lib.CBError) as e:
        lib.cb_lm_head(model, t, 1, t, t, 0, t)                 # vocab 0
    assert e.value.status == lib.CB_E_INVALID
