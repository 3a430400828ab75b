"""Quantized chunk caches (per-channel 8- and 4-bit codes, CacheGen
explainer, "チャネル別量子化") against the oracle:

* the encoder kernel (cb_quantize_kv) reproduces the oracle's codes, scales
  and zero points bit for bit (both decide in float32), ties included;
* decoding fused with the RoPE re-alignment (cb_dequant_rerotate) matches the
  oracle's decode + rotation (fp32 1e-4, bf16 2e-2 normwise);
* fusion with quantized chunks, device-resident or pinned host, alone or
  mixed with plain chunks in a batch, matches the oracle's fusion of the
  decoded chunks, and host staging gives the same bits as device chunks.
Inputs are seeded; every code handed to the library comes from the oracle's
encoder."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import make_case, make_batch_case, quantize_case, run_blend, rel_err
from tests.gpu_helpers import (make_model, run_gpu_blend, run_gpu_batch, quant_chunk, dev,
                               host, TORCH_DT)
from tests.gpu_helpers import compare
from workloads import TINY, WORKLOADS, BATCHED_TINY, ModelShape, round_to, make_batched_requests

pytestmark = pytest.mark.gpu
TW = WORKLOADS["tiny"]
TOL = {"f32": 1e-4, "bf16": 2e-2}


def gpu_quantize(lib, x, dt, bits, layer_stride=None):
    L, n, row = x.shape
    ls = n * row if layer_stride is None else layer_stride
    buf = np.zeros((L, ls), dtype=np.float64)
    buf[:, :n * row] = x.reshape(L, -1)
    xt = dev(buf, dt)
    codes = torch.full((L, n, row * bits // 8), 0xAB, dtype=torch.uint8, device="cuda")
    qp = torch.full((L, 4, row), float("nan"), dtype=torch.float32, device="cuda")
    lib.cb_quantize_kv(xt, L, n, row, ls, bits, codes, qp[:, 0], qp[:, 1], 4 * row)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), qp[:, 0].cpu().numpy(), qp[:, 1].cpu().numpy(), qp


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("L,n,row,pad", [(3, 37, 256, 0), (2, 5, 1032, 16), (1, 640, 4096, 0),
                                         (2, 1, 64, 8), (1, 3, 8, 0), (2, 129, 72, 0),
                                         (1, 25601, 64, 0)])
def test_quantize_kernel_bit_exact(lib, dt, bits, L, n, row, pad):
    print(f"[quantize] dt={dt} bits={bits} L={L} n={n} row={row}", flush=True)
    rng = np.random.default_rng(L * 1000 + n + row)
    x = (rng.standard_normal((L, n, row)) * rng.uniform(0.01, 4, size=(L, 1, row))
         + rng.uniform(-2, 2, size=(L, 1, row)))
    if row > 3:
        x[:, :, 3] = 0.625                              # a constant channel
    x = round_to(x, dt)
    codes, scale, zero = oracle.quantize_channels(x.reshape(L, n, 1, row), bits)
    gc, gs, gz, qp = gpu_quantize(lib, x, dt, bits, n * row + pad)
    np.testing.assert_array_equal(gc, oracle.pack_codes(codes, bits))
    np.testing.assert_array_equal(gs, scale)
    np.testing.assert_array_equal(gz, zero)
    # the other two parameter rows are left alone
    assert torch.isnan(qp[:, 2:]).all()


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_kernel_ties_round_half_even(lib, bits):
    """Values exactly halfway between two levels: both sides round to even."""
    rng = np.random.default_rng(21)
    L, n, row = 2, 64, 128
    top = 2 ** bits - 1
    s = 2.0 ** -6
    z = rng.integers(-50, 50, size=(L, 1, row)) * s
    q = rng.integers(0, top, size=(L, n, row)) + 0.5
    q[:, 0] = 0
    q[:, 1] = top
    x = z + q * s
    codes, scale, zero = oracle.quantize_channels(x.reshape(L, n, 1, row), bits)
    assert np.all(codes[:, 2:] % 2 == 0)
    gc, gs, gz, _ = gpu_quantize(lib, x, "f32", bits)
    np.testing.assert_array_equal(gc, oracle.pack_codes(codes, bits))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("H,dh,n,delta", [(4, 64, 45, 0), (4, 64, 45, 7), (2, 128, 17, 1000),
                                          (2, 128, 9, -3), (32, 128, 640, 3200)])
def test_dequant_rerotate_vs_oracle(lib, dt, bits, H, dh, n, delta):
    print(f"[dequant] dt={dt} bits={bits} H={H} dh={dh} n={n} delta={delta}", flush=True)
    rng = np.random.default_rng(n + H + abs(delta))
    k = round_to(rng.standard_normal((1, n, H, dh)), dt)
    v = round_to(rng.standard_normal((1, n, H, dh)) * 0.5, dt)
    kc, ks, kz = oracle.quantize_channels(k, bits)
    vc, vs, vz = oracle.quantize_channels(v, bits)
    want_k = oracle.rope_rotate(oracle.dequantize_channels(kc, ks, kz, H, dh)[0], delta, 1e4)
    want_v = oracle.dequantize_channels(vc, vs, vz, H, dh)[0]
    qp = torch.from_numpy(np.stack([ks[0], kz[0], vs[0], vz[0]])).cuda()
    kt = torch.from_numpy(oracle.pack_codes(kc, bits)[0]).cuda()
    vt = torch.from_numpy(oracle.pack_codes(vc, bits)[0]).cuda()
    ko = torch.full((n, H, dh), float("nan"), dtype=TORCH_DT[dt], device="cuda")
    vo = torch.full_like(ko, float("nan"))
    lib.cb_dequant_rerotate(1 if bits == 8 else 2, kt, vt, qp, ko, vo, n, H, dh, delta)
    torch.cuda.synchronize()
    assert rel_err(host(ko), want_k) < TOL[dt]
    assert rel_err(host(vo), want_v) < TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [8, 4])
def test_blend_quantized_chunks_vs_oracle(lib, dt, bits):
    case = make_case(TINY, TW.chunk_lens, TW.n_suffix, seed=5, dtype=dt)
    codes, dcase = quantize_case(case, bits)
    model = make_model(lib, case, dt)
    for r, kind in ((1500, "gradual"), (0, "gradual"), (10000, "fixed")):
        print(f"[blend-q] dt={dt} bits={bits} r={r} {kind}", flush=True)
        sched = oracle.schedule(case.n_chunk_tokens, r, kind, TINY.n_layers)
        gpu = run_gpu_blend(lib, model, dcase, dt, sched, quant=(codes, bits))
        compare(dcase, gpu, sched, dt)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantized_host_chunks_equal_device_chunks(lib, bits):
    """Host codes staged per layer decode to the same bits as device codes,
    also through the layer-stepped calls."""
    dt = "bf16"
    case = make_case(TINY, TW.chunk_lens, TW.n_suffix, seed=6, dtype=dt)
    codes, dcase = quantize_case(case, bits)
    model = make_model(lib, case, dt)
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", TINY.n_layers)
    a = run_gpu_blend(lib, model, dcase, dt, sched, quant=(codes, bits))
    b = run_gpu_blend(lib, model, dcase, dt, sched, quant=(codes, bits), on_host=True)
    c = run_gpu_blend(lib, model, dcase, dt, sched, quant=(codes, bits), on_host=True, plan=True)
    for key in ("fused_k", "fused_v", "sel", "hidden", "dev"):
        assert torch.equal(a[key].nan_to_num(7.0), b[key].nan_to_num(7.0)), key
        assert torch.equal(a[key].nan_to_num(7.0), c[key].nan_to_num(7.0)), key


def test_gqa_head_dim128_quantized_vs_oracle(lib):
    shape = ModelShape(2, 256, 14, 2, 128, 512, vocab=512)
    case = make_case(shape, (100, 37, 160), 19, seed=4, dtype="f32")
    codes, dcase = quantize_case(case, 8)
    model = make_model(lib, case, "f32")
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", 2)
    gpu = run_gpu_blend(lib, model, dcase, "f32", sched, quant=(codes, 8), on_host=True)
    compare(dcase, gpu, sched, "f32")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_batch_mixed_formats_vs_oracle(lib, dt):
    """A pool mixing plain device chunks, 8-bit device chunks, 4-bit host
    chunks and 8-bit host chunks; shared chunks are staged once per layer."""
    pool_lens, reqs = make_batched_requests(BATCHED_TINY, seed=0)
    bc = make_batch_case(TINY, pool_lens, reqs, seed=0, dtype=dt)
    model = make_model(lib, bc, dt)
    used = sorted({i for r in bc.requests for i in r["chunk_ids"]})
    fmt = {i: (None, 8, 4, 8)[j % 4] for j, i in enumerate(used)}
    where = {i: j % 4 >= 2 for j, i in enumerate(used)}
    decoded = list(bc.pool)
    chunks = {}
    for i in used:
        if fmt[i] is None:
            continue
        one = dataclasses.replace(bc.cases[0], chunks=[bc.pool[i]])
        codes, dcase = quantize_case(one, fmt[i])
        decoded[i] = dcase.chunks[0]
        chunks[i] = quant_chunk(codes[0], fmt[i], on_host=where[i])
    cases = [dataclasses.replace(c, chunks=[decoded[i] for i in r["chunk_ids"]])
             for c, r in zip(bc.cases, bc.requests)]
    dbc = dataclasses.replace(bc, pool=decoded, cases=cases)
    per, _ = run_gpu_batch(lib, model, dbc, dt, override=chunks)
    for b, case in enumerate(cases):
        sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", TINY.n_layers)
        assert per[b]["sel_count"] == sched[1:], b
        compare(case, per[b], sched, dt)


def test_quantized_chunk_validation(lib):
    case = make_case(TINY, (64, 40), 8, seed=7, dtype="bf16")
    codes, dcase = quantize_case(case, 8)
    model = make_model(lib, case, "bf16")
    L = TINY.n_layers
    N = case.n_tokens
    fk = torch.empty((L, N, TINY.n_kv_heads, TINY.head_dim), dtype=torch.bfloat16, device="cuda")
    fv = torch.empty_like(fk)
    x0 = dev(case.x0, "bf16")
    good = [quant_chunk(c, 8) for c in codes]
    for bad_field, value, status in (("qparams", None, lib.CB_E_INVALID),
                                     ("kv_format", 9, lib.CB_E_INVALID),
                                     ("layer_stride", 64 * 256 + 8, lib.CB_E_SHAPE)):
        chunks = [dict(c) for c in good]
        chunks[1][bad_field] = value
        with pytest.raises(lib.CBError) as e:
            lib.cb_blend(model, chunks, case.offsets, case.n_suffix, x0, fk, fv,
                         schedule=[case.n_chunk_tokens] * (L + 1))
        assert e.value.status == status, bad_field
    # device codes with host parameters
    chunks = [dict(c) for c in good]
    chunks[0]["qparams"] = chunks[0]["qparams"].cpu().pin_memory()
    with pytest.raises(lib.CBError) as e:
        lib.cb_blend(model, chunks, case.offsets, case.n_suffix, x0, fk, fv,
                     schedule=[case.n_chunk_tokens] * (L + 1))
    assert e.value.status == lib.CB_E_INVALID
