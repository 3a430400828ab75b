"""End-to-end parity of the fusion path (cb_blend, the layer-stepped API and
cb_prefill) against the oracle on seeded tiny workloads: 3 chunks x 128
tokens + 32 suffix tokens, 2 layers, d = 256 (several tiles and ragged
tails), in fp32 (tolerance 1e-4) and bf16 (2e-2), normwise max relative
error max|g - o| / max|o|."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import make_case, run_blend, run_full, rel_err
from tests.gpu_helpers import make_model, run_gpu_blend, dev, host, TORCH_DT, compare, TOL
from workloads import TINY, WORKLOADS, ModelShape

pytestmark = pytest.mark.gpu
TW = WORKLOADS["tiny"]


@pytest.fixture(scope="module", params=["f32", "bf16"])
def tiny(request, lib):
    dt = request.param
    case = make_case(TINY, TW.chunk_lens, TW.n_suffix, seed=0, dtype=dt)
    return dt, case, make_model(lib, case, dt)


@pytest.mark.parametrize("r,kind", [(1500, "gradual"), (1500, "fixed"), (500, "gradual"),
                                    (1800, "fixed"), (0, "gradual"), (10000, "gradual")])
def test_tiny_blend_vs_oracle(lib, tiny, r, kind):
    dt, case, model = tiny
    sched = oracle.schedule(case.n_chunk_tokens, r, kind, TINY.n_layers)
    gpu = run_gpu_blend(lib, model, case, dt, sched)
    assert gpu["sel_count"] == sched[1:]
    compare(case, gpu, sched, dt)


def test_tiny_full_recompute_equals_prefill(lib, tiny):
    """r = 100% through cb_blend equals cb_prefill on the whole prompt, and
    both match the oracle's full prefill."""
    dt, case, model = tiny
    N, L = case.n_tokens, TINY.n_layers
    sched = [case.n_chunk_tokens] * (L + 1)
    gpu = run_gpu_blend(lib, model, case, dt, sched)
    k = torch.empty_like(gpu["fused_k"])
    v = torch.empty_like(gpu["fused_v"])
    hid = torch.empty((N, TINY.d_model), device="cuda")
    lib.cb_prefill(model, dev(case.x0, dt), N, 0, k, v, hid)
    torch.cuda.synchronize()
    assert torch.equal(k, gpu["fused_k"]) and torch.equal(v, gpu["fused_v"])
    assert torch.equal(hid, gpu["hidden"])
    fk, fv, outs = run_full(case)
    assert rel_err(host(k), fk) < TOL[dt] and rel_err(host(v), fv) < TOL[dt]
    assert rel_err(host(hid), outs[-1]) < TOL[dt]


def test_prefill_at_offset_vs_oracle(lib, tiny):
    """Chunk precompute at chunk-local positions and prefill at pos0 > 0."""
    dt, case, model = tiny
    n = 200
    x = case.x0[:n]
    for pos0 in (0, 333):
        k = torch.empty((TINY.n_layers, n, TINY.n_kv_heads, TINY.head_dim),
                        dtype=TORCH_DT[dt], device="cuda")
        v = torch.empty_like(k)
        hid = torch.empty((n, TINY.d_model), device="cuda")
        lib.cb_prefill(model, dev(x, dt), n, pos0, k, v, hid)
        torch.cuda.synchronize()
        rk, rv, outs = oracle.prefill(case.weights, TINY, x, pos0=pos0)
        assert rel_err(host(k), rk) < TOL[dt]
        assert rel_err(host(v), rv) < TOL[dt]
        assert rel_err(host(hid), outs[-1]) < TOL[dt]


def test_layer_stepped_equals_one_shot(lib, tiny):
    dt, case, model = tiny
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", TINY.n_layers)
    a = run_gpu_blend(lib, model, case, dt, sched)
    b = run_gpu_blend(lib, model, case, dt, sched, plan=True)
    for key in ("fused_k", "fused_v", "sel", "hidden"):
        assert torch.equal(a[key], b[key]), key


def test_pinned_host_chunks_equal_device_chunks(lib, tiny):
    """Side-stream H2D + in-place rotation gives bit-identical results to
    device-resident chunks (event ordering check)."""
    dt, case, model = tiny
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", TINY.n_layers)
    a = run_gpu_blend(lib, model, case, dt, sched)
    b = run_gpu_blend(lib, model, case, dt, sched, on_host=True)
    for key in ("fused_k", "fused_v", "sel", "hidden", "dev"):
        assert torch.equal(a[key].nan_to_num(7.0), b[key].nan_to_num(7.0)), key


@pytest.mark.parametrize("mode,name", [(1, "K"), (2, "V")])
def test_dev_modes(lib, mode, name):
    case = make_case(TINY, TW.chunk_lens, TW.n_suffix, seed=1, dtype="f32")
    model = make_model(lib, case, "f32")
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "fixed", TINY.n_layers)
    gpu = run_gpu_blend(lib, model, case, "f32", sched, dev_mode=mode)
    compare(case, gpu, sched, "f32", dev_mode=name)


def test_gqa_head_dim128_blend_vs_oracle(lib):
    """GQA (7 query heads per KV head) with 128-wide heads, ragged chunks."""
    shape = ModelShape(2, 256, 14, 2, 128, 512, vocab=512)
    case = make_case(shape, (100, 37, 160), 19, seed=4, dtype="f32")
    model = make_model(lib, case, "f32")
    for r, kind in ((1500, "gradual"), (10000, "fixed")):
        sched = oracle.schedule(case.n_chunk_tokens, r, kind, 2)
        gpu = run_gpu_blend(lib, model, case, "f32", sched)
        compare(case, gpu, sched, "f32")


def test_single_chunk_r0_is_cache_bit_exact(lib):
    """One chunk at offset 0, no recompute: the fused cache is the input
    cache bit for bit (rotation by 0 is exact)."""
    case = make_case(TINY, (96,), 0, seed=2, dtype="bf16")
    model = make_model(lib, case, "bf16")
    gpu = run_gpu_blend(lib, model, case, "bf16", [0] * 3)
    np.testing.assert_array_equal(host(gpu["fused_k"]), case.chunks[0][0])
    np.testing.assert_array_equal(host(gpu["fused_v"]), case.chunks[0][1])


def test_seeds_and_schedule_sweep_fp32(lib):
    for seed in (1, 2, 3):
        case = make_case(TINY, TW.chunk_lens, TW.n_suffix, seed=seed, dtype="f32")
        model = make_model(lib, case, "f32")
        for r in (100, 1000, 5000):
            sched = oracle.schedule(case.n_chunk_tokens, r, "gradual", 2)
            gpu = run_gpu_blend(lib, model, case, "f32", sched)
            compare(case, gpu, sched, "f32")


def test_error_paths(lib, tiny):
    dt, case, model = tiny
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", TINY.n_layers)
    chunks = [dict(c) for c in __import__("tests.gpu_helpers", fromlist=["x"]).chunk_inputs(case, dt)]
    x0 = dev(case.x0, dt)
    fk = torch.empty((TINY.n_layers, case.n_tokens, TINY.n_kv_heads, TINY.head_dim),
                     dtype=TORCH_DT[dt], device="cuda")
    fv = torch.empty_like(fk)
    # pageable host memory for an on_host chunk
    bad = [dict(c) for c in chunks]
    bad[1]["k"] = bad[1]["k"].cpu()
    bad[1]["v"] = bad[1]["v"].cpu()
    bad[1]["on_host"] = 1
    with pytest.raises(lib.CBError) as e:
        lib.cb_blend(model, bad, case.offsets, case.n_suffix, x0, fk, fv, schedule=sched)
    assert e.value.status == lib.CB_E_NOT_PINNED
    # gaps between chunks
    with pytest.raises(lib.CBError) as e:
        lib.cb_blend(model, chunks, [0, 129, 256], case.n_suffix, x0, fk, fv, schedule=sched)
    assert e.value.status == lib.CB_E_INVALID
    # increasing schedule
    with pytest.raises(lib.CBError) as e:
        lib.cb_blend(model, chunks, case.offsets, case.n_suffix, x0, fk, fv,
                     schedule=[384, 50, 60])
    assert e.value.status == lib.CB_E_SCHEDULE
    # layer-stepped calls out of order
    p = lib.Plan(model, chunks, case.offsets, case.n_suffix, x0, fk, fv, schedule=sched)
    with pytest.raises(lib.CBError) as e:
        p.prefill_layer(1)
    assert e.value.status == lib.CB_E_BAD_STATE
    p.prefill_layer(0)
    p.prefill_layer(1)
    p.synchronize()
    p.destroy()


def test_long_context_bf16_blend_vs_oracle(lib):
    """A context long enough for the attention to split its keys over several
    workgroups (segments merged by the combine pass), ragged chunk lengths."""
    case = make_case(TINY, (500, 403, 611), 61, seed=5, dtype="bf16")
    model = make_model(lib, case, "bf16")
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", TINY.n_layers)
    gpu = run_gpu_blend(lib, model, case, "bf16", sched)
    compare(case, gpu, sched, "bf16")
    full = [case.n_chunk_tokens] * 3
    gpu = run_gpu_blend(lib, model, case, "bf16", full)
    compare(case, gpu, full, "bf16")


def test_binding_rejects_mismatched_outputs(lib, tiny):
    """Outputs of the wrong element type or too small for the request are
    rejected by the binding before any kernel is queued."""
    dt, case, model = tiny
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", TINY.n_layers)
    chunks = __import__("tests.gpu_helpers", fromlist=["x"]).chunk_inputs(case, dt)
    x0 = dev(case.x0, dt)
    L, N, Nc = TINY.n_layers, case.n_tokens, case.n_chunk_tokens
    shape = (L, N, TINY.n_kv_heads, TINY.head_dim)
    fk = torch.empty(shape, dtype=TORCH_DT[dt], device="cuda")
    fv = torch.empty_like(fk)
    other = torch.float32 if dt == "bf16" else torch.bfloat16
    cases = [
        dict(fused_k=torch.empty(shape, dtype=other, device="cuda")),
        dict(fused_v=fv[:, :N - 1].contiguous()),
        dict(sel_idx=torch.empty((L, Nc), dtype=torch.int64, device="cuda")),
        dict(hidden_out=torch.empty((case.n_suffix + sched[-1] - 1, TINY.d_model),
                                    device="cuda")),
        dict(deviation=torch.empty((L, Nc - 1), device="cuda")),
    ]
    for over in cases:
        kw = dict(fused_k=fk, fused_v=fv)
        kw.update(over)
        with pytest.raises(lib.CBError) as e:
            lib.cb_blend(model, chunks, case.offsets, case.n_suffix, x0, schedule=sched, **kw)
        assert e.value.status in (lib.CB_E_INVALID, lib.CB_E_SHAPE), over.keys()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["gradual", "fixed"])
def test_layers_keeping_every_row_in_place(lib, kind, dt):
    """Layers where every recomputed row is kept leave the row maps as they
    are, launch no selection and write their new K/V straight into the fused
    cache from the q/k/v epilogue when neither kept positions nor deviations
    are asked for; the fusion is bit-identical to one that asks for them
    (which runs the selection and the scatter at every layer), and matches
    the oracle."""
    shape = ModelShape(5, 256, 4, 4, 64, 512, vocab=512)
    case = make_case(shape, (100, 37, 160), 19, seed=6, dtype=dt)
    model = make_model(lib, case, dt)
    sched = oracle.schedule(case.n_chunk_tokens, 1500, kind, shape.n_layers)
    assert any(a == b for a, b in zip(sched, sched[1:]))
    full = run_gpu_blend(lib, model, case, dt, sched)
    L, N = shape.n_layers, case.n_tokens
    fk = torch.full((L, N, shape.n_kv_heads, shape.head_dim), float("nan"), dtype=TORCH_DT[dt],
                    device="cuda")
    fv = torch.full_like(fk, float("nan"))
    hid = torch.full((case.n_suffix + sched[-1], shape.d_model), float("nan"), device="cuda")
    from tests.gpu_helpers import chunk_inputs
    lib.cb_blend(model, chunk_inputs(case, dt), case.offsets, case.n_suffix,
                 dev(case.x0, dt), fk, fv, hidden_out=hid, schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(fk, full["fused_k"]) and torch.equal(fv, full["fused_v"])
    assert torch.equal(hid, full["hidden"])
    # kept positions asked for without deviations: in-place layers get the
    # positions of the last layer that selected, copied after the last layer
    sel = torch.full((L, case.n_chunk_tokens), -1, dtype=torch.int32, device="cuda")
    lib.cb_blend(model, chunk_inputs(case, dt), case.offsets, case.n_suffix,
                 dev(case.x0, dt), fk, fv, sel_idx=sel, schedule=sched)
    torch.cuda.synchronize()
    for l in range(L):
        k = sched[l + 1]
        assert torch.equal(sel[l, :k], full["sel"][l, :k]), l
    assert torch.equal(fk, full["fused_k"]) and torch.equal(fv, full["fused_v"])
    compare(case, full, sched, dt)
