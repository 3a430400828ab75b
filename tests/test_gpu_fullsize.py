"""Parity at the benchmark's full sizes.

* Llama-2-7B shape (d 4096, 32 x 128 heads, F 11008; 6 x 640 chunk tokens +
  256 suffix tokens), four layers, against the oracle at every layer: the
  launch shapes of every kernel are those of the benchmark's layers 0-3.
* Yi-34B width (GQA 56/8), three layers with given scores: bit-exact kept
  sets and every layer against the oracle.
* Llama-2-13B width (d 5120, 40 x 128 heads, F 13824), three layers on a
  reduced prompt, KV deviation at r = 15% and at r = 100% (the full
  prefill), every layer against the oracle.
* The full 32-layer benchmark configuration (bench.py's own input builder),
  through properties that hold at any size: schedule counts, nested
  ascending kept sets, the top-k property of the reported deviations, and
  every row outside the kept set equal to the re-rotated cache.
* Llama-2-13B shape at r = 100% is bit-identical to cb_prefill of the whole
  prompt (the pages' full-prefill special case), plus the r sweep.
* Yi-34B shape (GQA 56/8) with chunk caches streamed from pinned host memory
  is bit-identical to the same fusion with device-resident caches.
"""
import dataclasses
import gc

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import make_case, run_blend, rel_err
from tests.gpu_helpers import make_model, run_gpu_blend, host, compare, dev
from workloads import WORKLOADS, round_to

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def test_llama7b_width_four_layers_vs_oracle(lib):
    """Llama-2-7B width and the benchmark's prompt layout (6 x 640 chunk
    tokens + 256 suffix), four layers in bf16, KV deviation, gradual r = 15%
    (CacheBlend explainer (0h-n0), "選択的再計算" Steps 1-4 at every layer):
    layer 0 recomputes all 4096 rows, layer 1 is the check layer, layers 2-3
    run the steady launch shapes (~890-950 rows: 224x192 GEMM tiles, the
    gathered residual of the O and down products, split-key attention over
    4096 keys).  Every layer's fused K/V, deviations and kept set, and the
    last rows, are compared with the oracle replayed on the GPU's kept sets.
    Chunk caches are seeded stand-ins (the precompute is not what is tested
    here and would dominate the CPU time)."""
    w = WORKLOADS["llama7b-4k"]
    shape = dataclasses.replace(w.shape, n_layers=4)
    case = make_case(shape, w.chunk_lens, w.n_suffix, seed=0, dtype="bf16", random_caches=True)
    model = make_model(lib, case, "bf16")
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", 4)
    gpu = run_gpu_blend(lib, model, case, "bf16", sched)
    _, swaps, errs = compare(case, gpu, sched, "bf16", oracle_dtype=np.float32)
    print(f"llama7b width: layers compared 4, threshold swaps per layer {swaps}, errors {errs}",
          flush=True)
    assert sum(swaps) <= 0.02 * sum(sched[2:])
    # without kept positions or deviations asked for, layers that keep every
    # recomputed row write their K/V from the q/k/v epilogue straight into
    # the fused cache: bit-identical
    L, N = 4, case.n_tokens
    fk = torch.full_like(gpu["fused_k"], float("nan"))
    fv = torch.full_like(fk, float("nan"))
    hid = torch.full_like(gpu["hidden"], float("nan"))
    from tests.gpu_helpers import chunk_inputs
    lib.cb_blend(model, chunk_inputs(case, "bf16"), case.offsets, case.n_suffix,
                 dev(case.x0, "bf16"), fk, fv, hidden_out=hid, schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(fk, gpu["fused_k"]) and torch.equal(fv, gpu["fused_v"])
    assert torch.equal(hid, gpu["hidden"])
    del model, gpu, fk, fv, hid
    _free()


def test_yi34b_width_given_scores_vs_oracle(lib):
    """Yi-34B width (d 7168, F 20480, 56 query / 8 KV heads of 128) in bf16
    on a reduced prompt (4 x 512 chunk tokens + 256 suffix), ranked by
    seeded given scores so the kept sets must be bit-exact at every layer.
    Three layers (layer 2 runs the steady q/k/v launch at ~620 rows): kept
    sets and every layer's fused K/V against the oracle (float32).  The last
    rows are compared on the first two layers of the same model: bf16
    rounding of the activations grows the normwise max error with depth at
    this width (measured: 0.3% of K at layer 0, 1.3% at layer 1, 1.4% at
    layer 2; last rows 1.6% after two layers, 2.1% after three), so the
    2e-2 bar on layer outputs is applied where it holds."""
    w = WORKLOADS["yi34b-8k"]
    shape = dataclasses.replace(w.shape, n_layers=3)
    case = make_case(shape, (512, 512, 512, 512), 256, seed=1, dtype="bf16",
                     random_caches=True)
    nc = case.n_chunk_tokens
    scores = np.random.default_rng(11).standard_normal(nc).astype(np.float32)
    s_dev = torch.from_numpy(scores).cuda()
    two = dataclasses.replace(case, shape=dataclasses.replace(shape, n_layers=2),
                              weights=case.weights[:2],
                              chunks=[(k[:2], v[:2]) for k, v in case.chunks])
    for c, check_hidden in ((case, False), (two, True)):
        L = c.shape.n_layers
        model = make_model(lib, c, "bf16")
        sched = oracle.schedule(nc, 1500, "gradual", L)
        gpu = run_gpu_blend(lib, model, c, "bf16", sched, dev_mode=lib.CB_DEV_GIVEN,
                            given_scores=s_dev)
        _, _, errs = compare(c, gpu, sched, "bf16", dev_mode="GIVEN",
                             given_scores=scores.astype(np.float64), allow_swaps=False,
                             check_hidden=check_hidden, oracle_dtype=np.float32)
        print(f"yi34b width, {L} layers: errors {errs}", flush=True)
        del model, gpu
        _free()


def test_llama13b_width_vs_oracle(lib):
    """Llama-2-13B width in bf16 on a reduced prompt (6 x 512 chunk tokens +
    256 suffix), KV deviation (CacheBlend explainer (0h-n0), "選択的再計算"
    Steps 1-4): gradual r = 15% (layer 2 runs the steady launch shapes at ~730
    rows) with the oracle replayed on the GPU's kept sets, and r = 100%,
    where the fusion is the oracle's full prefill of the whole prompt.  Kept
    sets and every layer's fused K/V over three layers; the last rows on the
    first two layers of the same model, where the 2e-2 bar holds at this
    width (bf16 rounding of the activations grows the normwise error by
    ~0.5% per layer: 2.0% after three layers).  Float32 oracle, seeded
    stand-in chunk caches."""
    w = WORKLOADS["llama13b-8k"]
    shape = dataclasses.replace(w.shape, n_layers=3)
    case = make_case(shape, (512,) * 6, 256, seed=2, dtype="bf16", random_caches=True)
    two = dataclasses.replace(case, shape=dataclasses.replace(shape, n_layers=2),
                              weights=case.weights[:2],
                              chunks=[(k[:2], v[:2]) for k, v in case.chunks])
    nc = case.n_chunk_tokens
    for c, check_hidden in ((case, False), (two, True)):
        L = c.shape.n_layers
        model = make_model(lib, c, "bf16")
        for sched in (oracle.schedule(nc, 1500, "gradual", L), [nc] * (L + 1)):
            gpu = run_gpu_blend(lib, model, c, "bf16", sched)
            _, swaps, errs = compare(c, gpu, sched, "bf16", oracle_dtype=np.float32,
                                     check_hidden=check_hidden)
            print(f"llama13b width, {L} layers, schedule {sched}: swaps {swaps}, errors {errs}",
                  flush=True)
            assert sum(swaps) <= 0.02 * max(1, sum(sched[2:]))
            if sched[-1] == nc:
                assert sum(swaps) == 0
            del gpu
        del model
        _free()


def _properties(npk, w, chunks, fk, fv, sel, dev, sched, Nc, L, S, layers_to_check):
    cnt = sched[1:]
    sel_h = sel.cpu().numpy()
    dev_h = dev.cpu().numpy()
    prev = np.arange(Nc)
    for l in range(L):
        s = sel_h[l, :cnt[l]]
        assert np.all(np.diff(s) > 0) and (len(s) == 0 or (s[0] >= 0 and s[-1] < Nc))
        assert set(s.tolist()) <= set(prev.tolist())
        if sched[l] > cnt[l]:
            d = dev_h[l]
            kept = np.zeros(Nc, bool)
            kept[s] = True
            cand = np.zeros(Nc, bool)
            cand[prev] = True
            assert np.all(~np.isnan(d[cand]))
            assert np.min(d[kept]) >= np.max(d[cand & ~kept])
        prev = s
    # rows outside the kept set hold the re-rotated cache (sampled layers)
    rng = np.random.default_rng(0)
    for l in layers_to_check:
        kept = set(sel_h[l, :cnt[l]].tolist())
        rows = [j for j in rng.choice(Nc, size=64, replace=False) if j not in kept]
        for j in rows:
            c = int(np.searchsorted(np.array(w.offsets), j, side="right") - 1)
            t = j - w.offsets[c]
            kc = chunks[c]["k"][l, t].float().cpu().numpy().astype(np.float64)[None]
            vc = chunks[c]["v"][l, t]
            ref = oracle.rope_rotate(kc, w.offsets[c], S.rope_base)[0]
            got = fk[l, j].float().cpu().numpy()
            assert np.max(np.abs(got - ref)) <= 2 ** -7 * max(1.0, np.max(np.abs(ref))), (l, j)
            assert torch.equal(fv[l, j].cpu(), vc.cpu()), (l, j)


def _bench_setup(npk, name, seed=0):
    import bench
    w = WORKLOADS[name]
    model, layers, x0, chunks, _ = bench.make_inputs(npk, w, seed, torch)
    return w, model, layers, x0, chunks


def _outputs(w, S, dt=torch.bfloat16):
    L, N, Nc = S.n_layers, w.n_tokens, w.n_chunk_tokens
    fk = torch.empty((L, N, S.n_kv_heads, S.head_dim), dtype=dt, device="cuda")
    fv = torch.empty_like(fk)
    sel = torch.full((L, Nc), -1, dtype=torch.int32, device="cuda")
    dev = torch.full((L, Nc), float("nan"), device="cuda")
    return fk, fv, sel, dev


def test_llama7b_benchmark_configuration_properties(lib):
    w, model, layers, x0, chunks = _bench_setup(lib, "llama7b-4k")
    S = w.shape
    sched = lib.cb_schedule(w.n_chunk_tokens, 1500, lib.CB_SCHED_GRADUAL, S.n_layers)
    fk, fv, sel, dev = _outputs(w, S)
    hid = torch.empty((w.n_suffix + sched[-1], S.d_model), device="cuda")
    cnt = lib.cb_blend(model, chunks, list(w.offsets), w.n_suffix, x0, fk, fv, sel_idx=sel,
                       hidden_out=hid, deviation=dev, schedule=sched)
    torch.cuda.synchronize()
    assert cnt == sched[1:]
    assert torch.isfinite(hid).all()
    _properties(lib, w, chunks, fk, fv, sel, dev, sched, w.n_chunk_tokens, S.n_layers, S,
                layers_to_check=(1, 2, 17, 31))
    # the same fusion through the layer-stepped API is bit-identical
    fk2, fv2, sel2, dev2 = _outputs(w, S)
    p = lib.Plan(model, chunks, list(w.offsets), w.n_suffix, x0, fk2, fv2, sel_idx=sel2,
                 deviation=dev2, schedule=sched)
    for l in range(S.n_layers):
        if l + 2 < S.n_layers:
            p.fetch_kv(l + 2)
        p.prefill_layer(l)
    p.synchronize()
    p.destroy()
    assert torch.equal(fk, fk2) and torch.equal(fv, fv2) and torch.equal(sel, sel2)
    del model, layers, x0, chunks, fk, fv, fk2, fv2
    _free()


def test_llama13b_full_recompute_is_prefill_and_r_sweep(lib):
    w, model, layers, x0, chunks = _bench_setup(lib, "llama13b-8k")
    S = w.shape
    N, Nc, L = w.n_tokens, w.n_chunk_tokens, S.n_layers
    fk, fv, sel, dev = _outputs(w, S)
    hid = torch.empty((N, S.d_model), device="cuda")
    lib.cb_blend(model, chunks, list(w.offsets), w.n_suffix, x0, fk, fv, hidden_out=hid,
                 schedule=[Nc] * (L + 1))
    kp = torch.empty_like(fk)
    vp = torch.empty_like(fv)
    hp = torch.empty_like(hid)
    lib.cb_prefill(model, x0, N, 0, kp, vp, hp)
    torch.cuda.synchronize()
    assert torch.equal(fk, kp) and torch.equal(fv, vp) and torch.equal(hid, hp)
    del kp, vp, hp, hid
    for r in (500, 1000, 1500, 1800):
        sched = lib.cb_schedule(Nc, r, lib.CB_SCHED_GRADUAL, L)
        cnt = lib.cb_blend(model, chunks, list(w.offsets), w.n_suffix, x0, fk, fv, sel_idx=sel,
                           deviation=dev, schedule=sched)
        torch.cuda.synchronize()
        assert cnt == sched[1:]
        _properties(lib, w, chunks, fk, fv, sel, dev, sched, Nc, L, S, layers_to_check=(3,))
    del model, layers, x0, chunks, fk, fv
    _free()


def test_yi34b_host_streamed_equals_device_resident(lib):
    w, model, layers, x0, chunks = _bench_setup(lib, "yi34b-8k")
    assert all(c["on_host"] for c in chunks)
    S = w.shape
    Nc, L = w.n_chunk_tokens, S.n_layers
    sched = lib.cb_schedule(Nc, 1500, lib.CB_SCHED_GRADUAL, L)
    fk, fv, sel, dev = _outputs(w, S)
    lib.cb_blend(model, chunks, list(w.offsets), w.n_suffix, x0, fk, fv, sel_idx=sel,
                 deviation=dev, schedule=sched)
    dchunks = [dict(c, k=c["k"].cuda(), v=c["v"].cuda(), on_host=0) for c in chunks]
    fk2, fv2, sel2, dev2 = _outputs(w, S)
    lib.cb_blend(model, dchunks, list(w.offsets), w.n_suffix, x0, fk2, fv2, sel_idx=sel2,
                 deviation=dev2, schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(fk, fk2) and torch.equal(fv, fv2) and torch.equal(sel, sel2)
    assert torch.equal(dev.nan_to_num(-1.0), dev2.nan_to_num(-1.0))
    _properties(lib, w, dchunks, fk, fv, sel, dev, sched, Nc, L, S, layers_to_check=(1, 30, 59))
    del model, layers, x0, chunks, dchunks, fk, fv, fk2, fv2
    _free()
