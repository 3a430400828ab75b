"""Selection variants on the GPU against the oracle: the given-scores mode
(CB_DEV_GIVEN) ranks chunk tokens by caller-supplied scores through the same
exact top-k and gradual filtering, so with identical scores on both sides
every kept set is bit-exact, at every layer, alone and in a batch; the
fused K/V and outputs then match to the usual tolerance."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import make_case, make_batch_case, rel_err
from tests.gpu_helpers import make_model, run_gpu_blend, host, dev, chunk_inputs, TORCH_DT
from workloads import TINY, WORKLOADS, BATCHED_TINY, make_batched_requests

pytestmark = pytest.mark.gpu
TW = WORKLOADS["tiny"]
TOL = {"f32": 1e-4, "bf16": 2e-2}


def seeded_scores(n, seed, ties=False):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal(n).astype(np.float32)
    if ties:
        s = np.round(s * 2) / 2           # many exact ties -> position order decides
        s[rng.integers(0, n, size=3)] = np.nan
    return s


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("ties", [False, True])
def test_given_scores_blend_bit_exact_selection(lib, dt, ties):
    case = make_case(TINY, TW.chunk_lens, TW.n_suffix, seed=8, dtype=dt)
    model = make_model(lib, case, dt)
    nc = case.n_chunk_tokens
    scores = seeded_scores(nc, 9, ties)
    for r, kind in ((1500, "gradual"), (500, "fixed"), (10000, "gradual")):
        sched = oracle.schedule(nc, r, kind, TINY.n_layers)
        s_dev = torch.from_numpy(scores).cuda()
        out = run_gpu_blend_given(lib, model, case, dt, sched, s_dev)
        ref = oracle.blend(case.weights, case.shape, case.x0, case.chunks, case.offsets,
                           case.n_suffix, sched, dev_mode="GIVEN", given_scores=scores)
        for l in range(TINY.n_layers):
            k = sched[l + 1]
            np.testing.assert_array_equal(out["sel"][l, :k].cpu().numpy(), ref["sel"][l])
            assert rel_err(host(out["fused_k"][l]), ref["fused_k"][l]) < TOL[dt]
            assert rel_err(host(out["fused_v"][l]), ref["fused_v"][l]) < TOL[dt]
        assert rel_err(host(out["hidden"]), ref["hidden"]) < TOL[dt]


def run_gpu_blend_given(lib, model, case, dt, sched, scores):
    s = case.shape
    L, N, nc = s.n_layers, case.n_tokens, case.n_chunk_tokens
    fk = torch.full((L, N, s.n_kv_heads, s.head_dim), float("nan"), dtype=TORCH_DT[dt],
                    device="cuda")
    fv = torch.full_like(fk, float("nan"))
    sel = torch.full((L, max(1, nc)), -1, dtype=torch.int32, device="cuda")
    dv = torch.full((L, max(1, nc)), float("nan"), device="cuda")
    hid = torch.full((case.n_suffix + sched[-1], s.d_model), float("nan"), device="cuda")
    lib.cb_blend(model, chunk_inputs(case, dt), case.offsets, case.n_suffix, dev(case.x0, dt), fk,
                 fv, sel_idx=sel, hidden_out=hid, deviation=dv, schedule=sched,
                 dev_mode=lib.CB_DEV_GIVEN, given_scores=scores)
    torch.cuda.synchronize()
    return {"fused_k": fk, "fused_v": fv, "sel": sel, "hidden": hid, "dev": dv}


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_given_scores_batch_bit_exact(lib, dt):
    from tests.gpu_helpers import pool_inputs
    pool_lens, reqs = make_batched_requests(BATCHED_TINY, seed=0)
    bc = make_batch_case(TINY, pool_lens, reqs, seed=0, dtype=dt)
    model = make_model(lib, bc, dt)
    L = TINY.n_layers
    ncs = [c.n_chunk_tokens for c in bc.cases]
    scores = seeded_scores(sum(ncs), 12, ties=True)
    Ntot = sum(c.n_tokens for c in bc.cases)
    fk = torch.empty((L, Ntot, TINY.n_kv_heads, TINY.head_dim), dtype=TORCH_DT[dt], device="cuda")
    fv = torch.empty_like(fk)
    sel = torch.full((L, sum(ncs)), -1, dtype=torch.int32, device="cuda")
    pool = pool_inputs(bc, dt)
    req = [{"chunk_ids": r["chunk_ids"], "n_suffix": r["n_suffix"]} for r in bc.requests]
    cnt = lib.cb_blend_batch(model, pool, req, dev(bc.x0, dt), fk, fv, sel_idx=sel,
                             dev_mode=lib.CB_DEV_GIVEN,
                             given_scores=torch.from_numpy(scores).cuda())
    torch.cuda.synchronize()
    C = 0
    for b, case in enumerate(bc.cases):
        sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", L)
        ref = oracle.blend(case.weights, case.shape, case.x0, case.chunks, case.offsets,
                           case.n_suffix, sched, dev_mode="GIVEN",
                           given_scores=scores[C:C + ncs[b]])
        for l in range(L):
            k = sched[l + 1]
            np.testing.assert_array_equal(sel[l, C:C + k].cpu().numpy(), ref["sel"][l])
        C += ncs[b]


def test_given_scores_validation(lib):
    case = make_case(TINY, (64, 40), 8, seed=7, dtype="f32")
    model = make_model(lib, case, "f32")
    L, N = TINY.n_layers, case.n_tokens
    fk = torch.empty((L, N, TINY.n_kv_heads, TINY.head_dim), device="cuda")
    fv = torch.empty_like(fk)
    x0 = dev(case.x0, "f32")
    with pytest.raises(lib.CBError) as e:      # GIVEN without scores
        lib.cb_blend(model, chunk_inputs(case, "f32"), case.offsets, case.n_suffix, x0, fk, fv,
                     dev_mode=lib.CB_DEV_GIVEN)
    assert e.value.status == lib.CB_E_INVALID
    with pytest.raises(lib.CBError) as e:      # scores without GIVEN
        lib.cb_blend(model, chunk_inputs(case, "f32"), case.offsets, case.n_suffix, x0, fk, fv,
                     given_scores=torch.zeros(104, device="cuda"))
    assert e.value.status == lib.CB_E_INVALID
