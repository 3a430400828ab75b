"""Boundary details of the C ABI on the GPU: the plan workspace (the
library's own, from a caller's buffer, or under a byte limit that forces
CB_E_OOM before anything is queued) and the final RMSNorm gain given to
cb_model_create and used by cb_lm_head."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import make_case, rel_err
from tests.gpu_helpers import make_model, run_gpu_blend, chunk_inputs, dev, TORCH_DT
from workloads import TINY, WORKLOADS, round_to

pytestmark = pytest.mark.gpu
TW = WORKLOADS["tiny"]


def _blend(lib, model, case, dt, sched, plan=False):
    return run_gpu_blend(lib, model, case, dt, sched, plan=plan)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_caller_workspace_and_limit(lib, dt):
    case = make_case(TINY, TW.chunk_lens, TW.n_suffix, seed=2, dtype=dt)
    model = make_model(lib, case, dt)
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", TINY.n_layers)
    chunks = chunk_inputs(case, dt)
    need = model.workspace_size(chunks, case.offsets, case.n_suffix, dev(case.x0, dt),
                                schedule=sched)
    assert need > 0
    ref = _blend(lib, model, case, dt, sched)
    # the caller's buffer, exactly the size asked for: bit-identical results,
    # one-shot and layer-stepped
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    model.set_workspace(ws)
    for plan in (False, True):
        got = _blend(lib, model, case, dt, sched, plan=plan)
        for key in ("fused_k", "fused_v", "sel", "hidden"):
            assert torch.equal(got[key], ref[key]), (plan, key)
    # one byte short: refused with CB_E_OOM before anything is queued
    L, N = TINY.n_layers, case.n_tokens
    fk = torch.full((L, N, TINY.n_kv_heads, TINY.head_dim), float("nan"), dtype=TORCH_DT[dt],
                    device="cuda")
    fv = torch.full_like(fk, float("nan"))
    for ws_arg, nbytes in ((ws, need - 1), (None, need - 1)):
        model.set_workspace(ws_arg, nbytes)
        with pytest.raises(lib.CBError) as e:
            lib.cb_blend(model, chunks, case.offsets, case.n_suffix, dev(case.x0, dt), fk, fv,
                         schedule=sched)
        assert e.value.status == lib.CB_E_OOM
        torch.cuda.synchronize()
        assert torch.isnan(fk.float()).all() and torch.isnan(fv.float()).all()
    # a limit that fits, then the default again
    model.set_workspace(None, need)
    got = _blend(lib, model, case, dt, sched)
    assert torch.equal(got["fused_k"], ref["fused_k"])
    model.set_workspace(None, 0)
    got = _blend(lib, model, case, dt, sched)
    assert torch.equal(got["hidden"], ref["hidden"])
    with pytest.raises(lib.CBError) as e:                    # misaligned buffer
        model.set_workspace(ws.data_ptr() + 16, need)
    assert e.value.status == lib.CB_E_SHAPE


def test_model_final_norm_serves_lm_head(lib):
    """The gain given to cb_model_create is the one cb_lm_head applies when it
    is passed no final_norm; without either the call is refused."""
    dt = "bf16"
    case = make_case(TINY, (40,), 1, seed=3, dtype=dt)
    rng = np.random.default_rng(62)
    g = round_to(rng.uniform(0.5, 1.5, TINY.d_model), dt)
    w = round_to(rng.standard_normal((257, TINY.d_model)) * 0.05, dt)
    s = case.shape
    layers = [{k: dev(v, dt).contiguous() for k, v in lw.items()} for lw in case.weights]
    gd = dev(g, dt)
    model = lib.Model(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn_dim,
                      layers, final_norm=gd)
    x = torch.from_numpy(rng.standard_normal((2, TINY.d_model)).astype(np.float32)).cuda()
    a = torch.empty((2, 257), device="cuda")
    b = torch.empty_like(a)
    lib.cb_lm_head(model, x, 2, None, dev(w, dt), 257, a)
    lib.cb_lm_head(model, x, 2, gd, dev(w, dt), 257, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle.lm_head(x.cpu().numpy(), g, w, TINY.rms_eps)
    assert rel_err(a.cpu().numpy(), ref) < 2e-2
    plain = make_model(lib, case, dt)
    with pytest.raises(lib.CBError) as e:
        lib.cb_lm_head(plain, x, 2, None, dev(w, dt), 257, a)
    assert e.value.status == lib.CB_E_INVALID
