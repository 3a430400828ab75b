"""Selection by per-token attention deviation (CB_DEV_ATTN) against the
oracle: the CacheBlend explainer (0h-n0), "HKVD（High KV Deviation）トークン
選定", selects the first layer's tokens by attention deviation (eq. 2 of
"KVキャッシュの定義と偏差メトリクス" taken row by row) and later layers by KV
deviation.

* cb_attention_deviation (the measure alone) vs oracle.attention_deviation
  on the same bf16 inputs, with grouped-query heads, head dims 64 and 128,
  ragged lengths over several 64-key blocks and 128-query tiles; identical
  keys give zero up to float32 rounding.
* cb_blend / cb_blend_batch with CB_DEV_ATTN vs oracle.blend(dev_mode='ATTN')
  replayed on the GPU's kept sets: kept sets equal to the replay's top-k (or
  swapped within the rounding band), fused K/V and last rows in tolerance."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import make_case, make_batch_case, rel_err
from tests.gpu_helpers import make_model, run_gpu_blend, run_gpu_batch, dev, host, compare
from workloads import TINY, WORKLOADS, BATCHED_TINY, ModelShape, round_to, make_batched_requests

pytestmark = pytest.mark.gpu
TW = WORKLOADS["tiny"]


@pytest.mark.parametrize("n,hq,hkv,dh", [(1, 4, 4, 64), (7, 2, 1, 128), (130, 4, 2, 64),
                                         (300, 14, 2, 128), (1000, 8, 8, 128),
                                         (3840, 4, 4, 128)])
def test_attention_deviation_kernel_vs_oracle(lib, n, hq, hkv, dh):
    rng = np.random.default_rng(n + hq)
    q = round_to(rng.standard_normal((n, hq, dh)), "bf16")
    k1 = round_to(rng.standard_normal((n, hkv, dh)), "bf16")
    k0 = round_to(k1 + 0.3 * rng.standard_normal((n, hkv, dh)), "bf16")
    out = torch.full((n,), float("nan"), device="cuda")
    lib.cb_attention_deviation(dev(q, "bf16"), dev(k1, "bf16"), dev(k0, "bf16"), n, hq, hkv, dh,
                               out)
    same = torch.full((n,), float("nan"), device="cuda")
    lib.cb_attention_deviation(dev(q, "bf16"), dev(k1, "bf16"), dev(k1, "bf16"), n, hq, hkv, dh,
                               same)
    torch.cuda.synchronize()
    ref = oracle.attention_deviation(q, np.arange(n), k1, k0, np.arange(n))
    assert np.all(np.isfinite(host(out)))
    assert rel_err(host(out), ref) < 1e-3
    # the kernel sums A/l1^2 - 2B/(l1 l0) + C/l0^2 in one pass over the keys:
    # values that are zero by definition come out at float32 rounding level
    assert host(out)[0] <= 1e-6                      # row 0 sees one key under both
    assert float(same.abs().max()) <= 1e-6           # identical keys


def test_attention_deviation_validation(lib):
    R = lib.RAW["cb_attention_deviation"]
    assert R(lib.CB_F32, None, None, None, 5, 4, 4, 64, None, None) == lib.CB_E_UNSUPPORTED
    assert R(lib.CB_BF16, None, None, None, 5, 4, 3, 64, None, None) == lib.CB_E_SHAPE
    assert R(lib.CB_BF16, None, None, None, 5, 4, 4, 96, None, None) == lib.CB_E_UNSUPPORTED
    assert R(lib.CB_BF16, None, None, None, 5, 4, 4, 64, None, None) == lib.CB_E_INVALID
    assert R(lib.CB_BF16, None, None, None, 0, 4, 4, 64, None, None) == lib.CB_OK


@pytest.mark.parametrize("shape,lens,ns,seed", [
    (TINY, TW.chunk_lens, TW.n_suffix, 0),
    (ModelShape(4, 256, 14, 2, 128, 512, vocab=512), (100, 37, 160), 19, 4),
])
@pytest.mark.parametrize("r,kind", [(1500, "gradual"), (1800, "fixed"), (10000, "gradual")])
def test_blend_attention_deviation_vs_oracle(lib, shape, lens, ns, seed, r, kind):
    case = make_case(shape, lens, ns, seed=seed, dtype="bf16")
    model = make_model(lib, case, "bf16")
    sched = oracle.schedule(case.n_chunk_tokens, r, kind, shape.n_layers)
    gpu = run_gpu_blend(lib, model, case, "bf16", sched, dev_mode=lib.CB_DEV_ATTN)
    assert gpu["sel_count"] == sched[1:]
    ref, swaps, errs = compare(case, gpu, sched, "bf16", dev_mode="ATTN")
    # the check layer ranked by attention deviation: the first chunk (no
    # preceding context) deviates by rounding only
    if sched[1] > sched[2]:
        n0 = lens[0]
        d = host(gpu["dev"][1])
        assert np.max(d[:n0]) < 1e-2 * np.max(d[n0:])
    print(f"ATTN blend {shape.n_layers} layers r {r} {kind}: swaps {swaps}, errors {errs}",
          flush=True)


def test_batch_attention_deviation_vs_oracle(lib):
    """A batch mixing schedules: requests rank by attention deviation while
    all their chunk rows are candidates, by KV deviation afterwards; a
    request with no recompute has nothing to rank."""
    pool_lens, reqs = make_batched_requests(BATCHED_TINY, seed=3)
    reqs = reqs[:4]
    bc = make_batch_case(TINY, pool_lens, reqs, seed=3, dtype="bf16")
    model = make_model(lib, bc, "bf16")
    L = TINY.n_layers
    Nc = [c.n_chunk_tokens for c in bc.cases]
    scheds = [oracle.schedule(Nc[0], 1500, "gradual", L), oracle.schedule(Nc[1], 1800, "fixed", L),
              [0] * (L + 1), oracle.schedule(Nc[3], 500, "gradual", L)]
    per, _ = run_gpu_batch(lib, model, bc, "bf16", schedules=scheds, dev_mode=lib.CB_DEV_ATTN)
    for b, case in enumerate(bc.cases):
        assert per[b]["sel_count"] == scheds[b][1:]
        compare(case, per[b], scheds[b], "bf16", dev_mode="ATTN",
                check_hidden=case.n_suffix + scheds[b][-1] > 0)


def test_attention_deviation_mode_needs_bf16(lib):
    case = make_case(TINY, (64, 40), 8, seed=7, dtype="f32")
    model = make_model(lib, case, "f32")
    L, N = TINY.n_layers, case.n_tokens
    fk = torch.empty((L, N, TINY.n_kv_heads, TINY.head_dim), device="cuda")
    from tests.gpu_helpers import chunk_inputs
    with pytest.raises(lib.CBError) as e:
        lib.cb_blend(model, chunk_inputs(case, "f32"), case.offsets, case.n_suffix,
                     dev(case.x0, "f32"), fk, torch.empty_like(fk), dev_mode=lib.CB_DEV_ATTN)
    assert e.value.status == lib.CB_E_UNSUPPORTED
