"""cb_attention_noalloc (the attention call that allocates nothing: its
split-key partials live in a fixed scratch array inside the library) against
cb_attention, which allocates a workspace per call: bit-identical outputs on
two calls in a row, the second smaller, both large enough to split their keys
over several workgroups, and both within the bf16 tolerance of the oracle
(causal attention by real position, CacheBlend explainer (0h-n0), section
"選択的再計算", Step 4)."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import rel_err
from tests.gpu_helpers import dev, host
from workloads import round_to

pytestmark = pytest.mark.gpu


def _inputs(seed, nq, nkv, hq, hkv, dh):
    rng = np.random.default_rng(seed)
    qpos = np.sort(rng.choice(nkv, size=nq, replace=False))
    q = round_to(rng.standard_normal((nq, hq, dh)), "bf16")
    k = round_to(rng.standard_normal((nkv, hkv, dh)), "bf16")
    v = round_to(rng.standard_normal((nkv, hkv, dh)), "bf16")
    return qpos, q, k, v


@pytest.mark.parametrize("first,second", [
    ((832, 4096, 32, 32, 128), (300, 2000, 8, 2, 64)),
    ((640, 4096, 64, 8, 64), (97, 1500, 4, 1, 128)),
])
def test_noalloc_attention_equals_allocating_call(lib, first, second):
    for call, (nq, nkv, hq, hkv, dh) in enumerate((first, second)):
        print(f"noalloc call {call}: nq {nq} nkv {nkv} heads {hq}/{hkv} dh {dh}", flush=True)
        qpos, q, k, v = _inputs(17 + call, nq, nkv, hq, hkv, dh)
        qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        qp = torch.from_numpy(qpos.astype(np.int32)).cuda()
        a = torch.full((nq, hq, dh), float("nan"), dtype=torch.bfloat16, device="cuda")
        b = torch.full_like(a, float("nan"))
        lib.cb_attention(qd, qp, nq, kd, vd, nkv, hq, hkv, dh, a)
        lib.cb_attention_noalloc(qd, qp, nq, kd, vd, nkv, hq, hkv, dh, b)
        torch.cuda.synchronize()
        assert torch.equal(a, b), call
        ref = oracle.attention(q, qpos, k, v, np.arange(nkv))
        assert rel_err(host(b), ref) < 2e-2, call


def test_noalloc_attention_validation(lib):
    """Arguments are checked before anything is queued (bad head counts,
    NULL buffers), as for cb_attention."""
    R = lib.RAW["cb_attention_noalloc"]
    assert R(1, None, None, 5, None, None, 10, 4, 3, 128, None, None) == lib.CB_E_SHAPE
    assert R(1, None, None, 5, None, None, 10, 4, 4, 96, None, None) == lib.CB_E_UNSUPPORTED
    assert R(1, None, None, 5, None, None, 10, 4, 4, 128, None, None) == lib.CB_E_INVALID
    assert R(7, None, None, 5, None, None, 10, 4, 4, 128, None, None) == lib.CB_E_INVALID
