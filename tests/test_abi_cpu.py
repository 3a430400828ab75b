"""C-ABI checks that need no GPU: the library loads, exports every function
include/cacheblend.h declares, and its host-only logic (schedule, argument
validation) behaves as documented.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "cacheblend.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cb_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def npk():
    import non_prefix_kv_amd
    return non_prefix_kv_amd


def test_exports_every_declared_symbol(npk):
    lib = ctypes.CDLL(npk.LIB_PATH)
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(npk.EXPORTED)


def test_abi_version(npk):
    assert npk.cb_abi_version() == npk.CB_ABI_VERSION == 6


@pytest.mark.parametrize("n", [0, 1, 10, 384, 3840, 7680, 8192])
@pytest.mark.parametrize("r", [0, 1, 500, 1000, 1500, 1800, 5000, 9999, 10000])
@pytest.mark.parametrize("kind", ["gradual", "fixed"])
def test_schedule_matches_oracle(npk, n, r, kind):
    code = npk.CB_SCHED_GRADUAL if kind == "gradual" else npk.CB_SCHED_FIXED
    for L in (1, 2, 32, 40, 60):
        assert npk.cb_schedule(n, r, code, L) == oracle.schedule(n, r, kind, L)


def test_schedule_rejects_bad_args(npk):
    with pytest.raises(npk.CBError) as e:
        npk.cb_schedule(100, 10001, npk.CB_SCHED_FIXED, 4)
    assert e.value.status == npk.CB_E_SCHEDULE
    with pytest.raises(npk.CBError) as e:
        npk.cb_schedule(100, 100, 7, 4)
    assert e.value.status == npk.CB_E_INVALID
    assert "kind" in npk.cb_last_error()


def test_model_create_validation(npk):
    raw = npk.RAW["cb_model_create"]
    h = ctypes.c_void_p()
    assert raw(None, None, None, ctypes.byref(h)) == npk.CB_E_INVALID
    cfg = npk.cb_model_cfg(2, 256, 4, 4, 96, 1024, 1e4, 1e-5, npk.CB_BF16)
    assert raw(ctypes.byref(cfg), None, None, ctypes.byref(h)) == npk.CB_E_UNSUPPORTED
    cfg = npk.cb_model_cfg(2, 256, 4, 3, 64, 1024, 1e4, 1e-5, npk.CB_BF16)
    assert raw(ctypes.byref(cfg), None, None, ctypes.byref(h)) == npk.CB_E_SHAPE
    cfg = npk.cb_model_cfg(2, 250, 4, 4, 64, 1024, 1e4, 1e-5, npk.CB_BF16)
    assert raw(ctypes.byref(cfg), None, None, ctypes.byref(h)) == npk.CB_E_SHAPE
    cfg = npk.cb_model_cfg(2, 256, 4, 4, 64, 1024, 1e4, 1e-5, 5)
    assert raw(ctypes.byref(cfg), None, None, ctypes.byref(h)) == npk.CB_E_INVALID
    cfg = npk.cb_model_cfg(2, 256, 4, 4, 64, 1024, 1e4, 1e-5, npk.CB_F32)
    assert raw(ctypes.byref(cfg), None, None, ctypes.byref(h)) == npk.CB_E_INVALID   # NULL layers
    w = (npk.cb_layer_weights * 2)()
    assert raw(ctypes.byref(cfg), w, None, ctypes.byref(h)) == npk.CB_E_INVALID     # NULL weights
    assert not h.value


def test_kernel_entry_validation(npk):
    R = npk.RAW
    assert R["cb_topk_select"](None, 5, 6, None, None) == npk.CB_E_INVALID
    assert R["cb_topk_select"](None, -1, 0, None, None) == npk.CB_E_INVALID
    assert R["cb_gemm"](npk.CB_BF16, None, None, None, 8, 8, 48, None) == npk.CB_E_SHAPE
    assert R["cb_gemm"](3, None, None, None, 8, 8, 64, None) == npk.CB_E_INVALID
    assert R["cb_attention"](npk.CB_BF16, None, None, 4, None, None, 8, 4, 4, 96, None,
                             None) == npk.CB_E_UNSUPPORTED
    assert R["cb_attention"](npk.CB_BF16, None, None, 4, None, None, 8, 4, 3, 64, None,
                             None) == npk.CB_E_SHAPE
    assert R["cb_rope_rerotate"](npk.CB_BF16, None, None, None, None, 4, 2, 64, 3, 1e4,
                                 None) == npk.CB_E_INVALID
    assert R["cb_rope_rerotate"](npk.CB_BF16, 16, 16, None, None, 4, 2, 60, 3, 1e4,
                                 None) == npk.CB_E_SHAPE
    assert R["cb_deviation"](npk.CB_F32, 16, 16, 16, 16, 4, 64, 3, 16, None) == npk.CB_E_INVALID
    assert R["cb_gather_rows"](16, 16, 16, 4, 6, None) == npk.CB_E_SHAPE
    # quantized chunk entries: bit widths, formats, row sizes, alignment
    assert R["cb_quantize_kv"](npk.CB_BF16, 16, 2, 8, 64, 512, 6, 16, 16, 16, 256,
                               None) == npk.CB_E_INVALID
    assert R["cb_quantize_kv"](npk.CB_BF16, 16, 2, 8, 60, 480, 8, 16, 16, 16, 240,
                               None) == npk.CB_E_SHAPE
    assert R["cb_quantize_kv"](npk.CB_BF16, 16, 2, 8, 64, 100, 8, 16, 16, 16, 256,
                               None) == npk.CB_E_SHAPE
    assert R["cb_quantize_kv"](npk.CB_BF16, 8, 2, 8, 64, 512, 8, 16, 16, 16, 256,
                               None) == npk.CB_E_SHAPE
    assert R["cb_quantize_kv"](npk.CB_BF16, None, 2, 8, 64, 512, 4, 16, 16, 16, 256,
                               None) == npk.CB_E_INVALID
    assert R["cb_quantize_kv"](npk.CB_BF16, None, 0, 8, 64, 512, 4, None, None, None, 256,
                               None) == npk.CB_OK
    assert R["cb_dequant_rerotate"](npk.CB_BF16, npk.CB_KV_PLAIN, 16, 16, 16, 16, 16, 4, 2, 64, 3,
                                    1e4, None) == npk.CB_E_INVALID
    assert R["cb_dequant_rerotate"](npk.CB_BF16, npk.CB_KV_U8, 16, 16, None, 16, 16, 4, 2, 64, 3,
                                    1e4, None) == npk.CB_E_INVALID
    assert R["cb_dequant_rerotate"](npk.CB_BF16, npk.CB_KV_U4, 16, 16, 16, 16, 16, 4, 2, 60, 3,
                                    1e4, None) == npk.CB_E_SHAPE
    assert R["cb_dequant_rerotate"](npk.CB_BF16, npk.CB_KV_U8, 24, 16, 16, 16, 16, 4, 2, 64, 3,
                                    1e4, None) == npk.CB_E_SHAPE
    assert R["cb_rmsnorm"](npk.CB_F32, None, npk.CB_F32, None, None, 3, 8, 1e-5,
                           None) == npk.CB_E_INVALID
    assert R["cb_lm_head"](None, 16, 1, 16, 16, 10, 16, None, None) == npk.CB_E_INVALID
    assert R["cb_decode_step"](None, 16, 4, 16, 16, 4, 16, 16, 16, None) == npk.CB_E_INVALID
    # NULL handles are rejected, never dereferenced
    assert R["cb_fetch_kv"](None, 0) == npk.CB_E_INVALID
    assert R["cb_prefill_layer"](None, 0) == npk.CB_E_INVALID
    assert R["cb_synchronize"](None) == npk.CB_E_INVALID
    R["cb_plan_destroy"](None)
    R["cb_model_destroy"](None)


def test_chunk_descriptor_layout(npk, tmp_path):
    """The ctypes mirrors of the request structs have the C layout that a C
    compiler gives the header."""
    import subprocess
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "cacheblend.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu\\n", sizeof(cb_chunk_kv), '
                   'offsetof(cb_chunk_kv, kv_format), offsetof(cb_chunk_kv, qparams), '
                   'sizeof(cb_request), sizeof(cb_batch_request)); return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got == [ctypes.sizeof(npk.cb_chunk_kv), npk.cb_chunk_kv.kv_format.offset,
                   npk.cb_chunk_kv.qparams.offset, ctypes.sizeof(npk.cb_request),
                   ctypes.sizeof(npk.cb_batch_request)]


def test_binding_has_no_fallback():
    """The package refuses to import without the built library."""
    src = open(os.path.join(ROOT, "non_prefix_kv_amd", "__init__.py")).read()
    assert "raise ImportError" in src
    assert "oracle" not in src


# ------------------------------------------------------------ chunk store (host logic)
def test_controller_matches_oracle(npk):
    import numpy as np
    rng = np.random.default_rng(41)
    for _ in range(500):
        tp = float(rng.uniform(1e-4, 2.0))
        tok = float(rng.integers(512, 1 << 18))
        n = int(rng.integers(0, 1 << 17))
        thr = float(rng.uniform(1e8, 1e11))
        rmin = int(rng.integers(0, 10001))
        assert npk.cb_controller_ratio(tp, tok, n, thr, rmin) == \
            oracle.controller_ratio(tp, tok, n, thr, rmin)
    # the worked example of the pages (Llama-7B 4K: 3 ms at 15%, 16 ms load)
    assert npk.cb_controller_ratio(0.02, 16384, 4096, 16384 * 4096 / 0.016, 1500) == 8000


def test_controller_rejects_bad_args(npk):
    R = npk.RAW["cb_controller_ratio"]
    out = ctypes.c_int32()
    assert R(0.0, 1.0, 1, 1.0, 0, ctypes.byref(out)) == npk.CB_E_INVALID
    assert R(1.0, 1.0, -1, 1.0, 0, ctypes.byref(out)) == npk.CB_E_INVALID
    assert R(1.0, 1.0, 1, float("inf"), 0, ctypes.byref(out)) == npk.CB_E_INVALID
    assert R(1.0, 1.0, 1, 1.0, 10001, ctypes.byref(out)) == npk.CB_E_INVALID
    assert R(1.0, 1.0, 1, 1.0, 0, None) == npk.CB_E_INVALID


@pytest.mark.parametrize("seed", range(6))
def test_cache_replay_matches_oracle(npk, seed):
    """The tier's LRU decisions (hits and releases, in order) equal the
    oracle's replay on Zipf-distributed chunk streams of varied sizes and
    budgets."""
    import numpy as np
    rng = np.random.default_rng(seed)
    pool = 60
    p = np.arange(1, pool + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    size = {k: int(rng.integers(1, 40)) * 4096 for k in range(pool)}
    batches = []
    for _ in range(int(rng.integers(1, 30))):
        ids = rng.choice(pool, size=int(rng.integers(0, 12)), p=p)
        batches.append([(int(k) * 7919 + 3, size[int(k)]) for k in ids])
    for cap in (0, 4096, 20 * 4096, 200 * 4096, 10 ** 12):
        got = npk.cb_cache_replay(cap, batches)
        want = oracle.lru_replay(cap, batches)
        assert got == [(h, list(e)) for h, e in want], cap


def test_cache_replay_hand_example(npk):
    b = lambda *ks: [(k, 1) for k in ks]
    assert npk.cb_cache_replay(3, [b(1, 2, 3), b(1, 4), b(2, 3), b(1, 4, 1)]) == \
        [([False] * 3, []), ([True, False], [2]), ([False, True], [1]),
         ([False, True, False], [3])]
    # a batch's own entries are not released for its misses
    assert npk.cb_cache_replay(3, [b(1, 2, 3), b(1, 2, 5, 6), b(6)])[1:] == \
        [([True, True, False, False], [3]), ([False], [1])]


def test_cache_entry_validation(npk):
    R = npk.RAW
    h = ctypes.c_void_p()
    assert R["cb_cache_create"](0, 256, npk.CB_BF16, 1 << 20, ctypes.byref(h)) == npk.CB_E_SHAPE
    assert R["cb_cache_create"](2, 250, npk.CB_BF16, 1 << 20, ctypes.byref(h)) == npk.CB_E_SHAPE
    assert R["cb_cache_create"](2, 256, 7, 1 << 20, ctypes.byref(h)) == npk.CB_E_INVALID
    assert R["cb_cache_create"](2, 256, npk.CB_BF16, -1, ctypes.byref(h)) == npk.CB_E_SHAPE
    assert R["cb_cache_create"](2, 256, npk.CB_BF16, 1, None) == npk.CB_E_INVALID
    assert R["cb_cache_resolve"](None, 0, None, None, None, None, None) == npk.CB_E_INVALID
    assert R["cb_cache_commit"](None, 0, None) == npk.CB_E_INVALID
    assert R["cb_cache_stats"](None, None) == npk.CB_E_INVALID
    assert R["cb_cache_replay"](-1, 0, None, None, None, None, None, None) == npk.CB_E_INVALID
    R["cb_cache_destroy"](None)


def test_binding_rejects_bad_buffers_before_the_call(npk):
    """The binding checks kind, element type and extent of every tensor it
    turns into a raw pointer (the library cannot see sizes behind pointers)
    and raises CBError with the library's codes before anything is called:
    here with a stand-in model whose handle is never used."""
    import types
    import torch
    cfg = npk.cb_model_cfg(2, 64, 4, 2, 16, 128, 1e4, 1e-5, npk.CB_F32)
    model = types.SimpleNamespace(cfg=cfg, handle=None)
    k = torch.zeros((2, 8, 2, 16))
    chunks = [{"k": k, "v": k, "n_tokens": 8, "layer_stride": 8 * 32}]
    x0 = torch.zeros((12, 64))
    fk = torch.zeros((2, 12, 2, 16))
    with pytest.raises(npk.CBError) as e:       # device buffers given as host tensors
        npk.cb_blend(model, chunks, [0], 4, x0, fk, fk)
    assert e.value.status == npk.CB_E_INVALID and "device" in str(e.value)
    with pytest.raises(npk.CBError) as e:       # schedule of the wrong length
        npk.cb_blend(model, [], [], 4, None, None, None, schedule=[0, 0])
    assert e.value.status == npk.CB_E_SCHEDULE
    _need = npk._need
    with pytest.raises(npk.CBError) as e:
        _need(torch.zeros(10), "hidden_out", torch.float32, 11, device=False)
    assert e.value.status == npk.CB_E_SHAPE
    with pytest.raises(npk.CBError) as e:
        _need(torch.zeros(10, dtype=torch.int64), "sel_idx", torch.int32, 10, device=False)
    assert e.value.status == npk.CB_E_INVALID
    with pytest.raises(npk.CBError) as e:
        _need(torch.zeros(4, 4).t(), "x0", torch.float32, 16, device=False)
    assert e.value.status == npk.CB_E_INVALID
    _need(torch.zeros(10), "ok", torch.float32, 10, device=False)
    _need(12345, "address", torch.float32, 10**9)          # raw addresses pass unchecked
