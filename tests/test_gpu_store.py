"""The HBM tier of the chunk store (cb_cache_*) on the GPU: fusions whose
pinned-host chunks are staged into or served from the tier give the same
bits as fusions that stream every chunk from host memory; the tier's hits
and releases follow its LRU policy (checked against the oracle's replay,
which the CPU tests pin); quantized chunks are kept as codes."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import make_batch_case, quantize_case
from tests.gpu_helpers import make_model, run_gpu_batch, pool_inputs, quant_chunk
from workloads import TINY, BATCHED_TINY, make_batched_requests

pytestmark = pytest.mark.gpu


def entry_bytes(c, L, row, es):
    """Device bytes the tier charges for a chunk: K, V (codes or values) and
    parameters, each rounded up to 256 bytes."""
    r256 = lambda x: (x + 255) // 256 * 256
    elems = L * c["n_tokens"] * row
    fmt = c.get("kv_format", 0)
    b = elems * es if fmt == 0 else (elems if fmt == 1 else elems // 2)
    out = 2 * r256(b)
    if fmt:
        out += r256(L * 4 * row * 4)
    return out


def nan_eq(a, b):
    return torch.equal(a.nan_to_num(7.0), b.nan_to_num(7.0))


def batches_over_one_pool(dt):
    pool_lens, reqs = make_batched_requests(BATCHED_TINY, seed=0)
    parts = [reqs[0:3], reqs[3:6], reqs[1:4], reqs[0:6]]
    return [make_batch_case(TINY, pool_lens, p, seed=0, dtype=dt) for p in parts]


def quantize_pool(bc, bits_of):
    """Pinned-host pool descriptors; entries in bits_of become oracle codes."""
    pool = pool_inputs(bc, "bf16", on_host=True)
    for i, bits in bits_of.items():
        if bc.pool[i] is None:
            continue
        from dataclasses import replace
        one = replace(bc.cases[0], chunks=[bc.pool[i]])
        codes, _ = quantize_case(one, bits)
        pool[i] = quant_chunk(codes[0], bits, on_host=True)
    return pool


@pytest.mark.parametrize("cap_entries,quant", [(100, False), (2, False), (3, True), (0, False)])
def test_tier_fusions_bit_identical_and_lru(lib, cap_entries, quant):
    dt = "bf16"
    L, row, es = TINY.n_layers, TINY.kv_dim, 2
    cases = batches_over_one_pool(dt)
    model = make_model(lib, cases[0], dt)
    bits_of = {i: (8 if i % 2 else 4) for i in range(len(cases[0].pool))} if quant else {}
    sizes = None
    tier = None
    replay_batches = []
    for j, bc in enumerate(cases):
        print(f"[tier] cap_entries={cap_entries} quant={quant} batch={j}", flush=True)
        pool = quantize_pool(bc, bits_of)
        used = [i for i, c in enumerate(bc.pool) if c is not None]
        if sizes is None:
            fmt = lambda i: 0 if i not in bits_of else (1 if bits_of[i] == 8 else 2)
            sizes = {i: entry_bytes({"n_tokens": cases[-1].pool[i][0].shape[1],
                                     "kv_format": fmt(i)}, L, row, es)
                     for i, c in enumerate(cases[-1].pool) if c is not None}
            cap = cap_entries * max(sizes.values())
            tier = lib.ChunkCache(L, row, lib.CB_BF16, cap)
        for i in used:
            assert sizes[i] == entry_bytes(pool[i], L, row, es)
        # reference: every chunk streamed from pinned host memory
        _, want = run_gpu_batch(lib, model, bc, dt, pool=pool)
        keys = list(range(len(pool)))
        host_pool = [dict(c) for c in pool]
        for i, c in enumerate(host_pool):
            if i not in used:          # unused entries are never read; not looked up
                c["on_host"] = 0
        resolved, hits = tier.resolve(keys, host_pool)
        _, got = run_gpu_batch(lib, model, bc, dt, pool=resolved)
        tier.commit(keys)
        torch.cuda.synchronize()
        for key in want:
            assert nan_eq(got[key], want[key]), (j, key)
        replay_batches.append([(i, sizes[i]) for i in used])
        expect = lib.cb_cache_replay(cap, replay_batches)[-1]
        assert [hits[i] for i in used] == expect[0], j
        assert expect == (oracle.lru_replay(cap, replay_batches)[-1][0],
                          list(oracle.lru_replay(cap, replay_batches)[-1][1]))
    st = tier.stats()
    assert st["hits"] == sum(sum(h) for h, _ in lib.cb_cache_replay(cap, replay_batches))
    assert st["resident_bytes"] <= cap
    if cap_entries >= 100:
        assert st["evicted"] == 0 and st["hits"] > 0
    if cap_entries == 0:
        assert st["hits"] == 0 and st["admitted"] == 0
    tier.close()


def test_tier_single_request_and_validation(lib):
    """cb_blend (one request) through the tier: a staged miss, then a hit,
    both bit-identical to host streaming; an uncommitted reservation is
    dropped by the next lookup; descriptor checks."""
    from tests.helpers import make_case
    from tests.gpu_helpers import run_gpu_blend, chunk_inputs
    from workloads import WORKLOADS
    dt = "bf16"
    L, row = TINY.n_layers, TINY.kv_dim
    tw = WORKLOADS["tiny"]
    case = make_case(TINY, tw.chunk_lens, tw.n_suffix, seed=3, dtype=dt)
    model = make_model(lib, case, dt)
    sched = oracle.schedule(case.n_chunk_tokens, 1500, "gradual", L)
    host = chunk_inputs(case, dt, on_host=True)
    want = run_gpu_blend(lib, model, case, dt, sched, chunks=host)
    tier = lib.ChunkCache(L, row, lib.CB_BF16, 1 << 30)
    keys = [11, 12, 13]
    for rnd in range(3):
        resolved, hits = tier.resolve(keys, host)
        assert hits == [rnd > 0] * 3
        if rnd == 0:
            assert all(resolved[i].stage_k for i in range(3))
        got = run_gpu_blend(lib, model, case, dt, sched, chunks=resolved)
        tier.commit(keys)
        torch.cuda.synchronize()
        for key in ("fused_k", "fused_v", "sel", "hidden"):
            assert torch.equal(got[key], want[key]), (rnd, key)
    # a reservation that is never committed does not become a hit
    tier2 = lib.ChunkCache(L, row, lib.CB_BF16, 1 << 30)
    tier2.resolve(keys, host)
    _, hits = tier2.resolve(keys, host)
    assert hits == [False] * 3
    # same key, other length: rejected at lookup
    other = [dict(host[0], n_tokens=host[0]["n_tokens"] - 1)]
    with pytest.raises(lib.CBError) as e:
        tier.resolve([11], other)
    assert e.value.status == lib.CB_E_INVALID
    # staging on a device chunk is rejected by the fusion
    dev_chunks = chunk_inputs(case, dt)
    bad = [dict(c) for c in dev_chunks]
    bad[0]["stage_k"] = bad[1]["k"]
    bad[0]["stage_v"] = bad[1]["v"]
    with pytest.raises(lib.CBError) as e:
        run_gpu_blend(lib, model, case, dt, sched, chunks=bad)
    assert e.value.status == lib.CB_E_INVALID
    tier.close()
    tier2.close()
