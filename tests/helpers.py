"""Shared test fixtures: build a synthetic fused-prompt case and its oracle
results.  Inputs come from `workloads` (seeded draws); precomputed chunk KVs
come from the oracle's own prefill, so no oracle input is ever produced by the
HIP library."""
import dataclasses

import numpy as np

import oracle
from workloads import (make_weights_np, make_embedding_np, make_tokens, round_to,
                       ModelShape, make_chunk_caches_np)


@dataclasses.dataclass
class Case:
    shape: ModelShape
    weights: list
    x0: np.ndarray            # [N][d] float64 (already rounded to the run dtype)
    chunks: list              # [(K [L][n_c][Hkv][dh], V)] float64, rounded
    offsets: list
    n_suffix: int
    dtype: str

    @property
    def n_chunk_tokens(self):
        return int(sum(k.shape[1] for k, _ in self.chunks))

    @property
    def n_tokens(self):
        return self.n_chunk_tokens + self.n_suffix


def make_case(shape, chunk_lens, n_suffix, seed=0, dtype="f64", n_layers=None,
              precompute_dtype=np.float64, random_caches=False):
    """Weights/x0 drawn from the seeded generators and rounded to `dtype`;
    chunk KVs precomputed by the oracle alone at chunk-local positions and
    rounded to `dtype` as a stored cache would be (`precompute_dtype` only
    sets the arithmetic of that precompute, e.g. float32 at full width), or,
    with random_caches, seeded N(0, 1) stand-ins (full-width parity cases,
    where the precompute would dominate the test's CPU time)."""
    L = shape.n_layers if n_layers is None else n_layers
    if L != shape.n_layers:
        shape = dataclasses.replace(shape, n_layers=L)
    w = make_weights_np(shape, seed=seed, dtype=dtype)
    emb = make_embedding_np(shape, seed=seed, dtype=dtype)
    n = int(sum(chunk_lens)) + n_suffix
    x0 = emb[make_tokens(shape, n, seed=seed)]
    chunks, offsets, o = [], [], 0
    stand_ins = make_chunk_caches_np(shape, chunk_lens, seed, dtype) if random_caches else None
    for c, nc in enumerate(chunk_lens):
        if stand_ins is not None:
            chunks.append(stand_ins[c])
        else:
            k, v, _ = oracle.prefill(w, shape, x0[o:o + nc], pos0=0, dtype=precompute_dtype)
            chunks.append((round_to(k, dtype), round_to(v, dtype)))
        offsets.append(o)
        o += nc
    return Case(shape, w, x0, chunks, offsets, n_suffix, dtype)


def run_blend(case, sched, dev_mode="KV"):
    return oracle.blend(case.weights, case.shape, case.x0, case.chunks, case.offsets,
                        case.n_suffix, sched, dev_mode=dev_mode)


def run_full(case):
    return oracle.prefill(case.weights, case.shape, case.x0, pos0=0)


def rel_err(got, ref):
    """Normwise max relative error: max|g - o| / max|o|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


@dataclasses.dataclass
class BatchCase:
    shape: ModelShape
    weights: list
    pool: list                # [(K [L][n][Hkv][dh], V)] float64, rounded; None if unused
    requests: list            # [{"chunk_ids": [...], "n_suffix": int}]
    cases: list               # per request: Case over its own chunks (oracle input)
    x0: np.ndarray            # stacked [sum N][d]
    dtype: str


def make_batch_case(shape, pool_lens, requests, seed=0, dtype="f64", n_layers=None,
                    precompute_dtype=np.float64):
    """A batch over a chunk pool: each used pool chunk is precomputed once by
    the oracle at chunk-local positions from its own tokens; request b's
    prompt is its chunks' tokens in order then its suffix tokens."""
    from workloads import make_batch_tokens
    L = shape.n_layers if n_layers is None else n_layers
    if L != shape.n_layers:
        shape = dataclasses.replace(shape, n_layers=L)
    w = make_weights_np(shape, seed=seed, dtype=dtype)
    emb = make_embedding_np(shape, seed=seed, dtype=dtype)
    pool_tok, suf_tok = make_batch_tokens(shape, pool_lens, requests, seed=seed)
    used = sorted({i for r in requests for i in r["chunk_ids"]})
    pool = [None] * len(pool_lens)
    for i in used:
        k, v, _ = oracle.prefill(w, shape, emb[pool_tok[i]], pos0=0, dtype=precompute_dtype)
        pool[i] = (round_to(k, dtype), round_to(v, dtype))
    cases, xs = [], []
    for r, st in zip(requests, suf_tok):
        toks = np.concatenate([pool_tok[i] for i in r["chunk_ids"]] + [st]).astype(np.int64)
        x0 = emb[toks]
        offsets = list(np.cumsum([0] + [len(pool_tok[i]) for i in r["chunk_ids"]])[:-1])
        cases.append(Case(shape, w, x0, [pool[i] for i in r["chunk_ids"]],
                          [int(o) for o in offsets], int(r["n_suffix"]), dtype))
        xs.append(x0)
    return BatchCase(shape, w, pool, requests, cases, np.concatenate(xs, axis=0), dtype)


def quantize_case(case, bits):
    """The case's chunk caches stored as per-channel codes by the oracle's
    encoder.  Returns (codes, decoded case): codes per chunk as (K codes
    [L][n][C*bits/8] uint8, V codes, qparams [L][4][C] float32 = k scale,
    k zero, v scale, v zero), and a Case whose chunks are the oracle's
    decoded values (the oracle's input for the same fusion)."""
    s = case.shape
    codes, decoded = [], []
    for k, v in case.chunks:
        kc, ks, kz = oracle.quantize_channels(k, bits)
        vc, vs, vz = oracle.quantize_channels(v, bits)
        qp = np.stack([ks, kz, vs, vz], axis=1).astype(np.float32)
        codes.append((oracle.pack_codes(kc, bits), oracle.pack_codes(vc, bits), qp))
        decoded.append((oracle.dequantize_channels(kc, ks, kz, s.n_kv_heads, s.head_dim),
                        oracle.dequantize_channels(vc, vs, vz, s.n_kv_heads, s.head_dim)))
    return codes, dataclasses.replace(case, chunks=decoded)
