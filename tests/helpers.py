"""Shared test fixtures: build a synthetic fused-prompt case and its oracle
results.  Inputs come from `workloads` (seeded draws); precomputed chunk KVs
come from the oracle's own prefill, so no oracle input is ever produced by the
HIP library."""
import dataclasses

import numpy as np

import oracle
from workloads import (make_weights_np, make_embedding_np, make_tokens, round_to,
                       ModelShape)


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
              precompute_dtype=np.float64):
    """Weights/x0 drawn from the seeded generators and rounded to `dtype`;
    chunk KVs precomputed by the oracle alone at chunk-local positions and
    rounded to `dtype` as a stored cache would be (`precompute_dtype` only
    sets the arithmetic of that precompute, e.g. float32 at full width)."""
    L = shape.n_layers if n_layers is None else n_layers
    if L != shape.n_layers:
        shape = dataclasses.replace(shape, n_layers=L)
    w = make_weights_np(shape, seed=seed, dtype=dtype)
    emb = make_embedding_np(shape, seed=seed, dtype=dtype)
    n = int(sum(chunk_lens)) + n_suffix
    x0 = emb[make_tokens(shape, n, seed=seed)]
    chunks, offsets, o = [], [], 0
    for nc in chunk_lens:
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
