"""Seeded draws for the synthetic workloads (numpy PCG64, fixed draw order).

Every tensor gets its own PCG64 stream keyed by (seed, layer, tensor id), so a
test that needs only layer 3 draws exactly what a full-model run draws for
layer 3.  Weights are i.i.d. N(0, 0.02^2); RMSNorm gains are 1; token ids are
uniform over the vocabulary; the embedding rows of the prompt are the layer-0
input.
"""
import numpy as np

from .shapes import ModelShape, BatchedWorkload

WEIGHT_STD = 0.02
_TENSOR_IDS = {"embed": 0, "wq": 1, "wk": 2, "wv": 3, "wo": 4,
               "w_gate": 5, "w_up": 6, "w_down": 7, "tokens": 8,
               "batch_tokens": 9}


def _rng(seed: int, layer: int, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(layer) + 1,
                                                _TENSOR_IDS[tensor]]))


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round an array to the storage dtype ('f64', 'f32' or 'bf16', RNE) and
    return it widened to float64, so both sides start from identical values."""
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        # float32, then round to nearest even at bit 16 of the pattern
        # (finite inputs): the conversion torch and the GPU use for bf16
        f = np.array(a, dtype=np.float32, order="C")
        u = f.view(np.uint32)
        bias = u >> np.uint32(16)
        bias &= np.uint32(1)
        bias += np.uint32(0x7FFF)
        u += bias
        u &= np.uint32(0xFFFF0000)
        return f.astype(np.float64)
    raise ValueError(dtype)


def _normal(seed, layer, name, shape):
    return _rng(seed, layer, name).standard_normal(shape, dtype=np.float64) * WEIGHT_STD


def make_weights_np(shape: ModelShape, seed: int = 0, layers=None, dtype: str = "f64"):
    """Per-layer weight dicts, row-major [out][in], rounded to `dtype`.

    `layers` selects which layer indices to draw (default: all); entries for
    other layers are None, so indices keep their meaning.
    """
    sel = range(shape.n_layers) if layers is None else layers
    out = [None] * shape.n_layers
    d, qd, kvd, f = shape.d_model, shape.q_dim, shape.kv_dim, shape.ffn_dim
    for l in sel:
        out[l] = {
            "attn_norm": np.ones(d),
            "wq": round_to(_normal(seed, l, "wq", (qd, d)), dtype),
            "wk": round_to(_normal(seed, l, "wk", (kvd, d)), dtype),
            "wv": round_to(_normal(seed, l, "wv", (kvd, d)), dtype),
            "wo": round_to(_normal(seed, l, "wo", (d, qd)), dtype),
            "mlp_norm": np.ones(d),
            "w_gate": round_to(_normal(seed, l, "w_gate", (f, d)), dtype),
            "w_up": round_to(_normal(seed, l, "w_up", (f, d)), dtype),
            "w_down": round_to(_normal(seed, l, "w_down", (d, f)), dtype),
        }
    return out


def make_embedding_np(shape: ModelShape, seed: int = 0, dtype: str = "f64"):
    return round_to(_normal(seed, -1, "embed", (shape.vocab, shape.d_model)), dtype)


def make_tokens(shape: ModelShape, n_tokens: int, seed: int = 0) -> np.ndarray:
    return _rng(seed, -1, "tokens").integers(0, shape.vocab, size=n_tokens, dtype=np.int64)


def make_batched_requests(w: BatchedWorkload, seed: int = 0):
    """Batched serving slice: a pool of chunks with U{lo..hi} lengths, then per
    request n ~ U{4..8} distinct chunk ids from a truncated Zipf(s) over ranks
    1..pool (p proportional to k^-s) and a U{64..256} suffix.  Draw order: pool
    lengths, then per request (n, ids, suffix)."""
    g = np.random.Generator(np.random.PCG64([int(seed), 0, 99]))
    lo, hi = w.chunk_len_range
    pool_lens = g.integers(lo, hi + 1, size=w.pool_size)
    ranks = np.arange(1, w.pool_size + 1, dtype=np.float64)
    p = ranks ** (-w.zipf_s)
    p /= p.sum()
    reqs = []
    for _ in range(w.n_requests):
        n = int(g.integers(w.chunks_per_req[0], w.chunks_per_req[1] + 1))
        ids = g.choice(w.pool_size, size=n, replace=False, p=p)
        suffix = int(g.integers(w.suffix_range[0], w.suffix_range[1] + 1))
        reqs.append({"chunk_ids": [int(i) for i in ids], "n_suffix": suffix})
    return pool_lens.astype(np.int64), reqs


def make_request_stream(w: BatchedWorkload, seed: int = 0, n_batches: int = 1):
    """A stream of batches over one chunk pool: batch 0 is
    make_batched_requests(w, seed); batch j > 0 draws its requests the same
    way from its own generator (the pool lengths are batch 0's)."""
    pool_lens, first = make_batched_requests(w, seed)
    ranks = np.arange(1, w.pool_size + 1, dtype=np.float64)
    p = ranks ** (-w.zipf_s)
    p /= p.sum()
    batches = [first]
    for j in range(1, n_batches):
        g = np.random.Generator(np.random.PCG64([int(seed), int(j), 98]))
        reqs = []
        for _ in range(w.n_requests):
            n = int(g.integers(w.chunks_per_req[0], w.chunks_per_req[1] + 1))
            ids = g.choice(w.pool_size, size=n, replace=False, p=p)
            suffix = int(g.integers(w.suffix_range[0], w.suffix_range[1] + 1))
            reqs.append({"chunk_ids": [int(i) for i in ids], "n_suffix": suffix})
        batches.append(reqs)
    return pool_lens, batches


def make_batch_tokens(shape: ModelShape, pool_lens, reqs, seed: int = 0):
    """Token ids of every pool chunk and of every request's suffix (seeded;
    a chunk has the same tokens wherever it is used)."""
    g = _rng(seed, -1, "batch_tokens")
    pool_tokens = [g.integers(0, shape.vocab, size=int(n), dtype=np.int64) for n in pool_lens]
    suffix_tokens = [g.integers(0, shape.vocab, size=int(r["n_suffix"]), dtype=np.int64)
                     for r in reqs]
    return pool_tokens, suffix_tokens


def make_chunk_caches_np(shape: ModelShape, chunk_lens, seed: int = 0, dtype: str = "f64",
                         std: float = 1.0):
    """Seeded stand-in chunk caches: K and V [L][n_c][H_kv][d_head] drawn
    i.i.d. N(0, std^2) per chunk and rounded to `dtype`.  The fusion takes
    any cached values, so parity checks at full model width can skip the
    per-chunk precompute; std = 1 is the scale of a projected row of the
    N(0, 0.02^2) weights at these widths."""
    out = []
    for c, n in enumerate(chunk_lens):
        g = np.random.Generator(np.random.PCG64([int(seed), int(c), 97]))
        shp = (shape.n_layers, int(n), shape.n_kv_heads, shape.head_dim)
        k = round_to(g.standard_normal(shp, dtype=np.float64) * std, dtype)
        v = round_to(g.standard_normal(shp, dtype=np.float64) * std, dtype)
        out.append((k, v))
    return out
