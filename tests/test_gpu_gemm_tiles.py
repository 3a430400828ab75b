"""Projection tiles at full model width.

The GEMM launcher picks among three tile shapes (128x128, 224x192, 256x256)
by the number of rows and output columns.  The blend at r = 15% runs its
projections on ~832-947 rows, where the 224x192 tile takes the q/k/v and
gate/up products (Llama-2-7B shape) and the q/k/v, O and down products
(Llama-2-13B shape).  One-layer prefills at those row counts exercise each
epilogue on that tile (RoPE at real positions on q/k/v tiles that straddle
the q|k and k|v boundaries, SiLU(gate)*up on interleaved gate/up rows, the
gathered residual) against the oracle's prefill; at 947 rows the gate/up
product runs split, 896 rows on 224x192 tiles and 51 on 128x128.  A one-KV-head shape at
4000 rows puts q, k and v in one 224x192 tile column range.  A 16640-row
prefill runs every epilogue on the 4-stage 256x256 kernel of long launches."""
import dataclasses
import gc
import types

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import rel_err
from tests.gpu_helpers import dev, host, make_model
from workloads import WORKLOADS, ModelShape, make_weights_np, make_embedding_np, make_tokens

pytestmark = pytest.mark.gpu


# One KV head of 128 dims: the 224x192 q/k/v tiles 10 and 11 span q|k and
# k|v (the k block is 128 rows), at 4000 rows where that tile is chosen.
GQA_1KV = ModelShape(n_layers=1, d_model=2048, n_q_heads=16, n_kv_heads=1, head_dim=128,
                     ffn_dim=5504, vocab=1024)


@pytest.mark.parametrize("name,rows,pos0", [("llama7b-4k", 832, 0), ("llama7b-4k", 889, 1000),
                                            ("llama7b-4k", 947, 300),
                                            ("llama13b-8k", 1664, 77), ("gqa-1kv", 4000, 5)])
def test_prefill_projection_tiles_vs_oracle(lib, name, rows, pos0):
    base = GQA_1KV if name == "gqa-1kv" else WORKLOADS[name].shape
    shape = dataclasses.replace(base, n_layers=1)
    w = make_weights_np(shape, seed=3, dtype="bf16")
    x = make_embedding_np(shape, seed=3, dtype="bf16")[make_tokens(shape, rows, seed=3)]
    model = make_model(lib, types.SimpleNamespace(shape=shape, weights=w), "bf16")
    k = torch.empty((1, rows, shape.n_kv_heads, shape.head_dim), dtype=torch.bfloat16,
                    device="cuda")
    v = torch.empty_like(k)
    hid = torch.empty((rows, shape.d_model), device="cuda")
    lib.cb_prefill(model, dev(x, "bf16"), rows, pos0, k, v, hid)
    torch.cuda.synchronize()
    rk, rv, outs = oracle.prefill(w, shape, x, pos0=pos0, dtype=np.float32)
    assert rel_err(host(k), rk) < 2e-2
    assert rel_err(host(v), rv) < 2e-2
    assert rel_err(host(hid), outs[-1]) < 2e-2
    model.close()
    del model, k, v, hid
    gc.collect()
    torch.cuda.empty_cache()


def test_long_prefill_four_stage_tiles(lib):
    """Products of more than four rounds of 256x256 tiles take the 4-stage
    kernel (gemm_big4_kernel): a one-layer prefill of 16640 rows at the
    Llama-2-7B width runs its q/k/v + RoPE (65 x 48 tiles), O + residual and
    down + residual (65 x 16) and gate/up + SwiGLU (65 x 86) products there.
    Causality fixes the first 4096 rows to those of the 4096-row prefill of
    the same tokens, whose products run the 5-stage kernel (one to three
    rounds): same per-element accumulation order, so bit-identical.  The
    4096-row prefill is compared with the oracle's."""
    shape = dataclasses.replace(WORKLOADS["llama7b-4k"].shape, n_layers=1)
    w = make_weights_np(shape, seed=4, dtype="bf16")
    long_rows, short_rows = 16640, 4096
    x = make_embedding_np(shape, seed=4, dtype="bf16")[make_tokens(shape, long_rows, seed=4)]
    model = make_model(lib, types.SimpleNamespace(shape=shape, weights=w), "bf16")
    out = {}
    for rows in (long_rows, short_rows):
        k = torch.empty((1, rows, shape.n_kv_heads, shape.head_dim), dtype=torch.bfloat16,
                        device="cuda")
        v = torch.empty_like(k)
        hid = torch.empty((rows, shape.d_model), device="cuda")
        lib.cb_prefill(model, dev(x[:rows], "bf16"), rows, 0, k, v, hid)
        torch.cuda.synchronize()
        out[rows] = (k, v, hid)
    kl, vl, hl = out[long_rows]
    ks, vs, hs = out[short_rows]
    assert torch.equal(kl[:, :short_rows], ks) and torch.equal(vl[:, :short_rows], vs)
    assert torch.equal(hl[:short_rows], hs)
    rk, rv, outs = oracle.prefill(w, shape, x[:short_rows], pos0=0, dtype=np.float32)
    assert rel_err(host(ks), rk) < 2e-2
    assert rel_err(host(vs), rv) < 2e-2
    assert rel_err(host(hs), outs[-1]) < 2e-2
    model.close()
    del model, out, kl, vl, hl, ks, vs, hs
    gc.collect()
    torch.cuda.empty_cache()
