"""Seeded synthetic inputs shared by the CPU oracle tests, the GPU tests and bench.py.

This package holds shapes, random draws and dtype rounding only: none of the
fusion method's arithmetic lives here, so the oracle and the HIP path can both
take their inputs from it without sharing any computation.
"""
from .shapes import (ModelShape, Workload, TINY, LLAMA7B, LLAMA13B, YI34B,
                     WORKLOADS, BatchedWorkload, BATCHED_LLAMA7B, BATCHED_TINY,
                     BATCHED_WORKLOADS)
from .gen import (make_weights_np, make_tokens, make_embedding_np, round_to,
                  make_batched_requests, make_batch_tokens, make_request_stream,
                  make_chunk_caches_np)

__all__ = [
    "ModelShape", "Workload", "TINY", "LLAMA7B", "LLAMA13B", "YI34B", "WORKLOADS",
    "BatchedWorkload", "BATCHED_LLAMA7B", "BATCHED_TINY", "BATCHED_WORKLOADS",
    "make_weights_np", "make_tokens", "make_embedding_np", "round_to",
    "make_batched_requests", "make_batch_tokens", "make_request_stream",
    "make_chunk_caches_np",
]
