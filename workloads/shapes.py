"""Model shapes and prompt layouts of the synthetic workloads.

The model shapes are the Llama-2-7B / Llama-2-13B / Yi-34B families that the
CacheBlend explainers evaluate on (abeam CacheBlend page, section on
experiments and results); the prompt layout (independently precomputed chunks
in retrieval order followed by a query suffix) is the RAG input structure of
the 0h-n0 CacheBlend page (section on RAG prefill bottleneck and chunk
boundary handling).  No dataset item is used or recreated: token ids are
uniform random draws.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    rope_base: float = 10000.0
    rms_eps: float = 1e-5
    vocab: int = 32000

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    chunk_lens: Tuple[int, ...]
    n_suffix: int
    r_bp: int = 1500                 # recompute ratio in basis points (15%)
    schedule_kind: str = "gradual"
    kv_on_host: bool = False         # chunk KVs streamed from pinned host memory

    @property
    def n_chunk_tokens(self) -> int:
        return int(sum(self.chunk_lens))

    @property
    def n_tokens(self) -> int:
        return self.n_chunk_tokens + self.n_suffix

    @property
    def offsets(self) -> Tuple[int, ...]:
        out, o = [], 0
        for n in self.chunk_lens:
            out.append(o)
            o += n
        return tuple(out)


TINY = ModelShape(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                  ffn_dim=1024, vocab=1024)
LLAMA7B = ModelShape(n_layers=32, d_model=4096, n_q_heads=32, n_kv_heads=32,
                     head_dim=128, ffn_dim=11008)
LLAMA13B = ModelShape(n_layers=40, d_model=5120, n_q_heads=40, n_kv_heads=40,
                      head_dim=128, ffn_dim=13824)
YI34B = ModelShape(n_layers=60, d_model=7168, n_q_heads=56, n_kv_heads=8,
                   head_dim=128, ffn_dim=20480)

WORKLOADS = {
    # tiny fused prefill: 3 chunks x 128 + 32-token query suffix, fp32 on GPU
    "tiny": Workload("tiny-2L-d256-3x128+32", TINY, (128, 128, 128), 32),
    # Llama-2-7B shape, 4K context, chunk KVs resident in HBM
    "llama7b-4k": Workload("llama2-7b-shape-6x640+256", LLAMA7B, (640,) * 6, 256),
    # Llama-2-13B shape, 8K context
    "llama13b-8k": Workload("llama2-13b-shape-10x768+512", LLAMA13B, (768,) * 10, 512),
    # Yi-34B shape (GQA 56/8), chunk KVs streamed from pinned host memory
    "yi34b-8k": Workload("yi-34b-shape-8x1024+256", YI34B, (1024,) * 8, 256,
                         kv_on_host=True),
}


@dataclass(frozen=True)
class BatchedWorkload:
    name: str
    shape: ModelShape
    n_requests: int = 32
    pool_size: int = 200
    chunk_len_range: Tuple[int, int] = (256, 1024)
    chunks_per_req: Tuple[int, int] = (4, 8)
    suffix_range: Tuple[int, int] = (64, 256)
    zipf_s: float = 1.1
    r_bp: int = 1500
    schedule_kind: str = "gradual"


BATCHED_LLAMA7B = BatchedWorkload("batched-32req-llama2-7b-shape-zipf1.1", LLAMA7B)
# Small batch of the tiny model for parity tests: ragged chunks shared
# between requests, short suffixes.
BATCHED_TINY = BatchedWorkload("batched-6req-tiny", TINY, n_requests=6, pool_size=10,
                               chunk_len_range=(17, 150), chunks_per_req=(1, 4),
                               suffix_range=(1, 40))

BATCHED_WORKLOADS = {"batch-7b": BATCHED_LLAMA7B}
