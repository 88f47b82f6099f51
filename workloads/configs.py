"""The five synthetic decode workloads, as plain data.

Every workload is single-token (decode-step) grouped-query attention over a paged KV cache:
each sequence's keys and values live in fixed-size pages of one shared pool
``[num_pages, page_size, kv_heads, head_dim]`` and are reached through a per-sequence page table.
The shapes follow the Llama/Mistral/Qwen-style decoders that CacheIR targets (CacheIR page,
"Complete Tech Stack": Llama/Mistral/Qwen-style blocks with grouped-query attention) and the
page size of 16 that CacheIR's benchmark JSON reports (CacheIR page, "Benchmarks").  Prefix
sharing — many sequences whose page tables name the same physical pages — is the serving shape
TorchInferno describes as shared prefix-page reuse (TorchInferno page, "Design Coverage").

This module holds sizes and distributions only; it computes nothing of the attention itself.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

DTYPES = ("f32", "bf16", "f16")
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2}


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One decode-step workload.

    ``lengths`` selects how per-sequence context lengths are drawn:
      * ``("fixed", L)``            every sequence has L tokens;
      * ``("uniform", lo, hi)``     integers uniform in [lo, hi], inclusive;
      * ``("loguniform", lo, hi)``  round(exp(U(ln lo, ln hi))) clipped to [lo, hi];
      * ``("prefix", P, lo, hi)``   a P-token prefix shared by every sequence (same physical
                                    pages) plus a private suffix uniform in [lo, hi].
    With ``append`` the drawn length is the pre-append length L: one new token is written at
    position L and attention then covers L + 1 tokens.
    """

    name: str
    index: int                      # 1..5; also the default seed
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    lengths: Tuple
    pool_pages: Optional[int] = None   # explicit pool size; default ceil(1.1 * pages in use)
    append: bool = False
    partition_tokens: Optional[int] = None   # split-KV partition size, when the workload uses one
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def max_context(self) -> int:
        """Largest context (tokens attended) any draw can produce."""
        kind = self.lengths[0]
        if kind == "fixed":
            hi = self.lengths[1]
        elif kind in ("uniform", "loguniform"):
            hi = self.lengths[2]
        elif kind == "prefix":
            hi = self.lengths[1] + self.lengths[3]
        else:
            raise ValueError(kind)
        return hi + (1 if self.append else 0)

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.max_context // self.page_size)

    def scaled(self, batch: Optional[int] = None, lengths: Optional[Tuple] = None,
               name_suffix: str = "small") -> "DecodeConfig":
        """The same heads, dtype, page size and structure at a smaller batch / context."""
        return dataclasses.replace(
            self,
            name=f"{self.name}-{name_suffix}",
            batch=self.batch if batch is None else batch,
            lengths=self.lengths if lengths is None else lengths,
            pool_pages=None if lengths is not None or batch is not None else self.pool_pages,
        )


CONFIGS = {
    1: DecodeConfig(
        name="tiny-fp32", index=1, batch=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
        page_size=16, dtype="f32", lengths=("fixed", 128), pool_pages=32,
        description="tiny paged decode, fp32; 8 pages drawn from a permuted 32-page pool"),
    2: DecodeConfig(
        name="llama3-8b-bf16-b64", index=2, batch=64, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=16, dtype="bf16", lengths=("uniform", 512, 4096),
        partition_tokens=512,
        description="Llama-3-8B-shaped decode step, bf16, contexts uniform in [512, 4096]"),
    3: DecodeConfig(
        name="prefix-shared-fp16-b128", index=3, batch=128, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=16, dtype="f16", lengths=("prefix", 2048, 64, 512),
        description="128 sequences sharing one 2048-token prefix plus private suffixes, fp16"),
    4: DecodeConfig(
        name="qwen2-7b-gqa7-bf16-append", index=4, batch=32, num_q_heads=28, num_kv_heads=4,
        head_dim=128, page_size=32, dtype="bf16", lengths=("loguniform", 128, 8192),
        append=True,
        description="Qwen2-7B-shaped high-GQA decode with a one-token paged KV append, bf16"),
    5: DecodeConfig(
        name="long-context-splitkv-bf16-b8", index=5, batch=8, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=16, dtype="bf16", lengths=("uniform", 32768, 131072),
        partition_tokens=4096,
        description="long-context split-KV decode, partitions of 4096 tokens, bf16"),
}


def config(index_or_name) -> DecodeConfig:
    if isinstance(index_or_name, int):
        return CONFIGS[index_or_name]
    for c in CONFIGS.values():
        if c.name == index_or_name:
            return c
    raise KeyError(index_or_name)


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim); callers round it to float32 before use."""
    return 1.0 / math.sqrt(head_dim)
