"""Seeded synthetic inputs for paged decode attention.

The same arrays feed both the HIP library and the CPU oracle; nothing here computes any part of
attention.  Values are drawn as float32 standard normals and rounded once to the storage dtype
(round-to-nearest-even); those stored bits *are* the input for every consumer.

Random streams.  Every quantity has its own stream, so that changing the size of one does not
move the others, and large pools are filled in fixed chunks so the bits do not depend on the
thread count.  Stream ``k``, chunk ``c`` of seed ``s`` is ``PCG64(SeedSequence(s, spawn_key=(k, c)))``:

    k = 0 context lengths     k = 1 physical page permutation     k = 2 q
    k = 3 K pool              k = 4 V pool                        k = 5 new K rows (append)
    k = 6 new V rows (append)

Storage: ``f32`` -> ``numpy.float32``; ``f16`` -> ``numpy.float16``; ``bf16`` -> raw ``numpy.uint16``
bit patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

from .configs import DecodeConfig, default_scale

CHUNK = 1 << 22
STREAM_LENGTHS, STREAM_PERM, STREAM_Q, STREAM_K, STREAM_V, STREAM_KNEW, STREAM_VNEW = range(7)

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
NAN_BITS = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}


def _rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, chunk))))


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage dtype, round-to-nearest-even.  ``x`` may be overwritten."""
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    # bf16: add 0x7FFF plus the lowest kept bit, then drop the low half (finite inputs only).
    u = x.view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def _threads(threads: Optional[int]) -> int:
    if threads is not None:
        return max(1, threads)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill_normal(shape: Sequence[int], dtype: str, seed: int, stream: int,
                threads: Optional[int] = None) -> np.ndarray:
    """N(0,1) values rounded to ``dtype``, in fixed chunks of 2**22 elements."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=STORAGE[dtype])
    nchunks = -(-n // CHUNK)

    def work(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        x = _rng(seed, stream, c).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = _encode(x, dtype)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def draw_lengths(cfg: DecodeConfig, seed: int) -> np.ndarray:
    """Per-sequence *drawn* lengths (pre-append for append workloads), int64 [B]."""
    rng = _rng(seed, STREAM_LENGTHS)
    kind = cfg.lengths[0]
    B = cfg.batch
    if kind == "fixed":
        return np.full(B, cfg.lengths[1], dtype=np.int64)
    if kind == "uniform":
        lo, hi = cfg.lengths[1:3]
        return rng.integers(lo, hi + 1, size=B, dtype=np.int64)
    if kind == "loguniform":
        lo, hi = cfg.lengths[1:3]
        x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=B))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    if kind == "prefix":
        prefix, lo, hi = cfg.lengths[1:4]
        return prefix + rng.integers(lo, hi + 1, size=B, dtype=np.int64)
    raise ValueError(kind)


@dataclasses.dataclass
class Workload:
    """Inputs of one decode step.

    ``context_lens`` are the lengths attention covers.  For append workloads ``append_lens`` holds
    the pre-append lengths (the append call's argument; the new row lands at that position) and
    ``context_lens == append_lens + 1``.
    """

    cfg: DecodeConfig
    seed: int
    q: np.ndarray                 # [B, Hq, D]
    k_pool: np.ndarray            # [NP, PS, Hkv, D]
    v_pool: np.ndarray            # [NP, PS, Hkv, D]
    page_table: np.ndarray        # int32 [B, MP]
    context_lens: np.ndarray      # int32 [B]
    scale: np.float32
    append_lens: Optional[np.ndarray] = None   # int32 [B]
    k_new: Optional[np.ndarray] = None         # [B, Hkv, D]
    v_new: Optional[np.ndarray] = None         # [B, Hkv, D]
    shared_pages: int = 0                      # leading page-table entries shared by all rows

    @property
    def dtype(self) -> str:
        return self.cfg.dtype

    @property
    def shape(self) -> dict:
        B, Hq, D = self.q.shape
        NP, PS, Hkv, _ = self.k_pool.shape
        return dict(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=PS,
                    num_pages=NP, max_pages_per_seq=self.page_table.shape[1], dtype=self.dtype)

    def kv_bytes_per_token(self) -> int:
        _, _, Hkv, D = self.k_pool.shape
        return 2 * Hkv * D * self.cfg.elem_bytes

    def logical_tokens(self) -> int:
        return int(np.maximum(self.context_lens, 0).sum())

    def unique_tokens(self) -> int:
        """Tokens whose K/V rows are distinct physical slots (shared prefix counted once)."""
        L = np.maximum(self.context_lens.astype(np.int64), 0)
        if self.shared_pages == 0:
            return int(L.sum())
        shared_tok = self.shared_pages * self.cfg.page_size
        live = L > 0
        return int(np.minimum(L, shared_tok).max(initial=0) + (L[live] - shared_tok).clip(0).sum())


def make_workload(cfg: DecodeConfig, seed: Optional[int] = None, *, poison: bool = False,
                  pad_rows: Sequence[int] = (), threads: Optional[int] = None) -> Workload:
    """Build the inputs of ``cfg`` from ``seed`` (default: the config index).

    ``poison`` fills every pool page that no sequence uses, and every slot at or past a sequence's
    context length in its last page, with NaN, and sets unused page-table entries to -1.
    ``pad_rows`` become padding rows: context length 0 (append length -1), no pages, table all -1.
    """
    seed = cfg.index if seed is None else seed
    B, Hq, Hkv, D, PS = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    assert Hq % Hkv == 0

    drawn = draw_lengths(cfg, seed)
    pad = np.zeros(B, dtype=bool)
    pad[list(pad_rows)] = True
    extra = 1 if cfg.append else 0
    attn = np.where(pad, 0, drawn + extra)

    # Pages per row; with a shared prefix the first `shared` pages are common to every row.
    shared = 0
    if cfg.lengths[0] == "prefix":
        assert cfg.lengths[1] % PS == 0
        shared = cfg.lengths[1] // PS
    npages = -(-attn // PS)
    private = np.where(pad, 0, npages - shared) if shared else npages
    total = shared + int(private.sum())
    pool = cfg.pool_pages if cfg.pool_pages is not None else int(math.ceil(1.1 * total))
    assert pool >= total, (pool, total)
    perm = _rng(seed, STREAM_PERM).permutation(pool).astype(np.int32)

    MP = cfg.max_pages_per_seq
    table = np.full((B, MP), -1 if poison else 0, dtype=np.int32)
    cursor = shared
    for b in range(B):
        if pad[b]:
            table[b, :] = -1
            continue
        n = int(npages[b])
        row = np.empty(n, dtype=np.int32)
        row[:shared] = perm[:shared]
        k = n - shared
        row[shared:] = perm[cursor:cursor + k]
        cursor += k
        table[b, :n] = row
        if not poison and n < MP:
            table[b, n:] = row[-1]   # harmless in-range filler, never read

    q = fill_normal((B, Hq, D), cfg.dtype, seed, STREAM_Q, threads)
    k_pool = fill_normal((pool, PS, Hkv, D), cfg.dtype, seed, STREAM_K, threads)
    v_pool = fill_normal((pool, PS, Hkv, D), cfg.dtype, seed, STREAM_V, threads)
    k_new = v_new = append_lens = None
    if cfg.append:
        k_new = fill_normal((B, Hkv, D), cfg.dtype, seed, STREAM_KNEW, threads)
        v_new = fill_normal((B, Hkv, D), cfg.dtype, seed, STREAM_VNEW, threads)
        append_lens = np.where(pad, -1, drawn).astype(np.int32)

    if poison:
        nan = NAN_BITS[cfg.dtype]
        used = np.zeros(pool, dtype=bool)
        used[perm[:total]] = True
        k_pool[~used] = nan
        v_pool[~used] = nan
        for b in range(B):
            L = int(attn[b])
            if L == 0 or L % PS == 0:
                continue
            last = table[b, (L - 1) // PS]
            k_pool[last, L % PS:] = nan
            v_pool[last, L % PS:] = nan

    return Workload(cfg=cfg, seed=seed, q=q, k_pool=k_pool, v_pool=v_pool, page_table=table,
                    context_lens=attn.astype(np.int32), scale=np.float32(default_scale(D)),
                    append_lens=append_lens, k_new=k_new, v_new=v_new, shared_pages=shared)


# ----------------------------------------------------------------------------------------------
# Input transformations used by invariance checks.  They move bits; they compute nothing.
# ----------------------------------------------------------------------------------------------

def relabel_pages(w: Workload, seed: int) -> Workload:
    """Same logical content under a fresh random physical page numbering."""
    NP = w.k_pool.shape[0]
    new_of_old = np.random.Generator(np.random.PCG64(seed)).permutation(NP).astype(np.int32)
    k_pool = np.empty_like(w.k_pool)
    v_pool = np.empty_like(w.v_pool)
    k_pool[new_of_old] = w.k_pool
    v_pool[new_of_old] = w.v_pool
    table = np.where(w.page_table >= 0, new_of_old[np.clip(w.page_table, 0, NP - 1)], w.page_table)
    return dataclasses.replace(w, k_pool=k_pool, v_pool=v_pool, page_table=table.astype(np.int32))


def unshare_prefix(w: Workload) -> Workload:
    """Give every live row a private copy of the shared prefix pages (new pages appended)."""
    S = w.shared_pages
    assert S > 0
    live = [b for b in range(w.q.shape[0]) if w.context_lens[b] > 0]
    NP = w.k_pool.shape[0]
    extra = S * len(live)
    k_pool = np.concatenate([w.k_pool, np.empty((extra,) + w.k_pool.shape[1:], w.k_pool.dtype)])
    v_pool = np.concatenate([w.v_pool, np.empty((extra,) + w.v_pool.shape[1:], w.v_pool.dtype)])
    table = w.page_table.copy()
    nxt = NP
    for b in live:
        src = w.page_table[b, :S]
        k_pool[nxt:nxt + S] = w.k_pool[src]
        v_pool[nxt:nxt + S] = w.v_pool[src]
        table[b, :S] = np.arange(nxt, nxt + S, dtype=np.int32)
        nxt += S
    return dataclasses.replace(w, k_pool=k_pool, v_pool=v_pool, page_table=table, shared_pages=0)


def subset_rows(w: Workload, rows: Sequence[int]) -> Workload:
    """The same pool with only ``rows`` of the batch (for batch-independence checks)."""
    rows = list(rows)
    cfg = dataclasses.replace(w.cfg, batch=len(rows))
    return dataclasses.replace(
        w, cfg=cfg, q=w.q[rows].copy(), page_table=w.page_table[rows].copy(),
        context_lens=w.context_lens[rows].copy(),
        append_lens=None if w.append_lens is None else w.append_lens[rows].copy(),
        k_new=None if w.k_new is None else w.k_new[rows].copy(),
        v_new=None if w.v_new is None else w.v_new[rows].copy())


def rope_tables(positions: int, head_dim: int, base: float = 10000.0):
    """A rotary cache as a model holds it: float32 ``cos``, ``sin`` of shape
    ``[positions, head_dim / 2]`` with angle ``p * base ** (-2 i / head_dim)`` for row p, pair i,
    evaluated in float64 and rounded once to float32.  It is an input of the rotary step (the
    step applies it); nothing here rotates anything."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / head_dim)
    ang = np.arange(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
