"""Plain float64 CPU oracle for paged decode attention, the paged KV append and the split-KV merge.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's CPU-baseline leg
may import this module; the library never does, and nothing here is shared with the HIP code.

What is computed, and where the pages state it:

* A sequence's keys and values are materialised by walking its page table: logical token ``t``
  lives in physical page ``page_table[b, t // page_size]`` at slot ``t % page_size`` of a pool laid
  out ``[num_pages, page_size, kv_heads, head_dim]`` (TorchInferno page, "Runtime Scaffolds":
  ``runtime.paged`` allocates page-table-shaped KV storage and materialises it; CacheIR page,
  "Current Capabilities": paged KV cache metadata over shared page-backed pools).
* Decode attention for the one new query token of each sequence is the textbook
  ``softmax(scale * q K^T) V`` over the materialised rows (TorchInferno page, "Custom Kernels":
  ``paged_decode_attention`` / ``batched_paged_decode_attention`` with a torch reference; CacheIR
  page, "Compiler Example": decode lowers grouped-query attention to one
  ``paged_attention_decode`` call).  Grouped-query mapping: query head ``h`` reads KV head
  ``h // (Hq / Hkv)`` (CacheIR page, "Boundaries": page-table decode attention with GQA mapping;
  consecutive query heads sharing a KV head is the Llama/Mistral/Qwen convention).
* The append writes the new token's K and V rows, bit for bit, at logical position
  ``context_lens[b]`` before attention runs over ``context_lens[b] + 1`` tokens (CacheIR page,
  "Compiler Example": the decode op receives the new token's k and v; TorchInferno page,
  "OpenAI-Compatible Serving": a separate KV-append kernel precedes decode attention).
* Split-KV: attention restricted to token partitions ``[p*P, min((p+1)*P, L))`` yields a normalised
  partial output and its log-sum-exp; merging partials with weights ``exp(lse_p - max lse)`` is an
  identity that reproduces the full result (no page states it; it is the algebra of the softmax
  normaliser, and the flash-decoding form the benchmark spec names).

Precision: inputs are decoded exactly to float64 (bf16 from raw bits), arithmetic is float64, the
softmax scale is the float32 value the caller passes, widened exactly.

Multi-query decode (T new tokens per sequence, causal) is the decode of each query over its own
prefix of the sequence.

Parity pins live in tests/test_oracle.py: a loop-only brute force over contiguous K/V, closed forms
(one token, two tokens, constant V, zero query, identical keys), invariance under page relabelling
and prefix unsharing, GQA equal to MHA over repeated KV heads, and the LSE-merge identity.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------------------------
# Exact decoding of stored element bits to float64
# ----------------------------------------------------------------------------------------------

def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to float64 exactly.

    ``bf16`` arrives as raw ``uint16`` bit patterns: a bfloat16 is the top half of a float32, so
    shifting the 16 bits into the high half of a 32-bit word gives the identical float32 value.
    """
    if dtype in ("f32", "f16"):
        return np.asarray(x).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x).view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------------
# Page-table materialisation
# ----------------------------------------------------------------------------------------------

def gather_rows(pool: np.ndarray, table_row: np.ndarray, length: int, page_size: int,
                kv_head: Optional[int] = None, lo: int = 0) -> np.ndarray:
    """Contiguous rows ``[lo, length)`` of one sequence: ``[n, kv_heads, D]``, or ``[n, D]`` for
    one KV head.

    Logical token ``t`` is slot ``t % page_size`` of page ``table_row[t // page_size]``.  Only the
    table entries covering ``[lo, length)`` are read, and each must name a page of the pool.
    """
    if length <= lo:
        shape = pool.shape[2:] if kv_head is None else pool.shape[3:]
        return np.empty((0,) + shape, dtype=pool.dtype)
    first = lo // page_size
    last = (length - 1) // page_size
    ids = np.asarray(table_row[first:last + 1], dtype=np.int64)
    num_pages = pool.shape[0]
    if np.any(ids < 0) or np.any(ids >= num_pages):
        raise ValueError(f"page id out of range in table entries {first}..{last}: {ids}")
    pages = pool[ids] if kv_head is None else pool[ids, :, kv_head, :]
    rows = pages.reshape((len(ids) * page_size,) + pages.shape[2:])
    start = lo - first * page_size
    return rows[start:start + (length - lo)]


# ----------------------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------------------

def _softmax_attend(scores: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, float]:
    """``softmax(scores) @ values`` and ``log(sum(exp(scores)))``, float64."""
    m = scores.max()
    w = np.exp(scores - m)
    z = w.sum()
    return (w @ values) / z, float(m + math.log(z))


def paged_decode_attention(q, k_pool, v_pool, page_table, context_lens, scale, dtype,
                           token_range=None):
    """Decode attention of ``q [B, Hq, D]`` over each sequence's paged K/V.

    Returns ``(out [B, Hq, D], lse [B, Hq])`` in float64.  A sequence with ``context_lens[b] <= 0``
    attends to nothing: its output is 0 and its lse is -inf.  ``token_range(b, L) -> (lo, hi)``
    optionally restricts attention to logical tokens ``[lo, hi)`` (used for split-KV partials).
    """
    B, Hq, D = q.shape
    _, PS, Hkv, _ = k_pool.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    sc = float(np.float32(scale))
    qf = to_f64(q, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        lo, hi = (0, L) if token_range is None else token_range(b, L)
        if hi <= lo:
            continue
        for kvh in range(Hkv):
            K = to_f64(gather_rows(k_pool, page_table[b], hi, PS, kvh, lo), dtype)
            V = to_f64(gather_rows(v_pool, page_table[b], hi, PS, kvh, lo), dtype)
            for g in range(G):
                h = kvh * G + g
                out[b, h], lse[b, h] = _softmax_attend(sc * (K @ qf[b, h]), V)
    return out, lse


def paged_multi_query_attention(q, k_pool, v_pool, page_table, context_lens, scale, dtype):
    """Causal attention of T new query tokens per sequence, ``q [B, T, Hq, D]``.

    ``context_lens[b]`` counts every token of the sequence, the T new ones included (their K/V
    rows are already in the pages).  Query ``j`` sits at position ``L - T + j`` and attends to
    tokens ``[0, L - T + j]``: it is the decode of one query over ``L - T + 1 + j`` tokens.
    Returns ``(out [B, T, Hq, D], lse [B, T, Hq])``; a query with no tokens gets 0 / -inf.
    (Infinity docs, "Short shared prefix qualification": a tile of up to 32 query rows of
    suffix tokens after a cached context; the causal rule is that of decoder self-attention.)"""
    B, T, Hq, D = q.shape
    lens = np.asarray(context_lens, dtype=np.int64)
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    lse = np.full((B, T, Hq), -np.inf, dtype=np.float64)
    for j in range(T):
        Lj = np.where(lens > 0, np.maximum(lens - T + 1 + j, 0), 0)
        out[:, j], lse[:, j] = paged_decode_attention(np.ascontiguousarray(q[:, j]), k_pool,
                                                      v_pool, page_table, Lj, scale, dtype)
    return out, lse


def num_partitions(context_lens, partition_tokens: int) -> np.ndarray:
    """Partitions per sequence: ``ceil(L / P)`` (0 for empty rows)."""
    L = np.maximum(np.asarray(context_lens, dtype=np.int64), 0)
    return -(-L // partition_tokens)


def paged_decode_attention_partial(q, k_pool, v_pool, page_table, context_lens, scale, dtype,
                                   partition_tokens: int, max_partitions: Optional[int] = None):
    """Per-partition normalised outputs and log-sum-exps.

    Partition ``p`` of sequence ``b`` covers logical tokens ``[p*P, min((p+1)*P, L_b))``.
    Returns ``(partial_out [B, Hq, Pmax, D], partial_lse [B, Hq, Pmax])``; unused partitions hold
    output 0 and lse -inf.
    """
    B, Hq, D = q.shape
    nparts = num_partitions(context_lens, partition_tokens)
    Pmax = int(nparts.max(initial=0)) if max_partitions is None else max_partitions
    po = np.zeros((B, Hq, Pmax, D), dtype=np.float64)
    pl = np.full((B, Hq, Pmax), -np.inf, dtype=np.float64)
    for p in range(Pmax):
        def rng(b, L, p=p):
            return p * partition_tokens, min((p + 1) * partition_tokens, L)
        o, l = paged_decode_attention(q, k_pool, v_pool, page_table, context_lens, scale, dtype,
                                      token_range=rng)
        po[:, :, p] = o
        pl[:, :, p] = l
    return po, pl


def lse_merge(partial_out, partial_lse, nparts):
    """Combine partitions: ``out = sum_p w_p o_p / sum_p w_p`` with ``w_p = exp(lse_p - max lse)``.

    ``nparts[b]`` partitions of row ``b`` are read.  Returns ``(out [B, Hq, D], lse [B, Hq])``;
    a row with no partitions gives output 0 and lse -inf.
    """
    po = np.asarray(partial_out, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    B, Hq, _, D = po.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(nparts[b])
        if n <= 0:
            continue
        for h in range(Hq):
            ls = pl[b, h, :n]
            M = ls.max()
            if M == -np.inf:
                continue
            w = np.exp(ls - M)
            out[b, h] = (w @ po[b, h, :n]) / w.sum()
            lse[b, h] = M + math.log(w.sum())
    return out, lse


# ----------------------------------------------------------------------------------------------
# Append
# ----------------------------------------------------------------------------------------------

def paged_kv_append(k_pool, v_pool, k_new, v_new, page_table, append_lens):
    """New pools with row ``b``'s new K/V written at logical position ``append_lens[b]``.

    The write is a raw copy of the stored bits into page ``page_table[b, L // page_size]``, slot
    ``L % page_size``.  Rows with a negative length are padding and write nothing.  Every other
    byte of the pools is unchanged.
    """
    kp = k_pool.copy()
    vp = v_pool.copy()
    PS = k_pool.shape[1]
    for b in range(len(append_lens)):
        L = int(append_lens[b])
        if L < 0:
            continue
        page = int(page_table[b, L // PS])
        if not 0 <= page < k_pool.shape[0]:
            raise ValueError(f"row {b}: append page id {page} out of range")
        kp[page, L % PS] = k_new[b]
        vp[page, L % PS] = v_new[b]
    return kp, vp


# ----------------------------------------------------------------------------------------------
# Metadata validation (what the library's device-side validator must report)
# ----------------------------------------------------------------------------------------------

STATUS_PAGE_RANGE = 1        # a live page-table entry outside [0, num_pages)
STATUS_CAPACITY = 2          # a context (plus extra tokens) longer than the table can address
STATUS_APPEND_ALIAS = 4      # an append destination page also read by another live row


def validate_metadata(page_table, context_lens, num_pages: int, page_size: int,
                      extra_tokens: int = 0, check_append_unique: bool = False) -> int:
    """Status bits for the page-table preconditions of attention and append.

    Live rows are those with ``context_lens[b] + extra_tokens > 0``; each needs
    ``ceil((L + extra) / page_size)`` entries, all in range.  With ``check_append_unique`` the page
    receiving row ``b``'s appended token (entry ``L // page_size``) must not appear among the live
    entries of any other row.
    """
    B, MP = page_table.shape
    status = 0
    live_sets = []
    for b in range(B):
        L = int(context_lens[b]) + extra_tokens
        if L <= 0:
            live_sets.append(set())
            continue
        n = -(-L // page_size)
        if n > MP:
            status |= STATUS_CAPACITY
            n = MP
        ids = page_table[b, :n]
        if np.any(ids < 0) or np.any(ids >= num_pages):
            status |= STATUS_PAGE_RANGE
        live_sets.append(set(int(i) for i in ids))
    if check_append_unique:
        for b in range(B):
            L = int(context_lens[b])
            if L < 0 or L + extra_tokens <= 0:
                continue
            idx = L // page_size
            if idx >= MP:
                continue
            dest = int(page_table[b, idx])
            for b2 in range(B):
                if b2 != b and dest in live_sets[b2]:
                    status |= STATUS_APPEND_ALIAS
                    break
    return status
