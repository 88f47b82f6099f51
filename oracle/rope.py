"""Plain CPU oracle for the rotary position embedding (RoPE) of a decode step's new token.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's CPU-baseline leg
may import this module; the library never does, and nothing here is shared with the HIP code.

What is computed.  Before attention, the new token's query and key are rotated by their position
(CacheIR page, "Compiler Example": ``rope(q, k)`` feeds grouped-query attention, and
``fused_rmsnorm_qkv_rope`` feeds ``paged_attention_decode``; TorchInferno page,
"OpenAI-Compatible Serving": a decode rotary-append kernel writes the rotated key into the paged
cache).  The pages name the step but not its formula.  The reading used here is the rotate-half
form of the Llama/Mistral/Qwen decoders the pages target: for pair ``i < D/2`` of a head at
position ``p``, with ``c = cos_table[p, i]`` and ``s = sin_table[p, i]``,

    y[i]       = x[i] * c - x[i + D/2] * s
    y[i + D/2] = x[i + D/2] * c + x[i] * s

The cos/sin cache is an input, float32 ``[positions, D/2]``, as a model's rotary cache is; the new
token's position is its index in the sequence, ``context_lens[b]`` before the append.

Precision.  The rotated value is rounded to the element type, a decision made on a float, so the
oracle takes it in the kernel's precision: float32 products and sum, each rounded to nearest even
(no fused multiply-add), then float32 -> element type, round to nearest even.  The float64 complex
rotation in tests/test_oracle_rope.py pins this to the mathematics (within float32 rounding), and
pins the complex form itself by its algebra (angles add, norms are kept, scores depend only on
the position difference).
"""
from __future__ import annotations

import numpy as np


def _to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored element bits -> float32 (exact for every dtype here); "f64" stays float64."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def _from_f32(y: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> stored element bits, round to nearest even (bf16 NaN -> 0x7FC0)."""
    if dtype == "f64":
        return np.asarray(y, dtype=np.float64)
    y = np.asarray(y, dtype=np.float32)
    if dtype == "f32":
        return y.copy()
    if dtype == "f16":
        return y.astype(np.float16)
    if dtype == "bf16":
        u = y.view(np.uint32).astype(np.uint64)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        nan = np.isnan(y)
        r[nan] = np.uint16(0x7FC0)
        return r
    raise ValueError(dtype)


def rotate(x: np.ndarray, dtype: str, positions: np.ndarray, cos_table: np.ndarray,
           sin_table: np.ndarray) -> np.ndarray:
    """RoPE of ``x`` ``[B, H, D]`` (storage dtype) at ``positions[b]``; returns storage bits.
    ``dtype="f64"`` computes in float64 throughout (tables taken as given), for the pins."""
    xf = _to_f32(x, dtype)
    B, H, D = xf.shape
    half = D // 2
    ct = np.float64 if dtype == "f64" else np.float32
    c = np.asarray(cos_table, dtype=ct)[np.asarray(positions)][:, None, :]   # [B, 1, D/2]
    s = np.asarray(sin_table, dtype=ct)[np.asarray(positions)][:, None, :]
    x1, x2 = xf[..., :half], xf[..., half:]
    y1 = (x1 * c) - (x2 * s)          # float32 ops (float64 for "f64"), each rounded
    y2 = (x2 * c) + (x1 * s)
    return _from_f32(np.concatenate([y1, y2], axis=-1), dtype)


def rope_kv_append(q, k_pool, v_pool, k_new, v_new, page_table, context_lens, cos_table,
                   sin_table, dtype: str):
    """The fused rotary + append step: returns ``(q_rot, k_pool', v_pool')``.

    Rows with ``context_lens[b] < 0`` are padding: their q rows are returned unrotated and they
    write nothing.  Every other row's new token sits at position ``L = context_lens[b]``: its
    rotated key and its value are written, bit for bit, at slot ``L % PS`` of page
    ``page_table[b, L // PS]`` (the append of oracle.paged_attention, with the key rotated)."""
    lens = np.asarray(context_lens)
    live = lens >= 0
    pos = np.where(live, lens, 0)
    q_rot = np.array(q, copy=True)
    k_rot = rotate(k_new, dtype, pos, cos_table, sin_table)
    q_all = rotate(q, dtype, pos, cos_table, sin_table)
    q_rot[live] = q_all[live]
    kp, vp = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    PS = kp.shape[1]
    for b in np.nonzero(live)[0]:
        L = int(lens[b])
        page = int(page_table[b, L // PS])
        kp[page, L % PS] = k_rot[b]
        vp[page, L % PS] = v_new[b]
    return q_rot, kp, vp
