"""Paged decode attention, float64 (oracle; test infrastructure only).

What is computed ("PagedAttention: Efficient LLM Serving with vLLM", "How PagedAttention
Works" -> "The PagedAttention Algorithm", steps 4 and 5; "Efficient Memory Management for
Large Language Model Serving with PagedAttention", observer card, "Key ideas"): the KV cache
of a sequence is cut into fixed-size blocks placed anywhere in a physical pool; a per-sequence
block table maps logical block j to a physical block; attention gathers the sequence's K/V
pairs through that table.  Paging changes only where the bytes sit, so the result is ordinary
single-query attention over the sequence's tokens in logical order:

    z_t   = scale * <q, K_t>                 t = 0 .. L-1
    p     = softmax(z)
    out   = sum_t p_t V_t

Readings where the pages are silent:
  * token t (0-based) lives in physical block table[t // BS] at slot t % BS; the pages'
    "tokens 1-16" in the first block is the 1-based view of the same mapping;
  * pool layout [num_blocks][num_heads][block_size][head_dim], the same for K and V;
  * a sequence of length 0 attends to nothing and yields a zero vector;
  * ``scale`` is the binary32 value the kernel receives, widened to float64.
"""
from __future__ import annotations

import numpy as np

from .storage import decode


def gather_sequence(pool, table_row, length: int, head: int, block_size: int) -> np.ndarray:
    """Rows of ``pool`` for tokens 0..length-1 of one sequence and one head, in logical order.

    Token t comes from physical block ``table_row[t // block_size]``, slot
    ``t % block_size``.  Returns the stored elements (no conversion), shape [length, D].
    """
    length = int(length)
    t = np.arange(length)
    blocks = np.asarray(table_row)[t // block_size].astype(np.int64)
    assert np.all((blocks >= 0) & (blocks < pool.shape[0])), "block id out of range"
    return pool[blocks, head, t % block_size, :]


def attend(q64: np.ndarray, K64: np.ndarray, V64: np.ndarray, scale: float) -> np.ndarray:
    """Textbook single-query attention in float64: softmax(scale * K q) weighted sum of V."""
    if K64.shape[0] == 0:
        return np.zeros(V64.shape[1], np.float64)
    z = float(scale) * (K64 @ q64)
    m = z.max()
    w = np.exp(z - m)
    return (w @ V64) / w.sum()


def decode_unit(q, k_pool, v_pool, block_tables, context_lens, scale, dtype: str,
                s: int, h: int) -> np.ndarray:
    """Output of sequence ``s``, head ``h`` in float64 (shape [D])."""
    BS = k_pool.shape[2]
    L = int(context_lens[s])
    Kc = decode(gather_sequence(k_pool, block_tables[s], L, h, BS), dtype)
    Vc = decode(gather_sequence(v_pool, block_tables[s], L, h, BS), dtype)
    q64 = decode(q[s, h], dtype)
    return attend(q64, Kc, Vc, float(np.float32(scale)))


def paged_attention_decode(q, k_pool, v_pool, block_tables, context_lens, scale,
                           dtype: str, units=None) -> np.ndarray:
    """Float64 outputs [S][H][D] for storage inputs.

    q: [S][H][D]; k_pool, v_pool: [NB][H][BS][D]; block_tables: int [S][MB];
    context_lens: int [S]; ``units``: optional iterable of (s, h) to compute -- the rest
    of the result is NaN.
    """
    S, H, D = q.shape
    out = np.full((S, H, D), np.nan)
    if units is None:
        units = [(s, h) for s in range(S) for h in range(H)]
    for s, h in units:
        out[s, h] = decode_unit(q, k_pool, v_pool, block_tables, context_lens, scale,
                                dtype, s, h)
    return out
