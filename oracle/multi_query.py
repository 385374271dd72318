"""Multi-query paged attention, float64 (oracle; test infrastructure only).

When a request's prompt prefix is already in the prefix cache, only its remaining prompt
tokens are new ("PagedAttention: Efficient LLM Serving with vLLM", "Advanced Features" ->
"Prefix Caching": later requests reuse the cached prefix blocks and skip recomputing them).
The same holds for a chunk of a long prompt and for the draft tokens that a target model
checks under speculative decoding (same page, "Speculative Decoding Integration": both
models keep their caches in pages).  In each case one sequence brings several new tokens at
once, each new token needs attention over the cached blocks, and the blocks are reached
through the sequence's block table as in decode ("The PagedAttention Algorithm", step 5).

What is computed, for sequence s with L_s cached tokens of which the last n_s are its new
tokens (their K/V already written into their slots), and new token i = 0 .. n_s-1 at
position P = L_s - n_s + i:

    z_t   = scale * <q_i, K_t>          t = 0 .. P
    out_i = sum_t softmax(z)_t V_t

Readings where the pages are silent:
  * the pages state no rule for several new tokens of one sequence; a new token attends to
    every token before it and to itself, never to a later one (the autoregressive rule that
    single-token decoding follows, which is the case n_s = 1);
  * the new tokens' K/V are written into the cache before attention, so every key, cached
    or new, is read through the block table;
  * query rows are packed: the new tokens of sequence s are rows query_start[s] ..
    query_start[s+1]-1 of q and of the output; n_s = 0 is allowed and yields no rows.
"""
from __future__ import annotations

import numpy as np

from .attention import attend, gather_sequence
from .storage import decode


def query_position(context_lens, query_start, s: int, i: int) -> int:
    """Position of new token i of sequence s: its cached tokens come first."""
    n = int(query_start[s + 1]) - int(query_start[s])
    L = int(context_lens[s])
    assert 0 <= i < n <= L, "new tokens must be the last tokens of the context"
    return L - n + i


def multi_query_unit(q, k_pool, v_pool, block_tables, context_lens, query_start, scale,
                     dtype: str, s: int, i: int, h: int) -> np.ndarray:
    """Output of new token i of sequence s, head h, in float64 (shape [D])."""
    BS = k_pool.shape[2]
    P = query_position(context_lens, query_start, s, i)
    Kc = decode(gather_sequence(k_pool, block_tables[s], P + 1, h, BS), dtype)
    Vc = decode(gather_sequence(v_pool, block_tables[s], P + 1, h, BS), dtype)
    q64 = decode(q[int(query_start[s]) + i, h], dtype)
    return attend(q64, Kc, Vc, float(np.float32(scale)))


def paged_attention_multi_query(q, k_pool, v_pool, block_tables, context_lens, query_start,
                                scale, dtype: str, units=None) -> np.ndarray:
    """Float64 outputs [T][H][D] for storage inputs.

    q: [T][H][D] with T = query_start[-1]; k_pool, v_pool: [NB][H][BS][D];
    block_tables: int [S][MB]; context_lens: int [S]; query_start: int [S+1], nondecreasing
    from 0.  ``units``: optional iterable of (s, i, h) to compute -- the rest is NaN.
    """
    T, H, D = q.shape
    S = len(context_lens)
    assert len(query_start) == S + 1 and int(query_start[0]) == 0 and int(query_start[S]) == T
    out = np.full((T, H, D), np.nan)
    if units is None:
        units = [(s, i, h) for s in range(S)
                 for i in range(int(query_start[s + 1]) - int(query_start[s]))
                 for h in range(H)]
    for s, i, h in units:
        out[int(query_start[s]) + i, h] = multi_query_unit(
            q, k_pool, v_pool, block_tables, context_lens, query_start, scale, dtype, s, i, h)
    return out
