"""Cache writes and block copies as plain byte copies (oracle; test infrastructure only).

reshape_and_cache: "Generate tokens, fill block" ("PagedAttention: Efficient LLM Serving with
vLLM", "The PagedAttention Algorithm", step 2) -- a new token's K and V rows are written into
the slot the block manager gave it.  A slot number is physical_block * block_size + offset;
a negative slot means "no write" (reading).

copy_blocks: copy-on-write of a shared block ("PagedAttention: Efficient LLM Serving with
vLLM", "Advanced Features" -> "KV-Cache Sharing (Copy-on-Write)": blocks stay shared until a
holder writes, as the pages of a forked process do) -- the destination block receives the
source block's bytes, in every layer.

Both work on integer views of the storage so that every bit, NaN payloads included, is copied
unchanged; the result is compared bit for bit.
"""
from __future__ import annotations

import numpy as np


def _bits(a: np.ndarray) -> np.ndarray:
    return a.view({2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def reshape_and_cache(k, v, k_pool, v_pool, slot_mapping):
    """Return copies of (k_pool, v_pool) with token i's rows written at slot_mapping[i].

    k, v: [N][H][D] storage; pools [NB][H][BS][D]; slot_mapping: int [N].
    """
    BS = k_pool.shape[2]
    kp = k_pool.copy()
    vp = v_pool.copy()
    kb, vb = _bits(kp), _bits(vp)
    ks, vs = _bits(np.ascontiguousarray(k)), _bits(np.ascontiguousarray(v))
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), BS)
        assert block < kp.shape[0], "slot out of range"
        kb[block, :, offset, :] = ks[i]
        vb[block, :, offset, :] = vs[i]
    return kp, vp


def copy_blocks(pools, pairs):
    """Return copies of every pool in ``pools`` with pool[dst] = pool[src] for each pair.

    ``pairs`` is int [n][2] of (src, dst).  Destinations are distinct and no destination is
    also a source, so the order of the copies does not matter.
    """
    pairs = np.asarray(pairs, np.int64).reshape(-1, 2)
    dsts = pairs[:, 1].tolist()
    assert len(set(dsts)) == len(dsts), "duplicate destination"
    assert not set(dsts) & set(pairs[:, 0].tolist()), "destination is also a source"
    out = []
    for p in pools:
        c = p.copy()
        cb = _bits(c)
        pb = _bits(p)
        for src, dst in pairs.tolist():
            cb[dst] = pb[src]
        out.append(c)
    return out


def swap_blocks(src_pools, dst_pools, pairs):
    """Return copies of the destination pools with dst[d] = src[s] for each (s, d) pair, in
    every layer: the byte copy that moves blocks between HBM and host swap memory."""
    pairs = np.asarray(pairs, np.int64).reshape(-1, 2)
    dsts = pairs[:, 1].tolist()
    assert len(set(dsts)) == len(dsts), "duplicate destination"
    out = []
    for sp, dp in zip(src_pools, dst_pools):
        c = dp.copy()
        cb, sb = _bits(c), _bits(np.ascontiguousarray(sp))
        for s, d in pairs.tolist():
            cb[d] = sb[s]
        out.append(c)
    return out
