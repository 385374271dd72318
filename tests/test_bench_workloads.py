"""Host-side checks of bench.py's workloads (CPU): the fork step makes exactly the
copy-on-write work it claims on every step, without leaking blocks, and the prefix-hit batch
has the shape its description states."""
import types

import numpy as np

import bench
import paged_kv_cache_306_amd as pkv
import workloads as W


def _fork_step_manager():
    """The block-manager half of bench.DecodeBatch for the fork step (no GPU needed)."""
    sp = bench.workload_spec("fork_step", 2, 16, "permuted")
    b = types.SimpleNamespace(sp=sp, S=sp["S"], init_lens=sp["lens"],
                              seq_ids=np.arange(sp["S"], dtype=np.int64), next_id=sp["S"])
    b.alloc = pkv.BlockAllocator(sp["NB"], sp["BS"], free_order=sp["order"])
    b._fork_groups = types.MethodType(bench.DecodeBatch._fork_groups, b)
    b.recycle = types.MethodType(bench.DecodeBatch.recycle, b)
    b._fork_groups()
    b.grown = 0
    return sp, b


def test_fork_step_copies_224_blocks_every_step():
    sp, b = _fork_step_manager()
    assert sp["S"] == 256 and sp["groups"] == 32
    r = sp["prompts"] - 512
    assert r.min() >= 1 and r.max() <= 15          # the prompt's last block is partly filled
    free = []
    for _ in range(4):
        b.recycle()
        slots, pairs = b.alloc.append_slots(b.seq_ids)
        b.grown += 1
        # 8 holders of each group's partial block: the first 7 writers copy, the last writes
        # in place
        assert len(pairs) == 7 * 32
        assert len(set(int(s) for s in slots)) == sp["S"]
        srcs = [int(p[0]) for p in pairs]
        assert all(srcs.count(s) == 7 for s in set(srcs))
        free.append(b.alloc.num_free())
    assert len(set(free)) == 1                      # re-forking returns every block


def test_prefix_hit_batch_shape():
    w = W.prefix_hit()
    qs = w.extra["query_start"]
    n = np.diff(qs)
    assert w.S == 64 and int(qs[-1]) == 17396
    assert n.min() >= 16 and n.max() <= 512
    assert (w.lens - n == 1024).all()               # each context: its system prompt + turn
    # consecutive requests share a prompt: their first 64 blocks are the same physical ones
    for p in range(4):
        rows = w.tables[16 * p:16 * p + 16, :64]
        assert (rows == rows[0]).all()
    assert len({tuple(w.tables[16 * p, :64]) for p in range(4)}) == 4


def test_decode_tile_list_is_exactly_the_decode_reads():
    """bench.py --ceiling's own-tiles case reads every K and V (block, head) tile the decode
    launch reads, each once, and nothing else: ceil(L / 16) blocks per sequence, every head."""
    for wl in ("llama13b_layer", "full_step_40", "long_context"):
        idx, n_buf, tile, sp = bench.decode_tile_list(wl, 2)
        H, NB = sp["H"], sp["NB"]
        lens = sp["lens"] + 1
        nblk = -(-lens // 16)
        assert tile == 16 * 128 * 2 and n_buf == 2 * NB * H
        assert len(idx) == 2 * H * int(nblk.sum())
        assert len(np.unique(idx)) == len(idx) and idx.min() >= 0 and idx.max() < n_buf
        k, v = idx[idx < NB * H], idx[idx >= NB * H] - NB * H
        assert np.array_equal(np.sort(k), np.sort(v))            # K and V of the same tiles
        blocks = np.unique(k // H)
        assert len(blocks) == int(nblk.sum())                     # no block shared or skipped
        assert (np.bincount(k % H, minlength=H) == int(nblk.sum())).all()
