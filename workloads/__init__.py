"""Seeded synthetic inputs for the paged decode path.

This module is shared by the float64 oracle's tests and by the HIP path's tests and bench.
It holds none of the method's arithmetic (no attention, no cache write, no block
allocation policy): it draws context lengths, a physical placement for each sequence's
blocks and N(0,1) values, and lays them out as the arrays the calls take.

Shapes and distributions follow the LLaMA/OPT-13B-shaped decode workloads the PagedAttention
pages talk about ("Efficient Memory Management for Large Language Model Serving with
PagedAttention", Abstract; "PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention
Algorithm": 16-token blocks placed anywhere in GPU memory and reached through a page table).
The pages name no dataset; these recipes stand in for their workloads.

Storage arrays are numpy arrays holding the raw element bits' carrier type:
``f32`` -> float32, ``f16`` -> float16, ``bf16`` -> uint16 (the upper half of a binary32).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

# Quiet-NaN bit patterns used to poison memory that a correct kernel never reads.
_NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- values
def f32_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type, round-to-nearest-even."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        nan = np.isnan(x)
        lsb = (u >> 16) & 1
        r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
        r[nan] = _NAN_BITS["bf16"]
        return r
    raise ValueError(dtype)


def storage_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def nan_fill(dtype: str):
    """A scalar of the storage carrier type holding a quiet NaN."""
    if dtype == "f32":
        return np.array([_NAN_BITS["f32"]], np.uint32).view(np.float32)[0]
    if dtype == "f16":
        return np.array([_NAN_BITS["f16"]], np.uint16).view(np.float16)[0]
    return np.uint16(_NAN_BITS["bf16"])


def normal_values(g: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) drawn in float32, then rounded to the storage type."""
    return f32_to_storage(g.standard_normal(shape, dtype=np.float32), dtype)


# ----------------------------------------------------------------------------- lengths
def uniform_lens(g: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform in [lo, hi], both ends included."""
    return g.integers(lo, hi + 1, size=n).astype(np.int32)


def lognormal_lens(g: np.random.Generator, n: int, mean: float, sigma: float,
                   lo: int, hi: int) -> np.ndarray:
    """Lognormal lengths whose unclipped arithmetic mean is ``mean`` (log-sigma ``sigma``),
    rounded to the nearest integer and clipped to [lo, hi]."""
    mu = math.log(mean) - 0.5 * sigma * sigma
    x = np.rint(g.lognormal(mu, sigma, size=n))
    return np.clip(x, lo, hi).astype(np.int32)


# ----------------------------------------------------------------------------- placement
def nblocks_for(length: int, block_size: int) -> int:
    """Blocks a sequence of ``length`` tokens occupies (input layout, ceil division)."""
    return -(-int(length) // block_size)


def permuted_block_tables(g: np.random.Generator, lens, block_size: int,
                          pool_factor: float = 1.2, max_blocks: int | None = None,
                          num_blocks: int | None = None):
    """Give every sequence its own blocks, taken in (sequence, logical block) order from a
    seeded random permutation of a pool sized ``pool_factor`` x the total need.

    Returns ``(tables, num_blocks)``; ``tables`` is int32 [S][max_blocks] and holds -1 in
    every entry past a sequence's last block.
    """
    lens = np.asarray(lens)
    need = [nblocks_for(L, block_size) for L in lens]
    total = int(sum(need))
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(pool_factor * total)))
    assert num_blocks >= total
    if max_blocks is None:
        max_blocks = max(1, max(need) if need else 1)
    perm = g.permutation(num_blocks).astype(np.int32)
    tables = np.full((len(lens), max_blocks), -1, np.int32)
    k = 0
    for s, n in enumerate(need):
        tables[s, :n] = perm[k:k + n]
        k += n
    return tables, num_blocks


def identity_block_tables(lens, block_size: int, max_blocks: int | None = None):
    """Contiguous placement: sequence s's blocks follow those of s-1 in the pool."""
    need = [nblocks_for(L, block_size) for L in lens]
    if max_blocks is None:
        max_blocks = max(1, max(need) if need else 1)
    tables = np.full((len(lens), max_blocks), -1, np.int32)
    k = 0
    for s, n in enumerate(need):
        tables[s, :n] = np.arange(k, k + n, dtype=np.int32)
        k += n
    return tables, max(1, k)


def shared_prefix_tables(g: np.random.Generator, groups: int, per_group: int,
                         prefix_len: int, tail_lens, block_size: int,
                         pool_factor: float = 1.2):
    """Groups of ``per_group`` sequences whose first ``prefix_len`` tokens sit in the same
    physical blocks; each sequence then owns the blocks of its own tail.

    Only whole prefix blocks are shared: a prefix that ends inside a block gives every
    sequence its own copy of that last partial block (so the tail can follow it).
    Returns ``(tables, lens, num_blocks)``.
    """
    S = groups * per_group
    tail_lens = np.asarray(tail_lens, np.int64)
    assert tail_lens.shape == (S,)
    shared = prefix_len // block_size
    lens = (prefix_len + tail_lens).astype(np.int32)
    own = [nblocks_for(L, block_size) - shared for L in lens]
    total = groups * shared + int(sum(own))
    num_blocks = max(1, int(math.ceil(pool_factor * total)))
    perm = g.permutation(num_blocks).astype(np.int32)
    max_blocks = max(1, max(shared + o for o in own))
    tables = np.full((S, max_blocks), -1, np.int32)
    k = 0
    for gi in range(groups):
        pre = perm[k:k + shared]
        k += shared
        for j in range(per_group):
            s = gi * per_group + j
            tables[s, :shared] = pre
            tables[s, shared:shared + own[s]] = perm[k:k + own[s]]
            k += own[s]
    return tables, lens, num_blocks


def poison_unused(pool: np.ndarray, tables, lens, block_size: int, dtype: str) -> None:
    """Write NaN into every block no table references and into every slot of a referenced
    block that no sequence's length reaches.  ``pool`` is [NB][H][BS][D] storage."""
    nan = nan_fill(dtype)
    filled = np.zeros(pool.shape[0], np.int64)   # valid slots per physical block
    used = np.zeros(pool.shape[0], bool)
    for s, L in enumerate(lens):
        n = nblocks_for(L, block_size)
        for j in range(n):
            b = tables[s, j]
            used[b] = True
            filled[b] = max(filled[b], min(block_size, int(L) - j * block_size))
    pool[~used] = nan
    for b in np.nonzero(used & (filled < block_size))[0]:
        pool[b, :, filled[b]:, :] = nan


# ----------------------------------------------------------------------------- workloads
@dataclass
class DecodeShape:
    """One decode batch: S sequences, H heads of size D, blocks of BS tokens."""
    name: str
    S: int
    H: int
    D: int
    BS: int
    dtype: str
    lens: np.ndarray
    tables: np.ndarray
    num_blocks: int
    scale: float
    seed: int
    extra: dict = field(default_factory=dict)

    @property
    def max_blocks(self) -> int:
        return int(self.tables.shape[1])

    @property
    def max_len(self) -> int:
        return int(self.lens.max()) if len(self.lens) else 0

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode pass reads: 2 * sum(L) * H * D * e."""
        return int(2 * int(np.asarray(self.lens, np.int64).sum()) * self.H * self.D
                   * ELEM_BYTES[self.dtype])


def tiny_fp32(seed: int = 1) -> DecodeShape:
    """4 seqs, 4 heads, head_dim 64, block 16, lengths {1,15,16,37}, 32-block pool placed by a
    seeded random permutation; scale 1/sqrt(64)."""
    g = rng(seed)
    lens = np.array([1, 15, 16, 37], np.int32)
    tables, nb = permuted_block_tables(g, lens, 16, num_blocks=32)
    return DecodeShape("tiny_fp32", 4, 4, 64, 16, "f32", lens, tables, nb, 0.125, seed)


def llama13b_layer(seed: int = 2) -> DecodeShape:
    """LLaMA-13B-shaped single layer, fp16: 64 seqs, 40 heads, head_dim 128, block 16,
    lengths uniform in [128, 2048], pool 1.2x the need, seeded random permutation."""
    g = rng(seed)
    lens = uniform_lens(g, 64, 128, 2048)
    tables, nb = permuted_block_tables(g, lens, 16, pool_factor=1.2)
    return DecodeShape("llama13b_layer_fp16", 64, 40, 128, 16, "f16", lens, tables, nb,
                       float(np.float32(1.0 / math.sqrt(128))), seed)


def shared_prefix(seed: int = 3, groups: int = 32, per_group: int = 8,
                  prefix_len: int = 512, tail_max: int = 256) -> DecodeShape:
    """Parallel sampling: 32 groups x 8 seqs share a 512-token prefix (same physical blocks),
    then own tails of uniform [0, 256] tokens; fp16, 40 heads, head_dim 128, block 16."""
    g = rng(seed)
    tails = uniform_lens(g, groups * per_group, 0, tail_max)
    tables, lens, nb = shared_prefix_tables(g, groups, per_group, prefix_len, tails, 16)
    return DecodeShape("shared_prefix_fp16", groups * per_group, 40, 128, 16, "f16", lens,
                       tables, nb, float(np.float32(1.0 / math.sqrt(128))), seed,
                       extra={"groups": groups, "per_group": per_group,
                              "prefix_len": prefix_len})


def long_context(seed: int = 4, block_size: int = 16) -> DecodeShape:
    """Long-context stress, bf16: 8 seqs, 40 heads, head_dim 128, lengths uniform in
    [16384, 32768] (the same for every block size), block size in {8, 16, 32}."""
    g = rng(seed)
    lens = uniform_lens(g, 8, 16384, 32768)
    gp = rng(seed * 1000 + block_size)
    tables, nb = permuted_block_tables(gp, lens, block_size, pool_factor=1.2)
    return DecodeShape(f"long_context_bf16_bs{block_size}", 8, 40, 128, block_size, "bf16",
                       lens, tables, nb, float(np.float32(1.0 / math.sqrt(128))), seed)


def shared_prompt_runs(seed: int, groups, block_size: int, solo=()):
    """Consecutive sequences in groups, each group sharing the whole blocks of a prompt (a
    partly filled last block is each member's own, as a prefix cache keeps it), then a few
    cached tokens of each member's own and its new tokens; ``groups``: list of (members,
    prompt tokens, (lo, hi) new tokens per member); ``solo``: context lengths of sequences that
    share nothing, appended, each with U[1, L] new tokens.  Block ids are consecutive (callers
    permute them).  Returns ``(query_start, context_lens, tables)``; tables are padded with
    -1."""
    g = rng(seed)
    rows, lens, nxt = [], [], 0
    for members, prompt, (lo, hi) in groups:
        shared = list(range(nxt, nxt + prompt // block_size))
        nxt += len(shared)
        for _ in range(members):
            own = int(g.integers(0, 40))
            n = int(g.integers(lo, hi + 1))
            L = prompt + own + n
            k = nblocks_for(L, block_size) - len(shared)
            rows.append(shared + list(range(nxt, nxt + k)))
            nxt += k
            lens.append((L, n))
    for L in solo:
        n = int(g.integers(1, L + 1))
        k = nblocks_for(L, block_size)
        rows.append(list(range(nxt, nxt + k)))
        nxt += k
        lens.append((L, n))
    mb = max(len(r) for r in rows)
    tables = np.full((len(rows), mb), -1, np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    ctx = np.array([L for L, _ in lens], np.int32)
    n = np.array([n for _, n in lens], np.int64)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    return qs, ctx, tables


def prefix_hit(seed: int = 6, requests: int = 64, prompts: int = 4, system_len: int = 1024,
               user_lo: int = 16, user_hi: int = 512, block_size: int = 16,
               dtype: str = "f16") -> DecodeShape:
    """Chat requests after a prefix-cache hit, LLaMA-13B shapes (40 heads, head_dim 128): each
    request starts with one of ``prompts`` system prompts of ``system_len`` tokens whose
    blocks are cached and shared by every request with that prompt (consecutive requests
    share one), then brings a user turn of uniform [user_lo, user_hi] new tokens.  ``lens``
    are the context lengths (prompt + user turn); ``extra["query_start"]`` packs the new
    tokens (the user turns), int32 [requests + 1]."""
    g = rng(seed)
    user = uniform_lens(g, requests, user_lo, user_hi)
    tables, lens, nb = shared_prefix_tables(g, prompts, requests // prompts, system_len, user,
                                            block_size, pool_factor=1.05)
    qs = np.concatenate([[0], np.cumsum(user)]).astype(np.int32)
    return DecodeShape(f"prefix_hit_{dtype}", requests, 40, 128, block_size, dtype, lens,
                       tables, nb, float(np.float32(1.0 / math.sqrt(128))), seed,
                       extra={"query_start": qs, "prompts": prompts, "system_len": system_len,
                              "user_range": (user_lo, user_hi)})


def full_step_lens(seed: int = 5, S: int = 512) -> np.ndarray:
    """40-layer step: 512 context lengths, lognormal (mean 600, sigma 0.8), clipped to
    [1, 2048]."""
    return lognormal_lens(rng(seed), S, 600.0, 0.8, 1, 2048)


# ----------------------------------------------------------------------------- torch glue
def to_torch(arr: np.ndarray, dtype: str):
    """Host storage array -> CPU torch tensor of the matching torch dtype (same bits)."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr))


def from_torch(t, dtype: str) -> np.ndarray:
    """torch tensor (any device) -> host storage array (same bits)."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def device_normal(shape, dtype: str, seed: int, device):
    """N(0,1) values drawn on the device by torch's seeded generator, in the storage type.
    Used for pools too large to draw on the host; the oracle reads back the stored values."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return torch.randn(shape, dtype=torch_dtype(dtype), device=device, generator=gen)


def poison_unused_device(pool_t, tables, lens, block_size: int) -> None:
    """Device-tensor version of ``poison_unused``: NaN into unreferenced blocks and into
    slots of referenced blocks that no sequence's length reaches."""
    import torch
    nb = pool_t.shape[0]
    filled = np.zeros(nb, np.int64)
    used = np.zeros(nb, bool)
    for s, L in enumerate(np.asarray(lens).tolist()):
        n = nblocks_for(L, block_size)
        if n == 0:
            continue
        row = np.asarray(tables[s, :n], np.int64)
        used[row] = True
        counts = np.minimum(block_size, int(L) - np.arange(n) * block_size)
        np.maximum.at(filled, row, counts)
    dev = pool_t.device
    unused = torch.from_numpy(np.nonzero(~used)[0]).to(dev)
    if unused.numel():
        pool_t.index_fill_(0, unused, float("nan"))
    partial = np.nonzero(used & (filled < block_size))[0]
    for r in range(1, block_size):
        sel = partial[filled[partial] == r]
        if sel.size:
            idx = torch.from_numpy(sel).to(dev)
            sub = pool_t.index_select(0, idx)
            sub[:, :, r:, :] = float("nan")
            pool_t.index_copy_(0, idx, sub)


def fork_groups(seed: int = 3, groups: int = 32, per_group: int = 8, prefix_len: int = 512,
                rmax: int = 15):
    """Copy-on-write step of the parallel-sampling workload: each group's prompt is
    prefix_len + r_g tokens (r_g uniform in [1, rmax]), so its last prompt block is partly
    filled and shared by the group's sequences after forking.  Returns the prompt lengths."""
    g = rng(seed * 31 + 7)
    return (prefix_len + uniform_lens(g, groups, 1, rmax)).astype(np.int32)


def full_step(seed: int = 5, S: int = 512, block_size: int = 16, slack: float = 1.05):
    """40-layer decode step: lognormal lengths (mean 600, sigma 0.8, clipped to [1, 2048]);
    the pool holds every sequence's blocks after one appended token, plus ``slack``.
    Returns (lens, num_blocks, free_order)."""
    lens = full_step_lens(seed, S)
    need = int(sum(nblocks_for(int(L) + 1, block_size) for L in lens))
    nb = int(math.ceil(slack * need))
    order = rng(seed * 1000 + 17).permutation(nb).astype(np.int32)
    return lens, nb, order
