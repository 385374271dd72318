"""Block manager with reference counts and copy-on-write (oracle; test infrastructure only).

Model of the host-side KV block allocator, written from the pages:
  * "PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention Algorithm",
    steps 1-4: a request's first block is allocated when it starts; tokens fill the block;
    when the block is full the next one is taken from any free place in the pool; a page table
    records logical block -> physical block.
  * same page, "Memory Efficiency": blocks are allocated on demand, so the only waste is the
    unused tail of each sequence's last block (100 tokens -> 7 blocks of 16 -> 112 slots,
    12 unused).
  * same page, "Advanced Features" -> "KV-Cache Sharing (Copy-on-Write)": sequences that share
    a prefix share its blocks; tokens past the point where they differ go to new blocks; as with the pages of a
    forked Unix process, a block stays shared until one of its holders writes to it.
  * "Efficient Memory Management for Large Language Model Serving with PagedAttention",
    observer card, "Key ideas": prefix blocks are shared across sequences of one prompt
    (parallel sampling, beam search) via copy-on-write.

Readings where the pages are silent:
  * "any free place" is a free list whose initial order is an input (tests pass a
    seeded random permutation); a freed block goes back on top of the list and is handed out
    next (last in, first out); a freed sequence returns its blocks so that its logical block
    0 is on top;
  * a write to a block whose reference count is above one takes a fresh block, records the
    pair (src, dst) for the device copy and drops one reference from src; the last holder
    (count one) writes in place, as fork() does;
  * a write that starts a new block never copies anything, even if earlier blocks are shared;
  * wasted slots = for every physical block in use, block_size minus the largest number of
    valid tokens any sequence keeps in it.

Prefix cache ("PagedAttention: Efficient LLM Serving with vLLM", "Advanced Features" ->
"Prefix Caching": the KV blocks of a shared prompt prefix are cached by the first request and
reused by later ones, which skip recomputing it).  Readings:
  * a full prompt block is identified by its own block_size token ids together with the
    identity of the block before it (so equal token runs after different prefixes differ);
    identities are fresh numbers that are never reused;
  * the trailing partial block of a prompt is never cached;
  * a cached block whose last reference goes away is kept, parked in the order it was parked;
    new blocks come from the plain free list first and only then by evicting the block parked
    longest ago; a cache hit on a parked block takes it back.
"""
from __future__ import annotations

from collections import OrderedDict


class OutOfBlocks(Exception):
    """No free block is left in the pool."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._free = order[::-1]            # top of the stack = next block handed out
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.cache: dict[tuple, int] = {}     # (parent identity, tokens) -> block
        self.ident = [0] * num_blocks         # identity of a cached block, 0 if not cached
        self.key_of: dict[int, tuple] = {}
        self.parked: OrderedDict[int, None] = OrderedDict()   # oldest first
        self._next_ident = 1

    # -- free list ---------------------------------------------------------------------
    def _take(self) -> int:
        if self._free:
            b = self._free.pop()
        elif self.parked:
            b, _ = self.parked.popitem(last=False)      # parked longest ago
            del self.cache[self.key_of.pop(b)]
            self.ident[b] = 0
        else:
            raise OutOfBlocks()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        assert self.ref[b] > 0
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if self.ident[b]:
                self.parked[b] = None
            else:
                self._free.append(b)

    # -- sequences ---------------------------------------------------------------------
    def add_seq(self, seq: int, length: int) -> None:
        """A new sequence holding ``length`` tokens gets ceil(length / BS) blocks."""
        if seq in self.tables or length < 0:
            raise ValueError("bad sequence")
        n = -(-length // self.block_size)
        if n > self.num_free():
            raise OutOfBlocks()
        self.tables[seq] = [self._take() for _ in range(n)]
        self.lens[seq] = length

    def add_seq_cached(self, seq: int, tokens) -> int:
        """A new sequence whose prompt is ``tokens``: its leading full blocks that are in the
        prefix cache are shared (one more reference each); the rest are fresh, and the fresh
        full blocks are entered in the cache.  Returns the number of prompt tokens whose K/V
        is already present (the cached blocks' tokens)."""
        if seq in self.tables:
            raise ValueError("bad sequence")
        tokens = [int(t) for t in tokens]
        BS = self.block_size
        full, n = len(tokens) // BS, -(-len(tokens) // BS)
        hits, parent = [], 0
        for j in range(full):
            b = self.cache.get((parent, tuple(tokens[j * BS:(j + 1) * BS])))
            if b is None:
                break
            hits.append(b)
            parent = self.ident[b]
        if n - len(hits) > self.num_free() - sum(1 for b in hits if b in self.parked):
            raise OutOfBlocks()
        table = []
        for b in hits:
            self.parked.pop(b, None)
            self.ref[b] += 1
            table.append(b)
        for j in range(len(hits), n):
            b = self._take()
            table.append(b)
            if j < full:
                key = (parent, tuple(tokens[j * BS:(j + 1) * BS]))
                self.cache[key] = b
                self.key_of[b] = key
                self.ident[b] = self._next_ident
                self._next_ident += 1
                parent = self.ident[b]
        self.tables[seq] = table
        self.lens[seq] = len(tokens)
        return len(hits) * BS

    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent; each gains one reference."""
        if parent not in self.tables or child in self.tables:
            raise ValueError("bad sequence")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append_slot(self, seq: int):
        """Make room for one more token of ``seq``.

        Returns (slot, cow) where slot = physical_block * BS + offset for the new token and
        cow is None or the (src, dst) pair of blocks to copy before the write.
        """
        if seq not in self.tables:
            raise ValueError("bad sequence")
        table = self.tables[seq]
        L = self.lens[seq]
        j, offset = divmod(L, self.block_size)
        cow = None
        if j == len(table):
            table.append(self._take())
        else:
            src = table[j]
            if self.ref[src] > 1:
                dst = self._take()
                self.ref[src] -= 1
                table[j] = dst
                cow = (src, dst)
        self.lens[seq] = L + 1
        return table[j] * self.block_size + offset, cow

    def append_slots(self, seqs):
        """``append_slot`` for each sequence in order; stops at the first failure.

        Returns (slots, cow_pairs, n_done).
        """
        slots, pairs = [], []
        for i, s in enumerate(seqs):
            try:
                slot, cow = self.append_slot(s)
            except (OutOfBlocks, ValueError):
                return slots, pairs, i
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        return slots, pairs, len(slots)

    def append_need(self, seqs) -> int:
        """Blocks ``append_slots(seqs)`` would take from the pool (new blocks at a block
        boundary, fresh blocks for copy-on-write), found by running it on a copy of this
        manager that is given one spare block per append, and counting.  ValueError for an
        unknown sequence."""
        import copy
        seqs = [int(s) for s in seqs]
        if any(s not in self.tables for s in seqs):
            raise ValueError("bad sequence")
        twin = copy.deepcopy(self)
        spare = list(range(self.num_blocks, self.num_blocks + len(seqs)))
        twin.ref += [0] * len(spare)
        twin.ident += [0] * len(spare)
        twin._free = spare[::-1] + twin._free     # used only once the real pool is empty
        before = twin.num_free()
        twin.append_slots(seqs)
        return before - twin.num_free()

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise ValueError("bad sequence")
        for b in reversed(self.tables.pop(seq)):
            self._drop(b)
        del self.lens[seq]

    def move_seqs(self, to: "BlockManager", seqs):
        """Swap out / in: move the sequences to another manager; each distinct block they use
        gets one block there in first-use order.  Returns the (here, there) pairs.  Refused
        (ValueError) if a block is also used by a sequence not in the list."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs) or any(s not in self.tables or s in to.tables
                                               for s in seqs):
            raise ValueError("bad sequence")
        if to.block_size != self.block_size:
            raise ValueError("block sizes differ")
        order, uses = [], {}
        for s in seqs:
            for b in self.tables[s]:
                if b not in uses:
                    order.append(b)
                    uses[b] = 0
                uses[b] += 1
        if any(uses[b] != self.ref[b] for b in order):
            raise ValueError("a block is shared with a sequence that is not moved")
        if len(order) > to.num_free():
            raise OutOfBlocks()
        mapping = {}
        for b in order:
            d = to._take()
            to.ref[d] = 0
            mapping[b] = d
        for s in seqs:
            table = self.tables.pop(s)
            to.tables[s] = [mapping[b] for b in table]
            to.lens[s] = self.lens.pop(s)
            for b in table:
                to.ref[mapping[b]] += 1
            for b in reversed(table):
                self._drop(b)
        return [(b, mapping[b]) for b in order]

    # -- queries -----------------------------------------------------------------------
    def num_free(self) -> int:
        """Blocks that can be handed out: plain free ones and parked cached ones."""
        return len(self._free) + len(self.parked)

    def num_cached(self) -> int:
        return len(self.cache)

    def block_table(self, seq: int) -> list[int]:
        return list(self.tables[seq])

    def seq_len(self, seq: int) -> int:
        return self.lens[seq]

    def wasted_slots(self) -> int:
        fill: dict[int, int] = {}
        for s, table in self.tables.items():
            L = self.lens[s]
            for j, b in enumerate(table):
                fill[b] = max(fill.get(b, 0), min(self.block_size, L - j * self.block_size))
        return sum(self.block_size - f for f in fill.values())
