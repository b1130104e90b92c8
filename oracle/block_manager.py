"""Plain model of the paged KV block manager.

TEST INFRASTRUCTURE: only the tests import this module.  It shares no code
with the library's C++ block manager; it restates, in the simplest Python,
what the pages say the manager does:

  * the KV cache is cut into fixed-size blocks; a sequence's block table
    maps its logical blocks to physical blocks ("Why vLLM Uses
    PagedAttention", section "The mechanism");
  * blocks are allocated on demand: a new block only when the token count
    crosses a block boundary ("PagedAttention - Virtual Memory for the KV
    Cache" explainer, chapter "The Block Table"; "PagedAttention: how vLLM
    manages the KV cache", section "Walk one request through the allocator");
  * blocks come from a global free list and go back to it when the request
    finishes ("Paged Attention" placement notes, section "Paged Attention's
    Approach");
  * sequences that overlap point at the same physical blocks, a reference
    count tracks the sharers, and a shared block that needs a write is
    copied first, the count decremented and the writer diverges; only the
    block being written is copied ("Why vLLM Uses PagedAttention", section
    "The bonus"; "PagedAttention: how vLLM manages the KV cache", section
    "Copy-on-write makes shared prefixes practical": the other branch keeps
    the original);
  * under memory pressure a request can be swapped out and later brought
    back, like an evicted page ("PagedAttention - Virtual Memory for the KV
    Cache" explainer, chapter 05, card "Preemption & swapping"; deep dive,
    card "What Indirection Buys").  Swapped-out sequences sit in a second,
    host-side pool of blocks; every block they hold moves once, keeping its
    sharers.

Conventions fixed here (the pages leave them open): the free list is
a stack whose initial order hands out blocks 0, 1, 2, ...; a finished
sequence returns its blocks in reverse table order; a batch of appends is
served in order and either succeeds whole or changes nothing.  A swap moves
the distinct blocks of the listed sequences in order of first appearance,
each into the next free block of the other pool, and returns the old blocks
so that the first one moved is the next one handed out; it refuses to split
a shared block from a sharer that is not listed.
"""
from __future__ import annotations


class OutOfBlocks(Exception):
    pass


class Refused(Exception):
    """An operation the model refuses (the C++ manager returns a status)."""


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int,
                 num_host_blocks: int = 0):
        self.block_size = block_size
        self.free = list(range(num_blocks))[::-1]   # top of the stack = end
        self.ref = [0] * num_blocks
        self.host_free = list(range(num_host_blocks))[::-1]
        self.host_ref = [0] * num_host_blocks
        self.tables: dict[int, list[int]] = {}
        self.tokens: dict[int, int] = {}
        self.swapped: set[int] = set()

    # -- helpers -------------------------------------------------------------
    def _take(self) -> int:
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def slot(self, seq: int, t: int) -> int:
        return self.tables[seq][t // self.block_size] * self.block_size + \
            t % self.block_size

    # -- operations ----------------------------------------------------------
    def add_sequence(self, seq: int, num_tokens: int) -> list[int]:
        if seq in self.tables:
            raise KeyError("exists")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise OutOfBlocks
        self.tables[seq] = [self._take() for _ in range(need)]
        self.tokens[seq] = num_tokens
        return [self.slot(seq, t) for t in range(num_tokens)]

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables:
            raise KeyError("unknown")
        if child in self.tables:
            raise KeyError("exists")
        if parent in self.swapped:
            raise Refused("swapped")
        self.tables[child] = list(self.tables[parent])
        self.tokens[child] = self.tokens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def _append_one(self, seq: int):
        t = self.tokens[seq]
        copy = None
        if t % self.block_size == 0:
            self.tables[seq].append(self._take())
        else:
            last = self.tables[seq][-1]
            if self.ref[last] > 1:          # shared: copy before writing
                fresh = self._take()
                self.ref[last] -= 1
                self.tables[seq][-1] = fresh
                copy = (last, fresh)
        self.tokens[seq] = t + 1
        return self.slot(seq, t), copy

    def append_tokens(self, seqs):
        for s in seqs:
            if s not in self.tables:
                raise KeyError("unknown")
            if s in self.swapped:
                raise Refused("swapped")
        # all or nothing: run the batch on a copy first
        snapshot = (list(self.free), list(self.ref),
                    {k: list(v) for k, v in self.tables.items()},
                    dict(self.tokens))
        slots, copies = [], []
        try:
            for s in seqs:
                slot, copy = self._append_one(s)
                slots.append(slot)
                if copy is not None:
                    copies.append(copy)
        except IndexError:                     # the free list ran dry
            self.free, self.ref, self.tables, self.tokens = snapshot
            raise OutOfBlocks from None
        return slots, copies

    def free_sequence(self, seq: int) -> None:
        if seq not in self.tables:
            raise KeyError("unknown")
        ref, free = ((self.host_ref, self.host_free) if seq in self.swapped
                     else (self.ref, self.free))
        for b in reversed(self.tables[seq]):
            ref[b] -= 1
            if ref[b] == 0:
                free.append(b)
        del self.tables[seq]
        del self.tokens[seq]
        self.swapped.discard(seq)

    def _move(self, seqs, to_host: bool):
        ids = []
        for s in seqs:
            if s not in self.tables:
                raise KeyError("unknown")
            if (s in self.swapped) == to_host:
                raise Refused("swapped")
            if s not in ids:
                ids.append(s)
        if to_host:
            src_ref, src_free = self.ref, self.free
            dst_ref, dst_free = self.host_ref, self.host_free
        else:
            src_ref, src_free = self.host_ref, self.host_free
            dst_ref, dst_free = self.ref, self.free
        blocks = []
        for s in ids:
            for b in self.tables[s]:
                if b not in blocks:
                    blocks.append(b)
        for b in blocks:
            holders = sum(t.count(b) for s, t in self.tables.items()
                          if s in ids)
            if holders != src_ref[b]:
                raise Refused("shared with a sequence not listed")
        if len(blocks) > len(dst_free):
            raise OutOfBlocks
        new = {}
        for b in blocks:
            nb = dst_free.pop()
            dst_ref[nb] = src_ref[b]
            new[b] = nb
        for s in ids:
            self.tables[s] = [new[b] for b in self.tables[s]]
            if to_host:
                self.swapped.add(s)
            else:
                self.swapped.discard(s)
        for b in reversed(blocks):
            src_ref[b] = 0
            src_free.append(b)
        return [(b, new[b]) for b in blocks]

    def swap_out(self, seqs):
        """(device block, host block) pairs to copy."""
        return self._move(seqs, True)

    def swap_in(self, seqs):
        """(host block, device block) pairs to copy."""
        return self._move(seqs, False)

    def num_free_blocks(self) -> int:
        return len(self.free)
