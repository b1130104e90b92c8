"""The block-manager model (oracle/block_manager.py) pinned on its own,
with no C++ manager in the loop.

Pins:
  * the pages' worked allocator walk (tests/golden/worked_examples.json):
    a 30-token prompt takes 2 blocks of 16, the 33rd token a third
    ("PagedAttention: how vLLM manages the KV cache", section "Walk one
    request through the allocator");
  * copy-on-write: only the shared block about to be written is copied, the
    writer diverges, the other sharers keep the original; a fork at a block
    boundary copies nothing ("Why vLLM Uses PagedAttention", section "The
    bonus"; same page as above, section "Copy-on-write makes shared
    prefixes practical");
  * swapping moves each block once, keeps its sharers together and refuses
    to split a shared block from a sharer not listed ("PagedAttention -
    Virtual Memory for the KV Cache" explainer, chapter 05, card
    "Preemption & swapping");
  * what every one of these must preserve, checked by brute force over
    random operation streams: every sequence, read through its block table
    in the pool that holds it, returns exactly the tokens it was given, in
    order - the contents of every slot are simulated from the slots the
    model hands out, the copies it asks for and the blocks it swaps;
  * the bookkeeping invariants: a block's reference count is the number of
    table entries that hold it, and a block is free exactly when no table
    holds it.

Every pin takes the model class as an argument, so that
test_planted_mistake_in_the_model_is_caught can run them on a copy of the
model with one plausible mistake planted.
"""
import json
import os
import types

import numpy as np
import pytest

import oracle.block_manager as bmod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
REAL = (bmod.BlockManagerModel, bmod.OutOfBlocks, bmod.Refused)


# ---- the invariants and the content simulation ---------------------------

def check_invariants(m, nb, nh):
    """Reference counts are table references; free = unreferenced."""
    dev = [0] * nb
    host = [0] * nh
    for s, t in m.tables.items():
        for b in t:
            (host if s in m.swapped else dev)[b] += 1
    assert m.ref == dev, "device reference counts differ from table references"
    assert m.host_ref == host, "host reference counts differ from table references"
    assert sorted(m.free) == [b for b in range(nb) if dev[b] == 0]
    assert sorted(m.host_free) == [b for b in range(nh) if host[b] == 0]


class Contents:
    """Every slot's token, simulated from what the model hands out."""

    def __init__(self, nb, nh, bs):
        self.bs = bs
        self.dev = [[None] * bs for _ in range(nb)]
        self.host = [[None] * bs for _ in range(nh)]
        self.hist = {}
        self.next_id = 0

    def _new(self):
        self.next_id += 1
        return self.next_id

    def write(self, slot, tok):
        self.dev[slot // self.bs][slot % self.bs] = tok

    def add(self, seq, slots):
        self.hist[seq] = []
        for sl in slots:
            t = self._new()
            self.write(sl, t)
            self.hist[seq].append(t)

    def fork(self, parent, child):
        self.hist[child] = list(self.hist[parent])

    def append(self, seqs, slots, copies):
        for src, dst in copies:          # copies run before the writes
            self.dev[dst] = list(self.dev[src])
        for s, sl in zip(seqs, slots):
            t = self._new()
            self.write(sl, t)
            self.hist[s].append(t)

    def swap(self, pairs, to_host):
        src, dst = (self.dev, self.host) if to_host else (self.host, self.dev)
        for a, b in pairs:
            dst[b] = list(src[a])

    def check(self, m):
        for s, h in self.hist.items():
            pool = self.host if s in m.swapped else self.dev
            t = m.tables[s]
            view = [pool[t[i // self.bs]][i % self.bs] for i in range(m.tokens[s])]
            assert view == h, f"sequence {s} reads {view} through its table, wrote {h}"


def random_stream(M, seed, nb=24, nh=16, bs=4, steps=300):
    """Random adds, forks, appends, frees and swaps; after each, every
    sequence reads back its own tokens and the invariants hold."""
    Model, OutOfBlocks, Refused = M
    rng = np.random.default_rng([88, seed])
    m = Model(nb, bs, nh)
    c = Contents(nb, nh, bs)
    nxt = 0
    for _ in range(steps):
        live = sorted(m.tables)
        dev_live = [s for s in live if s not in m.swapped]
        op = rng.choice(["add", "fork", "append", "append", "append", "free",
                         "out", "in"])
        try:
            if op == "add" or not live:
                slots = m.add_sequence(nxt, int(rng.integers(1, 3 * bs)))
                c.add(nxt, slots)
                nxt += 1
            elif op == "fork" and dev_live:
                p = int(rng.choice(dev_live))
                m.fork(p, nxt)
                c.fork(p, nxt)
                nxt += 1
            elif op == "append" and dev_live:
                k = int(rng.integers(1, len(dev_live) + 1))
                seqs = [int(x) for x in rng.choice(dev_live, size=k, replace=False)]
                slots, copies = m.append_tokens(seqs)
                c.append(seqs, slots, copies)
            elif op == "free":
                s = int(rng.choice(live))
                m.free_sequence(s)
                del c.hist[s]
            elif op == "out" and dev_live:
                k = int(rng.integers(1, min(3, len(dev_live)) + 1))
                seqs = [int(x) for x in rng.choice(dev_live, size=k, replace=False)]
                c.swap(m.swap_out(seqs), True)
            elif op == "in" and m.swapped:
                sw = sorted(m.swapped)
                k = int(rng.integers(1, min(3, len(sw)) + 1))
                seqs = [int(x) for x in rng.choice(sw, size=k, replace=False)]
                c.swap(m.swap_in(seqs), False)
        except (OutOfBlocks, Refused):
            pass
        check_invariants(m, nb, nh)
        c.check(m)


# ---- the pins --------------------------------------------------------------

def pin_allocator_walk(M):
    Model = M[0]
    ex = json.load(open(GOLDEN))["allocator_walk"]
    bs = ex["block_size"]
    m = Model(16, bs)
    m.add_sequence(0, ex["prompt_tokens"])
    assert len(m.tables[0]) == ex["blocks_after_prompt"]
    assert ex["prompt_tokens"] - (len(m.tables[0]) - 1) * bs == \
        ex["tokens_in_second_block_after_prompt"]
    for _ in range(ex["empty_positions_after_prompt"]):
        _, copies = m.append_tokens([0])
        assert copies == []
    assert len(m.tables[0]) == ex["blocks_after_prompt"]   # filled, no new block
    assert m.tokens[0] == ex["tokens_when_second_block_full"]
    m.append_tokens([0])
    assert len(m.tables[0]) == ex["blocks_at_33_tokens"]
    m.append_tokens([0])
    assert m.tokens[0] == ex["final_tokens"]
    assert len(m.tables[0]) == ex["final_blocks"]
    assert m.tokens[0] - (ex["final_blocks"] - 1) * bs == \
        ex["live_positions_in_last_block"]
    assert m.num_free_blocks() == 16 - ex["final_blocks"]


def pin_only_the_written_block_is_copied(M):
    Model = M[0]
    bs = 16
    m = Model(32, bs)
    m.add_sequence(0, 3 * bs + 5)            # 3 full blocks + 1 partial
    for ch in range(1, 5):
        m.fork(0, ch)                        # 5 sharers
    shared = list(m.tables[0])
    assert all(m.ref[b] == 5 for b in shared)
    free0 = m.num_free_blocks()
    slots, copies = m.append_tokens([0, 1, 2, 3, 4])
    assert len(copies) == 4                  # 5 writers: the last keeps the original
    assert all(src == shared[3] for src, _ in copies)
    assert len({dst for _, dst in copies}) == 4
    assert m.num_free_blocks() == free0 - 4
    lasts = [m.tables[i][3] for i in range(5)]
    for i in range(5):
        assert m.tables[i][:3] == shared[:3]  # full blocks still shared
    assert len(set(lasts)) == 5 and shared[3] in lasts
    assert m.ref[shared[0]] == 5 and m.ref[shared[3]] == 1
    assert sorted(s % bs for s in slots) == [5] * 5
    assert sorted(s // bs for s in slots) == sorted(lasts)


def pin_fork_at_a_block_boundary_copies_nothing(M):
    Model = M[0]
    bs = 16
    m = Model(16, bs)
    m.add_sequence(0, 2 * bs)
    m.fork(0, 1)
    slots, copies = m.append_tokens([0, 1])
    assert copies == []
    assert slots[0] // bs != slots[1] // bs
    assert m.tables[0][:2] == m.tables[1][:2] and m.ref[m.tables[0][0]] == 2


def pin_free_returns_unshared_blocks_only(M):
    Model = M[0]
    m = Model(8, 4)
    m.add_sequence(0, 8)                     # blocks 0, 1
    m.fork(0, 1)
    m.free_sequence(0)
    assert m.num_free_blocks() == 6          # the fork still holds 0 and 1
    m.free_sequence(1)
    assert m.num_free_blocks() == 8
    slots = m.add_sequence(2, 5)             # the freed blocks come back
    assert sorted({s // 4 for s in slots}) == [0, 1]


def pin_swap_keeps_sharers_and_refuses_to_split_them(M):
    Model, OutOfBlocks, Refused = M
    bs = 4
    m = Model(16, bs, 16)
    m.add_sequence(0, 10)                    # 3 blocks, the last partial
    m.fork(0, 1)
    m.fork(0, 2)
    m.add_sequence(3, 5)
    _, copies = m.append_tokens([1])         # 1 diverges in its last block
    assert len(copies) == 1
    with pytest.raises(Refused):
        m.swap_out([0, 1])                   # 2 still shares 0's blocks
    assert len(m.host_free) == 16 and not m.swapped
    blocks = {b for s in (0, 1, 2) for b in m.tables[s]}
    pairs = m.swap_out([1, 0, 2, 1])
    assert len(pairs) == len(blocks) == 4    # each distinct block once
    assert {a for a, _ in pairs} == blocks
    for s in (0, 1, 2):
        assert s in m.swapped
    host_shared = m.tables[0][0]
    assert m.tables[1][0] == m.tables[2][0] == host_shared
    assert m.host_ref[host_shared] == 3
    back = m.swap_in([2, 0, 1])
    assert len(back) == 4 and not m.swapped
    assert m.tables[0][:2] == m.tables[1][:2] == m.tables[2][:2]
    assert m.ref[m.tables[0][0]] == 3 and len(m.host_free) == 16


def pin_random_streams(M, seeds=range(12)):
    for seed in seeds:
        random_stream(M, seed)


PINS = [pin_allocator_walk, pin_only_the_written_block_is_copied,
        pin_fork_at_a_block_boundary_copies_nothing,
        pin_free_returns_unshared_blocks_only,
        pin_swap_keeps_sharers_and_refuses_to_split_them, pin_random_streams]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(REAL)


@pytest.mark.parametrize("seed", range(12, 40))
def test_random_streams_keep_every_sequence_readable(seed):
    random_stream(REAL, seed)


# ---- planted mistakes in the model ------------------------------------------

MUTANTS = {
    "no_copy_before_writing_a_shared_block": (
        "if self.ref[last] > 1:", "if False:"),
    "copy_pair_reversed": ("copy = (last, fresh)", "copy = (fresh, last)"),
    "count_not_decremented_on_copy": (
        "                self.ref[last] -= 1\n", "                pass\n"),
    "fresh_block_one_token_late": (
        "if t % self.block_size == 0:", "if t % self.block_size == 1:"),
    "fork_does_not_count_the_child": (
        "        for b in self.tables[child]:\n            self.ref[b] += 1",
        "        for b in self.tables[child]:\n            pass"),
    "free_ignores_the_count": ("            if ref[b] == 0:", "            if True:"),
    "swap_splits_sharers": (
        "            if holders != src_ref[b]:", "            if False:"),
    "swap_drops_the_count": ("dst_ref[nb] = src_ref[b]", "dst_ref[nb] = 1"),
    "swap_moves_a_shared_block_twice": (
        "                if b not in blocks:\n                    blocks.append(b)",
        "                blocks.append(b)"),
}


def mutated_model(name):
    old, new = MUTANTS[name]
    src = open(bmod.__file__).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    mod = types.ModuleType(f"mutant_{name}")
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod.BlockManagerModel, mod.OutOfBlocks, mod.Refused


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_in_the_model_is_caught(name):
    M = mutated_model(name)
    caught = 0
    for pin in PINS:
        try:
            pin(M)
        except (AssertionError, pytest.fail.Exception, IndexError, KeyError,
                ValueError):
            caught += 1
            break
        except (M[1], M[2]):      # the mutant refused or ran dry where it must not
            caught += 1
            break
    assert caught, f"no pin caught the planted mistake {name}"
