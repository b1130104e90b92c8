"""The host planner of the shared-prefix decode (pkv_prefix_plan), on the
CPU: integer work, compared exactly with a plain statement of its rule.

The rule: sequences with at least one full block whose first table entry
is the same physical block form one set (sets in order of their first
member, members in sequence order); a set's prefix is the largest k such
that every member has k full blocks in its context and all members' first
k entries agree; sets of fewer than min_sharers members are dropped.
"""
import ctypes

import numpy as np
import pytest

from paged_kv_cache_309_amd import _lib

ERR = {v: k for k, v in _lib.STATUS.items()}


def plan(bt, cl, bs, min_sharers=2, capacity=None):
    bt = np.ascontiguousarray(bt, np.int32)
    cl = np.ascontiguousarray(cl, np.int32)
    S, MB = bt.shape
    cap = 4 * S + 1 if capacity is None else capacity
    out = np.full(max(cap, 1), -7, np.int32)
    info = _lib.PkvPrefixInfo()
    rc = _lib.lib().pkv_prefix_plan(bt.ctypes.data, cl.ctypes.data, S, MB, bs,
                                    min_sharers, out.ctypes.data, cap,
                                    ctypes.byref(info))
    return rc, out, info


def expected(bt, cl, bs, min_sharers=2):
    """The rule written out, scanning all members at once."""
    S, MB = bt.shape
    full = [min(max(int(L), 0) // bs, MB) for L in cl]
    keys, sets = [], {}
    for s in range(S):
        if full[s] < 1:
            continue
        key = int(bt[s, 0])
        if key not in sets:
            sets[key] = []
            keys.append(key)
        sets[key].append(s)
    seq_prefix = [0] * S
    starts, tokens, members = [0], [], []
    for key in keys:
        mem = sets[key]
        if len(mem) < min_sharers:
            continue
        k = 0
        while k < min(full[m] for m in mem) and \
                all(bt[m, k] == bt[mem[0], k] for m in mem):
            k += 1
        for m in mem:
            seq_prefix[m] = k * bs
        members += mem
        starts.append(len(members))
        tokens.append(k * bs)
    return seq_prefix + starts + tokens + members, len(tokens), len(members), \
        max([len(sets[k]) for k in keys if len(sets[k]) >= min_sharers], default=0), \
        max(tokens, default=0)


def check(bt, cl, bs, min_sharers=2):
    rc, out, info = plan(bt, cl, bs, min_sharers)
    assert rc == 0, _lib.STATUS.get(rc)
    arr, G, M, maxm, maxt = expected(bt, cl, bs, min_sharers)
    assert out[:len(arr)].tolist() == arr
    assert np.all(out[len(arr):] == -7)   # nothing written past the plan
    assert (info.num_seqs, info.num_groups, info.num_members, info.max_members,
            info.max_prefix_tokens) == (bt.shape[0], G, M, maxm, maxt)
    return out[:len(arr)], info


def forked_tables(rng, S, bs, max_blocks, fresh):
    """Tables built the way forks and shared system prompts build them:
    sequence s copies the first k entries of an earlier sequence's table
    (or starts afresh) and appends blocks of its own."""
    bt = np.full((S, max_blocks), -1, np.int32)
    cl = np.zeros(S, np.int32)
    nxt = 0
    for s in range(S):
        if s > 0 and rng.random() < 0.8:
            src = int(rng.integers(0, s))
            k = int(rng.integers(0, max(1, cl[src] // bs) + 1))
            bt[s, :k] = bt[src, :k]
        else:
            k = 0
        n = int(rng.integers(k, max_blocks + 1))
        for j in range(k, n):
            bt[s, j] = fresh[nxt]
            nxt += 1
        lo = max(k * bs, 1) if n else 0
        cl[s] = int(rng.integers(lo, max(lo, n * bs) + 1)) if n else 0
    return bt, cl


@pytest.mark.parametrize("seed", range(40))
def test_random_forest_of_forks(seed):
    rng = np.random.default_rng([610, seed])
    bs = int(rng.choice([16, 32]))
    S = int(rng.integers(1, 60))
    MB = int(rng.integers(1, 12))
    fresh = rng.permutation(100000).astype(np.int32)
    bt, cl = forked_tables(rng, S, bs, MB, fresh)
    for ms in (2, 3, 5):
        check(bt, cl, bs, ms)


def test_one_set_of_all_sequences():
    # 128 sequences over one 64-block prefix, suffixes of their own
    rng = np.random.default_rng(3)
    S, bs, pb = 128, 16, 64
    lens = 1024 + rng.integers(16, 513, S)
    MB = int(-(-lens.max() // bs))
    ids = rng.permutation(100000).astype(np.int32)
    bt = np.full((S, MB), -1, np.int32)
    bt[:, :pb] = ids[:pb]
    nxt = pb
    for s in range(S):
        n = -(-int(lens[s]) // bs)
        bt[s, pb:n] = ids[nxt:nxt + n - pb]
        nxt += n - pb
    out, info = check(bt, lens, bs)
    assert info.num_groups == 1 and info.num_members == S
    assert info.max_prefix_tokens == 1024
    assert np.all(out[:S] == 1024)


def test_worked_cases():
    bs = 16
    bt = np.array([[5, 6, 7, -1], [5, 6, 9, 10], [1, 2, 3, 4], [5, 6, 7, 8],
                   [1, 2, 0, -1], [8, 3, -1, -1]], np.int32)
    cl = np.array([40, 60, 64, 60, 40, 20], np.int32)
    out, info = check(bt, cl, bs)
    # {0, 1, 3} share [5, 6] (sequence 0 holds two full blocks); {2, 4}
    # share [1, 2]; sequence 5 shares nothing
    assert out.tolist() == [32, 32, 32, 32, 32, 0,   # seq_prefix
                            0, 3, 5,                 # starts
                            32, 32,                  # tokens
                            0, 1, 3, 2, 4]           # members
    # a sequence shorter than one block joins no set
    cl2 = cl.copy()
    cl2[4] = 15
    out, info = check(bt, cl2, bs)
    assert info.num_groups == 1 and out[4] == 0
    # min_sharers 3 keeps the first set only
    out, info = check(bt, cl, bs, 3)
    assert info.num_groups == 1 and info.num_members == 3
    # a partly filled shared block is not part of the prefix
    bt3 = np.array([[4, 5, -1], [4, 5, -1]], np.int32)
    out, info = check(bt3, np.array([20, 31], np.int32), bs)
    assert out[:2].tolist() == [16, 16]


def test_no_sharing_and_empty_batch():
    bt = np.arange(12, dtype=np.int32).reshape(4, 3)
    out, info = check(bt, np.array([48, 48, 10, 0], np.int32), 16)
    assert info.num_groups == 0 and out.tolist() == [0, 0, 0, 0, 0]
    rc, out, info = plan(np.zeros((0, 4), np.int32), np.zeros(0, np.int32), 16)
    assert rc == 0 and info.num_groups == 0 and out[0] == 0


def test_errors():
    bt = np.zeros((3, 2), np.int32)
    cl = np.full(3, 32, np.int32)
    assert plan(bt, cl, 16, capacity=3)[0] == ERR["PKV_ERR_CAPACITY"]
    assert plan(bt, cl, 16, capacity=4 + 2 + 3)[0] == 0   # S + 2G + 1 + M
    assert plan(bt, cl, 16, capacity=4 + 2 + 2)[0] == ERR["PKV_ERR_CAPACITY"]
    assert plan(bt, cl, 16, min_sharers=1)[0] == ERR["PKV_ERR_SHAPE"]
    assert plan(bt, cl, 0)[0] == ERR["PKV_ERR_BLOCK_SIZE"]
    info = _lib.PkvPrefixInfo()
    out = np.zeros(16, np.int32)
    assert _lib.lib().pkv_prefix_plan(None, cl.ctypes.data, 3, 2, 16, 2,
                                      out.ctypes.data, 16,
                                      ctypes.byref(info)) == ERR["PKV_ERR_NULL"]
    assert _lib.lib().pkv_prefix_plan(bt.ctypes.data, cl.ctypes.data, -1, 2, 16,
                                      2, out.ctypes.data, 16,
                                      ctypes.byref(info)) == ERR["PKV_ERR_SHAPE"]
