"""Structure of the seeded inputs: block placement, tables, slots, sharing,
length recipes and determinism."""
import math

import numpy as np
import pytest

import workloads as wl


def check_structure(w: wl.Workload, shared_prefix_blocks: int = 0):
    bs = w.block_size
    S = w.num_seqs
    assert w.block_tables.shape == (S, w.max_blocks_per_seq)
    used = []
    for s in range(S):
        L = int(w.context_lens[s])
        nb = -(-L // bs)
        row = w.block_tables[s]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < w.num_blocks)
        assert np.all(row[nb:] == -1)            # unused entries are -1
        used.append(row[shared_prefix_blocks:nb])
        assert len(w.token_rows[s]) == L
    own = np.concatenate(used) if used else np.zeros(0, np.int32)
    # private blocks are distinct and disjoint from the shared prefix
    pref = w.block_tables[0, :shared_prefix_blocks] if S else []
    assert len(np.unique(own)) == len(own)
    assert not np.intersect1d(own, pref).size
    # every token's slot is inside its table's block, and slots are unique
    assert len(np.unique(w.kv_slots)) == len(w.kv_slots)
    for s in range(S):
        t = np.arange(int(w.context_lens[s]))
        sl = w.kv_slots[w.token_rows[s]]
        assert np.array_equal(sl // bs, w.block_tables[s, t // bs])
        assert np.array_equal(sl % bs, t % bs)
    # refcounts count table references
    ref = np.zeros(w.num_blocks, np.int64)
    for s in range(S):
        nb = -(-int(w.context_lens[s]) // bs)
        np.add.at(ref, w.block_tables[s, :nb], 1)
    assert np.array_equal(ref, w.refcount)


def test_tiny_config():
    for seed in range(10):
        w = wl.tiny(seed)
        assert list(w.context_lens) == [5, 16, 17, 40]
        assert w.num_blocks == 16 and w.dtype == "f32" and w.head_dim == 64
        check_structure(w)
        # new tokens at positions 4, 15, 16, 39
        pos = [int(np.where(w.token_rows[s] == w.new_rows[s])[0][0])
               for s in range(4)]
        assert pos == [4, 15, 16, 39]
    # different seeds place blocks differently
    assert not np.array_equal(wl.tiny(0).block_tables, wl.tiny(1).block_tables)


def test_mha_pool_is_twice_the_need_and_lengths_in_range():
    w = wl.build("m", lens=np.random.default_rng(0).integers(128, 2048, 6,
                                                              endpoint=True),
                 num_heads=2, num_kv_heads=2, head_dim=8, block_size=16,
                 dtype="f16", seed=0, pool_factor=2.0)
    need = sum(-(-int(L) // 16) for L in w.context_lens)
    assert w.num_blocks == 2 * need
    check_structure(w)


def test_gqa_lengths_lognormal_recipe():
    w = wl.gqa70b(0, num_seqs=16)
    check_structure(w)
    assert w.num_heads == 64 and w.num_kv_heads == 8
    assert w.context_lens.min() >= 1 and w.context_lens.max() <= 8192
    # the recipe: clamp(round(exp(ln 1024 + sigma * z)), 1, 8192), z drawn
    # first from the seed's generator
    z = np.random.default_rng(0).standard_normal(16)
    want = np.clip(np.rint(np.exp(math.log(1024) + wl.GQA_SIGMA * z)), 1, 8192)
    assert np.array_equal(w.context_lens, want.astype(np.int32))


def test_long_context_outlier_keys():
    w = wl.long_split(0, num_seqs=2, ctx=1000)
    check_structure(w)
    base = wl.build("ref", lens=[1000, 1000], num_heads=32, num_kv_heads=32,
                    head_dim=128, block_size=16, dtype="bf16", seed=0,
                    max_blocks_per_seq=63,
                    rng=np.random.default_rng(0))
    kf = wl.storage_to_f32(w.kv_k, "bf16")
    kb = wl.storage_to_f32(base.kv_k, "bf16")
    for s in range(2):
        rows = w.token_rows[s]
        changed = np.any(kf[rows] != kb[rows], axis=(1, 2))
        assert changed.sum() == 10                    # floor(1% of 1000)
        r = rows[changed]
        assert np.array_equal(kf[r], kb[r] * 8)       # exact power of two


@pytest.mark.parametrize("bs", [16, 32])
def test_shared_prefix_blocks(bs):
    w = wl.shared_prefix(0, block_size=bs, num_seqs=6)
    pb = 1024 // bs
    check_structure(w, shared_prefix_blocks=pb)
    assert np.all(w.block_tables[:, :pb] == w.block_tables[0, :pb])
    assert np.all(w.refcount[w.block_tables[0, :pb]] == 6)
    # the written slot of the step lies in a block only its sequence holds
    new_blocks = w.new_slots() // bs
    assert np.all(w.refcount[new_blocks] == 1)
    # suffix lengths in [16, 512]
    assert np.all((w.context_lens >= 1040) & (w.context_lens <= 1536))


def test_zero_length_sequences_have_no_new_token():
    w = wl.build("z", lens=[0, 5, 0], num_heads=1, num_kv_heads=1,
                 head_dim=8, block_size=4, dtype="f32", seed=0,
                 max_blocks_per_seq=2)
    assert list(w.new_slots()[[0, 2]]) == [-1, -1]
    assert w.new_k().shape == (3, 1, 8)
    check_structure(w)


def test_chunked_draws_do_not_depend_on_thread_count(monkeypatch):
    n = 3 * (1 << 20) + 17
    a = wl.normal(n, "bf16", 5, 2)
    monkeypatch.setattr(wl, "_threads", lambda: 1)
    b = wl.normal(n, "bf16", 5, 2)
    assert np.array_equal(a, b)
    assert not np.array_equal(a[:100], wl.normal(100, "bf16", 6, 2))


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -2.00390625, 3.0]  # ties and exact
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(wl.f32_to_storage(x, "bf16").view(np.int16), want)
