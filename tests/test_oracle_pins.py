"""Pins of the oracle to things other than itself.

Each test checks the oracle (``oracle/``) against a fact fixed by the pages
or by mathematics: ordinary contiguous attention computed by NumPy/SciPy on
an un-paged copy of the keys and values, invariance under any physical
placement of the blocks, closed forms (identical keys, one-hot probes, a
single token), the worked examples printed on the pages, a NumPy-view
formulation of the cache write, and a library decoding of fp16/bf16.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "worked_examples.json")


# ---------------------------------------------------------------- helpers --

def lib_widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of a storage array through NumPy/torch conversions
    (not the oracle's decoders)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.view(torch.bfloat16).to(torch.float64).numpy()
    return np.asarray(a).astype(np.float64)


def oracle_pool(w: wl.Workload, slots=None):
    kc, vc = oracle.new_pool(w.num_blocks, w.num_kv_heads, w.block_size,
                             w.head_dim, w.dtype)
    oracle.reshape_and_cache(w.kv_k, w.kv_v, kc, vc,
                             w.kv_slots if slots is None else slots,
                             w.num_kv_heads, w.head_dim, w.block_size,
                             w.num_blocks, w.dtype)
    return kc, vc


def oracle_decode(w: wl.Workload, kc, vc, tables=None, lens=None, q=None,
                  threads=None):
    return oracle.paged_decode(
        w.q if q is None else q, kc, vc,
        w.block_tables if tables is None else tables,
        w.context_lens if lens is None else lens, w.scale, w.block_size,
        w.num_kv_heads, w.num_blocks, w.dtype, threads=threads)


def brute(w: wl.Workload, q=None, kv_k=None, kv_v=None) -> np.ndarray:
    """Ordinary attention on the un-paged, logically contiguous K/V of each
    sequence: softmax(K q * scale) @ V, KV heads repeated for GQA."""
    q = lib_widen(w.q if q is None else q, w.dtype)
    kk = lib_widen(w.kv_k if kv_k is None else kv_k, w.dtype)
    vv = lib_widen(w.kv_v if kv_v is None else kv_v, w.dtype)
    G = w.num_heads // w.num_kv_heads
    scale = np.float64(np.float32(w.scale))
    out = np.zeros((w.num_seqs, w.num_heads, w.head_dim))
    for s in range(w.num_seqs):
        rows = w.token_rows[s]
        if len(rows) == 0:
            continue
        K = np.repeat(kk[rows], G, axis=1)  # [L, Hq, D]
        V = np.repeat(vv[rows], G, axis=1)
        for h in range(w.num_heads):
            logits = (K[:, h, :] @ q[s, h]) * scale
            p = scipy.special.softmax(logits)
            out[s, h] = p @ V[:, h, :]
    return out


SWEEP = [
    # (dtype, block_size, Hq, Hkv, D, S, max_len)
    ("f32", 16, 2, 2, 64, 4, 60),
    ("f32", 4, 4, 1, 8, 5, 33),
    ("f16", 8, 8, 2, 64, 6, 100),
    ("f16", 16, 4, 4, 128, 3, 70),
    ("bf16", 32, 8, 1, 64, 4, 100),
    ("bf16", 16, 16, 2, 128, 3, 90),
    ("bf16", 12, 6, 3, 8, 5, 50),
]


# ----------------------------------------------------------------- pins ----

@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_matches_contiguous_attention(case):
    """Paging keeps the computation of ordinary attention ("PagedAttention:
    how vLLM manages the KV cache", section "PagedAttention changes
    addressing inside attention")."""
    dtype, bs, Hq, Hkv, D, S, max_len = SWEEP[case]
    w = wl.random_case(100 + case, num_seqs=S, max_len=max_len, num_heads=Hq,
                       num_kv_heads=Hkv, head_dim=D, block_size=bs,
                       dtype=dtype)
    kc, vc = oracle_pool(w)
    got = oracle_decode(w, kc, vc)
    want = brute(w)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_zero_length_gives_zeros():
    w = wl.build("z", lens=[0, 3, 0], num_heads=2, num_kv_heads=1,
                 head_dim=8, block_size=4, dtype="f32", seed=1,
                 max_blocks_per_seq=2)
    kc, vc = oracle_pool(w)
    got = oracle_decode(w, kc, vc)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert np.max(np.abs(got[1] - brute(w)[1])) <= 1e-12


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_physical_permutation_is_bitwise_invariant(dtype):
    """Correctness does not depend on where blocks live (the explainer's
    "The Block Table" chapter: attention walks the table, independent of
    layout).  The same logical order gives the same double operations, so
    the result is bit-identical."""
    w = wl.random_case(7, num_seqs=6, max_len=120, num_heads=4,
                       num_kv_heads=2, head_dim=64, block_size=16,
                       dtype=dtype, pool_factor=2.0)
    kc, vc = oracle_pool(w)
    base = oracle_decode(w, kc, vc)
    rng = np.random.default_rng(9)
    for _ in range(3):
        perm = rng.permutation(w.num_blocks)
        bs = w.block_size
        slots = np.where(w.kv_slots >= 0,
                         perm[w.kv_slots // bs] * bs + w.kv_slots % bs, -1)
        tables = np.where(w.block_tables >= 0,
                          perm[np.maximum(w.block_tables, 0)], -1)
        kc2, vc2 = oracle_pool(w, slots=slots)
        got = oracle_decode(w, kc2, vc2, tables=tables.astype(np.int32))
        assert np.array_equal(got, base)


def test_identical_keys_give_mean_of_values():
    """All logits equal: every weight is 1/L, so the output is the plain
    mean of the sequence's values."""
    w = wl.random_case(11, num_seqs=5, max_len=80, num_heads=4,
                       num_kv_heads=4, head_dim=64, block_size=16,
                       dtype="bf16", min_len=1)
    w.kv_k[:] = w.kv_k[0]
    kc, vc = oracle_pool(w)
    got = oracle_decode(w, kc, vc)
    vv = lib_widen(w.kv_v, w.dtype)
    for s in range(w.num_seqs):
        want = vv[w.token_rows[s]].mean(axis=0)  # [Hkv=Hq, D]
        assert np.max(np.abs(got[s] - want)) <= 1e-12


def one_hot_probe(w: wl.Workload, probe_pos: np.ndarray):
    """q = e_0 for every head; every key zero except the probed token's
    first component, 16384.  The probed logit exceeds the rest by
    16384*scale, far past the point where exp() underflows to 0, so the
    weights are exactly one and zeros and the output is exactly v_j."""
    q = np.zeros_like(w.q)
    one = wl.f32_to_storage(np.float32([1.0]), w.dtype)[0]
    big = wl.f32_to_storage(np.float32([16384.0]), w.dtype)[0]
    q[:, :, 0] = one
    kk = np.zeros_like(w.kv_k)
    for s in range(w.num_seqs):
        if w.context_lens[s] > 0:
            kk[w.token_rows[s][probe_pos[s]], :, 0] = big
    return q, kk


def test_one_hot_probe_every_position_bit_exact():
    """Block-table indexing, bit-exact: the probe recovers the value of the
    exact token it marks, for every token position of the tiny config."""
    for seed in range(3):
        w = wl.tiny(seed)
        G = w.num_heads // w.num_kv_heads
        vv = lib_widen(w.kv_v, w.dtype)
        for i in range(int(w.context_lens.max())):
            pos = np.minimum(i, w.context_lens - 1)
            q, kk = one_hot_probe(w, pos)
            kc, vc = oracle.new_pool(w.num_blocks, w.num_kv_heads,
                                     w.block_size, w.head_dim, w.dtype)
            oracle.reshape_and_cache(kk, w.kv_v, kc, vc, w.kv_slots,
                                     w.num_kv_heads, w.head_dim,
                                     w.block_size, w.num_blocks, w.dtype)
            got = oracle_decode(w, kc, vc, q=q)
            for s in range(w.num_seqs):
                row = w.token_rows[s][pos[s]]
                for h in range(w.num_heads):
                    assert np.array_equal(got[s, h], vv[row, h // G])


def test_single_token_returns_its_value_exactly():
    w = wl.build("one", lens=[1, 1, 1], num_heads=4, num_kv_heads=2,
                 head_dim=64, block_size=16, dtype="f16", seed=3,
                 pool_factor=3.0)
    kc, vc = oracle_pool(w)
    got = oracle_decode(w, kc, vc)
    vv = lib_widen(w.kv_v, w.dtype)
    for s in range(3):
        assert np.array_equal(got[s], np.repeat(vv[w.token_rows[s][0]], 2,
                                                axis=0))


def test_thread_count_does_not_change_result():
    w = wl.random_case(21, num_seqs=7, max_len=90, num_heads=4,
                       num_kv_heads=2, head_dim=64, block_size=16,
                       dtype="bf16")
    kc, vc = oracle_pool(w)
    a = oracle_decode(w, kc, vc, threads=1)
    b = oracle_decode(w, kc, vc, threads=5)
    assert np.array_equal(a, b)


def test_selected_pairs_match_full_output():
    w = wl.random_case(22, num_seqs=4, max_len=70, num_heads=6,
                       num_kv_heads=3, head_dim=64, block_size=16,
                       dtype="f16")
    kc, vc = oracle_pool(w)
    full = oracle_decode(w, kc, vc)
    sel = np.array([[3, 5], [0, 0], [2, 1]])
    part = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens,
                               w.scale, w.block_size, w.num_kv_heads,
                               w.num_blocks, w.dtype, sel=sel)
    for i, (s, h) in enumerate(sel):
        assert np.array_equal(part[i], full[s, h])


# ---------------------------------------------------- the online softmax ----

def online_model(logits2, values, part_size, n_states):
    """The running-max / running-sum recurrence (Milakov & Gimelshein,
    "Online normalizer calculation for softmax", 2018) with base-2 logits,
    tokens dealt round-robin in chunks of 4 over `n_states` partial states
    inside each partition, states merged by rescaling to the larger
    maximum, then partitions merged the same way."""
    L = len(logits2)

    def merge(states):
        live = [s for s in states if s[0] != -np.inf]
        if not live:
            return (-np.inf, 0.0, np.zeros(values.shape[1]))
        M = max(s[0] for s in live)
        lsum = sum(np.exp2(s[0] - M) * s[1] for s in live)
        acc = sum(np.exp2(s[0] - M) * s[2] for s in live)
        return (M, lsum, acc)

    parts = []
    for p0 in range(0, L, part_size):
        states = [[-np.inf, 0.0, np.zeros(values.shape[1])]
                  for _ in range(n_states)]
        for c, c0 in enumerate(range(p0, min(L, p0 + part_size), 4)):
            st = states[c % n_states]
            x = logits2[c0:min(c0 + 4, p0 + part_size, L)]
            m_new = max(st[0], x.max())
            alpha = np.exp2(st[0] - m_new)
            p = np.exp2(x - m_new)
            st[1] = st[1] * alpha + p.sum()
            st[2] = st[2] * alpha + p @ values[c0:c0 + len(x)]
            st[0] = m_new
        parts.append(merge([tuple(s) for s in states]))
    M, lsum, acc = merge(parts)
    return acc / lsum


@pytest.mark.parametrize("part_size,n_states", [(10 ** 9, 16), (128, 16),
                                                (256, 4), (512, 16),
                                                (1024, 1), (16, 3)])
def test_online_softmax_with_partitions_equals_oracle(part_size, n_states):
    """The device kernels compute the softmax with running maxima, in
    partial states merged at the end, and the long-context variant merges
    per-partition partials; mathematically this is the same softmax."""
    w = wl.random_case(31, num_seqs=3, max_len=1500, min_len=900,
                       num_heads=2, num_kv_heads=2, head_dim=64,
                       block_size=16, dtype="f32")
    kc, vc = oracle_pool(w)
    ref = oracle_decode(w, kc, vc)
    q = lib_widen(w.q, w.dtype)
    kk = lib_widen(w.kv_k, w.dtype)
    vv = lib_widen(w.kv_v, w.dtype)
    scale = np.float64(np.float32(w.scale))
    for s in range(w.num_seqs):
        rows = w.token_rows[s]
        for h in range(w.num_heads):
            x2 = (kk[rows, h] @ q[s, h]) * scale / np.log(2.0)
            got = online_model(x2, vv[rows, h], part_size, n_states)
            assert np.max(np.abs(got - ref[s, h])) <= 1e-12


# ---------------------------------------------------- the cache write ----

@pytest.mark.parametrize("dtype,bs,D", [("f32", 16, 64), ("f16", 32, 128),
                                        ("bf16", 16, 128), ("bf16", 8, 8)])
def test_cache_write_matches_numpy_view_scatter(dtype, bs, D):
    """The documented pool layouts, checked through NumPy array views:
    K pool viewed as [blocks, kv_heads, block_size, D], V pool viewed as
    [blocks, kv_heads, block_size/4, D, 4]; every other byte unchanged."""
    w = wl.random_case(41, num_seqs=5, max_len=70, num_heads=4,
                       num_kv_heads=2, head_dim=D, block_size=bs,
                       dtype=dtype, pool_factor=2.0)
    kc, vc = oracle.new_pool(w.num_blocks, w.num_kv_heads, bs, D, dtype)
    ek, ev = kc.copy(), vc.copy()
    oracle.reshape_and_cache(w.kv_k, w.kv_v, kc, vc, w.kv_slots,
                             w.num_kv_heads, D, bs, w.num_blocks, dtype)
    K5 = ek.reshape(w.num_blocks, w.num_kv_heads, bs, D)
    V5 = ev.reshape(w.num_blocks, w.num_kv_heads, bs // 4, D, 4)
    for i, slot in enumerate(w.kv_slots):
        p, o = divmod(int(slot), bs)
        K5[p, :, o, :] = w.kv_k[i]
        V5[p, :, o // 4, :, o % 4] = w.kv_v[i]
    u = np.uint32 if dtype == "f32" else np.uint16
    assert np.array_equal(kc.view(u), ek.view(u))
    assert np.array_equal(vc.view(u), ev.view(u))


def test_cache_write_rejects_duplicates_and_range_and_skips_negative():
    kc, vc = oracle.new_pool(4, 1, 16, 8, "f32", fill="zero")
    k = np.ones((3, 1, 8), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.reshape_and_cache(k, k, kc, vc, np.array([1, 5, 1]), 1, 8, 16,
                                 4, "f32")
    with pytest.raises(oracle.OracleError):
        oracle.reshape_and_cache(k, k, kc, vc, np.array([1, 64, 2]), 1, 8, 16,
                                 4, "f32")
    assert not kc.any() and not vc.any()  # rejected calls write nothing
    oracle.reshape_and_cache(k, k, kc, vc, np.array([-1, 3, -7]), 1, 8, 16, 4,
                             "f32")
    assert kc.sum() == 8 and vc.sum() == 8


def test_decode_rejects_bad_table_and_context():
    w = wl.tiny(0)
    kc, vc = oracle_pool(w)
    bad = w.block_tables.copy()
    bad[3, 1] = w.num_blocks
    with pytest.raises(oracle.OracleError):
        oracle_decode(w, kc, vc, tables=bad)
    lens = w.context_lens.copy()
    lens[0] = w.max_blocks_per_seq * w.block_size + 1
    with pytest.raises(oracle.OracleError):
        oracle_decode(w, kc, vc, lens=lens)


# ------------------------------------------------- the pages' examples ----

def _probe_table(table, L, bs, slots_of_tokens=None):
    """A one-sequence, one-head pool whose tokens 0..L-1 are placed through
    `table`; returns a function probe(j) -> oracle output of a one-hot
    probe at token j, and the value written for each token."""
    NB = max(table) + 1
    D = 8
    rng = np.random.default_rng(5)
    vals = rng.standard_normal((L, 1, D)).astype(np.float32)
    t = np.arange(L)
    slots = (np.asarray(table)[t // bs] * bs + t % bs
             if slots_of_tokens is None else np.asarray(slots_of_tokens))
    bt = np.full((1, len(table)), -1, np.int32)
    bt[0, :] = table

    def probe(j):
        kk = np.zeros((L, 1, D), np.float32)
        kk[j, 0, 0] = 16384.0
        kc, vc = oracle.new_pool(NB, 1, bs, D, "f32")
        oracle.reshape_and_cache(kk, vals, kc, vc, slots, 1, D, bs, NB, "f32")
        q = np.zeros((1, 1, D), np.float32)
        q[0, 0, 0] = 1.0
        return oracle.paged_decode(q, kc, vc, bt, np.array([L], np.int32),
                                   1.0 / np.sqrt(D), bs, 1, NB, "f32")[0, 0]
    return probe, vals, slots


def test_worked_request_walk():
    """Request 1 holds blocks [0, 5, 7]; its token #49 (index 48) opens
    logical block 3 in physical block 9, and attention spans tokens 0-48."""
    ex = json.load(open(GOLDEN))["request_walk"]
    bs = ex["block_size"]
    table = ex["block_table_before"] + [ex["new_block"]]
    L = ex["attended_tokens"][1] + 1
    assert ex["new_token_index"] // bs == ex["logical_block_of_new_token"]
    for lb, pb in ex["logical_to_physical"]:
        assert table[lb] == pb
    # the slots the pages' walk implies, written by the oracle's cache write
    slots = np.array([table[t // bs] * bs + t % bs for t in range(L)])
    for tok, slot in ex["token_slots"]:
        assert slots[tok] == slot
    probe, vals, _ = _probe_table(table, L, bs)
    # the oracle's walk reads token j back from the slot the page names
    for tok, _slot in ex["token_slots"]:
        assert np.array_equal(probe(tok), vals[tok, 0].astype(np.float64))
    for lo, hi in ex["token_ranges_of_logical_blocks"]:
        for tok in (lo, hi):
            assert np.array_equal(probe(tok), vals[tok, 0].astype(np.float64))


def test_scattered_table_diagram():
    """logical blocks [0,1,2,3] -> physical [7,2,9,1]: token t is read from
    physical block table[t // 16] at offset t % 16."""
    ex = json.load(open(GOLDEN))["scattered_table"]
    bs = ex["block_size"]
    table = ex["physical"]
    L = bs * len(table)
    # values written straight at the physical slots the diagram implies
    slots = [table[t // bs] * bs + t % bs for t in range(L)]
    probe, vals, _ = _probe_table(table, L, bs, slots_of_tokens=slots)
    for lb in ex["logical"]:
        for off in (0, 7, bs - 1):
            t = lb * bs + off
            assert np.array_equal(probe(t), vals[t, 0].astype(np.float64))


def test_allocator_walk_and_fragmentation_count():
    """Blocks are allocated on demand: ceil(tokens / 16) blocks, waste
    confined to the last block."""
    ex = json.load(open(GOLDEN))["allocator_walk"]
    bs = ex["block_size"]

    def blocks(n):
        w = wl.build("walk", lens=[n], num_heads=1, num_kv_heads=1,
                     head_dim=8, block_size=bs, dtype="f32", seed=0,
                     pool_factor=4.0)
        return int((w.block_tables[0] >= 0).sum())

    assert blocks(ex["prompt_tokens"]) == ex["blocks_after_prompt"]
    assert ex["prompt_tokens"] - bs == ex["tokens_in_second_block_after_prompt"]
    assert 2 * bs - ex["prompt_tokens"] == ex["empty_positions_after_prompt"]
    assert blocks(ex["tokens_when_second_block_full"]) == 2
    assert blocks(33) == ex["blocks_at_33_tokens"]
    n = ex["final_tokens"]
    assert blocks(n) == ex["final_blocks"]
    assert n - (blocks(n) - 1) * bs == ex["live_positions_in_last_block"]
    assert blocks(n) * bs - n == ex["unused_positions_in_last_block"]

    fc = json.load(open(GOLDEN))["fragmentation_count"]
    b = blocks(fc["tokens"])
    assert b == fc["blocks"] and b * bs == fc["slots"]
    assert b * bs - fc["tokens"] == fc["wasted_slots"]
    assert max(blocks(n) * bs - n for n in range(1, 200)) == \
        fc["max_wasted_per_request"]


# ------------------------------------------------------- element decoding ----

def test_fp16_decoding_exhaustive():
    h = np.arange(65536, dtype=np.uint16).view(np.float16)
    assert np.array_equal(oracle.widen(h, "f16"), h.astype(np.float64),
                          equal_nan=True)


def test_bf16_decoding_exhaustive():
    b = np.arange(65536, dtype=np.uint16)
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()
    assert np.array_equal(oracle.widen(b, "bf16"), want, equal_nan=True)
