"""Pins of the oracle's multi-query (chunked prefill) attention to things
other than itself: causal attention computed by NumPy/SciPy with an
explicit mask on the un-paged keys and values; one-token chunks equal to
decode, which is pinned on its own; the same prompt cut into different
chunks giving the same outputs; invariance under physical placement; and
tokens after a query never influencing it."""
import numpy as np
import pytest
import scipy.special

import oracle
import workloads as wl
from test_oracle_pins import lib_widen, oracle_pool


def oracle_prefill(w, kc, vc, tables=None, q=None, qsl=None, lens=None,
                   **kw):
    return oracle.paged_prefill(
        w.q if q is None else q, kc, vc,
        w.block_tables if tables is None else tables,
        w.context_lens if lens is None else lens,
        w.query_start_loc if qsl is None else qsl, w.scale, w.block_size,
        w.num_kv_heads, w.num_blocks, w.dtype, **kw)


def brute_causal(w, kv_k=None):
    """softmax(Q K^T * scale + M) V per sequence and head on the logical,
    contiguous K/V, with M = -inf above the causal diagonal: the chunk's
    query j sits at position L - C + j."""
    q = lib_widen(w.q, w.dtype)
    kk = lib_widen(w.kv_k if kv_k is None else kv_k, w.dtype)
    vv = lib_widen(w.kv_v, w.dtype)
    G = w.num_heads // w.num_kv_heads
    scale = np.float64(np.float32(w.scale))
    out = np.zeros((q.shape[0], w.num_heads, w.head_dim))
    qsl = w.query_start_loc
    for s in range(w.num_seqs):
        rows = w.token_rows[s]
        L, C = len(rows), int(qsl[s + 1] - qsl[s])
        if C == 0:
            continue
        K = np.repeat(kk[rows], G, axis=1)       # [L, Hq, D]
        V = np.repeat(vv[rows], G, axis=1)
        pos = L - C + np.arange(C)
        mask = np.where(np.arange(L)[None, :] <= pos[:, None], 0.0, -np.inf)
        for h in range(w.num_heads):
            logits = q[qsl[s]:qsl[s + 1], h, :] @ K[:, h, :].T * scale + mask
            out[qsl[s]:qsl[s + 1], h] = scipy.special.softmax(logits, axis=1) @ V[:, h, :]
    return out


SWEEP = [
    # dtype, bs, Hq, Hkv, D, S, max_prior, max_chunk
    ("f32", 16, 2, 2, 64, 4, 40, 24),
    ("f16", 16, 8, 2, 64, 5, 70, 40),
    ("bf16", 32, 8, 1, 128, 3, 60, 33),
    ("bf16", 4, 6, 3, 8, 6, 20, 20),
    ("f16", 8, 5, 5, 16, 4, 0, 30),      # whole prompts in one chunk
]


@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_matches_masked_contiguous_attention(case):
    dtype, bs, Hq, Hkv, D, S, mp, mc = SWEEP[case]
    w = wl.random_prefill_case(300 + case, num_seqs=S, max_prior=mp,
                               max_chunk=mc, num_heads=Hq, num_kv_heads=Hkv,
                               head_dim=D, block_size=bs, dtype=dtype)
    kc, vc = oracle_pool(w)
    got = oracle_prefill(w, kc, vc)
    want = brute_causal(w)
    assert got.shape == want.shape
    assert np.max(np.abs(got - want), initial=0.0) <= 1e-12


def test_one_token_chunks_are_decode():
    w = wl.random_case(310, num_seqs=6, max_len=80, num_heads=8,
                       num_kv_heads=2, head_dim=64, block_size=16,
                       dtype="bf16", min_len=1)
    kc, vc = oracle_pool(w)
    qsl = np.arange(w.num_seqs + 1, dtype=np.int32)
    got = oracle_prefill(w, kc, vc, qsl=qsl)
    want = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens,
                               w.scale, w.block_size, w.num_kv_heads,
                               w.num_blocks, w.dtype)
    assert np.array_equal(got, want)


def test_chunking_does_not_change_the_result():
    """One 90-token prompt processed whole, or as chunks of 30 + 45 + 15
    (each chunk after the earlier ones are in the cache): every token's
    output is bit-identical, since each depends only on its own prefix."""
    w = wl.build("p", lens=[90], num_heads=4, num_kv_heads=2, head_dim=32,
                 block_size=16, dtype="f16", seed=5, pool_factor=2.0,
                 chunk_lens=[90])
    kc, vc = oracle_pool(w)
    whole = oracle_prefill(w, kc, vc)
    parts = []
    start = 0
    for c in (30, 45, 15):
        lens = np.array([start + c], np.int32)
        qsl = np.array([0, c], np.int32)
        parts.append(oracle_prefill(w, kc, vc, q=w.q[start:start + c],
                                    qsl=qsl, lens=lens))
        start += c
    assert np.array_equal(np.concatenate(parts), whole)


def test_physical_permutation_is_bitwise_invariant():
    w = wl.random_prefill_case(320, num_seqs=5, max_prior=50, max_chunk=30,
                               num_heads=4, num_kv_heads=2, head_dim=64,
                               block_size=8, dtype="bf16", pool_factor=3.0)
    kc, vc = oracle_pool(w)
    base = oracle_prefill(w, kc, vc)
    rng = np.random.default_rng(1)
    perm = rng.permutation(w.num_blocks)       # block b moves to perm[b]
    tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1)
    slots = perm[w.kv_slots // w.block_size] * w.block_size + w.kv_slots % w.block_size
    kc2, vc2 = oracle_pool(w, slots=slots)
    got = oracle_prefill(w, kc2, vc2, tables=tables.astype(np.int32))
    assert np.array_equal(got, base)


def test_later_tokens_do_not_influence_a_query():
    """Changing the keys of the last token of a chunk changes only that
    token's own output (and nothing when the chunk has one token less)."""
    w = wl.build("c", lens=[40, 33], num_heads=2, num_kv_heads=1, head_dim=16,
                 block_size=8, dtype="f32", seed=9, pool_factor=1.5,
                 chunk_lens=[12, 33])
    kc, vc = oracle_pool(w)
    base = oracle_prefill(w, kc, vc)
    kk = w.kv_k.copy()
    last = w.token_rows[0][-1]
    kk[last] *= np.float32(3.0)
    w2 = wl.Workload(**{**w.__dict__, "kv_k": kk})
    kc2, vc2 = oracle_pool(w2)
    got = oracle_prefill(w2, kc2, vc2)
    assert np.array_equal(got[:11], base[:11])        # tokens before it
    assert not np.array_equal(got[11], base[11])      # the token itself
    assert np.array_equal(got[12:], base[12:])        # the other sequence
    assert np.max(np.abs(got - brute_causal(w2, kv_k=kk))) <= 1e-12


def test_selected_pairs_and_rejections():
    w = wl.random_prefill_case(330, num_seqs=4, max_prior=30, max_chunk=10,
                               num_heads=4, num_kv_heads=4, head_dim=32,
                               block_size=16, dtype="f32")
    kc, vc = oracle_pool(w)
    full = oracle_prefill(w, kc, vc)
    T = w.q.shape[0]
    sel = np.array([[0, 1], [T - 1, 3], [T // 2, 0]], np.int32)
    got = oracle_prefill(w, kc, vc, sel=sel)
    assert np.array_equal(got, full[sel[:, 0], sel[:, 1]])
    qsl = w.query_start_loc.copy()
    for bad in (qsl + 1, qsl[::-1].copy(), np.r_[qsl[:-1], T + 1]):
        with pytest.raises(oracle.OracleError):
            oracle_prefill(w, kc, vc, qsl=bad.astype(np.int32))
    lens = w.context_lens.copy()
    s = int(np.argmax(np.diff(qsl)))
    lens[s] = int(qsl[s + 1] - qsl[s]) - 1           # chunk longer than context
    with pytest.raises(oracle.OracleError):
        oracle_prefill(w, kc, vc, lens=lens)
