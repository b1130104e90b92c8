"""Seeded synthetic inputs for paged decode attention.

This module is shared by the tests, the benchmark and the smoke check, and
feeds both the oracle and the device library.  It holds none of the
method's arithmetic and no pool layout: it draws

  * context lengths,
  * a physical placement of every sequence's blocks (the host allocator's
    job: blocks are handed out on demand, one whenever a sequence's token
    count crosses a block boundary; "PagedAttention: how vLLM manages the
    KV cache", section "Walk one request through the allocator"),
  * block tables (logical block -> physical block, -1 where unused),
  * queries and every token's key and value in logical (per-token) order,
  * the slot of every token: physical_block * block_size + offset, the
    encoding the cache-write call consumes,

and casts values to the storage type.  Whoever consumes a workload builds
its own pool from these rows with its own cache write.

Value recipe: float32 draws from ``numpy.random.default_rng`` standard
normals, rounded to nearest-even into the storage type.  Large arrays are
drawn in fixed 2**20-element chunks, chunk c from the generator seeded by
(seed, stream, c), so the result does not depend on how many threads fill it.

Storage types: fp32 -> numpy.float32, fp16 -> numpy.float16, bf16 ->
numpy.uint16 holding the bfloat16 bit pattern.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
_CHUNK = 1 << 20
_STREAM_Q, _STREAM_K, _STREAM_V = 1, 2, 3


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- casts ----

def f32_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to nearest-even in the storage type."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "f16":
        return x.astype(np.float16)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))))
    out = (r >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a storage array to float32."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float32)


def normal(n: int, dtype: str, seed: int, stream: int) -> np.ndarray:
    """n standard-normal values in the storage type (flat)."""
    out = np.empty(n, STORAGE[dtype])
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        s, e = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.default_rng([seed, stream, c])
        tmp = np.empty(e - s, np.float32)
        g.standard_normal(out=tmp, dtype=np.float32)
        out[s:e] = f32_to_storage(tmp, dtype)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(min(_threads(), nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


# ------------------------------------------------------------- workload ----

@dataclass
class Workload:
    name: str
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    context_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray      # int32 [S, max_blocks_per_seq], -1 unused
    q: np.ndarray                 # [S, Hq, D] storage
    kv_k: np.ndarray              # [R, Hkv, D] storage: every token's key
    kv_v: np.ndarray              # [R, Hkv, D] storage
    kv_slots: np.ndarray          # int64 [R]: slot of each row
    token_rows: list              # per sequence: int64 [L] rows of tokens 0..L-1
    new_rows: np.ndarray          # int64 [S]: row of token L-1 (the new token)
    refcount: np.ndarray          # int32 [num_blocks]: tables referencing a block
    meta: dict = field(default_factory=dict)
    # multi-query (chunked prefill) workloads: q holds [T, Hq, D], one row
    # per chunk token; sequence s's rows are query_start_loc[s] ..
    # query_start_loc[s+1]-1, its last C_s tokens.  None for decode.
    query_start_loc: np.ndarray | None = None   # int32 [S+1]

    # -- chunked prefill: the chunk is the last C_s tokens of each sequence;
    # the step writes the chunk's K/V, then attends (causally) for every
    # chunk token.  The earlier context is written beforehand.
    def chunk_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int64)

    def chunk_rows(self) -> np.ndarray:
        return np.concatenate(
            [self.token_rows[s][len(self.token_rows[s]) - int(c):]
             for s, c in enumerate(self.chunk_lens())] + [np.zeros(0, np.int64)])

    def context_slots(self) -> np.ndarray:
        """Slots of every row, the chunk rows marked -1 (no write)."""
        s = self.kv_slots.copy()
        s[self.chunk_rows()] = -1
        return s

    def chunk_k(self) -> np.ndarray:
        return self.kv_k[self.chunk_rows()]

    def chunk_v(self) -> np.ndarray:
        return self.kv_v[self.chunk_rows()]

    def chunk_slots(self) -> np.ndarray:
        return self.kv_slots[self.chunk_rows()]

    def attended_pairs(self) -> int:
        """(query token, context token) pairs the causal chunks attend, per
        query head: sum over chunk tokens of their position + 1."""
        tot = 0
        for L, C in zip(self.context_lens.astype(np.int64), self.chunk_lens()):
            tot += int(C) * (int(L) - int(C)) + int(C) * (int(C) + 1) // 2
        return tot

    # The decode step writes each sequence's newest token, then attends.
    # Prefill = every other row; its slot list marks the new rows with -1
    # ("no write") so the full row arrays can be passed without copying.
    # A sequence with no tokens has no new token: its new row is -1, its
    # new slot -1 and its new K/V rows are zeros.
    def prefill_slots(self) -> np.ndarray:
        s = self.kv_slots.copy()
        s[self.new_rows[self.new_rows >= 0]] = -1
        return s

    def _new(self, a: np.ndarray) -> np.ndarray:
        out = np.zeros((self.num_seqs,) + a.shape[1:], a.dtype)
        ok = self.new_rows >= 0
        out[ok] = a[self.new_rows[ok]]
        return out

    def new_k(self) -> np.ndarray:
        return self._new(self.kv_k)

    def new_v(self) -> np.ndarray:
        return self._new(self.kv_v)

    def new_slots(self) -> np.ndarray:
        out = np.full(self.num_seqs, -1, np.int64)
        ok = self.new_rows >= 0
        out[ok] = self.kv_slots[self.new_rows[ok]]
        return out

    def kv_bytes(self, elem_bytes: int | None = None) -> int:
        """K and V bytes of every live token, each KV head once; elements of
        the workload's dtype unless `elem_bytes` says otherwise (1 for an
        8-bit cache)."""
        e = elem_bytes or np.dtype(STORAGE[self.dtype]).itemsize
        return int(self.context_lens.astype(np.int64).sum()) * \
            self.num_kv_heads * self.head_dim * e * 2


def _assign_blocks(rng, lens, bs, num_blocks, groups):
    """Physical placement: every sequence gets ceil(L/bs) blocks.  `groups`
    lists (members, prefix_blocks): the first prefix_blocks logical blocks
    of every member of a group are one shared set of physical blocks; the
    groups' sets come first in the draw, then every sequence's own blocks
    in sequence order."""
    S = len(lens)
    need = [-(-int(L) // bs) for L in lens]
    pref = [0] * S
    grp = [-1] * S
    for gi, (members, pb) in enumerate(groups):
        for s in members:
            assert grp[s] < 0, "a sequence in two groups"
            grp[s], pref[s] = gi, pb
    shared_total = sum(pb for _, pb in groups)
    private = sum(max(0, n - pref[s]) for s, n in enumerate(need))
    total = shared_total + private
    if num_blocks is None:
        num_blocks = total
    assert num_blocks >= total
    ids = rng.permutation(num_blocks)[:total].astype(np.int32)
    shared, nxt = [], 0
    for _, pb in groups:
        shared.append(ids[nxt:nxt + pb])
        nxt += pb
    tables = []
    for s in range(S):
        own = need[s] - pref[s]
        pre = shared[grp[s]] if grp[s] >= 0 else ids[:0]
        tables.append(np.concatenate([pre, ids[nxt:nxt + own]]))
        nxt += own
    return tables, num_blocks


def build(name: str, *, lens, num_heads: int, num_kv_heads: int,
          head_dim: int, block_size: int, dtype: str, seed: int,
          num_blocks=None, pool_factor: float = 1.0, max_blocks_per_seq=None,
          prefix_len: int = 0, key_outlier_frac: float = 0.0,
          key_outlier_mult: float = 8.0, scale=None, rng=None,
          meta=None, chunk_lens=None, prefix_groups=None) -> Workload:
    """Generic builder.  `lens` are the context lengths (new token
    included).  With prefix_len > 0 every sequence starts with the same
    prefix_len tokens held in shared blocks (prefix_len must be a multiple
    of block_size).  `prefix_groups` generalises this to several groups: a
    list of (member sequences, prefix tokens), each group's prefix held once
    in blocks its members share (members need at least that many tokens).
    The generator `rng` must already have drawn `lens` if the caller drew
    them from it (placement continues the same stream).  With `chunk_lens`
    (C_s <= L_s per sequence) the workload is a chunked prefill: q gets one
    row per chunk token."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    S = len(lens)
    bs = block_size
    if prefix_groups is None:
        assert prefix_len % bs == 0 and (prefix_len == 0 or lens.min() > prefix_len)
        prefix_groups = [(list(range(S)), prefix_len)] if prefix_len else []
    else:
        assert prefix_len == 0, "prefix_len or prefix_groups, not both"
    groups = []
    for members, plen in prefix_groups:
        assert plen % bs == 0 and all(lens[m] >= plen for m in members)
        groups.append((list(members), plen // bs))
    need_total = sum(-(-int(L) // bs) for L in lens)
    if num_blocks is None and pool_factor != 1.0:
        num_blocks = int(math.ceil(pool_factor * need_total))
    tables, NB = _assign_blocks(rng, lens, bs, num_blocks, groups)
    MB = max_blocks_per_seq or max(1, max(len(t) for t in tables))
    bt = np.full((S, MB), -1, np.int32)
    for s, t in enumerate(tables):
        assert len(t) <= MB
        bt[s, :len(t)] = t
    refcount = np.zeros(NB, np.int32)
    for t in tables:
        np.add.at(refcount, t, 1)

    # rows: each group's shared prefix once, then every sequence's own tokens
    base, R = [], 0
    for _, pb in groups:
        base.append(R)
        R += pb * bs
    pre_rows = [np.zeros(0, np.int64)] * S
    for gi, (members, pb) in enumerate(groups):
        for m in members:
            pre_rows[m] = np.arange(base[gi], base[gi] + pb * bs, dtype=np.int64)
    rows_per_seq = []
    for s, L in enumerate(lens):
        own = int(L) - len(pre_rows[s])
        rows_per_seq.append(np.concatenate([
            pre_rows[s], np.arange(R, R + own, dtype=np.int64)]))
        R += own
    Hq, Hkv, D = num_heads, num_kv_heads, head_dim
    qsl = None
    if chunk_lens is not None:
        chunk_lens = np.asarray(chunk_lens, np.int64)
        assert chunk_lens.shape == (S,) and np.all(chunk_lens >= 0)
        assert np.all(chunk_lens <= lens)
        qsl = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int32)
    T = S if qsl is None else int(qsl[-1])
    q = normal(T * Hq * D, dtype, seed, _STREAM_Q).reshape(T, Hq, D)
    kk = normal(R * Hkv * D, dtype, seed, _STREAM_K).reshape(R, Hkv, D)
    vv = normal(R * Hkv * D, dtype, seed, _STREAM_V).reshape(R, Hkv, D)

    if key_outlier_frac > 0.0:
        # per sequence, floor(frac * L) token positions drawn without
        # replacement; their keys (all heads) are multiplied by an exact
        # power of two after rounding to the storage type
        for s, L in enumerate(lens):
            n_out = int(math.floor(key_outlier_frac * int(L)))
            if n_out == 0:
                continue
            pos = rng.choice(int(L), size=n_out, replace=False)
            r = rows_per_seq[s][pos]
            kk[r] = f32_to_storage(storage_to_f32(kk[r], dtype)
                                   * np.float32(key_outlier_mult), dtype)

    slots = np.empty(R, np.int64)
    for s, L in enumerate(lens):
        t = np.arange(int(L), dtype=np.int64)
        slots[rows_per_seq[s]] = (bt[s, t // bs].astype(np.int64) * bs
                                  + t % bs)
    new_rows = np.array([r[-1] if len(r) else -1 for r in rows_per_seq],
                        np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Workload(name=name, dtype=dtype, num_seqs=S, num_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, block_size=bs,
                    num_blocks=NB, max_blocks_per_seq=MB, scale=float(scale),
                    context_lens=lens.astype(np.int32), block_tables=bt,
                    q=q, kv_k=kk, kv_v=vv, kv_slots=slots,
                    token_rows=rows_per_seq, new_rows=new_rows,
                    refcount=refcount, meta=dict(meta or {}, seed=seed),
                    query_start_loc=qsl)


# ----------------------------------------------------- the named configs ----

def tiny(seed: int = 0) -> Workload:
    """4 sequences with 5, 16, 17 and 40 tokens, 2 heads (MHA), head_dim 64,
    fp32, 16-token blocks, a pool of 16 blocks placed by a seeded permutation.
    The new tokens sit at positions 4, 15, 16 and 39: a block's last slot
    (15) and a fresh block's first slot (16) are both exercised."""
    rng = np.random.default_rng(seed)
    return build("tiny", lens=[5, 16, 17, 40], num_heads=2, num_kv_heads=2,
                 head_dim=64, block_size=16, dtype="f32", seed=seed,
                 num_blocks=16, max_blocks_per_seq=4, scale=1.0 / 8.0,
                 rng=rng)


def mha13b(seed: int = 0) -> Workload:
    """13B-class multi-head decode layer: 64 sequences, lengths uniform on
    [128, 2048], 40 heads, head_dim 128, fp16, 16-token blocks, a pool twice
    the blocks needed with blocks drawn at random from it."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 2048, size=64, endpoint=True)
    return build("mha13b", lens=lens, num_heads=40, num_kv_heads=40,
                 head_dim=128, block_size=16, dtype="f16", seed=seed,
                 pool_factor=2.0, max_blocks_per_seq=128, rng=rng)


GQA_SIGMA = 1.0


def gqa70b(seed: int = 0, num_seqs: int = 256) -> Workload:
    """70B-class grouped-query decode layer: 256 sequences, 64 query heads
    over 8 KV heads, head_dim 128, bf16, 16-token blocks, lengths
    log-normal with median 1024 and sigma 1.0, rounded and clamped to
    [1, 8192], every block at a random place in an exactly sized pool."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(num_seqs)
    lens = np.clip(np.rint(np.exp(math.log(1024.0) + GQA_SIGMA * z)), 1, 8192)
    return build("gqa70b", lens=lens.astype(np.int64), num_heads=64,
                 num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                 seed=seed, max_blocks_per_seq=512, rng=rng,
                 meta={"sigma": GQA_SIGMA})


def long_split(seed: int = 0, num_seqs: int = 8, ctx: int = 32768) -> Workload:
    """Long-context decode: 8 sequences of 32768 tokens, 32 heads (MHA),
    head_dim 128, bf16, 16-token blocks in a randomly permuted pool of
    exactly the 16384 blocks needed; 1% of every sequence's keys are
    multiplied by 8 to stretch the softmax range."""
    rng = np.random.default_rng(seed)
    return build("long_split", lens=[ctx] * num_seqs, num_heads=32,
                 num_kv_heads=32, head_dim=128, block_size=16, dtype="bf16",
                 seed=seed, key_outlier_frac=0.01,
                 max_blocks_per_seq=-(-ctx // 16), rng=rng)


def shared_prefix(seed: int = 0, block_size: int = 16,
                  num_seqs: int = 128) -> Workload:
    """128 sequences sharing one 1024-token prefix (the same physical
    blocks in every table, reference count 128) followed by private
    suffixes of uniform [16, 512] tokens; 32 heads (MHA), head_dim 128,
    bf16, 16- or 32-token blocks."""
    rng = np.random.default_rng(seed)
    suffix = rng.integers(16, 512, size=num_seqs, endpoint=True)
    lens = 1024 + suffix
    return build(f"shared_prefix_bs{block_size}", lens=lens, num_heads=32,
                 num_kv_heads=32, head_dim=128, block_size=block_size,
                 dtype="bf16", seed=seed, prefix_len=1024,
                 max_blocks_per_seq=(1024 + 512) // block_size, rng=rng)


def prefill70b(seed: int = 0, num_seqs: int = 16, chunk: int = 512) -> Workload:
    """Chunked prefill, 70B-class grouped-query layer: 16 sequences, each
    bringing a chunk of 512 prompt tokens after an earlier context uniform
    on [0, 3584] tokens; 64 query heads over 8 KV heads, head_dim 128,
    bf16, 16-token blocks at random places in an exactly sized pool."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(0, 3584, size=num_seqs, endpoint=True)
    lens = prior + chunk
    return build("prefill70b", lens=lens, num_heads=64, num_kv_heads=8,
                 head_dim=128, block_size=16, dtype="bf16", seed=seed,
                 max_blocks_per_seq=(3584 + chunk) // 16, rng=rng,
                 chunk_lens=[chunk] * num_seqs)


def prefill13b(seed: int = 0, num_seqs: int = 8, chunk: int = 512) -> Workload:
    """Chunked prefill, 13B-class multi-head layer: 8 sequences, chunks of
    512 tokens after an earlier context uniform on [0, 1536]; 40 heads,
    head_dim 128, fp16, 16-token blocks, a pool twice the blocks needed."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(0, 1536, size=num_seqs, endpoint=True)
    lens = prior + chunk
    return build("prefill13b", lens=lens, num_heads=40, num_kv_heads=40,
                 head_dim=128, block_size=16, dtype="f16", seed=seed,
                 pool_factor=2.0, max_blocks_per_seq=(1536 + chunk) // 16,
                 rng=rng, chunk_lens=[chunk] * num_seqs)


def random_prefill_case(seed: int, *, num_seqs: int, max_prior: int,
                        max_chunk: int, num_heads: int, num_kv_heads: int,
                        head_dim: int, block_size: int, dtype: str,
                        pool_factor: float = 1.5) -> Workload:
    """A small random chunked-prefill case: earlier context uniform on
    [0, max_prior], chunk uniform on [0, max_chunk] (zero allowed: that
    sequence has no query rows)."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(0, max_prior, size=num_seqs, endpoint=True)
    chunk = rng.integers(0, max_chunk, size=num_seqs, endpoint=True)
    lens = prior + chunk
    return build(f"prefill_random{seed}", lens=lens, num_heads=num_heads,
                 num_kv_heads=num_kv_heads, head_dim=head_dim,
                 block_size=block_size, dtype=dtype, seed=seed,
                 pool_factor=pool_factor, rng=rng, chunk_lens=chunk,
                 max_blocks_per_seq=max(1, -(-(max_prior + max_chunk)
                                             // block_size)))


CONFIGS = {
    "tiny": tiny,
    "mha13b": mha13b,
    "gqa70b": gqa70b,
    "long_split": long_split,
    "shared_prefix_bs16": lambda seed=0: shared_prefix(seed, 16),
    "shared_prefix_bs32": lambda seed=0: shared_prefix(seed, 32),
}

PREFILL_CONFIGS = {
    "prefill70b": prefill70b,
    "prefill13b": prefill13b,
}


def random_case(seed: int, *, num_seqs: int, max_len: int, num_heads: int,
                num_kv_heads: int, head_dim: int, block_size: int,
                dtype: str, pool_factor: float = 1.5, min_len: int = 0,
                prefix_len: int = 0) -> Workload:
    """A small random case for sweeps: lengths uniform on
    [min_len, max_len] (zero allowed)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len, size=num_seqs, endpoint=True)
    if prefix_len:
        lens = np.maximum(lens, prefix_len + 1)
    return build(f"random{seed}", lens=lens, num_heads=num_heads,
                 num_kv_heads=num_kv_heads, head_dim=head_dim,
                 block_size=block_size, dtype=dtype, seed=seed,
                 pool_factor=pool_factor, prefix_len=prefix_len, rng=rng,
                 max_blocks_per_seq=max(1, -(-max(int(max_len), 1)
                                             // block_size)))
