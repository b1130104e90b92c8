"""Pools larger than 4 GiB, through the C ABI.

A KV pool on one MI355X normally spans tens of GiB, so every kernel has to
address blocks whose byte offset inside a pool is past 2^31 and 2^32.  Each
case below builds a small random workload on the oracle's compact pool.  It
then places those blocks in a device pool of a little over 4 GiB per cache,
at physical ids just below and above the 2 GiB and 4 GiB byte marks and at
the pool's last block, and remaps the block table and the slots to them.
Every result must equal the oracle's on the compact pool:
- decode, single pass and split, on the vector and matrix-core kernels,
  over 16-bit, fp32 and 8-bit caches;
- chunked prefill;
- the shared-prefix decode (both prefix kernels);
- the cache write (bit-exact);
- the block copy (bit-exact);
- the swap out to pinned host memory and back (bit-exact).
Blocks of the big pool outside the mapping are never read; the cache-write
case checks that blocks next to the mapped ones stay unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import compare, host_bits, pool_bits, to_f64, to_torch, TORCH

pytestmark = pytest.mark.gpu
FP8 = torch.float8_e4m3fn
KS, VS = 0.5, 0.25  # scales of the 8-bit cases
STORE = {1: torch.uint8, 2: torch.int16, 4: torch.int32}


@pytest.fixture(autouse=True)
def _release_pools():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _elem_bytes(dtype, cache):
    return 1 if cache == "fp8" else {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def big_pool_ids(block_bytes, n, seed):
    """NB_big (the pool reaches a little past 4 GiB) and n distinct block ids
    around the 2 GiB and 4 GiB marks, the pool's last block among them."""
    lo2, lo4 = (1 << 31) // block_bytes, (1 << 32) // block_bytes
    nb_big = lo4 + 512
    zone = np.concatenate([np.arange(lo2 - 256, lo2 + 256), np.arange(lo4 - 256, nb_big - 1)])
    assert n <= zone.size
    rng = np.random.default_rng(seed)
    ids = rng.choice(zone, size=n, replace=False).astype(np.int64)
    ids[rng.integers(0, n)] = nb_big - 1
    assert ids.max() * block_bytes >= (1 << 32) and ids.min() * block_bytes < (1 << 32)
    return nb_big, ids


def torch_pool(flat, dtype, cache, NB, Hkv, bs, D, v):
    """A flat oracle pool as a device pool of the library's shape."""
    if cache == "fp8":
        t = torch.from_numpy(flat).view(FP8)
    else:
        t = to_torch(flat, dtype, device="cpu")
    shape = (NB, Hkv, bs // 4, D, 4) if v else (NB, Hkv, bs, D)
    return t.reshape(shape).cuda()


def place(small, nb_big, ids):
    """A device pool of nb_big blocks (contents undefined) holding the
    blocks of `small` at ids."""
    big = torch.empty((nb_big,) + tuple(small.shape[1:]), dtype=small.dtype, device="cuda")
    st = STORE[small.element_size()]
    big.view(st)[torch.from_numpy(ids).cuda()] = small.view(st)
    return big


def gather(big, ids):
    st = STORE[big.element_size()]
    return big.view(st)[torch.from_numpy(ids).cuda()]


def remap_table(bt, ids):
    out = bt.copy()
    ok = (bt >= 0) & (bt < ids.size)
    out[ok] = ids[bt[ok]]
    return out


def remap_slots(slots, ids, bs):
    out = slots.copy()
    ok = slots >= 0
    out[ok] = ids[slots[ok] // bs] * bs + slots[ok] % bs
    return out


def compact_pools(w, cache):
    """The oracle's pools after writing every row of the workload."""
    Hkv, bs, D, NB = w.num_kv_heads, w.block_size, w.head_dim, w.num_blocks
    if cache == "fp8":
        kc, vc = oracle.new_pool(NB, Hkv, bs, D, "fp8")
        oracle.reshape_and_cache_fp8(w.kv_k, w.kv_v, kc, vc, w.kv_slots, Hkv, D, bs,
                                     NB, w.dtype, KS, VS)
    else:
        kc, vc = oracle.new_pool(NB, Hkv, bs, D, w.dtype)
        oracle.reshape_and_cache(w.kv_k, w.kv_v, kc, vc, w.kv_slots, Hkv, D, bs, NB,
                                 w.dtype)
    return kc, vc


def big_pools(w, cache, kc, vc, seed):
    Hkv, bs, D, NB = w.num_kv_heads, w.block_size, w.head_dim, w.num_blocks
    bb = Hkv * bs * D * _elem_bytes(w.dtype, cache)
    nb_big, ids = big_pool_ids(bb, NB, seed)
    kd = place(torch_pool(kc, w.dtype, cache, NB, Hkv, bs, D, False), nb_big, ids)
    vd = place(torch_pool(vc, w.dtype, cache, NB, Hkv, bs, D, True), nb_big, ids)
    return kd, vd, ids


def _scales(cache):
    return {"k_scale": KS, "v_scale": VS} if cache == "fp8" else {}


# (I/O type, query heads, KV heads, cache, head_dim, block size): the
# matrix-core kernel for 16-bit queries in groups of 2..16, else the vector one
DECODE = [("bf16", 16, 2, "same", 128, 16), ("f16", 4, 4, "same", 128, 16),
          ("f32", 4, 2, "same", 64, 16), ("bf16", 16, 2, "fp8", 128, 16),
          ("f16", 4, 4, "fp8", 128, 32)]


@pytest.mark.parametrize("variant", ["single", "split"])
@pytest.mark.parametrize("dt,Hq,Hkv,cache,D,bs", DECODE)
def test_decode_past_4gib(dt, Hq, Hkv, cache, D, bs, variant):
    import paged_kv_cache_309_amd as pkv
    seed = 8100 + DECODE.index((dt, Hq, Hkv, cache, D, bs))
    w = wl.random_case(seed, num_seqs=5, max_len=300, num_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, block_size=bs, dtype=dt, pool_factor=1.5)
    kc, vc = compact_pools(w, cache)
    kd, vd, ids = big_pools(w, cache, kc, vc, seed)
    print(f"[large pool decode] {dt} Hq={Hq} Hkv={Hkv} cache={cache} D={D} bs={bs} "
          f"{variant} pool={kd.shape[0]} blocks ids {ids.min()}..{ids.max()}", flush=True)
    q = to_torch(w.q, dt)
    out = torch.empty_like(q)
    bt = torch.from_numpy(remap_table(w.block_tables, ids)).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    if variant == "single":
        pkv.paged_attention_decode(out, q, kd, vd, bt, cl, w.scale, **_scales(cache))
    else:
        part = 4 * bs
        ws = torch.empty(max(pkv.split_workspace_bytes(q, kd, bt, part), 16),
                         dtype=torch.uint8, device="cuda")
        pkv.paged_attention_decode_split(out, q, kd, vd, bt, cl, w.scale, part, ws,
                                         **_scales(cache))
    torch.cuda.synchronize()
    want = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                               bs, Hkv, w.num_blocks, dt,
                               cache_dtype="fp8" if cache == "fp8" else None,
                               **_scales(cache))
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    compare(got, want, dt, f"decode past 4 GiB {dt} {cache} {variant}")


@pytest.mark.parametrize("dt,Hq,Hkv,cache", [("bf16", 8, 4, "same"), ("f16", 8, 4, "fp8")])
def test_prefill_past_4gib(dt, Hq, Hkv, cache):
    import paged_kv_cache_309_amd as pkv
    D, bs = 128, 16
    seed = 8200 + (cache == "fp8")
    w = wl.random_prefill_case(seed, num_seqs=3, max_prior=200, max_chunk=90,
                               num_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                               block_size=bs, dtype=dt, pool_factor=1.5)
    kc, vc = compact_pools(w, cache)
    kd, vd, ids = big_pools(w, cache, kc, vc, seed)
    print(f"[large pool prefill] {dt} cache={cache} chunks={w.chunk_lens().tolist()} "
          f"pool={kd.shape[0]} blocks", flush=True)
    q = to_torch(w.q, dt)
    out = torch.empty_like(q)
    pkv.paged_attention_prefill(out, q, kd, vd,
                                torch.from_numpy(remap_table(w.block_tables, ids)).cuda(),
                                torch.from_numpy(w.context_lens).cuda(),
                                torch.from_numpy(w.query_start_loc).cuda(), w.scale,
                                **_scales(cache))
    torch.cuda.synchronize()
    want = oracle.paged_prefill(w.q, kc, vc, w.block_tables, w.context_lens,
                                w.query_start_loc, w.scale, bs, Hkv, w.num_blocks, dt,
                                cache_dtype="fp8" if cache == "fp8" else None,
                                **_scales(cache))
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    compare(got, want, dt, f"prefill past 4 GiB {dt} {cache}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2)])
def test_shared_prefix_past_4gib(Hq, Hkv):
    """The shared-prefix decode over blocks past the 4 GiB mark: the prefix
    products (multi-head: members as the columns; grouped-query: the chunked
    products) and the decode of the rest, against the oracle's decode on the
    compact pool."""
    import paged_kv_cache_309_amd as pkv
    D, bs, dt = 128, 16, "bf16"
    seed = 8500 + Hkv
    rng = np.random.default_rng(seed)
    lens = np.concatenate([rng.integers(1, 120, 6) + 320, rng.integers(1, 90, 4) + 160,
                           rng.integers(1, 400, 2)])
    w = wl.build(f"large_prefix{Hkv}", lens=lens, num_heads=Hq, num_kv_heads=Hkv,
                 head_dim=D, block_size=bs, dtype=dt, seed=seed, pool_factor=1.5,
                 prefix_groups=[([0, 1, 2, 3, 4, 5], 320), ([6, 7, 8, 9], 160)], rng=rng)
    kc, vc = compact_pools(w, "same")
    kd, vd, ids = big_pools(w, "same", kc, vc, seed)
    bt_host = remap_table(w.block_tables, ids)
    plan = pkv.PrefixPlan(bt_host, w.context_lens, bs)
    assert plan.info.num_groups == 2
    print(f"[large pool shared prefix] Hq={Hq} Hkv={Hkv} pool={kd.shape[0]} blocks "
          f"ids {ids.min()}..{ids.max()}", flush=True)
    q = to_torch(w.q, dt)
    out = torch.full_like(q, float("nan"))
    bt = torch.from_numpy(bt_host).cuda()
    ws = torch.empty(max(pkv.shared_prefix_workspace_bytes(q, kd, bt, plan), 16),
                     dtype=torch.uint8, device="cuda")
    pkv.paged_attention_decode_shared_prefix(out, q, kd, vd, bt,
                                             torch.from_numpy(w.context_lens).cuda(),
                                             w.scale, plan, ws)
    torch.cuda.synchronize()
    want = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                               bs, Hkv, w.num_blocks, dt)
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    compare(got, want, dt, f"shared-prefix decode past 4 GiB Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("dt,cache", [("bf16", "same"), ("f16", "fp8")])
def test_cache_write_past_4gib(dt, cache):
    """Every row of a workload written into blocks past the 4 GiB mark; the
    mapped blocks equal the oracle's pool bit for bit, and blocks next to
    them are untouched."""
    import paged_kv_cache_309_amd as pkv
    Hkv, D, bs = 8, 128, 16
    seed = 8300 + (cache == "fp8")
    w = wl.random_case(seed, num_seqs=6, max_len=200, num_heads=Hkv, num_kv_heads=Hkv,
                       head_dim=D, block_size=bs, dtype=dt, pool_factor=1.5)
    NB = w.num_blocks
    cdt = "fp8" if cache == "fp8" else dt
    k0, v0 = oracle.new_pool(NB, Hkv, bs, D, cdt)  # NaN patterns in every slot
    kd, vd, ids = big_pools(w, cache, k0, v0, seed)
    # a few blocks that are not mapped, with known contents
    free = np.setdiff1d(np.concatenate([ids - 1, ids + 1]), ids)
    free = free[(free >= 0) & (free < kd.shape[0])][:16]
    st = STORE[kd.element_size()]
    fidx = torch.from_numpy(free).cuda()
    kd.view(st)[fidx] = 0x55
    vd.view(st)[fidx] = 0x55
    print(f"[large pool write] {dt} cache={cache} rows={w.kv_k.shape[0]} "
          f"pool={kd.shape[0]} blocks", flush=True)
    slots = torch.from_numpy(remap_slots(w.kv_slots, ids, bs)).cuda()
    k = to_torch(w.kv_k, dt).reshape(-1, Hkv, D)
    v = to_torch(w.kv_v, dt).reshape(-1, Hkv, D)
    pkv.reshape_and_cache(k, v, kd, vd, slots, **_scales(cache))
    torch.cuda.synchronize()
    if cache == "fp8":
        oracle.reshape_and_cache_fp8(w.kv_k, w.kv_v, k0, v0, w.kv_slots, Hkv, D, bs, NB,
                                     dt, KS, VS)
    else:
        oracle.reshape_and_cache(w.kv_k, w.kv_v, k0, v0, w.kv_slots, Hkv, D, bs, NB, dt)
    assert np.array_equal(pool_bits(gather(kd, ids)), host_bits(k0))
    assert np.array_equal(pool_bits(gather(vd, ids)), host_bits(v0))
    assert bool((kd.view(st)[fidx] == 0x55).all()) and bool((vd.view(st)[fidx] == 0x55).all())


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_copy_and_swap_past_4gib(dt):
    """Copy-on-write pairs between blocks past the 4 GiB mark, then those
    blocks swapped out to a pinned host pool and back into other blocks past
    it: every pool equals the oracle's block copies bit for bit."""
    import paged_kv_cache_309_amd as pkv
    Hkv, D, bs, NB = 8, 128, 16, 96
    cache = "fp8" if dt == "fp8" else "same"
    n = NB * Hkv * bs * D
    rng = np.random.default_rng(8400)
    if dt == "fp8":
        kc = rng.integers(0, 256, n).astype(np.uint8)
        vc = rng.integers(0, 256, n).astype(np.uint8)
    else:
        kc, vc = wl.normal(n, dt, 8400, 1), wl.normal(n, dt, 8400, 2)
    bb = Hkv * bs * D * (1 if dt == "fp8" else 2)
    nb_big, ids = big_pool_ids(bb, NB, 8400 + (dt == "fp8"))
    kd = place(torch_pool(kc, dt, cache, NB, Hkv, bs, D, False), nb_big, ids)
    vd = place(torch_pool(vc, dt, cache, NB, Hkv, bs, D, True), nb_big, ids)
    print(f"[large pool copy/swap] {dt} pool={nb_big} blocks", flush=True)

    perm = rng.permutation(NB)
    pairs = np.stack([perm[:30], perm[30:60]], 1).astype(np.int64)
    pkv.copy_blocks(kd, vd, torch.from_numpy(ids[pairs]).cuda())
    oracle.copy_blocks(kc, vc, pairs, NB, "fp8" if dt == "fp8" else dt)
    torch.cuda.synchronize()
    assert np.array_equal(pool_bits(gather(kd, ids)), host_bits(kc))
    assert np.array_equal(pool_bits(gather(vd, ids)), host_bits(vc))

    # out: 36 mapped blocks to a pinned host pool of 64 blocks; in: back
    # into 36 other mapped blocks
    NH = 64
    tdt = FP8 if dt == "fp8" else TORCH[dt]
    hk, hv = pkv.new_kv_cache(NH, Hkv, bs, D, tdt, device="cpu", pin_memory=True)
    hk.view(STORE[hk.element_size()]).zero_()
    hv.view(STORE[hv.element_size()]).zero_()
    out_src = perm[60:]
    host_dst = rng.permutation(NH)[:out_src.size]
    m_out = np.stack([ids[out_src], host_dst], 1).astype(np.int64)
    pkv.swap_blocks(kd, vd, hk, hv, torch.from_numpy(m_out).cuda())
    torch.cuda.synchronize()
    hk0 = np.zeros(NH * Hkv * bs * D, kc.dtype)
    hv0 = np.zeros_like(hk0)
    odt = "fp8" if dt == "fp8" else dt
    oracle.swap_blocks(kc, vc, hk0, hv0, np.stack([out_src, host_dst], 1), NB, NH, odt)
    assert np.array_equal(pool_bits(hk), host_bits(hk0))
    assert np.array_equal(pool_bits(hv), host_bits(hv0))

    back = perm[:out_src.size]
    m_in = np.stack([host_dst, ids[back]], 1).astype(np.int64)
    pkv.swap_blocks(hk, hv, kd, vd, torch.from_numpy(m_in).cuda())
    torch.cuda.synchronize()
    oracle.swap_blocks(hk0, hv0, kc, vc, np.stack([host_dst, back], 1), NH, NB, odt)
    assert np.array_equal(pool_bits(gather(kd, ids)), host_bits(kc))
    assert np.array_equal(pool_bits(gather(vd, ids)), host_bits(vc))
