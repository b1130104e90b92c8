"""Every compiled kernel variant once, through the C ABI, against the oracle.

The decode and prefill kernels are templates over the query type, the cache
type (the query's or E4M3), head_dim (64, 128), block size (16, 32) and,
for decode, single pass or split; the call picks the vector kernel or the
matrix-core kernel from the query type and the group width G (matrix cores
for 16-bit queries with 2 <= G <= 16).  This sweep reaches each of those
instantiations on a small random case (ragged lengths, a zero-length
sequence possible, NaN in every unused slot), with non-unit scales for the
8-bit caches, and compares with the oracle within the output type's
tolerance.  The larger per-family tests cover the shapes in depth.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import TORCH, compare, to_f64, to_torch

pytestmark = pytest.mark.gpu
FP8 = torch.float8_e4m3fn
KS, VS = 0.5, 0.25  # scales of the 8-bit cases

# (query type, group width): the decode path each pair takes
DECODE_KINDS = [("f32", 2, "vector"), ("f16", 1, "vector"), ("f16", 4, "mfma"),
                ("bf16", 1, "vector"), ("bf16", 4, "mfma")]
DECODE = [(dt, G, path, cache, D, bs, variant)
          for (dt, G, path), cache, D, bs, variant in itertools.product(
              DECODE_KINDS, ("same", "fp8"), (64, 128), (16, 32), ("single", "split"))]
PREFILL = list(itertools.product(("f32", "f16", "bf16"), ("same", "fp8"), (64, 128),
                                 (16, 32)))


def _pools(w, cache):
    """The oracle's pools (host) after writing the workload's rows, and the
    same bytes on the device in the library's layouts."""
    Hkv, bs, D, NB = w.num_kv_heads, w.block_size, w.head_dim, w.num_blocks
    if cache == "fp8":
        kc, vc = oracle.new_pool(NB, Hkv, bs, D, "fp8")
        oracle.reshape_and_cache_fp8(w.kv_k, w.kv_v, kc, vc, w.kv_slots, Hkv, D, bs,
                                     NB, w.dtype, KS, VS)
        kd = torch.from_numpy(kc).view(FP8).reshape(NB, Hkv, bs, D).cuda()
        vd = torch.from_numpy(vc).view(FP8).reshape(NB, Hkv, bs // 4, D, 4).cuda()
    else:
        kc, vc = oracle.new_pool(NB, Hkv, bs, D, w.dtype)
        oracle.reshape_and_cache(w.kv_k, w.kv_v, kc, vc, w.kv_slots, Hkv, D, bs, NB,
                                 w.dtype)
        kd = to_torch(kc, w.dtype).reshape(NB, Hkv, bs, D)
        vd = to_torch(vc, w.dtype).reshape(NB, Hkv, bs // 4, D, 4)
    return kc, vc, kd, vd


def _scales(cache):
    return {"k_scale": KS, "v_scale": VS} if cache == "fp8" else {}


@pytest.mark.parametrize("dt,G,path,cache,D,bs,variant", DECODE)
def test_decode_instantiation(dt, G, path, cache, D, bs, variant):
    import paged_kv_cache_309_amd as pkv
    Hkv = 2
    seed = 7000 + DECODE.index((dt, G, path, cache, D, bs, variant))
    w = wl.random_case(seed, num_seqs=3, max_len=150, num_heads=G * Hkv,
                       num_kv_heads=Hkv, head_dim=D, block_size=bs, dtype=dt,
                       pool_factor=1.5)
    print(f"[inst decode] {dt} G={G} ({path}) cache={cache} D={D} bs={bs} {variant} "
          f"lens={w.context_lens.tolist()}", flush=True)
    kc, vc, kd, vd = _pools(w, cache)
    q = to_torch(w.q, dt)
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    if variant == "single":
        pkv.paged_attention_decode(out, q, kd, vd, bt, cl, w.scale, **_scales(cache))
    else:
        part = 2 * bs  # several partitions per sequence
        nbytes = pkv.split_workspace_bytes(q, kd, bt, part)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        pkv.paged_attention_decode_split(out, q, kd, vd, bt, cl, w.scale, part, ws,
                                         **_scales(cache))
    torch.cuda.synchronize()
    want = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                               bs, Hkv, w.num_blocks, dt,
                               cache_dtype="fp8" if cache == "fp8" else None,
                               **_scales(cache))
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    compare(got, want, dt, f"decode {dt} G={G} {cache} D={D} bs={bs} {variant}")


@pytest.mark.parametrize("dt,cache,D,bs", PREFILL)
def test_prefill_instantiation(dt, cache, D, bs):
    import paged_kv_cache_309_amd as pkv
    Hkv, G = 2, 2
    seed = 7500 + PREFILL.index((dt, cache, D, bs))
    w = wl.random_prefill_case(seed, num_seqs=3, max_prior=100, max_chunk=70,
                               num_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                               block_size=bs, dtype=dt, pool_factor=1.5)
    print(f"[inst prefill] {dt} cache={cache} D={D} bs={bs} "
          f"lens={w.context_lens.tolist()} chunks={w.chunk_lens().tolist()}", flush=True)
    kc, vc, kd, vd = _pools(w, cache)
    q = to_torch(w.q, dt)
    out = torch.empty_like(q)
    pkv.paged_attention_prefill(out, q, kd, vd, torch.from_numpy(w.block_tables).cuda(),
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
    compare(got, want, dt, f"prefill {dt} {cache} D={D} bs={bs}")


PLAIN = list(itertools.product(("f16", "bf16"), ("same", "fp8"), (64, 128), (16, 32)))


@pytest.mark.parametrize("dt,cache,D,bs", PLAIN)
def test_prefill_instantiation_plain_grid(dt, cache, D, bs):
    """The matrix-core prefill has a second instantiation for grids of more
    than 256 row blocks per XCD, which keep the grid order (the sweep above
    runs the longest-first one).  Many short chunks with max_query_len left
    at its default (all query tokens) give such a grid: about 300 sequences
    x 2 KV heads x 38 row blocks, most of them past their sequence's rows."""
    import paged_kv_cache_309_amd as pkv
    Hkv, G = 2, 2
    seed = 7600 + PLAIN.index((dt, cache, D, bs))
    w = wl.random_prefill_case(seed, num_seqs=300, max_prior=60, max_chunk=16,
                               num_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                               block_size=bs, dtype=dt, pool_factor=1.5)
    T = int(w.query_start_loc[-1])
    row_blocks = -(-T * G // 128)
    grid = 8 * -(-(w.num_seqs * Hkv) // 8) * row_blocks
    assert grid // 8 > 256, grid
    print(f"[inst prefill plain] {dt} cache={cache} D={D} bs={bs} T={T} grid={grid}",
          flush=True)
    kc, vc, kd, vd = _pools(w, cache)
    q = to_torch(w.q, dt)
    out = torch.empty_like(q)
    pkv.paged_attention_prefill(out, q, kd, vd, torch.from_numpy(w.block_tables).cuda(),
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
    compare(got, want, dt, f"prefill plain grid {dt} {cache} D={D} bs={bs}")
