"""Steps captured in a HIP graph (torch.cuda.CUDAGraph is a hipGraph on
ROCm): the library's calls only enqueue kernels on the caller's stream - no
allocation, memset or synchronisation - so they can be captured.  Covered:
the decode step (cache write + single-pass or split decode), the
shared-prefix decode, the chunked-prefill step (chunk write + prefill, both
kernels), the allocation-free split and a copy-on-write step (block copies +
decode).  Each graph is replayed several times with eager work and
synchronisations in between; every replay must equal the eager result bit
for bit, and the eager result matches the oracle."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import Dev, compare, oracle_out, oracle_pool, to_f64, to_torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["single", "split"])
@pytest.mark.parametrize("dtype,Hq,Hkv", [("bf16", 16, 2), ("f16", 8, 8)])
def test_decode_step_replays_in_a_graph(variant, dtype, Hq, Hkv):
    import paged_kv_cache_309_amd as pkv
    w = wl.random_case(8100 + Hq, num_seqs=6, max_len=500, num_heads=Hq,
                       num_kv_heads=Hkv, head_dim=128, block_size=16,
                       dtype=dtype, pool_factor=1.5, min_len=1)
    print(f"[graph] {dtype} Hq={Hq} Hkv={Hkv} {variant}", flush=True)
    dev = Dev(w)
    kc, vc = dev.cache_via_gpu_write()
    ws = None
    if variant == "split":
        nb = pkv.split_workspace_bytes(dev.q, kc, dev.block_tables, 128)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev.q)

    def step():
        pkv.reshape_and_cache(dev.new_k, dev.new_v, kc, vc, dev.new_slots)
        if variant == "single":
            pkv.paged_attention_decode(out, dev.q, kc, vc, dev.block_tables,
                                       dev.context_lens, w.scale)
        else:
            pkv.paged_attention_decode_split(out, dev.q, kc, vc, dev.block_tables,
                                             dev.context_lens, w.scale, 128, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    kh, vh = oracle_pool(w)
    compare(to_f64(eager), oracle_out(w, kh, vh), dtype, "eager step")
    for rep in range(4):
        out.fill_(float("nan"))                  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep


@pytest.mark.parametrize("Hkv", [2, 8])
def test_shared_prefix_decode_replays_in_a_graph(Hkv):
    """The shared-prefix decode (the prefix products, then the decode that
    starts from their partial states) captured with the cache write: every
    replay equals the eager call bit for bit, with the workspace scribbled
    over between replays, and the eager call matches the oracle."""
    import paged_kv_cache_309_amd as pkv
    bs = 16
    rng = np.random.default_rng(8200 + Hkv)
    lens = np.concatenate([320 + rng.integers(1, 200, 7), rng.integers(1, 400, 3)])
    w = wl.build(f"graph_shared{Hkv}", lens=lens, num_heads=8, num_kv_heads=Hkv,
                 head_dim=128, block_size=bs, dtype="bf16", seed=8300 + Hkv,
                 pool_factor=1.5, prefix_groups=[([0, 1, 2, 3], 320), ([4, 5, 6], 160)],
                 rng=rng)
    print(f"[graph] shared prefix Hkv={Hkv}", flush=True)
    dev = Dev(w)
    kc, vc = dev.cache_via_gpu_write()
    plan = pkv.PrefixPlan(w.block_tables, w.context_lens, bs)
    assert plan.info.num_groups == 2
    nb = pkv.shared_prefix_workspace_bytes(dev.q, kc, dev.block_tables, plan)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev.q)

    def step():
        pkv.reshape_and_cache(dev.new_k, dev.new_v, kc, vc, dev.new_slots)
        pkv.paged_attention_decode_shared_prefix(out, dev.q, kc, vc, dev.block_tables,
                                                 dev.context_lens, w.scale, plan, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    kh, vh = oracle_pool(w)
    compare(to_f64(eager), oracle_out(w, kh, vh), "bf16", "eager shared-prefix step")
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(255)                            # stale partials must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep


@pytest.mark.parametrize("dtype,Hq,Hkv", [("bf16", 16, 2), ("f32", 4, 2)])
def test_prefill_step_replays_in_a_graph(dtype, Hq, Hkv):
    """A chunked-prefill step (the chunk's cache write, then the prefill
    attention: the matrix-core kernel for bf16, the vector kernel's
    multi-query mode for fp32) captured and replayed; every replay equals
    the eager step bit for bit, and the eager step matches the oracle."""
    import oracle
    import paged_kv_cache_309_amd as pkv
    w = wl.random_prefill_case(8400 + Hq, num_seqs=4, max_prior=300, max_chunk=120,
                               num_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                               block_size=16, dtype=dtype, pool_factor=1.5)
    print(f"[graph] prefill {dtype} Hq={Hq} Hkv={Hkv} chunks={w.chunk_lens().tolist()}",
          flush=True)
    kc, vc = pkv.new_kv_cache(w.num_blocks, Hkv, 16, 128,
                              {"bf16": torch.bfloat16, "f32": torch.float32}[dtype],
                              fill=float("nan"))
    ctx = w.kv_slots.copy()
    ctx[w.chunk_rows()] = -1
    pkv.reshape_and_cache(to_torch(w.kv_k, dtype), to_torch(w.kv_v, dtype), kc, vc,
                          torch.from_numpy(ctx).cuda())
    ck, cv = to_torch(w.chunk_k(), dtype), to_torch(w.chunk_v(), dtype)
    cs = torch.from_numpy(w.kv_slots[w.chunk_rows()]).cuda()
    q = to_torch(w.q, dtype)
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    qsl = torch.from_numpy(w.query_start_loc).cuda()
    mq = int(w.chunk_lens().max())

    def step():
        pkv.reshape_and_cache(ck, cv, kc, vc, cs)
        pkv.paged_attention_prefill(out, q, kc, vc, bt, cl, qsl, w.scale, max_query_len=mq)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    kh, vh = oracle_pool(w)
    want = oracle.paged_prefill(w.q, kh, vh, w.block_tables, w.context_lens,
                                w.query_start_loc, w.scale, 16, Hkv, w.num_blocks, dtype)
    compare(to_f64(eager), want, dtype, "eager prefill step")
    st = torch.int16 if dtype == "bf16" else torch.int32
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(st), eager.view(st)), rep


def test_allocation_free_split_replays_in_a_graph():
    """The allocation-free split decode (partials in the library's static
    scratch, no workspace argument: the call meant for captured code) in a
    captured decode step; the scratch is rewritten by an eager call with
    other sizes between replays, and every replay equals the eager step bit
    for bit."""
    import paged_kv_cache_309_amd as pkv
    w = wl.random_case(8450, num_seqs=6, max_len=900, num_heads=16, num_kv_heads=2,
                       head_dim=128, block_size=16, dtype="bf16", pool_factor=1.5,
                       min_len=1)
    w2 = wl.random_case(8451, num_seqs=3, max_len=400, num_heads=8, num_kv_heads=8,
                        head_dim=64, block_size=16, dtype="bf16", pool_factor=1.5,
                        min_len=1)
    print("[graph] allocation-free split", flush=True)
    dev, dev2 = Dev(w), Dev(w2)
    kc, vc = dev.cache_via_gpu_write()
    kc2, vc2 = dev2.cache_via_gpu_write()
    out = torch.empty_like(dev.q)
    out2 = torch.empty_like(dev2.q)

    def step():
        pkv.reshape_and_cache(dev.new_k, dev.new_v, kc, vc, dev.new_slots)
        pkv.paged_attention_decode_split_static(out, dev.q, kc, vc, dev.block_tables,
                                                dev.context_lens, w.scale, 128)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    kh, vh = oracle_pool(w)
    compare(to_f64(eager), oracle_out(w, kh, vh), "bf16", "eager static split step")
    for rep in range(4):
        out.fill_(float("nan"))
        pkv.paged_attention_decode_split_static(out2, dev2.q, kc2, vc2, dev2.block_tables,
                                                dev2.context_lens, w2.scale, 64)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep


def test_copy_on_write_step_replays_in_a_graph():
    """copy_blocks (each sequence's first block copied to a free block, which
    the sequence's table then points to), the cache write and the decode,
    captured together.  The copies' targets are filled with NaN before every
    replay, so only the replay's own copies make the output right; every
    replay equals the eager step bit for bit, and that equals the decode
    over the original blocks."""
    import paged_kv_cache_309_amd as pkv
    w = wl.random_case(8460, num_seqs=5, max_len=300, num_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, dtype="bf16", pool_factor=2.0,
                       min_len=17)
    print("[graph] copy-on-write step", flush=True)
    dev = Dev(w)
    kc, vc = dev.cache_via_gpu_write()
    ref = dev.decode(kc, vc)
    torch.cuda.synchronize()
    used = set(int(b) for b in w.block_tables[w.block_tables >= 0].ravel())
    free = [b for b in range(w.num_blocks) if b not in used][:w.num_seqs]
    assert len(free) == w.num_seqs
    src = w.block_tables[:, 0].astype(np.int64)
    pairs = torch.from_numpy(np.stack([src, np.array(free, np.int64)], 1)).cuda()
    bt2 = w.block_tables.copy()
    bt2[:, 0] = free
    bt2 = torch.from_numpy(bt2).cuda()
    dst = torch.tensor(free, dtype=torch.long, device="cuda")
    out = torch.empty_like(dev.q)

    def step():
        pkv.copy_blocks(kc, vc, pairs)
        pkv.paged_attention_decode(out, dev.q, kc, vc, bt2, dev.context_lens, w.scale)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    assert torch.equal(eager.view(torch.int16), ref.view(torch.int16))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        out.fill_(float("nan"))
        kc[dst] = float("nan")
        vc[dst] = float("nan")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
