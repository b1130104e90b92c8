"""8-bit (E4M3) caches on the GPU, through the C ABI.

* The quantising cache write equals the oracle's, bit for bit, whole pools.
* The device widening of every E4M3 code is exact: a one-token decode
  returns code * v_scale exactly (fp32 output).
* Decode (single-pass and split, vector and matrix-core kernels) matches
  the oracle, which reads the same quantised pools, within the tolerance of
  the output type; the 13B-class and 70B-class workloads at full size.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import compare, split_parts_per_wave, to_f64, to_torch, TORCH

pytestmark = pytest.mark.gpu
FP8 = torch.float8_e4m3fn


def fp8_pool_to_dev(kc, vc, NB, Hkv, bs, D):
    kd = torch.from_numpy(kc).view(FP8).reshape(NB, Hkv, bs, D).cuda()
    vd = torch.from_numpy(vc).view(FP8).reshape(NB, Hkv, bs // 4, D, 4).cuda()
    return kd, vd


def dev_bits(t):
    return t.view(torch.uint8).cpu().numpy().reshape(-1)


def gpu_write(w, ks, vs, kc0, vc0):
    import paged_kv_cache_309_amd as pkv
    kd, vd = fp8_pool_to_dev(kc0, vc0, w.num_blocks, w.num_kv_heads,
                             w.block_size, w.head_dim)
    kk, vv = to_torch(w.kv_k, w.dtype), to_torch(w.kv_v, w.dtype)
    pkv.reshape_and_cache(kk, vv, kd, vd, torch.from_numpy(w.kv_slots).cuda(),
                          k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return kd, vd


def oracle_write(w, ks, vs, kc0, vc0):
    kc, vc = kc0.copy(), vc0.copy()
    oracle.reshape_and_cache_fp8(w.kv_k, w.kv_v, kc, vc, w.kv_slots,
                                 w.num_kv_heads, w.head_dim, w.block_size,
                                 w.num_blocks, w.dtype, ks, vs)
    return kc, vc


def decode(w, kd, vd, variant, part, ks, vs, q=None):
    import paged_kv_cache_309_amd as pkv
    q = to_torch(w.q, w.dtype) if q is None else q
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    out = torch.empty_like(q)
    if variant == "single":
        pkv.paged_attention_decode(out, q, kd, vd, bt, cl, w.scale,
                                   k_scale=ks, v_scale=vs)
    else:
        nb = pkv.split_workspace_bytes(q, kd, bt, part)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        pkv.paged_attention_decode_split(out, q, kd, vd, bt, cl, w.scale,
                                         part, ws, k_scale=ks, v_scale=vs)
    return out


CASES = [
    # dtype, bs, Hq, Hkv, D, S, max_len, k_scale, v_scale
    ("bf16", 16, 4, 4, 128, 6, 700, 1.0, 1.0),
    ("f16", 32, 8, 8, 64, 5, 400, 0.05, 0.25),
    ("f32", 16, 2, 2, 128, 4, 300, 2.0, 0.5),
    ("bf16", 16, 64, 8, 128, 5, 800, 0.02, 0.03),   # 70B-class heads, MFMA
    ("f16", 32, 16, 2, 128, 4, 500, 1.0, 1.0),      # MFMA, bs 32
    ("bf16", 16, 12, 3, 64, 5, 300, 0.5, 2.0),      # MFMA, D 64
    ("f32", 16, 40, 2, 64, 3, 200, 1.0, 1.0),       # 20 per KV head: vector
    ("f32", 16, 16, 2, 128, 4, 400, 0.5, 1.5),      # fp32 q, 8 per KV head: vector
]


def case(i, seed=0):
    dtype, bs, Hq, Hkv, D, S, max_len, ks, vs = CASES[i]
    w = wl.random_case(7000 + 10 * i + seed, num_seqs=S, max_len=max_len,
                       num_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       block_size=bs, dtype=dtype, pool_factor=1.6)
    return w, ks, vs


@pytest.mark.parametrize("i", range(len(CASES)))
def test_quantising_cache_write_bit_exact(i):
    w, ks, vs = case(i)
    print(f"[fp8 write] case {i} {w.dtype} lens {w.context_lens.tolist()}",
          flush=True)
    kc0, vc0 = oracle.new_pool(w.num_blocks, w.num_kv_heads, w.block_size,
                               w.head_dim, "fp8")
    kd, vd = gpu_write(w, ks, vs, kc0, vc0)
    kc, vc = oracle_write(w, ks, vs, kc0, vc0)
    assert np.array_equal(dev_bits(kd), kc)
    assert np.array_equal(dev_bits(vd), vc)


@pytest.mark.parametrize("i", [0, 3])
def test_quantising_cache_write_shuffled_order_bit_exact(i):
    """Tokens in a random order: no slot group is written whole by one
    token, every token writes its own value bytes."""
    w, ks, vs = case(i, seed=2)
    import paged_kv_cache_309_amd as pkv
    perm = np.random.default_rng(5).permutation(w.kv_slots.shape[0])
    kc0, vc0 = oracle.new_pool(w.num_blocks, w.num_kv_heads, w.block_size,
                               w.head_dim, "fp8")
    kd, vd = fp8_pool_to_dev(kc0, vc0, w.num_blocks, w.num_kv_heads,
                             w.block_size, w.head_dim)
    pkv.reshape_and_cache(to_torch(w.kv_k[perm], w.dtype),
                          to_torch(w.kv_v[perm], w.dtype), kd, vd,
                          torch.from_numpy(w.kv_slots[perm]).cuda(),
                          k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    kc, vc = kc0.copy(), vc0.copy()
    oracle.reshape_and_cache_fp8(w.kv_k[perm], w.kv_v[perm], kc, vc,
                                 w.kv_slots[perm], w.num_kv_heads, w.head_dim,
                                 w.block_size, w.num_blocks, w.dtype, ks, vs)
    assert np.array_equal(dev_bits(kd), kc)
    assert np.array_equal(dev_bits(vd), vc)


def test_cache_write_rounding_and_saturation_codes():
    """Values chosen to land on ties, subnormals and past the largest
    finite value go through the device encoder and match the oracle's."""
    Hkv, D, bs = 1, 64, 16
    mids = oracle.widen(np.arange(0, 127, dtype=np.uint8), "fp8")
    vals = np.concatenate([(mids[:-1] + mids[1:]) / 2, mids,
                           [448, 460, 464, 500, 1e30, np.inf, 2.0 ** -10,
                            2.0 ** -12, 0.0]]).astype(np.float32)
    vals = np.concatenate([vals, -vals, [np.nan]]).astype(np.float32)
    T = -(-vals.size // D)
    x = np.zeros(T * D, np.float32)
    x[:vals.size] = vals
    x = x.reshape(T, Hkv, D)
    NB = -(-T // bs)
    slots = np.arange(T, dtype=np.int64)
    kc0, vc0 = oracle.new_pool(NB, Hkv, bs, D, "fp8")
    import paged_kv_cache_309_amd as pkv
    kd, vd = fp8_pool_to_dev(kc0, vc0, NB, Hkv, bs, D)
    pkv.reshape_and_cache(torch.from_numpy(x).cuda(), torch.from_numpy(x).cuda(),
                          kd, vd, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kc, vc = kc0.copy(), vc0.copy()
    oracle.reshape_and_cache_fp8(x, x, kc, vc, slots, Hkv, D, bs, NB, "f32",
                                 1.0, 1.0)
    assert np.array_equal(dev_bits(kd), kc)
    assert np.array_equal(dev_bits(vd), vc)


@pytest.mark.parametrize("v_scale", [1.0, 0.375])
@pytest.mark.parametrize("qdtype,Hq", [("f32", 1), ("bf16", 8), ("f16", 8)])
def test_every_code_widens_exactly(v_scale, qdtype, Hq):
    """One-token sequences: the output is v * v_scale exactly; 128 dims x 2
    sequences carry all 256 codes.  An fp32 query runs the vector kernel; a
    16-bit query with 8 query heads per KV head runs the matrix-core kernel,
    which widens the codes to the query's type (exact for every E4M3 value,
    and so is the product with 0.375 in both 16-bit types)."""
    import paged_kv_cache_309_amd as pkv
    S, H, D, bs = 2, 1, 128, 16
    codes = np.arange(256, dtype=np.uint8).reshape(S, D)
    kc = np.zeros(S * H * bs * D, np.uint8)
    vc = np.zeros(S * H * bs * D, np.uint8)
    V5 = vc.reshape(S, H, bs // 4, D, 4)
    for s in range(S):
        V5[s, 0, 0, :, 0] = codes[s]          # token 0 of block s
    kd, vd = fp8_pool_to_dev(kc, vc, S, H, bs, D)
    q = torch.zeros((S, Hq, D), dtype=TORCH[qdtype], device="cuda")
    bt = torch.tensor([[0], [1]], dtype=torch.int32, device="cuda")
    cl = torch.tensor([1, 1], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    pkv.paged_attention_decode(out, q, kd, vd, bt, cl, 0.1, v_scale=v_scale)
    got = out.float().cpu().numpy().astype(np.float64)
    want = oracle.widen(codes.reshape(-1), "fp8").reshape(S, D) * v_scale
    for h in range(Hq):
        assert np.array_equal(got[:, h, :],
                              want.astype(np.float32).astype(np.float64),
                              equal_nan=True), h


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("variant,part", [("single", 0), ("split", 64),
                                          ("split", 512)])
def test_decode_matches_oracle(i, variant, part):
    w, ks, vs = case(i, seed=1)
    print(f"[fp8 decode] case {i} {variant} {part}", flush=True)
    kc0, vc0 = oracle.new_pool(w.num_blocks, w.num_kv_heads, w.block_size,
                               w.head_dim, "fp8")
    kc, vc = oracle_write(w, ks, vs, kc0, vc0)
    want = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens,
                               w.scale, w.block_size, w.num_kv_heads,
                               w.num_blocks, w.dtype, cache_dtype="fp8",
                               k_scale=ks, v_scale=vs)
    kd, vd = fp8_pool_to_dev(kc, vc, w.num_blocks, w.num_kv_heads,
                             w.block_size, w.head_dim)
    got = to_f64(decode(w, kd, vd, variant, part, ks, vs))
    assert np.all(np.isfinite(got))
    compare(got, want, w.dtype, f"fp8 case {i} {variant}{part}")


@pytest.mark.parametrize("name", ["mha13b", "gqa70b"])
def test_full_size_workloads(name):
    w = wl.CONFIGS[name](0)
    print(f"[fp8 full] {name}", flush=True)
    ks = vs = 1.0
    kc0, vc0 = oracle.new_pool(w.num_blocks, w.num_kv_heads, w.block_size,
                               w.head_dim, "fp8")
    kd, vd = gpu_write(w, ks, vs, kc0, vc0)
    kc, vc = oracle_write(w, ks, vs, kc0, vc0)
    del kc0, vc0
    assert np.array_equal(dev_bits(kd), kc) and np.array_equal(dev_bits(vd), vc)
    rng = np.random.default_rng(1)
    sel = np.array(sorted({(int(rng.integers(w.num_seqs)),
                            int(rng.integers(w.num_heads))) for _ in range(48)}),
                   np.int32)
    want = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens,
                               w.scale, w.block_size, w.num_kv_heads,
                               w.num_blocks, w.dtype, sel=sel,
                               cache_dtype="fp8", k_scale=ks, v_scale=vs)
    for variant in ("single", "split"):
        out = to_f64(decode(w, kd, vd, variant, 512, ks, vs))
        compare(out[sel[:, 0], sel[:, 1]], want, w.dtype, f"{name} {variant}")


def test_split_several_partitions_per_wave():
    """E4M3 caches on the vector kernel's split walk with one wave carried
    through four consecutive partitions (rows 2 and 3 park nothing: a row
    of 8-bit values holds 64 dims)."""
    ks, vs = 0.25, 2.0
    w = wl.random_case(7900, num_seqs=64, max_len=600, num_heads=8,
                       num_kv_heads=8, head_dim=128, block_size=16,
                       dtype="bf16", pool_factor=1.3)
    part = 16
    P = -(-(w.max_blocks_per_seq * w.block_size) // part)
    ppw = split_parts_per_wave(w.num_seqs, w.num_heads, P)
    print(f"[fp8 split ppw] P={P} parts/wave={ppw}", flush=True)
    if ppw < 2:
        pytest.skip("this device holds the whole grid at one partition per wave")
    kc0, vc0 = oracle.new_pool(w.num_blocks, w.num_kv_heads, w.block_size,
                               w.head_dim, "fp8")
    kc, vc = oracle_write(w, ks, vs, kc0, vc0)
    want = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens,
                               w.scale, w.block_size, w.num_kv_heads,
                               w.num_blocks, w.dtype, cache_dtype="fp8",
                               k_scale=ks, v_scale=vs)
    kd, vd = fp8_pool_to_dev(kc, vc, w.num_blocks, w.num_kv_heads,
                             w.block_size, w.head_dim)
    got = to_f64(decode(w, kd, vd, "split", part, ks, vs))
    compare(got, want, w.dtype, f"fp8 split{part} parts/wave={ppw}")
