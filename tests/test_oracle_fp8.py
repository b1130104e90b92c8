"""Pins of the oracle's 8-bit (E4M3) cache functions to things other than
itself: torch's float8_e4m3fn conversions (a library routine), the format's
fixed points (largest finite value, NaN codes, saturation), a NumPy-view
formulation of the quantising cache write, and ordinary attention on the
dequantised, un-paged keys and values."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads as wl


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_every_code():
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(oracle.widen(codes, "fp8"), torch_decode(codes),
                          equal_nan=True)
    v = oracle.widen(codes, "fp8")
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6


def test_encode_matches_library_in_range_including_ties():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(20),
        rng.standard_normal(20000).astype(np.float32) * np.float32(0.003),
        oracle.widen(np.arange(0, 127, dtype=np.uint8), "fp8").astype(np.float32),
    ])
    # every midpoint between neighbouring codes: a tie that must go to the
    # even fraction
    vals = oracle.widen(np.arange(0, 127, dtype=np.uint8), "fp8")
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    x = np.concatenate([x, mids, -mids])
    keep = np.abs(x) < 464
    assert np.array_equal(oracle.e4m3_encode(x[keep]), torch_encode(x[keep]))


def test_encode_saturates_and_keeps_nan():
    x = np.float32([448, 449, 463.9, 464, 1e4, np.inf, -500, -np.inf, np.nan])
    got = oracle.e4m3_encode(x)
    assert list(got[:6]) == [0x7E] * 6
    assert list(got[6:8]) == [0xFE, 0xFE]
    assert got[8] == 0x7F


@pytest.mark.parametrize("in_dtype,scale", [("bf16", 1.0), ("f16", 0.05),
                                            ("f32", 3.0)])
def test_quantising_cache_write_matches_view_scatter(in_dtype, scale):
    w = wl.random_case(51, num_seqs=4, max_len=60, num_heads=4,
                       num_kv_heads=2, head_dim=64, block_size=16,
                       dtype=in_dtype, pool_factor=2.0)
    NB, Hkv, bs, D = w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim
    kc, vc = oracle.new_pool(NB, Hkv, bs, D, "fp8")
    ek, ev = kc.copy(), vc.copy()
    oracle.reshape_and_cache_fp8(w.kv_k, w.kv_v, kc, vc, w.kv_slots, Hkv, D,
                                 bs, NB, in_dtype, scale, scale * 2)
    xk = wl.storage_to_f32(w.kv_k, in_dtype) / np.float32(scale)
    xv = wl.storage_to_f32(w.kv_v, in_dtype) / np.float32(scale * 2)
    qk = torch_encode(np.clip(xk, -448, 448))
    qv = torch_encode(np.clip(xv, -448, 448))
    K5 = ek.reshape(NB, Hkv, bs, D)
    V5 = ev.reshape(NB, Hkv, bs // 4, D, 4)
    for i, slot in enumerate(w.kv_slots):
        p, o = divmod(int(slot), bs)
        K5[p, :, o, :] = qk[i]
        V5[p, :, o // 4, :, o % 4] = qv[i]
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


@pytest.mark.parametrize("q_dtype,Hq,Hkv", [("bf16", 8, 2), ("f16", 4, 4),
                                             ("f32", 6, 3)])
def test_decode_on_quantised_cache_is_attention_on_dequantised_values(
        q_dtype, Hq, Hkv):
    w = wl.random_case(52, num_seqs=5, max_len=90, num_heads=Hq,
                       num_kv_heads=Hkv, head_dim=64, block_size=16,
                       dtype=q_dtype, pool_factor=1.5)
    ks, vs = 0.04, 0.5
    kc, vc = oracle.new_pool(w.num_blocks, Hkv, 16, 64, "fp8")
    oracle.reshape_and_cache_fp8(w.kv_k, w.kv_v, kc, vc, w.kv_slots, Hkv, 64,
                                 16, w.num_blocks, q_dtype, ks, vs)
    got = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens,
                              w.scale, 16, Hkv, w.num_blocks, q_dtype,
                              cache_dtype="fp8", k_scale=ks, v_scale=vs)
    # reference: torch-quantised, torch-dequantised logical K and V
    xk = wl.storage_to_f32(w.kv_k, q_dtype) / np.float32(ks)
    xv = wl.storage_to_f32(w.kv_v, q_dtype) / np.float32(vs)
    K = torch_decode(torch_encode(np.clip(xk, -448, 448))) * np.float64(np.float32(ks))
    V = torch_decode(torch_encode(np.clip(xv, -448, 448))) * np.float64(np.float32(vs))
    q = wl.storage_to_f32(w.q, q_dtype).astype(np.float64)
    G = Hq // Hkv
    sc = np.float64(np.float32(w.scale))
    for s in range(w.num_seqs):
        rows = w.token_rows[s]
        for h in range(Hq):
            if len(rows) == 0:
                assert np.all(got[s, h] == 0)
                continue
            p = scipy.special.softmax(K[rows, h // G] @ q[s, h] * sc)
            assert np.max(np.abs(p @ V[rows, h // G] - got[s, h])) <= 1e-12
