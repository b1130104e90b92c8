"""Pins of the oracle's whole-block copies (copy-on-write and swapping) to
a NumPy formulation: a pool viewed as [num_blocks, block elements], and a
block copy as one row assignment.  Also the rejections the oracle applies
(indices outside a pool, a destination written twice, for copy-on-write a
destination that is also a source)."""
import numpy as np
import pytest

import oracle
import workloads as wl


def pools(nb, Hkv, bs, D, dtype, seed):
    n = nb * Hkv * bs * D
    return wl.normal(n, dtype, seed, 1), wl.normal(n, dtype, seed, 2)


@pytest.mark.parametrize("dtype,nb,Hkv,bs,D,npairs", [
    ("f32", 12, 2, 16, 64, 5), ("bf16", 40, 4, 32, 128, 17),
    ("f16", 3, 1, 16, 64, 1)])
def test_copy_blocks_is_row_assignment(dtype, nb, Hkv, bs, D, npairs):
    kc, vc = pools(nb, Hkv, bs, D, dtype, 21)
    rng = np.random.default_rng(5)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:npairs], perm[npairs:2 * npairs]], 1)
    ek, ev = kc.reshape(nb, -1).copy(), vc.reshape(nb, -1).copy()
    for s, d in pairs:
        ek[d] = ek[s]
        ev[d] = ev[s]
    oracle.copy_blocks(kc, vc, pairs, nb, dtype)
    assert np.array_equal(kc.reshape(nb, -1), ek)
    assert np.array_equal(vc.reshape(nb, -1), ev)


def test_copy_blocks_fp8_and_rejections():
    nb, blk = 6, 2 * 16 * 64
    kc = np.arange(nb * blk, dtype=np.uint8)
    vc = (np.arange(nb * blk) * 7 % 251).astype(np.uint8)
    k0, v0 = kc.copy(), vc.copy()
    for bad in ([[0, 6]], [[-1, 2]], [[0, 2], [1, 2]], [[0, 2], [2, 3]]):
        with pytest.raises(oracle.OracleError):
            oracle.copy_blocks(kc, vc, bad, nb, "fp8")
        assert np.array_equal(kc, k0) and np.array_equal(vc, v0)
    oracle.copy_blocks(kc, vc, [[5, 0]], nb, "fp8")
    assert np.array_equal(kc[:blk], k0[5 * blk:]) and np.array_equal(kc[blk:], k0[blk:])
    assert np.array_equal(vc[:blk], v0[5 * blk:])


@pytest.mark.parametrize("dtype,src_nb,dst_nb,npairs", [
    ("bf16", 30, 10, 7), ("f32", 5, 40, 5), ("fp8", 16, 16, 16)])
def test_swap_blocks_is_row_assignment(dtype, src_nb, dst_nb, npairs):
    Hkv, bs, D = 2, 16, 64
    if dtype == "fp8":
        rng = np.random.default_rng(1)
        sk = rng.integers(0, 256, src_nb * Hkv * bs * D).astype(np.uint8)
        sv = rng.integers(0, 256, src_nb * Hkv * bs * D).astype(np.uint8)
        dk = np.zeros(dst_nb * Hkv * bs * D, np.uint8)
        dv = np.ones_like(dk)
    else:
        sk, sv = pools(src_nb, Hkv, bs, D, dtype, 31)
        dk, dv = pools(dst_nb, Hkv, bs, D, dtype, 32)
    rng = np.random.default_rng(9)
    src = rng.choice(src_nb, npairs, replace=False)
    dst = rng.choice(dst_nb, npairs, replace=False)
    pairs = np.stack([src, dst], 1)
    ek, ev = dk.reshape(dst_nb, -1).copy(), dv.reshape(dst_nb, -1).copy()
    ek[dst] = sk.reshape(src_nb, -1)[src]
    ev[dst] = sv.reshape(src_nb, -1)[src]
    s0 = sk.copy()
    oracle.swap_blocks(sk, sv, dk, dv, pairs, src_nb, dst_nb, dtype)
    assert np.array_equal(dk.reshape(dst_nb, -1), ek)
    assert np.array_equal(dv.reshape(dst_nb, -1), ev)
    assert np.array_equal(sk, s0)


def test_swap_blocks_round_trip_and_rejections():
    """Out to a second pool and back into other blocks: the blocks' bytes
    are the same; a bad mapping writes nothing."""
    nb, nh, Hkv, bs, D = 10, 6, 1, 16, 64
    kc, vc = pools(nb, Hkv, bs, D, "f16", 41)
    hk, hv = pools(nh, Hkv, bs, D, "f16", 42)
    h0 = hk.copy()
    for bad in ([[0, 6]], [[10, 0]], [[0, 1], [2, 1]]):
        with pytest.raises(oracle.OracleError):
            oracle.swap_blocks(kc, vc, hk, hv, bad, nb, nh, "f16")
        assert np.array_equal(hk, h0)
    out = [[7, 0], [2, 1], [9, 2]]
    oracle.swap_blocks(kc, vc, hk, hv, out, nb, nh, "f16")
    back = [[0, 3], [1, 4], [2, 5]]
    k2, v2 = kc.copy(), vc.copy()
    oracle.swap_blocks(hk, hv, k2, v2, back, nh, nb, "f16")
    K, K2 = kc.reshape(nb, -1), k2.reshape(nb, -1)
    V, V2 = vc.reshape(nb, -1), v2.reshape(nb, -1)
    for (s, _), (_, d) in zip(out, back):
        assert np.array_equal(K2[d], K[s]) and np.array_equal(V2[d], V[s])
    untouched = [b for b in range(nb) if b not in (3, 4, 5)]
    assert np.array_equal(K2[untouched], K[untouched])
