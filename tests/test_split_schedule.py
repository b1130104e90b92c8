"""The vector kernel's split walk, modelled on the CPU.

Wave w of workgroup z walks the tiles of partitions (4z + w) * k .. + k - 1
(k partitions per wave) as one stream and parks a partition's row states
at the partition's last tile.  This model restates that schedule - the
same integer steps as the kernel's walk - and checks what the kernel's
memory accesses rely on, for every block size, partition size, table
width, k and a spread of lengths:

* every partition holding a token is parked exactly once, at its own last
  tile, and none other is;
* a wave parks at most k <= 4 partitions, so its LDS slot stays inside the
  64 row states a workgroup holds;
* the grid covers every partition;
* the launcher's choice of k (resident grid, at most 4, at most a quarter
  of the partitions) stays in 1..4.
"""
import numpy as np
import pytest

WAVES = 4
MAX_PPW = 4


def parts_per_wave(num_seqs, num_heads, num_parts, cus):
    ppw = -(-num_seqs * num_heads * num_parts // (cus * 4 * WAVES))
    ppw = min(ppw, max(1, num_parts // WAVES))
    return max(1, min(ppw, MAX_PPW))


def walk(L, part_tokens, num_parts, ppw):
    """Partitions parked, in order, with the tile each was parked at."""
    tpp = part_tokens >> 4
    per_wg = WAVES * ppw
    parked = []
    for z in range(-(-num_parts // per_wg)):
        for w in range(WAVES):
            part0 = (z * WAVES + w) * ppw
            if part0 >= num_parts:
                continue
            tok_begin = part0 * part_tokens
            tok_end = min(L, min(num_parts, part0 + ppw) * part_tokens)
            if tok_begin >= tok_end:
                continue
            st_begin, st_end = tok_begin >> 4, (tok_end + 15) >> 4
            flush_at = min(st_end, st_begin + tpp) - 1
            n_flushed = 0
            for k in range(st_begin, st_end):
                if k == flush_at:
                    slot = (w * MAX_PPW + n_flushed) * 4 + 3  # the last row's slot
                    assert slot < WAVES * MAX_PPW * 4
                    assert n_flushed < ppw
                    parked.append((part0 + n_flushed, k))
                    n_flushed += 1
                    flush_at = min(st_end - 1, flush_at + tpp)
    return parked


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("mult", [1, 2, 3, 32])
@pytest.mark.parametrize("max_blocks", [1, 5, 64, 200])
@pytest.mark.parametrize("ppw", [1, 2, 3, 4])
def test_every_partition_parked_once_at_its_last_tile(bs, mult, max_blocks, ppw):
    part_tokens = bs * mult
    ctx = max_blocks * bs
    num_parts = max(1, -(-ctx // part_tokens))
    rng = np.random.default_rng(bs * 1000 + mult * 100 + max_blocks + ppw)
    lens = {0, 1, 15, 16, 17, part_tokens - 1, part_tokens, part_tokens + 1,
            ctx - 1, ctx} | set(rng.integers(0, ctx + 1, size=6).tolist())
    for L in sorted(x for x in lens if 0 <= x <= ctx):
        parked = walk(L, part_tokens, num_parts, ppw)
        parts = [p for p, _ in parked]
        assert sorted(parts) == [p for p in range(num_parts) if p * part_tokens < L]
        tpp = part_tokens // 16
        for p, k in parked:
            # the partition's last tile: the one holding its last live token
            assert k == (min(L, (p + 1) * part_tokens) - 1) // 16
            assert k // tpp == p


@pytest.mark.parametrize("S,H,P", [(8, 32, 64), (64, 40, 4), (1, 1, 1), (256, 64, 16),
                                   (4096, 64, 65535), (1, 1, 65535)])
@pytest.mark.parametrize("cus", [1, 80, 256, 304])
def test_parts_per_wave_in_range(S, H, P, cus):
    k = parts_per_wave(S, H, P, cus)
    assert 1 <= k <= MAX_PPW
    assert k == 1 or k <= P // WAVES
    if (S, H, P, cus) == (8, 32, 64, 256):
        assert k == 4  # the long-context workload: 1024 resident workgroups
