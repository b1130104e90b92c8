"""Host-side pieces of bench.py: the per-kernel source digest that keys the
stored HBM-counter readings, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = ["decode_vector_kernel", "decode_mfma_kernel", "prefill_mfma_kernel",
           "copy_blocks_kernel", "partition_reduce_kernel",
           "reshape_and_cache_kernel", "reshape_and_cache_fp8_kernel"]


@pytest.mark.parametrize("kernel", KERNELS)
def test_every_kernel_has_a_digest(kernel):
    d = bench.source_digest(kernel)
    assert len(d) == 16 and d == bench.source_digest(kernel)


def test_digests_separate_kernels_in_different_files():
    assert bench.source_digest("decode_vector_kernel") != \
        bench.source_digest("prefill_mfma_kernel")
    # two kernels of one file share the file's digest
    assert bench.source_digest("reshape_and_cache_kernel") == \
        bench.source_digest("partition_reduce_kernel")


def test_unknown_kernel_is_an_error():
    with pytest.raises(ValueError):
        bench.source_digest("no_such_kernel")


def test_stored_traffic_keys_name_real_kernels():
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        pytest.skip("no stored counter readings")
    for key in json.load(open(path)):
        kernel, workload = key.split(":")
        bench.source_digest(kernel)          # raises if the kernel is gone
        assert workload


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_digest_ignores_comments_not_code():
    a = b"int f(int x) { return x + 1; } // one\n/* two */"
    b = b"int f(int x) {\n  return x + 1;  // changed comment\n}"
    c = b"int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    # a comment marker inside a string literal is code
    assert b"//" in bench._code_only(b'const char *u = "a//b";')


def test_unique_kv_bytes_equal_logical_without_sharing():
    import workloads as wl
    w = wl.random_case(31, num_seqs=5, max_len=300, num_heads=4, num_kv_heads=2,
                       head_dim=64, block_size=16, dtype="f16", pool_factor=1.5)
    assert bench.unique_kv_bytes(w, 2) == w.kv_bytes()


def test_unique_kv_bytes_count_a_shared_prefix_once():
    """Sequences over one 64-token prefix: the prefix's tokens count once,
    every sequence's own tokens once each."""
    import numpy as np
    import workloads as wl
    lens = [70, 100, 65, 200]
    w = wl.build("prefix", lens=lens, num_heads=2, num_kv_heads=2, head_dim=64,
                 block_size=16, dtype="bf16", seed=3, pool_factor=1.0, prefix_len=64)
    shared = w.block_tables[:, :4]
    assert (shared == shared[0]).all()  # the prefix blocks are one set
    tokens = 64 + sum(L - 64 for L in lens)
    assert bench.unique_kv_bytes(w, 2) == tokens * 2 * 64 * 2 * 2
    assert bench.unique_kv_bytes(w, 2) < w.kv_bytes()
