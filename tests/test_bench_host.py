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


def test_stored_traffic_was_read_from_the_current_kernels():
    """Every stored HBM-counter reading (and the profile beside it) was taken
    on kernels whose code is the code in the tree: a kernel changed since its
    counters were read must be profiled again (bench_probe/collect_counters.sh,
    then bench.py --reduce-counters)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        pytest.skip("no stored counter readings")
    stale = [key for key, rec in json.load(open(path)).items()
             if rec["source_digest"] != bench.source_digest(key.split(":")[0])]
    assert not stale, f"counter readings older than their kernels: {stale}"


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


def test_reduce_counters_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    """A synthetic pair of counter passes: the kernel's mean reading in KiB,
    times 1024, times 1 GiB over the copy's reading, per launch; kernels of
    one attention (here the split's partial and reduce kernels) add up."""
    root = tmp_path / "runs"
    d = root / "ls"
    (d / "kt").mkdir(parents=True)
    (d / "FETCH_SIZE").mkdir()
    (d / "WRITE_SIZE").mkdir()
    (d / "args.txt").write_text("--workload long_split --variant split")
    rec = {"metric": "m", "ms_per_step": 0.7, "dtype": "bf16", "steps": 50,
           "config": {"workload": "long_split"},
           "roofline": {"kernel": "decode_vector_kernel + partition_reduce_kernel",
                        "mean_launch_ms": 0.68, "achieved": 6300.0, "frac": 0.79,
                        "peak": 8000.0, "unit": "GB/s",
                        "algorithmic_bytes_per_launch": 4.0e9}}
    (d / "kt.json").write_text("noise\n" + json.dumps(rec) + "\n")
    (d / "kt" / "run_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void pkv::decode_vector_kernel<2, 2, 128, 16, true, false>(pkv::DecodeArgs)",'
        '50,33000000,660000,97.0,650000,700000,1000\n')

    # a trace of 60 partial-kernel launches, the first ten slow (clock ramp),
    # and 60 reduce launches: the bench's last timed pass is the last 50
    vk_name = "void pkv::decode_vector_kernel<2, 2, 128, 16, true, false>(pkv::DecodeArgs)"
    rows = ['"Kernel_Name","Start_Timestamp","End_Timestamp"']
    t0 = 1000
    for i in range(60):
        dur = 700000 if i < 10 else 650000
        rows.append(f'"{vk_name}",{t0},{t0 + dur}')
        rows.append(f'"void pkv::partition_reduce_kernel<2, 128>(pkv::DecodeArgs)",'
                    f'{t0 + dur + 100},{t0 + dur + 5100}')
        t0 += dur + 10000
    (d / "kt" / "run_kernel_trace.csv").write_text("\n".join(rows) + "\n")

    def passes(counter, kern_vals, copy_val):
        rows = ["Kernel_Name,Counter_Name,Counter_Value"]
        for name, vals in kern_vals.items():
            rows += [f'"{name}",{counter},{v}' for v in vals]
        rows.append(f'"__amd_rocclr_copyBuffer",{counter},{copy_val}')
        return "\n".join(rows) + "\n"
    vk = "void pkv::decode_vector_kernel<2, 2, 128, 16, true, false>(pkv::DecodeArgs)"
    rk = "void pkv::partition_reduce_kernel<2, 128>(pkv::DecodeArgs)"
    (d / "FETCH_SIZE" / "run_counter_collection.csv").write_text(
        passes("FETCH_SIZE", {vk: [2000000, 2000002], rk: [4000]}, 524288))
    (d / "WRITE_SIZE" / "run_counter_collection.csv").write_text(
        passes("WRITE_SIZE", {vk: [8000], rk: [64]}, 1048576))
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    bench.reduce_counters(str(root))
    t = json.load(open(prof / "traffic.json"))
    e = t["decode_vector_kernel+partition_reduce_kernel:long_split"]
    assert e["calibration_factor_fetch"] == 2.0 and e["calibration_factor_write"] == 1.0
    assert e["read_bytes"] == round((2000001 + 4000) * 1024 * 2.0)
    assert e["write_bytes"] == (8000 + 64) * 1024
    assert e["source_digest"] == bench.source_digest(
        "decode_vector_kernel+partition_reduce_kernel")
    md = (prof / "decode_vector_kernel+partition_reduce_kernel_long_split.md").read_text()
    assert "--workload long_split --variant split" in md and "| 50 | 660.0 |" in md
    # the trace mean of the last 50 launches of each kernel, added: 650 + 5 us
    assert "the last 50 launches" in md and "attention): 655.0 us." in md
