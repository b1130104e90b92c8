"""Benchmark of one paged decode step on one MI355X.

A step is the whole hot path over one batch: the cache write of every
sequence's new token (reshape_and_cache), then decode attention over the
paged cache (single-pass, or split into partitions plus the reduce).  The
default workload is the 13B-class multi-head decode layer: 64 sequences with
context lengths uniform on [128, 2048], 40 heads, head_dim 128, fp16,
16-token blocks, a pool twice the blocks needed with blocks at random places.
All inputs are seeded synthetic data already resident in HBM when the timed
region starts.

Prints one JSON line on stdout:
  value          effective KV bandwidth of the step: live K/V bytes / step time
  roofline       the attention kernel's algorithmic bytes / its mean duration
                 (HIP events around each launch), against the 8 TB/s HBM peak
  cpu_baseline   the fp64 oracle timed on host cores for the same step

    python bench.py [--steps K] [--warmup W] [--workload mha13b]
                    [--variant single|split] [--partition 512]
                    [--kv-dtype same|fp8]

With --kv-dtype fp8 the caches hold 8-bit E4M3 values (per-tensor scales
of 1); the queries and outputs keep the workload's dtype.
"""
from __future__ import annotations

import argparse
import hashlib
import importlib.util
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("paged decode attention effective KV GB/s (% of HBM peak) + "
          "decode tokens/s")
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=None,
                   choices=["tiny", "mha13b", "gqa70b", "long_split",
                            "shared_prefix_bs16", "shared_prefix_bs32",
                            "prefill70b", "prefill13b"],
                   help="default: mha13b (decode), prefill70b (prefill)")
    p.add_argument("--variant", default="single",
                   choices=["single", "split", "shared"],
                   help="single-pass, split (partitions + reduce), or shared "
                        "(each sharer set's prefix computed once)")
    p.add_argument("--partition", type=int, default=512)
    p.add_argument("--kv-dtype", default="same", choices=["same", "fp8"],
                   help="cache element type: the workload's (default) or "
                        "8-bit E4M3")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--mode", default="decode",
                   choices=["decode", "copy_blocks", "swap", "prefill"],
                   help="decode: the decode step (default); copy_blocks: the "
                        "copy-on-write block copy; swap: blocks out to pinned "
                        "host memory and back; prefill: chunked-prefill "
                        "attention (--workload prefill70b|prefill13b)")
    p.add_argument("--pairs", type=int, default=2048,
                   help="copy_blocks mode: block pairs copied per launch")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after the timed region, run one plain device copy "
                        "of this many MiB (to scale HBM counters)")
    p.add_argument("--no-configs", action="store_true",
                   help="time the headline workload only (the default run "
                        "also times the other decode workloads)")
    p.add_argument("--reduce-counters", metavar="DIR", default=None,
                   help="no GPU: turn the rocprofv3 runs under DIR (written by "
                        "bench_probe/collect_counters.sh) into profiles/*.md "
                        "and profiles/traffic.json")
    return p.parse_args()


def _code_only(src: bytes) -> bytes:
    """C/C++ source without comments and with whitespace runs collapsed, so
    that an edit of a comment leaves a kernel's digest unchanged.  String
    and character literals are kept as they are."""
    out, i, n = bytearray(), 0, len(src)
    while i < n:
        c = src[i:i + 1]
        if c in (b'"', b"'"):
            j = i + 1
            while j < n and src[j:j + 1] != c:
                j += 2 if src[j:j + 1] == b"\\" else 1
            out += src[i:j + 1]
            i = j + 1
        elif src.startswith(b"//", i):
            j = src.find(b"\n", i)
            i = n if j < 0 else j
        elif src.startswith(b"/*", i):
            j = src.find(b"*/", i + 2)
            i = n if j < 0 else j + 2
            out += b" "
        else:
            out += c
            i += 1
    return b" ".join(bytes(out).split())


def source_digest(kernel: str | None = None) -> str:
    """Hash of the code a kernel is built from (comments and layout left
    out): the file that defines it, the local headers it includes
    (transitively), the dispatcher, and each file's compile flags; with no
    kernel named, every kernel source.  Stored
    HBM-counter readings are used only while it matches."""
    csrc = os.path.join(ROOT, "paged_kv_cache_309_amd", "csrc")
    text = {f: open(os.path.join(csrc, f), "rb").read()
            for f in sorted(os.listdir(csrc))}
    if kernel is None:
        files = sorted(text)
    else:
        files = []
        for k in kernel.split("+"):   # several kernels: "a+b"
            pat = re.compile(rb"__global__[^;{]*?\b" + re.escape(k.encode())
                             + rb"\s*\(", re.S)
            found = [f for f in sorted(text) if pat.search(text[f])]
            if not found:
                raise ValueError(f"no kernel named {k} in {csrc}")
            files += [f for f in found if f not in files]
        todo = list(files) + ["abi.hip"]
        files = []
        while todo:
            f = todo.pop()
            if f in files or f not in text:
                continue
            files.append(f)
            todo += [m.decode() for m in
                     re.findall(rb'#include "([^"]+)"', text[f])]
        files.sort()
    # the build script by path: no need to load the library for its flags
    spec = importlib.util.spec_from_file_location(
        "pkv_build_flags", os.path.join(ROOT, "paged_kv_cache_309_amd", "build.py"))
    build_mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build_mod)
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode() + _code_only(text[f]))
        # the compile line of this file (the flags every file gets, plus its own)
        flags = build_mod.HIPCC_FLAGS + build_mod.FILE_FLAGS.get(f, [])
        h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def unique_kv_bytes(w, elem_bytes: int) -> int:
    """K and V bytes of every live token, counted once per physical slot:
    a block that several sequences' tables share (a common prefix) holds
    its bytes once in HBM.  Equal to the logical bytes when no block is
    shared."""
    bs = w.block_size
    live = {}
    for s, L in enumerate(w.context_lens.tolist()):
        for j in range(-(-int(L) // bs)):
            p = int(w.block_tables[s, j])
            live[p] = max(live.get(p, 0), min(bs, int(L) - j * bs))
    return sum(live.values()) * w.num_kv_heads * w.head_dim * elem_bytes * 2


def kernel_names(desc: str) -> list:
    """The kernels of a roofline `kernel` description ("a (note) + b")."""
    return [part.split()[0] for part in desc.split(" + ")]


def stored_traffic(kernel: str, workload: str):
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


# The other decode workloads timed in the default run, after the headline
# (13B-class multi-head) line: (workload, variant).
EXTRA_CONFIGS = [("gqa70b", "single"), ("long_split", "split"),
                 ("shared_prefix_bs16", "single"), ("shared_prefix_bs16", "shared"),
                 ("shared_prefix_bs32", "single"), ("shared_prefix_bs32", "shared"),
                 ("tiny", "single")]


def decode_kernel_name(w, variant):
    """The kernel the library picks: matrix cores for 2..16 query heads per
    KV head in fp16/bf16, the vector kernel otherwise."""
    k = ("decode_vector_kernel" if w.num_heads == w.num_kv_heads
         or w.dtype == "f32" or w.num_heads // w.num_kv_heads > 16
         else "decode_mfma_kernel")
    if variant == "shared":
        pre = ("decode_mfma_kernel (prefix partials)" if w.num_heads == w.num_kv_heads
               else "prefill_mfma_kernel (prefix partials)")
        return f"{pre} + {k}"
    return k + (" + partition_reduce_kernel" if variant == "split" else "")


def measure_decode(w, variant, partition, fp8, steps, warmup):
    """One decode step (the cache write of every sequence's new token, then
    attention) of workload w, timed: `steps` steps with no events in them,
    then the same number with HIP events around each of the two launches on
    the launch stream.  Returns the timings and the byte counts."""
    import numpy as np
    import torch

    import paged_kv_cache_309_amd as pkv
    import workloads as wl

    tdt = {"f32": torch.float32, "f16": torch.float16,
           "bf16": torch.bfloat16}[w.dtype]
    cdt = torch.float8_e4m3fn if fp8 else tdt
    if variant == "shared" and (fp8 or w.dtype == "f32"):
        raise SystemExit("--variant shared takes 16-bit caches and queries")

    def dev(a):
        a = np.ascontiguousarray(a)
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    t0 = time.time()
    q = dev(w.q)
    tables = torch.from_numpy(w.block_tables).cuda()
    lens = torch.from_numpy(w.context_lens).cuda()
    new_k, new_v = dev(w.new_k()), dev(w.new_v())
    new_slots = torch.from_numpy(w.new_slots()).cuda()
    k_cache, v_cache = pkv.new_kv_cache(w.num_blocks, w.num_kv_heads,
                                        w.block_size, w.head_dim, cdt, fill=0.0)
    # prefill: every earlier token written by the library's cache write
    kk, vv = dev(w.kv_k), dev(w.kv_v)
    pkv.reshape_and_cache(kk, vv, k_cache, v_cache,
                          torch.from_numpy(w.prefill_slots()).cuda())
    del kk, vv
    out = torch.empty_like(q)
    ws = None
    plan = None
    plan_ms = None
    if variant == "split":
        nbytes = pkv.split_workspace_bytes(q, k_cache, tables, partition)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    elif variant == "shared":
        # the sharer sets, found on the host from the host tables (built by
        # the harness like the tables themselves; timed apart)
        t_plan = time.perf_counter()
        plan = pkv.PrefixPlan(w.block_tables, w.context_lens, w.block_size)
        plan_ms = (time.perf_counter() - t_plan) * 1e3
        nbytes = pkv.shared_prefix_workspace_bytes(q, k_cache, tables, plan)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        log(f"[bench] prefix plan: {plan.info.num_groups} sets, "
            f"{plan.info.num_members} members, prefix "
            f"{plan.info.max_prefix_tokens} tokens, built in {plan_ms:.3f} ms")
    torch.cuda.synchronize()
    log(f"[bench] {w.name} ({variant}) inputs resident in HBM after "
        f"{time.time()-t0:.1f}s")

    stream = torch.cuda.current_stream()
    ev = []

    def step(record: bool):
        if record:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
        pkv.reshape_and_cache(new_k, new_v, k_cache, v_cache, new_slots)
        if record:
            e[1].record(stream)
        if variant == "single":
            pkv.paged_attention_decode(out, q, k_cache, v_cache, tables, lens,
                                       w.scale)
        elif variant == "shared":
            pkv.paged_attention_decode_shared_prefix(out, q, k_cache, v_cache,
                                                     tables, lens, w.scale,
                                                     plan, ws)
        else:
            pkv.paged_attention_decode_split(out, q, k_cache, v_cache, tables,
                                             lens, w.scale, partition, ws)
        if record:
            e[2].record(stream)
            ev.append(e)

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    # the timed steps carry the work only; the launch times of the two
    # kernels come from a second pass with events between the launches
    start.record(stream)
    for _ in range(steps):
        step(False)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    rac_ms = [e[0].elapsed_time(e[1]) for e in ev]
    att_ms = [e[1].elapsed_time(e[2]) for e in ev]
    log(f"[bench] {w.name} ({variant}): {steps} steps in {total_ms:.2f} ms")
    del k_cache, v_cache, ws, out, q
    torch.cuda.empty_cache()

    e = np.dtype(wl.STORAGE[w.dtype]).itemsize
    kv_bytes = w.kv_bytes(1 if fp8 else None)
    # the roofline counts each physical K/V byte once: shared prefix blocks
    # are read by every sharer but held once; the metric's effective GB/s
    # stays on logical bytes
    kv_unique = unique_kv_bytes(w, 1 if fp8 else e)
    nblk = int(sum(-(-int(L) // w.block_size) for L in w.context_lens))
    qo_bytes = 2 * w.num_seqs * w.num_heads * w.head_dim * e
    table_bytes = 4 * nblk + 4 * w.num_seqs
    return {"ms_step": total_ms / steps, "att_ms": att_ms, "rac_ms": rac_ms,
            "kv_bytes": kv_bytes, "kv_unique": kv_unique,
            "alg_bytes": kv_unique + qo_bytes + table_bytes, "plan_ms": plan_ms}


def config_summary(w, variant, partition, fp8, m):
    """The per-workload figures of the default run's `configs` object."""
    import numpy as np
    att = float(np.mean(m["att_ms"]))
    kernel = decode_kernel_name(w, variant)
    tag = w.name + ("_fp8" if fp8 else "")
    traffic = stored_traffic("+".join(kernel_names(kernel)), tag)
    return {
        "variant": variant, "partition": partition if variant == "split" else None,
        "kernel": kernel,
        "attention_us": round(att * 1e3, 2),
        "attention_median_us": round(float(np.median(m["att_ms"])) * 1e3, 2),
        "step_us": round(m["ms_step"] * 1e3, 2),
        "kv_gbs": round(m["kv_bytes"] / (att * 1e-3) / 1e9, 1),
        "roofline_frac": round(m["alg_bytes"] / (att * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "traffic_ratio": (round(traffic / m["alg_bytes"], 4) if traffic else None),
        "kv_bytes": m["kv_bytes"], "kv_bytes_unique": m["kv_unique"],
        "decode_tokens_per_s": round(w.num_seqs / (m["ms_step"] * 1e-3), 1),
        "prefix_plan_ms": round(m["plan_ms"], 4) if m["plan_ms"] is not None else None,
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; "
              "run it with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.reduce_counters:
        return reduce_counters(args.reduce_counters)

    import numpy as np
    import torch

    import paged_kv_cache_309_amd as pkv  # noqa: F401  (fails if not built)
    import workloads as wl

    torch.cuda.set_device(0)
    if args.mode == "copy_blocks":
        return bench_copy_blocks(args)
    if args.mode == "swap":
        return bench_swap(args)
    if args.mode == "prefill":
        return bench_prefill(args)
    headline = args.workload is None
    args.workload = args.workload or "mha13b"
    if args.workload not in wl.CONFIGS:
        raise SystemExit(f"{args.workload} is a prefill workload: use --mode prefill")
    t0 = time.time()
    w = wl.CONFIGS[args.workload](args.seed)
    log(f"[bench] workload {w.name}: S={w.num_seqs} Hq={w.num_heads} "
        f"Hkv={w.num_kv_heads} D={w.head_dim} bs={w.block_size} "
        f"dtype={w.dtype} NB={w.num_blocks} generated in {time.time()-t0:.1f}s")
    fp8 = args.kv_dtype == "fp8"
    m = measure_decode(w, args.variant, args.partition, fp8, args.steps, args.warmup)

    calibration_copy(args.calib_copy_mib)
    ceiling = read_ceiling()

    kv_bytes, kv_unique, att_alg_bytes = m["kv_bytes"], m["kv_unique"], m["alg_bytes"]
    ms_step = m["ms_step"]
    att_ms, rac_ms = m["att_ms"], m["rac_ms"]
    att_mean_ms = float(np.mean(att_ms))
    achieved = att_alg_bytes / (att_mean_ms * 1e-3) / 1e9
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    tok_s = w.num_seqs / (ms_step * 1e-3)
    kernel = decode_kernel_name(w, args.variant)
    tag = w.name + ("_fp8" if fp8 else "")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": stored_traffic("+".join(kernel_names(kernel)), tag),
                "kernel": kernel,
                "algorithmic_bytes_per_launch": att_alg_bytes,
                "mean_launch_ms": round(att_mean_ms, 5),
                "logical_kv_gbs": round(kv_bytes / (att_mean_ms * 1e-3) / 1e9, 1)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, kv_bytes, fp8)
        cpu["gpu_speedup"] = round(value / cpu["value"], 1)

    configs = None
    if headline and not args.no_configs and not fp8 and args.variant == "single":
        # the other workloads, each timed the same way after the headline,
        # with at least 50 warm-up and 50 timed steps: the workloads served
        # from L2 and the MALL (shared prefixes) read up to 13% slow in the
        # first tens of steps
        configs = {"steps": max(args.steps, 50), "warmup": max(args.warmup, 50)}
        for name, variant in EXTRA_CONFIGS:
            t1 = time.time()
            wx = wl.CONFIGS[name](args.seed)
            log(f"[bench] config {name} ({variant}) generated in {time.time()-t1:.1f}s")
            mx = measure_decode(wx, variant, args.partition, False, configs["steps"],
                                configs["warmup"])
            configs[f"{name}:{variant}"] = config_summary(wx, variant, args.partition,
                                                          False, mx)
            del wx

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": f"{w.dtype}, e4m3 kv" if fp8 else w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs,
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size,
                   "num_blocks": w.num_blocks, "seed": args.seed,
                   "mean_context": float(w.context_lens.mean()),
                   "variant": args.variant,
                   "kv_dtype": "e4m3" if fp8 else w.dtype,
                   "partition": args.partition if args.variant == "split" else None,
                   "prefix_plan_ms": (round(m["plan_ms"], 4)
                                      if m["plan_ms"] is not None else None),
                   "accumulate": "f32", "kv_bytes_per_step": kv_bytes,
                   "kv_bytes_unique_per_step": kv_unique},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(tok_s, 1),
        "kernels_ms": {"reshape_and_cache": round(float(np.mean(rac_ms)), 5),
                       "attention": round(att_mean_ms, 5),
                       "attention_median": round(float(np.median(att_ms)), 5),
                       "attention_p10": round(float(np.percentile(att_ms, 10)), 5),
                       "attention_p90": round(float(np.percentile(att_ms, 90)), 5)},
        "roofline": roofline,
        "context": {"random_4k_tile_read_gbs": ceiling,
                    "note": "a trivial kernel reading random 4 KiB tiles of a "
                            "4 GiB buffer (the paged walk's access pattern, no "
                            "arithmetic) on this GPU, for comparison with "
                            "roofline.achieved; null if its helper is not built"},
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(rec), flush=True)


def _find(d, suffix):
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    return f[0] if f else None


def _last_json(path):
    for line in reversed(open(path).read().splitlines()):
        if line.startswith("{"):
            return json.loads(line)
    return None


def _counter(d, name):
    """Per-kernel lists of one counter's per-dispatch values (rocprofv3 CSV)."""
    import csv
    out = {}
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] == name:
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _pick(vals, sub):
    return [x for k, v in vals.items() if sub in k for x in v]


def reduce_counters(root):
    """Turn rocprofv3 runs into profiles/<kernel>_<workload>.md summaries and
    profiles/traffic.json.  `root` holds one folder per workload, as
    bench_probe/collect_counters.sh writes them: args.txt (the bench
    arguments), kt.json + kt/ (a --kernel-trace --stats run), and FETCH_SIZE/,
    WRITE_SIZE/ (one --pmc pass each, every run ending with a plain 1 GiB
    device copy).  HBM bytes per launch = the kernel's mean counter value in
    KiB x 1024 x (1 GiB / the copy's reading of the same counter)."""
    import csv
    tj = os.path.join(PROFILES, "traffic.json")
    traffic = json.load(open(tj)) if os.path.exists(tj) else {}
    for tag in sorted(os.listdir(root)):
        d = os.path.join(root, tag)
        if not os.path.exists(os.path.join(d, "args.txt")):
            continue
        args = open(os.path.join(d, "args.txt")).read().strip()
        rec = _last_json(os.path.join(d, "kt.json"))
        roof = rec["roofline"]
        kernels = kernel_names(roof["kernel"])
        kernel = "+".join(kernels)
        wtag = rec["config"]["workload"] + ("_fp8" if "e4m3" in rec["dtype"] else "")
        if kernel == "copy_blocks_kernel":
            wtag = rec["config"]["workload"]
        stats = list(csv.DictReader(open(_find(os.path.join(d, "kt"), "kernel_stats.csv"))))
        kt_cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats "
                  "--output-format csv -d <out> -o run -- python3 <repo>/bench.py "
                  f"--steps 50 --warmup 5 --no-cpu-baseline {args}").strip()

        def pmc_cmd(c):
            return ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc "
                    f"{c} --output-format csv -d <out> -o run -- python3 "
                    "<repo>/bench.py --steps 5 --warmup 2 --no-cpu-baseline "
                    f"--calib-copy-mib 1024 {args}").strip()
        L = [f"# {kernel} on the {wtag} workload", "",
             "Kernel-trace statistics (run from the repository root on one MI355X; "
             "`bench_probe/collect_counters.sh` runs these commands, "
             "`python bench.py --reduce-counters <out>` writes this file):",
             "", "```", kt_cmd, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|"]
        for r in stats:
            name = r["Name"]
            short = (name[5:] if name.startswith("void ") else name).split("(")[0]
            if "read_tiles_kernel" in name:
                short = ("read_tiles_kernel (bench_probe: random 4 KiB tile read "
                         "ceiling, context only)")
            L.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} | "
                     f"{float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
        L.append("")
        # the launches of the bench's last timed pass (the event-timed one in
        # the decode and prefill modes): the last `steps` of each kernel in
        # the trace, so that the clock ramp of the first launches stays out
        trace_path = _find(os.path.join(d, "kt"), "kernel_trace.csv")
        last_us = None
        if trace_path and "steps" in rec:
            trace = list(csv.DictReader(open(trace_path)))
            steps = int(rec["steps"])
            last_us = 0.0
            for k in kernels:
                rows = sorted((r for r in trace if k in r["Kernel_Name"]),
                              key=lambda r: int(r["Start_Timestamp"]))[-steps:]
                last_us += sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                               for r in rows) / len(rows) / 1e3
            L += [f"Kernel-trace mean of the last {steps} launches of `{kernel}` (the "
                  f"bench's last timed pass, each kernel's mean added for a two-launch "
                  f"attention): {last_us:.1f} us.", ""]
        if any("reshape_and_cache" in r["Name"] for r in stats):
            L += ["The reshape_and_cache average includes the one large call that "
                  "fills the earlier context; the per-step calls are the minimum.", ""]
        mean_us = roof["mean_launch_ms"] * 1e3
        unit = roof["unit"]
        L.append(f"bench.py in the same run (HIP events on the launch stream): mean "
                 f"launch {mean_us:.1f} us, roofline {roof['achieved']:.0f} {unit} = "
                 f"{100*roof['frac']:.1f}% of {roof['peak']:.0f} {unit}, step "
                 f"{rec['ms_per_step']*1e3:.1f} us." + (
                     f" The events add the launch gaps to the kernel time "
                     f"({100 * (mean_us / last_us - 1):+.1f}% against the trace mean "
                     f"above); the table's averages also hold the warm-up launches, the "
                     f"first of them at rising clocks." if last_us else ""))
        L += ["", "HBM traffic per launch, from two counter passes:", "", "```",
              pmc_cmd("FETCH_SIZE"), pmc_cmd("WRITE_SIZE"), "```", ""]
        f = _counter(os.path.join(d, "FETCH_SIZE"), "FETCH_SIZE")
        wr = _counter(os.path.join(d, "WRITE_SIZE"), "WRITE_SIZE")
        cf, cw = max(_pick(f, "copyBuffer")), max(_pick(wr, "copyBuffer"))
        kf, kw = 1048576.0 / cf, 1048576.0 / cw
        L.append(f"Calibration: the 1 GiB device copy reads FETCH_SIZE = {cf:.0f} KiB "
                 f"and WRITE_SIZE = {cw:.0f} KiB, so the counters are scaled by "
                 f"{kf:.3f} and {kw:.3f}.")
        # every launch of the attention: the mean per dispatch of each kernel,
        # added up
        fr = sum(sum(_pick(f, k)) / len(_pick(f, k)) for k in kernels)
        wrr = sum(sum(_pick(wr, k)) / len(_pick(wr, k)) for k in kernels)
        rb, wb = fr * 1024 * kf, wrr * 1024 * kw
        L += ["", "| kernel | FETCH_SIZE (KiB, raw) | WRITE_SIZE (KiB, raw) | read bytes "
              "(scaled) | written bytes (scaled) | algorithmic bytes | traffic / "
              "algorithmic |", "|---|---|---|---|---|---|---|"]
        if "algorithmic_bytes_per_launch" in roof:
            alg = roof["algorithmic_bytes_per_launch"]
            L.append(f"| `{kernel}` | {fr:.0f} | {wrr:.1f} | {rb:.4g} | {wb:.4g} | "
                     f"{alg:.4g} | {(rb+wb)/alg:.3f} |")
        else:
            L.append(f"| `{kernel}` | {fr:.0f} | {wrr:.1f} | {rb:.4g} | {wb:.4g} | "
                     f"(flop-bound: {roof['algorithmic_flops_per_launch']:.4g} flops) | - |")
        L.append("")
        open(os.path.join(PROFILES, f"{kernel}_{wtag}.md"), "w").write("\n".join(L))
        traffic[f"{kernel}:{wtag}"] = {
            "bytes_per_launch": int(round(rb + wb)), "read_bytes": int(round(rb)),
            "write_bytes": int(round(wb)), "fetch_size_kib_raw": fr,
            "write_size_kib_raw": wrr, "calibration_factor_fetch": kf,
            "calibration_factor_write": kw, "source_digest": source_digest(kernel),
            "commands": [c.replace("cd /tmp && export TMPDIR=/tmp && ", "")
                         .replace("--output-format csv -d <out> -o run ", "... ")
                         .replace("<repo>/", "")
                         for c in (pmc_cmd("FETCH_SIZE"), pmc_cmd("WRITE_SIZE"))]}
        print(f"{tag}: {kernel} on {wtag}, mean launch {mean_us:.1f} us, traffic / "
              f"algorithmic {(rb + wb) / roof.get('algorithmic_bytes_per_launch', float('nan')):.3f}",
              flush=True)
    json.dump(traffic, open(tj, "w"), indent=1)


def read_ceiling():
    """Read bandwidth of the bench_probe tile-read kernel, or None when its
    helper library is not built."""
    import bench_probe
    if not os.path.exists(bench_probe.LIB):
        log("[bench] bench_probe not built: no read ceiling")
        return None
    return bench_probe.random_tile_read_gbs()


def calibration_copy(mib: int):
    """One plain device copy of `mib` MiB, so that HBM counters read in the
    same run can be scaled to bytes."""
    if not mib:
        return
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy of {n} bytes done")


def bench_copy_blocks(args):
    """Copy-on-write block copies: `pairs` disjoint (source, destination)
    block pairs of the shared-prefix workload's shape (32 KV heads, 16-token
    blocks, head_dim 128, bf16: 128 KiB per block per pool), both pools."""
    import numpy as np
    import torch

    import paged_kv_cache_309_amd as pkv

    nb, hkv, bs, d = 8192, 32, 16, 128
    k_cache, v_cache = pkv.new_kv_cache(nb, hkv, bs, d, torch.bfloat16, fill=1.0)
    rng = np.random.default_rng(args.seed)
    perm = rng.permutation(nb)
    n = min(args.pairs, nb // 2)
    pairs = np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int64)
    mapping = torch.from_numpy(pairs).cuda()
    for _ in range(args.warmup):
        pkv.copy_blocks(k_cache, v_cache, mapping)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        pkv.copy_blocks(k_cache, v_cache, mapping)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    calibration_copy(args.calib_copy_mib)
    block_bytes = hkv * bs * d * 2
    moved = 2 * 2 * n * block_bytes            # K and V, read and written
    gbs = moved / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        kc = np.zeros(nb * hkv * bs * d, np.uint16)
        vc = np.zeros_like(kc)
        t1 = time.perf_counter()
        oracle.copy_blocks(kc, vc, pairs, nb, "bf16")
        dt = time.perf_counter() - t1
        cpu = {"value": round(moved / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "seconds": round(dt, 4),
               "sample": f"the same {n} block pairs copied by the oracle"}
    rec = {"metric": "copy_blocks effective GB/s (K and V blocks read and written)",
           "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "copy_blocks", "pairs": n, "num_blocks": nb,
                      "num_kv_heads": hkv, "block_size": bs, "head_dim": d,
                      "block_bytes_per_pool": block_bytes},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": stored_traffic("copy_blocks_kernel", "copy_blocks"),
                        "kernel": "copy_blocks_kernel",
                        "algorithmic_bytes_per_launch": moved,
                        "mean_launch_ms": round(ms, 5)},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


HOST_LINK_GBS = 64.0   # PCIe 5.0 x16, one direction
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # dense, no sparsity


def bench_prefill(args):
    """Chunked prefill: every sequence brings a chunk of prompt tokens; the
    step writes the chunk's K/V (reshape_and_cache) and then runs
    paged_attention_prefill for every chunk token (causal).  Work is counted
    as 4 * head_dim flops per (query token, query head, attended token)."""
    import numpy as np
    import torch

    import paged_kv_cache_309_amd as pkv
    import workloads as wl

    name = args.workload or "prefill70b"
    if name not in wl.PREFILL_CONFIGS:
        raise SystemExit(f"{name} is not a prefill workload")
    t0 = time.time()
    w = wl.PREFILL_CONFIGS[name](args.seed)
    T = w.q.shape[0]
    log(f"[bench] workload {w.name}: S={w.num_seqs} T={T} Hq={w.num_heads} "
        f"Hkv={w.num_kv_heads} D={w.head_dim} dtype={w.dtype} "
        f"generated in {time.time()-t0:.1f}s")
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    fp8 = args.kv_dtype == "fp8"
    cdt = torch.float8_e4m3fn if fp8 else tdt

    def dev(a):
        a = np.ascontiguousarray(a)
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    kc, vc = pkv.new_kv_cache(w.num_blocks, w.num_kv_heads, w.block_size,
                              w.head_dim, cdt, fill=0.0)
    pkv.reshape_and_cache(dev(w.kv_k), dev(w.kv_v), kc, vc,
                          torch.from_numpy(w.context_slots()).cuda())
    ck, cv = dev(w.chunk_k()), dev(w.chunk_v())
    cslots = torch.from_numpy(w.chunk_slots()).cuda()
    q = dev(w.q)
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    qsl = torch.from_numpy(w.query_start_loc).cuda()
    mq = int(w.chunk_lens().max())
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = []

    def step(record):
        if record:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
        pkv.reshape_and_cache(ck, cv, kc, vc, cslots)
        if record:
            e[1].record(stream)
        pkv.paged_attention_prefill(out, q, kc, vc, bt, cl, qsl, w.scale,
                                    max_query_len=mq)
        if record:
            e[2].record(stream)
            ev.append(e)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    # the timed steps carry the work only; the launch times come from a
    # second pass with events between the launches
    a.record(stream)
    for _ in range(args.steps):
        step(False)
    b.record(stream)
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / args.steps
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    att_ms = [e[1].elapsed_time(e[2]) for e in ev]
    rac_ms = [e[0].elapsed_time(e[1]) for e in ev]
    calibration_copy(args.calib_copy_mib)
    flops = 4.0 * w.head_dim * w.num_heads * w.attended_pairs()
    att_mean = float(np.mean(att_ms))
    achieved = flops / (att_mean * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    tok_s = T / (ms_step * 1e-3)
    cpu = None
    tag = w.name + ("_fp8" if fp8 else "")
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_prefill(w, flops, fp8=fp8)
        cpu["gpu_speedup"] = round(flops / (ms_step * 1e-3) / 1e12 / cpu["value"], 1)
    rec = {"metric": "chunked-prefill attention TFLOP/s (causal, "
                     "4*head_dim flops per attended (token, head, key)) + "
                     "prefill tokens/s",
           "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": f"{w.dtype}, e4m3 kv" if fp8 else w.dtype, "data": "synthetic",
           "config": {"workload": w.name, "num_seqs": w.num_seqs,
                      "query_tokens": T, "num_heads": w.num_heads,
                      "kv_dtype": "e4m3" if fp8 else w.dtype,
                      "num_kv_heads": w.num_kv_heads,
                      "head_dim": w.head_dim, "block_size": w.block_size,
                      "num_blocks": w.num_blocks, "seed": args.seed,
                      "chunk": mq,
                      "mean_context": float(w.context_lens.mean()),
                      "attended_pairs_per_head": w.attended_pairs(),
                      "accumulate": "f32"},
           "prefill_tokens_per_s": round(tok_s, 1),
           "kernels_ms": {"reshape_and_cache": round(float(np.mean(rac_ms)), 5),
                          "attention": round(att_mean, 5),
                          "attention_median": round(float(np.median(att_ms)), 5),
                          "attention_p10": round(float(np.percentile(att_ms, 10)), 5),
                          "attention_p90": round(float(np.percentile(att_ms, 90)), 5)},
           "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                        "peak": peak, "unit": "TFLOP/s",
                        "frac": round(achieved / peak, 4),
                        "traffic": stored_traffic("prefill_mfma_kernel", tag),
                        "kernel": "prefill_mfma_kernel",
                        "algorithmic_flops_per_launch": flops,
                        "mean_launch_ms": round(att_mean, 5)},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def cpu_baseline_prefill(w, flops_total, sample_rows=512, fp8=False):
    """The oracle on a bounded sample: every query head of `sample_rows`
    chunk tokens spread over the batch; flop rate scaled by the sampled
    tokens' share of the work."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    cdt = "fp8" if fp8 else w.dtype
    kc, vc = oracle.new_pool(w.num_blocks, w.num_kv_heads, w.block_size,
                             w.head_dim, cdt, fill="zero")
    if fp8:
        oracle.reshape_and_cache_fp8(w.kv_k, w.kv_v, kc, vc, w.kv_slots,
                                     w.num_kv_heads, w.head_dim, w.block_size,
                                     w.num_blocks, w.dtype, 1.0, 1.0)
    else:
        oracle.reshape_and_cache(w.kv_k, w.kv_v, kc, vc, w.kv_slots,
                                 w.num_kv_heads, w.head_dim, w.block_size,
                                 w.num_blocks, w.dtype)
    T = w.q.shape[0]
    rows = np.linspace(0, T - 1, sample_rows).astype(np.int64)
    sel = np.stack([np.repeat(rows, w.num_heads),
                    np.tile(np.arange(w.num_heads), rows.size)], 1).astype(np.int32)
    # attended tokens of each sampled row
    qsl = w.query_start_loc
    seq = np.searchsorted(qsl, rows, side="right") - 1
    pos = w.context_lens[seq].astype(np.int64) - np.diff(qsl)[seq] + (rows - qsl[seq])
    flops = 4.0 * w.head_dim * w.num_heads * float(np.sum(pos + 1))
    t1 = time.perf_counter()
    out = oracle.paged_prefill(w.q, kc, vc, w.block_tables, w.context_lens,
                               qsl, w.scale, w.block_size, w.num_kv_heads,
                               w.num_blocks, w.dtype, sel=sel, threads=threads,
                               cache_dtype=cdt)
    dt = time.perf_counter() - t1
    assert np.all(np.isfinite(out))
    log(f"[bench] oracle sample {dt:.2f}s")
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{sample_rows} chunk tokens x {w.num_heads} heads of "
                      f"{w.name} ({flops / flops_total:.4f} of the step's "
                      f"attention work)"}


def bench_swap(args):
    """Swapping: `pairs` scattered blocks of the 13B-class shape (40 KV
    heads, 16-token blocks, head_dim 128, fp16: 160 KiB per block per pool)
    copied from the device pools to pinned host pools (out), then back into
    other device blocks (in), one swap_blocks launch each.  For context, the
    same blocks moved by one DMA copy per block (torch copy_, non-blocking)
    and one contiguous DMA copy of the same byte count."""
    import numpy as np
    import torch

    import paged_kv_cache_309_amd as pkv

    nb, hkv, bs, d = 2048, 40, 16, 128
    n = min(args.pairs, nb // 2)
    kd, vd = pkv.new_kv_cache(nb, hkv, bs, d, torch.float16, fill=1.0)
    hk, hv = pkv.new_kv_cache(n, hkv, bs, d, torch.float16, device="cpu",
                              pin_memory=True, fill=0.0)
    rng = np.random.default_rng(args.seed)
    perm = rng.permutation(nb)
    out_pairs = np.stack([perm[:n], np.arange(n)], 1).astype(np.int64)
    in_pairs = np.stack([np.arange(n), perm[n:2 * n]], 1).astype(np.int64)
    m_out = torch.from_numpy(out_pairs).cuda()
    m_in = torch.from_numpy(in_pairs).cuda()
    stream = torch.cuda.current_stream()
    block_bytes = hkv * bs * d * 2
    moved = 2 * n * block_bytes                # K and V, one direction

    def timed(fn, steps):
        for _ in range(max(1, args.warmup // 4)):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    steps = max(1, min(args.steps, 20))
    ms_out = timed(lambda: pkv.swap_blocks(kd, vd, hk, hv, m_out), steps)
    ms_in = timed(lambda: pkv.swap_blocks(hk, hv, kd, vd, m_in), steps)

    def per_block_dma():
        for s_, t_ in out_pairs[:, :].tolist():
            hk[t_].copy_(kd[s_], non_blocking=True)
            hv[t_].copy_(vd[s_], non_blocking=True)
    ms_dma = timed(per_block_dma, max(1, steps // 4))
    flat = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
    src = torch.empty(moved, dtype=torch.uint8, device="cuda")
    ms_flat = timed(lambda: flat.copy_(src, non_blocking=True), steps)
    calibration_copy(args.calib_copy_mib)

    # the copies are bit copies: one sampled block checked after the run
    torch.cuda.synchronize()
    assert torch.equal(hk[0].cuda(), kd[int(out_pairs[0, 0])])

    gbs = lambda ms: moved / (ms * 1e-3) / 1e9
    both = 2 * moved / ((ms_out + ms_in) * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        blk = hkv * bs * d
        src_k = np.zeros(nb * blk, np.float16)
        src_v = np.zeros_like(src_k)
        dst_k = np.zeros(n * blk, np.float16)
        dst_v = np.zeros_like(dst_k)
        t1 = time.perf_counter()
        oracle.swap_blocks(src_k, src_v, dst_k, dst_v, out_pairs, nb, n, "f16")
        dt = time.perf_counter() - t1
        cpu = {"value": round(moved / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "seconds": round(dt, 4),
               "sample": f"the same {n} swap-out block pairs copied by the "
                         f"oracle between host arrays"}
    rec = {"metric": "swap_blocks GB/s over the host link (K and V blocks, "
                     "device to pinned host and back)",
           "value": round(both, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": steps, "warmup": args.warmup,
           "ms_per_step": round(ms_out + ms_in, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "data": "synthetic",
           "config": {"workload": "swap", "pairs": n, "num_blocks": nb,
                      "num_kv_heads": hkv, "block_size": bs, "head_dim": d,
                      "block_bytes_per_pool": block_bytes,
                      "bytes_each_way": moved},
           "swap_out_gbs": round(gbs(ms_out), 2),
           "swap_in_gbs": round(gbs(ms_in), 2),
           "context": {"dma_one_copy_per_block_out_gbs": round(gbs(ms_dma), 2),
                       "dma_contiguous_out_gbs": round(gbs(ms_flat), 2)},
           "roofline": {"bound": "host_link", "achieved": round(both, 2),
                        "peak": HOST_LINK_GBS, "unit": "GB/s",
                        "frac": round(both / HOST_LINK_GBS, 4),
                        "traffic": None, "kernel": "copy_blocks_kernel",
                        "algorithmic_bytes_per_launch": moved,
                        "mean_launch_ms": round((ms_out + ms_in) / 2, 4)},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def cpu_baseline(w, kv_bytes, fp8=False):
    """The oracle, as it stands, on host cores: the same decode step (the
    cache write of the new tokens, then attention for every sequence and
    head).  The pool it reads is built untimed beforehand."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    t0 = time.time()
    cdt = "fp8" if fp8 else w.dtype
    kc, vc = oracle.new_pool(w.num_blocks, w.num_kv_heads, w.block_size,
                             w.head_dim, cdt, fill="zero")

    def write(k, v, slots):
        if fp8:
            oracle.reshape_and_cache_fp8(k, v, kc, vc, slots, w.num_kv_heads,
                                         w.head_dim, w.block_size,
                                         w.num_blocks, w.dtype, 1.0, 1.0)
        else:
            oracle.reshape_and_cache(k, v, kc, vc, slots, w.num_kv_heads,
                                     w.head_dim, w.block_size, w.num_blocks,
                                     w.dtype)

    write(w.kv_k, w.kv_v, w.prefill_slots())
    log(f"[bench] oracle pool built in {time.time()-t0:.1f}s; timing the "
        f"oracle on {threads} threads")
    # whole steps, repeated until about 10 s of CPU work (at most 50)
    t1 = time.perf_counter()
    reps = 0
    while True:
        write(w.new_k(), w.new_v(), w.new_slots())
        out = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.context_lens,
                                  w.scale, w.block_size, w.num_kv_heads,
                                  w.num_blocks, w.dtype, threads=threads,
                                  cache_dtype="fp8" if fp8 else None)
        reps += 1
        if time.perf_counter() - t1 >= 10.0 or reps >= 50:
            break
    dt = (time.perf_counter() - t1) / reps
    assert np.all(np.isfinite(out))
    log(f"[bench] oracle step {dt:.2f}s (mean of {reps})")
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3), "repetitions": reps,
            "sample": f"full decode steps of {w.name} (cache write of "
                      f"{w.num_seqs} new tokens + attention for all "
                      f"{w.num_seqs}x{w.num_heads} (sequence, head) pairs), "
                      f"repeated {reps} times; seconds is one step"}


if __name__ == "__main__":
    main()
