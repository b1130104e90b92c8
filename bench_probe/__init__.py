"""Measurement helper of bench.py: a trivial tile-read kernel that gives
the read bandwidth the GPU delivers to the paged decode's access pattern
(independent 4 KiB tiles at random places), as context for the roofline.
Built by build(); not part of the library."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libpkv_probe.so")


def build() -> str:
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    cmd = [cc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wl,-z,defs", "-o", LIB + ".tmp", os.path.join(HERE, "read_probe.hip")]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def random_tile_read_gbs(gib: int = 4, tiles: int = 1 << 19, reps: int = 10) -> float:
    """GB/s of `tiles` random 4 KiB tiles (a permutation sample) of a
    `gib` GiB device buffer."""
    import numpy as np
    import torch
    lib = ctypes.CDLL(LIB)
    lib.pkv_probe_read_tiles.restype = ctypes.c_int
    lib.pkv_probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    n_all = (gib << 30) // 4096
    buf = torch.ones((gib << 30) // 2, dtype=torch.float16, device="cuda")
    order = torch.from_numpy(np.random.default_rng(0).permutation(n_all)[:tiles]
                             .astype(np.int64)).cuda()
    grid = 2048
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        rc = lib.pkv_probe_read_tiles(buf.data_ptr(), order.data_ptr(), tiles, grid,
                                      sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"probe launch failed: {rc}")
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del buf
    return round(tiles * 4096 / (ms * 1e-3) / 1e9, 1)
