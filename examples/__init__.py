"""Programs that use the library the way a C caller would, and their build.

build(): compiles examples/decode_step.c with the host C compiler against
the HIP runtime and the in-tree libpkv.so (host code only: the kernels are
in the library).  The binary sits next to its source and finds the library
through a relative run path.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "decode_step.c")
EXE = os.path.join(HERE, "decode_step")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler to build the examples")
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", SRC,
           f"-L{ROOT}/paged_kv_cache_309_amd", "-lpkv", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../paged_kv_cache_309_amd", f"-Wl,-rpath,{ROCM}/lib",
           "-lm", "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building examples/decode_step failed:\n" + r.stdout + r.stderr)
    return EXE
