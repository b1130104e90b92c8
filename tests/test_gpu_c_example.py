"""The C ABI from a plain C program: examples/decode_step.c allocates with
the HIP runtime, calls reshape_and_cache, paged_attention_decode and
paged_attention_decode_split on a stream of its own (no Python or torch in
that process), and dumps its inputs and both outputs; here they are checked
against the oracle on the same inputs."""
import os
import subprocess

import numpy as np
import pytest

import examples
import oracle
from gpu_util import compare

pytestmark = pytest.mark.gpu


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_c_program_decode_step_matches_oracle(tmp_path):
    if not os.path.exists(examples.EXE):
        examples.build()
    dump = tmp_path / "decode_step.bin"
    print("[c example] running examples/decode_step", flush=True)
    r = subprocess.run([examples.EXE, str(dump)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    print(r.stdout.strip(), flush=True)

    raw = dump.read_bytes()
    pos = 0

    def take(dtype, count):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=pos)
        pos += a.nbytes
        return a.copy()
    S, Hq, Hkv, D, bs, NB, MB, T, part, _ = take(np.int32, 10).tolist()
    scale = float(take(np.float32, 1)[0])
    lens = take(np.int32, S)
    tables = take(np.int32, S * MB).reshape(S, MB)
    slots = take(np.int64, T)
    k_rows = take(np.uint16, T * Hkv * D).reshape(T, Hkv, D)
    v_rows = take(np.uint16, T * Hkv * D).reshape(T, Hkv, D)
    q = take(np.uint16, S * Hq * D).reshape(S, Hq, D)
    out_single = take(np.uint16, S * Hq * D).reshape(S, Hq, D)
    out_split = take(np.uint16, S * Hq * D).reshape(S, Hq, D)
    assert pos == len(raw)
    assert (S, Hq, Hkv, D, bs, part) == (3, 8, 2, 64, 16, 16)

    kc, vc = oracle.new_pool(NB, Hkv, bs, D, "bf16")
    oracle.reshape_and_cache(k_rows, v_rows, kc, vc, slots, Hkv, D, bs, NB, "bf16")
    want = oracle.paged_decode(q, kc, vc, tables, lens, scale, bs, Hkv, NB, "bf16")
    compare(bf16_to_f64(out_single), want, "bf16", "C program, single pass")
    compare(bf16_to_f64(out_split), want, "bf16", "C program, split")
