"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/paged_oracle.c`` (on the
CPU, in a temporary build), points the oracle wrapper at that build, and
requires at least one of the pins in ``test_oracle_pins`` to fail.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_blocks as blockpins
import test_oracle_fp8 as fp8pins
import test_oracle_prefill as prefillpins
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "paged_oracle.c")

MUTANTS = {
    "k_layout_heads_offsets_swapped": (
        "return ((p * hkv + g) * bs + o) * hd + d;",
        "return ((p * bs + o) * hkv + g) * hd + d;"),
    "v_layout_untransposed": (
        "(o / 4) * 4 * hd + d * 4 + (o % 4);",
        "o * hd + d;"),
    "slot_block_offset_swapped": (
        "size_t p = (size_t)(s / block_size), o = (size_t)(s % block_size);",
        "size_t o = (size_t)(s / block_size), p = (size_t)(s % block_size);"),
    "table_indexed_by_offset": (
        "    int p = table[t / bs];\n    int o = t % bs;\n    if (p < 0",
        "    int p = table[t % bs < jb->max_blocks_per_seq ? t % bs : 0];\n"
        "    int o = t % bs;\n    if (p < 0"),
    "scale_dropped": ("x[t] = jb->scale * dot;", "x[t] = dot;"),
    "max_sign_flipped": ("double w = exp(x[t] - m);",
                         "double w = exp(m - x[t]);"),
    "last_token_dropped": ("for (int t = 0; t < L; ++t) {\n    int p = table[t / bs];\n    int o = t % bs;\n    double w",
                           "for (int t = 0; t < L - 1; ++t) {\n    int p = table[t / bs];\n    int o = t % bs;\n    double w"),
    "gqa_interleaved": ("const int g = h / group;",
                        "const int g = h % jb->num_kv_heads;"),
    "not_normalised": ("out[d] /= z;", "out[d] /= 1.0;"),
    "fp16_exponent_bias": ("ex - 25);", "ex - 24);"),
    "bf16_wrong_half": ("uint32_t u = (uint32_t)b << 16;",
                        "uint32_t u = (uint32_t)b << 15;"),
    "query_head_ignored": ("qbase = ((size_t)qrow * jb->num_heads + h) * hd;",
                           "qbase = ((size_t)qrow * jb->num_heads) * hd;"),
    "e4m3_exponent_bias": ("ldexp((double)(8 + fr), ex - 10)",
                           "ldexp((double)(8 + fr), ex - 11)"),
    "e4m3_ties_to_odd": ("(a - vlo == vhi - a && (lo & 1))",
                         "(a - vlo == vhi - a && !(lo & 1))"),
    "key_scale_dropped": ("              jb->k_scale);", "              1.0);"),
    "cache_scale_multiplied": ("e4m3_encode(xk / jb->k_scale)",
                               "e4m3_encode(xk * jb->k_scale)"),
    "copy_blocks_reversed": (
        "memcpy((char *)k_cache + d * bytes, (const char *)k_cache + s * bytes, bytes);",
        "memcpy((char *)k_cache + s * bytes, (const char *)k_cache + d * bytes, bytes);"),
    "causal_excludes_self": (
        "L = (int)(jb->context_lens[s] - C + (r - qsl[s]) + 1);",
        "L = (int)(jb->context_lens[s] - C + (r - qsl[s]));"),
    "chunk_at_the_start": (
        "L = (int)(jb->context_lens[s] - C + (r - qsl[s]) + 1);",
        "L = (int)((r - qsl[s]) + 1);"),
    "swap_values_from_keys": (
        "memcpy((char *)dst_v + d * bytes, (const char *)src_v + s * bytes, bytes);",
        "memcpy((char *)dst_v + d * bytes, (const char *)src_k + s * bytes, bytes);"),
}


def _pin_calls():
    calls = [lambda c=c: pins.test_matches_contiguous_attention(c)
             for c in range(len(pins.SWEEP))]
    calls += [
        pins.test_one_hot_probe_every_position_bit_exact,
        pins.test_worked_request_walk,
        pins.test_scattered_table_diagram,
        pins.test_fp16_decoding_exhaustive,
        pins.test_bf16_decoding_exhaustive,
        pins.test_single_token_returns_its_value_exactly,
    ]
    calls += [lambda a=a: pins.test_cache_write_matches_numpy_view_scatter(*a)
              for a in [("f32", 16, 64), ("bf16", 8, 8)]]
    calls += [fp8pins.test_decode_every_code,
              fp8pins.test_encode_matches_library_in_range_including_ties,
              fp8pins.test_encode_saturates_and_keeps_nan]
    calls += [lambda a=a: fp8pins.test_quantising_cache_write_matches_view_scatter(*a)
              for a in [("bf16", 1.0), ("f16", 0.05)]]
    calls += [lambda a=a: fp8pins.test_decode_on_quantised_cache_is_attention_on_dequantised_values(*a)
              for a in [("bf16", 8, 2)]]
    calls += [lambda: blockpins.test_copy_blocks_is_row_assignment("f32", 12, 2, 16, 64, 5),
              lambda: blockpins.test_swap_blocks_is_row_assignment("bf16", 30, 10, 7),
              blockpins.test_swap_blocks_round_trip_and_rejections]
    calls += [lambda c=c: prefillpins.test_matches_masked_contiguous_attention(c)
              for c in (0, 2)]
    return calls


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    # a mistake in a formula the oracle writes out more than once is planted
    # everywhere that formula appears
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread",
                    "-w", "-o", str(lib), str(mutated), "-lm"], check=True)
    caught = 0
    with oracle.use_library(str(lib)):
        for call in _pin_calls():
            try:
                call()
            except (AssertionError, oracle.OracleError):
                caught += 1
                break
    assert caught, f"no pin caught the planted mistake {name}"
