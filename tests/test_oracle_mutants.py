"""Planted mistakes in the oracle must be caught by its pins.

Each case edits one line of a private copy of oracle/oracle.c (a dropped term, a
wrong sign, a wrong or transposed index, ...), builds it into a temporary
library, and runs every pin against it: at least one pin has to fail. This shows
the pins can tell a wrong oracle from a right one. Nothing here touches the GPU.
"""
import ctypes
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import oracle_pins as P  # noqa: E402
from oracle.build import SRC, build

MUTANTS = {
    "block_index_uses_offset": ("block_tables[(long)b * max_blocks + t / bs]",
                                "block_tables[(long)b * max_blocks + t % bs]"),
    "offset_off_by_one": ("(size_t)(t % bs)) * D", "(size_t)((t + 1) % bs)) * D"),
    "gqa_interleaved_heads": ("int g = h / G;", "int g = h % Hkv;"),
    "scale_dropped": ("s[t] = scale * acc;", "s[t] = acc;"),
    "softmax_sign": ("s[t] = exp(s[t] - mx);", "s[t] = exp(mx - s[t]);"),
    "normaliser_wrong": ("o[d] /= denom;", "o[d] /= denom + 1.0;"),
    "first_token_dropped_from_sum": ("denom += s[t];", "denom += t ? s[t] : 0.0;"),
    "keys_and_values_swapped": ("elem(q, qoff + d, q_dtype) * (elem(k_cache",
                                "elem(q, qoff + d, q_dtype) * (elem(v_cache"),
    "last_token_skipped": ("for (int t = 0; t < n; ++t) {\n        int phys",
                           "for (int t = 0; t < n - 1; ++t) {\n        int phys"),
    "slot_block_offset_swapped": ("int64_t blk = slot / bs, off = slot % bs;",
                                  "int64_t blk = slot % bs, off = slot / bs;"),
    "negative_slot_written": ("if (slot < 0) continue;", "if (slot < 0) slot = 0;"),
    "copy_direction_reversed": ("int src = pairs[2 * i], dst = pairs[2 * i + 1];",
                                "int dst = pairs[2 * i], src = pairs[2 * i + 1];"),
    "bf16_shift_wrong": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "f16_bias_wrong": ("expo - 25", "expo - 24"),
    # 8-bit cache: decoder, quantiser, scales, quantising append
    "chunk_causal_off_by_one": ("const int n = context_lens[b] - T + j + 1;",
                                "const int n = context_lens[b] - T + j;"),
    "chunk_not_causal": ("const int n = context_lens[b] - T + j + 1;",
                         "const int n = context_lens[b];"),
    "chunk_rows_reversed": ("const int j = r - query_start[b];",
                            "const int j = query_start[b + 1] - 1 - r;"),
    "chunk_query_row_of_sequence": ("((size_t)r * Hq + h) * D", "((size_t)b * Hq + h) * D"),
    "chunk_row_owner_wrong": ("while (query_start[b + 1] <= r) ++b;",
                              "while (query_start[b + 1] < r) ++b;"),
    "swap_pools_exchanged": ("memcpy((char*)dst_pool + (size_t)to * block_bytes,\n"
                             "               (const char*)src_pool + (size_t)from * block_bytes,",
                             "memcpy((char*)dst_pool + (size_t)from * block_bytes,\n"
                             "               (const char*)src_pool + (size_t)to * block_bytes,"),
    "swap_first_pair_skipped": ("for (int i = 0; i < n; ++i) {\n        const int from",
                                "for (int i = 1; i < n; ++i) {\n        const int from"),
    "fp8_bias_wrong": ("expo - 10", "expo - 9"),
    "fp8_subnormal_step_wrong": ("ldexp((double)mant, -9)", "ldexp((double)mant, -10)"),
    "fp8_ties_away_from_zero": ("(int)nearbyint((2.0 * f - 1.0) * 8.0)",
                                "(int)round((2.0 * f - 1.0) * 8.0)"),
    "fp8_no_saturation": ("if (a >= 448.0) return sign | 0x7E;",
                          "if (a >= 480.0) return sign | 0x7E;"),
    "fp8_subnormal_bound_wrong": ("if (a < ldexp(1.0, -6)) {", "if (a < ldexp(1.0, -7)) {"),
    "fp8_key_scale_dropped": ("(elem(k_cache, at[t] + d, kv_dtype) * k_scale)",
                              "elem(k_cache, at[t] + d, kv_dtype)"),
    "fp8_value_scale_dropped": ("(elem(v_cache, at[t] + d, kv_dtype) * v_scale)",
                                "elem(v_cache, at[t] + d, kv_dtype)"),
    "fp8_append_scales_swapped": ("(float)elem(k, src + d, src_dtype) * k_inv_scale",
                                  "(float)elem(k, src + d, src_dtype) * v_inv_scale"),
    "fp8_append_offset_wrong": ("offset = slot - block * bs;", "offset = slot - block;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib_path = build(str(path), str(tmp_path / f"lib_{name}.so"), extra=("-Wno-error",))
    # Run the pins in a child process: a wrong index may also crash the mutant,
    # which counts as caught.
    proc = subprocess.run([sys.executable, os.path.abspath(__file__), lib_path],
                          capture_output=True, text=True, timeout=600,
                          cwd=os.path.dirname(os.path.abspath(__file__)))
    crashed = proc.returncode < 0                       # killed by a signal (e.g. SIGSEGV)
    flagged = proc.returncode == 1 and "PINS-FAILED" in proc.stdout
    assert crashed or flagged, \
        f"no pin catches the planted mistake {name}:\n{proc.stdout}\n{proc.stderr[-2000:]}"


def test_unmodified_oracle_passes_in_child(tmp_path):
    """Control: the same child-process check passes on the real oracle, so a
    failing mutant is a caught mistake and not a broken harness."""
    lib_path = build(SRC, str(tmp_path / "lib_control.so"))
    proc = subprocess.run([sys.executable, os.path.abspath(__file__), lib_path],
                          capture_output=True, text=True, timeout=600,
                          cwd=os.path.dirname(os.path.abspath(__file__)))
    assert proc.returncode == 0, proc.stdout + proc.stderr


def _run_all_pins(lib_path):
    """Child-process entry: exit 0 only if every pin passes on this library."""
    lib = oracle._bind(ctypes.CDLL(lib_path))
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError) as e:
            failed.append(f"{pin.__name__}: {e}")
    print("PINS-FAILED\n" + "\n".join(failed) if failed else "all pins passed")
    sys.exit(1 if failed else 0)


if __name__ == "__main__":
    _run_all_pins(sys.argv[1])
