"""Plants plausible mistakes in copies of the CPU oracle and checks that the pins
in test_oracle_pins.py catch every one of them.

Each mutant is the oracle's C source with one textual change, compiled with gcc
into a temporary library and swapped in for the real one while the pin checks
run. A mutant that passes every pin would mean the pins cannot tell that mistake
from the definition.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
import test_oracle_pins as pins

MUTANTS = {
    "nibble_order_reversed": ("(word >> (4 * (k % 8)))", "(word >> (4 * (7 - k % 8)))"),
    "group_index_always_zero": ("            int g = k / ORACLE_GROUP;\n            double sc",
                                "            int g = 0 * k;\n            double sc"),
    "bias_dropped": ("sc * (double)oracle_nibble(Wq, K, n, k) + bi;",
                     "sc * (double)oracle_nibble(Wq, K, n, k);"),
    "scale_bias_swapped": ("double sc = oracle_bf16_value(scale[(size_t)n * G + g]);\n"
                           "            double bi = oracle_bf16_value(bias[(size_t)n * G + g]);",
                           "double sc = oracle_bf16_value(bias[(size_t)n * G + g]);\n"
                           "            double bi = oracle_bf16_value(scale[(size_t)n * G + g]);"),
    "operand_k_reversed": ("part += arow[k] * brow[k];", "part += arow[k] * brow[j->K - 1 - k];"),
    "last_group_dropped": ("*g_end = (p + 1) * (G / s);", "*g_end = (p + 1) * (G / s) - (p == s - 1);"),
    "granule_bounds_ceil": ("*u_begin = (int)(((long long)p * U) / s);",
                            "*u_begin = (int)(((long long)p * U + s - 1) / s);"),
    "reduce_in_double": ("float acc = (float)oracle_bf16_value(partials[i]);\n"
                         "        for (int p = 1; p < s; ++p) acc = acc + (float)oracle_bf16_value(partials[(size_t)p * MN + i]);",
                         "double acc = oracle_bf16_value(partials[i]);\n"
                         "        for (int p = 1; p < s; ++p) acc = acc + oracle_bf16_value(partials[(size_t)p * MN + i]);"),
    "round_ties_away": ("(frac == 0.5 && fmod(fl, 2.0) != 0.0)", "(frac == 0.5)"),
    "round_truncates": ("if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;", ""),
    "code_order_reversed": ("(word >> (bits * (k % per_word)))", "(word >> (bits * (per_word - 1 - k % per_word)))"),
    "code_mask_four_bits": ("& ((1u << bits) - 1u));", "& 0xFu);"),
    "format_group_index_128": ("    int g = k / group;\n", "    int g = k / 128;\n"),
    "format_group_count_128": ("    int G = K / group;\n    int g", "    int G = K / 128;\n    int g"),
    "attn_head_map_modulo": ("(size_t)(h / G)) * (size_t)Lmax", "(size_t)(h % Hkv)) * (size_t)Lmax"),
    "attn_mask_off_by_one": ("int nkeys = len[b] - Mq + 1 + i;", "int nkeys = len[b] - Mq + i + (i > 0);"),
    "attn_scale_dropped": ("sc[j] = scale * dot;", "sc[j] = dot;"),
    "attn_not_normalised": ("o[d] = acc / denom;", "o[d] = acc;"),
    "attn_values_from_keys": ("acc += sc[j] * oracle_bf16_value(V[kv", "acc += sc[j] * oracle_bf16_value(K[kv"),
    "format_bias_dropped": ("return sc * (double)oracle_code(Wq, bits, K, n, k) + bi;",
                            "return sc * (double)oracle_code(Wq, bits, K, n, k);"),
}

# The pin checks run against each mutant (a representative of every pin family).
CHECKS = [
    (pins.test_bf16_round_matches_torch_on_fp32, {}),
    (pins.test_bf16_round_ties_to_even_by_hand, {}),
    (pins.test_nibble_order_golden, {}),
    (pins.test_dequant_matches_generator_fields_exactly, {}),
    (pins.test_bruteforce_exact_rationals, dict(M=2, N=3, K=256)),
    (pins.test_bruteforce_dense_exact_rationals, {}),
    (pins.test_closed_form_zero_weights, dict(s=4)),
    (pins.test_closed_form_ones_times_nine, {}),
    (pins.test_closed_form_one_hot_rows, dict(s=2)),
    (pins.test_integer_weights_equal_numpy_matmul, {}),
    (pins.test_dense_equals_numpy_matmul_and_split_invariant, {}),
    (pins.test_reduce_bf16_matches_torch, dict(s=5, M=48, N=1000)),
    (pins.test_reduce_bf16_is_fp32_then_one_cast, {}),
    (pins.test_reduce_f32_matches_torch, dict(s=6, M=32, N=40)),
    (pins.test_granule_partitions_near_equal, {}),
    (pins.test_group_partitions_equal_and_covering, {}),
    (pins.test_code_order_golden, {}),
    (pins.test_format_dequant_matches_generator_fields, dict(bits=8, group=32)),
    (pins.test_format_bruteforce_exact_rationals, dict(bits=8, group=64)),
    (pins.test_format_one_hot_rows, dict(bits=4, group=32)),
    (pins.test_format_integer_weights_equal_numpy_matmul, dict(bits=8)),
    (pins.test_attn_single_key_returns_its_value_row, {}),
    (pins.test_attn_zero_query_averages_the_allowed_values, {}),
    (pins.test_attn_two_keys_closed_form, {}),
    (pins.test_attn_query_heads_share_their_group_key_value_head, {}),
    (pins.test_attn_causal_queries_match_shorter_histories, {}),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, "mutation anchor for %s not found exactly once" % name
    path_c = os.path.join(str(tmp_path), name + ".c")
    path_so = os.path.join(str(tmp_path), name + ".so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", *obuild.CFLAGS, path_c, "-o", path_so, "-lm"], check=True)
    return path_so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    so = _build_mutant(tmp_path, name, old, new)
    real = oracle._lib()
    mutant = ctypes.CDLL(so)
    # copy the ctypes signatures of the real library onto the mutant
    for fn in ("oracle_bf16_value", "oracle_bf16_round", "oracle_nibble", "oracle_dequant_w4a16",
               "oracle_partition_groups", "oracle_partition_granules", "oracle_qmm_w4a16",
               "oracle_qmm_w4a16_points", "oracle_qmm_dense", "oracle_reduce_bf16", "oracle_reduce_f32",
               "oracle_code", "oracle_dequant_wq", "oracle_qmm_wq", "oracle_qmm_wq_points", "oracle_attn_decode"):
        getattr(mutant, fn).argtypes = getattr(real, fn).argtypes
        getattr(mutant, fn).restype = getattr(real, fn).restype
    caught = []
    oracle._LIB = mutant
    try:
        for fn, kw in CHECKS:
            try:
                fn(**kw)
            except (AssertionError, ValueError):
                caught.append(fn.__name__)
    finally:
        oracle._LIB = real
    assert caught, "mutant %s passed every pin" % name
