"""The pins must catch plausible slips in the oracle.

Each case copies ``oracle/oracle.c`` to a temporary directory, plants one
mistake by text substitution, builds it with gcc, swaps the mutant in for the
real library and runs the pin suite's key checks.  Every mutant must fail at
least one of them.  CPU only; the real oracle is restored afterwards.
"""

import ctypes
import os
import subprocess

import pytest

import oracle as oracle_pkg

from tests import test_oracle_pins as pins

MUTANTS = {
    "kv_head_modulo": ("kv_heads, h / group, head_dim", "kv_heads, h % kv_heads, head_dim"),
    "causal_offset": ("int64_t p = (int64_t)seq_lens[b] - n + (t - q_start[b]);",
                      "int64_t p = (int64_t)seq_lens[b] - n + (t - q_start[b]) - 1 + (n > 1);"),
    "positions_ignore_cache": ("int64_t p = (int64_t)seq_lens[b] - n + (t - q_start[b]);",
                               "int64_t p = (n > 1) ? (t - q_start[b]) : (int64_t)seq_lens[b] - 1;"),
    "no_max_subtraction": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "no_normalisation": ("out[c] /= l;", "out[c] /= 1.0;"),
    "scores_from_v": ("dot += orc_load(q, q_off + c, dtype) * orc_load(k_pool, base + c, dtype);",
                      "dot += orc_load(q, q_off + c, dtype) * orc_load(v_pool, base + c, dtype);"),
    "strict_mask": ("for (int64_t j = 0; j <= p; ++j) {\n        int64_t base = (int64_t)pt_row[j] * row_elems + kv * head_dim;\n        double dot",
                    "for (int64_t j = 0; j < p || j == 0; ++j) {\n        int64_t base = (int64_t)pt_row[j] * row_elems + kv * head_dim;\n        double dot"),
    "no_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "bf16_widening": ("<< 16;", "<< 15;"),
    "v_head_offset": ("        int64_t base = (int64_t)pt_row[j] * row_elems + kv * head_dim;\n        for (int64_t c = 0; c < head_dim; ++c)\n            out[c] +=",
                      "        int64_t base = (int64_t)pt_row[j] * row_elems;\n        for (int64_t c = 0; c < head_dim; ++c)\n            out[c] +="),
    "lse_without_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "store_swaps_pools": ("memcpy(v_pool + (int64_t)out_loc[t] * row_bytes, v_new",
                          "memcpy(v_pool + (int64_t)out_loc[t] * row_bytes, k_new"),
    "query_row_of_first_token": ("orc_one(dtype, q, (t * q_heads + h) * head_dim",
                                 "orc_one(dtype, q, (q_start[b] * q_heads + h) * head_dim"),
    "rope_sign": ("out[row + i] = x1 * cos(a) - x2 * sin(a);", "out[row + i] = x1 * cos(a) + x2 * sin(a);"),
    "rope_adjacent_pairs": ("double x2 = orc_load(x, row + i + half, dtype);",
                            "double x2 = orc_load(x, row + (i + 1) % head_dim, dtype);"),
    "rope_frequency_exponent": ("pow(base, -2.0 * (double)i / (double)head_dim)",
                                "pow(base, -1.0 * (double)i / (double)head_dim)"),
    "rope_one_angle": ("double a = p * pow(base, -2.0 * (double)i / (double)head_dim);", "double a = p;"),
    "rope_token_index_as_position": ("double p = (double)positions[t];", "double p = (double)t;"),
    "rope_swapped_halves": ("out[row + i + half] = x2 * cos(a) + x1 * sin(a);",
                            "out[row + i + half] = x1 * cos(a) + x2 * sin(a);"),
    "vocab_range_inclusive_end": ("if (r >= 0 && r < rows)", "if (r >= 0 && r <= rows)"),
    "vocab_no_start_offset": ("int64_t r = (int64_t)ids[t] - vocab_start;", "int64_t r = (int64_t)ids[t];"),
    "vocab_stale_rows": ("            memset(out + t * row_bytes, 0, (size_t)row_bytes);", "            ;"),
}

CHECKS = [
    ("bruteforce_decode", lambda o: pins.test_bruteforce_tiny(o, "decode")),
    ("bruteforce_prefill", lambda o: pins.test_bruteforce_tiny(o, "prefill")),
    ("sdpa", pins.test_sdpa_contiguous),
    ("logit_shift", pins.test_logit_shift_invariance),
    ("row_sums", pins.test_row_sums_from_lse),
    ("store_kv", pins.test_store_kv_definition),
    ("bf16", pins.test_bf16_widening_is_exact),
    ("length_one", pins.test_length_one_returns_v),
    ("rope_identity", pins.test_rope_position_zero_is_identity),
    ("rope_complex", pins.test_rope_two_dims_is_complex_rotation),
    ("rope_frequencies", pins.test_rope_four_dims_frequencies),
    ("rope_lengths", pins.test_rope_keeps_pair_lengths),
    ("rope_distance", pins.test_rope_scores_depend_on_distance_only),
    ("vocab_hand", pins.test_vocab_embed_hand_worked),
    ("vocab_full", pins.test_vocab_embed_full_table_is_embedding),
    ("vocab_shards", lambda o: pins.test_vocab_embed_shards_sum_to_full_table(o, 3)),
]


def _build_mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle_pkg.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique / not found"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                           str(path), "-lm"])
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, oracle_mod, name):
    so = _build_mutant(tmp_path, name)
    real = oracle_pkg._load()
    lib = ctypes.CDLL(so)
    for fn in ("oracle_store_kv", "oracle_attention", "oracle_rope", "oracle_vocab_embed",
               "oracle_set_threads", "oracle_num_threads"):
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        getattr(lib, fn).restype = getattr(real, fn).restype
    oracle_pkg._lib = lib
    caught = []
    try:
        for cname, check in CHECKS:
            try:
                check(oracle_pkg)
            except (AssertionError, RuntimeError, ValueError):
                caught.append(cname)
    finally:
        oracle_pkg._lib = real
    assert caught, f"mutant {name} passed every pin"
