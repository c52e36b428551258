"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of oracle/fd_oracle.c with one plausible mistake
planted in it, compiled with gcc into a temporary directory.  The pins of
test_oracle_pins.py (not the regression snapshot) are run against it; at
least one of them must fail, otherwise that mistake would go unnoticed.
"""
import os
import subprocess
import tempfile

import pytest

import test_oracle_pins as pins
from oracle import oracle as oracle_py

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(
    __file__))), "oracle", "fd_oracle.c")

# (name, text in fd_oracle.c, replacement); every occurrence is replaced.
MUTANTS = [
    ("f16_exponent_bias", "v = ldexp((double)(m | 0x400), e - 25);",
     "v = ldexp((double)(m | 0x400), e - 24);"),
    ("f16_subnormal_scale", "v = ldexp((double)m, -24);",
     "v = ldexp((double)m, -25);"),
    ("f16_implicit_bit_dropped", "v = ldexp((double)(m | 0x400), e - 25);",
     "v = ldexp((double)m, e - 25);"),
    ("lse_in_base2", "*lse = m + log(l);", "*lse = m + log2(l);"),
    ("lse_without_max", "*lse = m + log(l);", "*lse = log(l);"),
    ("scale_dropped", "double s = scale * dot;", "double s = dot;"),
    ("gqa_map_h_mod_hkv", "int g = h / G;", "int g = h % Hkv;"),
    ("q_row_from_kv_head", "size_t q_off = ((size_t)b * Hq + h) * D;",
     "size_t q_off = ((size_t)b * Hq + g) * D;"),
    ("k_and_v_swapped", "load_elem(k, r + d, dtype)",
     "load_elem(v, r + d, dtype)"),
    ("exp_sign_flipped", "double p = exp(scratch[j] - m);",
     "double p = exp(m - scratch[j]);"),
    ("not_normalised", "        out[d] /= l;\n", "\n"),
    ("last_key_dropped",
     "for (int j = 0; j < L; ++j) {\n        const size_t r = row_off ? "
     "row_off[j] : kv_off + (size_t)j * D;\n        double p",
     "for (int j = 0; j < L - 1; ++j) {\n        const size_t r = row_off ? "
     "row_off[j] : kv_off + (size_t)j * D;\n        double p"),
    ("seqlens_ignored", "    if (!seqlens)\n        return Lmax;",
     "    return Lmax;"),
    ("merge_weight_sign", "double w = exp(pl[c] - M);",
     "double w = exp(M - pl[c]);"),
    ("merge_not_normalised", "            out[d] /= W;\n", "\n"),
    ("merge_lse_no_max", "*lse = M + log(W);", "*lse = log(W);"),
    ("chunk_offset_in_rows", "(size_t)lo * D, NULL", "(size_t)lo, NULL"),
    ("chunk_tail_dropped", "        if (n > chunk)\n            n = chunk;",
     "        if (n > chunk || n < chunk)\n            n = chunk < n ? chunk : n - 1;"),
    ("paged_token_index", "size_t t = (size_t)(j % page_size);",
     "size_t t = (size_t)(j / page_size);"),
    ("paged_head_ignored", "((pg * page_size + t) * Hkv + g)",
     "((pg * page_size + t) * Hkv + 0)"),
    ("paged_head_major_ignored", "if (head_major)\n                    roff",
     "if (0)\n                    roff"),
    ("paged_head_major_wrong_head", "((pg * Hkv + g) * page_size + t)",
     "((pg * Hkv + (Hkv - 1 - g)) * page_size + t)"),
    ("paged_page_of_token_zero", "                                j / page_size];",
     "                                0];"),
    ("multiquery_not_causal", "- (Tq - 1 - t);", "- 0;"),
    ("paged_multiquery_not_causal", "L -= Tq - 1 - tok;", "L -= 0;"),
    ("paged_multiquery_token_ignored", "int tok = (int)((r / Hq) % Tq);",
     "int tok = Tq - 1;"),
    ("paged_multiquery_q_row", "attend_row(q, (size_t)r * D, k_pages",
     "attend_row(q, (size_t)(r % ((long)Tq * Hq) % Hq) * D, k_pages"),
    ("multiquery_causal_reversed", "- (Tq - 1 - t);", "- t;"),
    ("multiquery_q_row", "attend_row(q, (size_t)r * D, k, v, kv_off",
     "attend_row(q, (size_t)(r % Hq) * D, k, v, kv_off"),
]

PINS = [
    (pins.test_single_key_returns_its_value_row, ("bf16",)),
    (pins.test_single_key_returns_its_value_row, ("f32",)),
    (pins.test_scale_zero_gives_mean_of_values, ()),
    (pins.test_identical_keys_give_mean_and_shifted_lse, ()),
    (pins.test_two_keys_closed_form, ()),
    (pins.test_dominant_key_returns_its_row, ()),
    (pins.test_gqa_head_map_is_h_div_group, ()),
    (pins.test_padding_beyond_seqlen_is_never_read, ()),
    (pins.test_seqlen_zero_and_clamping, ()),
    (pins.test_nan_inside_valid_prefix_propagates, ()),
    (pins.test_joint_permutation_of_rows_is_invisible, ()),
    (pins.test_affine_map_of_values_passes_through, ()),
    (pins.test_common_score_shift_moves_lse_only, ()),
    (pins.test_split_and_merge_equals_unsplit, (100, 7, 0)),
    (pins.test_split_and_merge_equals_unsplit, (100, 33, 3)),
    (pins.test_split_and_merge_equals_unsplit, (257, 64, 0)),
    (pins.test_split_batch_twin_matches_batch, ()),
    (pins.test_torch_fp64_attention_agrees, ()),
    (pins.test_mpmath_brute_force_50_digits, ()),
    (pins.test_paged_equals_contiguous_after_scatter, (32, False, "bf16")),
    (pins.test_paged_equals_contiguous_after_scatter, (64, False, "bf16")),
    (pins.test_paged_equals_contiguous_after_scatter, (32, True, "bf16")),
    (pins.test_paged_equals_contiguous_after_scatter, (16, False, "f32")),
    (pins.test_paged_multiquery_equals_contiguous_after_scatter,
     (False, "bf16")),
    (pins.test_paged_multiquery_equals_contiguous_after_scatter,
     (False, "f32")),
    (pins.test_multiquery_single_token_is_decode, ("bf16",)),
    (pins.test_f16_decoding_matches_numpy_for_every_bit_pattern, ()),
    (pins.test_multiquery_single_token_is_decode, ("f32",)),
    (pins.test_multiquery_identical_keys_closed_form, ()),
    (pins.test_multiquery_query_never_sees_later_tokens, ()),
]


def _build(src_text: str, out_dir: str, name: str) -> str:
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off",
                    "-shared", "-fPIC", c, "-o", so, "-lm"], check=True)
    return so


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_planted_mistake_fails_a_pin(name, old, new):
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as d:
        variant = oracle_py.Variant(_build(src.replace(old, new), d, name))
        caught = []
        for fn, args in PINS:
            try:
                fn(variant, *args)
            except (AssertionError, ValueError):
                caught.append(fn.__name__)
                break
        assert caught, f"mutant {name} passed every pin"


def test_unmutated_source_passes_every_pin():
    with tempfile.TemporaryDirectory() as d:
        variant = oracle_py.Variant(_build(open(SRC).read(), d, "clean"))
        for fn, args in PINS:
            fn(variant, *args)
