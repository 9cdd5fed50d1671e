"""Negative controls for the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle source, builds
it, and checks that at least one pin from test_oracle_pins fails against the
mutant.  A pin set that lets a planted mistake through would be too weak.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "kv4_oracle.c")

# (name, text to replace, replacement, pins that must catch it)
MUTATIONS = [
    ("scores_drop_rope", "for (i = 0; i < D; ++i) acc +=", "for (i = 0; i < a->n_latent; ++i) acc +=",
     ["dense", "rope"]),
    ("nibble_order_swapped", "if (e & 1) codes[e >> 1] |= (uint8_t)(c << 4);\n            else       codes[e >> 1] |= c;",
     "if (e & 1) codes[e >> 1] |= c;\n            else       codes[e >> 1] |= (uint8_t)(c << 4);",
     ["roundtrip", "closed_bytes"]),
    ("e2m1_ties_away", "(d == bestd && (code & 1) == 0 && (best & 1) == 1)) {\n            bestd = d;\n            best = (uint8_t)code;\n        }\n    }\n    return (uint8_t)(best | (signbit(y)",
     "(d == bestd)) {\n            bestd = d;\n            best = (uint8_t)code;\n        }\n    }\n    return (uint8_t)(best | (signbit(y)",
     ["e2m1_grid"]),
    ("scale_by_reciprocal", "scale_f = amax / 6.0f;", "scale_f = amax * (1.0f / 6.0f);", ["scale_division"]),
    ("scale_amax_over_4", "scale_f = amax / 6.0f;", "scale_f = amax / 4.0f;", ["scale_argmin", "roundtrip"]),
    ("lse_without_log", "= m + log(l);", "= m + l;", ["closed_forms"]),
    ("sm_scale_dropped", "s[j] = a->sm_scale * acc;", "s[j] = acc;", ["dense", "closed_forms"]),
    ("page_offset_wrong", "slot = (int64_t)phys * page_size + pos % page_size;",
     "slot = (int64_t)phys * page_size + pos / page_size;", ["translate", "dense"]),
    ("values_include_rope", "o[d] += p * K[(int64_t)j * D + d];", "o[d] += p * K[(int64_t)j * D + d + 64];",
     ["dense", "closed_forms"]),
    ("dedup_keeps_last", "if (j == 0 || pairs[j].v != pairs[j - 1].v) keep[nk++] = pairs[j].pos;",
     "if (j == np - 1 || pairs[j].v != pairs[j + 1].v) keep[nk++] = pairs[j].pos;", ["dedup"]),
    ("merge_weight_sign", "w = exp(ls - M);", "w = exp(M - ls);", ["merge"]),
    ("compact_rank_skips_one", "rank[s] = count;", "rank[s] = count + (count > 0);", ["compact"]),
    ("compact_keeps_first_page_only", "if (slot >= 0) seen[slot] = 1;", "if (slot >= 0 && slot < 64) seen[slot] = 1;",
     ["compact"]),
    ("mse_ties_to_largest_code", "if (err < best_err) {", "if (err <= best_err) {", ["mse_hand"]),
    ("mse_search_starts_at_base", "for (code = 0; code <= 0x7E; ++code) {\n        float err",
     "for (code = base; code <= 0x7E; ++code) {\n        float err", ["mse_brute"]),
    ("mse_error_skips_last_value", "for (i = 0; i < 16; ++i) {\n        float cd",
     "for (i = 0; i < 15; ++i) {\n        float cd", ["mse_brute", "mse_exact"]),
    ("mse_absolute_error", "s = fmaf(e, e, s);", "s = s + fabsf(e);", ["mse_brute"]),
    ("rope_scaled_like_latent", "for (i = 0; i < n_rope; ++i) rope[i] = o_e4m3_encode(x[n_latent + i]);",
     "for (i = 0; i < n_rope; ++i) rope[i] = o_e4m3_encode(x[n_latent + i] / 6.0f);", ["roundtrip", "scale_argmin"]),
]

PINS = {
    "dense": lambda: P.test_attention_equals_dense_when_topk_covers_context(0),
    "rope": P.test_attention_rope_dims_enter_scores_only,
    "roundtrip": P.test_quantize_roundtrip_exact_on_representable_rows,
    "closed_bytes": P.test_quantize_closed_form_bytes,
    "e2m1_grid": P.test_e2m1_encode_grid_and_ties,
    "scale_argmin": P.test_quantize_scale_is_nearest_e4m3_of_amax_over_6_and_codes_are_argmin,
    "scale_division": lambda: P.test_scale_uses_fp32_division_at_e4m3_midpoints(),
    "closed_forms": P.test_attention_closed_forms,
    "translate": P.test_translate_matches_page_arithmetic,
    "dedup": lambda: P.test_dedup_matches_brute_force(300),
    "merge": P.test_merge_of_split_lists_equals_whole_list,
    "compact": lambda: P.test_global_compact_matches_brute_force(0),
    "mse_hand": P.test_mse_scale_hand_worked_block,
    "mse_exact": P.test_mse_exact_fit_blocks_round_trip,
    "mse_brute": lambda: [P.test_mse_scale_minimizes_squared_error_brute_force(k) for k in ("normal", "outlier")],
}


@pytest.mark.parametrize("name,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, pins):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found: " + name
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mut.c")
        so = os.path.join(d, "libmut.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-shared",
                               "-fPIC", c, "-o", so, "-lm"])
        caught = []
        with oracle.using_library(so):
            for p in pins:
                try:
                    PINS[p]()
                except AssertionError:
                    caught.append(p)
        assert caught, "planted mistake %s passed every pin %s" % (name, pins)
