"""Plant plausible mistakes in a copy of oracle.c and check the pins catch each.

Every mutant is a one-line textual change to a temporary copy of the oracle
source (the real oracle.c is never touched), compiled into its own shared
library; the pins of test_oracle.py then run against it, and at least one
must fail. This is what gives the pins their power: a pin suite that a
dropped scale or an h % Hkv head map slips through would not be worth much.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle as pins
from tests import test_oracle_rope as rope_pins
from tests import test_oracle_serving as serving_pins

MUTANTS = {
    "gqa_interleaved_prefill": ("uint32_t g = h / heads_per_kv;",
                                "uint32_t g = h % (num_q_heads / heads_per_kv);"),
    "gqa_interleaved_decode": ("uint32_t g = h / repeat;",
                               "uint32_t g = h % kv_heads;"),
    "causal_excludes_diagonal": ("(size_t)i + 1, head_dim, scale",
                                 "(size_t)i, head_dim, scale"),
    "causal_one_extra_key": ("(size_t)i + 1, head_dim, scale",
                             "(size_t)i + 2 > m ? m : (size_t)i + 2, head_dim, scale"),
    "scale_dropped": ("scores[j] = scale * dot;", "scores[j] = dot;"),
    "scale_squared": ("scores[j] = scale * dot;", "scores[j] = scale * scale * dot;"),
    "prefill_scale_wrong": ("return 1.0f / sqrtf((float)head_dim);",
                            "return 1.0f / (float)head_dim;"),
    "exp_sign_flipped": ("scores[j] = exp(scores[j] - mu);",
                         "scores[j] = exp(mu - scores[j]);"),
    "no_normalisation": ("double w = scores[j] / z;", "double w = scores[j];"),
    "max_is_min": ("if (scores[j] > mu)", "if (scores[j] < mu || mu == -INFINITY)"),
    "window_off_by_one": ("? total_seq - window : 0;",
                          "? total_seq - window + 1 : 0;"),
    "window_ignored": ("(window > 0 && total_seq > window)",
                       "(0 && total_seq > window)"),
    "value_stride_transposed": ("const float *vj = v0 + j * row_stride;",
                                "const float *vj = v0 + j * d;"),
    "key_element_fixed": ("dot += (double)q[e] * (double)kj[e];",
                          "dot += (double)q[e] * (double)kj[0];"),
    "query_head_offset": ("const float *qi = q + (size_t)i * q_stride + (size_t)h * head_dim;",
                          "const float *qi = q + (size_t)i * q_stride + (size_t)g * head_dim;"),
    "append_wrong_row": ("+ position)\n                         * head_dim;",
                         "+ position + 1 - (position + 1 == max_seq))\n                         * head_dim;"),
    "append_v_from_k": ("v_cache[dst + e] = v_src[src + e];",
                        "v_cache[dst + e] = k_src[src + e];"),
    "rope_sign": ("out[i] = a * c - b * s;", "out[i] = a * c + b * s;"),
    "rope_pair_index": ("double a = x[i], b = x[i + half]", "double a = x[i], b = x[half - 1 - i]"),
    "rope_step_raw_k": ("dot += qh[e] * kn[e];", "dot += qh[e] * (double)k_raw[((size_t)b * kv_heads + g) * d + e];"),
    "rows_src_ignores_stride": ("size_t src = (size_t)j * kv_stride + (size_t)g * head_dim;",
                                "size_t src = (size_t)j * kv_heads * head_dim + (size_t)g * head_dim;"),
    "rows_dst_row_major": ("size_t dst = ((size_t)g * max_seq + position + j) * head_dim;",
                           "size_t dst = ((size_t)j * kv_heads + g + position) * head_dim;"),
    "rows_v_from_k": ("v_cache[dst + e] = v_src[src + e];\n            }\n        }\n    return 0;\n}\n\n/*\n * Decode of a batch",
                      "v_cache[dst + e] = k_src[src + e];\n            }\n        }\n    return 0;\n}\n\n/*\n * Decode of a batch"),
    "varlen_first_length": ("uint32_t len = seq_lens[b];", "uint32_t len = seq_lens[0];"),
    "varlen_window_ignored": ("(window > 0 && len > window)", "(0 && len > window)"),
    "varlen_idle_skipped": ("o[e] = 0.0;", "o[e] = o[e];"),
}

PIN_CALLS = [
    ("decode_total_seq_one", lambda o, g: pins.test_decode_total_seq_one_is_v_row0(o, g)),
    ("prefill_row0", lambda o, g: pins.test_prefill_row0_is_v_row0(o)),
    ("prefill_scale", lambda o, g: pins.test_prefill_scale_is_f32_inverse_sqrt(o)),
    ("decode_closed_form", lambda o, g: pins.test_decode_closed_form_scores_0_1_2(o)),
    ("prefill_closed_form", lambda o, g: pins.test_prefill_closed_form_scale(o)),
    ("extreme_scores", lambda o, g: pins.test_extreme_scores_stay_finite(o)),
    ("zero_q", lambda o, g: pins.test_prefill_zero_q_is_cumulative_mean(o)),
    ("identical_keys", lambda o, g: pins.test_identical_keys_give_mean_of_v(o)),
    ("future", lambda o, g: pins.test_prefill_future_independence(o)),
    ("gqa_prefill", lambda o, g: pins.test_prefill_gqa_is_mha_with_consecutive_repeat(o)),
    ("gqa_decode", lambda o, g: pins.test_decode_gqa_is_mha_with_consecutive_repeat(o)),
    ("window_trunc", lambda o, g: pins.test_window_equals_truncated_cache(o)),
    ("window_edges", lambda o, g: pins.test_window_edge_values(o)),
    ("cross_mode", lambda o, g: pins.test_cross_mode_decode_equals_prefill_row(o)),
    ("convex", lambda o, g: pins.test_outputs_are_convex_combinations(o)),
    ("sdpa_prefill", lambda o, g: pins.test_prefill_matches_torch_sdpa_fp64(o, 33, 6, 3, 64, 32, 64)),
    ("sdpa_decode", lambda o, g: pins.test_decode_matches_torch_sdpa_fp64(o, 1, 8, 2, 64, 20, 11, 3)),
    ("kv_append", lambda o, g: pins.test_kv_append_writes_only_position(o)),
    ("rope_complex", lambda o, g: rope_pins.test_rope_is_complex_rotation(o)),
    ("rope_special", lambda o, g: rope_pins.test_rope_special_angles(o)),
    ("rope_norms", lambda o, g: rope_pins.test_rope_preserves_pair_norms_and_composes(o)),
    ("rope_relative", lambda o, g: rope_pins.test_rope_relative_position(o)),
    ("rope_step", lambda o, g: rope_pins.test_decode_rope_append_is_rotate_append_decode(o)),
    ("rows_slice", lambda o, g: serving_pins.test_kv_append_rows_is_a_slice_copy(o)),
    ("rows_bounds", lambda o, g: serving_pins.test_kv_append_rows_bounds(o)),
    ("rows_prefill_decode", lambda o, g: serving_pins.test_prefill_then_bulk_append_then_decode(o)),
    ("varlen_sdpa", lambda o, g: serving_pins.test_decode_varlen_matches_sdpa_per_sequence(o, 6)),
    ("varlen_equal", lambda o, g: serving_pins.test_decode_varlen_equal_lengths_is_decode(o)),
    ("varlen_indep", lambda o, g: serving_pins.test_decode_varlen_sequences_are_independent(o)),
]


def _failing_pins(orc, golden):
    failed = []
    for name, call in PIN_CALLS:
        try:
            call(orc, golden)
        except Exception:  # an assertion, or a NaN/shape error from the mutant
            failed.append(name)
    return failed


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("oracle_mutants")


def test_unmutated_copy_passes_every_pin(mutant_dir, golden):
    src = os.path.join(mutant_dir, "same.c")
    with open(oracle.__file__.replace("__init__.py", "oracle.c")) as f:
        text = f.read()
    with open(src, "w") as f:
        f.write(text)
    so = oracle.build(src=src, so_path=os.path.join(mutant_dir, "same.so"))
    assert _failing_pins(oracle.Oracle(so), golden) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(mutant_dir, golden, name):
    old, new = MUTANTS[name]
    with open(oracle.__file__.replace("__init__.py", "oracle.c")) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation anchor for {name} not found"
    src = os.path.join(mutant_dir, f"{name}.c")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    try:
        so = oracle.build(src=src, so_path=os.path.join(mutant_dir, f"{name}.so"))
    except subprocess.CalledProcessError:
        pytest.fail(f"mutant {name} did not compile")
    failed = _failing_pins(oracle.Oracle(so), golden)
    assert failed, f"no pin caught mutant {name}"
