"""Pins are strong enough: each plausible mistake planted in a copy of the
oracle's C source (on the CPU, in a temporary directory) must make at least
one pin fail.  The oracle itself is never modified."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

from oracle import oracle as O

MUTANTS = {
    "relu_dropped": ("head_sum += (dot > 0.0) ? dot : 0.0;", "head_sum += dot;"),
    "relu_after_head_sum": ("head_sum += (dot > 0.0) ? dot : 0.0;",
                            "head_sum += dot; if (h == 3 && head_sum < 0) head_sum = 0;"),
    "scale_as_divisor": ("return (float)(head_sum * (double)scale);",
                         "return (float)(head_sum / (double)scale);"),
    "head_dropped": ("for (int h = 0; h < QSA_ORACLE_HEADS; ++h) {",
                     "for (int h = 0; h < QSA_ORACLE_HEADS - 1; ++h) {"),
    "head_stride_ignored": ("q_off + h * q_stride_head + d, q_format)", "q_off + h * QSA_ORACLE_DIM + d, q_format)"),
    "feature_index_shifted": ("double kv = element(k, k_off + d, k_format);",
                              "double kv = element(k, k_off + (d + 1) % QSA_ORACLE_DIM, k_format);"),
    "bf16_widening_wrong": ("uint32_t u = ((uint32_t)bits) << 16;",
                            "uint32_t u = ((uint32_t)bits) << 15;"),
    "visible_off_by_one": ("int64_t by_pos = floor_div(pos + 1, compress_ratio);",
                           "int64_t by_pos = floor_div(pos, compress_ratio);"),
    "position_ignores_request_start": ("+ (t - query_start_loc[req]);", "+ t;"),
    "decode_mask_inclusive": ("if (c < seen) {", "if (c <= seen && c < comp_lens[r]) {"),
    "decode_no_comp_clamp": ("if (seen > comp_lens[r]) seen = comp_lens[r];", ""),
    "page_slot_swapped": ("int64_t slot = c / page_size;", "int64_t slot = c % page_size;"),
    "page_row_wrong": ("(page * page_size + (c % page_size))", "(page * page_size + (c / page_size))"),
    "page_range_unchecked": ("if (page >= 0 && page < num_pages) {", "if (page >= 0) {"),
    "page_table_width_unchecked": ("if (slot < page_table_cols) {", "if (slot < page_table_cols + 1) {"),
    "decode_row_request_wrong": ("int32_t r = row / dql;", "int32_t r = row % dql;"),
    "intervals_offset_by_token": ("int32_t start = key_offsets[token_to_req[t]];",
                                  "int32_t start = key_offsets[t % 4];"),
    "intervals_end_without_offset": ("row_k_end[t] = start + visible[t];", "row_k_end[t] = visible[t];"),
    "intervals_end_one_short": ("row_k_end[t] = start + visible[t];", "row_k_end[t] = start + visible[t] - 1;"),
    "ring_null_block_written": ("if (block <= 0) break;\n            slot = block * ring_size", "if (block < 0) break;\n            slot = block * ring_size"),
    "ring_every_token_writes": ("if ((int64_t)t + ring_size < query_end) break;", ""),
    "ring_row_by_division": ("slot = block * ring_size + pos % ring_size;", "slot = block * ring_size + pos / ring_size;"),
    "ring_column_one": ("int64_t block = block_table[r * block_table_stride];", "int64_t block = block_table[r * block_table_stride + 1];"),
    "ring_negative_positions_written": ("if (pos < 0) break;\n            if ((int64_t)t + ring_size", "if (pos < -1) break;\n            if ((int64_t)t + ring_size"),
    "write_e4m3_scale_multiplies": ("float_to_e4m3_bits((float)bf16_bits_to_double(src[d]) / scale)",
                                    "float_to_e4m3_bits((float)bf16_bits_to_double(src[d]) * scale)"),
    "write_positions_axes_swapped": ("int64_t v = positions[a * pos_stride_axis + (int64_t)t * pos_stride_token];",
                                     "int64_t v = positions[(2 - a) * pos_stride_axis + (int64_t)t * pos_stride_token];"),
    "write_slot_upper_bound_unchecked": ("if (s < 0 || s >= num_slots) continue;", "if (s < 0) continue;"),
    "write_key_stride_ignored": ("const uint16_t *src = keys + (int64_t)t * key_stride;",
                                 "const uint16_t *src = keys + (int64_t)t * 64;"),
    "prefill_absolute_columns": ("int64_t n = (int64_t)row_k_start[t] + c;", "int64_t n = c;"),
    "prefill_end_inclusive": ("n < row_k_end[t])", "n <= row_k_end[t])"),
    "prefill_no_lower_bound": ("if (n >= 0 && n < num_keys", "if (n >= -2 && n < num_keys"),
    "topk_ties_high_index": ("return (x->col > y->col) - (x->col < y->col);\n}\n\nstatic int by_col",
                             "return (x->col < y->col) - (x->col > y->col);\n}\n\nstatic int by_col"),
    "topk_keeps_neg_inf": ("if (row[c] > neg_inf()) {", "if (row[c] >= neg_inf()) {"),
    "topk_descending_output": ("qsort(cand, (size_t)keep, sizeof(oracle_cand), by_col);", ""),
    "fp16_exponent_bias_wrong": ("v = ldexp((double)(1024 + fraction), exponent - 25);",
                                 "v = ldexp((double)(1024 + fraction), exponent - 24);"),
    "fp16_subnormal_scale_wrong": ("v = ldexp((double)fraction, -24);", "v = ldexp((double)fraction, -25);"),
    "fp16_sign_dropped": ("    return sign ? -v : v;\n}\n\n/* OCP", "    return v;\n}\n\n/* OCP"),
    "e4m3_bias_of_fnuz": ("v = ldexp((double)(8 + fraction), exponent - 10);",
                          "v = ldexp((double)(8 + fraction), exponent - 11);"),
    "e4m3_subnormal_scale_wrong": ("v = ldexp((double)fraction, -9);", "v = ldexp((double)fraction, -10);"),
    "e4m3_no_implicit_one": ("ldexp((double)(8 + fraction), exponent - 10)", "ldexp((double)(fraction), exponent - 7)"),
    "e4m3_top_binade_as_nan": ("if (exponent == 15 && fraction == 7)", "if (exponent == 15)"),
    "k_scale_divides": ("if (k_format == ORACLE_FP8_E4M3) kv *= k_scale;",
                        "if (k_format == ORACLE_FP8_E4M3) kv /= k_scale;"),
    "k_scale_ignored": ("if (k_format == ORACLE_FP8_E4M3) kv *= k_scale;", ""),
    "typed_query_read_as_bf16": ("dot += element(q, q_off + h * q_stride_head + d, q_format) * kv;",
                                 "dot += element(q, q_off + h * q_stride_head + d, ORACLE_BF16) * kv;"),
    "typed_prefill_key_stride_ignored": ("n * k_stride, k_format, k_scale, scale);",
                                         "n * QSA_ORACLE_DIM, k_format, k_scale, scale);"),
    "typed_decode_page_row_wrong": ("int64_t k_off = (page * page_size + (c % page_size)) * QSA_ORACLE_DIM;",
                                    "int64_t k_off = (page * page_size + (c / page_size)) * QSA_ORACLE_DIM;"),
    "slot_closing_test_shifted": ("if (pos < 0 || (pos + 1) % compress_ratio != 0) break;",
                                  "if (pos < 0 || pos % compress_ratio != 0) break;"),
    "slot_row_in_block_wrong": ("slot = block * storage_block_size + cp % storage_block_size;",
                                "slot = block * storage_block_size + cp / storage_block_size;"),
    "slot_table_width_unchecked": ("if (logical_block >= block_table_cols) break;",
                                   "if (logical_block > block_table_cols) break;"),
    "slot_block_zero_rejected": ("if (block < 0) break;", "if (block <= 0) break;"),
    "slot_main_cache_ignored": ("if (common_slot_mapping && common_slot_mapping[t] < 0) break;", ""),
    "slot_compressed_position_wrong": ("int64_t cp = pos / compress_ratio;", "int64_t cp = (pos + 1) / compress_ratio;"),
    "work_no_minimum_item": ("int64_t count = groups > 1 ? groups : 1;", "int64_t count = groups;"),
    "work_empty_requests_counted": ("if (query_len <= 0) continue;", "if (query_len < 0) continue;"),
    "work_chunk_start_wrong": ("floor_div((int64_t)seq_lens[r] - query_len, compress_ratio);",
                               "floor_div((int64_t)seq_lens[r] - query_len + 1, compress_ratio);"),
    "topk_smallest": ("if (x->value > y->value) return -1;\n    if (x->value < y->value) return 1;",
                      "if (x->value < y->value) return -1;\n    if (x->value > y->value) return 1;"),
    "prep_gain_without_one": ("float gain = (float)element(weight, d, weight_format) + 1.0f;",
                              "float gain = (float)element(weight, d, weight_format);"),
    "prep_eps_dropped": ("(float)sum_sq / (float)PREP_DIM + eps;", "(float)sum_sq / (float)PREP_DIM;"),
    "prep_sum_not_averaged": ("(float)sum_sq / (float)PREP_DIM + eps;", "(float)sum_sq + eps;"),
    "prep_rotation_sign": ("o[j] = in_type(in_type(lo * c, rot_format) - in_type(hi * s, rot_format)",
                           "o[j] = in_type(in_type(lo * c, rot_format) + in_type(hi * s, rot_format)"),
    "prep_partner_wrong": ("float lo = y[j], hi = y[j + PREP_PAIRS];",
                           "float lo = y[j], hi = y[j + 2 * PREP_PAIRS];"),
    "prep_cos_sin_swapped": ("c = (float)element(cos_sin, p * 2 * PREP_PAIRS + j, rot_format);",
                             "c = (float)element(cos_sin, p * 2 * PREP_PAIRS + PREP_PAIRS + j, rot_format);"),
    "prep_table_row_stride": ("s = (float)element(cos_sin, p * 2 * PREP_PAIRS + PREP_PAIRS + j, rot_format);",
                              "s = (float)element(cos_sin, p * PREP_PAIRS + PREP_PAIRS + j, rot_format);"),
    "prep_mrope_height_residue": ("if (j % 3 == 1 && j < 3 * section[1]) return 1;",
                                  "if (j % 3 == 0 && j < 3 * section[1]) return 1;"),
    "prep_mrope_sections_swapped": ("if (j % 3 == 2 && j < 3 * section[2]) return 2;",
                                    "if (j % 3 == 2 && j < 3 * section[1]) return 2;"),
    "prep_no_per_op_rounding": ("o[j] = in_type(in_type(lo * c, rot_format) - in_type(hi * s, rot_format), rot_format);",
                                "o[j] = in_type(lo * c - hi * s, rot_format);"),
    "prep_y_not_rounded": ("y[d] = in_type((x[d] * rrms) * gain, rot_format);", "y[d] = (x[d] * rrms) * gain;"),
    "prep_passthrough_from_rotated": ("for (int d = 2 * PREP_PAIRS; d < PREP_DIM; ++d) o[d] = y[d];",
                                      "for (int d = 2 * PREP_PAIRS; d < PREP_DIM; ++d) o[d] = y[d - 64];"),
    "prep_fp8_scale_multiplies": ("float_to_e4m3_bits((float)bf16_bits_to_double(v) / out_scale)",
                                  "float_to_e4m3_bits((float)bf16_bits_to_double(v) * out_scale)"),
    "prep_fp8_skips_bf16": ("float_to_e4m3_bits((float)bf16_bits_to_double(v) / out_scale)",
                            "float_to_e4m3_bits(o[d] / out_scale)"),
    "prep_head_stride_wrong": ("(int64_t)h * PREP_DIM;\n", "(int64_t)h * 64;\n"),
    "prep_position_axis_ignored": ("int64_t p = pos[mrope_section ? mrope_axis(j, mrope_section) : 0];",
                                   "int64_t p = pos[0];"),
    "prep_range_unchecked_high": ("if (p >= 0 && p < cos_sin_rows) {", "if (p >= 0 && p <= cos_sin_rows) {"),
    "bf16_ties_away": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;",
                       "if (dropped >= 0x8000u) kept += 1u;"),
    "e4m3_ties_odd": ("if (err < best_err || (err == best_err && (code & 1) == 0)) {",
                      "if (err < best_err || (err == best_err && (code & 1) == 1)) {"),
    "e4m3_no_saturation": ("if (a > 448.0) a = 448.0;", "if (a > 448.0) return 0x7F;"),
}


RUNNER = """
import sys
sys.path.insert(0, {root!r})
from oracle import oracle as O
O._lib = O.load({lib!r})
from tests import oracle_pins as P
# One failing pin is enough; the slowest pins (library comparisons, brute
# force) run last.
slow = ("pin_bf16_rounding_matches_library", "pin_fp16_decoding_all_codes", "pin_bruteforce_numpy_decode")
failed = []
for pin in sorted(P.ALL_PINS, key=lambda f: f.__name__ in slow):
    try:
        pin()
    except AssertionError:
        failed.append(pin.__name__)
        break
print("FAILED_PINS", ",".join(failed))
"""


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="qsa_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    """Each mutant runs in its own process: a mutant that reads out of bounds
    may die on a signal, which also counts as caught; any other error fails
    the test."""
    old, new = MUTANTS[name]
    src = open(O.SRC).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib_path = O.build(path, os.path.join(workdir, f"lib_{name}.so"))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = RUNNER.format(root=root, lib=lib_path)
    env = dict(os.environ, QSA_ORACLE_THREADS="1")
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=300, env=env)
    if proc.returncode < 0:
        return  # killed by a signal (an out-of-bounds read): caught
    assert proc.returncode == 0, proc.stderr[-2000:]
    line = [x for x in proc.stdout.splitlines() if x.startswith("FAILED_PINS")][-1]
    failed = [x for x in line.split(" ", 1)[1].split(",") if x]
    assert failed, f"no pin caught mutant {name}"
