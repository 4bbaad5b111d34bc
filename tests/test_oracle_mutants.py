"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of oracle/oracle.c with one textual change (a dropped
term, a wrong sign, a wrong tie rule, a transposed index, ...), compiled with
gcc into a temporary library on the CPU.  The pins of tests/pins.py are run
against it; a mutant that passes every pin would show a hole in the pins.
"""
import os
import subprocess

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text to replace, replacement) -- each replacement keeps memory accesses in bounds.
MUTANTS = [
    ("drop_first_row_of_sum", "for (int64_t r = lo; r < hi; ++r) {\n                        const double x",
     "for (int64_t r = lo + 1; r < hi; ++r) {\n                        const double x"),
    ("drop_first_row_of_int_sum", "for (int64_t r = lo; r < hi; ++r)\n                        sum += load_bits",
     "for (int64_t r = lo + 1; r < hi; ++r)\n                        sum += load_bits"),
    ("float_sum_wrong_sign", "sum += x;", "sum -= x;"),
    ("magnitude_not_absolute", "mag += x < 0 ? -x : x;", "mag += x;"),
    ("mean_wrong_length", "sum / (double)(hi - lo)", "sum / (double)(hi - lo + 1)"),
    ("ties_to_higher_row_min", "(k < best_key)", "(k <= best_key)"),
    ("ties_to_higher_row_max", "(k > best_key)", "(k >= best_key)"),
    ("min_max_swapped", "(op == ORC_MIN) ? (k < best_key) : (k > best_key)",
     "(op == ORC_MIN) ? (k > best_key) : (k < best_key)"),
    ("float_key_negatives_unflipped", "        return ~bits;", "        return bits;"),
    ("int_key_unsigned", "return bits ^ 0x80000000u;\n    if (bits", "return bits;\n    if (bits"),
    ("empty_value_nonzero", "store_bits(out, o, 0u);", "store_bits(out, o, 1u);"),
    ("empty_arg_not_minus_one", "arg_out[o] = -1;", "arg_out[o] = lo;"),
    ("output_transposed", "const int64_t o = s * feat + f;", "const int64_t o = f * num_segments + s;"),
    ("feature_stride_dropped", "load_bits(values, r * feat + f));\n                        sum",
     "load_bits(values, r + f));\n                        sum"),
    ("arg_relative_to_segment", "arg_out[o] = best_row;", "arg_out[o] = best_row - lo;"),
    ("rle_only_increasing_boundaries", "keys[i] != keys[i - 1]", "keys[i] > keys[i - 1]"),
    ("rle_last_offset_short", "offsets[c] = n;\n    for (int64_t r", "offsets[c] = n - (n > 0);\n    for (int64_t r"),
    ("scatter_drops_output_zero", "if (s < 0 || s >= dim_size)\n            continue;\n        count",
     "if (s < 1 || s >= dim_size)\n            continue;\n        count"),
    ("scatter_drops_first_row", "for (int64_t r = 0; r < rows; ++r) {\n        const int64_t s = index[r];\n        if (s < 0",
     "for (int64_t r = 1; r < rows; ++r) {\n        const int64_t s = index[r];\n        if (s < 0"),
    ("index_offsets_drop_first_row", "for (int64_t r = 0; r < rows; ++r) {\n        const int64_t s = index[r];\n        if (s >= 0",
     "for (int64_t r = 1; r < rows; ++r) {\n        const int64_t s = index[r];\n        if (s >= 0"),
    ("scatter_int_sum_overwrites", "isum[cell] += b;", "isum[cell] = b;"),
    ("scatter_float_sum_wrong_sign", "sum[cell] += x;", "sum[cell] -= x;"),
    ("scatter_mean_wrong_count", "sum[cell] / (double)count[s]", "sum[cell] / (double)(count[s] + 1)"),
    ("scatter_ties_to_later_row", "(k < best_key[cell]) : (k > best_key[cell])",
     "(k <= best_key[cell]) : (k >= best_key[cell])"),
    ("scatter_min_max_swapped", "(k < best_key[cell]) : (k > best_key[cell])",
     "(k > best_key[cell]) : (k < best_key[cell])"),
    ("scatter_feature_stride_dropped", "const uint32_t b = load_bits(values, r * feat + f);",
     "const uint32_t b = load_bits(values, r + f * (r + 1 < rows));"),
    ("index_offsets_shifted", "offsets[s + 1] += 1;", "offsets[s] += 1;"),
    ("index_offsets_not_cumulative", "offsets[s + 1] += offsets[s];", "offsets[s + 1] = offsets[s + 1];"),
    ("unique_only_increasing", "keys[i] != values[c - 1]", "keys[i] > values[c - 1]"),
    ("unique_compares_first_kept", "keys[i] != values[c - 1]", "keys[i] != values[0]"),
    ("flags_low_bit_only", "if (flags[i] != 0)", "if ((flags[i] & 1u) != 0)"),
    ("flags_offset_shifted", "offsets[c++] = i;", "offsets[c++] = i + (i + 1 < n);"),
    ("flags_last_offset_short", "offsets[c] = n;\n    *count = c;", "offsets[c] = n - (n > 0);\n    *count = c;"),
    ("scan_exclusive_block_inverted", "if (exclusive) {\n                    /* the prefix", "if (!exclusive) {\n                    /* the prefix"),
    ("scan_float_sum_wrong_sign", "run += x;", "run -= x;"),
    ("scan_magnitude_not_absolute", "run_abs += x < 0 ? -x : x;", "run_abs += x;"),
    ("scan_min_max_swapped", "((op == ORC_MAX) ? (k > top_key) : (k < top_key))",
     "((op == ORC_MAX) ? (k < top_key) : (k > top_key))"),
    ("scan_exclusive_start_not_zero", "seen ? top_bits : 0u", "seen ? top_bits : b"),
    ("scan_feature_stride_dropped", "const int64_t o = r * feat + f;\n                const uint32_t b",
     "const int64_t o = r + f;\n                const uint32_t b"),
    ("scan_int_sum_overwrites", "run_int += b;", "run_int = b;"),
    ("lb_upper_bound", "(bits_to_float(vb) < bits_to_float(qb)) : (vb < qb)",
     "(bits_to_float(vb) <= bits_to_float(qb)) : (vb <= qb)"),
    ("lb_signed_compare", ": (vb < qb);", ": ((int32_t)vb < (int32_t)qb);"),
    ("lb_relative_position", "out[qo + k] = p;", "out[qo + k] = p - vo;"),
    ("lb_order_ignored", "const int64_t row = order ? (int64_t)order[p] : p;", "const int64_t row = p;"),
    ("lb_stride_ignored", "load_bits(values, row * stride);", "load_bits(values, row);"),
    ("lb_decrease_across_tiles", "if (k % T != 0) {", "if (k != 0) {"),
    ("lb_no_tile_stop", "k = (k / T + 1) * T - 1; /* the rest of this tile is skipped */", "/* no stop */"),
    ("lb_capacity_ignored", " || qc > max_qc;", ";"),
    ("rle_length_off_by_one", "(uint32_t)(offsets[r + 1] - offsets[r])", "(uint32_t)(offsets[r + 1] - offsets[r] - 1)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: anchor text not found exactly once"
    mutant_src = tmp_path / "oracle_mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "liboracle_mutant.so")
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", str(mutant_src), "-o", lib_path], check=True)
    lib = oracle.load(lib_path)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake '{name}' passed every pin"
