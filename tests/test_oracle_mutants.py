"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

Every mutant is compiled from a textual edit of the oracle source into a
temporary directory; the edits keep all memory accesses inside the buffers.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "wgrad_ref.c")

# name -> (function whose body the edit applies to, text, replacement)
WG = "oracle_wgrad2_accumulate"
MUTANTS = {
    "pad_sign_h": (WG, "ho * stride_h + r * dil_h - pad_h", "ho * stride_h + r * dil_h + pad_h"),
    "r_for_s_in_w": (WG, "wo * stride_w + s * dil_w - pad_w", "wo * stride_w + r * dil_w - pad_w"),
    "no_stride_w": (WG, "wo * stride_w + s * dil_w - pad_w", "wo + s * dil_w - pad_w"),
    "no_dilation_w": (WG, "wo * stride_w + s * dil_w - pad_w", "wo * stride_w + s - pad_w"),
    "row_pad_on_columns": (WG, "wo * stride_w + s * dil_w - pad_w", "wo * stride_w + s * dil_w - pad_h"),
    "row_stride_on_columns": (WG, "wo * stride_w + s * dil_w - pad_w", "wo * stride_h + s * dil_w - pad_w"),
    "row_dilation_on_columns": (WG, "wo * stride_w + s * dil_w - pad_w", "wo * stride_w + s * dil_h - pad_w"),
    "column_pad_on_rows": (WG, "ho * stride_h + r * dil_h - pad_h", "ho * stride_h + r * dil_h - pad_w"),
    "wo_from_row_geometry": (WG, "oracle_out_size(W, S, pad_w, stride_w, dil_w)",
                             "oracle_out_size(W, S, pad_h, stride_h, dil_h)"),
    "dropped_group_offset": (WG, "* C + grp * Cg;", "* C;"),
    "transposed_taps": (WG, "((k * R + r) * S + s) * Cg;\n              double* a",
                        "((k * S + s) * R + r) * Cg;\n              double* a"),
    "abs_of_product_dropped": (WG, "a[c] += fabs(g) * fabs(v);", "a[c] += g * v;"),
    "last_row_dropped": (WG, "if (h < 0 || h >= H) continue", "if (h < 0 || h >= H - 1) continue"),
    "out_size_off_by_one": ("oracle_out_size", "return span / stride + 1;", "return span / stride;"),
    "single_thread_copy_only": (WG, "for (int t = 0; t < nthreads; ++t) {", "for (int t = 0; t < 1; ++t) {"),
    "bgrad_last_pixel_dropped": ("oracle_bgrad_accumulate", "for (int64_t l = 0; l < pixels; ++l) {",
                                 "for (int64_t l = 0; l < pixels - 1; ++l) {"),
    "bgrad_abs_summed": ("oracle_bgrad_accumulate", "db[k] += (double)g[k];", "db[k] += fabs((double)g[k]);"),
    "bgrad_signed_denominator": ("oracle_bgrad_accumulate", "absacc[k] += fabs((double)g[k]);",
                                 "absacc[k] += (double)g[k];"),
    "bgrad_channel_stride": ("oracle_bgrad_accumulate", "const float* g = dy + l * K;",
                             "const float* g = dy + (l / K) * K;"),
    # forward
    "fwd_pad_sign": ("oracle_fwd", "ho * stride_h + r * dil_h - pad_h", "ho * stride_h + r * dil_h + pad_h"),
    "fwd_row_pad_on_columns": ("oracle_fwd", "wo * stride_w + s * dil_w - pad_w", "wo * stride_w + s * dil_w - pad_h"),
    "fwd_no_column_stride": ("oracle_fwd", "wo * stride_w + s * dil_w - pad_w", "wo + s * dil_w - pad_w"),
    "fwd_filter_taps_transposed": ("oracle_fwd", "((k * R + r) * S + s) * Cg", "((k * S + s) * R + r) * Cg"),
    "fwd_group_offset_dropped": ("oracle_fwd", "* C + grp * Cg;", "* C;"),
    "fwd_last_channel_dropped": ("oracle_fwd", "for (int64_t c = 0; c < Cg; ++c) {",
                                 "for (int64_t c = 0; c < Cg - 1; ++c) {"),
    "fwd_abs_dropped": ("oracle_fwd", "aacc += fabs((double)xp[c]) * fabs((double)wp[c]);",
                        "aacc += (double)xp[c] * (double)wp[c];"),
    # data gradient
    "dgrad_pad_sign": ("oracle_dgrad", "ho * stride_h + r * dil_h - pad_h", "ho * stride_h + r * dil_h + pad_h"),
    "dgrad_no_row_dilation": ("oracle_dgrad", "ho * stride_h + r * dil_h - pad_h", "ho * stride_h + r - pad_h"),
    "dgrad_column_stride_on_rows": ("oracle_dgrad", "ho * stride_h + r * dil_h - pad_h",
                                    "ho * stride_w + r * dil_h - pad_h"),
    "dgrad_filter_not_flipped_wrt_taps": ("oracle_dgrad", "((k * R + r) * S + s) * Cg",
                                          "((k * R + (R - 1 - r)) * S + s) * Cg"),
    "dgrad_group_offset_dropped": ("oracle_dgrad", "* C + grp * Cg;\n              double* a",
                                   "* C;\n              double* a"),
    "dgrad_last_row_dropped": ("oracle_dgrad", "if (hi < 0 || hi >= H) continue", "if (hi < 0 || hi >= H - 1) continue"),
}


def _function_span(src, func):
    """[start, end) of the definition of func (from its signature to its closing brace)."""
    start = src.index("\n" + ("int64_t " if func == "oracle_out_size" else "int ") + func + "(")
    end = src.index("\n}\n", start) + 3
    return start, end


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    func, old, new = MUTANTS[name]
    src = open(SRC).read()
    a, b = _function_span(src, func)
    body = src[a:b]
    assert body.count(old) == 1, name
    mutated = tmp_path / ("wgrad_%s.c" % name)
    mutated.write_text(src[:a] + body.replace(old, new) + src[b:])
    lib_path = str(tmp_path / ("lib_%s.so" % name))
    oracle.build(force=True, src=str(mutated), out=lib_path, strict=False)
    lib = oracle.load(lib_path)
    # The pins of the mutated function's own direction first (they catch it soonest).
    key = {"oracle_fwd": ("fwd", "adjoint"), "oracle_dgrad": ("dgrad", "adjoint")}.get(func, ())
    pins = sorted(P.ALL_PINS, key=lambda f: not any(k in f.__name__ for k in key))
    for pin in pins:
        try:
            pin(lib)
        except (AssertionError, ValueError, RuntimeError):
            return  # caught
    pytest.fail("mutant %s passed every pin" % name)


def test_unmutated_source_builds_and_passes(tmp_path):
    lib_path = str(tmp_path / "lib_clean.so")
    oracle.build(force=True, src=SRC, out=lib_path)
    lib = oracle.load(lib_path)
    for pin in P.ALL_PINS:
        pin(lib)
