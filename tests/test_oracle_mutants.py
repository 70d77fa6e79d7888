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

MUTANTS = {
    "pad_sign_h": ("ho * stride_h + r * dil_h - pad_h", "ho * stride_h + r * dil_h + pad_h"),
    "r_for_s_in_w": ("wo * stride_w + s * dil_w - pad_w", "wo * stride_w + r * dil_w - pad_w"),
    "no_stride_w": ("wo * stride_w + s * dil_w - pad_w", "wo + s * dil_w - pad_w"),
    "no_dilation_w": ("wo * stride_w + s * dil_w - pad_w", "wo * stride_w + s - pad_w"),
    "row_pad_on_columns": ("wo * stride_w + s * dil_w - pad_w", "wo * stride_w + s * dil_w - pad_h"),
    "row_stride_on_columns": ("wo * stride_w + s * dil_w - pad_w", "wo * stride_h + s * dil_w - pad_w"),
    "row_dilation_on_columns": ("wo * stride_w + s * dil_w - pad_w", "wo * stride_w + s * dil_h - pad_w"),
    "column_pad_on_rows": ("ho * stride_h + r * dil_h - pad_h", "ho * stride_h + r * dil_h - pad_w"),
    "wo_from_row_geometry": ("oracle_out_size(W, S, pad_w, stride_w, dil_w)",
                             "oracle_out_size(W, S, pad_h, stride_h, dil_h)"),
    "dropped_group_offset": ("* C + grp * Cg;", "* C;"),
    "transposed_taps": ("((k * R + r) * S + s) * Cg;\n              double* a",
                        "((k * S + s) * R + r) * Cg;\n              double* a"),
    "abs_of_product_dropped": ("a[c] += fabs(g) * fabs(v);", "a[c] += g * v;"),
    "last_row_dropped": ("if (h < 0 || h >= H) continue", "if (h < 0 || h >= H - 1) continue"),
    "out_size_off_by_one": ("return span / stride + 1;", "return span / stride;"),
    "single_thread_copy_only": ("for (int t = 0; t < nthreads; ++t) {", "for (int t = 0; t < 1; ++t) {"),
    "bgrad_last_pixel_dropped": ("for (int64_t l = 0; l < pixels; ++l) {",
                                 "for (int64_t l = 0; l < pixels - 1; ++l) {"),
    "bgrad_abs_summed": ("db[k] += (double)g[k];", "db[k] += fabs((double)g[k]);"),
    "bgrad_signed_denominator": ("absacc[k] += fabs((double)g[k]);", "absacc[k] += (double)g[k];"),
    "bgrad_channel_stride": ("const float* g = dy + l * K;", "const float* g = dy + (l / K) * K;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / ("wgrad_%s.c" % name)
    mutated.write_text(src.replace(old, new))
    lib_path = str(tmp_path / ("lib_%s.so" % name))
    oracle.build(force=True, src=str(mutated), out=lib_path, strict=False)
    lib = oracle.load(lib_path)
    for pin in P.ALL_PINS:
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
