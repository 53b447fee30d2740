"""Helpers of the full-size sampled parity tests: sampled slots of ragged groups, and the oracle's
quantization of selected rows placed in full-size arrays (the requantization keys its random bits
by the element's index in the whole source matrix, so windows must come from full-size arrays)."""
import numpy as np

import oracle as O


def oracle_quant_rows(x_rows, total_rows, first_row, rows_per_outer, four_six):
    """The oracle's NVFP4 quantization of rows [first_row, first_row + n) of a [total_rows x C]
    matrix, placed in full-size arrays whose other rows stay zero (and are never read)."""
    q = O.nvfp4_quantize(x_rows, rows_per_outer, four_six)
    n, half = q["codes"].shape
    assert first_row % rows_per_outer == 0 and n % rows_per_outer == 0
    codes = np.zeros((total_rows, half), np.uint8)
    scales = np.zeros((total_rows, half // 8), np.uint8)
    outer = np.ones(total_rows // rows_per_outer, np.float32)
    codes[first_row:first_row + n] = q["codes"]
    scales[first_row:first_row + n] = q["scales"]
    outer[first_row // rows_per_outer:(first_row + n) // rows_per_outer] = q["outer"]
    return dict(codes=codes, scales=scales, outer=outer, rows_per_outer=rows_per_outer)


def sample_slots(offsets, groups, per_group, rng):
    s = []
    for g in groups:
        a, b = int(offsets[g]), int(offsets[g + 1])
        s += [a, b - 1] + list(rng.integers(a, b, per_group - 2))
    return np.array(s, np.int64)
