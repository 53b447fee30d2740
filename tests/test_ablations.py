"""Numerical ablations of the combine format, measured with the oracle on the CPU.

The AREX article's section "计算提速后,NVLink 通信成了新瓶颈" reports that the combine was first
sent in MXFP8, which represented outliers badly, and then as a 32-point randomized Hadamard
transform followed by block-scaled S2F6, which spreads the outliers before quantizing. These
tests measure the three encodings on the same rows:
  MXFP8      E4M3 codes + one E8M0 per 32 (round to nearest even);
  S2F6       int8 codes c/64 + one E8M0 per 32, no transform;
  RHT+S2F6   the same after the transform (inverted exactly on decode).
Data (bf16 rows, 256 x 1024, seeded): N(0,1); N(0,1) with 8 rows x 50 (outlier rows, as in the
transpose figure); N(0,1) with one value per 32-chunk x 30 (an outlier in every chunk);
Student-t(3). Errors are relative Frobenius errors over all values, and over the values other
than the planted outliers.
"""
import numpy as np
import torch

import oracle as O

R, C, MASK = 256, 1024, 0x5A5A0F0F


def _rows(kind, rng):
    y = rng.standard_normal((R, C))
    planted = np.zeros((R, C), bool)
    if kind == "outlier_rows":
        rows = rng.choice(R, 8, replace=False)
        y[rows] *= 50
        planted[rows] = True
    elif kind == "chunk_outliers":
        idx = rng.integers(0, 32, (R, C // 32))
        v = y.reshape(R, C // 32, 32)
        p = planted.reshape(R, C // 32, 32)
        v[np.arange(R)[:, None], np.arange(C // 32)[None, :], idx] *= 30
        p[np.arange(R)[:, None], np.arange(C // 32)[None, :], idx] = True
    elif kind == "student_t3":
        y = rng.standard_t(3, (R, C))
    return torch.tensor(y, dtype=torch.float32).to(torch.bfloat16), planted


def errors(kind, seed=3):
    x, planted = _rows(kind, np.random.default_rng(seed))
    y = x.float().numpy().astype(np.float64)
    q, e = O.mxfp8_quantize_rows(x)
    mx = O.mxfp8_dequantize(q, e)
    c, e2 = O.s2f6_quantize(y.astype(np.float32))
    s2 = O.s2f6_dequantize(c, e2)
    c, e3 = O.rht32_s2f6_quantize(y.astype(np.float32), MASK)
    rh = O.rht32_s2f6_decode(c, e3, MASK)
    rest = ~planted

    def rel(a, m=None):
        if m is None:
            return np.linalg.norm(a - y) / np.linalg.norm(y)
        return np.linalg.norm((a - y)[m]) / np.linalg.norm(y[m])
    return {name: (rel(a), rel(a, rest)) for name, a in (("mxfp8", mx), ("s2f6", s2), ("rht_s2f6", rh))}


def test_rht_s2f6_beats_mxfp8_on_every_recipe():
    """Over all values RHT+S2F6 has well under half MXFP8's error on every recipe (MXFP8 keeps
    3 mantissa bits, about 2.65% here, and large values dominate the error). On the ordinary
    values it is also better, by 3x and more, except when every chunk carries an outlier: the
    transform then spreads the outlier over the chunk and the others keep about MXFP8's error."""
    for kind in ("gaussian", "outlier_rows", "chunk_outliers", "student_t3"):
        r = errors(kind)
        assert r["rht_s2f6"][0] < 0.4 * r["mxfp8"][0], (kind, r)
        assert r["rht_s2f6"][1] < r["mxfp8"][1], (kind, r)
        if kind != "chunk_outliers":
            assert r["rht_s2f6"][1] < 0.35 * r["mxfp8"][1], (kind, r)


def test_the_transform_is_what_protects_s2f6_from_outliers():
    """With an outlier in every chunk, plain S2F6 spends its uniform grid on the outlier and the
    other 31 values lose most of their bits; after the transform they keep them."""
    r = errors("chunk_outliers")
    assert r["s2f6"][1] > 3 * r["rht_s2f6"][1], r
    assert r["s2f6"][0] > 3 * r["rht_s2f6"][0], r
    # without outliers the transform changes little
    g = errors("gaussian")
    assert 0.5 < g["s2f6"][0] / g["rht_s2f6"][0] < 2.0, g


if __name__ == "__main__":      # prints the table of errors (run from the repository root)
    for kind in ("gaussian", "outlier_rows", "chunk_outliers", "student_t3"):
        r = errors(kind)
        print(kind, {k: (round(a, 5), round(b, 5)) for k, (a, b) in r.items()})


# ------------------------------------------------------------------------------------------
# The transpose problem ([AREX] "转置打散分组,随机舍入保住期望值"): zeros after the transpose under
# outlier rows, for 1D blocks re-quantized by rounding to nearest, 16 x 16 blocks, and the
# pages' method (dequantize, transpose, stochastic rounding to MXFP8). Workload: X [256 x 512]
# N(0,1) with two rows x 50 (the single-expert inputs).
# ------------------------------------------------------------------------------------------

def _fp4_vals(codes):
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    c = np.zeros((codes.shape[0], codes.shape[1] * 2), np.int64)
    c[:, 0::2], c[:, 1::2] = codes & 15, codes >> 4
    return np.where(c & 8, -1.0, 1.0) * grid[c & 7]


def _nvfp4_values(q):
    """fp64 values of an NVFP4 matrix (codes x E4M3 scale x outer)."""
    s = torch.from_numpy(q["scales"]).view(torch.float8_e4m3fn).double().numpy()
    outer = np.repeat(q["outer"], q["rows_per_outer"])
    return _fp4_vals(q["codes"]) * np.repeat(s, 16, axis=1) * outer[:, None]


def transpose_zero_fractions():
    from precision_moe_numerics_amd import inputs as I
    d = I.single_expert("cpu")
    x, rows = d["x"], d["outlier_rows"]
    R, C = x.shape
    fwd = O.nvfp4_quantize(x, 1, True)                         # forward: 1D, per token, 4/6
    v = _nvfp4_values(fwd)                                      # the saved forward values
    live = (v != 0)
    # blocks that hold an outlier-row value after the transpose: every 16-block of columns that
    # spans one of the outlier rows, i.e. rows (16 * (r // 16)) .. + 15 of each column
    band = np.zeros((R, C), bool)
    for r in rows:
        band[16 * (r // 16):16 * (r // 16) + 16] = True
    ordinary = band & live & ~np.isin(np.arange(R), rows)[:, None]
    res = {}
    # (1) 1D blocks, re-quantized by RTN along the transposed direction (weight mode: no 4/6)
    vt = torch.tensor(v.T, dtype=torch.float32).to(torch.bfloat16)
    naive = _nvfp4_values(O.nvfp4_quantize(vt, rows_per_outer=C, four_six=False)).T
    res["1d_rtn_transposed"] = float((naive[ordinary] == 0).mean())
    # (2) 16 x 16 blocks: the forward itself already shares the outlier's scale over the tile
    q2 = O.nvfp4_quantize_2d(x, R)
    v2 = _nvfp4_values(q2)
    res["2d_16x16"] = float((v2[ordinary] == 0).mean())
    # (3) the method: dequantize -> transpose -> SR to MXFP8 (and, for reference, to the E2M1 grid)
    q = dict(codes=fwd["codes"], scales=fwd["scales"], outer=fwd["outer"], rows_per_outer=1)
    t8, e8 = O.requant_transpose_sr(q, seed=7, stream=1)
    m8 = O.mxfp8_dequantize(t8, e8)[:, :R].T
    res["sr_mxfp8"] = float((m8[ordinary] == 0).mean())
    t4, e4 = O.requant_transpose_sr(q, target=O.TARGET_E2M1, seed=7, stream=1)
    m4 = (np.where(t4 & 8, -1.0, 1.0) * np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])[t4 & 7]
          * np.repeat(2.0 ** (e4.astype(np.float64) - 127), 32, axis=1))[:, :R].T
    res["sr_e2m1"] = float((m4[ordinary] == 0).mean())
    res["ordinary_values"] = int(ordinary.sum())
    res["forward_zero_fraction"] = float((v[band & ~np.isin(np.arange(R), rows)[:, None]] == 0).mean())
    return res


def test_transpose_zero_fractions_under_outlier_rows():
    """1D blocks re-quantized after the transpose and 16 x 16 blocks both lose most ordinary values
    of the blocks an outlier row crosses; the method (SR to MXFP8 after dequantizing) keeps them."""
    r = transpose_zero_fractions()
    assert r["1d_rtn_transposed"] > 0.5, r
    assert r["2d_16x16"] > 0.5, r
    assert r["sr_mxfp8"] < 0.01, r
    assert r["forward_zero_fraction"] < 0.2, r
