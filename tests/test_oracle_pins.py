"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Sources of truth used here: values the pages print (tests/golden/pages_facts.json), the
published Philox4x32-10 known-answer vectors (tests/golden/philox_kat.json), library routines
(torch's float8_e4m3fn cast, numpy matmul, numpy's stable argsort), closed forms, invariants
and brute force on tiny inputs. Each test is chosen so that a plausible mistake in the oracle
(a dropped term, a wrong sign, a transposed operand, a wrong tie rule) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FACTS = json.load(open(os.path.join(GOLD, "pages_facts.json")))


def bf16(a):
    return torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16)


# ------------------------------------------------------------------------------------------
# codecs
# ------------------------------------------------------------------------------------------

def test_fp4_grid_is_the_pages_grid():
    mags = FACTS["fp4_grid"]["magnitudes"]
    assert [O.fp4_value(c) for c in range(8)] == mags
    assert [O.fp4_value(8 + c) for c in range(8)] == [-m for m in mags]
    # nothing above 6 is representable: everything larger saturates to code 7
    assert O.fp4_encode(6.5) == 7 and O.fp4_encode(1e30) == 7 and O.fp4_encode(-7.0) == 15


def test_rtn_example_3_2_to_3():
    f = FACTS["rtn_example"]
    # on a grid where only 3 and 4 exist around 3.2 (the FP4 grid), RTN gives 3, error -0.2
    c = O.fp4_encode(f["value"])
    assert O.fp4_value(c) == f["rounded"]
    assert math.isclose(O.fp4_value(c) - f["value"], f["error"], abs_tol=1e-6)


def _fp4_bruteforce(y):
    """Nearest of the pages' 16 FP4 values, ties to the even magnitude index, saturating."""
    mags = np.array(FACTS["fp4_grid"]["magnitudes"])
    a = np.abs(y.astype(np.float64))[:, None]
    d = np.abs(a - mags[None, :])
    best = np.argmin(d, axis=1)
    # ties: argmin takes the lower index; replace by the even one when two are equally near
    nxt = np.minimum(best + 1, 7)
    tie = (d[np.arange(len(y)), nxt] == d[np.arange(len(y)), best]) & (nxt != best)
    best = np.where(tie & (best % 2 == 1), nxt, best)
    return (best | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


def test_fp4_encode_matches_bruteforce():
    rng = np.random.default_rng(1)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    around = np.concatenate([np.nextafter(mids, 0), mids, np.nextafter(mids, 10)])
    y = np.concatenate([rng.uniform(-8, 8, 200000).astype(np.float32), around, -around,
                        np.array([0.0, -0.0, 6.0, -6.0, 1e-30, -1e-30], np.float32)])
    got = O.fp4_encode_array(y)
    assert np.array_equal(got, _fp4_bruteforce(y))


def test_e4m3_encode_matches_torch_cast():
    """RNE E4M3 against torch's float8_e4m3fn cast (a library routine) for |x| < 464."""
    allbf = np.arange(65536, dtype=np.uint32) << 16
    rng = np.random.default_rng(2)
    rnd = rng.integers(0, 2**32, 3_000_000, dtype=np.uint64).astype(np.uint32)
    grid = np.array([O.e4m3_value(c) for c in range(127)], np.float32)
    mids = ((grid[:-1].astype(np.float64) + grid[1:]) / 2).astype(np.float32)
    y = np.concatenate([allbf.view(np.float32), rnd.view(np.float32), mids, -mids,
                        np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    y = y[np.isfinite(y) & (np.abs(y) < 464)]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode_array(y)
    assert np.array_equal(got, ref)


def test_e4m3_saturates_above_torch_range():
    for v in (464.0, 480.0, 1e6, 3e38):
        assert O.e4m3_encode(v) == 0x7E and O.e4m3_encode(-v) == 0xFE
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0 ** -9


def test_e8m0_rule_bruteforce():
    rng = np.random.default_rng(3)
    vals = np.concatenate([np.ldexp(rng.uniform(0.5, 1.0, 2000), rng.integers(-140, 128, 2000)),
                           [448.0, 449.0, 6.0, 6.0000005, 127 / 64, 2.0, 1e-45]]).astype(np.float32)
    for M in (448.0, 6.0, 127 / 64):
        for a in vals:
            if not np.isfinite(a) or a == 0:
                continue
            e = O.e8m0_exponent(float(a), M)
            assert -127 <= e <= 127
            assert float(a) <= M * 2.0 ** e or e == 127
            if e > -127:
                assert float(a) > M * 2.0 ** (e - 1), (a, M, e)
    assert O.e8m0_exponent(0.0, 448.0) == -127


# ------------------------------------------------------------------------------------------
# stochastic rounding and the RNG
# ------------------------------------------------------------------------------------------

def test_philox_known_answers():
    kat = json.load(open(os.path.join(GOLD, "philox_kat.json")))["vectors"]
    for v in kat:
        out = O.philox4x32_10([int(x, 16) for x in v["ctr"]], [int(x, 16) for x in v["key"]])
        assert [f"{int(w):08x}" for w in out] == v["out"]


def test_rand16_slices_the_philox_output():
    seed, stream = 0x1234_5678_9ABC_DEF0, 7
    for blk in (0, 1, 5, 2**32 + 3):
        w = O.philox4x32_10([blk & 0xFFFFFFFF, blk >> 32, stream, 0], [seed & 0xFFFFFFFF, seed >> 32])
        for lane in range(8):
            word = int(w[lane >> 1])
            want = (word >> 16) if lane & 1 else (word & 0xFFFF)
            assert O.rand16(seed, stream, blk * 8 + lane) == want


def test_sr_worked_example_exact_probability():
    f = FACTS["sr_example"]
    y = f["value"] / f["new_scale"]
    assert y == f["scaled"]
    assert O.fp4_value(O.fp4_encode(y)) == f["rtn"]
    r = np.arange(65536, dtype=np.uint32)
    codes = O.fp4_encode_array(np.full(65536, y, np.float32), sr=True, r16=r)
    vals = np.array([O.fp4_value(c) for c in range(16)])[codes]
    assert set(np.unique(vals)) == {f["sr_low"], f["sr_high"]}
    assert np.sum(vals == f["sr_high"]) == int(f["p_high"] * 65536)
    assert np.sum(vals == f["sr_low"]) == int(f["p_low"] * 65536)
    assert vals.mean() * f["new_scale"] == f["expectation"]


def test_sr_e4m3_neighbours_and_expectation():
    rng = np.random.default_rng(4)
    y = np.ldexp(rng.uniform(1, 2, 300), rng.integers(-12, 8, 300)).astype(np.float32)
    grid = np.array([O.e4m3_value(c) for c in range(127)])
    r = np.arange(0, 65536, 16, dtype=np.uint32)
    for v in y:
        codes = O.e4m3_encode_array(np.full(r.size, v, np.float32), sr=True, r16=r)
        vals = grid[codes & 0x7F]
        lo = grid[grid <= v].max()
        hi = grid[grid >= v].min()
        assert set(np.unique(vals)) <= {lo, hi}
        if hi > lo:
            f = (float(v) - lo) / (hi - lo)
            assert abs(vals.mean() - float(v)) <= (hi - lo) * (1 / 4096 + 1e-12) + 1e-30, (v, f)


# ------------------------------------------------------------------------------------------
# NVFP4 quantization
# ------------------------------------------------------------------------------------------

def _block_with(values):
    x = np.zeros(16, np.float32)
    x[: len(values)] = values
    return x


def test_worked_example_block_max_and_5_4():
    bs, fw = FACTS["block_scale_example"], FACTS["forward_value_example"]
    x = _block_with([bs["block_max"], fw["value"], 1.0, -2.0, 0.3])
    q = O.nvfp4_quantize(bf16(x[None, :]), four_six=False, outer_in=[1.0])
    assert q["scales"][0, 0] == 0x51 and O.e4m3_value(0x51) == bs["scale"]
    nib = lambda i: (q["codes"][0, i // 2] >> (4 * (i & 1))) & 15
    assert O.fp4_value(nib(0)) == bs["code_value"]
    assert O.fp4_value(nib(1)) == fw["code_value"]
    deq = O.nvfp4_dequantize(q)
    assert deq[0, 1] == fw["dequant"]


def test_worked_example_with_computed_outer_scale():
    """With the outer scale computed from the data the codes are the same (effective scale ~9)."""
    bs, fw = FACTS["block_scale_example"], FACTS["forward_value_example"]
    x = _block_with([bs["block_max"], fw["value"]])
    q = O.nvfp4_quantize(bf16(x[None, :]), four_six=False)
    assert math.isclose(q["outer"][0], 54.0 / 2688.0, rel_tol=1e-7)
    assert O.e4m3_value(q["scales"][0, 0]) == 448.0
    deq = O.nvfp4_dequantize(q)
    assert math.isclose(deq[0, 0], -54.0, rel_tol=1e-6) and math.isclose(deq[0, 1], 4.5, rel_tol=1e-6)


def test_four_over_six_hand_case():
    # block [6, 4.5 x 15] with unit outer scale: candidate 6 keeps scale 1 and rounds every 4.5
    # to 4 (squared error 15 * 0.25 = 3.75); candidate 4 takes scale 1.5 and represents 6 = 4*1.5
    # and 4.5 = 3*1.5 exactly (error 0), so 4 is kept.
    x = np.array([6.0] + [4.5] * 15, np.float32)[None, :]
    q46 = O.nvfp4_quantize(bf16(x), four_six=True, outer_in=[1.0])
    q6 = O.nvfp4_quantize(bf16(x), four_six=False, outer_in=[1.0])
    assert O.e4m3_value(q6["scales"][0, 0]) == 1.0
    assert np.sum((O.nvfp4_dequantize(q6) - x) ** 2) == 3.75
    assert q46["chose4"][0, 0] == 1 and O.e4m3_value(q46["scales"][0, 0]) == 1.5
    assert np.array_equal(O.nvfp4_dequantize(q46), x)
    # a block already on the scale-6 grid keeps 6
    y = np.array([6, 4, 3, 2, 1.5, 1, 0.5, 0] * 2, np.float32)[None, :]
    qy = O.nvfp4_quantize(bf16(y), four_six=True, outer_in=[1.0])
    assert qy["chose4"][0, 0] == 0 and np.array_equal(O.nvfp4_dequantize(qy), y)


def test_four_over_six_exact_tie_keeps_six():
    """An exact tie between the two candidates keeps candidate 6 (the strict '<' of the rule).

    Row [2688, 0 x 15 | 6, 0 x 15] in activation mode: the row amax 2688 = 6 * 448 gives the
    outer scale exactly 1. In the second block candidate 6 takes scale 1 (E4M3 0x38) and stores 6
    as code 6; candidate 4 takes scale 1.5 (0x3C) and stores 6 as code 4 (4 * 1.5 = 6). Both
    reproduce the block with zero error, so only the tie rule decides: 0x38 under '<', 0x3C under
    '<='. The first block saturates both candidates to 448 (0x7E), an identical pair.
    """
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 16] = 2688.0, 6.0
    # the tie is real: both candidates' dequantized blocks equal the input, computed here from
    # the FP4 grid and the E4M3 values 1 and 1.5 alone
    grid = FACTS["fp4_grid"]["magnitudes"]
    assert 6.0 in grid and 4.0 in grid and grid[grid.index(6.0)] * 1.0 == 6.0 and 4.0 * 1.5 == 6.0
    for outer_in in (None, [1.0]):
        q = O.nvfp4_quantize(bf16(x), four_six=True, outer_in=outer_in)
        assert q["outer"][0] == 1.0
        assert list(q["scales"][0]) == [0x7E, 0x38]
        assert list(q["chose4"][0]) == [0, 0]
        assert q["codes"][0, 0] == 0x07 and q["codes"][0, 8] == 0x07      # code 6 = magnitude index 7
        assert np.array_equal(O.nvfp4_dequantize(q), x)


def _dequant_block_fp64(codes, scale_byte, s_o):
    """Independent decode: the pages' grid and the OCP E4M3 layout, written out here."""
    mags = FACTS["fp4_grid"]["magnitudes"]
    e, m = (scale_byte >> 3) & 15, scale_byte & 7
    sb = (m / 8 * 2 ** -6) if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return np.array([(-1 if c & 8 else 1) * mags[c & 7] for c in codes]) * sb * s_o


def test_nvfp4_properties_random():
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, size=(64, 256)) * 0.5).astype(np.float32)
    xb = bf16(x)
    xf = xb.float().numpy().astype(np.float64)
    for four_six in (False, True):
        q = O.nvfp4_quantize(xb, four_six=four_six)
        # outer scale: row amax / 2688, so the row's largest block has scale byte 448 (candidate 6)
        amax = np.abs(xf).max(axis=1)
        assert np.allclose(q["outer"], amax / 2688.0, rtol=1e-7)
        deq = O.nvfp4_dequantize(q)
        for r in range(0, 64, 7):
            for b in range(16):
                nib = [(q["codes"][r, (b * 16 + i) // 2] >> (4 * (i & 1))) & 15 for i in range(16)]
                ind = _dequant_block_fp64(nib, int(q["scales"][r, b]), float(q["outer"][r]))
                assert np.allclose(ind, deq[r, b * 16:(b + 1) * 16], rtol=1e-6, atol=0)
                # every element is within half an FP4 step (in units of the block scale) of x,
                # except where the block max saturates the grid
                d = abs(float(q["outer"][r]) * O.e4m3_value(int(q["scales"][r, b])))
                blk = xf[r, b * 16:(b + 1) * 16]
                err = np.abs(blk - ind)
                step = np.where(np.abs(blk) / d < 2, 0.5, np.where(np.abs(blk) / d < 4, 1.0, 2.0)) * d
                assert np.all(err <= step / 2 * (1 + 1e-5) + np.maximum(np.abs(blk) / d - 6, 0) * d)
        if four_six:
            # the kept candidate has the smaller squared error (recomputed independently in fp64)
            q6 = O.nvfp4_quantize(xb, four_six=False)
            d46 = O.nvfp4_dequantize(q)
            d6 = O.nvfp4_dequantize(q6)
            e46 = ((d46 - xf) ** 2).reshape(64, 16, 16).sum(-1)
            e6 = ((d6 - xf) ** 2).reshape(64, 16, 16).sum(-1)
            assert np.all(e46 <= e6 * (1 + 1e-5) + 1e-30)
            assert q["chose4"].mean() > 0.05


def test_weight_mode_one_outer_per_group():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((8, 64)) * 0.02).astype(np.float32)
    xb = bf16(x)
    q = O.nvfp4_quantize(xb, rows_per_outer=4, four_six=False)
    xf = xb.float().numpy()
    assert q["outer"].shape == (2,)
    assert np.isclose(q["outer"][0], np.abs(xf[:4]).max() / 2688, rtol=1e-7)
    assert np.isclose(q["outer"][1], np.abs(xf[4:]).max() / 2688, rtol=1e-7)
    assert q["chose4"].sum() == 0


def test_all_zero_and_tiny_blocks():
    x = np.zeros((2, 32), np.float32)
    x[1, 16:] = 1e-38
    q = O.nvfp4_quantize(bf16(x), four_six=True)
    assert q["outer"][0] == 1.0
    assert np.all(O.nvfp4_dequantize(q)[0] == 0)
    assert np.all(np.isfinite(O.nvfp4_dequantize(q)))


def test_bits_per_value():
    bits = FACTS["bits_per_value"]
    n = 4096
    q = O.nvfp4_quantize(bf16(np.ones((1, n))), four_six=False)
    nvfp4_bits = 8 * (q["codes"].nbytes + q["scales"].nbytes) / n
    assert nvfp4_bits == bits["nvfp4"]
    c, e = O.rht32_s2f6_quantize(np.ones((1, n), np.float32), 0)
    assert 8 * (c.nbytes + e.nbytes) / n == bits["s2f6_combine"]
    m, me = O.mxfp8_quantize_rows(bf16(np.ones((1, n))))
    assert 8 * (m.nbytes + me.nbytes) / n == bits["mxfp8"]


# ------------------------------------------------------------------------------------------
# requantization (dequant -> transpose -> SR)
# ------------------------------------------------------------------------------------------

def test_requant_sr_worked_example_through_the_transpose():
    """4.5 (code 0.5 in a scale-9 block) re-blocked with a block max of 9 gets E8M0 scale 2 on the
    E2M1 grid and becomes 2 or 3 times 2; the choice follows the element's random bits."""
    rows = 32
    x = np.zeros((rows, 16), np.float32)
    x[:, 0] = -54.0            # every row's block max -> effective scale 9 with s_o = 1
    x[:, 1] = 5.4              # stored as 0.5 * 9 = 4.5
    x[3, 1] = 9.0              # the new column block (column 1) has max 9 -> scale 2 on E2M1
    q = O.nvfp4_quantize(bf16(x), four_six=False, outer_in=np.ones(rows))
    for seed in range(6):
        out, oe = O.requant_transpose_sr(q, target=O.TARGET_E2M1, seed=seed, stream=3)
        assert oe[1, 0] == 127 + 1
        for s in range(rows):
            if s == 3:
                continue
            v = O.fp4_value(out[1, s]) * 2
            r16 = O.rand16(seed, 3, s * 16 + 1)
            assert v == (6.0 if r16 < 16384 else 4.0)


def test_requant_layout_groups_padding_and_gather():
    rng = np.random.default_rng(7)
    R, Cc = 50, 48
    x = rng.standard_normal((R, Cc)).astype(np.float32)
    q = O.nvfp4_quantize(bf16(x), four_six=True)
    gather = rng.integers(0, R, 70).astype(np.int32)
    offsets = np.array([0, 5, 5, 40, 70], np.int64)        # includes an empty group
    out, oe = O.requant_transpose_sr(q, gather=gather, offsets=offsets, seed=9, stream=1)
    P = [0, 32, 0, 64, 32]
    assert out.shape == (Cc, sum(P)) and oe.shape == (Cc, sum(P) // 32)
    deq = O.nvfp4_dequantize(q)
    e4 = np.array([O.e4m3_value(c) for c in range(256)])
    po = np.cumsum([0] + P[1:])
    for g in range(4):
        s0, s1 = offsets[g], offsets[g + 1]
        for c in range(Cc):
            for j in range(P[g + 1]):
                val = out[c, po[g] + j]
                if s0 + j >= s1:
                    assert val == 0
                    continue
                v = deq[gather[s0 + j], c]
                got = e4[val] * 2.0 ** (int(oe[c, (po[g] + j) // 32]) - 127)
                # SR lands on one of the two E4M3 neighbours of v at this block's scale
                sc = 2.0 ** (int(oe[c, (po[g] + j) // 32]) - 127)
                y = v / sc
                grid = np.concatenate([-e4[126::-1], e4[1:127]])
                lo, hi = grid[grid <= y].max(), grid[grid >= y].min()
                assert got / sc in (lo, hi)


def test_requant_unbiased():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    q = O.nvfp4_quantize(bf16(x), four_six=True)
    deq = O.nvfp4_dequantize(q).astype(np.float64)
    acc = np.zeros((32, 64))
    n = 200
    for seed in range(n):
        out, oe = O.requant_transpose_sr(q, seed=seed)
        acc += O.mxfp8_dequantize(out, oe)
    mean = acc / n
    err = mean - deq.T
    # per-element SR variance <= spacing^2 / 4; z-score of the mean over all elements
    sp = np.abs(deq.T) * 2 ** -3 + 1e-30
    z = err.sum() / np.sqrt(np.sum(sp ** 2 / 4) / n)
    assert abs(z) < 5
    assert np.abs(err).max() < 0.2 * np.abs(deq).max()


def test_requant_is_deterministic_in_seed_and_stream():
    rng = np.random.default_rng(9)
    q = O.nvfp4_quantize(bf16(rng.standard_normal((40, 64))), four_six=True)
    a, _ = O.requant_transpose_sr(q, seed=1, stream=0)
    b, _ = O.requant_transpose_sr(q, seed=1, stream=0)
    c, _ = O.requant_transpose_sr(q, seed=1, stream=1)
    d, _ = O.requant_transpose_sr(q, seed=2, stream=0)
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)


def test_mxfp8_quant_rows_and_cols_agree_on_transpose():
    rng = np.random.default_rng(10)
    x = bf16(rng.standard_normal((64, 96)) * 1e-3)
    rq, re = O.mxfp8_quantize_rows(x)
    cq, ce = O.mxfp8_quantize_cols(x.t().contiguous())
    assert np.array_equal(rq, cq) and np.array_equal(re, ce)
    # RTN error within half an E4M3 step of the block scale
    v = O.mxfp8_dequantize(rq, re)
    xf = x.float().numpy()
    assert np.all(np.abs(v - xf) <= np.abs(xf) * 2 ** -4 + 2.0 ** -9 * np.repeat(2.0 ** (re.astype(int) - 127), 32, 1))
    # scale rule: block amax / 2^e in (224, 448]
    am = np.abs(xf).reshape(64, 3, 32).max(-1)
    ratio = am / 2.0 ** (re.astype(int) - 127)
    assert np.all((ratio > 224) & (ratio <= 448))


# ------------------------------------------------------------------------------------------
# RHT + S2F6
# ------------------------------------------------------------------------------------------

def _sylvester32():
    i = np.arange(32)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def test_rht_matches_sylvester_and_is_self_inverse():
    rng = np.random.default_rng(11)
    H = _sylvester32()
    for mask in (0, 0xFFFFFFFF, 0x5A5A1234):
        D = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(32)])
        y = rng.integers(-50, 50, 32).astype(np.float32)       # integers: every sum is exact
        z = O.rht32(y, mask)
        assert np.array_equal(z, H @ (D * y))
        back = D * (H @ z) / 32
        assert np.array_equal(back, y)
    assert np.array_equal(H @ H, 32 * np.eye(32))


def test_s2f6_range_and_error_bound():
    f = FACTS["s2f6_range"]
    rng = np.random.default_rng(12)
    y = (rng.standard_t(3, size=(40, 256)) * np.exp(rng.uniform(-20, 20, (40, 1)))).astype(np.float32)
    y[0, :32] = 0.0
    mask = 0xC0FFEE11
    codes, e = O.rht32_s2f6_quantize(y, mask)
    assert codes.min() >= -127 and codes.max() <= 127
    assert codes.min() / 64 >= f["min"] and codes.max() / 64 <= f["max"]
    absmax = np.abs(codes.astype(int)).reshape(40, 8, 32).max(-1)
    assert np.all((absmax[1:] >= 64) & (absmax[1:] <= 127))
    xh = O.rht32_s2f6_decode(codes, e, mask)
    err = np.sqrt(((xh - y.astype(np.float64)) ** 2).reshape(40, 8, 32).sum(-1))
    bound = 2.0 ** (e.astype(np.float64) - 127) / 128
    scale = np.sqrt((y.astype(np.float64) ** 2).reshape(40, 8, 32).sum(-1))
    assert np.all(err <= bound * (1 + 1e-6) + scale * 1e-6)
    assert np.all(xh[0, :32] == 0)


def test_s2f6_outlier_spread():
    """A single outlier in a chunk: after the RHT every value carries 1/sqrt(32) of it, so the
    other values keep far more resolution than with plain per-32 scaling."""
    y = np.full((1, 32), 0.01, np.float32)
    y[0, 5] = 100.0
    codes, e = O.rht32_s2f6_quantize(y, 0x0F0F0F0F)
    xh = O.rht32_s2f6_decode(codes, e, 0x0F0F0F0F)
    plain_step = 100.0 / 127
    assert np.abs(xh[0] - y[0]).max() < plain_step / 2


# ------------------------------------------------------------------------------------------
# GEMMs
# ------------------------------------------------------------------------------------------

def test_nvfp4_gemm_all_ones_closed_form():
    K, N = 256, 8
    x = bf16(np.ones((4, K)))
    w = bf16(np.ones((2 * N, K)))
    xq = O.nvfp4_quantize(x, four_six=True)
    wq = O.nvfp4_quantize(w, rows_per_outer=N, four_six=False)
    Y = O.gemm_nvfp4_grouped(xq, wq, [0, 2, 4], N, K)
    assert np.allclose(Y, K, rtol=1e-6)


def test_nvfp4_gemm_one_hot_weights_select_columns():
    rng = np.random.default_rng(13)
    K, N = 64, 16
    x = bf16(rng.standard_normal((6, K)))
    perm = rng.permutation(K)[:N]
    w = np.zeros((N, K), np.float32)
    w[np.arange(N), perm] = 1.0
    xq = O.nvfp4_quantize(x, four_six=True)
    wq = O.nvfp4_quantize(bf16(w), rows_per_outer=N, four_six=False)
    Y = O.gemm_nvfp4_grouped(xq, wq, [0, 6], N, K)
    deq = O.nvfp4_dequantize(xq)
    wdeq = O.nvfp4_dequantize(wq)
    assert np.allclose(wdeq[np.arange(N), perm], 1.0, rtol=1e-6)
    assert np.allclose(Y, deq[:, perm], rtol=2e-6, atol=1e-30)


def test_nvfp4_gemm_bruteforce_small_with_gather():
    rng = np.random.default_rng(14)
    K, N, T = 32, 4, 5
    x = bf16(rng.standard_normal((T, K)))
    w = bf16(rng.standard_normal((2 * N, K)) * 0.02)
    xq = O.nvfp4_quantize(x, four_six=True)
    wq = O.nvfp4_quantize(w, rows_per_outer=N, four_six=False)
    gather = np.array([4, 0, 2, 2, 1, 3], np.int32)
    offsets = [0, 2, 6]
    Y = O.gemm_nvfp4_grouped(xq, wq, offsets, N, K, gather=gather)
    mags = FACTS["fp4_grid"]["magnitudes"]

    def val(q, r, k):
        c = (q["codes"][r, k // 2] >> (4 * (k & 1))) & 15
        sb = q["scales"][r, k // 16]
        e, m = (sb >> 3) & 15, sb & 7
        s = (m / 8 * 2 ** -6) if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        return (-1 if c & 8 else 1) * mags[c & 7] * s

    for s in range(6):
        g = 0 if s < 2 else 1
        for n in range(N):
            acc = sum(val(xq, gather[s], k) * val(wq, g * N + n, k) for k in range(K))
            want = acc * xq["outer"][gather[s]] * wq["outer"][(g * N + n) // N]
            assert math.isclose(Y[s, n], want, rel_tol=1e-6, abs_tol=1e-30)


def test_nvfp4_gemm_vs_numpy_matmul():
    rng = np.random.default_rng(15)
    K, N = 128, 48
    x = bf16(rng.standard_normal((40, K)))
    w = bf16(rng.standard_normal((3 * N, K)) * 0.02)
    xq = O.nvfp4_quantize(x, four_six=True)
    wq = O.nvfp4_quantize(w, rows_per_outer=N, four_six=False)
    offsets = [0, 7, 7, 40]
    Y = O.gemm_nvfp4_grouped(xq, wq, offsets, N, K)
    xd = O.nvfp4_dequantize(xq).astype(np.float64)
    wd = O.nvfp4_dequantize(wq).astype(np.float64)
    for g in range(3):
        s0, s1 = offsets[g], offsets[g + 1]
        ref = xd[s0:s1] @ wd[g * N:(g + 1) * N].T
        assert np.allclose(Y[s0:s1], ref, rtol=1e-5, atol=1e-6)
    # the sampled form agrees with the full form
    rows, cols = [0, 20, 39], [0, 13, 47]
    el = O.gemm_nvfp4_elems(xq, wq, offsets, N, K, rows, cols)
    assert np.allclose(el, Y[rows, cols], rtol=1e-6)


def test_mxfp8_gemms_vs_dense_products():
    rng = np.random.default_rng(16)
    G, N, K = 3, 64, 96
    offsets = np.array([0, 10, 10, 75], np.int64)
    M = int(offsets[-1])
    dy = bf16(rng.standard_normal((M, N)) * 1e-3)
    w = bf16(rng.standard_normal((G * N, K)) * 0.02)
    x = bf16(rng.standard_normal((M, K)))
    wq = O.nvfp4_quantize(w, rows_per_outer=N, four_six=False)
    xq = O.nvfp4_quantize(x, four_six=True)
    dq, de = O.mxfp8_quantize_rows(dy)
    wt, wte = O.requant_transpose_sr(wq, offsets=np.arange(G + 1) * N, seed=3, stream=1)
    dX = O.gemm_mxfp8_dgrad(dq, de, wt, wte, offsets, N, K)
    dyv = O.mxfp8_dequantize(dq, de)
    wtv = O.mxfp8_dequantize(wt, wte)                       # [K x G*N]
    for g in range(G):
        s0, s1 = offsets[g], offsets[g + 1]
        ref = dyv[s0:s1] @ wtv[:, g * N:(g + 1) * N].T
        assert np.allclose(dX[s0:s1], ref, rtol=1e-6, atol=1e-12)
    dt, dte = O.mxfp8_quantize_cols(dy, offsets=offsets)
    xt, xte = O.requant_transpose_sr(xq, offsets=offsets, seed=3, stream=2)
    dW = O.gemm_mxfp8_wgrad(dt, dte, xt, xte, offsets, N, K)
    dtv = O.mxfp8_dequantize(dt, dte)
    xtv = O.mxfp8_dequantize(xt, xte)
    P = [32, 0, 96]
    po = [0, 32, 32]
    for g in range(G):
        ref = dtv[:, po[g]:po[g] + P[g]] @ xtv[:, po[g]:po[g] + P[g]].T
        assert np.allclose(dW[g * N:(g + 1) * N], ref, rtol=1e-6, atol=1e-12)
    assert np.all(dW[N:2 * N] == 0)


# ------------------------------------------------------------------------------------------
# SwiGLU, routing
# ------------------------------------------------------------------------------------------

def test_swiglu_closed_forms_and_derivative():
    F = 4
    h = np.array([[0.0, 1.0, -2.0, 3.0, 5.0, 2.0, 1.0, -1.0]], np.float32)
    a = O.swiglu(h, F)
    sig = lambda v: 1 / (1 + math.exp(-v))
    for j in range(F):
        h1, h3 = float(h[0, j]), float(h[0, F + j])
        assert math.isclose(a[0, j], h1 * sig(h1) * h3, rel_tol=1e-12)
    assert a[0, 0] == 0.0
    # backward against central finite differences of the forward
    rng = np.random.default_rng(17)
    h13 = bf16(rng.standard_normal((3, 2 * F)))
    hf = h13.float().numpy()
    da = rng.standard_normal((3, F)).astype(np.float32)
    g = O.swiglu_bwd(da, h13, F)
    eps = 1e-6
    for j in range(2 * F):
        hp, hm = hf.astype(np.float64).copy(), hf.astype(np.float64).copy()
        hp[:, j] += eps
        hm[:, j] -= eps
        fp = (hp[:, :F] / (1 + np.exp(-hp[:, :F])) * hp[:, F:] * da).sum(1)
        fm = (hm[:, :F] / (1 + np.exp(-hm[:, :F])) * hm[:, F:] * da).sum(1)
        assert np.allclose(g[:, j], (fp - fm) / (2 * eps), rtol=1e-5, atol=1e-7)


def test_routing_vs_stable_argsort():
    rng = np.random.default_rng(18)
    T, E, k = 50, 12, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[7, 2] = logits[7, 9]                                 # a tie: lower expert first
    r = O.route_topk(logits, k)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert np.array_equal(r["ids"], order)
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(r["gates"], np.take_along_axis(p, order, 1), rtol=1e-6)
    flat = r["ids"].reshape(-1)
    keys = flat.astype(np.int64) * T + np.repeat(np.arange(T), k)
    srt = np.argsort(keys, kind="stable")
    assert np.array_equal(r["gather"], srt // k)
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(r["slot_of"][srt], np.arange(T * k))


_ROCRAND_PROBE = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
struct probe : rocrand_device::philox4x32_10_engine {
  probe() : rocrand_device::philox4x32_10_engine(0, 0, 0) {}
  uint4 run(uint4 c, uint2 k) { return ten_rounds(c, k); }
};
int main() {
  probe eng;
  unsigned c[4], k[2];
  while (scanf("%x %x %x %x %x %x", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
    uint4 r = eng.run(uint4{c[0], c[1], c[2], c[3]}, uint2{k[0], k[1]});
    printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
}
"""


def test_philox_vs_rocrand_header(tmp_path):
    """Cross-check against the open-source rocRAND Philox4x32-10 (host-compiled header)."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = tmp_path / "probe.cpp"
    src.write_text(_ROCRAND_PROBE)
    exe = tmp_path / "probe"
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-host-only", str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    rng = np.random.default_rng(19)
    vecs = rng.integers(0, 2**32, (300, 6), dtype=np.uint64)
    inp = "\n".join(" ".join(f"{int(v):x}" for v in row) for row in vecs) + "\n"
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    for row, line in zip(vecs, out):
        want = O.philox4x32_10(row[:4], row[4:])
        assert line == " ".join(f"{int(w):08x}" for w in want)


def test_requant_window_matches_full_output():
    rng = np.random.default_rng(20)
    q = O.nvfp4_quantize(bf16(rng.standard_t(3, size=(200, 64))), four_six=True)
    full, fe = O.requant_transpose_sr(q, seed=4, stream=2)
    w, we = O.requant_window(q, 64, 96, seed=4, stream=2)
    assert np.array_equal(w, full[:, 64:160]) and np.array_equal(we, fe[:, 2:5])
    tail, te = O.requant_window(q, 192, 8, seed=4, stream=2)
    assert np.array_equal(tail, full[:, 192:224]) and np.array_equal(te, fe[:, 6:7])


# ------------------------------------------------------------------------------------------
# combine (receiver side of the w2 output exchange)
# ------------------------------------------------------------------------------------------

def test_combine_one_hot_code_closed_form():
    """A chunk whose only nonzero code is c at position 0 decodes to D (c 2^(e-133)) H[:, 0] / 32,
    and the first Hadamard column is all ones: every value is +-c 2^(e-138), signed by the mask."""
    H, mask = 64, 0x80000003
    codes = np.zeros((3, H), np.int8)
    e8m0 = np.full((3, H // 32), 127, np.uint8)
    codes[1, 32] = -100
    e8m0[1, 1] = 130
    slot_of = np.array([[1]], np.int32)
    out = O.moe_combine_s2f6(codes, e8m0, mask, slot_of, np.array([[0.75]], np.float32))
    D = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(32)])
    assert np.all(out[0, :32] == 0)
    assert np.array_equal(out[0, 32:], 0.75 * D * (-100.0 * 2.0 ** (130 - 138)))


def test_combine_round_trip_and_gate_linearity():
    """Slots that carry a token's rows scaled by its gates: the combine returns their weighted sum
    within the S2F6 error bound of each slot; duplicated routes add their gates."""
    rng = np.random.default_rng(21)
    T, k, H, mask = 24, 3, 128, 0x13579BDF
    M = T * k
    y = (rng.standard_normal((M, H)) * np.exp(rng.uniform(-6, 6, (M, 1)))).astype(np.float32)
    codes, e = O.rht32_s2f6_quantize(y, mask)
    perm = rng.permutation(M).astype(np.int32).reshape(T, k)
    gates = rng.dirichlet(np.ones(k), T).astype(np.float32)
    out = O.moe_combine_s2f6(codes, e, mask, perm, gates)
    ref = np.einsum("tk,tkh->th", gates.astype(np.float64), y.astype(np.float64)[perm])
    # per slot and chunk the decode error is at most 2^(e-127)/128 in the 2-norm
    bound = (2.0 ** (e.astype(np.float64) - 127) / 128)[perm]                  # [T, k, H/32]
    err = np.sqrt(((out - ref) ** 2).reshape(T, H // 32, 32).sum(-1))
    assert np.all(err <= (gates[..., None] * bound).sum(1) * (1 + 1e-6))
    # two routes to one slot behave as one route with the summed gate
    dup = np.stack([perm[:, 0], perm[:, 0]], 1)
    g2 = np.stack([gates[:, 0], gates[:, 1]], 1)
    one = O.moe_combine_s2f6(codes, e, mask, perm[:, :1], (gates[:, 0] + gates[:, 1])[:, None])
    assert np.allclose(O.moe_combine_s2f6(codes, e, mask, dup, g2), one, rtol=1e-6, atol=0)
    # k = 1 with gate 1 is the plain decode, un-permuted
    dec = O.rht32_s2f6_decode(codes, e, mask)
    assert np.array_equal(O.moe_combine_s2f6(codes, e, mask, perm[:, :1], np.ones((T, 1), np.float32)),
                          dec[perm[:, 0]])


def test_plain_s2f6_grid_values_round_trip_and_bound():
    """Plain per-32 S2F6: values on the grid (largest |c| in [64, 127]) come back exactly with the
    scale they were built with; others are within half a step, 2^(e-127)/128."""
    rng = np.random.default_rng(22)
    c = rng.integers(-127, 128, (6, 64))
    c[:, 0] = 127
    c[:, 32] = -64
    s = rng.integers(-20, 20, (6, 2))
    y = (c.reshape(6, 2, 32) / 64.0 * 2.0 ** s[..., None]).reshape(6, 64).astype(np.float32)
    codes, e = O.s2f6_quantize(y)
    assert np.array_equal(codes, c) and np.array_equal(e.astype(int), s + 127)
    assert np.array_equal(O.s2f6_dequantize(codes, e), y.astype(np.float64))
    y = (rng.standard_t(3, (40, 256)) * np.exp(rng.uniform(-10, 10, (40, 1)))).astype(np.float32)
    codes, e = O.s2f6_quantize(y)
    half = np.repeat(2.0 ** (e.astype(np.float64) - 127) / 128, 32, axis=1)
    assert np.all(np.abs(O.s2f6_dequantize(codes, e) - y) <= half)
    assert np.all(np.abs(codes.astype(int)).reshape(40, 8, 32).max(-1) >= 64)


def _e4m3_by_torch(codes, e8m0):
    """MXFP8 values decoded by torch's float8_e4m3fn type (independent of the oracle's decoder)."""
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    R, Cc = c.shape
    return (c.reshape(R, Cc // 32, 32) * 2.0 ** (np.asarray(e8m0, np.float64) - 127)[..., None]).reshape(R, Cc)


def test_mxfp8_forward_vs_library_decode_and_matmul():
    """Grouped MXFP8 forward with a gather, an empty group and ragged groups, against torch's E4M3
    decode and a numpy matmul per group."""
    rng = np.random.default_rng(23)
    G, N, K, T = 4, 64, 96, 50
    offsets = np.array([0, 17, 17, 60, 71], np.int64)
    M = int(offsets[-1])
    gather = rng.integers(0, T, M).astype(np.int32)
    x = bf16(rng.standard_t(4, (T, K)))
    w = bf16(rng.standard_normal((G * N, K)) * 0.02)
    xq, xe = O.mxfp8_quantize_rows(x)
    wq, we = O.mxfp8_quantize_rows(w)
    Y = O.gemm_mxfp8_fwd(xq, xe, wq, we, offsets, N, K, gather=gather)
    xv, wv = _e4m3_by_torch(xq, xe), _e4m3_by_torch(wq, we)
    for g in range(G):
        s0, s1 = offsets[g], offsets[g + 1]
        ref = xv[gather[s0:s1]] @ wv[g * N:(g + 1) * N].T
        assert np.allclose(Y[s0:s1], ref, rtol=1e-12, atol=1e-300)
    # without a gather the slot is the row (one group of 41 slots)
    Y2 = O.gemm_mxfp8_fwd(xq[:41], xe[:41], wq, we, [0, 41], N, K)
    assert np.allclose(Y2, xv[:41] @ wv[:N].T, rtol=1e-12, atol=1e-300)


def test_mxfp8_forward_one_hot_closed_form():
    """X all ones (each quantizes exactly: 1 = 256 * 2^-8) and W rows one-hot with E4M3-exact values:
    Y[s, n] is the nonzero value of W row g N + n."""
    G, N, K = 2, 32, 64
    offsets = np.array([0, 5, 9], np.int64)
    x = bf16(np.ones((9, K)))
    vals = np.array([1.5, -0.25, 3.0, -448.0, 0.0078125, 6.0, -1.0, 2.75] * 8)   # 64 rows
    w = np.zeros((G * N, K))
    w[np.arange(G * N), np.arange(G * N) % K] = vals
    xq, xe = O.mxfp8_quantize_rows(x)
    wq, we = O.mxfp8_quantize_rows(bf16(w))
    Y = O.gemm_mxfp8_fwd(xq, xe, wq, we, offsets, N, K)
    for s in range(9):
        g = 0 if s < 5 else 1
        assert np.array_equal(Y[s], vals[g * N:(g + 1) * N])


# ------------------------------------------------------------------------------------------
# MX with E2M1 elements (the FP4 backward)
# ------------------------------------------------------------------------------------------

def _fp4_decode(codes, e8m0):
    """E2M1 codes (one per byte) x 2^(e - 127) from the pages' grid (independent of the oracle)."""
    grid = np.array(FACTS["fp4_grid"]["magnitudes"])
    c = np.asarray(codes).astype(int)
    v = np.where(c & 8, -1.0, 1.0) * grid[c & 7]
    return v * np.repeat(2.0 ** (np.asarray(e8m0, np.float64) - 127), 32, axis=1)


def test_mxfp4_quant_rule_rows_cols_and_nearest():
    rng = np.random.default_rng(24)
    x = bf16(rng.standard_t(4, (64, 96)))
    rq, re = O.mxfp8_quantize_rows(x, target=O.TARGET_E2M1)
    cq, ce = O.mxfp8_quantize_cols(x.t().contiguous(), target=O.TARGET_E2M1)
    assert np.array_equal(rq, cq) and np.array_equal(re, ce)
    assert rq.max() <= 15
    xf = x.float().numpy().astype(np.float64)
    # scale rule with M = 6: block amax / 2^e in (3, 6]
    am = np.abs(xf).reshape(64, 3, 32).max(-1)
    ratio = am / 2.0 ** (re.astype(int) - 127)
    assert np.all((ratio > 3) & (ratio <= 6))
    # RNE: each value is a nearest grid point (brute force over the 15 candidates of its block)
    v = _fp4_decode(rq, re)
    grid = np.array(FACTS["fp4_grid"]["magnitudes"])
    cand = np.concatenate([-grid[::-1], grid])[None, None, :] * np.repeat(2.0 ** (re.astype(int) - 127), 32, 1)[..., None]
    best = np.abs(cand - xf[..., None]).min(-1)
    assert np.all(np.abs(v - xf) == best)


def test_mxfp4_sr_is_unbiased():
    rng = np.random.default_rng(25)
    x = bf16(rng.standard_normal((4, 64)))
    xf = x.float().numpy().astype(np.float64)
    acc = np.zeros_like(xf)
    n = 400
    for s in range(n):
        q, e = O.mxfp8_quantize_rows(x, sr=True, seed=s, stream=3, target=O.TARGET_E2M1)
        acc += _fp4_decode(q, e)
    mean = acc / n
    # per element the SR error is at most one grid step (<= 2^(e-127) * 2); z-test on the sum
    step = np.repeat(2.0 ** (O.mxfp8_quantize_rows(x, target=O.TARGET_E2M1)[1].astype(int) - 127), 32, 1) * 2
    z = (mean - xf).sum() / np.sqrt((step ** 2 / 4).sum() / n)
    assert abs(z) < 5


def test_mxfp4_gemms_vs_dense_products():
    """FP4 dgrad and wgrad (the requantized operands on the E2M1 grid) against the pages' grid
    decode and numpy matmuls."""
    rng = np.random.default_rng(26)
    G, N, K = 3, 64, 96
    offsets = np.array([0, 10, 10, 75], np.int64)
    M = int(offsets[-1])
    dy = bf16(rng.standard_normal((M, N)) * 1e-3)
    w = bf16(rng.standard_normal((G * N, K)) * 0.02)
    x = bf16(rng.standard_normal((M, K)))
    wq = O.nvfp4_quantize(w, rows_per_outer=N, four_six=False)
    xq = O.nvfp4_quantize(x, four_six=True)
    dq, de = O.mxfp8_quantize_rows(dy, sr=True, seed=4, stream=6, target=O.TARGET_E2M1)
    wt, wte = O.requant_transpose_sr(wq, offsets=np.arange(G + 1) * N, target=O.TARGET_E2M1, seed=3, stream=1)
    dX = O.gemm_mxfp8_dgrad(dq, de, wt, wte, offsets, N, K, target=O.TARGET_E2M1)
    dyv, wtv = _fp4_decode(dq, de), _fp4_decode(wt, wte)
    for g in range(G):
        s0, s1 = offsets[g], offsets[g + 1]
        ref = dyv[s0:s1] @ wtv[:, g * N:(g + 1) * N].T
        assert np.allclose(dX[s0:s1], ref, rtol=1e-6, atol=1e-12)
    dt, dte = O.mxfp8_quantize_cols(dy, offsets=offsets, sr=True, seed=4, stream=7, target=O.TARGET_E2M1)
    xt, xte = O.requant_transpose_sr(xq, offsets=offsets, target=O.TARGET_E2M1, seed=3, stream=2)
    dW = O.gemm_mxfp8_wgrad(dt, dte, xt, xte, offsets, N, K, target=O.TARGET_E2M1)
    dtv, xtv = _fp4_decode(dt, dte), _fp4_decode(xt, xte)
    P, po = [32, 0, 96], [0, 32, 32]
    for g in range(G):
        ref = dtv[:, po[g]:po[g] + P[g]] @ xtv[:, po[g]:po[g] + P[g]].T
        assert np.allclose(dW[g * N:(g + 1) * N], ref, rtol=1e-6, atol=1e-12)
    # one sampled element through the generic dot
    assert np.isclose(O.mxfp8_dot(dt, dte, xt, xte, 5, 7, 32, 96, target=O.TARGET_E2M1), dW[2 * N + 5, 7], rtol=1e-6)


# ------------------------------------------------------------------------------------------
# 16 x 16 square blocks
# ------------------------------------------------------------------------------------------

def _nibbles(codes):
    c = np.asarray(codes)
    out = np.zeros((c.shape[0], c.shape[1] * 2), np.uint8)
    out[:, 0::2], out[:, 1::2] = c & 15, c >> 4
    return out


def test_2d_blocks_transpose_bit_identity_and_tile_scales():
    """Quantizing X^T gives exactly the transpose of X's codes and (tile) scales: a square block
    is the same set of values either way ([AREX S3])."""
    rng = np.random.default_rng(27)
    x = bf16(rng.standard_t(3, (64, 96)))
    a = O.nvfp4_quantize_2d(x, 64)
    b = O.nvfp4_quantize_2d(x.t().contiguous(), 96)
    assert np.array_equal(_nibbles(b["codes"]), _nibbles(a["codes"]).T)
    assert a["outer"][0] == b["outer"][0]
    tiles = a["scales"].reshape(4, 16, 6)
    assert np.all(tiles == tiles[:, :1, :])                   # one scale per tile
    assert np.array_equal(tiles[:, 0, :].T, b["scales"].reshape(6, 16, 4)[:, 0, :])


def test_2d_blocks_reduce_to_1d_when_tile_rows_repeat():
    """If the 16 rows of every tile are equal, each tile's amax is its rows' block amax and the 2D
    result equals the 1D weight-mode quantization."""
    rng = np.random.default_rng(28)
    base = rng.standard_normal((4, 128)) * np.exp(rng.uniform(-3, 3, (4, 1)))
    x = bf16(np.repeat(base, 16, axis=0))
    a = O.nvfp4_quantize_2d(x, 32)
    b = O.nvfp4_quantize(x, rows_per_outer=32, four_six=False)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    assert np.array_equal(a["outer"], b["outer"])
