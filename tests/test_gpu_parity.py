"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact for every code, scale byte, index and integer output; GEMM outputs within 2e-3
relative Frobenius error of the oracle. Inputs are seeded synthetic tensors from
precision_moe_numerics_amd.inputs (or seeded numpy draws), sized so the oracle finishes in
seconds while the kernels still see several tiles and ragged tails. The oracle always starts from
the same original inputs as the library (it quantizes them itself); no output of the library is
ever an input of the oracle. Library outputs are read back only through the small test-side
decoders in tests/decoders.py.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decoders import decode_s2f6_rows, fp4_value, unblock

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def P():
    import precision_moe_numerics_amd as P
    return P


@pytest.fixture(scope="module")
def I():
    from precision_moe_numerics_amd import inputs as I
    return I


def npy(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bf16_np(a):
    return torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16)


def rel_fro(got, ref):
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)


def assert_nvfp4_equal(q, ref, rows=None):
    codes, scales, outer = npy(q.codes), npy(q.scales), npy(q.outer)
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    assert np.array_equal(scales, ref["scales"]), "scale bytes differ"
    assert np.array_equal(codes, ref["codes"]), "codes differ"
    if rows is None:
        assert np.array_equal(outer, ref["outer"]), "outer scales differ"


# ------------------------------------------------------------------------------------------
# NVFP4 quantization
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,nu", [(256, 512, 0), (300, 7168, 3), (130, 1536, 4), (67, 16, 3),
                                          (33, 8208, 3), (5, 4096, 0)])
@pytest.mark.parametrize("four_six", [True, False])
def test_nvfp4_quantize_rows(P, I, rows, cols, nu, four_six):
    x = I.student_t((rows, cols), nu, 0.5, 11) if nu else I.normal((rows, cols), 1.0, 12)
    q = P.nvfp4_quantize(x.to(DEV), P.NVFP4_ACT if four_six else P.NVFP4_WEIGHT)
    ref = O.nvfp4_quantize(x, 1, four_six)
    assert_nvfp4_equal(q, ref)


@pytest.mark.parametrize("rpo", [256, 512, 32])
def test_nvfp4_quantize_weight_groups(P, I, rpo):
    w = I.normal((4 * 256 + 512, 512), 0.02, 13)[: (4 * 256 + 512) // rpo * rpo]
    q = P.nvfp4_quantize(w.to(DEV), P.NVFP4_WEIGHT, rows_per_outer=rpo)
    ref = O.nvfp4_quantize(w, rpo, False)
    assert_nvfp4_equal(q, ref)


@pytest.mark.parametrize("four_six", [False, True])
def test_nvfp4_large_weight_groups(P, I, four_six):
    """13 groups of 2048 x 7168 (29.4 MB of bf16 each, the size of one expert's w1 or w3): the
    group amax pass spreads each group over many workgroups that fold into one atomic max, so a
    group whose amax is one isolated value checks the fold. Sampled groups, bit-exact."""
    G, R, Cc = 13, 2048, 7168
    w = I.normal((G * R, Cc), 0.02, 31, DEV)
    w[4 * R + 17, 5] = 0.75                              # a group whose amax is an isolated outlier
    q = P.nvfp4_quantize(w, P.NVFP4_ACT if four_six else P.NVFP4_WEIGHT, rows_per_outer=R)
    codes, scales, outer = npy(q.codes), npy(q.scales), npy(q.outer)
    for g in (0, 4, 5, 9, 10, 12):
        ref = O.nvfp4_quantize(w[g * R:(g + 1) * R].cpu(), R, four_six)
        assert np.array_equal(scales[g * R:(g + 1) * R], ref["scales"]), g
        assert np.array_equal(codes[g * R:(g + 1) * R], ref["codes"]), g
        assert outer[g] == ref["outer"][0], g


def test_nvfp4_worked_example_with_outer_hook(P):
    x = np.zeros((1, 16), np.float32)
    x[0, :5] = [-54.0, 5.4, 1.0, -2.0, 0.3]
    q = P.nvfp4_quantize(bf16_np(x).to(DEV), P.NVFP4_WEIGHT, outer_in=torch.ones(1, device=DEV))
    assert npy(q.scales)[0, 0] == 0x51
    c = npy(q.codes)[0]
    assert c[0] & 15 == 0xF and (c[0] >> 4) == 0x1        # -6 and 0.5


def test_nvfp4_edge_values(P):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    x[0] = 0.0                                  # all-zero row: outer 1, zero codes
    x[1, :16] = 1e-38                           # tiny values
    x[2, 16:32] = -0.0
    x[3] *= 1e30                                # large values
    x[4, ::16] = 3e38                           # bf16 near max
    x[5, :] = 6.0
    xb = bf16_np(x)
    for four_six in (True, False):
        q = P.nvfp4_quantize(xb.to(DEV), P.NVFP4_ACT if four_six else P.NVFP4_WEIGHT)
        assert_nvfp4_equal(q, O.nvfp4_quantize(xb, 1, four_six))


@pytest.mark.parametrize("cols", [32, 1024, 2048, 4096, 8192, 8208])
def test_nvfp4_four_over_six_exact_tie_keeps_six(P, cols):
    """[2688, 0 x 15 | 6, 0 x 15]: both candidates of the second block are exact, the tie keeps 6
    (scale byte 0x38; a '<=' rule would store 0x3C). Checked through the one-wavefront row kernel
    (every row-length instantiation and the long-row fallback) and through the outer-scale hook."""
    x = np.zeros((3, cols), np.float32)
    for r in range(3):
        x[r, 0], x[r, 16] = 2688.0, 6.0
        x[r, cols - 16] = 6.0 if cols > 32 else x[r, cols - 16]     # a tie in the row's last block
    xb = bf16_np(x)
    ref = O.nvfp4_quantize(xb, 1, True)
    assert ref["scales"][0, 1] == 0x38
    for outer_in in (None, torch.ones(3, device=DEV)):
        q = P.nvfp4_quantize(xb.to(DEV), P.NVFP4_ACT, outer_in=outer_in)
        assert_nvfp4_equal(q, ref)
        assert npy(q.scales)[0, 1] == 0x38 and npy(q.scales)[2, cols // 16 - 1] == 0x38


def test_nvfp4_division_free_reciprocal_is_exact(P):
    """The activation quantizer forms 1/d as the hardware reciprocal plus one Newton step on rows
    whose outer scale is at least 2^-96; d then lies in [2^-105, 2^126). Over every fp32 value of
    that range the result equals the IEEE quotient 1.0f / d bit for bit."""
    assert P.probe_recip_check(0x0B000000, 0x7E7FFFFF) == 0


@pytest.mark.parametrize("four_six", [True, False])
def test_nvfp4_rows_on_both_sides_of_the_exact_division_switch(P, I, four_six):
    """Rows scaled by powers of two from 2^-120 to 2^100: outer scales below 2^-96 take the IEEE
    division sequences, the others the division-free quotients; all bit-exact with the oracle."""
    x = I.normal((16, 7168), 1.0, 41).float()
    pw = [-120, -100, -90, -86, -85, -84, -83, -60, -20, 0, 0, 20, 60, 90, 100, -127]
    x = (x * torch.tensor([2.0 ** p for p in pw])[:, None]).to(torch.bfloat16)
    q = P.nvfp4_quantize(x.to(DEV), P.NVFP4_ACT if four_six else P.NVFP4_WEIGHT)
    ref = O.nvfp4_quantize(x, 1, four_six)
    assert_nvfp4_equal(q, ref)
    so = ref["outer"]
    assert (so < 2.0 ** -96).sum() >= 4 and (so >= 2.0 ** -96).sum() >= 8


def test_nvfp4_empty(P):
    q = P.nvfp4_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV))
    assert q.codes.shape == (0, 32)


def test_nvfp4_full_size_quantizer_workload_sampled_rows(P, I):
    """8192 x 7168 Student-t(3) * 0.5, ACT mode with 4/6: sampled rows checked bit for bit."""
    x = I.quantizer(DEV)["x"]
    q = P.nvfp4_quantize(x, P.NVFP4_ACT)
    rows = np.sort(np.random.default_rng(5).choice(8192, 48, replace=False))
    ref = O.nvfp4_quantize(x[torch.as_tensor(rows, device=DEV)].cpu(), 1, True)
    assert_nvfp4_equal(q, ref, rows=rows)
    assert np.array_equal(npy(q.outer)[rows], ref["outer"])
    # the same call twice gives the same bits
    q2 = P.nvfp4_quantize(x, P.NVFP4_ACT)
    assert torch.equal(q.codes, q2.codes) and torch.equal(q.scales, q2.scales)


# ------------------------------------------------------------------------------------------
# Requantization (dequant -> transpose -> SR) and MXFP8 gradients
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols", [(256, 512), (97, 4096), (64, 16), (1, 32)])
def test_requant_ungrouped(P, I, rows, cols):
    x = I.student_t((rows, cols), 3, 0.5, 21)
    q = P.nvfp4_quantize(x.to(DEV), P.NVFP4_ACT)
    out, oe, po = P.requant_transpose_sr_mxfp8(q, seed=7, rng_stream=3, want_padded_offsets=True)
    ro, roe = O.requant_transpose_sr(O.nvfp4_quantize(x, 1, True), seed=7, stream=3)
    Pt = ro.shape[1]
    assert np.array_equal(npy(out)[:, :Pt], ro) and np.array_equal(npy(oe)[:, :Pt // 32], roe)
    assert list(npy(po)) == [0, Pt]


def test_requant_grouped_gathered_ragged(P, I):
    rng = np.random.default_rng(22)
    x = I.student_t((300, 1536), 4, 1.0, 23)
    q = P.nvfp4_quantize(x.to(DEV), P.NVFP4_ACT)
    counts = [37, 0, 300, 1, 64, 298]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    gather = rng.integers(0, 300, offsets[-1]).astype(np.int32)
    out, oe, po = P.requant_transpose_sr_mxfp8(q, gather=torch.as_tensor(gather, device=DEV),
                                               offsets=torch.as_tensor(offsets, device=DEV), seed=11,
                                               rng_stream=5, want_padded_offsets=True)
    ro, roe = O.requant_transpose_sr(O.nvfp4_quantize(x, 1, True), gather=gather, offsets=offsets, seed=11, stream=5)
    Pt = ro.shape[1]
    assert np.array_equal(npy(out)[:, :Pt], ro) and np.array_equal(npy(oe)[:, :Pt // 32], roe)
    assert list(npy(po)) == list(np.concatenate([[0], np.cumsum([(c + 31) // 32 * 32 for c in counts])]))


def test_requant_weights(P, I):
    w = I.normal((3 * 256, 512), 0.02, 24)
    q = P.nvfp4_quantize(w.to(DEV), P.NVFP4_WEIGHT, rows_per_outer=256)
    out, oe, _ = P.requant_transpose_sr_mxfp8(q, seed=2, rng_stream=1, ld=768)
    ro, roe = O.requant_transpose_sr(O.nvfp4_quantize(w, 256, False), seed=2, stream=1)
    assert np.array_equal(npy(out), ro) and np.array_equal(npy(oe), roe)


def test_requant_e2m1_worked_example(P):
    rows = 64
    x = np.zeros((rows, 16), np.float32)
    x[:, 0] = -54.0
    x[:, 1] = 5.4
    x[3, 1] = 9.0
    q = P.nvfp4_quantize(bf16_np(x).to(DEV), P.NVFP4_WEIGHT, outer_in=torch.ones(rows, device=DEV))
    out, oe, _ = P.requant_transpose_sr_mxfp8(q, target=P.TARGET_E2M1, seed=5, rng_stream=3)
    rq = O.nvfp4_quantize(bf16_np(x), 1, False, outer_in=np.ones(rows, np.float32))
    ro, roe = O.requant_transpose_sr(rq, target=O.TARGET_E2M1, seed=5, stream=3)
    assert np.array_equal(npy(out)[:, :64], ro) and np.array_equal(npy(oe)[:, :2], roe)
    # column 1, block 0 has max 9 -> E8M0 scale 2; every 4.5 (rows other than 3) became 2 or 3
    assert npy(oe)[1, 0] == 128
    vals = {fp4_value(int(c)) for j, c in enumerate(npy(out)[1, :32]) if j != 3}
    assert vals <= {2.0, 3.0}


def test_requant_full_size_windows_and_unbiased(P, I):
    """Requant of the 8192 x 7168 quantizer workload (seed 1, stream 0): windows of 32-slot
    blocks bit for bit, and the SR mean over the whole tensor unbiased against the dequantized
    forward values."""
    data = I.quantizer(DEV)
    q = P.nvfp4_quantize(data["x"], P.NVFP4_ACT)
    out, oe, _ = P.requant_transpose_sr_mxfp8(q, seed=data["seed"], rng_stream=data["stream"])
    ref_q = O.nvfp4_quantize(data["x"].cpu(), 1, True)
    for s0 in (0, 4096, 8160):
        ro, roe = O.requant_window(ref_q, s0, 32, seed=data["seed"], stream=data["stream"])
        assert np.array_equal(npy(out[:, s0:s0 + 32]), ro)
        assert np.array_equal(npy(oe[:, s0 // 32:s0 // 32 + 1]), roe)
    # unbiasedness on sampled columns: the mean of (requant - forward value) over many
    # elements is within a few standard errors of zero
    cols = torch.arange(0, 7168, 97, device=DEV)
    e4 = torch.tensor([O.e4m3_value(c) if (c & 0x7F) != 0x7F else 0.0 for c in range(256)], dtype=torch.float64,
                      device=DEV)
    got = e4[out[cols].long()] * torch.pow(2.0, oe[cols].double() - 127).repeat_interleave(32, dim=1)
    deq = torch.from_numpy(O.nvfp4_dequantize(dict(codes=ref_q["codes"][:, :], scales=ref_q["scales"],
                                                   outer=ref_q["outer"], rows_per_outer=1))).to(DEV).double()
    fwd = deq[:, cols].t()
    d = (got[:, :8192] - fwd)
    spacing = torch.pow(2.0, torch.floor(torch.log2(fwd.abs().clamp_min(1e-30))) - 3)
    z = d.sum() / torch.sqrt((spacing ** 2 / 4).sum())
    assert abs(z.item()) < 5


def test_gemm_fwd_many_groups(P, I):
    """200 experts (the group lookup scans them 64 at a time), most with 0..40 slots and a few
    with several tiles; F32 against the oracle, SwiGLU's h13 against it."""
    rng = np.random.default_rng(31)
    counts = [int(c) for c in rng.integers(0, 41, 200)]
    counts[7], counts[150], counts[199] = 300, 0, 513
    N, K = 256, 128
    d = _moe_small(P, I, counts, N, K, gather_rows=None, seed=90)
    y = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_F32)
    ref = O.gemm_nvfp4_grouped(d["rxq"], d["rwq"], d["offsets"], N, K)
    assert rel_fro(npy(y), ref) <= 1e-5
    a, h13 = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_SWIGLU, save_h13=True)
    assert torch.equal(h13, y.to(torch.bfloat16))
    assert rel_fro(npy(a.float()), O.swiglu(ref, N // 2)) <= 2e-3


@pytest.mark.parametrize("counts,N,K,gather_rows", [([70, 300, 129, 128, 1], 768, 320, None),
                                                    ([5, 0, 600], 512, 448, 700)])
def test_gemm_fwd_short_units(P, I, counts, N, K, gather_rows):
    """Slot units of at most 128 slots (an expert's last) run as 512 weight rows x 128 slots,
    covering two weight tiles; with an odd number of weight tiles the last one keeps the
    256 x 256 shape. K = 64 mod 128 leaves a half-full last k-stage. All four epilogues."""
    d = _moe_small(P, I, counts, N, K, gather_rows, seed=80)
    F = N // 2
    y = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_F32, gather=d["ggather"])
    ref = O.gemm_nvfp4_grouped(d["rxq"], d["rwq"], d["offsets"], N, K, gather=d["gather"])
    assert rel_fro(npy(y), ref) <= 1e-5          # exact products, fp32 accumulation
    yb = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_BF16, gather=d["ggather"])
    assert torch.equal(yb, y.to(torch.bfloat16))
    a, h13 = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_SWIGLU, gather=d["ggather"],
                                    save_h13=True)
    assert rel_fro(npy(a.float()), O.swiglu(ref, F)) <= 2e-3
    assert torch.equal(h13, y.to(torch.bfloat16))
    mask = I.sign_mask(3)
    c, e = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_RHT32_S2F6, gather=d["ggather"],
                                  rht_sign_mask=mask)
    sc, se = P.rht32_s2f6_quantize(y, mask)
    assert torch.equal(c, sc) and torch.equal(e, se)


@pytest.mark.parametrize("counts,N,K,gather_rows", [([70, 300, 129, 1], 288, 96, None),
                                                    ([5, 0, 600, 128], 352, 160, 700),
                                                    ([300, 40], 320, 32, None),
                                                    ([129, 257], 64, 224, 300),
                                                    ([200, 3], 96, 320, None)])
def test_gemm_fwd_edge_shapes(P, I, counts, N, K, gather_rows):
    """Weight rows per expert that are not a multiple of 256 (a partial last weight tile: 32, 96
    or 64 of its rows exist) and contractions that are not a multiple of 64 (the last k-stage
    holds 32 or 96 values; rows of scales then sit at 2-byte alignment), with short slot units.
    All four epilogues where the shape allows them (SwiGLU needs F = N / 2 a multiple of 32)."""
    d = _moe_small(P, I, counts, N, K, gather_rows, seed=85)
    y = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_F32, gather=d["ggather"])
    ref = O.gemm_nvfp4_grouped(d["rxq"], d["rwq"], d["offsets"], N, K, gather=d["gather"])
    assert rel_fro(npy(y), ref) <= 1e-5          # exact products, fp32 accumulation
    yb = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_BF16, gather=d["ggather"])
    assert torch.equal(yb, y.to(torch.bfloat16))
    mask = I.sign_mask(3)
    c, e = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_RHT32_S2F6, gather=d["ggather"],
                                  rht_sign_mask=mask)
    sc, se = P.rht32_s2f6_quantize(y, mask)
    assert torch.equal(c, sc) and torch.equal(e, se)
    if N % 64 == 0:
        a, h13 = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_SWIGLU, gather=d["ggather"],
                                        save_h13=True)
        assert torch.equal(h13, y.to(torch.bfloat16))
        assert rel_fro(npy(a.float()), O.swiglu(ref, N // 2)) <= 2e-3
    else:
        with pytest.raises(RuntimeError):
            P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_SWIGLU, gather=d["ggather"])


@pytest.mark.parametrize("sr", [False, True])
def test_mxfp8_quantize_rows_and_cols(P, I, sr):
    dy = I.normal((600, 512), 1e-3, 31)
    rnd = P.SR if sr else P.RNE
    q, e, _ = P.mxfp8_quantize(dy.to(DEV), P.ROWWISE, rounding=rnd, seed=3, rng_stream=9)
    rq, re = O.mxfp8_quantize_rows(dy, sr=sr, seed=3, stream=9)
    assert np.array_equal(npy(q), rq) and np.array_equal(npy(e), re)
    offsets = np.array([0, 100, 100, 433, 600], np.int64)
    t, te, _ = P.mxfp8_quantize(dy.to(DEV), P.COLWISE, offsets=torch.as_tensor(offsets, device=DEV), rounding=rnd,
                                seed=3, rng_stream=9)
    rt, rte = O.mxfp8_quantize_cols(dy, offsets=offsets, sr=sr, seed=3, stream=9)
    Pt = rt.shape[1]
    assert np.array_equal(npy(t)[:, :Pt], rt) and np.array_equal(npy(te)[:, :Pt // 32], rte)


# ------------------------------------------------------------------------------------------
# RHT32 + S2F6
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rht32_s2f6(P, I, dtype):
    x = I.student_t((333, 1024), 3, 1.0, 41).to(dtype)
    x[0, :32] = 0
    mask = I.sign_mask(3)
    c, e = P.rht32_s2f6_quantize(x.to(DEV), mask)
    rc, re = O.rht32_s2f6_quantize(x.float().numpy(), mask)
    assert np.array_equal(npy(c), rc) and np.array_equal(npy(e), re)
    xh = decode_s2f6_rows(npy(c), npy(e), mask)
    assert rel_fro(xh, x.float().numpy()) < 0.02
    # per 32-chunk: the transform is orthogonal up to its factor 32, so the decoded chunk lies within
    # half a code step, 2^(e-127)/128, of the input in the 2-norm (up to the fp32 transform's rounding)
    xr = x.float().numpy().astype(np.float64)
    R, Cc = xr.shape
    ee = npy(e).astype(np.float64)
    err = np.sqrt(((xh - xr) ** 2).reshape(R, Cc // 32, 32).sum(-1))
    nrm = np.sqrt((xr ** 2).reshape(R, Cc // 32, 32).sum(-1))
    assert np.all(err <= 2.0 ** (ee - 127) / 128 * (1 + 1e-6) + 1e-6 * nrm)


# ------------------------------------------------------------------------------------------
# Grouped GEMMs
# ------------------------------------------------------------------------------------------

def _moe_small(P, I, counts, N, K, gather_rows=None, seed=50):
    rng = np.random.default_rng(seed)
    G = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    T = gather_rows or M
    x = I.student_t((T, K), 4, 1.0, seed + 1)
    w = I.normal((G * N, K), 0.02, seed + 2)
    gather = rng.integers(0, T, M).astype(np.int32) if gather_rows else None
    rpo = N // 2 if N % 64 == 0 else N
    xq = P.nvfp4_quantize(x.to(DEV), P.NVFP4_ACT)
    wq = P.nvfp4_quantize(w.to(DEV), P.NVFP4_WEIGHT, rows_per_outer=rpo)
    # the oracle's own quantization of the same inputs
    rxq = O.nvfp4_quantize(x, 1, True)
    rwq = O.nvfp4_quantize(w, rpo, False)
    return dict(offsets=offsets, M=M, x=x, w=w, gather=gather, xq=xq, wq=wq, rxq=rxq, rwq=rwq,
                goff=torch.as_tensor(offsets, device=DEV),
                ggather=None if gather is None else torch.as_tensor(gather, device=DEV))


@pytest.mark.parametrize("counts,N,K,gather_rows", [([300], 256, 192, None), ([10, 0, 300, 77], 512, 256, 200),
                                                    ([256, 513], 256, 1024, 1000)])
def test_gemm_fwd_f32_bf16(P, I, counts, N, K, gather_rows):
    d = _moe_small(P, I, counts, N, K, gather_rows)
    y = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_F32, gather=d["ggather"])
    ref = O.gemm_nvfp4_grouped(d["rxq"], d["rwq"], d["offsets"], N, K, gather=d["gather"])
    assert rel_fro(npy(y), ref) <= 2e-3
    assert rel_fro(npy(y), ref) <= 1e-5          # exact products, fp32 accumulation
    yb = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_BF16, gather=d["ggather"])
    assert torch.equal(yb, y.to(torch.bfloat16))


def test_gemm_fwd_swiglu(P, I):
    counts, F, K = [130, 0, 301], 128, 256
    d = _moe_small(P, I, counts, 2 * F, K, gather_rows=250, seed=60)
    a, h13 = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], 2 * F, P.EPI_SWIGLU, gather=d["ggather"],
                                    save_h13=True)
    y = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], 2 * F, P.EPI_F32, gather=d["ggather"])
    ref = O.gemm_nvfp4_grouped(d["rxq"], d["rwq"], d["offsets"], 2 * F, K, gather=d["gather"])
    aref = O.swiglu(ref, F)
    assert rel_fro(npy(a.float()), aref) <= 2e-3
    assert torch.equal(h13, y.to(torch.bfloat16))


def test_gemm_fwd_rht_epilogue_bit_exact(P, I):
    counts, N, K = [70, 256, 3], 512, 192
    d = _moe_small(P, I, counts, N, K, gather_rows=120, seed=70)
    mask = I.sign_mask(3)
    y = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_F32, gather=d["ggather"])
    c, e = P.moe_grouped_gemm_fwd(d["xq"], d["wq"], d["goff"], d["M"], N, P.EPI_RHT32_S2F6, gather=d["ggather"],
                                  rht_sign_mask=mask)
    # the fused epilogue equals the library's standalone transform of the same fp32 rows (which
    # is bit-exact with the oracle in test_rht32_s2f6), and decodes to the oracle's product
    sc, se = P.rht32_s2f6_quantize(y, mask)
    assert torch.equal(c, sc) and torch.equal(e, se)
    ref = O.gemm_nvfp4_grouped(d["rxq"], d["rwq"], d["offsets"], N, K, gather=d["gather"])
    # per 32-chunk: the S2F6 bound ||x_hat - x||_2 <= 2^(e-127)/128 around the fp32 result, which
    # is itself within the GEMM tolerance of the oracle's fp64 product
    M = d["M"]
    dec = decode_s2f6_rows(npy(c), npy(e), mask)
    ee = npy(e).astype(np.float64)
    err = np.sqrt(((dec - ref) ** 2).reshape(M, N // 32, 32).sum(-1))
    nrm = np.sqrt((ref ** 2).reshape(M, N // 32, 32).sum(-1))
    assert np.all(err <= 2.0 ** (ee - 127) / 128 * (1 + 1e-6) + 2e-3 * nrm)
    assert rel_fro(npy(y), ref) <= 1e-5


@pytest.mark.parametrize("counts,N,K", [([40, 0, 333, 227], 256, 128), ([1, 64, 65, 0, 130], 288, 96),
                                         ([300, 5, 700], 1024, 64), ([0, 129], 7168, 32)])
def test_gemm_bwd_dy_both_ways_in_one_read(P, I, counts, N, K):
    """With both gradients (E4M3, dY by RNE) the call quantizes dY row-wise and column-wise from
    one read of dY. Its workspace parts equal those of the one-gradient calls, which quantize each
    orientation separately, byte for byte (the parts the one-gradient call does not write aside):
    N of 288 (an odd k-block count and a partial last column tile), groups of 1, 64, 65 and 129
    slots (a padded unit of padding only), empty groups, and 7168 columns."""
    d = _moe_small(P, I, counts, N, K, seed=90)
    M, G = d["M"], len(counts)
    dy = I.normal((M, N), 1e-3, 91).to(DEV)
    size = P.moe_grouped_gemm_bwd_workspace_size(M, G, N, K, 3)
    views = {}
    for flags in (3, 1, 2):
        ws = torch.zeros((size,), dtype=torch.uint8, device=DEV)
        P.moe_grouped_gemm_bwd(dy, d["xq"], d["wq"], d["goff"], M, N, flags=flags, seed=3, workspace=ws)
        views[flags] = P.bwd_workspace_views(ws, M, G, N, K)
    torch.cuda.synchronize()
    for name, flags in (("dq", 1), ("de", 1), ("dt", 2), ("dte", 2)):
        assert torch.equal(views[3][name], views[flags][name]), name


@pytest.mark.parametrize("counts,N,K,gather_rows", [([40, 0, 333, 227], 256, 128, 400), ([1, 64, 65, 0, 130], 320, 96, None)])
def test_gemm_bwd_swiglu_equals_swiglu_then_bwd(P, I, counts, N, K, gather_rows):
    """moe_grouped_gemm_bwd_swiglu (dh13 formed inside dY's quantization, never written) gives the
    gradients and workspace parts of swiglu_bwd followed by moe_grouped_gemm_bwd, bit for bit; F
    of 160 leaves the last 256-feature tile partial."""
    d = _moe_small(P, I, counts, N, K, gather_rows=gather_rows, seed=95)
    M, G, F = d["M"], len(counts), N // 2
    da = I.normal((M, F), 1e-3, 96, DEV, dtype=torch.float32)
    h13 = I.student_t((M, N), 4, 1.0, 97, DEV)
    size = P.moe_grouped_gemm_bwd_workspace_size(M, G, N, K, 3)
    ws1 = torch.zeros((size,), dtype=torch.uint8, device=DEV)
    ws2 = torch.zeros((size,), dtype=torch.uint8, device=DEV)
    dh13 = P.swiglu_bwd(da, h13)
    dx1, dw1, _ = P.moe_grouped_gemm_bwd(dh13, d["xq"], d["wq"], d["goff"], M, N, gather=d["ggather"], seed=4,
                                         workspace=ws1)
    dx2, dw2, _ = P.moe_grouped_gemm_bwd_swiglu(da, h13, d["xq"], d["wq"], d["goff"], M, N, gather=d["ggather"],
                                                seed=4, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2) and torch.equal(dw1, dw2)
    v1, v2 = P.bwd_workspace_views(ws1, M, G, N, K), P.bwd_workspace_views(ws2, M, G, N, K)
    for name in ("dq", "de", "dt", "dte", "wt", "wte", "xt", "xte"):
        assert torch.equal(v1[name], v2[name]), name


@pytest.mark.parametrize("sr", [False, True])
def test_gemm_bwd_intermediates_and_gradients(P, I, sr):
    """Both gradients in one call: dY's row-wise and column-wise MXFP8 (RNE, or SR on streams 6
    and 7), W^T and A^T from the SR requant, and the two gradients."""
    counts, N, K = [40, 0, 333, 227], 256, 512
    d = _moe_small(P, I, counts, N, K, gather_rows=400, seed=80)
    M, G = d["M"], len(counts)
    dy = I.normal((M, N), 1e-3, 81)
    da, db, ws = P.moe_grouped_gemm_bwd(dy.to(DEV), d["xq"], d["wq"], d["goff"], M, N, gather=d["ggather"],
                                        dy_rounding=P.SR if sr else P.RNE, seed=9, rng_stream_a=4, rng_stream_b=1,
                                        rng_stream_dy=6)
    v = P.bwd_workspace_views(ws, M, G, N, K)
    # The library pads each group to 64 slots and keeps the code parts blocked; the oracle pads
    # to 32 and is row-major. E8M0 parts are k-block-major; the row-wise dY codes and scales sit
    # at padded slot rows / columns.
    off = np.asarray(d["offsets"], dtype=np.int64)
    cnt = np.diff(off)
    po32 = np.concatenate([[0], np.cumsum((cnt + 31) // 32 * 32)])
    po = np.concatenate([[0], np.cumsum((cnt + 63) // 64 * 64)])
    assert np.array_equal(npy(v["po"]), po)
    Pb = v["de"].shape[1]
    grp = np.searchsorted(off, np.arange(M), side="right") - 1
    pcol = po[grp] + np.arange(M) - off[grp]
    rq, re = O.mxfp8_quantize_rows(dy, sr=sr, seed=9, stream=6)
    assert np.array_equal(unblock(npy(v["dq"]), Pb, N)[pcol], rq)
    assert np.array_equal(npy(v["de"])[:, pcol].T, re)
    rwt, rwte = O.requant_transpose_sr(d["rwq"], seed=9, stream=1)
    assert np.array_equal(unblock(npy(v["wt"]), K, G * N), rwt) and np.array_equal(npy(v["wte"]).T, rwte)
    rt, rte = O.mxfp8_quantize_cols(dy, offsets=d["offsets"], sr=sr, seed=9, stream=7)
    rxt, rxte = O.requant_transpose_sr(d["rxq"], gather=d["gather"], offsets=d["offsets"], seed=9, stream=4)
    for name, ref, ref_e in (("dt", rt, rte), ("xt", rxt, rxte)):
        got = unblock(npy(v[name]), ref.shape[0], Pb)
        got_e = npy(v[name + "e"]).T
        for g in range(G):
            n32 = po32[g + 1] - po32[g]
            a, a32 = po[g], po32[g]
            assert np.array_equal(got[:, a:a + n32], ref[:, a32:a32 + n32]), (name, g)
            assert np.array_equal(got_e[:, a // 32:(a + n32) // 32], ref_e[:, a32 // 32:(a32 + n32) // 32]), (name, g)
            assert np.all(got[:, a + n32:po[g + 1]] == 0), (name, g)   # a block of padding only
    da_ref = O.gemm_mxfp8_dgrad(rq, re, rwt, rwte, d["offsets"], N, K)
    db_ref = O.gemm_mxfp8_wgrad(rt, rte, rxt, rxte, d["offsets"], N, K)
    assert rel_fro(npy(da), da_ref) <= 2e-3
    assert rel_fro(npy(db), db_ref) <= 2e-3
    assert np.all(npy(db)[N:2 * N] == 0)          # the empty expert gets a zero gradient


@pytest.mark.parametrize("fp4", [False, True])
def test_gemm_bwd_many_small_groups(P, I, fp4):
    """96 experts with 0..40 slots each (many empty, most smaller than one 64- or 128-slot padded
    stage): both gradients against the oracle, whose operands are its own quantizations."""
    rng = np.random.default_rng(97)
    counts = [int(c) if rng.random() > 0.25 else 0 for c in rng.integers(1, 41, 96)]
    N, K = 256, 256
    d = _moe_small(P, I, counts, N, K, gather_rows=900, seed=98)
    M = d["M"]
    dy = I.normal((M, N), 1e-3, 99)
    flags = P.BWD_DGRAD | P.BWD_WGRAD | (P.BWD_FP4 if fp4 else 0)
    da, db, _ = P.moe_grouped_gemm_bwd(dy.to(DEV), d["xq"], d["wq"], d["goff"], M, N, flags=flags,
                                       gather=d["ggather"], seed=13, rng_stream_a=2, rng_stream_b=3, rng_stream_dy=4)
    target = O.TARGET_E2M1 if fp4 else O.TARGET_E4M3
    rq, re = O.mxfp8_quantize_rows(dy, target=target)
    rwt, rwte = O.requant_transpose_sr(d["rwq"], target=target, seed=13, stream=3)
    rt, rte = O.mxfp8_quantize_cols(dy, offsets=d["offsets"], target=target)
    rxt, rxte = O.requant_transpose_sr(d["rxq"], gather=d["gather"], offsets=d["offsets"], target=target, seed=13,
                                       stream=2)
    assert rel_fro(npy(da), O.gemm_mxfp8_dgrad(rq, re, rwt, rwte, d["offsets"], N, K, target=target)) <= 2e-3
    assert rel_fro(npy(db), O.gemm_mxfp8_wgrad(rt, rte, rxt, rxte, d["offsets"], N, K, target=target)) <= 2e-3
    off = d["offsets"]
    for g in range(len(counts)):
        if off[g + 1] == off[g]:
            assert np.all(npy(db)[g * N:(g + 1) * N] == 0)


@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("counts,N,K,gather_rows", [([40, 0, 333, 227], 288, 96, 400), ([129, 70], 96, 352, None)])
def test_gemm_bwd_edge_shapes(P, I, counts, N, K, gather_rows, fp4):
    """N and K that are not multiples of 256 (nor N of 64): dgrad contracts over N rounded up to a
    whole stage (W^T re-quantized per expert, each expert's columns padded with zero codes; dY's
    last block column half or partly empty), and the last row / column tiles of dX and dW are
    partial. Both gradients against the oracle; the padded W^T bit-exact with the oracle's."""
    d = _moe_small(P, I, counts, N, K, gather_rows, seed=87)
    M, G = d["M"], len(counts)
    dy = I.normal((M, N), 1e-3, 88)
    flags = P.BWD_DGRAD | P.BWD_WGRAD | (P.BWD_FP4 if fp4 else 0)
    da, db, ws = P.moe_grouped_gemm_bwd(dy.to(DEV), d["xq"], d["wq"], d["goff"], M, N, flags=flags,
                                        gather=d["ggather"], seed=13, rng_stream_a=2, rng_stream_b=3, rng_stream_dy=4)
    target = O.TARGET_E2M1 if fp4 else O.TARGET_E4M3
    rq, re = O.mxfp8_quantize_rows(dy, target=target)
    rwt, rwte = O.requant_transpose_sr(d["rwq"], target=target, seed=13, stream=3)
    rt, rte = O.mxfp8_quantize_cols(dy, offsets=d["offsets"], target=target)
    rxt, rxte = O.requant_transpose_sr(d["rxq"], gather=d["gather"], offsets=d["offsets"], target=target, seed=13,
                                       stream=2)
    assert rel_fro(npy(da), O.gemm_mxfp8_dgrad(rq, re, rwt, rwte, d["offsets"], N, K, target=target)) <= 2e-3
    assert rel_fro(npy(db), O.gemm_mxfp8_wgrad(rt, rte, rxt, rxte, d["offsets"], N, K, target=target)) <= 2e-3
    if not fp4:
        Nk = (N + 63) // 64 * 64
        v = P.bwd_workspace_views(ws, M, G, N, K)
        wt = unblock(npy(v["wt"]), K, G * Nk)
        wte = npy(v["wte"]).T
        for g in range(G):
            assert np.array_equal(wt[:, g * Nk:g * Nk + N], rwt[:, g * N:(g + 1) * N]), g
            assert np.all(wt[:, g * Nk + N:(g + 1) * Nk] == 0), g
            assert np.array_equal(wte[:, g * Nk // 32:(g * Nk + N) // 32], rwte[:, g * N // 32:(g + 1) * N // 32]), g


def test_gemm_bwd_sr_gradients_deterministic(P, I):
    counts, N, K = [200, 56], 256, 256
    d = _moe_small(P, I, counts, N, K, seed=90)
    dy = I.normal((d["M"], N), 1e-3, 91).to(DEV)
    a1 = P.moe_grouped_gemm_bwd(dy, d["xq"], d["wq"], d["goff"], d["M"], N, dy_rounding=P.SR, seed=3)
    a2 = P.moe_grouped_gemm_bwd(dy, d["xq"], d["wq"], d["goff"], d["M"], N, dy_rounding=P.SR, seed=3)
    assert torch.equal(a1[0], a2[0]) and torch.equal(a1[1], a2[1])


def test_swiglu_bwd(P, I):
    M, F = 300, 256
    da = I.normal((M, F), 1.0, 95, dtype=torch.float32)
    h13 = I.normal((M, 2 * F), 2.0, 96)
    g = P.swiglu_bwd(da.to(DEV), h13.to(DEV))
    ref = O.swiglu_bwd(da.numpy(), h13, F)
    assert rel_fro(npy(g.float()), ref) <= 2e-3


# ------------------------------------------------------------------------------------------
# Routing
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1000, 32, 8), (257, 48, 8), (3, 8, 8), (50, 384, 8)])
def test_route_topk(P, I, T, E, k):
    logits = torch.randn((T, E), generator=torch.Generator().manual_seed(T + E), dtype=torch.float32)
    r = P.moe_route_topk(logits.to(DEV), k)
    ref = O.route_topk(logits.numpy(), k)
    for key in ("ids", "offsets", "gather", "slot_of"):
        assert np.array_equal(npy(r[key]), ref[key]), key
    assert np.allclose(npy(r["gates"]), ref["gates"], rtol=1e-5, atol=1e-7)


def test_gemm_bwd_odd_stage_counts_and_half_stages(P, I):
    """wgrad groups padded to whole 64-slot stages, with odd and even stage counts and mostly
    padding in the last stage (150 -> 192 slots: 3 stages, 22 real slots in the last; 1 -> 64: 1
    stage of 1 real slot; 95 -> 128: 2 stages; 33 -> 64: 1 stage)."""
    counts, N, K = [150, 1, 95, 33], 256, 256
    d = _moe_small(P, I, counts, N, K, gather_rows=300, seed=95)
    M = d["M"]
    dy = I.normal((M, N), 1e-3, 96)
    da, db, _ = P.moe_grouped_gemm_bwd(dy.to(DEV), d["xq"], d["wq"], d["goff"], M, N, gather=d["ggather"],
                                       seed=4, rng_stream_a=2, rng_stream_b=3, rng_stream_dy=5)
    rq, re = O.mxfp8_quantize_rows(dy)
    rwt, rwte = O.requant_transpose_sr(d["rwq"], seed=4, stream=3)
    rt, rte = O.mxfp8_quantize_cols(dy, offsets=d["offsets"], stream=6)
    rxt, rxte = O.requant_transpose_sr(d["rxq"], gather=d["gather"], offsets=d["offsets"], seed=4, stream=2)
    assert rel_fro(npy(da), O.gemm_mxfp8_dgrad(rq, re, rwt, rwte, d["offsets"], N, K)) <= 2e-3
    assert rel_fro(npy(db), O.gemm_mxfp8_wgrad(rt, rte, rxt, rxte, d["offsets"], N, K)) <= 2e-3


def test_empty_layer_gemms(P, I):
    """A layer with no routed slots (M = 0, three experts): the forward GEMMs return empty outputs
    and the backward gives an empty dgrad and zero weight gradients, in MXFP8 and in FP4."""
    G, N, K = 3, 256, 256
    offsets = torch.zeros(G + 1, dtype=torch.int64, device=DEV)
    w = I.normal((G * N, K), 0.02, 5).to(DEV)
    wq = P.nvfp4_quantize(w, P.NVFP4_WEIGHT, N // 2)
    x = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    xq = P.nvfp4_quantize(x, P.NVFP4_ACT)
    assert P.moe_grouped_gemm_fwd(xq, wq, offsets, 0, N, P.EPI_F32).shape == (0, N)
    a, h13 = P.moe_grouped_gemm_fwd(xq, wq, offsets, 0, N, P.EPI_SWIGLU, save_h13=True)
    assert a.shape == (0, N // 2) and h13.shape == (0, N)
    assert P.moe_grouped_gemm_fwd_mxfp8(x, w, offsets, 0, N, P.EPI_F32).shape == (0, N)
    dy = torch.empty((0, N), dtype=torch.bfloat16, device=DEV)
    for flags in (P.BWD_DGRAD | P.BWD_WGRAD, P.BWD_DGRAD | P.BWD_WGRAD | P.BWD_FP4):
        db = torch.full((G * N, K), float("nan"), dtype=torch.float32, device=DEV)
        da, db, _ = P.moe_grouped_gemm_bwd(dy, xq, wq, offsets, 0, N, flags=flags, db=db)
        torch.cuda.synchronize()
        assert da.shape == (0, K)
        assert torch.count_nonzero(db).item() == 0     # every expert's gradient written as zero


def test_binding_rejects_mismatched_tensors(P, I):
    """The C ABI takes sizes as integers; the binding refuses tensors whose shape or dtype
    disagrees with them (PmnError), before anything is launched."""
    G, N, K, M = 2, 256, 256, 64
    x = I.normal((M, K), 1.0, 90).to(DEV)
    w = I.normal((G * N, K), 0.02, 91).to(DEV)
    xq = P.nvfp4_quantize(x, P.NVFP4_ACT)
    wq = P.nvfp4_quantize(w, P.NVFP4_WEIGHT, rows_per_outer=N)
    off = torch.tensor([0, 30, M], dtype=torch.int64, device=DEV)
    bad = [
        lambda: P.moe_grouped_gemm_fwd(xq, wq, off, M, 2 * N),                                   # wq rows != G*N
        lambda: P.moe_grouped_gemm_fwd(xq, P.nvfp4_quantize(w[:, :128].contiguous(), P.NVFP4_WEIGHT, N),
                                       off, M, N),                                               # K differs
        lambda: P.moe_grouped_gemm_fwd(xq, wq, off, M, N, out=torch.empty((M, N - 1), device=DEV)),
        lambda: P.moe_grouped_gemm_fwd(xq, wq, off, M, N, gather=torch.zeros(M, dtype=torch.int64, device=DEV)),
        lambda: P.moe_grouped_gemm_fwd(xq, wq, off.to(torch.int32), M, N),
        lambda: P.moe_grouped_gemm_fwd(xq, wq, off, M, N, P.EPI_RHT32_S2F6,
                                       out_e8m0=torch.empty((M, N // 16), dtype=torch.uint8, device=DEV)),
        lambda: P.moe_grouped_gemm_bwd(torch.zeros((M, N + 32), dtype=torch.bfloat16, device=DEV), xq, wq, off, M, N),
        lambda: P.moe_grouped_gemm_bwd(torch.zeros((M, N), dtype=torch.bfloat16, device=DEV), xq, wq, off, M, N,
                                       db=torch.empty((G * N, K - 1), device=DEV)),
        lambda: P.requant_transpose_sr_mxfp8(xq, out=torch.empty((K, 32), dtype=torch.uint8, device=DEV)),
        lambda: P.swiglu_bwd(torch.zeros((M, N), device=DEV), torch.zeros((M, N), dtype=torch.bfloat16, device=DEV)),
        lambda: P.moe_combine_s2f6(torch.zeros((M, N), dtype=torch.int8, device=DEV),
                                   torch.zeros((M, N // 16), dtype=torch.uint8, device=DEV), 0,
                                   torch.zeros(M, dtype=torch.int32, device=DEV), torch.ones((M, 1), device=DEV)),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(P.PmnError):
            call()
    # a well-formed call still runs
    y = P.moe_grouped_gemm_fwd(xq, wq, off, M, N)
    torch.cuda.synchronize()
    assert y.shape == (M, N)
