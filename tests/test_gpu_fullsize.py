"""Parity at the full size of the 48-expert layer step, in the launch configuration the bench times.

The layer is built as the bench builds it: 65536 routed slots with Zipf(1.1) loads over 48
experts, hidden 7168, FFN 2048, weights N(0, 0.02) quantized per (expert, matrix), activations
Student-t(4) quantized per token with 4/6. The oracle cannot redo the whole layer in seconds, so
outputs are sampled. Every sampled value is recomputed by the oracle from the original bf16
inputs (drawn by the seeded generators): the oracle quantizes the sampled token rows and the
sampled experts' matrices itself, requantizes its own windows and takes fp64 dot products. No
tensor produced by the HIP library is ever an input of the oracle. Activation quantization is
per token row and weight quantization per (expert, matrix), so quantizing only the sampled rows or
experts gives the same codes as quantizing everything; the requantization keys its random bits by
the element's index in the whole source matrix, so the oracle's windows are taken from full-size
arrays in which only the sampled rows are filled. Samples include the first and last slot of
ragged groups and the first and last output column. The bar is the GEMM tolerance, relative
Frobenius error <= 2e-3 over the samples, and for bf16 outputs one bf16 rounding (2^-8 of the
value) per element.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decoders import decode_s2f6_rows
from fullsize_helpers import oracle_quant_rows, sample_slots as _sample_slots

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def npy(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel_fro(got, ref):
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)


def host_bf16(t):
    torch.cuda.synchronize()
    return t.detach().cpu()


@pytest.fixture(scope="module")
def layer():
    import precision_moe_numerics_amd as P
    from precision_moe_numerics_amd import inputs as I
    sh = I.EP48
    E, H, F = sh.experts, sh.hidden, sh.ffn
    counts = I.moe_loads(sh)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    x = I.moe_activations(sh, DEV)
    w13, w2 = I.moe_weights(sh, DEV)
    d = dict(P=P, I=I, E=E, H=H, F=F, M=M, counts=np.asarray(counts), offsets=offsets, x=x, w13=w13, w2=w2,
             goff=torch.as_tensor(offsets, device=DEV), seed=sh.seeds["sr"], mask=I.sign_mask(sh.seeds["rht"]))
    d["xq"] = P.nvfp4_quantize(x, P.NVFP4_ACT)
    d["w13q"] = P.nvfp4_quantize(w13.view(E * 2 * F, H), P.NVFP4_WEIGHT, F)
    d["w2q"] = P.nvfp4_quantize(w2.view(E * H, F), P.NVFP4_WEIGHT, H)
    torch.cuda.synchronize()
    return d


def test_ep48_forward_w13_swiglu_sampled(layer):
    P, L = layer["P"], layer
    M, H, F, E = L["M"], L["H"], L["F"], L["E"]
    a, h13 = P.moe_grouped_gemm_fwd(L["xq"], L["w13q"], L["goff"], M, 2 * F, P.EPI_SWIGLU, save_h13=True)
    hg, ag = npy(h13.float()), npy(a.float())
    rng = np.random.default_rng(11)
    fcols = np.concatenate([[0, F - 1], rng.integers(0, F, 6)])
    got_h1, got_h3, ref_h1, ref_h3, got_a = [], [], [], [], []
    for g in (0, 1, 23, E - 1):
        slots = _sample_slots(L["offsets"], [g], 6, rng)
        xq = O.nvfp4_quantize(host_bf16(L["x"][torch.as_tensor(slots, device=DEV)]), 1, True)
        wq = O.nvfp4_quantize(host_bf16(L["w13"][g]), F, False)
        n = len(slots)
        rows = np.repeat(np.arange(n), len(fcols))
        cols = np.tile(fcols, n)
        ref_h1.append(O.gemm_nvfp4_elems(xq, wq, [0, n], 2 * F, H, rows, cols))
        ref_h3.append(O.gemm_nvfp4_elems(xq, wq, [0, n], 2 * F, H, rows, cols + F))
        got_h1.append(hg[slots[rows], cols])
        got_h3.append(hg[slots[rows], cols + F])
        got_a.append(ag[slots[rows], cols])
    h1, h3 = np.concatenate(ref_h1), np.concatenate(ref_h3)
    g1, g3, ga = np.concatenate(got_h1), np.concatenate(got_h3), np.concatenate(got_a)
    assert rel_fro(g1, h1) <= 2e-3 and rel_fro(g3, h3) <= 2e-3
    # bf16 outputs: each within one bf16 rounding of the fp64 value
    assert np.all(np.abs(g1 - h1) <= 2.0 ** -8 * np.abs(h1) + 1e-30)
    assert np.all(np.abs(g3 - h3) <= 2.0 ** -8 * np.abs(h3) + 1e-30)
    # A = silu(h1) h3, also bf16: within one bf16 rounding of the fp64 value
    a_ref = h1 / (1.0 + np.exp(-h1)) * h3
    assert np.all(np.abs(ga - a_ref) <= 2.0 ** -8 * np.abs(a_ref) + 1e-30)


def test_ep48_forward_w2_rht_s2f6_sampled(layer):
    """The w2 GEMM on a synthetic A (Student-t(4) x 0.05, the scale of SwiGLU outputs here): F32
    rows against the oracle; the fused RHT32 + S2F6 codes bit-exact with the library's standalone
    transform of the same F32 rows (whose parity with the oracle is tested bit for bit elsewhere)
    and, decoded, within the S2F6 error bound of the oracle's fp64 rows."""
    P, I, L = layer["P"], layer["I"], layer
    M, H, F, E = L["M"], L["H"], L["F"], L["E"]
    A = I.student_t((M, F), 4, 0.05, 611, DEV)
    aq = P.nvfp4_quantize(A, P.NVFP4_ACT)
    y = P.moe_grouped_gemm_fwd(aq, L["w2q"], L["goff"], M, H, P.EPI_F32)
    c, e = P.moe_grouped_gemm_fwd(aq, L["w2q"], L["goff"], M, H, P.EPI_RHT32_S2F6, rht_sign_mask=L["mask"])
    sc, se = P.rht32_s2f6_quantize(y, L["mask"])
    assert torch.equal(c, sc) and torch.equal(e, se)
    rng = np.random.default_rng(12)
    got, ref = [], []
    for g in (0, 7, E - 1):
        slots = _sample_slots(L["offsets"], [g], 3, rng)
        xq = O.nvfp4_quantize(host_bf16(A[torch.as_tensor(slots, device=DEV)]), 1, True)
        wq = O.nvfp4_quantize(host_bf16(L["w2"][g]), H, False)
        n = len(slots)
        rows = np.repeat(np.arange(n), H)
        cols = np.tile(np.arange(H), n)
        yr = O.gemm_nvfp4_elems(xq, wq, [0, n], H, F, rows, cols).reshape(n, H)
        ref.append(yr)
        got.append(npy(y[torch.as_tensor(slots, device=DEV)]))
        dec = decode_s2f6_rows(npy(c[torch.as_tensor(slots, device=DEV)]), npy(e[torch.as_tensor(slots, device=DEV)]),
                               L["mask"])
        # per 32-chunk: S2F6 error bound 2^(e-127)/128 (2-norm) plus the GEMM tolerance
        ee = npy(e[torch.as_tensor(slots, device=DEV)]).astype(np.float64)
        err = np.sqrt(((dec - yr) ** 2).reshape(n, H // 32, 32).sum(-1))
        nrm = np.sqrt((yr ** 2).reshape(n, H // 32, 32).sum(-1))
        assert np.all(err <= 2.0 ** (ee - 127) / 128 * (1 + 1e-6) + 2e-3 * nrm)
    assert rel_fro(np.concatenate(got), np.concatenate(ref)) <= 2e-3


def test_ep48_backward_w13_sampled(layer):
    P, I, L = layer["P"], layer["I"], layer
    M, H, F, E = L["M"], L["H"], L["F"], L["E"]
    N, K = 2 * F, H
    dy = I.normal((M, N), 1e-3, 602, DEV)
    da, db, _ = P.moe_grouped_gemm_bwd(dy, L["xq"], L["w13q"], L["goff"], M, N, seed=L["seed"], rng_stream_a=4,
                                       rng_stream_b=1, rng_stream_dy=8)
    off, seed = L["offsets"], L["seed"]
    dyh = dy.cpu()
    rng = np.random.default_rng(13)
    # dgrad: da[s, k] = sum_n dq[s, n] wt[k, g N + n]; W^T of expert g is the oracle's window of
    # its own quantization of W13_g (rows g N .. g N + N - 1 of the [E N x K] weight matrix)
    got, ref = [], []
    for g in (0, E - 1):
        wh = oracle_quant_rows(host_bf16(L["w13"][g]), E * N, g * N, F, False)
        wt, wte = O.requant_window(wh, g * N, N, seed=seed, stream=1)
        for s in _sample_slots(off, [g], 4, rng):
            dq, de = O.mxfp8_quantize_rows(dyh[int(s):int(s) + 1])
            for k in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dq, de, wt, wte, 0, k, 0, N))
                got.append(float(da[int(s), k]))
    assert rel_fro(got, ref) <= 2e-3
    # wgrad: db[g N + n, k] = sum over the group's padded slots of dt[n, s] xt[k, s]
    got, ref = [], []
    for g in (E - 1, E - 2, 20):
        a, b = int(off[g]), int(off[g + 1])
        dt, dte = O.mxfp8_quantize_cols(dyh[a:b])
        xh = oracle_quant_rows(host_bf16(L["x"][a:b]), M, a, 1, True)
        xt, xte = O.requant_window(xh, a, b - a, seed=seed, stream=4)
        Pg = dt.shape[1]
        for n in (0, N - 1, int(rng.integers(0, N))):
            for k in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dt, dte, xt, xte, n, k, 0, Pg))
                got.append(float(db[g * N + n, k]))
    assert rel_fro(got, ref) <= 2e-3


@pytest.mark.parametrize("fp4", [False, True], ids=["mxfp8", "fp4"])
def test_ep48_backward_w2_sampled(layer, fp4):
    """The w2 backward as the bench runs it: dY [65536 x 7168] N(0, 1e-3) (the bench's gradient),
    the saved NVFP4 A of a synthetic Student-t(4) x 0.05 activation, contraction N = 7168 in dgrad,
    RNG streams a = 5 (A^T), b = 3 (W2^T), dY = 6, in MXFP8 and in the FP4 variant. dA samples
    use the oracle's own W2_g^T windows (from its quantization of W2_g in a full-size array); dW2
    samples use its A^T windows and column-wise dY of the sampled group (sampled feature columns,
    each column quantizes on its own). Samples take in the first and last slot of the largest and
    the smallest group and the first and last column of both gradients."""
    P, I, L = layer["P"], layer["I"], layer
    M, H, F, E = L["M"], L["H"], L["F"], L["E"]
    N, K = H, F
    tgt = O.TARGET_E2M1 if fp4 else O.TARGET_E4M3
    A = I.student_t((M, F), 4, 0.05, 611, DEV)
    aq = P.nvfp4_quantize(A, P.NVFP4_ACT)
    dy = I.moe_grad(I.EP48, M, DEV)
    flags = P.BWD_DGRAD | P.BWD_WGRAD | (P.BWD_FP4 if fp4 else 0)
    da, db, _ = P.moe_grouped_gemm_bwd(dy, aq, L["w2q"], L["goff"], M, N, flags=flags, seed=L["seed"],
                                       rng_stream_a=5, rng_stream_b=3, rng_stream_dy=6)
    off, seed = L["offsets"], L["seed"]
    rng = np.random.default_rng(14 + fp4)

    def at(t, rows, cols):
        return npy(t[torch.as_tensor(rows, device=DEV), torch.as_tensor(cols, device=DEV)]).astype(np.float64)
    # dgrad: da[s, k] = sum_n dq[s, n] W2_g^T[k, n] over all 7168 n
    ij, ref = [], []
    for g in (0, E - 1):
        wh = oracle_quant_rows(host_bf16(L["w2"][g]), E * N, g * N, N, False)
        wt, wte = O.requant_window(wh, g * N, N, target=tgt, seed=seed, stream=3)
        for s in _sample_slots(off, [g], 4, rng):
            dq, de = O.mxfp8_quantize_rows(host_bf16(dy[int(s):int(s) + 1]), target=tgt)
            for k in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dq, de, wt, wte, 0, k, 0, N, target=tgt))
                ij.append((int(s), k))
    got = at(da, [i for i, _ in ij], [j for _, j in ij])
    assert rel_fro(got, ref) <= 2e-3
    # wgrad: db[g N + n, k] = sum over the group's padded slots of dt[n, s] at[k, s]
    ncols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 30)]))
    ij, ref = [], []
    for g in (0, E - 1, 20):
        a, b = int(off[g]), int(off[g + 1])
        dt, dte = O.mxfp8_quantize_cols(host_bf16(dy[a:b][:, torch.as_tensor(ncols, device=DEV)]), target=tgt)
        ah = oracle_quant_rows(host_bf16(A[a:b]), M, a, 1, True)
        xt, xte = O.requant_window(ah, a, b - a, target=tgt, seed=seed, stream=5)
        Pg = dt.shape[1]
        for jj, n in enumerate(ncols.tolist()):
            for k in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dt, dte, xt, xte, jj, k, 0, Pg, target=tgt))
                ij.append((g * N + n, k))
    got = at(db, [i for i, _ in ij], [j for _, j in ij])
    assert rel_fro(got, ref) <= 2e-3
    # the largest group's first and last slot rows of dA are finite and not all zero
    edge = npy(da[torch.as_tensor([0, int(off[1]) - 1], device=DEV)])
    assert np.all(np.isfinite(edge)) and np.any(edge[0] != 0)
