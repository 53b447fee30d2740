"""Parity at the full size of the 48-expert layer step, in the launch configuration the bench times.

The layer is built as the bench builds it: 65536 routed slots with Zipf(1.1) loads over 48
experts, hidden 7168, FFN 2048, weights N(0, 0.02) quantized per (expert, matrix), activations
Student-t(4) quantized per token with 4/6. The oracle cannot redo the whole layer in seconds, so
outputs are sampled: every sampled value is recomputed by the oracle from the original inputs
(its own quantization, requantization windows and fp64 dot products), never from an intermediate
of the HIP path. Samples include the first and last slot of ragged groups and the first and last
output column. The bar is the GEMM tolerance, relative Frobenius error <= 2e-3 over the samples,
and for bf16 outputs one bf16 rounding (2^-8 of the value) per element; the fused RHT32 + S2F6
codes are bit-exact with the oracle transform of the same kernel's fp32 rows.
"""
import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def npy(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel_fro(got, ref):
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)


def host_q(q):
    return dict(codes=npy(q.codes), scales=npy(q.scales), outer=npy(q.outer), rows_per_outer=q.rows_per_outer)


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
    d = dict(P=P, I=I, E=E, H=H, F=F, M=M, counts=np.asarray(counts), offsets=offsets,
             goff=torch.as_tensor(offsets, device=DEV), seed=sh.seeds["sr"], mask=I.sign_mask(sh.seeds["rht"]))
    d["xq"] = P.nvfp4_quantize(x, P.NVFP4_ACT)
    d["w13q"] = P.nvfp4_quantize(w13.view(E * 2 * F, H), P.NVFP4_WEIGHT, F)
    d["w2q"] = P.nvfp4_quantize(w2.view(E * H, F), P.NVFP4_WEIGHT, H)
    del x, w13, w2
    torch.cuda.synchronize()
    return d


def _sample_slots(offsets, groups, per_group, rng):
    s = []
    for g in groups:
        a, b = int(offsets[g]), int(offsets[g + 1])
        s += [a, b - 1] + list(rng.integers(a, b, per_group - 2))
    return np.array(s, np.int64)


def test_ep48_forward_w13_swiglu_sampled(layer):
    P, L = layer["P"], layer
    M, H, F, E = L["M"], L["H"], L["F"], L["E"]
    a, h13 = P.moe_grouped_gemm_fwd(L["xq"], L["w13q"], L["goff"], M, 2 * F, P.EPI_SWIGLU, save_h13=True)
    rng = np.random.default_rng(11)
    slots = _sample_slots(L["offsets"], [0, 1, 23, E - 1], 6, rng)
    fcols = np.concatenate([[0, F - 1], rng.integers(0, F, 6)])
    rows = np.repeat(slots, len(fcols))
    cols = np.tile(fcols, len(slots))
    xh, wh = host_q(L["xq"]), host_q(L["w13q"])
    h1 = O.gemm_nvfp4_elems(xh, wh, L["offsets"], 2 * F, H, rows, cols)
    h3 = O.gemm_nvfp4_elems(xh, wh, L["offsets"], 2 * F, H, rows, cols + F)
    hg = npy(h13.float())
    assert rel_fro(hg[rows, cols], h1) <= 2e-3 and rel_fro(hg[rows, cols + F], h3) <= 2e-3
    # bf16 outputs: each within bf16 rounding of the fp64 value
    assert np.all(np.abs(hg[rows, cols] - h1) <= 2.0 ** -8 * np.abs(h1) + 1e-30)
    # A = silu(h1) h3 is a bf16 output too: within one bf16 rounding of the fp64 value (bf16 keeps
    # 8 significant bits, so rounding alone moves a value by up to 2^-9 of itself)
    a_ref = h1 / (1.0 + np.exp(-h1)) * h3
    ag = npy(a.float())[rows, cols]
    assert np.all(np.abs(ag - a_ref) <= 2.0 ** -8 * np.abs(a_ref) + 1e-30)


def test_ep48_forward_w2_rht_s2f6_sampled(layer):
    P, L = layer["P"], layer
    M, H, F, E = L["M"], L["H"], L["F"], L["E"]
    a, _ = P.moe_grouped_gemm_fwd(L["xq"], L["w13q"], L["goff"], M, 2 * F, P.EPI_SWIGLU)
    aq = P.nvfp4_quantize(a, P.NVFP4_ACT)
    y = P.moe_grouped_gemm_fwd(aq, L["w2q"], L["goff"], M, H, P.EPI_F32)
    c, e = P.moe_grouped_gemm_fwd(aq, L["w2q"], L["goff"], M, H, P.EPI_RHT32_S2F6, rht_sign_mask=L["mask"])
    rng = np.random.default_rng(12)
    slots = _sample_slots(L["offsets"], [0, 7, E - 1], 3, rng)
    yr = npy(y)[slots]
    # the fused epilogue equals the oracle transform of the same fp32 rows, bit for bit
    rc, re = O.rht32_s2f6_quantize(yr, L["mask"])
    assert np.array_equal(npy(c)[slots], rc) and np.array_equal(npy(e)[slots], re)
    # and those fp32 rows match the oracle's fp64 GEMM on the same quantized operands
    cols = np.concatenate([[0, H - 1], rng.integers(0, H, 62)])
    rows = np.repeat(slots, len(cols))
    ref = O.gemm_nvfp4_elems(host_q(aq), host_q(L["w2q"]), L["offsets"], H, F, rows, np.tile(cols, len(slots)))
    assert rel_fro(yr[:, cols].reshape(-1), ref) <= 2e-3


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
    # dgrad: da[s, k] = sum_n dq[s, n] wt[k, g N + n]; W^T of expert g is rebuilt as a window
    wh = host_q(L["w13q"])
    got, ref = [], []
    for g in (0, E - 1):
        wt, wte = O.requant_window(wh, g * N, N, seed=seed, stream=1)
        for s in _sample_slots(off, [g], 4, rng):
            dq, de = O.mxfp8_quantize_rows(dyh[int(s):int(s) + 1])
            for k in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dq, de, wt, wte, 0, k, 0, N))
                got.append(float(da[int(s), k]))
    assert rel_fro(got, ref) <= 2e-3
    # wgrad: db[g N + n, k] = sum over the group's padded slots of dt[n, s] xt[k, s]
    xh = host_q(L["xq"])
    got, ref = [], []
    for g in (E - 1, E - 2, 20):
        a, b = int(off[g]), int(off[g + 1])
        dt, dte = O.mxfp8_quantize_cols(dyh[a:b])
        xt, xte = O.requant_window(xh, a, b - a, seed=seed, stream=4)
        Pg = dt.shape[1]
        for n in (0, N - 1, int(rng.integers(0, N))):
            for k in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dt, dte, xt, xte, n, k, 0, Pg))
                got.append(float(db[g * N + n, k]))
    assert rel_fro(got, ref) <= 2e-3
