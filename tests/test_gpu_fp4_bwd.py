"""Parity of the FP4 backward variant (moe_grouped_gemm_bwd with PMN_BWD_FP4) with the CPU oracle.

Every operand is quantized to MXFP4 (E2M1 codes, one E8M0 per 32 values, no saturation): dY
row-wise and column-wise per group (round to nearest even or stochastic), W^T and A^T requantized
from the saved NVFP4 operands by stochastic rounding. The workspace's packed codes and scales are
compared bit for bit with the oracle's own quantization of the same original inputs (packed two
per byte by the test); dgrad and wgrad within 2e-3 relative Frobenius error of the oracle's fp64
products (products of E2M1 values are exact; only the fp32 accumulation rounds).
"""
import numpy as np
import pytest
import torch

import oracle as O
from decoders import unblock

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
E2M1 = O.TARGET_E2M1


def npy(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel_fro(got, ref):
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)


def pack(codes):
    """One E2M1 code per byte -> two per byte, element 2j in the low nibble."""
    c = np.asarray(codes, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


@pytest.fixture(scope="module")
def P():
    import precision_moe_numerics_amd as P
    return P


def _layer(counts, N, K, gather_rows, seed):
    from precision_moe_numerics_amd import inputs as I
    import precision_moe_numerics_amd as P
    rng = np.random.default_rng(seed)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M, G = int(offsets[-1]), len(counts)
    T = gather_rows or M
    x = I.student_t((T, K), 4, 1.0, seed + 1)
    w = I.normal((G * N, K), 0.02, seed + 2)
    dy = I.normal((M, N), 1e-3, seed + 3)
    gather = rng.integers(0, T, M).astype(np.int32) if gather_rows else None
    rpo = N // 2
    d = dict(offsets=offsets, M=M, G=G, x=x, w=w, dy=dy, gather=gather,
             xq=P.nvfp4_quantize(x.to(DEV), P.NVFP4_ACT), wq=P.nvfp4_quantize(w.to(DEV), P.NVFP4_WEIGHT, rpo),
             rxq=O.nvfp4_quantize(x, 1, True), rwq=O.nvfp4_quantize(w, rpo, False),
             goff=torch.as_tensor(offsets, device=DEV),
             ggather=None if gather is None else torch.as_tensor(gather, device=DEV))
    return d


@pytest.mark.parametrize("counts,N,K,gather_rows,sr", [([40, 0, 333, 227], 256, 512, 400, False),
                                                        ([150, 1, 95, 33], 256, 256, 300, True),
                                                        ([700], 512, 256, None, False)])
def test_fp4_backward_operands_and_gradients(P, counts, N, K, gather_rows, sr):
    d = _layer(counts, N, K, gather_rows, seed=300 + len(counts))
    M, G = d["M"], d["G"]
    seed, sa, sb, sdy = 11, 4, 1, 6
    da, db, ws = P.moe_grouped_gemm_bwd(d["dy"].to(DEV), d["xq"], d["wq"], d["goff"], M, N,
                                        flags=P.BWD_DGRAD | P.BWD_WGRAD | P.BWD_FP4, gather=d["ggather"],
                                        dy_rounding=P.SR if sr else P.RNE, seed=seed, rng_stream_a=sa,
                                        rng_stream_b=sb, rng_stream_dy=sdy)
    v = P.bwd_workspace_views(ws, M, G, N, K, fp4=True)
    # The library pads each group to 128 slots (one 64-byte block column of packed codes) and
    # keeps the code parts blocked; the oracle pads to 32 and is row-major.
    off = d["offsets"]
    cnt = np.diff(off)
    po32 = np.concatenate([[0], np.cumsum((cnt + 31) // 32 * 32)])
    po = np.concatenate([[0], np.cumsum((cnt + 127) // 128 * 128)])
    assert np.array_equal(npy(v["po"]), po)
    Pb = v["de"].shape[1]
    grp = np.searchsorted(off, np.arange(M), side="right") - 1
    pcol = po[grp] + np.arange(M) - off[grp]
    # dY row-wise (the dgrad's A) and column-wise per group (the wgrad's A)
    rq, re = O.mxfp8_quantize_rows(d["dy"], sr=sr, seed=seed, stream=sdy, target=E2M1)
    assert np.array_equal(unblock(npy(v["dq"]), Pb, N // 2)[pcol], pack(rq))
    assert np.array_equal(npy(v["de"])[:, pcol].T, re)
    rt, rte = O.mxfp8_quantize_cols(d["dy"], offsets=off, sr=sr, seed=seed, stream=sdy + 1, target=E2M1)
    # W^T and A^T requantized by SR onto the E2M1 grid
    rwt, rwte = O.requant_transpose_sr(d["rwq"], target=E2M1, seed=seed, stream=sb)
    assert np.array_equal(unblock(npy(v["wt"]), K, G * N // 2), pack(rwt)) and np.array_equal(npy(v["wte"]).T, rwte)
    rxt, rxte = O.requant_transpose_sr(d["rxq"], gather=d["gather"], offsets=off, target=E2M1, seed=seed, stream=sa)
    for name, ref, ref_e in (("dt", rt, rte), ("xt", rxt, rxte)):
        got = unblock(npy(v[name]), ref.shape[0], Pb // 2)
        got_e = npy(v[name + "e"]).T
        pref = pack(ref)
        for g in range(G):
            n32 = po32[g + 1] - po32[g]
            a, a32 = po[g], po32[g]
            assert np.array_equal(got[:, a // 2:(a + n32) // 2], pref[:, a32 // 2:(a32 + n32) // 2]), (name, g)
            assert np.array_equal(got_e[:, a // 32:(a + n32) // 32], ref_e[:, a32 // 32:(a32 + n32) // 32]), (name, g)
            assert np.all(got[:, (a + n32) // 2:po[g + 1] // 2] == 0), (name, g)   # blocks of padding only
    # gradients on the FP4 MFMA
    da_ref = O.gemm_mxfp8_dgrad(rq, re, rwt, rwte, off, N, K, target=E2M1)
    db_ref = O.gemm_mxfp8_wgrad(rt, rte, rxt, rxte, off, N, K, target=E2M1)
    assert rel_fro(npy(da), da_ref) <= 2e-3
    assert rel_fro(npy(db), db_ref) <= 2e-3
    for g in range(G):
        if off[g + 1] == off[g]:
            assert np.all(npy(db)[g * N:(g + 1) * N] == 0)     # an empty expert gets a zero gradient


def test_fp4_backward_deterministic_and_separate_flags(P):
    d = _layer([200, 56], 256, 256, None, seed=330)
    M = d["M"]
    f = P.BWD_DGRAD | P.BWD_WGRAD | P.BWD_FP4
    a1 = P.moe_grouped_gemm_bwd(d["dy"].to(DEV), d["xq"], d["wq"], d["goff"], M, 256, flags=f, dy_rounding=P.SR, seed=3)
    a2 = P.moe_grouped_gemm_bwd(d["dy"].to(DEV), d["xq"], d["wq"], d["goff"], M, 256, flags=f, dy_rounding=P.SR, seed=3)
    assert torch.equal(a1[0], a2[0]) and torch.equal(a1[1], a2[1])
    only_d = P.moe_grouped_gemm_bwd(d["dy"].to(DEV), d["xq"], d["wq"], d["goff"], M, 256,
                                    flags=P.BWD_DGRAD | P.BWD_FP4, dy_rounding=P.SR, seed=3)
    only_w = P.moe_grouped_gemm_bwd(d["dy"].to(DEV), d["xq"], d["wq"], d["goff"], M, 256,
                                    flags=P.BWD_WGRAD | P.BWD_FP4, dy_rounding=P.SR, seed=3)
    assert torch.equal(only_d[0], a1[0]) and torch.equal(only_w[1], a1[1])
    # FP4 alone, without a gradient, is not a request
    with pytest.raises(P.PmnError):
        P.moe_grouped_gemm_bwd(d["dy"].to(DEV), d["xq"], d["wq"], d["goff"], M, 256, flags=P.BWD_FP4)


def test_fp4_backward_full_size_ep48_sampled(P):
    """The 48-expert layer's w13 backward in FP4, in the launch configuration the bench times:
    sampled dX and dW values against the oracle's own quantization of the original inputs (W_g^T
    and X^T windows taken from full-size arrays in which only the sampled rows are filled). dY is
    rounded to nearest here, so a sampled row or group quantizes on its own; stochastic dY
    rounding is covered bit for bit by the smaller cases above."""
    from precision_moe_numerics_amd import inputs as I
    from fullsize_helpers import oracle_quant_rows, sample_slots as _sample_slots
    sh = I.EP48
    E, H, F = sh.experts, sh.hidden, sh.ffn
    N, K = 2 * F, H
    off = np.concatenate([[0], np.cumsum(I.moe_loads(sh))]).astype(np.int64)
    M = int(off[-1])
    x = I.moe_activations(sh, DEV)
    w13, _ = I.moe_weights(sh, DEV)
    xq = P.nvfp4_quantize(x, P.NVFP4_ACT)
    wq = P.nvfp4_quantize(w13.view(E * N, H), P.NVFP4_WEIGHT, F)
    dy = I.normal((M, N), 1e-3, 602, DEV)
    seed = sh.seeds["sr"]
    da, db, _ = P.moe_grouped_gemm_bwd(dy, xq, wq, torch.as_tensor(off, device=DEV), M, N,
                                       flags=P.BWD_DGRAD | P.BWD_WGRAD | P.BWD_FP4, dy_rounding=P.RNE, seed=seed,
                                       rng_stream_a=4, rng_stream_b=1, rng_stream_dy=8)
    dyh = dy.cpu()
    rng = np.random.default_rng(41)
    got, ref = [], []
    for g in (0, E - 1):
        wh = oracle_quant_rows(w13[g].cpu(), E * N, g * N, F, False)
        wt, wte = O.requant_window(wh, g * N, N, target=E2M1, seed=seed, stream=1)
        for s in _sample_slots(off, [g], 4, rng):
            dq, de = O.mxfp8_quantize_rows(dyh[int(s):int(s) + 1], target=E2M1)
            for k in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dq, de, wt, wte, 0, k, 0, N, target=E2M1))
                got.append(float(da[int(s), k]))
    assert rel_fro(got, ref) <= 2e-3
    got, ref = [], []
    for g in (E - 1, E - 2, 20):
        a, b = int(off[g]), int(off[g + 1])
        dt, dte = O.mxfp8_quantize_cols(dyh[a:b], target=E2M1)
        xh = oracle_quant_rows(x[a:b].cpu(), M, a, 1, True)
        xt, xte = O.requant_window(xh, a, b - a, target=E2M1, seed=seed, stream=4)
        Pg = dt.shape[1]
        for n in (0, N - 1, int(rng.integers(0, N))):
            for k in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dt, dte, xt, xte, n, k, 0, Pg, target=E2M1))
                got.append(float(db[g * N + n, k]))
    assert rel_fro(got, ref) <= 2e-3

