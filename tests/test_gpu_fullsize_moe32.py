"""Parity at the full size of the 32-expert routed layer: 16384 tokens, top-8 of 32 experts,
131072 slots, hidden 4096, FFN 1536.

Routing is the oracle's top-8 of softmax over the seeded N(0, 1) logits, so the group offsets and
the gather index (slot -> token) come from the oracle. Activations are quantized once per token
(N(0, 1), 4/6); every GEMM reads its slot rows through the gather index, which the 48-expert
tests (slots already grouped) do not exercise at full size. Sampled outputs are recomputed by the
oracle from the bf16 inputs, as in the 48-expert tests: the oracle quantizes the sampled tokens
and experts itself, and the requantized windows of gathered activations are keyed by slot index.
The bar is the GEMM tolerance (relative Frobenius error <= 2e-3 over the samples) and, for bf16
outputs, one bf16 rounding per element.
"""
import numpy as np
import pytest
import torch

import oracle as O
from fullsize_helpers import oracle_quant_rows, sample_slots

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
def routed():
    import precision_moe_numerics_amd as P
    from precision_moe_numerics_amd import inputs as I
    sh = I.MOE32
    E, H, F, T, k = sh.experts, sh.hidden, sh.ffn, sh.tokens, sh.top_k
    r = O.route_topk(I.moe_logits(sh, "cpu").numpy(), k)
    offsets = r["offsets"].astype(np.int64)
    gather = r["gather"].astype(np.int32)
    M = int(offsets[-1])
    assert M == T * k
    x = I.moe_activations(sh, DEV)
    w13, w2 = I.moe_weights(sh, DEV)
    d = dict(P=P, I=I, E=E, H=H, F=F, T=T, M=M, offsets=offsets, gather=gather, x=x, w13=w13,
             goff=torch.as_tensor(offsets, device=DEV), ggather=torch.as_tensor(gather, device=DEV),
             seed=sh.seeds["sr"])
    d["xq"] = P.nvfp4_quantize(x, P.NVFP4_ACT)
    d["w13q"] = P.nvfp4_quantize(w13.view(E * 2 * F, H), P.NVFP4_WEIGHT, F)
    torch.cuda.synchronize()
    return d


def test_moe32_forward_w13_swiglu_gathered(routed):
    P, L = routed["P"], routed
    M, H, F, E = L["M"], L["H"], L["F"], L["E"]
    a, h13 = P.moe_grouped_gemm_fwd(L["xq"], L["w13q"], L["goff"], M, 2 * F, P.EPI_SWIGLU, gather=L["ggather"],
                                    save_h13=True)
    hg, ag = npy(h13.float()), npy(a.float())
    rng = np.random.default_rng(21)
    fcols = np.concatenate([[0, F - 1], rng.integers(0, F, 6)])
    got_h1, got_h3, ref_h1, ref_h3, got_a = [], [], [], [], []
    for g in (0, 15, E - 1):
        slots = sample_slots(L["offsets"], [g], 6, rng)
        tokens = L["gather"][slots]
        xq = O.nvfp4_quantize(host_bf16(L["x"][torch.as_tensor(tokens, device=DEV, dtype=torch.int64)]), 1, True)
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
    assert np.all(np.abs(g1 - h1) <= 2.0 ** -8 * np.abs(h1) + 1e-30)
    assert np.all(np.abs(g3 - h3) <= 2.0 ** -8 * np.abs(h3) + 1e-30)
    a_ref = h1 / (1.0 + np.exp(-h1)) * h3
    assert np.all(np.abs(ga - a_ref) <= 2.0 ** -8 * np.abs(a_ref) + 1e-30)


def test_moe32_backward_w13_gathered(routed):
    P, I, L = routed["P"], routed["I"], routed
    M, H, F, E = L["M"], L["H"], L["F"], L["E"]
    N, K = 2 * F, H
    dy = I.normal((M, N), 1e-3, 400, DEV)
    da, db, _ = P.moe_grouped_gemm_bwd(dy, L["xq"], L["w13q"], L["goff"], M, N, gather=L["ggather"], seed=L["seed"],
                                       rng_stream_a=4, rng_stream_b=1, rng_stream_dy=8)
    off, seed, gather = L["offsets"], L["seed"], L["gather"]
    dyh = dy.cpu()
    rng = np.random.default_rng(23)
    # dgrad: the weights' windows as in the 48-expert test
    got, ref = [], []
    for g in (0, E - 1):
        wh = oracle_quant_rows(host_bf16(L["w13"][g]), E * N, g * N, F, False)
        wt, wte = O.requant_window(wh, g * N, N, seed=seed, stream=1)
        for s in sample_slots(off, [g], 4, rng):
            dq, de = O.mxfp8_quantize_rows(dyh[int(s):int(s) + 1])
            for kk in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dq, de, wt, wte, 0, kk, 0, N))
                got.append(float(da[int(s), kk]))
    assert rel_fro(got, ref) <= 2e-3
    # wgrad: X^T of group g holds the group's slots in order, each slot reading its token's row;
    # its random bits are keyed by slot index, so the oracle quantizes the gathered token rows and
    # places them at the group's slot positions of a full-size [M x K] source
    got, ref = [], []
    for g in (3, E - 1):
        a, b = int(off[g]), int(off[g + 1])
        dt, dte = O.mxfp8_quantize_cols(dyh[a:b])
        xrows = host_bf16(L["x"][torch.as_tensor(gather[a:b], device=DEV, dtype=torch.int64)])
        xh = oracle_quant_rows(xrows, M, a, 1, True)
        xt, xte = O.requant_window(xh, a, b - a, seed=seed, stream=4)
        Pg = dt.shape[1]
        for n in (0, N - 1, int(rng.integers(0, N))):
            for kk in (0, K - 1, int(rng.integers(0, K))):
                ref.append(O.mxfp8_dot(dt, dte, xt, xte, n, kk, 0, Pg))
                got.append(float(db[g * N + n, kk]))
    assert rel_fro(got, ref) <= 2e-3
