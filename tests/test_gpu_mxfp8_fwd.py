"""Parity of the MXFP8 forward (moe_grouped_gemm_fwd_mxfp8, the layers that keep MXFP8) with the
CPU oracle, through the C ABI.

The oracle quantizes the original bf16 inputs itself (row-wise MXFP8, round to nearest even) and
takes fp64 products; the library's quantized operands in the workspace are checked bit for bit
against the oracle's. Products of two E4M3 values are exact in fp32, so the GEMM is compared at
the GEMM tolerance (relative Frobenius error <= 2e-3, observed about 2e-5). The epilogues are
checked against the library's own F32 result (bf16 rounding, the standalone RHT32 + S2F6
transform) and against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decoders import decode_s2f6_rows, unblock

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def npy(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel_fro(got, ref):
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)


@pytest.fixture(scope="module")
def P():
    import precision_moe_numerics_amd as P
    return P


def _layer(counts, N, K, gather_rows=None, seed=200):
    from precision_moe_numerics_amd import inputs as I
    rng = np.random.default_rng(seed)
    G = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    T = gather_rows or M
    x = I.student_t((T, K), 4, 1.0, seed + 1)
    w = I.normal((G * N, K), 0.02, seed + 2)
    gather = rng.integers(0, T, M).astype(np.int32) if gather_rows else None
    xq, xe = O.mxfp8_quantize_rows(x)
    wq, we = O.mxfp8_quantize_rows(w)
    return dict(offsets=offsets, M=M, G=G, x=x, w=w, gather=gather, xq=xq, xe=xe, wq=wq, we=we,
                goff=torch.as_tensor(offsets, device=DEV),
                ggather=None if gather is None else torch.as_tensor(gather, device=DEV))


def swiglu_bound(h1, h3, aref):
    dh = 1e-4 * max(np.abs(h1).max(), np.abs(h3).max())
    sg = 1.0 / (1.0 + np.exp(-h1))
    return 2.0 ** -8 * np.abs(aref) + (np.abs(sg * (1 + h1 * (1 - sg)) * h3) + np.abs(h1 * sg)) * dh + 1e-30


CASES = [([300], 256, 192, None), ([10, 0, 300, 77], 512, 256, 200), ([256, 513], 256, 1024, 1000),
         ([37, 1, 90], 512, 96, None), ([64, 0, 5], 256, 160, 40), ([1], 256, 32, None),
         # N not a multiple of 256: a partial last feature tile (32 or 96 of its rows exist)
         ([70, 300, 1], 288, 96, None), ([5, 0, 600], 352, 160, 700)]


@pytest.mark.parametrize("counts,N,K,gather_rows", CASES)
def test_mxfp8_fwd_f32_bf16_and_operands(P, counts, N, K, gather_rows):
    """Ragged and empty groups, a gather, K a multiple of 64 and K = 32 mod 64 (a half-full last
    stage), one and several tiles per dimension, N not a multiple of 256."""
    d = _layer(counts, N, K, gather_rows)
    M, G = d["M"], d["G"]
    ws = torch.empty((P._lib.moe_grouped_gemm_fwd_mxfp8_workspace_size(M, G, N, K),), dtype=torch.uint8, device=DEV)
    y = P.moe_grouped_gemm_fwd_mxfp8(d["x"].to(DEV), d["w"].to(DEV), d["goff"], M, N, P.EPI_F32, gather=d["ggather"],
                                     workspace=ws)
    ref = O.gemm_mxfp8_fwd(d["xq"], d["xe"], d["wq"], d["we"], d["offsets"], N, K, gather=d["gather"])
    assert rel_fro(npy(y), ref) <= 2e-3
    # products are exact; the block-scaled MFMA's internal sums round a little more than a plain
    # fp32 chain (about 2e-5 observed); a wrong k-block or scale would show at the 1e-1 level
    assert rel_fro(npy(y), ref) <= 1e-4
    yb = P.moe_grouped_gemm_fwd_mxfp8(d["x"].to(DEV), d["w"].to(DEV), d["goff"], M, N, P.EPI_BF16,
                                      gather=d["ggather"])
    assert torch.equal(yb, y.to(torch.bfloat16))
    # the quantized operands in the workspace: X in slot order at padded rows, W row-wise, both
    # blocked with rows of K rounded up to 64 bytes (zero codes past K); E8M0 k-block-major
    w8 = npy(ws)
    Pb = P.padded_bound(M, G)
    Kp = (K + 63) // 64 * 64
    r256 = lambda b: (b + 255) // 256 * 256
    o_xq, o_xe = 0, r256(Pb * Kp)
    o_wq = o_xe + r256(K // 32 * Pb)
    o_we = o_wq + r256(G * N * Kp)
    off = d["offsets"]
    po = np.concatenate([[0], np.cumsum((np.diff(off) + 31) // 32 * 32)])
    grp = np.searchsorted(off, np.arange(M), side="right") - 1
    pcol = po[grp] + np.arange(M) - off[grp]
    rows = d["gather"] if d["gather"] is not None else np.arange(M)
    xb = unblock(w8[o_xq:o_xq + Pb * Kp], Pb, Kp)[pcol]
    wb = unblock(w8[o_wq:o_wq + G * N * Kp], G * N, Kp)
    assert np.array_equal(xb[:, :K], d["xq"][rows]) and np.all(xb[:, K:] == 0)
    assert np.array_equal(wb[:, :K], d["wq"]) and np.all(wb[:, K:] == 0)
    assert np.array_equal(w8[o_we:o_we + K // 32 * G * N].reshape(K // 32, G * N).T, d["we"])
    assert np.array_equal(w8[o_xe:o_xe + K // 32 * Pb].reshape(K // 32, Pb)[:, pcol].T, d["xe"][rows])


@pytest.mark.parametrize("counts,F,K,gather_rows", [([130, 0, 301], 128, 256, 250), ([40, 300], 256, 96, None),
                                                    ([40, 300], 160, 96, None)])
def test_mxfp8_fwd_swiglu(P, counts, F, K, gather_rows):
    d = _layer(counts, 2 * F, K, gather_rows, seed=210)
    M = d["M"]
    a, h13 = P.moe_grouped_gemm_fwd_mxfp8(d["x"].to(DEV), d["w"].to(DEV), d["goff"], M, 2 * F, P.EPI_SWIGLU,
                                          gather=d["ggather"], save_h13=True)
    y = P.moe_grouped_gemm_fwd_mxfp8(d["x"].to(DEV), d["w"].to(DEV), d["goff"], M, 2 * F, P.EPI_F32,
                                     gather=d["ggather"])
    assert torch.equal(h13, y.to(torch.bfloat16))       # h1 | h3 are the bf16 of the same fp32 sums
    ref = O.gemm_mxfp8_fwd(d["xq"], d["xe"], d["wq"], d["we"], d["offsets"], 2 * F, K, gather=d["gather"])
    aref = O.swiglu(ref.astype(np.float32), F)
    assert rel_fro(npy(a.float()), aref) <= 2e-3
    # per value: one bf16 rounding plus the GEMM error (absolute, at most 1e-4 of the largest |h|)
    # carried through SwiGLU's partial derivatives
    assert np.all(np.abs(npy(a.float()) - aref) <= swiglu_bound(ref[:, :F], ref[:, F:], aref))
    # without out_aux only A is written
    a2, none = P.moe_grouped_gemm_fwd_mxfp8(d["x"].to(DEV), d["w"].to(DEV), d["goff"], M, 2 * F, P.EPI_SWIGLU,
                                            gather=d["ggather"])
    assert none is None and torch.equal(a2, a)


@pytest.mark.parametrize("counts,N,K", [([70, 256, 3], 512, 192), ([300, 1], 256, 96), ([300, 1], 288, 96)])
def test_mxfp8_fwd_rht_epilogue(P, counts, N, K):
    from precision_moe_numerics_amd import inputs as I
    d = _layer(counts, N, K, gather_rows=120, seed=220)
    M = d["M"]
    mask = I.sign_mask(3)
    y = P.moe_grouped_gemm_fwd_mxfp8(d["x"].to(DEV), d["w"].to(DEV), d["goff"], M, N, P.EPI_F32, gather=d["ggather"])
    c, e = P.moe_grouped_gemm_fwd_mxfp8(d["x"].to(DEV), d["w"].to(DEV), d["goff"], M, N, P.EPI_RHT32_S2F6,
                                        gather=d["ggather"], rht_sign_mask=mask)
    sc, se = P.rht32_s2f6_quantize(y, mask)
    assert torch.equal(c, sc) and torch.equal(e, se)
    ref = O.gemm_mxfp8_fwd(d["xq"], d["xe"], d["wq"], d["we"], d["offsets"], N, K, gather=d["gather"])
    dec = decode_s2f6_rows(npy(c), npy(e), mask)
    err = np.sqrt(((dec - ref) ** 2).reshape(M, N // 32, 32).sum(-1))
    nrm = np.sqrt((ref ** 2).reshape(M, N // 32, 32).sum(-1))
    assert np.all(err <= 2.0 ** (npy(e).astype(np.float64) - 127) / 128 * (1 + 1e-6) + 1e-5 * nrm)


def test_mxfp8_fwd_argument_errors(P):
    lib = P._lib
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((256, 256), dtype=torch.bfloat16, device=DEV)
    off = torch.tensor([0, 64], dtype=torch.int64, device=DEV)
    out = torch.empty((64 * 256 + 16,), dtype=torch.float32, device=DEV)
    oe = torch.empty((64 * 8 + 16,), dtype=torch.uint8, device=DEV)
    need = lib.moe_grouped_gemm_fwd_mxfp8_workspace_size(64, 1, 256, 256)
    ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
    p = lambda t: t.data_ptr()
    s = P._stream()
    call = lambda N, K, epi=0, o=None, e=None, wsb=need: lib.moe_grouped_gemm_fwd_mxfp8(
        p(x), 64, None, p(w), p(off), 1, 64, N, K, epi, 0, o if o is not None else p(out), e, None, p(ws), wsb, s)
    assert call(144, 256) == -2                       # N % 32
    assert call(96, 256, epi=2) == -2                 # SwiGLU: N % 64
    assert call(256, 48) == -2                        # K % 32
    assert call(256, 256, epi=7) == -1                # epilogue
    assert call(256, 256, epi=3) == -1                # RHT without out_e8m0
    assert call(256, 256, wsb=need - 1) == -4         # workspace
    assert call(256, 256, o=p(out) + 4) == -3         # alignment
    assert call(256, 256, epi=3, e=p(oe) + 4) == -3
    assert call(256, 256) == 0
    torch.cuda.synchronize()


def test_mxfp8_fwd_full_size_ep48_sampled(P):
    """The 48-expert layer (65536 slots, Zipf loads, H 7168, F 2048) in MXFP8: w13 with SwiGLU and
    w2 with RHT32 + S2F6, in the launch configuration the bench times; sampled slots of ragged
    groups (first and last), first and last features, against the oracle's own quantization of
    the sampled rows and experts."""
    from precision_moe_numerics_amd import inputs as I
    sh = I.EP48
    E, H, F = sh.experts, sh.hidden, sh.ffn
    counts = I.moe_loads(sh)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(off[-1])
    goff = torch.as_tensor(off, device=DEV)
    x = I.moe_activations(sh, DEV)
    w13, w2 = I.moe_weights(sh, DEV)
    a, h13 = P.moe_grouped_gemm_fwd_mxfp8(x, w13.view(E * 2 * F, H), goff, M, 2 * F, P.EPI_SWIGLU, save_h13=True)
    A = I.student_t((M, F), 4, 0.05, 611, DEV)
    c, e = P.moe_grouped_gemm_fwd_mxfp8(A, w2.view(E * H, F), goff, M, H, P.EPI_RHT32_S2F6,
                                        rht_sign_mask=I.sign_mask(sh.seeds["rht"]))
    y2 = P.moe_grouped_gemm_fwd_mxfp8(A, w2.view(E * H, F), goff, M, H, P.EPI_F32)
    sc, se = P.rht32_s2f6_quantize(y2, I.sign_mask(sh.seeds["rht"]))
    assert torch.equal(c, sc) and torch.equal(e, se)
    rng = np.random.default_rng(31)
    hg, ag = npy(h13.float()), npy(a.float())
    got1, got3, ref1, ref3, gota, goty, refy = [], [], [], [], [], [], []
    for g in (0, 1, 23, E - 1):
        a0, b0 = int(off[g]), int(off[g + 1])
        slots = np.array([a0, b0 - 1] + list(rng.integers(a0, b0, 3)))
        xq, xe = O.mxfp8_quantize_rows(x[torch.as_tensor(slots, device=DEV)].cpu())
        wq, we = O.mxfp8_quantize_rows(w13[g].cpu())
        for li, s in enumerate(slots):
            for n in (0, F - 1, int(rng.integers(0, F))):
                ref1.append(O.mxfp8_dot(xq, xe, wq, we, li, n, 0, H))
                ref3.append(O.mxfp8_dot(xq, xe, wq, we, li, F + n, 0, H))
                got1.append(hg[s, n])
                got3.append(hg[s, F + n])
                gota.append(ag[s, n])
        aq, ae = O.mxfp8_quantize_rows(A[torch.as_tensor(slots, device=DEV)].cpu())
        w2q, w2e = O.mxfp8_quantize_rows(w2[g].cpu())
        yrows = npy(y2[torch.as_tensor(slots, device=DEV)])
        for li in range(len(slots)):
            for n in (0, H - 1, int(rng.integers(0, H))):
                refy.append(O.mxfp8_dot(aq, ae, w2q, w2e, li, n, 0, F))
                goty.append(yrows[li, n])
    r1, r3 = np.array(ref1), np.array(ref3)
    assert rel_fro(got1, r1) <= 2e-3 and rel_fro(got3, r3) <= 2e-3 and rel_fro(goty, refy) <= 2e-3
    assert np.all(np.abs(np.array(got1) - r1) <= 2.0 ** -8 * np.abs(r1) + 1e-4 * np.abs(r1).max())
    aref = r1 / (1.0 + np.exp(-r1)) * r3
    assert np.all(np.abs(np.array(gota) - aref) <= swiglu_bound(r1, r3, aref))
