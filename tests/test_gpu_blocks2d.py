"""NVFP4 with 16 x 16 square blocks (nvfp4_quantize, PMN_NVFP4_WEIGHT_2D) against the CPU oracle:
bit-exact codes, scales and outer scales; the transpose bit-identity on the device; and the
result used as an ordinary NVFP4 operand by the grouped GEMM."""
import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def npy(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def nibbles(codes):
    c = np.asarray(codes)
    out = np.zeros((c.shape[0], c.shape[1] * 2), np.uint8)
    out[:, 0::2], out[:, 1::2] = c & 15, c >> 4
    return out


@pytest.fixture(scope="module")
def P():
    import precision_moe_numerics_amd as P
    return P


@pytest.mark.parametrize("rows,cols,rpo,kind", [(64, 96, 64, "t3"), (48, 80, 16, "t3"), (256, 512, 256, "outliers"),
                                                (16, 16, 16, "normal"), (4096, 7168, 4096, "weights")])
def test_nvfp4_2d_vs_oracle(P, rows, cols, rpo, kind):
    from precision_moe_numerics_amd import inputs as I
    if kind == "outliers":
        x = I.single_expert("cpu")["x"]
    elif kind == "weights":
        x = I.normal((rows, cols), 0.02, 501)
    elif kind == "t3":
        x = I.student_t((rows, cols), 3, 1.0, rows + cols)
    else:
        x = I.normal((rows, cols), 1.0, 7)
    q = P.nvfp4_quantize(x.to(DEV), P.NVFP4_WEIGHT_2D, rows_per_outer=rpo)
    ref = O.nvfp4_quantize_2d(x, rpo)
    assert np.array_equal(npy(q.codes), ref["codes"])
    assert np.array_equal(npy(q.scales), ref["scales"])
    assert np.array_equal(npy(q.outer), ref["outer"])


def test_nvfp4_2d_transpose_bit_identity_on_device(P):
    from precision_moe_numerics_amd import inputs as I
    x = I.single_expert("cpu")["x"].to(DEV)
    a = P.nvfp4_quantize(x, P.NVFP4_WEIGHT_2D, rows_per_outer=256)
    b = P.nvfp4_quantize(x.t().contiguous(), P.NVFP4_WEIGHT_2D, rows_per_outer=512)
    assert np.array_equal(nibbles(npy(b.codes)), nibbles(npy(a.codes)).T)
    sa, sb = npy(a.scales), npy(b.scales)
    assert np.array_equal(sa[::16], sb[::16].T)
    assert npy(a.outer)[0] == npy(b.outer)[0]


def test_nvfp4_2d_weights_in_the_grouped_gemm(P):
    """2D-quantized weights are an ordinary NVFP4 operand: the forward GEMM on them matches the
    oracle's product of the oracle's own 2D quantization."""
    from precision_moe_numerics_amd import inputs as I
    counts, N, K = [100, 37], 256, 512
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    x = I.student_t((M, K), 4, 1.0, 61)
    w = I.normal((2 * N, K), 0.02, 62)
    xq = P.nvfp4_quantize(x.to(DEV), P.NVFP4_ACT)
    wq = P.nvfp4_quantize(w.to(DEV), P.NVFP4_WEIGHT_2D, rows_per_outer=N)
    y = P.moe_grouped_gemm_fwd(xq, wq, torch.as_tensor(offsets, device=DEV), M, N, P.EPI_F32)
    ref = O.gemm_nvfp4_grouped(O.nvfp4_quantize(x, 1, True), O.nvfp4_quantize_2d(w, N), offsets, N, K)
    err = np.linalg.norm(npy(y) - ref) / np.linalg.norm(ref)
    assert err <= 2e-3


def test_nvfp4_2d_shape_errors(P):
    x = torch.zeros((40, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(P.PmnError):
        P.nvfp4_quantize(x, P.NVFP4_WEIGHT_2D, rows_per_outer=40)      # rows not a multiple of 16
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(P.PmnError):
        P.nvfp4_quantize(x, P.NVFP4_WEIGHT_2D, rows_per_outer=8)       # groups not a multiple of 16
