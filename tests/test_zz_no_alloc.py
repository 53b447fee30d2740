"""moe_grouped_gemm_bwd_noalloc (workspace in the library's static device scratch) against
moe_grouped_gemm_bwd (caller's workspace), through the C ABI: two calls in a row on one device, the
second with smaller sizes, so the second runs on scratch that still holds the first call's
contents. The two entry points launch the same kernels on the same inputs, so the gradients must be
bit-identical (stronger than the GEMM tolerance of the oracle comparisons)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def P():
    import precision_moe_numerics_amd as P
    return P


def _case(P, counts, N, K, T, seed):
    from precision_moe_numerics_amd import inputs as I
    rng = np.random.default_rng(seed)
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(off[-1])
    x = I.student_t((T, K), 4, 1.0, seed + 1).to(DEV)
    w = I.normal((G * N, K), 0.02, seed + 2).to(DEV)
    gather = torch.as_tensor(rng.integers(0, T, M).astype(np.int32), device=DEV)
    dy = I.normal((M, N), 1e-3, seed + 3).to(DEV)
    xq = P.nvfp4_quantize(x, P.NVFP4_ACT)
    wq = P.nvfp4_quantize(w, P.NVFP4_WEIGHT, rows_per_outer=N)
    return dict(M=M, N=N, K=K, G=G, off=torch.as_tensor(off, device=DEV), gather=gather, dy=dy, xq=xq, wq=wq)


def test_noalloc_matches_workspace_call_twice_second_smaller(P):
    assert P._lib.pmn_noalloc_scratch_bytes() == 256 << 20
    cases = [(_case(P, [700, 0, 513, 1, 286], 512, 768, 900, 810), P.BWD_DGRAD | P.BWD_WGRAD, P.RNE),
             (_case(P, [130, 2, 57], 256, 512, 150, 820), P.BWD_DGRAD | P.BWD_WGRAD | P.BWD_FP4, P.SR)]
    for d, flags, rnd in cases:
        assert P.moe_grouped_gemm_bwd_workspace_size(d["M"], d["G"], d["N"], d["K"], flags) <= 256 << 20
        kw = dict(flags=flags, gather=d["gather"], dy_rounding=rnd, seed=9, rng_stream_a=4, rng_stream_b=1,
                  rng_stream_dy=6)
        da0, db0, _ = P.moe_grouped_gemm_bwd(d["dy"], d["xq"], d["wq"], d["off"], d["M"], d["N"], **kw)
        da1, db1 = P.moe_grouped_gemm_bwd_noalloc(d["dy"], d["xq"], d["wq"], d["off"], d["M"], d["N"], **kw)
        torch.cuda.synchronize()
        assert torch.equal(da0, da1) and torch.equal(db0, db1)
        assert torch.isfinite(da1).all() and torch.isfinite(db1).all() and da1.abs().max() > 0

