"""GPU test of pmn_check_indices, the device-side check of the index contract the grouped calls
assume (offsets non-decreasing from 0 to M, gather indices inside the gathered matrix), through
the C ABI. The expected masks come from the rules written out in numpy on the host copies; the
check only reads offsets[0..G] and gather[0..n), so corrupted arrays are safe to pass to it (and
are never passed to a GEMM)."""
import numpy as np
import pytest
import torch

DEV = torch.device("cuda:0")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import precision_moe_numerics_amd as P
    return P


def rules(P, offsets, M, gather=None, src_rows=0):
    """The contract of include/pmn.h, rule by rule."""
    bad = 0
    if offsets is not None:
        o = np.asarray(offsets, np.int64)
        if o[0] != 0:
            bad |= P.CHECK_OFFSETS_START
        if o[-1] != M:
            bad |= P.CHECK_OFFSETS_END
        if np.any(np.diff(o) < 0):
            bad |= P.CHECK_OFFSETS_ORDER
        if np.any((o < 0) | (o > M)):
            bad |= P.CHECK_OFFSETS_RANGE
    if gather is not None:
        g = np.asarray(gather, np.int64)
        if np.any((g < 0) | (g >= src_rows)):
            bad |= P.CHECK_GATHER_RANGE
    return bad


def run(P, offsets, M, gather=None, src_rows=0):
    o = None if offsets is None else torch.as_tensor(np.asarray(offsets, np.int64), device=DEV)
    g = None if gather is None else torch.as_tensor(np.asarray(gather, np.int32), device=DEV)
    got = P.check_indices(o, M, g, src_rows)
    assert got == rules(P, offsets, M, gather, src_rows), (got, offsets if offsets is None else offsets[:8])
    return got


def test_routing_output_satisfies_the_contract(P):
    """moe_route_topk's offsets and token gather (16384 tokens, top-8 of 32 experts) break no rule."""
    torch.manual_seed(0)
    T, E, k = 16384, 32, 8
    logits = torch.randn(T, E, device=DEV)
    r = P.moe_route_topk(logits, k)
    offsets, gather = r["offsets"], r["gather"]
    assert P.check_indices(offsets, T * k, gather, T) == 0
    assert run(P, offsets.cpu().numpy(), T * k, gather.cpu().numpy(), T) == 0


@pytest.mark.parametrize("G", [1, 5, 1500])
def test_each_rule(P, G):
    """Every rule alone and in combination, with more groups and gather entries than the check's
    1024 threads (so that its loops wrap), and empty groups."""
    rng = np.random.default_rng(G)
    counts = rng.integers(0, 9, G)
    counts[G // 2] = 0
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    src = 3000
    gather = rng.integers(0, src, max(M, 1)).astype(np.int32)[:M]
    assert run(P, offsets, M, gather, src) == 0
    cases = []
    o = offsets.copy(); o[0] = 1; cases.append(o)                     # start (and order if offsets[1] == 0)
    o = offsets.copy(); o[-1] = M + 3; cases.append(o)                # end and range
    o = offsets.copy(); o[-1] = M - 1 if M > 0 else 1; cases.append(o)
    if G > 2:
        o = offsets.copy(); o[1], o[2] = o[2] + 1, o[1]; cases.append(o)   # order
        o = offsets.copy(); o[G // 3] = -5; cases.append(o)           # range and order
    for o in cases:
        assert run(P, o, M) != 0
    if M > 0:
        for v in (src, -1, 2 ** 31 - 1):
            g = gather.copy(); g[rng.integers(0, M)] = v
            assert run(P, offsets, M, g, src) == P.CHECK_GATHER_RANGE
            assert run(P, None, M, g, src) == P.CHECK_GATHER_RANGE
        g = gather.copy(); g[0] = src
        assert run(P, cases[0], M, g, src) == rules(P, cases[0], M, g, src)


def test_debug_switch_refuses_bad_offsets_before_the_gemm(P, monkeypatch):
    """With the binding's index check switched on, a GEMM call with bad offsets raises before
    launching, and one with good offsets runs as usual."""
    from precision_moe_numerics_amd import inputs as I
    monkeypatch.setattr(P, "CHECK_INDICES", True)
    M, N, K = 96, 256, 64
    x = I.normal((M, K), 1.0, 5, DEV)
    w = I.normal((2 * N, K), 0.02, 6, DEV)
    xq = P.nvfp4_quantize(x, P.NVFP4_ACT)
    wq = P.nvfp4_quantize(w, P.NVFP4_WEIGHT, rows_per_outer=N)
    good = torch.tensor([0, 40, M], dtype=torch.int64, device=DEV)
    y = P.moe_grouped_gemm_fwd(xq, wq, good, M, N)
    torch.cuda.synchronize()
    assert y.shape == (M, N)
    for bad in ([0, 40, M + 1], [0, 60, 40], [1, 40, M]):
        with pytest.raises(P.PmnError, match="index arrays"):
            P.moe_grouped_gemm_fwd(xq, wq, torch.tensor(bad, dtype=torch.int64, device=DEV), M, N)
    gather = torch.arange(M, dtype=torch.int32, device=DEV)
    gather[7] = M
    with pytest.raises(P.PmnError, match="gather index"):
        P.moe_grouped_gemm_fwd(xq, wq, good, M, N, gather=gather)
