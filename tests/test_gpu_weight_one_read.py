"""The weight quantization that reads x once (nvfp4_quantize_ws): bit-exact with the oracle and
bit-identical with the two-read path of nvfp4_quantize, on group counts that exercise every
branch of its round schedule (1, 2, 3 and more groups), on groups whose amax is zero or one
isolated value, at the 48-expert layer's full w13 and w2 sizes, and over repeated calls that
alternate shapes through one workspace (the cross-workgroup words of one call must never be
taken for another's). Modes and shapes it does not take fall back to the two reads."""
import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
FLAG_OFFSET = 4 * 512 * 4          # the workspace's flag word (set if a wait was ever abandoned)


@pytest.fixture(scope="module")
def P():
    import precision_moe_numerics_amd as P
    return P


@pytest.fixture(scope="module")
def I():
    from precision_moe_numerics_amd import inputs as I
    return I


@pytest.fixture(scope="module")
def ws(P):
    return torch.zeros((P.nvfp4_quantize_ws_size(),), dtype=torch.uint8, device=DEV)


def npy(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def flag(ws):
    torch.cuda.synchronize()
    return int(ws[FLAG_OFFSET:FLAG_OFFSET + 4].view(torch.int32).item())


def identical(a, b):
    return (torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
            and torch.equal(a.outer.view(torch.int32), b.outer.view(torch.int32)))


@pytest.mark.parametrize("G,rpo,cols", [(1, 16, 256), (2, 32, 512), (3, 16, 1024), (5, 96, 1024), (8, 64, 2048)])
def test_one_read_matches_oracle(P, I, ws, G, rpo, cols):
    x = I.normal((G * rpo, cols), 0.02, 41 + G)
    if G >= 2:
        x[rpo:2 * rpo] = 0                                   # a group of zeros (outer 1)
    if G >= 3:
        x[2 * rpo:3 * rpo] *= 1e-3
        x[2 * rpo + 5, 17] = 0.5                             # one isolated value sets the amax
    q = P.nvfp4_quantize(x.to(DEV), P.NVFP4_WEIGHT, rows_per_outer=rpo, workspace=ws)
    ref = O.nvfp4_quantize(x, rpo, False)
    assert np.array_equal(npy(q.scales), ref["scales"])
    assert np.array_equal(npy(q.codes), ref["codes"])
    assert np.array_equal(npy(q.outer), ref["outer"])
    assert flag(ws) == 0


def test_one_read_large_groups_with_outlier(P, I, ws):
    """13 groups of 2048 x 7168 (one expert's w1 or w3 each, the largest group the one-read path
    holds on 256 compute units): sampled groups against the oracle, all against the two reads."""
    G, R, Cc = 13, 2048, 7168
    w = I.normal((G * R, Cc), 0.02, 31, DEV)
    w[4 * R + 17, 5] = 0.75
    q = P.nvfp4_quantize(w, P.NVFP4_WEIGHT, rows_per_outer=R, workspace=ws)
    assert identical(q, P.nvfp4_quantize(w, P.NVFP4_WEIGHT, rows_per_outer=R))
    codes, scales, outer = npy(q.codes), npy(q.scales), npy(q.outer)
    for g in (0, 4, 12):
        ref = O.nvfp4_quantize(w[g * R:(g + 1) * R].cpu(), R, False)
        assert np.array_equal(scales[g * R:(g + 1) * R], ref["scales"]), g
        assert np.array_equal(codes[g * R:(g + 1) * R], ref["codes"]), g
        assert outer[g] == ref["outer"][0], g
    assert flag(ws) == 0


def test_one_read_full_layer_weights(P, I, ws):
    """The 48-expert layer's w13 (96 groups of 2048 x 7168) and w2 (48 of 7168 x 2048), as the
    benchmark quantizes them: identical to the two reads."""
    sh = I.EP48
    E, H, F = sh.experts, sh.hidden, sh.ffn
    w13, w2 = I.moe_weights(sh, DEV)
    for x, rpo in ((w13.view(E * 2 * F, H), F), (w2.view(E * H, F), H)):
        assert identical(P.nvfp4_quantize(x, P.NVFP4_WEIGHT, rpo, workspace=ws), P.nvfp4_quantize(x, P.NVFP4_WEIGHT, rpo))
    assert flag(ws) == 0


def test_one_read_repeated_calls_alternate_shapes(P, I, ws):
    shapes = [(64, 256, 16), (16, 256, 16), (32, 256, 16), (4096, 1024, 512), (16, 256, 16)]
    xs = [I.normal((r, c), 0.01 * (1 + i), 60 + i, DEV) for i, (r, c, _) in enumerate(shapes)]
    refs = [P.nvfp4_quantize(x, P.NVFP4_WEIGHT, rpo) for x, (_, _, rpo) in zip(xs, shapes)]
    for _ in range(10):
        for x, (_, _, rpo), ref in zip(xs, shapes, refs):
            assert identical(P.nvfp4_quantize(x, P.NVFP4_WEIGHT, rpo, workspace=ws), ref)
    assert flag(ws) == 0


def test_workspace_calls_of_the_other_modes_and_shapes(P, I, ws):
    """Activations (4/6), 16 x 16 blocks, caller-given outer scales and a group larger than the
    one-read path holds (4096 x 7168) take the two reads: the same outputs as nvfp4_quantize."""
    x = I.normal((256, 512), 1.0, 71, DEV)
    assert identical(P.nvfp4_quantize(x, P.NVFP4_ACT, workspace=ws), P.nvfp4_quantize(x, P.NVFP4_ACT))
    assert identical(P.nvfp4_quantize(x, P.NVFP4_WEIGHT_2D, 128, workspace=ws), P.nvfp4_quantize(x, P.NVFP4_WEIGHT_2D, 128))
    o = torch.tensor([0.5, 2.0], device=DEV)
    assert identical(P.nvfp4_quantize(x, P.NVFP4_WEIGHT, 128, outer_in=o, workspace=ws),
                     P.nvfp4_quantize(x, P.NVFP4_WEIGHT, 128, outer_in=o))
    big = I.normal((2 * 4096, 7168), 0.02, 72, DEV)
    assert identical(P.nvfp4_quantize(big, P.NVFP4_WEIGHT, 4096, workspace=ws), P.nvfp4_quantize(big, P.NVFP4_WEIGHT, 4096))


def test_captured_call_takes_the_two_reads(P, I, ws):
    """Under stream capture the call takes the two reads (a replayed graph would not guarantee the
    co-residency of a cooperative launch). Each replay, with eager work between replays, gives
    the eager outputs."""
    x = I.normal((4 * 256, 512), 0.02, 81, DEV)
    ref = P.nvfp4_quantize(x, P.NVFP4_WEIGHT, 256)
    out = P.nvfp4_quantize(x, P.NVFP4_WEIGHT, 256)          # buffers the graph writes into
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                           # warm-up before capture
        P.nvfp4_quantize(x, P.NVFP4_WEIGHT, 256, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.nvfp4_quantize(x, P.NVFP4_WEIGHT, 256, out=out, workspace=ws)
    for i in range(3):
        out.codes.zero_()
        out.scales.zero_()
        out.outer.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert identical(out, ref), i
        P.nvfp4_quantize(x, P.NVFP4_ACT)                    # eager work between replays
