"""Parity of the combine's receiver side (moe_combine_s2f6) with the CPU oracle.

The HIP kernel sums a token's k slots on the scaled codes in fp32 and transforms once; the oracle
decodes every slot in fp64 and sums. The tolerance follows from that arithmetic, per output value
of a token t and 32-chunk: with S = sum_i |g_i| 2^(e_i - 138), every fp32 intermediate is at most
32 * 127 * S = 4064 S in magnitude, the k fmas and five butterfly stages add at most (k + 5) unit
roundings (2^-24) of it, and the bf16 store rounds once more (at most 2^-8 of the value):
    |got - ref| <= E + 2^-8 (|ref| + E),   E = 1.01 (k + 5) 4064 2^-24 S
plus an absolute 2^-133 (half a bf16 subnormal step) and, where a gate times 2^(e - 138) falls
below the fp32 normal range, k 4064 2^-149 for its rounding. A wrong sign, slot, gate or scale
moves values by O(|ref|), far outside this. The GEMM bar (relative Frobenius error <= 2e-3) is
checked as well.
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


def check(got_bf16, codes, e8m0, mask, slot_of, gates):
    """Compare a bf16 combine output with the oracle at the bound stated above."""
    so = np.asarray(slot_of, np.int32)
    g = np.asarray(gates, np.float32)
    T, k = g.shape
    ref = O.moe_combine_s2f6(codes, e8m0, mask, so, g)
    got = got_bf16.float().cpu().numpy().astype(np.float64)
    e = np.asarray(e8m0, np.float64)[so]                                          # [T, k, H/32]
    S = (np.abs(g.astype(np.float64))[..., None] * 2.0 ** (e - 138)).sum(1)        # [T, H/32]
    E = np.repeat(1.01 * (k + 5) * 4064 * 2.0 ** -24 * S, 32, axis=1)
    bound = E + 2.0 ** -8 * (np.abs(ref) + E) + 2.0 ** -133 + k * 4064 * 2.0 ** -149
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{bad.sum()} values outside the bound, first at {np.argwhere(bad)[0]}"
    nr = np.linalg.norm(ref)
    if nr > 0:
        assert np.linalg.norm(got - ref) / nr <= 2e-3
    return ref


def payload(M, H, seed):
    from precision_moe_numerics_amd import inputs as I
    c, e = I.s2f6_payload(M, H, seed)
    return c.numpy(), e.numpy()


def routes(T, k, M, seed, dup=False):
    """slot_of [T x k] (a permutation of the M = T k slots, or with repeats) and gates [T x k]."""
    rng = np.random.default_rng(seed)
    so = rng.permutation(M)[: T * k] if not dup else rng.integers(0, M, T * k)
    gates = rng.dirichlet(np.ones(k), T).astype(np.float32)
    return so.astype(np.int32).reshape(T, k), gates


def run(P, codes, e8m0, mask, so, gates):
    return P.moe_combine_s2f6(torch.as_tensor(codes, device=DEV), torch.as_tensor(e8m0, device=DEV), mask,
                              torch.as_tensor(so, device=DEV), torch.as_tensor(gates, device=DEV))


@pytest.mark.parametrize("T,k,H", [(37, 3, 96), (130, 8, 256), (9, 11, 64), (5, 1, 32), (64, 16, 128),
                                   (300, 8, 4096), (3, 64, 224)])
def test_combine_vs_oracle(T, k, H):
    """Several workgroups and a ragged last one (T H / 32 not a multiple of 256), k below, at and
    above the 8-slot batch (tails 1..7 and two full batches), H from one chunk to 128."""
    import precision_moe_numerics_amd as P
    M = T * k
    codes, e8m0 = payload(M, H, 1000 + T + k)
    mask = 0x9E3779B9 ^ (T * 7919)
    so, gates = routes(T, k, M, T * 31 + k)
    out = run(P, codes, e8m0, mask, so, gates)
    check(out, codes, e8m0, mask & 0xFFFFFFFF, so, gates)


def test_combine_repeated_slots_and_unnormalized_gates():
    """Slots read by several tokens (and twice by one token), gates that do not sum to one."""
    import precision_moe_numerics_amd as P
    T, k, H, M = 50, 6, 160, 40
    codes, e8m0 = payload(M, H, 77)
    so, gates = routes(T, k, M, 78, dup=True)
    so[0, 1] = so[0, 0]
    gates = (gates * np.linspace(0.1, 3.0, T, dtype=np.float32)[:, None]).astype(np.float32)
    out = run(P, codes, e8m0, 0x0F0F1234, so, gates)
    check(out, codes, e8m0, 0x0F0F1234, so, gates)


def test_combine_k1_is_the_decode():
    """k = 1 with gate 1: each output row is the exact inverse transform of its slot, rounded once."""
    import precision_moe_numerics_amd as P
    T, H = 200, 512
    codes, e8m0 = payload(T, H, 5)
    so = np.random.default_rng(6).permutation(T).astype(np.int32).reshape(T, 1)
    ones = np.ones((T, 1), np.float32)
    out = run(P, codes, e8m0, 0xDEADBEEF, so, ones)
    dec = O.rht32_s2f6_decode(codes, e8m0, 0xDEADBEEF)[so[:, 0]]
    check(out, codes, e8m0, 0xDEADBEEF, so, ones)
    # a single slot has exact fp32 intermediates, so only the bf16 rounding remains
    ref_bf16 = torch.from_numpy(dec.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(out.cpu(), ref_bf16)


def test_combine_out_of_range_slots_add_nothing():
    import precision_moe_numerics_amd as P
    T, k, H = 40, 5, 128
    M = T * k
    codes, e8m0 = payload(M, H, 9)
    so, gates = routes(T, k, M, 10)
    so[0, 0], so[3, 4], so[7, 2], so[39, 1] = -1, M, 2**31 - 1, -(2**31)
    out = run(P, codes, e8m0, 0x12345678, so, gates)
    ok = (so >= 0) & (so < M)
    check(out, codes, e8m0, 0x12345678, np.where(ok, so, 0), np.where(ok, gates, 0.0).astype(np.float32))


def test_combine_extreme_scales():
    """E8M0 from 0 (gate x 2^-138 below the normal range) to 230 (values near 2^100)."""
    import precision_moe_numerics_amd as P
    T, k, H = 16, 4, 128
    M = T * k
    codes, _ = payload(M, H, 11)
    e8m0 = np.random.default_rng(12).choice(np.array([0, 1, 11, 12, 60, 127, 200, 230], np.uint8), (M, H // 32))
    so, gates = routes(T, k, M, 13)
    out = run(P, codes, e8m0, 0xFFFFFFFF, so, gates)
    check(out, codes, e8m0, 0xFFFFFFFF, so, gates)


def test_combine_empty_and_degenerate():
    import precision_moe_numerics_amd as P
    H = 64
    codes, e8m0 = payload(8, H, 14)
    # no tokens: nothing launched, empty output
    out = P.moe_combine_s2f6(torch.as_tensor(codes, device=DEV), torch.as_tensor(e8m0, device=DEV), 0,
                             torch.zeros((0,), dtype=torch.int32, device=DEV),
                             torch.zeros((0, 3), dtype=torch.float32, device=DEV))
    assert out.shape == (0, H)
    # no slots (M = 0): every route is out of range, the output is zero
    so = torch.zeros((4, 2), dtype=torch.int32, device=DEV)
    g = torch.ones((4, 2), dtype=torch.float32, device=DEV)
    out = P.moe_combine_s2f6(torch.zeros((0, H), dtype=torch.int8, device=DEV),
                             torch.zeros((0, H // 32), dtype=torch.uint8, device=DEV), 0, so, g)
    assert torch.count_nonzero(out).item() == 0
    # all-zero codes decode to zero whatever the scale
    z = np.zeros_like(codes)
    out = run(P, z, e8m0, 0xFFFFFFFF, np.arange(8, dtype=np.int32).reshape(4, 2), np.ones((4, 2), np.float32))
    assert torch.count_nonzero(out).item() == 0


def test_combine_argument_errors():
    import precision_moe_numerics_amd as P
    lib = P._lib
    c = torch.zeros((4, 64), dtype=torch.int8, device=DEV)
    e = torch.zeros((4, 2), dtype=torch.uint8, device=DEV)
    so = torch.zeros((4,), dtype=torch.int32, device=DEV)
    g = torch.ones((4,), dtype=torch.float32, device=DEV)
    out = torch.empty((4 * 64 + 8,), dtype=torch.bfloat16, device=DEV)
    p = lambda t: t.data_ptr()
    s = P._stream()
    assert lib.moe_combine_s2f6(p(c), p(e), 4, 48, 0, p(so), p(g), 4, 1, p(out), s) == -2     # H % 32
    assert lib.moe_combine_s2f6(p(c), p(e), 4, 64, 0, p(so), p(g), 4, 0, p(out), s) == -2     # k = 0
    assert lib.moe_combine_s2f6(p(c), p(e), 4, 64, 0, p(so), p(g), 1, 65, p(out), s) == -2    # k > 64
    assert lib.moe_combine_s2f6(p(c), p(e), 4, 64, 0, None, p(g), 4, 1, p(out), s) == -1      # null
    assert lib.moe_combine_s2f6(p(c), p(e), 4, 64, 0, p(so), p(g), 4, 1, p(out) + 2, s) == -3  # alignment
    assert lib.moe_combine_s2f6(p(c) + 8, p(e), 4, 64, 0, p(so), p(g), 4, 1, p(out), s) == -3


def test_combine_full_size_sampled():
    """16384 tokens, top-8 of 32 experts (routing of the oracle on the seeded logits), 131072 slot
    rows of hidden 4096 -- the launch the benchmark times; sampled tokens, all their values."""
    import precision_moe_numerics_amd as P
    from precision_moe_numerics_amd import inputs as I
    sh = I.MOE32
    T, k, H = sh.tokens, sh.top_k, sh.hidden
    r = O.route_topk(I.moe_logits(sh, "cpu").numpy(), k)
    so, gates = r["slot_of"].reshape(T, k), r["gates"]
    codes_d, e_d = I.s2f6_payload(T * k, H, sh.seeds["payload"], DEV)
    mask = I.sign_mask(sh.seeds["rht"])
    out = P.moe_combine_s2f6(codes_d, e_d, mask, torch.as_tensor(so, device=DEV), torch.as_tensor(gates, device=DEV))
    again = P.moe_combine_s2f6(codes_d, e_d, mask, torch.as_tensor(so, device=DEV), torch.as_tensor(gates, device=DEV))
    assert torch.equal(out, again)                                   # deterministic
    rng = np.random.default_rng(14)
    toks = np.concatenate([[0, 1, T - 1], rng.integers(0, T, 45)])
    check(out[torch.as_tensor(toks, device=DEV)], npy(codes_d), npy(e_d), mask, so[toks], gates[toks])
