"""Seeded synthetic inputs for the quantized MoE expert layer.

This module holds none of the method's arithmetic. It only draws the tensors that the HIP
path, the CPU oracle and the benchmark all consume: bf16 activations and weights with the
stated distributions, router logits, Zipf-skewed expert loads, RHT sign masks and RNG seeds.

Workloads (all synthetic; the pages measure on no dataset):
  single_expert   X bf16 [256 x 512] ~ N(0,1) with two seeded rows scaled by 50 (outlier rows,
                  as in the transpose discussion of the AREX article's section "转置打散分组,
                  随机舍入保住期望值"); W bf16 read as [K=512 x N=1024] ~ N(0, 0.02), stored
                  transposed [N x K] for the NT product Y = X W.
  quantizer       X bf16 [8192 x 7168] = 0.5 * StudentT(nu=3).
  moe32           T = 16384 tokens, H = 4096, F = 1536, 32 experts, top-8 of softmax(N(0,1)
                  logits); X ~ N(0,1); w1, w3 [F x H], w2 [H x F] ~ N(0, 0.02); dY ~ N(0, 1e-3).
  ep48            48 local experts, 65536 routed slots with Zipf(s = 1.1) loads, H = 7168,
                  F = 2048; X_recv ~ StudentT(nu=4); W ~ N(0, 0.02); dY ~ N(0, 1e-3).
  combine         the receive side on moe32's routing: 131072 slot rows of S2F6 codes [x 4096]
                  with one E8M0 byte per 32 codes, gathered back to 16384 tokens by top-8 gates.
Student-t samples are drawn as Z / sqrt(V / nu) with V a sum of nu squared normals.
S2F6 payload rows (the w2 outputs after the 32-point transform) are drawn directly as codes:
c = clamp(round(32 N(0,1)), -127, 127), so a 32-chunk's largest |c| is typically 60..110, near the
top of the code range as the E8M0 rule places it; E8M0 = 123 + round(2 N(0,1)) per row +
round(N(0,1)) per chunk, clamped to [100, 150] (values of order 2^-4, spread over rows and chunks).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std: float, seed: int, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    g = _gen(seed, device)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(dtype)


def student_t(shape, nu: int, scale: float, seed: int, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    g = _gen(seed, device)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(nu):
        n = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        v.addcmul_(n, n)
    z.div_(torch.sqrt(v / nu)).mul_(scale)
    return z.to(dtype)


def sign_mask(seed: int) -> int:
    """32 random sign bits for the randomized Hadamard transform (one mask for every chunk)."""
    g = _gen(seed, "cpu")
    return int(torch.randint(0, 2**32, (1,), generator=g, dtype=torch.int64).item())


def zipf_counts(total: int, experts: int, s: float) -> list:
    """Deterministic Zipf(s) expert loads: largest-remainder rounding of total * k^-s / H."""
    w = [k ** (-s) for k in range(1, experts + 1)]
    h = sum(w)
    raw = [total * x / h for x in w]
    base = [math.floor(r) for r in raw]
    rest = total - sum(base)
    order = sorted(range(experts), key=lambda i: (-(raw[i] - base[i]), i))
    for i in order[:rest]:
        base[i] += 1
    return base


def offsets_from_counts(counts, device="cpu") -> torch.Tensor:
    o = [0]
    for c in counts:
        o.append(o[-1] + int(c))
    return torch.tensor(o, dtype=torch.int64, device=device)


def single_expert(device="cpu"):
    """X [256 x 512] with two outlier rows, W^T [1024 x 512] (NT layout of W [512 x 1024])."""
    x = normal((256, 512), 1.0, 100, device)
    rows = torch.randperm(256, generator=_gen(102, "cpu"))[:2].tolist()
    xf = x.float()
    for r in rows:
        xf[r] *= 50.0
    x = xf.to(torch.bfloat16)
    w = normal((512, 1024), 0.02, 101, device)
    return dict(x=x, w_t=w.t().contiguous(), outlier_rows=rows, seed=0)


def quantizer(device="cpu", rows=8192, cols=7168):
    return dict(x=student_t((rows, cols), 3, 0.5, 200, device), seed=1, stream=0)


@dataclass
class MoEShape:
    name: str
    experts: int
    hidden: int
    ffn: int
    tokens: int = 0          # tokens before routing (0: slots arrive already grouped)
    top_k: int = 8
    slots: int = 0           # routed slots when the loads are given directly
    zipf_s: float = 0.0
    x_nu: int = 0            # 0: N(0,1) activations, else Student-t dof
    seeds: dict = field(default_factory=dict)


MOE32 = MoEShape("moe32", experts=32, hidden=4096, ffn=1536, tokens=16384, top_k=8,
                 seeds=dict(x=300, w=301, logits=302, dy=400, sr=2, rht=3, payload=303))
EP48 = MoEShape("ep48", experts=48, hidden=7168, ffn=2048, slots=65536, zipf_s=1.1, x_nu=4,
                seeds=dict(x=500, w=501, dy=502, sr=5, rht=3))


def moe_weights(shape: MoEShape, device="cpu", experts=None):
    """w13 [E x 2F x H] (rows 0..F-1 = w1, F..2F-1 = w3) and w2 [E x H x F], ~N(0, 0.02)."""
    E = shape.experts if experts is None else experts
    F, H = shape.ffn, shape.hidden
    w13 = normal((E, 2 * F, H), 0.02, shape.seeds["w"], device)
    w2 = normal((E, H, F), 0.02, shape.seeds["w"] + 1000, device)
    return w13, w2


def moe_activations(shape: MoEShape, device="cpu", rows=None):
    """Token activations: X [T x H] for routed shapes, X_recv [slots x H] for grouped ones."""
    n = rows if rows is not None else (shape.tokens if shape.tokens else shape.slots)
    if shape.x_nu:
        return student_t((n, shape.hidden), shape.x_nu, 1.0, shape.seeds["x"], device)
    return normal((n, shape.hidden), 1.0, shape.seeds["x"], device)


def moe_logits(shape: MoEShape, device="cpu", tokens=None):
    T = shape.tokens if tokens is None else tokens
    g = _gen(shape.seeds["logits"], device)
    return torch.randn((T, shape.experts), generator=g, device=device, dtype=torch.float32)


def moe_loads(shape: MoEShape):
    return zipf_counts(shape.slots, shape.experts, shape.zipf_s)


def moe_grad(shape: MoEShape, slots: int, device="cpu"):
    return normal((slots, shape.hidden), 1e-3, shape.seeds["dy"], device)


def s2f6_payload(rows: int, hidden: int, seed: int, device="cpu"):
    """int8 codes [rows x hidden] and uint8 E8M0 [rows x hidden/32] of S2F6 payload rows."""
    g = _gen(seed, device)
    codes = torch.randn((rows, hidden), generator=g, device=device, dtype=torch.float32).mul_(32.0).round_()
    codes = codes.clamp_(-127, 127).to(torch.int8)
    row = torch.randn((rows, 1), generator=g, device=device, dtype=torch.float32).mul_(2.0).round_()
    chunk = torch.randn((rows, hidden // 32), generator=g, device=device, dtype=torch.float32).round_()
    e8m0 = (123.0 + row + chunk).clamp_(100, 150).to(torch.uint8)
    return codes, e8m0
