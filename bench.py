"""Benchmark of the quantized MoE expert layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input, by default the
one-GPU expert share (48 local experts, 65536 routed slots with Zipf(1.1) loads, hidden 7168,
FFN 2048, SwiGLU):
  weights:  NVFP4 quantization of w13 and w2 (one outer scale per expert and matrix)
  forward:  NVFP4 quantization of X (per-token outer scale, 4/6) -> grouped GEMM w13 with the
            SwiGLU epilogue (h13 saved) -> NVFP4 quantization of A -> grouped GEMM w2 with the
            fused RHT32 + S2F6 epilogue (the combine payload)
  backward: w2 backward (dY MXFP8 row/column quantization, SR requantization of W2^T and A^T,
            MXFP8 dgrad and wgrad) -> SwiGLU backward -> w13 backward (same steps with X^T, W13^T)
Inputs are generated on the GPU from fixed seeds before the timed region and stay resident in
HBM. Per-call device time comes from HIP events on the stream the kernels run on.

Also reported: the memory-bound quantizer workload (8192 x 7168 activations, 0.5 * StudentT(3)):
nvfp4_quantize with 4/6 and requant_transpose_sr_mxfp8 of its output, each timed over rotating
input buffers larger than the 256 MB Infinity Cache, as GB/s of algorithmic bytes.

Also reported: the MXFP8 forward of the layers that keep MXFP8, on the same layer shape (w13 with
SwiGLU, w2 with RHT32 + S2F6, each call including its MXFP8 quantization), as TFLOP/s.

Also reported: the FP4 backward variant on the same layer (every backward operand in MXFP4, the
GEMMs on the block-scaled FP4 MFMA), as TFLOP/s.

Also reported: the receiver side of the combine (moe_combine_s2f6) on the routed shape, 16384
tokens with top-8 of 32 experts gathered back from 131072 S2F6 rows of hidden 4096, as GB/s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ep48|moe32]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4/MXFP8-SR quantize GB/s + MoE grouped GEMM TFLOPS, % of MI355X roofline"
PEAK_HBM_GBS = 8000.0          # MI355X published HBM3E bandwidth
PEAK_F16_TFLOPS = 2500.0       # MI355X dense MFMA fp16/bf16
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense MFMA fp8
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MFMA fp4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ep48", choices=["ep48", "moe32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quant-iters", type=int, default=20)
    return ap.parse_args()


class Timer:
    """HIP events around each ABI call on torch's current stream (the calls' stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.events = []

    def run(self, name, fn, *a, **k):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        r = fn(*a, **k)
        e1.record()
        self.events.append((name, e0, e1))
        return r

    def collect(self):
        out = {}
        for name, e0, e1 in self.events:
            ms = e0.elapsed_time(e1)
            s = out.setdefault(name, [0.0, 0])
            s[0] += ms
            s[1] += 1
        self.events = []
        return {k: v[0] / v[1] for k, v in out.items()}


class Layer:
    def __init__(self, P, I, torch, shape, dev):
        self.P, self.torch = P, torch
        self.shape = shape
        E, H, F = shape.experts, shape.hidden, shape.ffn
        self.E, self.H, self.F = E, H, F
        if shape.tokens:        # routed workload: route on the device, activations gathered
            logits = I.moe_logits(shape, dev)
            r = P.moe_route_topk(logits, shape.top_k)
            torch.cuda.synchronize()
            self.offsets = r["offsets"]
            self.gather = r["gather"]
            self.M = shape.tokens * shape.top_k
            self.x = I.moe_activations(shape, dev)
        else:
            counts = I.moe_loads(shape)
            self.offsets = I.offsets_from_counts(counts, dev)
            self.gather = None
            self.M = sum(counts)
            self.x = I.moe_activations(shape, dev)
        w13, w2 = I.moe_weights(shape, dev)
        self.w13 = w13.view(E * 2 * F, H)
        self.w2 = w2.view(E * H, F)
        self.dy = I.moe_grad(shape, self.M, dev)
        self.mask = I.sign_mask(shape.seeds["rht"])
        self.seed = shape.seeds["sr"]
        M = self.M
        # one workspace per matrix, large enough for the MXFP8 and the FP4 backward layouts
        def ws(N, K):
            n = max(P.moe_grouped_gemm_bwd_workspace_size(M, E, N, K, f) for f in (3, 3 | P.BWD_FP4))
            return torch.empty(n, dtype=torch.uint8, device=dev)
        self.ws13 = ws(2 * F, H)
        self.ws2 = ws(H, F)
        torch.cuda.synchronize()

    def flops(self):
        M, H, F = self.M, self.H, self.F
        fwd13 = 2.0 * M * 2 * F * H
        fwd2 = 2.0 * M * H * F
        return dict(fwd13=fwd13, fwd2=fwd2, fwd=fwd13 + fwd2, bwd=2 * (fwd13 + fwd2), step=3 * (fwd13 + fwd2))

    def step(self, T):
        P = self.P
        E, H, F, M = self.E, self.H, self.F, self.M
        w13q = T.run("nvfp4_quantize[w13]", P.nvfp4_quantize, self.w13, P.NVFP4_WEIGHT, F)
        w2q = T.run("nvfp4_quantize[w2]", P.nvfp4_quantize, self.w2, P.NVFP4_WEIGHT, H)
        xq = T.run("nvfp4_quantize[x]", P.nvfp4_quantize, self.x, P.NVFP4_ACT)
        a, h13 = T.run("moe_grouped_gemm_fwd[w13+swiglu]", P.moe_grouped_gemm_fwd, xq, w13q, self.offsets, M, 2 * F,
                       P.EPI_SWIGLU, gather=self.gather, save_h13=True)
        aq = T.run("nvfp4_quantize[a]", P.nvfp4_quantize, a, P.NVFP4_ACT)
        yc, ye = T.run("moe_grouped_gemm_fwd[w2+rht32_s2f6]", P.moe_grouped_gemm_fwd, aq, w2q, self.offsets, M, H,
                       P.EPI_RHT32_S2F6, rht_sign_mask=self.mask)
        da, dw2, _ = T.run("moe_grouped_gemm_bwd[w2]", P.moe_grouped_gemm_bwd, self.dy, aq, w2q, self.offsets, M, H,
                           seed=self.seed, rng_stream_a=5, rng_stream_b=3, rng_stream_dy=6, workspace=self.ws2)
        dh13 = T.run("swiglu_bwd", P.swiglu_bwd, da, h13)
        dx, dw13, _ = T.run("moe_grouped_gemm_bwd[w13]", P.moe_grouped_gemm_bwd, dh13, xq, w13q, self.offsets, M,
                            2 * F, gather=self.gather, seed=self.seed, rng_stream_a=4, rng_stream_b=1,
                            rng_stream_dy=8, workspace=self.ws13)
        return yc, dx, dw13, dw2


def quantizer_workload(P, I, torch, dev, iters):
    """GB/s of nvfp4_quantize (4/6, per-token outer) and requant_transpose_sr_mxfp8 on the
    8192 x 7168 activation workload, rotating inputs so the Infinity Cache cannot serve them."""
    R, Cc = 8192, 7168
    base = I.quantizer(dev)
    nbuf = 4
    xs = [base["x"]] + [base["x"].roll(shifts=97 * i, dims=1).contiguous() for i in range(1, nbuf)]
    qs = [P.nvfp4_quantize(x, P.NVFP4_ACT) for x in xs]
    nq = 12
    qs = [qs[i % nbuf] for i in range(nq)]
    qbuf = []
    for i in range(nq):     # distinct copies of the quantized tensors (> 256 MB in total)
        q = qs[i]
        qbuf.append(P.NVFP4(q.codes.clone(), q.scales.clone(), q.outer.clone(), q.rows_per_outer))
    ld = P.padded_bound(R, 0)
    out = torch.empty((Cc, ld), dtype=torch.uint8, device=dev)
    oe = torch.empty((Cc, ld // 32), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    res = {}
    # nvfp4_quantize
    for i in range(3):
        P.nvfp4_quantize(xs[i % nbuf], P.NVFP4_ACT)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(iters):
        P.nvfp4_quantize(xs[i % nbuf], P.NVFP4_ACT)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = R * Cc * (2 + 0.5 + 1 / 16) + R * 4
    res["nvfp4_quantize"] = dict(us=ms * 1e3, bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9)
    # requant
    def rq(q):
        P.requant_transpose_sr_mxfp8(q, seed=base["seed"], rng_stream=base["stream"], ld=ld, out=out, out_e8m0=oe)

    for i in range(3):
        rq(qbuf[i])
    torch.cuda.synchronize()
    e0.record()
    for i in range(iters):
        rq(qbuf[i % nq])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = R * Cc * (0.5 + 1 / 16 + 1 + 1 / 32) + R * 4
    res["requant_transpose_sr_mxfp8"] = dict(us=ms * 1e3, bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9)
    # measured copy bandwidth (device-to-device copy of 1 GiB, read + write)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    res["hbm_copy_gbs"] = 2 * (1 << 30) / (ms * 1e-3) / 1e9
    del src, dst
    return res


def combine_workload(P, I, torch, dev, iters):
    """GB/s of moe_combine_s2f6 on the routed shape (16384 tokens, top-8 of 32 experts, 131072 slot
    rows of hidden 4096): routing on the device from the seeded logits, two S2F6 payloads of
    553 MB each used in turn so the Infinity Cache cannot serve them."""
    sh = I.MOE32
    T, k, H = sh.tokens, sh.top_k, sh.hidden
    M = T * k
    r = P.moe_route_topk(I.moe_logits(sh, dev), k)
    so, gates = r["slot_of"], r["gates"]
    mask = I.sign_mask(sh.seeds["rht"])
    pay = [I.s2f6_payload(M, H, sh.seeds["payload"] + i, dev) for i in range(2)]
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for i in range(3):
        P.moe_combine_s2f6(*pay[i % 2], mask, so, gates, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(iters):
        P.moe_combine_s2f6(*pay[i % 2], mask, so, gates, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    # per token: k rows of H codes + H/32 E8M0 bytes, k slot indices and gates; H bf16 out
    nbytes = T * (k * (H + H // 32) + 8 * k + 2 * H)
    del pay
    return dict(us=ms * 1e3, bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9, tokens=T, top_k=k, hidden=H,
                slots=M, frac_of_8TBs=nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS)


def mxfp8_forward_workload(P, I, torch, layer, iters):
    """The MXFP8 forward of the layers that keep MXFP8, on the same layer shape: w13 with the
    SwiGLU epilogue and w2 with the RHT32 + S2F6 epilogue, each call including the row-wise MXFP8
    quantization of its activations and weights. TFLOP/s of the GEMMs against the fp8 peak."""
    M, E, H, F = layer.M, layer.E, layer.H, layer.F
    A = I.student_t((M, F), 4, 0.05, 611, layer.x.device)
    ws13 = torch.empty((P._lib.moe_grouped_gemm_fwd_mxfp8_workspace_size(M, E, 2 * F, H),), dtype=torch.uint8,
                       device=A.device)
    ws2 = torch.empty((P._lib.moe_grouped_gemm_fwd_mxfp8_workspace_size(M, E, H, F),), dtype=torch.uint8,
                      device=A.device)
    a_out = torch.empty((M, F), dtype=torch.bfloat16, device=A.device)
    h13 = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=A.device)
    c = torch.empty((M, H), dtype=torch.int8, device=A.device)
    ce = torch.empty((M, H // 32), dtype=torch.uint8, device=A.device)

    def w13():
        P.moe_grouped_gemm_fwd_mxfp8(layer.x, layer.w13, layer.offsets, M, 2 * F, P.EPI_SWIGLU, gather=layer.gather,
                                     workspace=ws13, out=a_out, out_aux=h13)

    def w2():
        P.moe_grouped_gemm_fwd_mxfp8(A, layer.w2, layer.offsets, M, H, P.EPI_RHT32_S2F6, rht_sign_mask=layer.mask,
                                     workspace=ws2, out=c, out_e8m0=ce)
    res = {}
    for name, fn, flops in (("w13+swiglu", w13, 2.0 * M * 2 * F * H), ("w2+rht32_s2f6", w2, 2.0 * M * H * F)):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        t = flops / (ms * 1e-3) / 1e12
        res[name] = dict(ms_incl_quant=ms, tflops_incl_quant=t, frac_fp8_peak=t / PEAK_FP8_TFLOPS)
    del ws13, ws2, A
    return res


def fp4_backward_workload(P, torch, layer, iters):
    """The FP4 backward variant on the same layer: w2 and w13 backward with every operand in MXFP4
    (E2M1 + E8M0/32, SR) and the GEMMs on the block-scaled FP4 MFMA, each call including its
    quantization and requantization. TFLOP/s of the GEMM work against the FP4 peak."""
    M, H, F = layer.M, layer.H, layer.F
    w13q = P.nvfp4_quantize(layer.w13, P.NVFP4_WEIGHT, F)
    w2q = P.nvfp4_quantize(layer.w2, P.NVFP4_WEIGHT, H)
    xq = P.nvfp4_quantize(layer.x, P.NVFP4_ACT)
    a, h13 = P.moe_grouped_gemm_fwd(xq, w13q, layer.offsets, M, 2 * F, P.EPI_SWIGLU, gather=layer.gather,
                                     save_h13=True)
    aq = P.nvfp4_quantize(a, P.NVFP4_ACT)
    dh13 = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=a.device).normal_(0, 1e-3)
    flags = P.BWD_DGRAD | P.BWD_WGRAD | P.BWD_FP4

    def w2():
        P.moe_grouped_gemm_bwd(layer.dy, aq, w2q, layer.offsets, M, H, flags=flags, seed=layer.seed, rng_stream_a=5,
                                rng_stream_b=3, rng_stream_dy=6, workspace=layer.ws2)

    def w13():
        P.moe_grouped_gemm_bwd(dh13, xq, w13q, layer.offsets, M, 2 * F, flags=flags, gather=layer.gather,
                                seed=layer.seed, rng_stream_a=4, rng_stream_b=1, rng_stream_dy=8, workspace=layer.ws13)
    res = {}
    fl = layer.flops()
    for name, fn, flops in (("w2", w2, 2 * fl["fwd2"]), ("w13", w13, 2 * fl["fwd13"])):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        t = flops / (ms * 1e-3) / 1e12
        res[name] = dict(ms_incl_quant=ms, tflops_incl_quant=t, frac_fp4_peak=t / PEAK_FP4_TFLOPS)
    return res


def cpu_baseline(I, shape):
    """The CPU oracle (as it stands) on a bounded sample of the same step: 16 slots of one expert
    through the whole layer, forward and backward. Returns TFLOP/s of that sample."""
    import numpy as np
    import torch

    import oracle as O
    S, H, F = 16, shape.hidden, shape.ffn
    x = I.moe_activations(shape, "cpu", rows=S)
    w13 = I.normal((2 * F, H), 0.02, shape.seeds["w"])
    w2 = I.normal((H, F), 0.02, shape.seeds["w"] + 1000)
    dy = I.moe_grad(shape, S, "cpu")
    mask = I.sign_mask(shape.seeds["rht"])
    off = [0, S]
    t0 = time.perf_counter()
    xq = O.nvfp4_quantize(x, 1, True)
    w13q = O.nvfp4_quantize(w13, F, False)
    w2q = O.nvfp4_quantize(w2, H, False)
    h13 = O.gemm_nvfp4_grouped(xq, w13q, off, 2 * F, H)
    a = torch.from_numpy(O.swiglu(h13, F)).to(torch.bfloat16)
    aq = O.nvfp4_quantize(a, 1, True)
    y = O.gemm_nvfp4_grouped(aq, w2q, off, H, F)
    O.rht32_s2f6_quantize(y, mask)
    dq, de = O.mxfp8_quantize_rows(dy)
    w2t, w2te = O.requant_transpose_sr(w2q, seed=5, stream=3)
    da = O.gemm_mxfp8_dgrad(dq, de, w2t, w2te, off, H, F)
    dt, dte = O.mxfp8_quantize_cols(dy, offsets=off)
    at, ate = O.requant_transpose_sr(aq, offsets=off, seed=5, stream=5)
    O.gemm_mxfp8_wgrad(dt, dte, at, ate, off, H, F)
    h13b = torch.from_numpy(h13).to(torch.bfloat16)
    dh = torch.from_numpy(O.swiglu_bwd(da, h13b, F)).to(torch.bfloat16)
    gq, ge = O.mxfp8_quantize_rows(dh)
    w13t, w13te = O.requant_transpose_sr(w13q, seed=5, stream=1)
    O.gemm_mxfp8_dgrad(gq, ge, w13t, w13te, off, 2 * F, H)
    gt, gte = O.mxfp8_quantize_cols(dh, offsets=off)
    xt, xte = O.requant_transpose_sr(xq, offsets=off, seed=5, stream=4)
    O.gemm_mxfp8_wgrad(gt, gte, xt, xte, off, 2 * F, H)
    dt_s = time.perf_counter() - t0
    flops = 3 * 2.0 * S * (2 * F * H + H * F)
    return dict(value=flops / dt_s / 1e12, unit="TFLOP/s", cores=O.threads(), kind="oracle", seconds=dt_s,
                sample=f"{S} routed slots of one expert through the whole layer (NVFP4 quantize of X, w13, w2; "
                       f"w13 GEMM + SwiGLU; A quantize; w2 GEMM; RHT32+S2F6; MXFP8 dY quantize; SR requant of "
                       f"W2^T, A^T, W13^T, X^T; dgrad and wgrad of both GEMMs), H={H}, F={F}")


def measured_traffic():
    """HBM bytes per launch of the w13 forward GEMM from the committed PMC profile (FETCH_SIZE and
    WRITE_SIZE runs, scaled by the copy-kernel calibration), or None when the kernel's source has
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_gemm_fwd.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])).hexdigest()
    if h != rec["source_sha256"]:
        return None
    return rec["traffic_bytes_per_launch"]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch

    import precision_moe_numerics_amd as P
    from precision_moe_numerics_amd import inputs as I

    dev = torch.device("cuda:0")
    shape = I.EP48 if args.workload == "ep48" else I.MOE32
    layer = Layer(P, I, torch, shape, dev)
    T = Timer(torch)
    for _ in range(args.warmup):
        layer.step(T)
    torch.cuda.synchronize()
    T.collect()
    t0 = time.perf_counter()
    # one event per step boundary: the first and last bracket the timed region
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        layer.step(T)
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = T.collect()
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    steps_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))

    def pct(q):
        return steps_ms[min(len(steps_ms) - 1, int(round(q * (len(steps_ms) - 1))))]
    fl = layer.flops()
    value = fl["step"] / (ms_step * 1e-3) / 1e12

    k13 = per_call["moe_grouped_gemm_fwd[w13+swiglu]"]
    k2 = per_call["moe_grouped_gemm_fwd[w2+rht32_s2f6]"]
    ach = fl["fwd13"] / (k13 * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "k_nvfp4_grouped_gemm<SWIGLU> (w13 forward, fp16 MFMA after exact "
                                           "NVFP4 dequant)",
                "achieved": ach, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_F16_TFLOPS,
                "traffic": measured_traffic() if args.workload == "ep48" else None,
                "flops_per_launch": fl["fwd13"], "ms_per_launch": k13,
                # the same rate against the FP4-class peak, above this exact path's own roof
                "frac_fp4_class": ach / PEAK_FP4_TFLOPS}
    kernels = {name: {"ms": ms} for name, ms in per_call.items()}
    kernels["moe_grouped_gemm_fwd[w13+swiglu]"].update(tflops=ach, frac_f16_peak=ach / PEAK_F16_TFLOPS)
    a2 = fl["fwd2"] / (k2 * 1e-3) / 1e12
    kernels["moe_grouped_gemm_fwd[w2+rht32_s2f6]"].update(tflops=a2, frac_f16_peak=a2 / PEAK_F16_TFLOPS)
    for nm, f in (("moe_grouped_gemm_bwd[w2]", 2 * fl["fwd2"]), ("moe_grouped_gemm_bwd[w13]", 2 * fl["fwd13"])):
        t = f / (per_call[nm] * 1e-3) / 1e12
        kernels[nm].update(tflops_incl_quant=t, frac_fp8_peak=t / PEAK_FP8_TFLOPS)

    quant = quantizer_workload(P, I, torch, dev, args.quant_iters)
    for k in ("nvfp4_quantize", "requant_transpose_sr_mxfp8"):
        quant[k]["frac_of_8TBs"] = quant[k]["gbs"] / PEAK_HBM_GBS
        quant[k]["frac_of_measured_copy"] = quant[k]["gbs"] / quant["hbm_copy_gbs"]

    # 16 x 16 square-block NVFP4 of the w13 weights, beside the 1D weight mode of the same call
    sq = {}
    for name, mode in (("weight_1d", P.NVFP4_WEIGHT), ("weight_16x16", P.NVFP4_WEIGHT_2D)):
        for _ in range(2):
            P.nvfp4_quantize(layer.w13, mode, layer.F)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            P.nvfp4_quantize(layer.w13, mode, layer.F)
        e1.record()
        torch.cuda.synchronize()
        sq[name] = dict(ms=e0.elapsed_time(e1) / 5)
    mx8 = mxfp8_forward_workload(P, I, torch, layer, max(args.quant_iters // 4, 3))
    fp4b = fp4_backward_workload(P, torch, layer, max(args.quant_iters // 4, 3))
    comb = combine_workload(P, I, torch, dev, args.quant_iters)
    comb["frac_of_measured_copy"] = comb["gbs"] / quant["hbm_copy_gbs"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(I, shape)

    cfg = {"workload": (f"{shape.name}: {shape.experts} local experts, {layer.M} routed slots"
                        + (f" (top-{shape.top_k} of {shape.tokens} tokens)" if shape.tokens else
                           f" with Zipf({shape.zipf_s}) loads")
                        + f", hidden {shape.hidden}, FFN {shape.ffn}, SwiGLU, forward + backward"),
           "experts": shape.experts, "slots": layer.M, "hidden": shape.hidden, "ffn": shape.ffn,
           "step_tflop": fl["step"] / 1e12}
    line = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step,
            "step_ms": {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9), "min": steps_ms[0],
                        "max": steps_ms[-1]},
            "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "nvfp4->f16 MFMA fwd, e4m3 MFMA bwd, fp32 accumulate",
            "data": "synthetic (seeded, generated on the GPU)", "config": cfg, "roofline": roofline,
            "cpu_baseline": cpu, "kernels": kernels, "quantizer_workload": quant, "combine_workload": comb,
            "mxfp8_forward": mx8, "fp4_backward": fp4b, "nvfp4_w13_blocking": sq,
            "wall_s_timed": wall}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
