"""Benchmark of the quantized MoE expert layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input, by default the
one-GPU expert share (48 local experts, 65536 routed slots with Zipf(1.1) loads, hidden 7168,
FFN 2048, SwiGLU):
  weights:  NVFP4 quantization of w13 and w2 (one outer scale per expert and matrix) and, from
            the same read, the SR requantization of W13^T and W2^T for the backward's dgrad
  forward:  NVFP4 quantization of X (per-token outer scale, 4/6) -> grouped GEMM w13 with the
            SwiGLU epilogue (h13 saved) -> NVFP4 quantization of A -> grouped GEMM w2 with the
            fused RHT32 + S2F6 epilogue (the combine payload)
  backward: w2 backward (dY MXFP8 row/column quantization, SR requantization of A^T, MXFP8 dgrad
            and wgrad) -> w13 backward (the same with X^T, its dY the SwiGLU backward formed
            inside the dY quantization)
Inputs are generated on the GPU from fixed seeds before the timed region and stay resident in
HBM. Per-call device time comes from HIP events on the stream the kernels run on.

Also reported, each in its own object of the JSON line:
  moe32              the same step on the routed 32-expert layer (16384 tokens, top-8 of 32
                     experts, hidden 4096, FFN 1536), activations gathered through the routing
  hw_measured        roofs measured in this run on this chip: HBM bandwidth of a streaming kernel
                     for each kernel's read:write byte mix (nontemporal 16-byte accesses, buffers
                     larger than the 256 MB Infinity Cache) and the throughput of every MFMA
                     instruction the grouped GEMMs issue
  memory_kernels     every memory-bound call (layer and workloads) as GB/s of algorithmic bytes,
                     against 8 TB/s and against the measured roof of its own mix
  quantizer_workload nvfp4_quantize with 4/6 and requant_transpose_sr_mxfp8 on 8192 x 7168
                     activations (0.5 * StudentT(3)), rotating inputs larger than the cache
  mxfp8_forward      the forward of the layers that keep MXFP8 (w13 + SwiGLU, w2 + RHT32/S2F6)
  fp4_backward       the FP4 backward variant (every backward operand in MXFP4)
  combine_workload   the combine's receiver, 16384 tokens x top-8 of 131072 S2F6 rows of 4096
  cpu_baseline       the CPU oracle on a bounded sample of the layer, and on the full 8192 x 7168
                     quantizer workload with all host threads and with one

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ep48|moe32]
       python bench.py --summarize-profiles DIR   (writes profiles/*.md from rocprofv3 CSVs in DIR)
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

# Read:write byte mixes of the memory-bound kernels, as KB read : KB written per streamed unit.
STREAM_MIXES = {
    "read": (1, 0),
    "write": (0, 1),
    "copy": (1, 1),
    "nvfp4_quantize": (32, 9),      # bf16 in (2 B) : codes + E4M3 scales out (0.5 + 1/16 B) per element
    "requant": (6, 11),             # codes + scales in (0.5 + 1/16 B) : E4M3 + E8M0 out (1 + 1/32 B)
    "mxfp8_quantize": (64, 33),     # bf16 in (2 B) : E4M3 + E8M0 out (1 + 1/32 B); also bf16 RHT32 + S2F6
    "weights_bwd": (64, 51),        # bf16 in (2 B) : NVFP4 codes + scales and W^T E4M3 + E8M0 out (1.59375 B)
    "combine": (33, 8),             # 8 slots x (4096 + 128) B + 64 B of index/gate in : 8192 B out per token
    "swiglu_bwd": (2, 1),           # da fp32 + h13 bf16 in (8 B) : dh13 bf16 out (4 B) per FFN element
}
CALIB_GRID = 4097                   # grid of the one calibration copy (1 GiB read + 1 GiB written)
# the roofline kernel in the traces: the NVFP4 forward with the SwiGLU epilogue, K a multiple of 64
ROOF_KERNEL = "pmn::k_nvfp4_grouped_gemm<2, false>"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ep48", choices=["ep48", "moe32"])
    ap.add_argument("--moe32-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quant-iters", type=int, default=20)
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None)
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
        # the weight quantizer's workspace (one read of the bf16 weights)
        self.wsq = torch.empty(P.nvfp4_quantize_ws_size(), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def flops(self):
        M, H, F = self.M, self.H, self.F
        fwd13 = 2.0 * M * 2 * F * H
        fwd2 = 2.0 * M * H * F
        return dict(fwd13=fwd13, fwd2=fwd2, fwd=fwd13 + fwd2, bwd=2 * (fwd13 + fwd2), step=3 * (fwd13 + fwd2))

    def step(self, T):
        P = self.P
        E, H, F, M = self.E, self.H, self.F, self.M
        # weights for both passes: NVFP4 for the forward, W^T requantized by SR for the dgrad
        w13b = T.run("nvfp4_quantize_weights_bwd[w13]", P.nvfp4_quantize_weights_bwd, self.w13, F, seed=self.seed,
                     rng_stream=1, workspace=self.wsq)
        w2b = T.run("nvfp4_quantize_weights_bwd[w2]", P.nvfp4_quantize_weights_bwd, self.w2, H, seed=self.seed,
                    rng_stream=3, workspace=self.wsq)
        w13q, w2q = w13b.q, w2b.q
        xq = T.run("nvfp4_quantize[x]", P.nvfp4_quantize, self.x, P.NVFP4_ACT)
        a, h13 = T.run("moe_grouped_gemm_fwd[w13+swiglu]", P.moe_grouped_gemm_fwd, xq, w13q, self.offsets, M, 2 * F,
                       P.EPI_SWIGLU, gather=self.gather, save_h13=True)
        aq = T.run("nvfp4_quantize[a]", P.nvfp4_quantize, a, P.NVFP4_ACT)
        yc, ye = T.run("moe_grouped_gemm_fwd[w2+rht32_s2f6]", P.moe_grouped_gemm_fwd, aq, w2q, self.offsets, M, H,
                       P.EPI_RHT32_S2F6, rht_sign_mask=self.mask)
        da, dw2, _ = T.run("moe_grouped_gemm_bwd[w2]", P.moe_grouped_gemm_bwd, self.dy, aq, w2b, self.offsets, M, H,
                           seed=self.seed, rng_stream_a=5, rng_stream_b=3, rng_stream_dy=6, workspace=self.ws2)
        # the SwiGLU backward runs inside the w13 backward's dY quantization (dh13 is not written)
        dx, dw13, _ = T.run("moe_grouped_gemm_bwd_swiglu[w13]", P.moe_grouped_gemm_bwd_swiglu, da, h13, xq, w13b,
                            self.offsets, M, 2 * F, gather=self.gather, seed=self.seed, rng_stream_a=4,
                            rng_stream_b=1, workspace=self.ws13)
        return yc, dx, dw13, dw2


def swiglu_workload(P, I, torch, layer):
    """ms of the standalone SwiGLU backward on the layer's shape (the step runs it inside the w13
    backward's dY quantization)."""
    M, F = layer.M, layer.F
    dev = layer.x.device
    da = I.normal((M, F), 1e-3, 51, dev, dtype=torch.float32)
    h13 = I.student_t((M, 2 * F), 4, 1.0, 52, dev)
    for _ in range(2):
        P.swiglu_bwd(da, h13)
    return _time_ms(torch, lambda: P.swiglu_bwd(da, h13), 5)


def _time_ms(torch, fn, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def hardware_roofs(P, torch, dev):
    """Roofs measured in this run: the streaming kernel's HBM bandwidth for each read:write mix
    (best of three grid sizes and the four load/store cache hints; 2 GiB read, or written when
    nothing is read, so every buffer is far larger than the 256 MB Infinity Cache), torch's
    1 GiB device-to-device copy, and each MFMA instruction's throughput at 1 and 2 wavefronts per
    SIMD (one workgroup per compute unit). One copy launch with the grid CALIB_GRID moves exactly
    1 GiB each way: the profile summaries calibrate the PMC byte counters on it."""
    src = torch.empty(2 << 30, dtype=torch.uint8, device=dev).fill_(7)
    dst = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    hbm = {}
    for name, (rv, wv) in STREAM_MIXES.items():
        units = (2 << 20) // (rv if rv else wv)          # 2 GiB read (or written)
        nbytes = units * (rv + wv) * 1024.0
        best, how = 0.0, None
        for hints in (0, 1, 2, 3):
            for grid in (1024, 4096, 16384):
                def run(g=grid, h=hints):
                    P.probe_stream(src, dst, units, rv, wv, grid=g, hints=h)
                run()
                gbs = nbytes / (_time_ms(torch, run, 3) * 1e-3) / 1e9
                if gbs > best:
                    best, how = gbs, dict(grid=grid, nontemporal_loads=bool(hints & 1),
                                          nontemporal_stores=bool(hints & 2))
        hbm[name] = dict(gbs=best, read_kb=rv, write_kb=wv, best_launch=how)
    P.probe_stream(src, dst, 1 << 20, 1, 1, grid=CALIB_GRID, hints=3)      # the calibration copy
    src1, dst1 = src[: 1 << 30], dst[: 1 << 30]
    dst1.copy_(src1)
    torch_copy = 2.0 * (1 << 30) / (_time_ms(torch, lambda: dst1.copy_(src1), 3) * 1e-3) / 1e9
    del src, dst, src1, dst1
    sink = torch.empty(P._lib.pmn_probe_mfma_sink_floats(2, 256), dtype=torch.float32, device=dev)
    guess = {0: 2.0e15, 1: 2.2e15, 2: 4.5e15, 3: 4.5e15, 4: 9.0e15, 5: 1.8e15, 6: 1.5e15}   # only sizes the launches
    mfma = {}
    for kind, name in P.PROBE_MFMA_KINDS.items():
        for wps in ((1,) if kind >= 5 else (1, 2)):   # kinds 5, 6: the GEMM's register budget, one wave per SIMD
            per_iter = P.probe_mfma(kind, wps, 256, 2, sink) / 2
            iters = max(200, int(4e-3 * guess[kind] / per_iter)) // 2 * 2
            P.probe_mfma(kind, wps, 256, 50, sink)
            fl = [0.0]

            def run(k=kind, w=wps, it=iters):
                fl[0] = P.probe_mfma(k, w, 256, it, sink)
            ms = _time_ms(torch, run, 2)
            mfma.setdefault(name, {})[f"{wps}_wave_per_simd"] = fl[0] / (ms * 1e-3) / 1e12
    del sink
    return dict(hbm_gbs=hbm, torch_copy_gbs=torch_copy, mfma_tflops=mfma,
                note="streaming kernel: 16-byte loads/stores, one contiguous KB per instruction, best of "
                     "ordinary and nontemporal accesses; "
                     "MFMA: independent accumulator chains on constant operands, no memory traffic")


def library_reference(torch, dev, shape):
    """The vendor library's dense GEMM on this chip, as a calibration of what the matrix cores reach
    on plain operands of the layer's sizes (not a path of this library): hipBLASLt through torch,
    fp16 for the forward shapes and fp8 E4M3 with unit per-tensor scales and fp32 output for the
    backward shapes, M = all routed slots in one group. TFLOP/s per shape."""
    M, H, F = shape.slots or shape.tokens * shape.top_k, shape.hidden, shape.ffn
    res = {}

    def rate(fn, flops, it=5):
        fn()
        ms = _time_ms(torch, fn, it)
        return flops / (ms * 1e-3) / 1e12
    for name, (m, n, k) in (("fwd_w13 fp16", (M, 2 * F, H)), ("fwd_w2 fp16", (M, H, F))):
        a = torch.randn(m, k, device=dev, dtype=torch.float16)
        b = torch.randn(k, n, device=dev, dtype=torch.float16)
        res[name] = rate(lambda: torch.matmul(a, b), 2.0 * m * n * k)
        del a, b
    one = torch.ones((), device=dev)
    for name, (m, n, k) in (("dgrad_w13 fp8", (M, H, 2 * F)), ("wgrad_w13 fp8", (2 * F, H, M))):
        try:
            a = torch.randn(m, k, device=dev).to(torch.float8_e4m3fn)
            b = torch.randn(n, k, device=dev).to(torch.float8_e4m3fn)
            res[name] = rate(lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.float32),
                             2.0 * m * n * k)
            del a, b
        except Exception as ex:   # the library may not offer this fp8 product
            res[name] = None
            res[name + " error"] = type(ex).__name__
    return res


def quantizer_workload(P, I, torch, dev, iters):
    """GB/s of nvfp4_quantize (4/6, per-token outer) and requant_transpose_sr_mxfp8 on the
    8192 x 7168 activation workload. Inputs and outputs both rotate over buffer sets larger than the
    256 MB Infinity Cache, so neither the reads nor the writes can be served or absorbed by it."""
    R, Cc = 8192, 7168
    base = I.quantizer(dev)
    nbuf = 4
    xs = [base["x"]] + [base["x"].roll(shifts=97 * i, dims=1).contiguous() for i in range(1, nbuf)]
    nq = 12
    qbuf = [P.nvfp4_quantize(xs[i % nbuf], P.NVFP4_ACT) for i in range(nq)]   # 12 x 33 MB of outputs
    ld = P.padded_bound(R, 0)
    nr = 8
    outs = [(torch.empty((Cc, ld), dtype=torch.uint8, device=dev),
             torch.empty((Cc, ld // 32), dtype=torch.uint8, device=dev)) for _ in range(nr)]   # 8 x 61 MB
    torch.cuda.synchronize()
    res = {}
    it = [0]

    def quant():
        i = it[0]
        it[0] += 1
        P.nvfp4_quantize(xs[i % nbuf], P.NVFP4_ACT, out=qbuf[i % nq])
    for _ in range(3):
        quant()
    ms = _time_ms(torch, quant, iters)
    nbytes = R * Cc * (2 + 0.5 + 1 / 16) + R * 4
    res["nvfp4_quantize"] = dict(us=ms * 1e3, bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9)

    def rq():
        i = it[0]
        it[0] += 1
        o, oe = outs[i % nr]
        P.requant_transpose_sr_mxfp8(qbuf[i % nq], seed=base["seed"], rng_stream=base["stream"], ld=ld, out=o,
                                     out_e8m0=oe)
    for _ in range(3):
        rq()
    ms = _time_ms(torch, rq, iters)
    nbytes = R * Cc * (0.5 + 1 / 16 + 1 + 1 / 32) + R * 4
    res["requant_transpose_sr_mxfp8"] = dict(us=ms * 1e3, bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9)
    return res


def combine_workload(P, I, torch, dev, iters):
    """GB/s of moe_combine_s2f6 on the routed shape (16384 tokens, top-8 of 32 experts, 131072 slot
    rows of hidden 4096): routing on the device from the seeded logits, two S2F6 payloads of
    553 MB each used in turn and four 134 MB outputs in turn, so the Infinity Cache can neither
    serve the reads nor absorb the writes."""
    sh = I.MOE32
    T, k, H = sh.tokens, sh.top_k, sh.hidden
    M = T * k
    r = P.moe_route_topk(I.moe_logits(sh, dev), k)
    so, gates = r["slot_of"], r["gates"]
    mask = I.sign_mask(sh.seeds["rht"])
    pay = [I.s2f6_payload(M, H, sh.seeds["payload"] + i, dev) for i in range(2)]
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(4)]
    it = [0]

    def run():
        i = it[0]
        it[0] += 1
        P.moe_combine_s2f6(*pay[i % 2], mask, so, gates, out=outs[i % 4])
    for _ in range(3):
        run()
    ms = _time_ms(torch, run, iters)
    # per token: k rows of H codes + H/32 E8M0 bytes, k slot indices and gates; H bf16 out
    nbytes = T * (k * (H + H // 32) + 8 * k + 2 * H)
    del pay, outs
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
    """The CPU oracle (as it stands, never tuned for speed) on bounded samples of the same work:
    16 slots of one expert through the whole layer, forward and backward (the `value`, TFLOP/s of
    the sample's GEMM work), and the full 8192 x 7168 quantizer workload (nvfp4_quantize with 4/6
    and requant_transpose_sr_mxfp8 of its output) with all host threads and with one thread, as
    GB/s of the same algorithmic bytes the GPU is rated on."""
    import numpy as np  # noqa: F401
    import torch

    import oracle as O
    threads = O.threads()
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
    # the memory-bound workload at full size
    base = I.quantizer("cpu")
    R, Cc = base["x"].shape
    qbytes = R * Cc * (2 + 0.5 + 1 / 16) + R * 4
    rbytes = R * Cc * (0.5 + 1 / 16 + 1 + 1 / 32) + R * 4
    quant = {}
    for nt in (threads, 1):
        O.set_threads(nt)
        t1 = time.perf_counter()
        q = O.nvfp4_quantize(base["x"], 1, True)
        t2 = time.perf_counter()
        O.requant_transpose_sr(q, seed=base["seed"], stream=base["stream"])
        t3 = time.perf_counter()
        quant[f"threads_{nt}"] = dict(nvfp4_quantize_s=t2 - t1, nvfp4_quantize_gbs=qbytes / (t2 - t1) / 1e9,
                                      requant_s=t3 - t2, requant_gbs=rbytes / (t3 - t2) / 1e9)
    O.set_threads(threads)
    return dict(value=flops / dt_s / 1e12, unit="TFLOP/s", cores=threads, kind="oracle", seconds=dt_s,
                sample=f"{S} routed slots of one expert through the whole layer (NVFP4 quantize of X, w13, w2; "
                       f"w13 GEMM + SwiGLU; A quantize; w2 GEMM; RHT32+S2F6; MXFP8 dY quantize; SR requant of "
                       f"W2^T, A^T, W13^T, X^T; dgrad and wgrad of both GEMMs), H={H}, F={F}",
                quantizer_workload=dict(shape=[R, Cc], **quant,
                                        note="full size, the same inputs and algorithmic bytes as the GPU's "
                                             "quantizer_workload"))


def moe32_workload(P, I, torch, dev, steps, warmup=2):
    """The layer step on the routed 32-expert layer (16384 tokens, top-8 of 32 experts, hidden
    4096, FFN 1536; routing on the device from the seeded logits, activations gathered)."""
    layer = Layer(P, I, torch, I.MOE32, dev)
    T = Timer(torch)
    for _ in range(warmup):
        layer.step(T)
    torch.cuda.synchronize()
    T.collect()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        layer.step(T)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    per_call = T.collect()
    fl = layer.flops()
    kern = {name: {"ms": v} for name, v in per_call.items()}
    for nm, f, pk in (("moe_grouped_gemm_fwd[w13+swiglu]", fl["fwd13"], PEAK_F16_TFLOPS),
                      ("moe_grouped_gemm_fwd[w2+rht32_s2f6]", fl["fwd2"], PEAK_F16_TFLOPS),
                      ("moe_grouped_gemm_bwd[w2]", 2 * fl["fwd2"], PEAK_FP8_TFLOPS),
                      ("moe_grouped_gemm_bwd_swiglu[w13]", 2 * fl["fwd13"], PEAK_FP8_TFLOPS)):
        t = f / (per_call[nm] * 1e-3) / 1e12
        kern[nm].update(tflops=t, frac_of_dtype_peak=t / pk)
    fwd_ms = sum(per_call[k] for k in per_call if "fwd" in k or k in ("nvfp4_quantize[x]", "nvfp4_quantize[a]"))
    bwd_ms = sum(per_call[k] for k in per_call if k.startswith("moe_grouped_gemm_bwd"))
    res = dict(workload=f"moe32: 32 experts, {layer.M} routed slots (top-8 of 16384 tokens), hidden 4096, FFN 1536",
               steps=steps, ms_per_step=ms, tflops=fl["step"] / (ms * 1e-3) / 1e12, step_tflop=fl["step"] / 1e12,
               forward_ms=fwd_ms, forward_tflops=fl["fwd"] / (fwd_ms * 1e-3) / 1e12,
               backward_ms=bwd_ms, backward_tflops=fl["bwd"] / (bwd_ms * 1e-3) / 1e12, kernels=kern)
    del layer
    return res


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


# ---- profile summaries ---------------------------------------------------------------------

PROFILE_COMMANDS = {
    "kernel_trace": ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof/kt -o ep48 -- "
                     "python3 bench.py --steps 10 --warmup 3 --no-cpu-baseline"),
    "fetch": ("rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof/fetch -o ep48 -- "
              "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --quant-iters 2 --moe32-steps 1"),
    "write": ("rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof/write -o ep48 -- "
              "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --quant-iters 2 --moe32-steps 1"),
    "clock": ("rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA "
              "SQ_ACTIVE_INST_VALU --output-format csv -d gpurun_out/prof/clock -o ep48 -- "
              "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --quant-iters 1 --moe32-steps 1"),
    "valu": ("rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_VALU_CVT "
             "SQ_INSTS_LDS SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_INSTS_SALU --output-format csv -d gpurun_out/prof/valu "
             "-o ep48 -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --quant-iters 1 --moe32-steps 1"),
    "bench": "python3 bench.py --no-cpu-baseline > gpurun_out/prof/bench.json",
}
TRAFFIC_SOURCES = ["precision_moe_numerics_amd/csrc/gemm_fwd.hip", "precision_moe_numerics_amd/csrc/pmn_dev.hpp"]


def _kname(n):
    n = n.replace("(anonymous namespace)::", "").strip()
    n = n[5:] if n.startswith("void ") else n
    return n.split("(")[0].strip()


def _find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def summarize_profiles(d, out_dir=None):
    """Write profiles/*.md (and the forward GEMM's traffic record) from the rocprofv3 CSVs of the
    PROFILE_COMMANDS runs under d (subfolders kt, fetch, write, clock, valu, and bench.json: the
    benchmark line of the same lease); out_dir defaults to the repository's profiles/."""
    import csv
    import hashlib
    from collections import defaultdict
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    bench = None
    bp = os.path.join(d, "bench.json")
    if os.path.exists(bp):
        lines = [l for l in open(bp) if l.strip().startswith("{")]
        bench = json.loads(lines[-1]) if lines else None
    # kernel trace + stats
    stats = list(csv.DictReader(open(_find_csv(os.path.join(d, "kt"), "kernel_stats.csv"))))
    trace = list(csv.DictReader(open(_find_csv(os.path.join(d, "kt"), "kernel_trace.csv"))))
    md = ["# Kernel time of the 48-expert layer step and the workloads bench.py reports", "",
          "Command (from the repository root, one MI355X; the bench line below ran in the same lease):", "",
          "```", PROFILE_COMMANDS["kernel_trace"], PROFILE_COMMANDS["bench"], "```", "",
          "rocprofv3 `--stats` summary (every kernel of the profiled run, input generation included):", "",
          "| kernel | calls | avg us | min us | max us | % time |", "|---|---:|---:|---:|---:|---:|"]
    for r in stats:
        n = _kname(r["Name"])
        n = n if len(n) <= 70 else n[:67] + "..."
        md.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                  f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    agg = defaultdict(list)
    for r in trace:
        n = r["Kernel_Name"]
        if "pmn::" not in n and "k_stream_mix" not in n and "k_mfma_probe" not in n:
            continue
        key = (_kname(n), r.get("Grid_Size_X", r.get("Grid_Size", "")), r.get("Grid_Size_Y", "1"))
        agg[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    md += ["", "Library kernels by launch shape (grid in work-items x, y):", "",
           "| kernel | grid | launches | avg us |", "|---|---|---:|---:|"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1]) / len(kv[1])):
        md.append(f"| `{k[0]}` | {k[1]},{k[2]} | {len(v)} | {sum(v) / len(v) / 1e3:.1f} |")
    if bench:
        r = bench["roofline"]
        gem = [v for k, v in agg.items() if k[0].startswith(ROOF_KERNEL)]
        if gem:
            v = max(gem, key=len)
            avg = sum(v) / len(v) / 1e6
            md += ["", f"Dominant kernel: `{ROOF_KERNEL[5:]}` (w13 forward + SwiGLU) averages {avg:.3f} ms per "
                       f"launch in this trace; bench.py in the same lease measured {r['ms_per_launch']:.3f} ms by HIP "
                       f"events ({r['achieved']:.0f} TFLOP/s, frac {r['frac']:.3f} of {r['peak']:.0f}); from the "
                       f"trace: {r['flops_per_launch'] / (avg * 1e-3) / 1e12:.0f} TFLOP/s, frac "
                       f"{r['flops_per_launch'] / (avg * 1e-3) / 1e12 / r['peak']:.3f}.",
                   "", f"Bench line of the same lease: {bench['ms_per_step']:.2f} ms per step, {bench['value']:.0f} "
                       f"TFLOP/s."]
    open(os.path.join(out_dir, "ep48_layer_step_kernel_stats.md"), "w").write("\n".join(md) + "\n")

    # HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), calibrated on the probe's copy
    def load(sub):
        dd = defaultdict(list)
        for r in csv.DictReader(open(_find_csv(os.path.join(d, sub), "counter_collection.csv"))):
            dd[(_kname(r["Kernel_Name"]), r["Grid_Size"])].append(float(r["Counter_Value"]))
        return dd
    fe, wr = load("fetch"), load("write")
    cal = str(CALIB_GRID * 256)
    ck = [k for k in fe if "k_stream_mix" in k[0] and k[1] == cal]
    assert ck, "the calibration copy (k_stream_mix, grid CALIB_GRID) is missing from the PMC runs"
    gib_kib = float(1 << 20)
    ff = gib_kib / (sum(fe[ck[0]]) / len(fe[ck[0]]))
    fw = gib_kib / (sum(wr[ck[0]]) / len(wr[ck[0]]))
    tc = [k for k in fe if "copyBuffer" in k[0]]
    tmd = ["# HBM traffic per kernel launch (48-expert layer step and the workloads)", "",
           "Commands (from the repository root, one MI355X, one counter per run):", "", "```",
           PROFILE_COMMANDS["fetch"], PROFILE_COMMANDS["write"], "```", "",
           f"Calibration: the probe copy `k_stream_mix` launched with grid {CALIB_GRID} x 256 reads and writes exactly "
           f"1 GiB (1048576 KiB) with nontemporal 16-byte accesses; it reads FETCH_SIZE = {gib_kib / ff:.1f} KiB and "
           f"WRITE_SIZE = {gib_kib / fw:.1f} KiB, so HBM bytes = FETCH_SIZE x {ff:.3f} KiB and WRITE_SIZE x {fw:.3f} KiB."
           + (f" (torch's 1 GiB copy reads FETCH_SIZE = {max(max(fe[k]) for k in tc):.1f} KiB.)" if tc else ""), "",
           "| kernel | grid | launches | read GB (scaled) | written GB (scaled) |", "|---|---:|---:|---:|---:|"]
    for k in sorted(fe, key=lambda k: -max(fe[k])):
        if "pmn::" not in k[0]:
            continue
        f = sum(fe[k]) / len(fe[k]) * ff * 1024 / 1e9
        w = sum(wr.get(k, [0.0])) / max(len(wr.get(k, [])), 1) * fw * 1024 / 1e9
        tmd.append(f"| `{k[0]}` | {k[1]} | {len(fe[k])} | {f:.3f} | {w:.3f} |")
    open(os.path.join(out_dir, "ep48_layer_step_hbm_traffic.md"), "w").write("\n".join(tmd) + "\n")
    key = [k for k in fe if k[0].startswith(ROOF_KERNEL)]
    key = max(key, key=lambda k: int(k[1]))
    fetch = sum(fe[key]) / len(fe[key]) * ff * 1024
    write = sum(wr[key]) / len(wr[key]) * fw * 1024
    M, E, H, F = 65536, 48, 7168, 2048
    alg = M * H * (0.5 + 1 / 16) + E * 2 * F * H * (0.5 + 1 / 16) + M * F * 2 + M * 2 * F * 2
    h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in TRAFFIC_SOURCES)).hexdigest()
    rec = {"kernel": f"k_nvfp4_grouped_gemm<PMN_EPI_SWIGLU> (w13 forward of the 48-expert layer step, "
                     f"{int(key[1]) // 256} workgroups)",
           "source_sha256": h, "sources": TRAFFIC_SOURCES, "fetch_bytes_per_launch": fetch,
           "write_bytes_per_launch": write, "traffic_bytes_per_launch": fetch + write,
           "algorithmic_bytes_per_launch": alg,
           "calibration": f"FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {fw:.3f} (probe copy of 1 GiB each way)",
           "commands": [PROFILE_COMMANDS["fetch"], PROFILE_COMMANDS["write"]]}
    json.dump(rec, open(os.path.join(out_dir, "traffic_gemm_fwd.json"), "w"), indent=1)

    # clock, MFMA and VALU busy
    rows = list(csv.DictReader(open(_find_csv(os.path.join(d, "clock"), "counter_collection.csv"))))
    ag = defaultdict(dict)
    for r in rows:
        n = _kname(r["Kernel_Name"])
        if "pmn::" not in n:
            continue
        v = ag[(int(r["Dispatch_Id"]), n, r["Grid_Size"])]
        v[r["Counter_Name"]] = float(r["Counter_Value"])
        v["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
    cmd = ["# Clock and matrix-core / VALU utilisation per kernel (48-expert layer step and workloads)", "",
           "Command (from the repository root, one MI355X):", "", "```", PROFILE_COMMANDS["clock"], "```", "",
           "GRBM_GUI_ACTIVE sums the 8 XCDs, so the clock is GRBM_GUI_ACTIVE / 8 / kernel time. "
           "SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of the 1024 SIMDs, so MFMA busy = MFMA_BUSY / 1024 / "
           "(GRBM_GUI_ACTIVE / 8) at the running clock. SQ_ACTIVE_INST_VALU counts quad-cycles issuing VALU work "
           "(MFMA included): VALU busy = 4 x ACTIVE_INST_VALU / 1024 / (GRBM_GUI_ACTIVE / 8). Kernels under "
           "0.02 ms are omitted. Two limits of these figures: launches shorter than about 0.05 ms read clocks "
           "above the 2.4 GHz maximum, because the counters run over a longer window than the dispatch's "
           "timestamps; and SQ_ACTIVE_INST_VALU is accumulated per wavefront, so a kernel whose wavefronts "
           "share a SIMD can read a VALU busy above 1, which means its vector units are saturated.", "",
           "| kernel | grid | ms | clock GHz | MFMA busy (at that clock) | MFMA busy vs 2.4 GHz | VALU busy |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for k, v in sorted(ag.items()):
        if v["dur"] < 2e-5 or "GRBM_GUI_ACTIVE" not in v:
            continue
        clk = v["GRBM_GUI_ACTIVE"] / 8 / v["dur"]
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024 / (v["GRBM_GUI_ACTIVE"] / 8)
        busy24 = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024 / (2.4e9 * v["dur"])
        valu = 4 * v.get("SQ_ACTIVE_INST_VALU", 0.0) / 1024 / (v["GRBM_GUI_ACTIVE"] / 8)
        cmd.append(f"| `{k[1]}` | {k[2]} | {v['dur'] * 1e3:.3f} | {clk / 1e9:.2f} | {busy:.2f} | {busy24:.2f} | "
                   f"{valu:.2f} |")
    open(os.path.join(out_dir, "ep48_layer_step_clock_mfma.md"), "w").write("\n".join(cmd) + "\n")

    # VALU instruction counts: what the VALU-bound kernels spend their issue cycles on
    vd = os.path.join(d, "valu")
    if os.path.isdir(vd):
        rows = list(csv.DictReader(open(_find_csv(vd, "counter_collection.csv"))))
        ag = defaultdict(dict)
        for r in rows:
            n = _kname(r["Kernel_Name"])
            if "pmn::" not in n:
                continue
            v = ag[(int(r["Dispatch_Id"]), n, r["Grid_Size"])]
            v[r["Counter_Name"]] = float(r["Counter_Value"])
            v["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
        md = ["# VALU instructions per kernel (48-expert layer step and workloads)", "",
              "Command (from the repository root, one MI355X):", "", "```", PROFILE_COMMANDS["valu"], "```", "",
              "SQ_INSTS_VALU counts wavefront VALU instructions (MFMA included) and SQ_ACTIVE_INST_VALU the "
              "quad-cycles spent issuing them, so 4 x ACTIVE / INSTS is the SIMD cycles per VALU instruction and "
              "4 x ACTIVE / 1024 / (GRBM_GUI_ACTIVE / 8) the share of SIMD cycles issuing VALU work (VALU busy). "
              "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES is the share of wavefront time spent waiting on a dependency "
              "(s_waitcnt). Kernels under 0.02 ms are omitted.", "",
              "| kernel | grid | ms | waves | VALU instr (M) | per wave | cycles / instr | VALU busy | converts (M) | "
              "LDS instr (M) | waiting |", "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
        for k, v in sorted(ag.items()):
            if v["dur"] < 2e-5 or "GRBM_GUI_ACTIVE" not in v or not v.get("SQ_INSTS_VALU"):
                continue
            cyc = v["GRBM_GUI_ACTIVE"] / 8
            md.append(f"| `{k[1]}` | {k[2]} | {v['dur'] * 1e3:.3f} | {v.get('SQ_WAVES', 0):.0f} | "
                      f"{v['SQ_INSTS_VALU'] / 1e6:.1f} | {v['SQ_INSTS_VALU'] / max(v.get('SQ_WAVES', 1), 1):.0f} | "
                      f"{4 * v['SQ_ACTIVE_INST_VALU'] / v['SQ_INSTS_VALU']:.2f} | "
                      f"{4 * v['SQ_ACTIVE_INST_VALU'] / 1024 / cyc:.2f} | {v.get('SQ_INSTS_VALU_CVT', 0) / 1e6:.1f} | "
                      f"{v.get('SQ_INSTS_LDS', 0) / 1e6:.1f} | "
                      f"{v.get('SQ_WAIT_INST_ANY', 0) / max(v.get('SQ_WAVE_CYCLES', 1), 1):.2f} |")
        open(os.path.join(out_dir, "ep48_layer_step_valu_instructions.md"), "w").write("\n".join(md) + "\n")
    print(f"wrote profiles/ from {d}: forward w13 traffic {(fetch + write) / 1e9:.3f} GB per launch "
          f"(algorithmic {alg / 1e9:.3f} GB)")


# ---- the benchmark ---------------------------------------------------------------------------

def _mem(nbytes, ms, mix, roofs):
    gbs = nbytes / (ms * 1e-3) / 1e9
    roof = roofs["hbm_gbs"][mix]["gbs"]
    return dict(ms=ms, bytes=nbytes, gbs=gbs, frac_of_8TBs=gbs / PEAK_HBM_GBS, mix=mix, measured_roof_gbs=roof,
                frac_of_measured_roof=gbs / roof)


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1 (the multi-GPU design, expert "
                                   "parallelism over RCCL all-to-alls, is not implemented here)"}))
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

    roofs = hardware_roofs(P, torch, dev)
    f16_ceiling = roofs["mfma_tflops"][P.PROBE_MFMA_KINDS[0]]["1_wave_per_simd"]
    # the same instruction with the kernel's dequantization interleaved, without memory traffic
    dequant_ceiling = roofs["mfma_tflops"][P.PROBE_MFMA_KINDS[5]]["1_wave_per_simd"]
    k13 = per_call["moe_grouped_gemm_fwd[w13+swiglu]"]
    k2 = per_call["moe_grouped_gemm_fwd[w2+rht32_s2f6]"]
    ach = fl["fwd13"] / (k13 * 1e-3) / 1e12
    roofline = {"bound": "mfma",
                "kernel": "k_nvfp4_grouped_gemm<SWIGLU> (w13 forward: NVFP4 operands dequantized exactly to fp16, "
                          "products on the fp16 matrix cores)",
                "achieved": ach, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_F16_TFLOPS,
                "traffic": measured_traffic() if args.workload == "ep48" else None,
                "peak_basis": "MI355X dense fp16 MFMA (2.5 PFLOP/s), the dtype this exact path computes in; "
                              "frac_fp4_class rates the same kernel against the 10.1 PFLOP/s FP4-class peak",
                "flops_per_launch": fl["fwd13"], "ms_per_launch": k13,
                "frac_of_measured_f16_ceiling": ach / f16_ceiling,
                "frac_of_measured_dequant_ceiling": ach / dequant_ceiling,
                "frac_fp4_class": ach / PEAK_FP4_TFLOPS}
    kernels = {name: {"ms": ms} for name, ms in per_call.items()}
    kernels["moe_grouped_gemm_fwd[w13+swiglu]"].update(tflops=ach, frac_f16_peak=ach / PEAK_F16_TFLOPS)
    a2 = fl["fwd2"] / (k2 * 1e-3) / 1e12
    kernels["moe_grouped_gemm_fwd[w2+rht32_s2f6]"].update(tflops=a2, frac_f16_peak=a2 / PEAK_F16_TFLOPS)
    for nm, f in (("moe_grouped_gemm_bwd[w2]", 2 * fl["fwd2"]),
                  ("moe_grouped_gemm_bwd_swiglu[w13]", 2 * fl["fwd13"])):
        t = f / (per_call[nm] * 1e-3) / 1e12
        kernels[nm].update(tflops_incl_quant=t, frac_fp8_peak=t / PEAK_FP8_TFLOPS)

    quant = quantizer_workload(P, I, torch, dev, args.quant_iters)
    # 16 x 16 square-block NVFP4 of the w13 weights, beside the 1D weight mode of the same call
    # (both with two reads of the weights) and the 1D mode with one read (the step's call)
    sq = {}
    for name, mode, kw in (("weight_1d", P.NVFP4_WEIGHT, {}), ("weight_16x16", P.NVFP4_WEIGHT_2D, {}),
                           ("weight_1d_one_read", P.NVFP4_WEIGHT, {"workspace": layer.wsq})):
        for _ in range(2):
            P.nvfp4_quantize(layer.w13, mode, layer.F, **kw)
        sq[name] = dict(ms=_time_ms(torch, lambda m=mode, k=kw: P.nvfp4_quantize(layer.w13, m, layer.F, **k), 5))
    # the step's call: the same one read, also writing the backward's W13^T operand
    sq["weight_1d_one_read_with_wt"] = dict(ms=_time_ms(
        torch, lambda: P.nvfp4_quantize_weights_bwd(layer.w13, layer.F, seed=layer.seed, rng_stream=1,
                                                    workspace=layer.wsq), 5))
    mx8 = mxfp8_forward_workload(P, I, torch, layer, max(args.quant_iters // 4, 3))
    fp4b = fp4_backward_workload(P, torch, layer, max(args.quant_iters // 4, 3))
    comb = combine_workload(P, I, torch, dev, args.quant_iters)

    # memory-bound calls, each against 8 TB/s and the measured roof of its read:write mix
    M, E, H, F = layer.M, layer.E, layer.H, layer.F
    w13_el, w2_el = E * 2 * F * H, E * H * F
    mem = {
        "nvfp4_quantize_weights_bwd[w13]": _mem(w13_el * (2.5625 + 1.03125) + E * 2 * 4,
                                                per_call["nvfp4_quantize_weights_bwd[w13]"], "weights_bwd", roofs),
        "nvfp4_quantize_weights_bwd[w2]": _mem(w2_el * (2.5625 + 1.03125) + E * 4,
                                               per_call["nvfp4_quantize_weights_bwd[w2]"], "weights_bwd", roofs),
        "nvfp4_quantize[x]": _mem(layer.x.numel() * 2.5625 + layer.x.shape[0] * 4,
                                  per_call["nvfp4_quantize[x]"], "nvfp4_quantize", roofs),
        "nvfp4_quantize[a]": _mem(M * F * 2.5625 + M * 4, per_call["nvfp4_quantize[a]"], "nvfp4_quantize",
                                  roofs),
        "swiglu_bwd": _mem(M * F * 12.0, swiglu_workload(P, I, torch, layer), "swiglu_bwd", roofs),
        "quantizer_workload.nvfp4_quantize": _mem(quant["nvfp4_quantize"]["bytes"],
                                                  quant["nvfp4_quantize"]["us"] * 1e-3, "nvfp4_quantize", roofs),
        "quantizer_workload.requant_transpose_sr_mxfp8": _mem(
            quant["requant_transpose_sr_mxfp8"]["bytes"], quant["requant_transpose_sr_mxfp8"]["us"] * 1e-3,
            "requant", roofs),
        "combine_workload.moe_combine_s2f6": _mem(comb["bytes"], comb["us"] * 1e-3, "combine", roofs),
    }
    for k in ("nvfp4_quantize", "requant_transpose_sr_mxfp8"):
        quant[k].update({kk: mem[f"quantizer_workload.{k}"][kk] for kk in
                         ("frac_of_8TBs", "measured_roof_gbs", "frac_of_measured_roof")})
    comb.update({kk: mem["combine_workload.moe_combine_s2f6"][kk] for kk in ("measured_roof_gbs",
                                                                             "frac_of_measured_roof")})
    over = [k for k, v in mem.items() if v["frac_of_measured_roof"] > 1.0]

    moe32 = moe32_workload(P, I, torch, dev, args.moe32_steps) if args.moe32_steps > 0 else None
    lib = library_reference(torch, dev, shape)
    roofs["library_gemm_tflops"] = lib
    for nm, ln in (("moe_grouped_gemm_fwd[w13+swiglu]", "fwd_w13 fp16"),
                   ("moe_grouped_gemm_fwd[w2+rht32_s2f6]", "fwd_w2 fp16")):
        if lib.get(ln):
            kernels[nm]["frac_of_library_dense_gemm"] = kernels[nm]["tflops"] / lib[ln]
    if lib.get("fwd_w13 fp16"):
        roofline["frac_of_library_dense_gemm"] = ach / lib["fwd_w13 fp16"]

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
            "cpu_baseline": cpu, "kernels": kernels, "memory_kernels": mem,
            "memory_roof_check": "ok" if not over else f"above the measured roof: {over}",
            "hw_measured": roofs, "quantizer_workload": quant, "combine_workload": comb,
            "moe32": moe32, "mxfp8_forward": mx8, "fp4_backward": fp4b, "nvfp4_w13_blocking": sq,
            "wall_s_timed": wall}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
