"""CPU oracle for the quantized MoE expert layer (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
It wraps ``pmn_oracle.c`` (plain C, built by :func:`build`) with numpy arrays; it never imports
the HIP library or the product package, and the product never imports it.

Every function states the passage of the pages it follows in the C source; the pages are
  [AREX] AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向传播
         贯穿预训练到最后一次 RL rollout" (sections cited by heading in the C source), and
  [LHC]  lhc.media note "Le calcul en 4 bits dès le préentraînement d'Inkling 2 Small".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pmn_oracle.c")
_LIB = os.path.join(_HERE, "libpmn_oracle.so")

# Target codes of the requantizer (E4M3 for MXFP8, E2M1 for the worked example's grid).
TARGET_E4M3 = 0
TARGET_E2M1 = 1


# Sanitizer flags of the checking build: AddressSanitizer (every out-of-bounds or use-after-free
# access aborts) and UndefinedBehaviorSanitizer (signed overflow, bad shifts, misaligned or null
# accesses, float-to-int overflow abort: nothing recovers).
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fsanitize=float-cast-overflow",
                  "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(out: str | None = None, sanitize: bool = False) -> str:
    """Compile the oracle with strict IEEE semantics (no contraction, no fast-math).

    ``sanitize`` adds ASan + UBSan (a checking build; the process that loads it needs the ASan
    runtime first in LD_PRELOAD). ``out`` is the library path (default: next to the source).
    """
    out = out or _LIB
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-Wall"] + (SANITIZE_FLAGS if sanitize else []) + ["-o", out, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def lib():
    """The loaded oracle library: PMN_ORACLE_LIB if set (e.g. a sanitizer build), else the
    default build, rebuilt when the source is newer."""
    global _lib
    if _lib is None:
        path = os.environ.get("PMN_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        _lib = C.CDLL(path)
        _declare(_lib)
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_get_threads())


def set_threads(n: int) -> None:
    """Set the OpenMP threads of the oracle's parallel loops (timing only; results do not change)."""
    lib().orc_set_threads(int(n))


P = C.c_void_p
I64 = C.c_int64
I32 = C.c_int
U32 = C.c_uint32
U64 = C.c_uint64


def _declare(L):
    sig = {
        "orc_bf16_to_f32": (C.c_float, [C.c_uint16]),
        "orc_f32_to_bf16": (C.c_uint16, [C.c_float]),
        "orc_e4m3_value": (C.c_double, [C.c_uint8]),
        "orc_fp4_value": (C.c_double, [C.c_uint8]),
        "orc_e4m3_encode": (C.c_uint8, [C.c_float, I32, U32]),
        "orc_fp4_encode": (C.c_uint8, [C.c_float, I32, U32]),
        "orc_e8m0_exponent": (I32, [C.c_float, C.c_double]),
        "orc_philox4x32_10": (None, [P, P, P]),
        "orc_rand16": (U32, [U64, U32, U64]),
        "orc_outer_scale": (C.c_float, [C.c_float]),
        "orc_nvfp4_quantize": (None, [P, I64, I64, I64, I32, P, P, P, P, P]),
        "orc_nvfp4_dequantize": (None, [P, P, P, I64, I64, I64, P]),
        "orc_padded_total": (I64, [P, I32, I64]),
        "orc_requant_transpose_sr": (None, [P, P, P, I64, I64, P, P, I32, I64, I32, U64, U32, P, P]),
        "orc_mxfp8_quantize_rows": (None, [P, I64, I64, I32, U64, U32, P, P]),
        "orc_mxfp8_quantize_cols": (None, [P, I64, I64, P, I32, I32, U64, U32, P, P]),
        "orc_rht32": (None, [P, U32, P]),
        "orc_s2f6_block": (None, [P, P, P]),
        "orc_rht32_s2f6_quantize": (None, [P, I64, I64, U32, P, P]),
        "orc_rht32_s2f6_decode": (None, [P, P, I64, I64, U32, P]),
        "orc_gemm_nvfp4_grouped": (None, [P, P, P, I64, P, P, P, P, I64, P, I32, I64, I64, P]),
        "orc_gemm_nvfp4_elem": (C.c_double, [P, P, P, I64, P, P, P, P, I64, P, I32, I64, I64, I64, I64]),
        "orc_mxfp8_dot": (C.c_double, [P, P, I64, P, P, I64, I64, I64, I64, I64]),
        "orc_moe_combine_s2f6": (None, [P, P, I64, I64, U32, P, P, I64, I32, P]),
        "orc_s2f6_quantize": (None, [P, I64, I64, P, P]),
        "orc_gemm_mxfp8_fwd": (None, [P, P, P, P, P, P, I32, I64, I64, P]),
        "orc_nvfp4_quantize_2d": (None, [P, I64, I64, I64, P, P, P]),
        "orc_mx_quantize_rows": (None, [P, I64, I64, I32, I32, U64, U32, P, P]),
        "orc_mx_quantize_cols": (None, [P, I64, I64, P, I32, I32, I32, U64, U32, P, P]),
        "orc_gemm_mx_dgrad": (None, [P, P, P, P, P, I32, I64, I64, I32, P]),
        "orc_gemm_mx_wgrad": (None, [P, P, P, P, P, I32, I64, I64, I32, P]),
        "orc_mx_dot": (C.c_double, [P, P, I64, P, P, I64, I64, I64, I64, I64, I32]),
        "orc_gemm_mxfp8_dgrad": (None, [P, P, P, P, P, I32, I64, I64, P]),
        "orc_gemm_mxfp8_wgrad": (None, [P, P, P, P, P, I32, I64, I64, P]),
        "orc_swiglu": (None, [P, I64, I64, P]),
        "orc_swiglu_bwd": (None, [P, P, I64, I64, P]),
        "orc_route_topk": (None, [P, I64, I32, I32, P, P, P, P, P]),
        "orc_e4m3_encode_array": (None, [P, I64, I32, P, P]),
        "orc_fp4_encode_array": (None, [P, I64, I32, P, P]),
        "orc_rand16_array": (None, [U64, U32, P, I64, P]),
        "orc_requant_window": (None, [P, P, P, I64, I64, I64, I64, I64, I32, U64, U32, P, P]),
        "orc_set_threads": (None, [I32]),
        "orc_get_threads": (I32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _u16(x):
    """bf16 data as raw uint16 (accepts a torch bf16 tensor or a uint16 array)."""
    if hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch
        return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    return np.ascontiguousarray(x, dtype=np.uint16)


# ---------------------------------------------------------------------------------------------
# scalar codecs
# ---------------------------------------------------------------------------------------------

def e4m3_value(c: int) -> float:
    return lib().orc_e4m3_value(c)


def fp4_value(c: int) -> float:
    return lib().orc_fp4_value(c)


def e4m3_encode(y: float, sr: bool = False, r16: int = 0) -> int:
    return lib().orc_e4m3_encode(y, 1 if sr else 0, r16)


def fp4_encode(y: float, sr: bool = False, r16: int = 0) -> int:
    return lib().orc_fp4_encode(y, 1 if sr else 0, r16)


def e4m3_encode_array(y, sr: bool = False, r16=None) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    r = None if r16 is None else np.ascontiguousarray(r16, np.uint32)
    out = np.zeros(y.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(y), y.size, 1 if sr else 0, _p(r), _p(out))
    return out


def fp4_encode_array(y, sr: bool = False, r16=None) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    r = None if r16 is None else np.ascontiguousarray(r16, np.uint32)
    out = np.zeros(y.shape, np.uint8)
    lib().orc_fp4_encode_array(_p(y), y.size, 1 if sr else 0, _p(r), _p(out))
    return out


def rand16_array(seed: int, stream: int, idx) -> np.ndarray:
    i = np.ascontiguousarray(idx, np.uint64)
    out = np.zeros(i.shape, np.uint32)
    lib().orc_rand16_array(seed, stream, _p(i), i.size, _p(out))
    return out


def e8m0_exponent(amax: float, M: float) -> int:
    return lib().orc_e8m0_exponent(amax, M)


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def rand16(seed: int, stream: int, i: int) -> int:
    return lib().orc_rand16(seed, stream, i)


def outer_scale(amax: float) -> float:
    return lib().orc_outer_scale(amax)


# ---------------------------------------------------------------------------------------------
# tensors
# ---------------------------------------------------------------------------------------------

def nvfp4_quantize(x_bf16, rows_per_outer: int = 1, four_six: bool = True, outer_in=None):
    """Returns dict(codes [R, C/2] u8, scales [R, C/16] u8, outer [R/rpo] f32, chose4)."""
    x = _u16(x_bf16)
    R, Cc = x.shape
    assert Cc % 16 == 0 and R % rows_per_outer == 0
    codes = np.zeros((R, Cc // 2), np.uint8)
    scales = np.zeros((R, Cc // 16), np.uint8)
    outer = np.zeros(R // rows_per_outer, np.float32)
    chose4 = np.zeros((R, Cc // 16), np.uint8)
    oin = None if outer_in is None else np.ascontiguousarray(outer_in, dtype=np.float32)
    lib().orc_nvfp4_quantize(_p(x), R, Cc, rows_per_outer, 1 if four_six else 0, _p(oin),
                             _p(codes), _p(scales), _p(outer), _p(chose4))
    return dict(codes=codes, scales=scales, outer=outer, chose4=chose4, rows_per_outer=rows_per_outer)


def nvfp4_dequantize(q) -> np.ndarray:
    codes, scales, outer = (np.ascontiguousarray(q[k]) for k in ("codes", "scales", "outer"))
    R, half = codes.shape
    out = np.zeros((R, half * 2), np.float32)
    lib().orc_nvfp4_dequantize(_p(codes), _p(scales), _p(np.ascontiguousarray(outer, np.float32)),
                               R, half * 2, q["rows_per_outer"], _p(out))
    return out


def padded_total(offsets, M: int) -> int:
    if offsets is None:
        return lib().orc_padded_total(None, 0, M)
    o = np.ascontiguousarray(offsets, np.int64)
    return lib().orc_padded_total(_p(o), len(o) - 1, M)


def nvfp4_quantize_2d(x_bf16, rows_per_outer: int):
    """NVFP4 with 16 x 16 blocks: dict(codes, scales [R, C/16] equal within a tile, outer)."""
    x = _u16(x_bf16)
    R, Cc = x.shape
    assert R % 16 == 0 and Cc % 16 == 0 and rows_per_outer % 16 == 0 and R % rows_per_outer == 0
    codes = np.zeros((R, Cc // 2), np.uint8)
    scales = np.zeros((R, Cc // 16), np.uint8)
    outer = np.zeros(R // rows_per_outer, np.float32)
    lib().orc_nvfp4_quantize_2d(_p(x), R, Cc, rows_per_outer, _p(codes), _p(scales), _p(outer))
    return dict(codes=codes, scales=scales, outer=outer, rows_per_outer=rows_per_outer)


def requant_transpose_sr(q, gather=None, offsets=None, M=None, target=TARGET_E4M3, seed=0, stream=0):
    """NVFP4 -> dequant -> transpose (grouped, padded to 32) -> SR to E4M3/E2M1 + E8M0."""
    codes, scales = np.ascontiguousarray(q["codes"]), np.ascontiguousarray(q["scales"])
    outer = np.ascontiguousarray(q["outer"], np.float32)
    R, half = codes.shape
    cols = half * 2
    g = None if gather is None else np.ascontiguousarray(gather, np.int32)
    o = None if offsets is None else np.ascontiguousarray(offsets, np.int64)
    if M is None:
        M = int(o[-1]) if o is not None else (len(g) if g is not None else R)
    G = 0 if o is None else len(o) - 1
    Ptot = padded_total(o, M)
    out = np.zeros((cols, Ptot), np.uint8)
    oe = np.zeros((cols, Ptot // 32), np.uint8)
    lib().orc_requant_transpose_sr(_p(codes), _p(scales), _p(outer), cols, q["rows_per_outer"],
                                   _p(g), _p(o), G, M, target, seed, stream, _p(out), _p(oe))
    return out, oe


def requant_window(q, s_begin, count, target=TARGET_E4M3, seed=0, stream=0):
    """Requantized output columns for slots [s_begin, s_begin + count) of an ungrouped source."""
    codes, scales = np.ascontiguousarray(q["codes"]), np.ascontiguousarray(q["scales"])
    outer = np.ascontiguousarray(q["outer"], np.float32)
    R, half = codes.shape
    cols = half * 2
    Pw = (count + 31) // 32 * 32
    out = np.zeros((cols, Pw), np.uint8)
    oe = np.zeros((cols, Pw // 32), np.uint8)
    lib().orc_requant_window(_p(codes), _p(scales), _p(outer), cols, q["rows_per_outer"], s_begin, count, R,
                             target, seed, stream, _p(out), _p(oe))
    return out, oe


def mxfp8_quantize_rows(x_bf16, sr=False, seed=0, stream=0, target=TARGET_E4M3):
    """Row-wise MX quantization: codes [M, N] (E4M3 bytes, or E2M1 one per byte), E8M0 [M, N/32]."""
    x = _u16(x_bf16)
    M, N = x.shape
    out = np.zeros((M, N), np.uint8)
    oe = np.zeros((M, N // 32), np.uint8)
    lib().orc_mx_quantize_rows(_p(x), M, N, target, 1 if sr else 0, seed, stream, _p(out), _p(oe))
    return out, oe


def mxfp8_quantize_cols(x_bf16, offsets=None, sr=False, seed=0, stream=0, target=TARGET_E4M3):
    x = _u16(x_bf16)
    M, N = x.shape
    o = None if offsets is None else np.ascontiguousarray(offsets, np.int64)
    G = 0 if o is None else len(o) - 1
    Ptot = padded_total(o, M)
    out = np.zeros((N, Ptot), np.uint8)
    oe = np.zeros((N, Ptot // 32), np.uint8)
    lib().orc_mx_quantize_cols(_p(x), M, N, _p(o), G, target, 1 if sr else 0, seed, stream, _p(out), _p(oe))
    return out, oe


def mxfp8_dequantize(codes, e8m0) -> np.ndarray:
    """fp64 values of an MXFP8 matrix with blocks of 32 along rows (test helper)."""
    e4 = np.array([lib().orc_e4m3_value(c) for c in range(256)], dtype=np.float64)
    v = e4[codes]
    sc = np.ldexp(1.0, e8m0.astype(np.int32) - 127)
    return v * np.repeat(sc, 32, axis=1)


def rht32(y, mask: int):
    y = np.ascontiguousarray(y, np.float32)
    z = np.zeros(32, np.float32)
    lib().orc_rht32(_p(y), mask, _p(z))
    return z


def rht32_s2f6_quantize(y, mask: int):
    y = np.ascontiguousarray(y, np.float32)
    R, Cc = y.shape
    codes = np.zeros((R, Cc), np.int8)
    e = np.zeros((R, Cc // 32), np.uint8)
    lib().orc_rht32_s2f6_quantize(_p(y), R, Cc, mask, _p(codes), _p(e))
    return codes, e


def rht32_s2f6_decode(codes, e8m0, mask: int):
    codes = np.ascontiguousarray(codes, np.int8)
    e8m0 = np.ascontiguousarray(e8m0, np.uint8)
    R, Cc = codes.shape
    out = np.zeros((R, Cc), np.float64)
    lib().orc_rht32_s2f6_decode(_p(codes), _p(e8m0), R, Cc, mask, _p(out))
    return out


def s2f6_quantize(y):
    """Plain per-32 S2F6 (no transform): codes int8 [R, C], E8M0 [R, C/32]."""
    y = np.ascontiguousarray(y, np.float32)
    R, Cc = y.shape
    codes = np.zeros((R, Cc), np.int8)
    e = np.zeros((R, Cc // 32), np.uint8)
    lib().orc_s2f6_quantize(_p(y), R, Cc, _p(codes), _p(e))
    return codes, e


def s2f6_dequantize(codes, e8m0):
    """fp64 values c 2^(e - 127 - 6) of plain S2F6 blocks."""
    c = np.asarray(codes, np.float64)
    R, Cc = c.shape
    return (c.reshape(R, Cc // 32, 32) * 2.0 ** (np.asarray(e8m0, np.float64) - 133)[..., None]).reshape(R, Cc)


def moe_combine_s2f6(codes, e8m0, mask: int, slot_of, gates):
    """Receiver side of the combine: out[t] = sum_i gates[t, i] * decode(codes[slot_of[t, i]]), fp64."""
    codes = np.ascontiguousarray(codes, np.int8)
    e8m0 = np.ascontiguousarray(e8m0, np.uint8)
    so = np.ascontiguousarray(slot_of, np.int32)
    g = np.ascontiguousarray(gates, np.float32)
    M, H = codes.shape
    T, k = so.shape
    out = np.zeros((T, H), np.float64)
    lib().orc_moe_combine_s2f6(_p(codes), _p(e8m0), M, H, mask, _p(so), _p(g), T, k, _p(out))
    return out


def gemm_nvfp4_grouped(xq, wq, offsets, N, K, gather=None):
    o = np.ascontiguousarray(offsets, np.int64)
    G = len(o) - 1
    M = int(o[-1])
    g = None if gather is None else np.ascontiguousarray(gather, np.int32)
    Y = np.zeros((M, N), np.float32)
    lib().orc_gemm_nvfp4_grouped(_p(np.ascontiguousarray(xq["codes"])), _p(np.ascontiguousarray(xq["scales"])),
                                 _p(np.ascontiguousarray(xq["outer"], np.float32)), xq["rows_per_outer"], _p(g),
                                 _p(np.ascontiguousarray(wq["codes"])), _p(np.ascontiguousarray(wq["scales"])),
                                 _p(np.ascontiguousarray(wq["outer"], np.float32)), wq["rows_per_outer"],
                                 _p(o), G, N, K, _p(Y))
    return Y


def gemm_nvfp4_elems(xq, wq, offsets, N, K, rows, cols, gather=None):
    """Sampled outputs (s, n) of the NVFP4 grouped forward, fp64."""
    o = np.ascontiguousarray(offsets, np.int64)
    g = None if gather is None else np.ascontiguousarray(gather, np.int32)
    arrs = [np.ascontiguousarray(a) for a in (xq["codes"], xq["scales"])]
    xo = np.ascontiguousarray(xq["outer"], np.float32)
    warr = [np.ascontiguousarray(a) for a in (wq["codes"], wq["scales"])]
    wo = np.ascontiguousarray(wq["outer"], np.float32)
    f = lib().orc_gemm_nvfp4_elem
    return np.array([f(_p(arrs[0]), _p(arrs[1]), _p(xo), xq["rows_per_outer"], _p(g), _p(warr[0]), _p(warr[1]),
                       _p(wo), wq["rows_per_outer"], _p(o), len(o) - 1, N, K, int(s), int(n))
                     for s, n in zip(rows, cols)])


def gemm_mxfp8_fwd(xq, xe, wq, we, offsets, N, K, gather=None):
    """MXFP8 grouped forward, fp64: Y[s, n] = sum_k X[gather[s] or s, k] W[g N + n, k]."""
    o = np.ascontiguousarray(offsets, np.int64)
    G = len(o) - 1
    g = None if gather is None else np.ascontiguousarray(gather, np.int32)
    Y = np.zeros((int(o[-1]), N), np.float64)
    arrs = [np.ascontiguousarray(a) for a in (xq, xe, wq, we)]
    lib().orc_gemm_mxfp8_fwd(_p(arrs[0]), _p(arrs[1]), _p(g), _p(arrs[2]), _p(arrs[3]), _p(o), G, N, K, _p(Y))
    return Y


def gemm_mxfp8_dgrad(dq, de, wt, wte, offsets, N, K, target=TARGET_E4M3):
    o = np.ascontiguousarray(offsets, np.int64)
    G = len(o) - 1
    dX = np.zeros((int(o[-1]), K), np.float32)
    lib().orc_gemm_mx_dgrad(*[_p(np.ascontiguousarray(a)) for a in (dq, de, wt, wte, o)], G, N, K, target, _p(dX))
    return dX


def gemm_mxfp8_wgrad(dt, dte, xt, xte, offsets, N, K, target=TARGET_E4M3):
    o = np.ascontiguousarray(offsets, np.int64)
    G = len(o) - 1
    dW = np.zeros((G * N, K), np.float32)
    lib().orc_gemm_mx_wgrad(*[_p(np.ascontiguousarray(a)) for a in (dt, dte, xt, xte, o)], G, N, K, target, _p(dW))
    return dW


def mxfp8_dot(a, ae, b, be, m, n, k0, kn, target=TARGET_E4M3):
    a, ae, b, be = (np.ascontiguousarray(t) for t in (a, ae, b, be))
    return lib().orc_mx_dot(_p(a), _p(ae), a.shape[1], _p(b), _p(be), b.shape[1], m, n, k0, kn, target)


def swiglu(h13, F):
    h = np.ascontiguousarray(h13, np.float32)
    M = h.shape[0]
    a = np.zeros((M, F), np.float64)
    lib().orc_swiglu(_p(h), M, F, _p(a))
    return a


def swiglu_bwd(da, h13_bf16, F):
    d = np.ascontiguousarray(da, np.float32)
    h = _u16(h13_bf16)
    M = d.shape[0]
    out = np.zeros((M, 2 * F), np.float64)
    lib().orc_swiglu_bwd(_p(d), _p(h), M, F, _p(out))
    return out


def route_topk(logits, k):
    l = np.ascontiguousarray(logits, np.float32)
    T, E = l.shape
    ids = np.zeros((T, k), np.int32)
    gates = np.zeros((T, k), np.float32)
    offsets = np.zeros(E + 1, np.int64)
    gather = np.zeros(T * k, np.int32)
    slot_of = np.zeros(T * k, np.int32)
    lib().orc_route_topk(_p(l), T, E, k, _p(ids), _p(gates), _p(offsets), _p(gather), _p(slot_of))
    return dict(ids=ids, gates=gates, offsets=offsets, gather=gather, slot_of=slot_of)


def bf16_to_f32(h: int) -> float:
    return lib().orc_bf16_to_f32(h)


def f32_to_bf16(f: float) -> int:
    return lib().orc_f32_to_bf16(f)
