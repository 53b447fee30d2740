"""Quantized MoE expert layer for AMD Instinct MI355X (gfx950).

Python binding of the C ABI in include/pmn.h (libpmn.so, built by ``build.py``). The functions
below have the ABI's names and only marshal arguments: they allocate outputs with torch on the
current device, pass raw pointers and torch's current HIP stream, and check the status code.
Every step of the computation runs in the library's HIP kernels; if the library is not built
the import fails.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpmn.so")

P, I64, I32, U32, U64, SZ = C.c_void_p, C.c_int64, C.c_int, C.c_uint32, C.c_uint64, C.c_size_t

_SIGS = {
    "pmn_strerror": (C.c_char_p, [I32]),
    "pmn_version": (I32, []),
    "pmn_padded_bound": (I64, [I64, I32]),
    "nvfp4_quantize": (I32, [P, I64, I64, I32, I64, P, P, P, P, P]),
    "nvfp4_quantize_ws_size": (SZ, []),
    "nvfp4_quantize_ws": (I32, [P, I64, I64, I32, I64, P, P, P, P, P, SZ, P]),
    "nvfp4_quantize_weights_bwd": (I32, [P, I64, I64, I64, P, P, P, P, P, U64, U32, P, SZ, P]),
    "requant_transpose_sr_mxfp8": (I32, [P, P, P, I64, I64, I64, P, I64, P, I32, I32, U64, U32, P, P, I64, P, P]),
    "mxfp8_quantize": (I32, [P, I64, I64, I32, P, I32, I32, U64, U32, P, P, I64, P, P]),
    "rht32_s2f6_quantize": (I32, [P, I32, I64, I64, U32, P, P, P]),
    "moe_grouped_gemm_fwd": (I32, [P, P, P, I64, I64, P, P, P, P, I64, P, I32, I64, I64, I64, I32, U32, P, P, P, P]),
    "moe_grouped_gemm_bwd_workspace_size": (SZ, [I64, I32, I64, I64, I32]),
    "moe_grouped_gemm_bwd": (I32, [P, P, P, P, I64, I64, P, P, P, P, I64, P, I32, I64, I64, I64, I32, I32, U64,
                                   U32, U32, U32, P, P, P, SZ, P]),
    "moe_grouped_gemm_bwd_swiglu": (I32, [P, P, P, P, P, I64, I64, P, P, P, P, I64, P, I32, I64, I64, I64, I32, U64,
                                          U32, U32, P, P, P, SZ, P]),
    "moe_grouped_gemm_fwd_mxfp8_workspace_size": (SZ, [I64, I32, I64, I64]),
    "moe_grouped_gemm_fwd_mxfp8": (I32, [P, I64, P, P, P, I32, I64, I64, I64, I32, U32, P, P, P, P, SZ, P]),
    "swiglu_bwd": (I32, [P, P, I64, I64, P, P]),
    "moe_route_topk": (I32, [P, I64, I32, I32, P, P, P, P, P, P]),
    "moe_combine_s2f6": (I32, [P, P, I64, I64, U32, P, P, I64, I32, P, P]),
    "pmn_check_indices": (I32, [P, I32, I64, P, I64, I64, P, P]),
    "pmn_noalloc_scratch_bytes": (SZ, []),
    "moe_grouped_gemm_bwd_noalloc": (I32, [P, P, P, P, I64, I64, P, P, P, P, I64, P, I32, I64, I64, I64, I32, I32,
                                           U64, U32, U32, U32, P, P, P]),
    # measurement kernels (include/pmn_probe.h)
    "pmn_probe_stream": (I32, [P, P, I64, I32, I32, I32, I32, P]),
    "pmn_probe_mfma_sink_floats": (SZ, [I32, I32]),
    "pmn_probe_mfma": (I32, [I32, I32, I32, I32, P, P, P]),
    "pmn_probe_recip_check": (I32, [U32, U32, P, P]),
}

ABI_FUNCTIONS = tuple(n for n in _SIGS if not n.startswith("pmn_"))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()

# ---- constants of include/pmn.h -------------------------------------------------------------
NVFP4_WEIGHT, NVFP4_ACT, NVFP4_WEIGHT_2D = 0, 1, 2
TARGET_E4M3, TARGET_E2M1 = 0, 1
ROWWISE, COLWISE = 0, 1
RNE, SR = 0, 1
DTYPE_BF16, DTYPE_F32 = 0, 1
EPI_F32, EPI_BF16, EPI_SWIGLU, EPI_RHT32_S2F6 = 0, 1, 2, 3
BWD_DGRAD, BWD_WGRAD, BWD_FP4, BWD_W_PREPARED = 1, 2, 4, 8


CHECK_OFFSETS_START, CHECK_OFFSETS_END, CHECK_OFFSETS_ORDER, CHECK_OFFSETS_RANGE, CHECK_GATHER_RANGE = 1, 2, 4, 8, 16
_CHECK_RULES = ((CHECK_OFFSETS_START, "offsets[0] != 0"), (CHECK_OFFSETS_END, "offsets[G] != M"),
                (CHECK_OFFSETS_ORDER, "offsets decrease"), (CHECK_OFFSETS_RANGE, "an offset outside [0, M]"),
                (CHECK_GATHER_RANGE, "a gather index outside the gathered matrix"))

# PMN_CHECK_INDICES=1 in the environment: every grouped call first checks its device index arrays
# with pmn_check_indices (one small launch and a synchronization) and refuses bad ones
CHECK_INDICES = os.environ.get("PMN_CHECK_INDICES", "") not in ("", "0")


class PmnError(RuntimeError):
    pass


def _check(st: int, what: str):
    if st != 0:
        raise PmnError(f"{what}: {_lib.pmn_strerror(st).decode()} (status {st})")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise PmnError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise PmnError("tensor must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


# ---- argument checks of the binding: the C ABI takes sizes as integers and cannot see the
# tensors, so tensors whose shape or dtype disagrees with those integers are refused here
def _need(cond: bool, what: str):
    if not cond:
        raise PmnError(what)


def _tensor(t: Optional[torch.Tensor], shape, dtype, name: str):
    _need(t is not None and t.dtype == dtype and tuple(t.shape) == tuple(shape),
          f"{name} must be {dtype} of shape {tuple(shape)}"
          + ("" if t is None else f", got {t.dtype} of shape {tuple(t.shape)}"))


def _index(t: Optional[torch.Tensor], n: int, dtype, name: str):
    if t is not None:
        _need(t.dtype == dtype and t.numel() == n, f"{name} must hold {n} values of {dtype}")


def _nvfp4(q: "NVFP4", name: str):
    _need(q.codes.dtype == torch.uint8 and q.codes.dim() == 2, f"{name}.codes must be uint8 [rows, cols/2]")
    R, C = q.rows, q.cols
    _tensor(q.scales, (R, C // 16), torch.uint8, f"{name}.scales")
    _need(q.rows_per_outer >= 1 and q.outer.dtype == torch.float32 and q.outer.numel() * q.rows_per_outer >= R,
          f"{name}.outer must be fp32 with one value per {q.rows_per_outer} rows")


def check_indices(offsets: Optional[torch.Tensor] = None, M: int = 0, gather: Optional[torch.Tensor] = None,
                  src_rows: int = 0) -> int:
    """pmn_check_indices: the mask of CHECK_* rules that the device arrays offsets [G+1] (int64)
    and gather (int32, indexing a matrix of src_rows rows) break, 0 if none. Synchronizes."""
    _need(offsets is not None or gather is not None, "check_indices needs offsets or gather")
    _need(offsets is None or (offsets.dtype == torch.int64 and offsets.numel() >= 2), "offsets must be int64 [G+1]")
    _need(gather is None or gather.dtype == torch.int32, "gather must be int32")
    dev = (offsets if offsets is not None else gather).device
    res = torch.empty(1, dtype=torch.int32, device=dev)
    G = offsets.numel() - 1 if offsets is not None else 0
    n = gather.numel() if gather is not None else 0
    _check(_lib.pmn_check_indices(_ptr(offsets), G, M, _ptr(gather), n, src_rows, _ptr(res), _stream()),
           "pmn_check_indices")
    return int(res.item()) & 0xFFFFFFFF


def _debug_indices(what: str, offsets, M: int, gather=None, src_rows: int = 0):
    if not CHECK_INDICES or (offsets is None and gather is None):
        return
    bad = check_indices(offsets, M, gather, src_rows)
    if bad:
        raise PmnError(f"{what}: the device index arrays break the contract: "
                       + ", ".join(t for b, t in _CHECK_RULES if bad & b))


def version() -> int:
    return _lib.pmn_version()


def padded_bound(M: int, G: int) -> int:
    return _lib.pmn_padded_bound(M, G)


@dataclass
class NVFP4:
    """An NVFP4 matrix [rows x cols]: codes u8 [rows, cols/2], scales u8 (E4M3) [rows, cols/16],
    outer fp32 [rows / rows_per_outer]."""
    codes: torch.Tensor
    scales: torch.Tensor
    outer: torch.Tensor
    rows_per_outer: int

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def cols(self) -> int:
        return self.codes.shape[1] * 2


def nvfp4_quantize_ws_size() -> int:
    return _lib.nvfp4_quantize_ws_size()


def nvfp4_quantize(x: torch.Tensor, mode: int = NVFP4_ACT, rows_per_outer: int = 1,
                   outer_in: Optional[torch.Tensor] = None, out: Optional[NVFP4] = None,
                   workspace: Optional[torch.Tensor] = None) -> NVFP4:
    """NVFP4 of x; `out` (optional) supplies the output tensors to write into. With `workspace`
    (uint8, at least nvfp4_quantize_ws_size() bytes) the call goes through nvfp4_quantize_ws: the
    same outputs, weights taken in one read of x."""
    _need(x.dtype == torch.bfloat16 and x.dim() == 2, "x must be bf16 [rows, cols]")
    R, Cc = x.shape
    dev = x.device
    n_outer = max(R // max(rows_per_outer, 1), 0)
    if out is None:
        codes = torch.empty((R, Cc // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((R, Cc // 16), dtype=torch.uint8, device=dev)
        outer = torch.empty((n_outer,), dtype=torch.float32, device=dev)
    else:
        codes, scales, outer = out.codes, out.scales, out.outer
        _tensor(codes, (R, Cc // 2), torch.uint8, "out.codes")
        _tensor(scales, (R, Cc // 16), torch.uint8, "out.scales")
        _tensor(outer, (n_outer,), torch.float32, "out.outer")
    if workspace is None:
        _check(_lib.nvfp4_quantize(_ptr(x), R, Cc, mode, rows_per_outer, _ptr(outer_in), _ptr(codes),
                                   _ptr(scales), _ptr(outer), _stream()), "nvfp4_quantize")
    else:
        _need(workspace.dtype == torch.uint8, "workspace must be uint8")
        _check(_lib.nvfp4_quantize_ws(_ptr(x), R, Cc, mode, rows_per_outer, _ptr(outer_in), _ptr(codes),
                                      _ptr(scales), _ptr(outer), _ptr(workspace), workspace.numel(), _stream()),
               "nvfp4_quantize_ws")
    return NVFP4(codes, scales, outer, rows_per_outer)


@dataclass
class WeightsBwd:
    """Weights quantized for both passes (nvfp4_quantize_weights_bwd): q, the NVFP4 matrix for
    the forward, and the backward's W^T operand, wt u8 [cols, rows] (E4M3 codes, blocked layout)
    with wte u8 [rows/32, cols] (E8M0), drawn with (seed, rng_stream). The backward calls take it
    in place of the NVFP4 weights."""
    q: NVFP4
    wt: torch.Tensor
    wte: torch.Tensor
    seed: int
    rng_stream: int


def nvfp4_quantize_weights_bwd(w: torch.Tensor, rows_per_outer: int, seed: int = 0, rng_stream: int = 2,
                               workspace: Optional[torch.Tensor] = None) -> WeightsBwd:
    """nvfp4_quantize_weights_bwd: w bf16 [rows, cols] (rows % 64 == 0) in weight mode with one
    outer scale per rows_per_outer rows, and its W^T operand for the backward's dgrad."""
    _need(w.dtype == torch.bfloat16 and w.dim() == 2, "w must be bf16 [rows, cols]")
    R, Cc = w.shape
    dev = w.device
    if workspace is None:
        workspace = torch.empty((nvfp4_quantize_ws_size(),), dtype=torch.uint8, device=dev)
    _need(workspace.dtype == torch.uint8, "workspace must be uint8")
    codes = torch.empty((R, Cc // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((R, Cc // 16), dtype=torch.uint8, device=dev)
    outer = torch.empty((R // max(rows_per_outer, 1),), dtype=torch.float32, device=dev)
    wt = torch.empty((Cc, R), dtype=torch.uint8, device=dev)
    wte = torch.empty((R // 32, Cc), dtype=torch.uint8, device=dev)
    _check(_lib.nvfp4_quantize_weights_bwd(_ptr(w), R, Cc, rows_per_outer, _ptr(codes), _ptr(scales), _ptr(outer),
                                           _ptr(wt), _ptr(wte), seed, rng_stream, _ptr(workspace),
                                           workspace.numel(), _stream()), "nvfp4_quantize_weights_bwd")
    return WeightsBwd(NVFP4(codes, scales, outer, rows_per_outer), wt, wte, seed, rng_stream)


def _bwd_weights(wq, G: int, N: int, K: int):
    """(codes, scales, outer, rows_per_outer, extra flags) of the backward's weight operand: the
    NVFP4 weights, or a WeightsBwd's prepared W^T (PMN_BWD_W_PREPARED)."""
    if isinstance(wq, WeightsBwd):
        _need(wq.q.cols == K and wq.q.rows == G * N, f"wq must be [G*N, K] = [{G * N}, {K}]")
        _tensor(wq.wt, (K, G * N), torch.uint8, "wq.wt")
        _tensor(wq.wte, (G * N // 32, K), torch.uint8, "wq.wte")
        return _ptr(wq.wt), _ptr(wq.wte), None, 1, BWD_W_PREPARED
    _nvfp4(wq, "wq")
    _need(wq.cols == K and wq.rows == G * N, f"wq must be [G*N, K] = [{G * N}, {K}], got [{wq.rows}, {wq.cols}]")
    return _ptr(wq.codes), _ptr(wq.scales), _ptr(wq.outer), wq.rows_per_outer, 0


def requant_transpose_sr_mxfp8(q: NVFP4, gather: Optional[torch.Tensor] = None,
                               offsets: Optional[torch.Tensor] = None, M: Optional[int] = None,
                               target: int = TARGET_E4M3, seed: int = 0, rng_stream: int = 0,
                               ld: Optional[int] = None, want_padded_offsets: bool = False,
                               out: Optional[torch.Tensor] = None, out_e8m0: Optional[torch.Tensor] = None):
    """Returns (out [cols, ld] u8, out_e8m0 [cols, ld/32] u8, padded_offsets or None); columns
    past the padded total are not written."""
    if M is None:
        M = gather.numel() if gather is not None else q.rows
    G = 0 if offsets is None else offsets.numel() - 1
    if ld is None:
        ld = padded_bound(M, G)
    dev = q.codes.device
    _nvfp4(q, "q")
    _index(gather, M, torch.int32, "gather")
    _index(offsets, G + 1, torch.int64, "offsets")
    _debug_indices("requant_transpose_sr_mxfp8", offsets, M, gather, q.rows)
    out = torch.empty((q.cols, ld), dtype=torch.uint8, device=dev) if out is None else out
    oe = torch.empty((q.cols, ld // 32), dtype=torch.uint8, device=dev) if out_e8m0 is None else out_e8m0
    _tensor(out, (q.cols, ld), torch.uint8, "out")
    _tensor(oe, (q.cols, ld // 32), torch.uint8, "out_e8m0")
    po = torch.zeros((max(G, 1) + 1,), dtype=torch.int64, device=dev) if want_padded_offsets else None
    _check(_lib.requant_transpose_sr_mxfp8(_ptr(q.codes), _ptr(q.scales), _ptr(q.outer), q.rows, q.cols,
                                           q.rows_per_outer, _ptr(gather), M, _ptr(offsets), G, target, seed,
                                           rng_stream, _ptr(out), _ptr(oe), ld, _ptr(po), _stream()),
           "requant_transpose_sr_mxfp8")
    return out, oe, po


def mxfp8_quantize(x: torch.Tensor, layout: int = ROWWISE, offsets: Optional[torch.Tensor] = None,
                   rounding: int = RNE, seed: int = 0, rng_stream: int = 0, ld: Optional[int] = None,
                   want_padded_offsets: bool = False):
    _need(x.dtype == torch.bfloat16 and x.dim() == 2, "x must be bf16 [M, N]")
    M, N = x.shape
    dev = x.device
    G = 0 if offsets is None else offsets.numel() - 1
    _index(offsets, G + 1, torch.int64, "offsets")
    _debug_indices("mxfp8_quantize", offsets, M)
    po = None
    if layout == ROWWISE:
        out = torch.empty((M, N), dtype=torch.uint8, device=dev)
        oe = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
        ld = N
    else:
        if ld is None:
            ld = padded_bound(M, G)
        out = torch.empty((N, ld), dtype=torch.uint8, device=dev)
        oe = torch.empty((N, ld // 32), dtype=torch.uint8, device=dev)
        po = torch.zeros((max(G, 1) + 1,), dtype=torch.int64, device=dev) if want_padded_offsets else None
    _check(_lib.mxfp8_quantize(_ptr(x), M, N, layout, _ptr(offsets), G, rounding, seed, rng_stream, _ptr(out),
                               _ptr(oe), ld, _ptr(po), _stream()), "mxfp8_quantize")
    return out, oe, po


def rht32_s2f6_quantize(x: torch.Tensor, sign_mask: int):
    _need(x.dim() == 2 and x.dtype in (torch.bfloat16, torch.float32), "x must be bf16 or fp32 [rows, cols]")
    R, Cc = x.shape
    codes = torch.empty((R, Cc), dtype=torch.int8, device=x.device)
    e = torch.empty((R, Cc // 32), dtype=torch.uint8, device=x.device)
    _check(_lib.rht32_s2f6_quantize(_ptr(x), DTYPE_F32 if x.dtype == torch.float32 else DTYPE_BF16, R, Cc,
                                    sign_mask & 0xFFFFFFFF, _ptr(codes), _ptr(e), _stream()), "rht32_s2f6_quantize")
    return codes, e


def moe_grouped_gemm_fwd(xq: NVFP4, wq: NVFP4, offsets: torch.Tensor, M: int, N: int,
                         epilogue: int = EPI_F32, gather: Optional[torch.Tensor] = None,
                         rht_sign_mask: int = 0, save_h13: bool = False, out=None, out_e8m0=None,
                         out_aux=None):
    """Y = grouped NVFP4 product; returns the epilogue's outputs (see include/pmn.h)."""
    K = xq.cols
    G = offsets.numel() - 1
    dev = xq.codes.device
    _nvfp4(xq, "xq")
    _nvfp4(wq, "wq")
    _need(wq.cols == K and wq.rows == G * N, f"wq must be [G*N, K] = [{G * N}, {K}], got [{wq.rows}, {wq.cols}]")
    _index(offsets, G + 1, torch.int64, "offsets")
    _index(gather, M, torch.int32, "gather")
    _debug_indices("moe_grouped_gemm_fwd", offsets, M, gather, xq.rows)
    if out is None:
        if epilogue == EPI_F32:
            out = torch.empty((M, N), dtype=torch.float32, device=dev)
        elif epilogue == EPI_BF16:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        elif epilogue == EPI_SWIGLU:
            out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
        else:
            out = torch.empty((M, N), dtype=torch.int8, device=dev)
    if epilogue == EPI_RHT32_S2F6 and out_e8m0 is None:
        out_e8m0 = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
    if epilogue == EPI_SWIGLU and save_h13 and out_aux is None:
        out_aux = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _epilogue_outputs(epilogue, M, N, out, out_e8m0, out_aux)
    _check(_lib.moe_grouped_gemm_fwd(_ptr(xq.codes), _ptr(xq.scales), _ptr(xq.outer), xq.rows, xq.rows_per_outer,
                                     _ptr(gather), _ptr(wq.codes), _ptr(wq.scales), _ptr(wq.outer),
                                     wq.rows_per_outer, _ptr(offsets), G, M, N, K, epilogue,
                                     rht_sign_mask & 0xFFFFFFFF, _ptr(out), _ptr(out_e8m0), _ptr(out_aux), _stream()),
           "moe_grouped_gemm_fwd")
    if epilogue == EPI_RHT32_S2F6:
        return out, out_e8m0
    if epilogue == EPI_SWIGLU:
        return out, out_aux
    return out


def _epilogue_outputs(epilogue: int, M: int, N: int, out, out_e8m0, out_aux):
    shape, dtype = {EPI_F32: ((M, N), torch.float32), EPI_BF16: ((M, N), torch.bfloat16),
                    EPI_SWIGLU: ((M, N // 2), torch.bfloat16)}.get(epilogue, ((M, N), torch.int8))
    _tensor(out, shape, dtype, "out")
    if epilogue == EPI_RHT32_S2F6:
        _tensor(out_e8m0, (M, N // 32), torch.uint8, "out_e8m0")
    if epilogue == EPI_SWIGLU and out_aux is not None:
        _tensor(out_aux, (M, N), torch.bfloat16, "out_aux")


def moe_grouped_gemm_bwd_workspace_size(M: int, G: int, N: int, K: int, flags: int) -> int:
    return _lib.moe_grouped_gemm_bwd_workspace_size(M, G, N, K, flags)


def moe_grouped_gemm_fwd_mxfp8(x: torch.Tensor, w: torch.Tensor, offsets: torch.Tensor, M: int, N: int,
                               epilogue: int = EPI_F32, gather: Optional[torch.Tensor] = None,
                               rht_sign_mask: int = 0, save_h13: bool = False, workspace=None, out=None,
                               out_e8m0=None, out_aux=None):
    """MXFP8 forward (row-wise RNE quantization of x and w inside the call); returns the
    epilogue's outputs as moe_grouped_gemm_fwd does."""
    K = x.shape[1]
    G = offsets.numel() - 1
    dev = w.device
    _need(x.dtype == torch.bfloat16 and x.dim() == 2, "x must be bf16 [rows, K]")
    _tensor(w, (G * N, K), torch.bfloat16, "w")
    _index(offsets, G + 1, torch.int64, "offsets")
    _index(gather, M, torch.int32, "gather")
    _debug_indices("moe_grouped_gemm_fwd_mxfp8", offsets, M, gather, x.shape[0])
    if workspace is None:
        workspace = torch.empty((_lib.moe_grouped_gemm_fwd_mxfp8_workspace_size(M, G, N, K),), dtype=torch.uint8,
                                device=dev)
    if out is None:
        if epilogue == EPI_F32:
            out = torch.empty((M, N), dtype=torch.float32, device=dev)
        elif epilogue == EPI_BF16:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        elif epilogue == EPI_SWIGLU:
            out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=dev)
        else:
            out = torch.empty((M, N), dtype=torch.int8, device=dev)
    if epilogue == EPI_RHT32_S2F6 and out_e8m0 is None:
        out_e8m0 = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
    if epilogue == EPI_SWIGLU and save_h13 and out_aux is None:
        out_aux = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _epilogue_outputs(epilogue, M, N, out, out_e8m0, out_aux)
    _need(workspace.dtype == torch.uint8 and workspace.dim() == 1, "workspace must be a 1-D uint8 tensor")
    _check(_lib.moe_grouped_gemm_fwd_mxfp8(_ptr(x), x.shape[0], _ptr(gather), _ptr(w), _ptr(offsets), G, M, N, K,
                                           epilogue, rht_sign_mask & 0xFFFFFFFF, _ptr(out), _ptr(out_e8m0),
                                           _ptr(out_aux), _ptr(workspace), workspace.numel(), _stream()),
           "moe_grouped_gemm_fwd_mxfp8")
    if epilogue == EPI_RHT32_S2F6:
        return out, out_e8m0
    if epilogue == EPI_SWIGLU:
        return out, out_aux
    return out


def moe_grouped_gemm_bwd(dy: torch.Tensor, xq: NVFP4, wq, offsets: torch.Tensor, M: int, N: int,
                         flags: int = BWD_DGRAD | BWD_WGRAD, gather: Optional[torch.Tensor] = None,
                         dy_rounding: int = RNE, seed: int = 0, rng_stream_a: int = 1, rng_stream_b: int = 2,
                         rng_stream_dy: int = 3, workspace: Optional[torch.Tensor] = None, da=None, db=None):
    """wq: the NVFP4 weights [G*N, K], or a WeightsBwd (its prepared W^T, PMN_BWD_W_PREPARED).
    Returns (da [M, K] fp32 or None, db [G*N, K] fp32 or None, workspace)."""
    K = xq.cols
    G = offsets.numel() - 1
    dev = dy.device
    _tensor(dy, (M, N), torch.bfloat16, "dy")
    _nvfp4(xq, "xq")
    bc, bs, bo, brpo, wflag = _bwd_weights(wq, G, N, K)
    flags |= wflag
    _index(offsets, G + 1, torch.int64, "offsets")
    _index(gather, M, torch.int32, "gather")
    _debug_indices("moe_grouped_gemm_bwd", offsets, M, gather, xq.rows)
    ws_bytes = moe_grouped_gemm_bwd_workspace_size(M, G, N, K, flags)
    if workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    if da is None and flags & BWD_DGRAD:
        da = torch.empty((M, K), dtype=torch.float32, device=dev)
    if db is None and flags & BWD_WGRAD:
        db = torch.empty((G * N, K), dtype=torch.float32, device=dev)
    if flags & BWD_DGRAD:
        _tensor(da, (M, K), torch.float32, "da")
    if flags & BWD_WGRAD:
        _tensor(db, (G * N, K), torch.float32, "db")
    _need(workspace.dtype == torch.uint8 and workspace.dim() == 1, "workspace must be a 1-D uint8 tensor")
    _check(_lib.moe_grouped_gemm_bwd(_ptr(dy), _ptr(xq.codes), _ptr(xq.scales), _ptr(xq.outer), xq.rows,
                                     xq.rows_per_outer, _ptr(gather), bc, bs, bo, brpo, _ptr(offsets), G, M, N, K,
                                     flags, dy_rounding, seed,
                                     rng_stream_a, rng_stream_b, rng_stream_dy, _ptr(da), _ptr(db),
                                     _ptr(workspace), workspace.numel(), _stream()), "moe_grouped_gemm_bwd")
    return da, db, workspace


def moe_grouped_gemm_bwd_swiglu(da_act: torch.Tensor, h13: torch.Tensor, xq: NVFP4, wq,
                                offsets: torch.Tensor, M: int, N: int, gather: Optional[torch.Tensor] = None,
                                seed: int = 0, rng_stream_a: int = 1, rng_stream_b: int = 2,
                                workspace: Optional[torch.Tensor] = None, dx=None, dw=None):
    """The w1||w3 backward with the SwiGLU backward folded into dY's quantization: the results of
    swiglu_bwd(da_act, h13) followed by moe_grouped_gemm_bwd(..., both gradients, RNE).
    Returns (dx [M, K] fp32, dw [G*N, K] fp32, workspace)."""
    K = xq.cols
    G = offsets.numel() - 1
    dev = h13.device
    _tensor(da_act, (M, N // 2), torch.float32, "da_act")
    _tensor(h13, (M, N), torch.bfloat16, "h13")
    _nvfp4(xq, "xq")
    bc, bs, bo, brpo, wflag = _bwd_weights(wq, G, N, K)
    _index(offsets, G + 1, torch.int64, "offsets")
    _index(gather, M, torch.int32, "gather")
    _debug_indices("moe_grouped_gemm_bwd_swiglu", offsets, M, gather, xq.rows)
    ws_bytes = moe_grouped_gemm_bwd_workspace_size(M, G, N, K, BWD_DGRAD | BWD_WGRAD)
    if workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    dx = torch.empty((M, K), dtype=torch.float32, device=dev) if dx is None else dx
    dw = torch.empty((G * N, K), dtype=torch.float32, device=dev) if dw is None else dw
    _tensor(dx, (M, K), torch.float32, "dx")
    _tensor(dw, (G * N, K), torch.float32, "dw")
    _need(workspace.dtype == torch.uint8 and workspace.dim() == 1, "workspace must be a 1-D uint8 tensor")
    _check(_lib.moe_grouped_gemm_bwd_swiglu(_ptr(da_act), _ptr(h13), _ptr(xq.codes), _ptr(xq.scales), _ptr(xq.outer),
                                            xq.rows, xq.rows_per_outer, _ptr(gather), bc, bs, bo, brpo,
                                            _ptr(offsets), G, M, N, K, wflag, seed, rng_stream_a, rng_stream_b,
                                            _ptr(dx), _ptr(dw),
                                            _ptr(workspace), workspace.numel(), _stream()),
           "moe_grouped_gemm_bwd_swiglu")
    return dx, dw, workspace


def moe_grouped_gemm_bwd_noalloc(dy: torch.Tensor, xq: "NVFP4", wq, offsets: torch.Tensor, M: int, N: int,
                                 flags: int = BWD_DGRAD | BWD_WGRAD, gather: Optional[torch.Tensor] = None,
                                 dy_rounding: int = RNE, seed: int = 0, rng_stream_a: int = 1, rng_stream_b: int = 2,
                                 rng_stream_dy: int = 3, da=None, db=None):
    """moe_grouped_gemm_bwd with the library's static scratch as its workspace (no workspace
    argument; the C call allocates nothing). Returns (da or None, db or None)."""
    K = xq.cols
    G = offsets.numel() - 1
    dev = dy.device
    _tensor(dy, (M, N), torch.bfloat16, "dy")
    _nvfp4(xq, "xq")
    bc, bs, bo, brpo, wflag = _bwd_weights(wq, G, N, K)
    flags |= wflag
    _index(offsets, G + 1, torch.int64, "offsets")
    _index(gather, M, torch.int32, "gather")
    _debug_indices("moe_grouped_gemm_bwd_noalloc", offsets, M, gather, xq.rows)
    if da is None and flags & BWD_DGRAD:
        da = torch.empty((M, K), dtype=torch.float32, device=dev)
    if db is None and flags & BWD_WGRAD:
        db = torch.empty((G * N, K), dtype=torch.float32, device=dev)
    if flags & BWD_DGRAD:
        _tensor(da, (M, K), torch.float32, "da")
    if flags & BWD_WGRAD:
        _tensor(db, (G * N, K), torch.float32, "db")
    _check(_lib.moe_grouped_gemm_bwd_noalloc(_ptr(dy), _ptr(xq.codes), _ptr(xq.scales), _ptr(xq.outer), xq.rows,
                                             xq.rows_per_outer, _ptr(gather), bc, bs, bo, brpo, _ptr(offsets), G, M,
                                             N, K, flags,
                                             dy_rounding, seed, rng_stream_a, rng_stream_b, rng_stream_dy, _ptr(da),
                                             _ptr(db), _stream()), "moe_grouped_gemm_bwd_noalloc")
    return da, db


def bwd_workspace_views(workspace: torch.Tensor, M: int, G: int, N: int, K: int, fp4: bool = False):
    """Views of the backward workspace parts, in the order include/pmn.h documents them: groups
    padded to U = 64 slots (E4M3) or 128 (FP4: E2M1 codes packed two per byte, rows of half the
    bytes) and the code parts (dq at padded slot rows, wt, dt, xt) in the blocked layout, viewed
    here as raw bytes of the matrix's shape."""
    U = 128 if fp4 else 64
    Pb = (M + U - 1) // U * U + U * G
    h = 2 if fp4 else 1
    Nk = (N + U - 1) // U * U   # dgrad's contraction: N rounded up to a whole stage (64 E4M3 / 128 E2M1 values)
    sizes = [("dq", Pb * Nk // h, (Pb, Nk // h)), ("de", N // 32 * Pb, (N // 32, Pb)),
             ("wt", K * G * Nk // h, (K, G * Nk // h)), ("wte", K * G * Nk // 32, (G * Nk // 32, K)),
             ("dt", N * Pb // h, (N, Pb // h)), ("dte", N * Pb // 32, (Pb // 32, N)),
             ("xt", K * Pb // h, (K, Pb // h)), ("xte", K * Pb // 32, (Pb // 32, K)), ("po", (G + 1) * 8, None),
             ("woff", (G + 1) * 8, None)]
    off, views = 0, {}
    for name, nbytes, shape in sizes:
        used = nbytes if shape is None else shape[0] * shape[1]
        part = workspace[off:off + used]
        views[name] = part.view(torch.int64) if shape is None else part.view(*shape)
        off += (nbytes + 255) // 256 * 256
    return views


def swiglu_bwd(da: torch.Tensor, h13: torch.Tensor) -> torch.Tensor:
    _need(da.dtype == torch.float32 and da.dim() == 2, "da must be fp32 [M, F]")
    M, F = da.shape
    _tensor(h13, (M, 2 * F), torch.bfloat16, "h13")
    out = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=da.device)
    _check(_lib.swiglu_bwd(_ptr(da), _ptr(h13), M, F, _ptr(out), _stream()), "swiglu_bwd")
    return out


def moe_route_topk(logits: torch.Tensor, k: int):
    """Returns dict(ids, gates, offsets, gather, slot_of) on the device."""
    _need(logits.dtype == torch.float32 and logits.dim() == 2, "logits must be fp32 [T, E]")
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int64, device=dev)
    gather = torch.empty((T * k,), dtype=torch.int32, device=dev)
    slot_of = torch.empty((T * k,), dtype=torch.int32, device=dev)
    _check(_lib.moe_route_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(gates), _ptr(offsets), _ptr(gather),
                               _ptr(slot_of), _stream()), "moe_route_topk")
    return dict(ids=ids, gates=gates, offsets=offsets, gather=gather, slot_of=slot_of)


def moe_combine_s2f6(codes: torch.Tensor, e8m0: torch.Tensor, sign_mask: int, slot_of: torch.Tensor,
                     gates: torch.Tensor, out=None):
    """Receiver side of the combine: bf16 [T x H], row t = sum_j gates[t, j] * decode(codes[slot_of[t, j]])."""
    _need(codes.dtype == torch.int8 and codes.dim() == 2, "codes must be int8 [M, H]")
    M, H = codes.shape
    _tensor(e8m0, (M, H // 32), torch.uint8, "e8m0")
    _need(gates.dtype == torch.float32 and gates.dim() == 2, "gates must be fp32 [T, k]")
    T, k = gates.shape
    _index(slot_of, T * k, torch.int32, "slot_of")
    _need(slot_of is not None, "slot_of is required")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=codes.device)
    _tensor(out, (T, H), torch.bfloat16, "out")
    _check(_lib.moe_combine_s2f6(_ptr(codes), _ptr(e8m0), M, H, sign_mask & 0xFFFFFFFF, _ptr(slot_of), _ptr(gates),
                                 T, k, _ptr(out), _stream()), "moe_combine_s2f6")
    return out


# ---- measurement kernels of include/pmn_probe.h ---------------------------------------------

PROBE_MFMA_KINDS = {0: "v_mfma_f32_32x32x16_f16", 1: "v_mfma_f32_16x16x32_f16",
                    2: "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3)", 3: "v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3)",
                    4: "v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1)",
                    5: "v_mfma_f32_32x32x16_f16 + FP4 dequantization", 6: "v_mfma_f32_16x16x32_f16 + FP4 dequantization"}


def probe_stream(src: Optional[torch.Tensor], dst: Optional[torch.Tensor], units: int, read_kb: int, write_kb: int,
                 grid: int = 8192, hints: int = 3):
    """Stream `units` units of read_kb KB read from src and write_kb KB written to dst (hints: bit 0
    nontemporal loads, bit 1 nontemporal stores)."""
    if read_kb:
        _need(src is not None and src.numel() * src.element_size() >= units * read_kb * 1024, "src too small")
    if write_kb:
        _need(dst is not None and dst.numel() * dst.element_size() >= units * write_kb * 1024, "dst too small")
    _check(_lib.pmn_probe_stream(_ptr(src) if read_kb else None, _ptr(dst) if write_kb else None, units, read_kb,
                                 write_kb, grid, hints, _stream()), "pmn_probe_stream")


def probe_mfma(kind: int, waves_per_simd: int, workgroups: int, iters: int, sink: torch.Tensor) -> float:
    """Launch the MFMA throughput probe; returns the launch's FLOPs (time it on the current stream)."""
    n = _lib.pmn_probe_mfma_sink_floats(waves_per_simd, workgroups)
    _need(sink.dtype == torch.float32 and sink.numel() >= n, f"sink must hold {n} floats")
    fl = C.c_double(0.0)
    _check(_lib.pmn_probe_mfma(kind, waves_per_simd, workgroups, iters, _ptr(sink), C.byref(fl), _stream()),
           "pmn_probe_mfma")
    return fl.value


def probe_recip_check(first_bits: int, last_bits: int) -> int:
    """Number of fp32 values with bit patterns in [first_bits, last_bits] whose division-free
    reciprocal (the activation quantizer's) differs from the IEEE quotient 1/d."""
    count = torch.zeros(1, dtype=torch.int64, device=torch.device("cuda", torch.cuda.current_device()))
    _check(_lib.pmn_probe_recip_check(first_bits, last_bits, _ptr(count), _stream()), "pmn_probe_recip_check")
    return int(count.item())
