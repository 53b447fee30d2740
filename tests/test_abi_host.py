"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every entry point
that include/pmn.h declares, and rejects bad arguments before launching anything."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_functions():
    names = []
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?(?:int|int64_t|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_five_hot_path_calls():
    names = declared_functions()
    for n in ("nvfp4_quantize", "requant_transpose_sr_mxfp8", "moe_grouped_gemm_fwd", "moe_grouped_gemm_bwd",
              "rht32_s2f6_quantize"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import precision_moe_numerics_amd as P
    lib = C.CDLL(P.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(P.ABI_FUNCTIONS) <= set(declared_functions())


def test_library_has_gfx950_code_only():
    import precision_moe_numerics_amd as P
    data = open(P.LIB_PATH, "rb").read()
    assert b"gfx950" in data
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in data


@pytest.fixture(scope="module")
def lib():
    import precision_moe_numerics_amd as P
    return P._lib


def test_argument_errors_without_launch(lib):
    fake = C.c_void_p(0x1000)     # never dereferenced: every call below fails its host checks
    # bad shapes
    assert lib.nvfp4_quantize(fake, 4, 15, 1, 1, None, fake, fake, fake, None) == -2
    assert lib.nvfp4_quantize(fake, 6, 32, 1, 4, None, fake, fake, fake, None) == -2
    assert lib.nvfp4_quantize(fake, 4, 32, 7, 1, None, fake, fake, fake, None) == -1
    assert lib.nvfp4_quantize(None, 4, 32, 1, 1, None, fake, fake, fake, None) == -1
    assert lib.nvfp4_quantize(C.c_void_p(0x1001), 4, 32, 1, 1, None, fake, fake, fake, None) == -3
    # requant: ld too small for the groups, offsets/G mismatch
    assert lib.requant_transpose_sr_mxfp8(fake, fake, fake, 64, 32, 1, None, 64, fake, 2, 0, 0, 0, fake, fake,
                                          64, None, None) == -2
    assert lib.requant_transpose_sr_mxfp8(fake, fake, fake, 64, 32, 1, None, 64, None, 2, 0, 0, 0, fake, fake,
                                          256, None, None) == -2
    assert lib.requant_transpose_sr_mxfp8(fake, fake, fake, 64, 32, 1, None, 64, None, 0, 5, 0, 0, fake, fake,
                                          64, None, None) == -1
    # rht: cols not a multiple of 32
    assert lib.rht32_s2f6_quantize(fake, 0, 2, 48, 0, fake, fake, None) == -2
    # gemm fwd: N or K not a multiple of 32; SwiGLU with N not a multiple of 64
    assert lib.moe_grouped_gemm_fwd(fake, fake, fake, 64, 1, None, fake, fake, fake, 128, fake, 1, 64, 144, 64, 0,
                                    0, fake, None, None, None) == -2
    assert lib.moe_grouped_gemm_fwd(fake, fake, fake, 64, 1, None, fake, fake, fake, 128, fake, 1, 64, 256, 80, 0,
                                    0, fake, None, None, None) == -2
    assert lib.moe_grouped_gemm_fwd(fake, fake, fake, 64, 1, None, fake, fake, fake, 96, fake, 1, 64, 96, 64, 2,
                                    0, fake, None, None, None) == -2
    assert lib.moe_grouped_gemm_fwd(fake, fake, fake, 64, 1, None, fake, fake, fake, 128, fake, 1, 64, 256, 64, 3,
                                    0, fake, None, None, None) == -1
    # gemm bwd: workspace too small
    ws = lib.moe_grouped_gemm_bwd_workspace_size(64, 1, 256, 256, 3)
    assert ws > 0
    assert lib.moe_grouped_gemm_bwd(fake, fake, fake, fake, 64, 1, None, fake, fake, fake, 256, fake, 1, 64, 256, 256,
                                    3, 0, 0, 1, 2, 3, fake, fake, fake, ws - 1, None) == -4
    assert lib.moe_grouped_gemm_bwd(fake, fake, fake, fake, 64, 1, None, fake, fake, fake, 256, fake, 1, 64, 256, 256,
                                    0, 0, 0, 1, 2, 3, fake, fake, fake, ws, None) == -1
    # routing: k > E
    assert lib.moe_route_topk(fake, 4, 4, 8, fake, fake, fake, fake, fake, None) == -2
    assert lib.pmn_strerror(-4) == b"workspace missing or too small"
    assert lib.pmn_padded_bound(33, 2) == 64 + 64


def test_quantize_with_workspace_argument_errors(lib):
    """nvfp4_quantize_ws checks its shapes like nvfp4_quantize, then its workspace (missing or
    smaller than nvfp4_quantize_ws_size(): PMN_EWORKSPACE; not 16-byte aligned: PMN_EALIGN),
    before any launch."""
    fake = C.c_void_p(0x1000)     # never dereferenced
    n = lib.nvfp4_quantize_ws_size()
    assert n >= 4 * 512 * 4
    assert lib.nvfp4_quantize_ws(fake, 4, 15, 0, 1, None, fake, fake, fake, fake, n, None) == -2
    assert lib.nvfp4_quantize_ws(fake, 4096, 256, 0, 2048, None, fake, fake, fake, None, n, None) == -4
    assert lib.nvfp4_quantize_ws(fake, 4096, 256, 0, 2048, None, fake, fake, fake, fake, n - 1, None) == -4
    assert lib.nvfp4_quantize_ws(fake, 4096, 256, 0, 2048, None, fake, fake, fake, C.c_void_p(0x1008), n, None) == -3
    assert lib.nvfp4_quantize_ws(None, 0, 32, 0, 1, None, None, None, None, None, 0, None) == 0


def test_weights_bwd_argument_errors(lib):
    """nvfp4_quantize_weights_bwd checks shapes (rows a multiple of 64 and of rows_per_outer, cols
    of 16), pointers, the workspace and alignment before any launch; the backward refuses the
    prepared operand with the FP4 variant or an N that is not a multiple of 64, and the SwiGLU
    backward any flag but PMN_BWD_W_PREPARED."""
    fake = C.c_void_p(0x1000)     # never dereferenced
    n = lib.nvfp4_quantize_ws_size()
    args = lambda rows, cols, rpo, wt=fake, ws=fake, nb=n: (fake, rows, cols, rpo, fake, fake, fake, wt, fake, 0, 0, ws,
                                                         nb, None)
    assert lib.nvfp4_quantize_weights_bwd(*args(96, 64, 32)) == -2
    assert lib.nvfp4_quantize_weights_bwd(*args(128, 40, 64)) == -2
    assert lib.nvfp4_quantize_weights_bwd(*args(128, 64, 48)) == -2
    assert lib.nvfp4_quantize_weights_bwd(*args(128, 64, 64, wt=None)) == -1
    assert lib.nvfp4_quantize_weights_bwd(*args(128, 64, 64, ws=None)) == -4
    assert lib.nvfp4_quantize_weights_bwd(*args(128, 64, 64, nb=n - 1)) == -4
    assert lib.nvfp4_quantize_weights_bwd(*args(128, 64, 64, wt=C.c_void_p(0x1008))) == -3
    assert lib.nvfp4_quantize_weights_bwd(*args(0, 64, 64)) == 0
    ws = lib.moe_grouped_gemm_bwd_workspace_size(64, 1, 256, 256, 3)
    bwd = lambda flags, N: lib.moe_grouped_gemm_bwd(fake, fake, fake, fake, 64, 1, None, fake, fake, None, 1, fake, 1,
                                                   64, N, 256, flags, 0, 0, 0, 0, 0, fake, fake, fake, ws, None)
    assert bwd(1 | 8 | 4, 256) == -1
    assert bwd(1 | 8, 288) == -2
    assert bwd(1 | 16, 256) == -1
    swi = lambda flags: lib.moe_grouped_gemm_bwd_swiglu(fake, fake, fake, fake, fake, 64, 1, None, fake, fake, fake,
                                                        1, fake, 1, 64, 256, 256, flags, 0, 0, 0, fake, fake, fake,
                                                        ws, None)
    assert swi(1) == -1 and swi(4) == -1


def test_probe_argument_errors(lib):
    """The MFMA probe refuses unknown kinds (PMN_EINVAL), and the dequantization kinds 5 and 6 at
    two wavefronts per SIMD or with an odd iteration count (PMN_ESHAPE), before any launch."""
    fake = C.c_void_p(0x1000)     # never dereferenced
    fl = C.c_double(0.0)
    assert lib.pmn_probe_mfma(7, 1, 256, 10, fake, C.byref(fl), None) == -1
    assert lib.pmn_probe_mfma(5, 2, 256, 10, fake, C.byref(fl), None) == -2
    assert lib.pmn_probe_mfma(6, 1, 256, 11, fake, C.byref(fl), None) == -2
    assert lib.pmn_probe_mfma(0, 3, 256, 10, fake, C.byref(fl), None) == -2


def test_check_indices_argument_errors(lib):
    """pmn_check_indices refuses, before any launch: no result or neither array (PMN_EINVAL), no
    groups or a negative M with offsets, a negative count or row bound with gather (PMN_ESHAPE),
    and a result not 4-byte aligned (PMN_EALIGN)."""
    fake = C.c_void_p(0x1000)     # never dereferenced
    assert lib.pmn_check_indices(None, 0, 0, None, 0, 0, fake, None) == -1
    assert lib.pmn_check_indices(fake, 1, 4, None, 0, 0, None, None) == -1
    assert lib.pmn_check_indices(fake, 0, 4, None, 0, 0, fake, None) == -2
    assert lib.pmn_check_indices(fake, 2, -1, None, 0, 0, fake, None) == -2
    assert lib.pmn_check_indices(None, 0, 0, fake, -1, 8, fake, None) == -2
    assert lib.pmn_check_indices(None, 0, 0, fake, 4, -8, fake, None) == -2
    assert lib.pmn_check_indices(fake, 1, 4, fake, 4, 8, C.c_void_p(0x1002), None) == -3


def test_zero_size_calls_are_no_ops(lib):
    assert lib.nvfp4_quantize(None, 0, 32, 1, 1, None, None, None, None, None) == 0
    assert lib.rht32_s2f6_quantize(None, 0, 0, 64, 0, None, None, None) == 0


def test_blocked_layout_reader_matches_the_documented_offsets():
    """The test-side reader of the backward's blocked code parts against the byte offset the
    header states, element by element: (rb * C/64 + kb) * 1024 + 64 r + 16 (c ^ ((r/4) % 4)) + b
    for row 16 rb + r and column 64 kb + 16 c + b."""
    import numpy as np
    from decoders import unblock
    R, Cc = 48, 192
    m = np.random.default_rng(5).integers(0, 256, (R, Cc), dtype=np.uint8)
    raw = np.zeros(R * Cc, dtype=np.uint8)
    for i in range(R):
        for j in range(Cc):
            rb, r = divmod(i, 16)
            kb, within = divmod(j, 64)
            c, b = divmod(within, 16)
            raw[(rb * (Cc // 64) + kb) * 1024 + 64 * r + 16 * (c ^ ((r // 4) % 4)) + b] = m[i, j]
    assert np.array_equal(unblock(raw, R, Cc), m)


def test_binding_refuses_mismatched_tensors_on_the_host():
    """The Python binding checks tensor shapes and dtypes against the sizes it passes to the C
    ABI before it takes any pointer, so the checks run (and fail) without a GPU."""
    import torch
    import precision_moe_numerics_amd as P
    G, N, K, M = 2, 256, 256, 64

    def nv(rows, cols, rpo=1):
        return P.NVFP4(torch.zeros((rows, cols // 2), dtype=torch.uint8), torch.zeros((rows, cols // 16), dtype=torch.uint8),
                       torch.ones((rows // rpo,), dtype=torch.float32), rpo)

    xq, wq = nv(M, K), nv(G * N, K, N)
    off = torch.tensor([0, 30, M], dtype=torch.int64)
    cases = [
        (lambda: P.moe_grouped_gemm_fwd(xq, nv(G * N, K - 64, N), off, M, N), "wq must be"),
        (lambda: P.moe_grouped_gemm_fwd(xq, nv(G * N + 256, K, N), off, M, N), "wq must be"),
        (lambda: P.moe_grouped_gemm_fwd(xq, wq, off.to(torch.int32), M, N), "offsets"),
        (lambda: P.moe_grouped_gemm_fwd(xq, wq, off, M, N, gather=torch.zeros(M, dtype=torch.int64)), "gather"),
        (lambda: P.moe_grouped_gemm_fwd(xq, wq, off, M, N, out=torch.empty((M, N), dtype=torch.bfloat16)), "out"),
        (lambda: P.moe_grouped_gemm_fwd(P.NVFP4(xq.codes, xq.scales[:, :8].contiguous(), xq.outer, 1), wq, off, M, N),
         "xq.scales"),
        (lambda: P.moe_grouped_gemm_bwd(torch.zeros((M, N + 1), dtype=torch.bfloat16), xq, wq, off, M, N), "dy"),
        (lambda: P.swiglu_bwd(torch.zeros((M, N)), torch.zeros((M, N), dtype=torch.bfloat16)), "h13"),
        (lambda: P.requant_transpose_sr_mxfp8(xq, out=torch.empty((K, 32), dtype=torch.uint8)), "out"),
    ]
    for call, what in cases:
        with pytest.raises(P.PmnError, match=what):
            call()


def test_noalloc_entry_rejects_sizes_beyond_its_scratch_on_the_host(lib):
    """moe_grouped_gemm_bwd_noalloc checks its sizes against the static scratch before touching the
    device: the 48-expert w2 backward (far above 256 MiB of workspace) returns PMN_ESCRATCH."""
    fake = C.c_void_p(0x1000)     # never dereferenced
    M, G, N, K = 65536, 48, 7168, 2048
    lib.moe_grouped_gemm_bwd_noalloc.restype = C.c_int
    assert lib.pmn_noalloc_scratch_bytes() == 256 << 20
    assert lib.moe_grouped_gemm_bwd_workspace_size(M, G, N, K, 3) > 256 << 20
    st = lib.moe_grouped_gemm_bwd_noalloc(fake, fake, fake, fake, M, 1, None, fake, fake, fake, N, fake, G, M, N, K,
                                          3, 0, 0, 1, 2, 3, fake, fake, None)
    assert st == -6 and b"scratch" in lib.pmn_strerror(st)
    # argument errors come first, as in moe_grouped_gemm_bwd
    assert lib.moe_grouped_gemm_bwd_noalloc(fake, fake, fake, fake, 64, 1, None, fake, fake, fake, 256, fake, 1, 64,
                                            250, 256, 3, 0, 0, 1, 2, 3, fake, fake, None) == -2
