// abi.hip -- the C ABI of include/pmn.h: host-side argument checks, workspace layout and the
// launch sequence of each call. No call allocates, frees or synchronizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmn.h"
#include "pmn_kernels.hpp"

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline int status(hipError_t e) { return e == hipSuccess ? PMN_OK : PMN_ELAUNCH; }
inline hipStream_t hs(pmn_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

struct BwdLayout {
    size_t dq, de, wt, wte, dt, dte, xt, xte, po, woff, total;
    int64_t Pb, Nk;
};

// Bound on the padded slot count when every group is padded to a multiple of `unit`.
static int64_t padded_bound_unit(int64_t M, int G, int64_t unit)
{
    return ((M + unit - 1) & ~(unit - 1)) + unit * (int64_t)(G > 0 ? G : 0);
}

// The backward keeps its operands in the blocked layout with groups padded to 64 slots (E4M3) or
// 128 slots (packed E2M1); the row-wise dY codes sit at padded rows. dgrad contracts over N in
// stages of 64 E4M3 / 128 E2M1 values, so dY's rows and each expert's columns of W^T are Nk wide:
// N rounded up to a whole stage (equal to N for the pages' shapes).
BwdLayout bwd_layout(int64_t M, int G, int64_t N, int64_t K, bool fp4 = false)
{
    BwdLayout L{};
    L.Pb = padded_bound_unit(M, G, pmn::blocked_unit(fp4));
    const int64_t vpb = fp4 ? 2 : 1;   // code values per byte
    const int64_t stage = 64 * vpb;
    L.Nk = (N + stage - 1) / stage * stage;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += round256(bytes); return o; };
    L.dq = take((size_t)(L.Pb * L.Nk / vpb));
    L.de = take((size_t)(N / 32 * L.Pb));
    L.wt = take((size_t)(K * G * L.Nk / vpb));
    L.wte = take((size_t)(K * G * L.Nk / 32));
    L.dt = take((size_t)(N * L.Pb / vpb));
    L.dte = take((size_t)(N * L.Pb / 32));
    L.xt = take((size_t)(K * L.Pb / vpb));
    L.xte = take((size_t)(K * L.Pb / 32));
    L.po = take((size_t)(G + 1) * sizeof(int64_t));
    L.woff = take((size_t)(G + 1) * sizeof(int64_t));
    L.total = off;
    return L;
}

struct FwdMx8Layout {
    size_t xq, xe, wq, we, po, total;
    int64_t Pb;
};

FwdMx8Layout fwd_mx8_layout(int64_t M, int G, int64_t N, int64_t K)
{
    FwdMx8Layout L{};
    L.Pb = pmn_padded_bound(M, G);
    const int64_t Kp = (K + 63) & ~(int64_t)63;   // blocked rows: whole 64-byte block columns
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += round256(bytes); return o; };
    L.xq = take((size_t)(L.Pb * Kp));
    L.xe = take((size_t)(K / 32 * L.Pb));
    L.wq = take((size_t)((int64_t)G * N * Kp));
    L.we = take((size_t)(K / 32 * (int64_t)G * N));
    L.po = take((size_t)(G + 1) * sizeof(int64_t));
    L.total = off;
    return L;
}

}  // namespace

namespace pmn {

int grouped_gemm_bwd_run(const void* dy, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                         int64_t a_rows, int64_t a_rows_per_outer, const int32_t* gather, const uint8_t* b_codes,
                         const uint8_t* b_scales, const float* b_outer, int64_t b_rows_per_outer,
                         const int64_t* offsets, int G, int64_t M, int64_t N, int64_t K, int flags, int dy_rounding,
                         uint64_t seed, uint32_t rng_stream_a, uint32_t rng_stream_b, uint32_t rng_stream_dy,
                         float* da, float* db, void* workspace, size_t workspace_bytes, pmn_stream_t stream,
                         size_t* workspace_needed, bool swiglu, const float* swi_da, const void* swi_h13)
{
    const bool swi = swiglu;
    // W^T operand prepared by nvfp4_quantize_weights_bwd: b_codes / b_scales are its E4M3 codes
    // and E8M0 scales, and no requant of the weights runs here
    const bool prepared = flags & PMN_BWD_W_PREPARED;
    if (swi) {
        // dY formed from the SwiGLU backward inside the fused dY quantization only
        if ((flags & ~PMN_BWD_W_PREPARED) != (PMN_BWD_DGRAD | PMN_BWD_WGRAD) || dy_rounding != PMN_RNE)
            return PMN_EINVAL;
        if (N % 64 != 0) return PMN_ESHAPE;
        if (M > 0 && (!swi_da || !swi_h13)) return PMN_EINVAL;
        if (M > 0 && (!aligned(swi_da, 16) || !aligned(swi_h13, 16))) return PMN_EALIGN;
        dy = swi_h13;   // stands in for dY in the checks below (not read as dY)
    }
    if ((flags & ~(PMN_BWD_DGRAD | PMN_BWD_WGRAD | PMN_BWD_FP4 | PMN_BWD_W_PREPARED)) != 0 ||
        (flags & (PMN_BWD_DGRAD | PMN_BWD_WGRAD)) == 0)
        return PMN_EINVAL;
    if (prepared && (flags & PMN_BWD_FP4)) return PMN_EINVAL;
    if (prepared && N % 64 != 0) return PMN_ESHAPE;
    if (dy_rounding != PMN_RNE && dy_rounding != PMN_SR) return PMN_EINVAL;
    if (G < 1 || M < 0 || a_rows < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return PMN_ESHAPE;
    if (a_rows_per_outer < 1 || (!prepared && b_rows_per_outer < 1)) return PMN_ESHAPE;
    if (!gather && M > a_rows) return PMN_ESHAPE;
    // with no slots (M == 0) dy, da and the activations may be null: dgrad has no rows and
    // wgrad writes zero gradients
    if (!offsets || (M > 0 && !dy)) return PMN_EINVAL;
    const bool dgrad = flags & PMN_BWD_DGRAD, wgrad = flags & PMN_BWD_WGRAD;
    if (dgrad && (!b_codes || !b_scales || (!prepared && !b_outer) || (M > 0 && !da))) return PMN_EINVAL;
    if (wgrad && (!db || (M > 0 && (!a_codes || !a_scales || !a_outer)))) return PMN_EINVAL;
    const bool fp4 = flags & PMN_BWD_FP4;
    const BwdLayout L = bwd_layout(M, G, N, K, fp4);
    if (workspace_needed) {
        // the caller supplies the workspace once it knows the size (the scratch-free entry point)
        *workspace_needed = L.total;
        return PMN_OK;
    }
    if (!workspace || workspace_bytes < L.total) return PMN_EWORKSPACE;
    if (!aligned(workspace, 16) || !aligned(dy, 16) || (da && !aligned(da, 16)) || (db && !aligned(db, 16)) ||
        (a_codes && !aligned(a_codes, 16)) || (b_codes && !aligned(b_codes, 16)))
        return PMN_EALIGN;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const hipStream_t s = hs(stream);
    const bool sr = dy_rounding == PMN_SR;
    const bool blocked = true;
    const int target = fp4 ? pmn::TARGET_E2M1_PACKED : PMN_TARGET_E4M3;
    int64_t* po = reinterpret_cast<int64_t*>(ws + L.po);
    hipError_t e = pmn::launch_padded_offsets(offsets, G, M, po, s, pmn::blocked_unit(fp4));
    if (e != hipSuccess) return PMN_ELAUNCH;
    // both gradients of an E4M3 backward with dY rounded to nearest: dY's row-wise and column-wise
    // codes from one read of dY (the same bytes as the two separate quantizations)
    const bool dy_both = dgrad && wgrad && !fp4 && !sr && M > 0;
    if (dy_both) {
        e = swi ? pmn::launch_swiglu_bwd_mxfp8_rows_cols(swi_da, static_cast<const uint16_t*>(swi_h13), M, N / 2,
                                                         offsets, po, G, L.Pb, ws + L.dq, ws + L.de, ws + L.dt,
                                                         ws + L.dte, s)
                : pmn::launch_mxfp8_rows_cols(static_cast<const uint16_t*>(dy), M, N, offsets, po, G, L.Pb,
                                              ws + L.dq, ws + L.de, ws + L.dt, ws + L.dte, s);
        if (e != hipSuccess) return PMN_ELAUNCH;
    }
    if (dgrad && M > 0) {
        if (!dy_both) {
            e = pmn::launch_mxfp8_rows(static_cast<const uint16_t*>(dy), M, N, sr, seed, rng_stream_dy, ws + L.dq,
                                       ws + L.de, offsets, G, po, L.Pb, s, nullptr, fp4, blocked);
            if (e != hipSuccess) return PMN_ELAUNCH;
        }
        const uint8_t* wt = ws + L.wt;
        const uint8_t* wte = ws + L.wte;
        if (prepared) {
            wt = b_codes;
            wte = b_scales;
        } else if (L.Nk == N) {
            e = pmn::launch_requant(b_codes, b_scales, b_outer, K, b_rows_per_outer, nullptr, (int64_t)G * N, nullptr,
                                    0, target, seed, rng_stream_b, ws + L.wt, ws + L.wte, (int64_t)G * N, true,
                                    nullptr, s, blocked);
        } else {
            // every expert's N rows form a group, padded to Nk columns of W^T; the random bits and
            // the codes of the real columns are those of the ungrouped call
            int64_t* woff = reinterpret_cast<int64_t*>(ws + L.woff);
            e = pmn::launch_iota_offsets(woff, G, N, s);
            if (e != hipSuccess) return PMN_ELAUNCH;
            e = pmn::launch_requant(b_codes, b_scales, b_outer, K, b_rows_per_outer, nullptr, (int64_t)G * N, woff, G,
                                    target, seed, rng_stream_b, ws + L.wt, ws + L.wte, (int64_t)G * L.Nk, true,
                                    nullptr, s, blocked);
        }
        if (e != hipSuccess) return PMN_ELAUNCH;
        e = pmn::launch_mxfp8_dgrad(ws + L.dq, ws + L.de, wt, wte, offsets, po, L.Pb, G, M, N, K, da, s, fp4, L.Nk);
        if (e != hipSuccess) return PMN_ELAUNCH;
    }
    if (wgrad) {
        if (!dy_both) {
            e = pmn::launch_mxfp8_cols(static_cast<const uint16_t*>(dy), M, N, offsets, G, sr, seed,
                                       rng_stream_dy + 1, ws + L.dt, ws + L.dte, L.Pb, true, nullptr, s, target,
                                       blocked);
            if (e != hipSuccess) return PMN_ELAUNCH;
        }
        e = pmn::launch_requant(a_codes, a_scales, a_outer, K, a_rows_per_outer, gather, M, offsets, G, target, seed,
                                rng_stream_a, ws + L.xt, ws + L.xte, L.Pb, true, nullptr, s, blocked);
        if (e != hipSuccess) return PMN_ELAUNCH;
        e = pmn::launch_mxfp8_wgrad(ws + L.dt, ws + L.dte, ws + L.xt, ws + L.xte, L.Pb, po, G, N, K, db, s, fp4);
        if (e != hipSuccess) return PMN_ELAUNCH;
    }
    return PMN_OK;
}

}  // namespace pmn

extern "C" {

const char* pmn_strerror(int s)
{
    switch (s) {
    case PMN_OK: return "ok";
    case PMN_EINVAL: return "invalid argument (null pointer or bad enum)";
    case PMN_ESHAPE: return "bad shape (negative, not a block multiple, or inconsistent)";
    case PMN_EALIGN: return "pointer not aligned as required";
    case PMN_EWORKSPACE: return "workspace missing or too small";
    case PMN_ELAUNCH: return "kernel launch failed";
    case PMN_ESCRATCH: return "the sizes need more scratch than the library's static scratch array holds";
    default: return "unknown status";
    }
}

int pmn_version(void) { return 100; }

int64_t pmn_padded_bound(int64_t M, int G) { return ((M + 31) & ~(int64_t)31) + 32 * (int64_t)(G > 0 ? G : 0); }

int nvfp4_quantize(const void* x, int64_t rows, int64_t cols, int mode, int64_t rows_per_outer,
                   const float* outer_in, uint8_t* codes, uint8_t* scales, float* outer_out,
                   pmn_stream_t stream)
{
    if (mode != PMN_NVFP4_WEIGHT && mode != PMN_NVFP4_ACT && mode != PMN_NVFP4_WEIGHT_2D) return PMN_EINVAL;
    if (rows < 0 || cols <= 0 || cols % 16 != 0 || rows_per_outer < 1 || rows % rows_per_outer != 0)
        return PMN_ESHAPE;
    if (mode == PMN_NVFP4_WEIGHT_2D && (rows % 16 != 0 || rows_per_outer % 16 != 0)) return PMN_ESHAPE;
    if (rows == 0) return PMN_OK;
    if (!x || !codes || !scales || !outer_out) return PMN_EINVAL;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(outer_out, 4) || (outer_in && !aligned(outer_in, 4)))
        return PMN_EALIGN;
    return status(pmn::launch_nvfp4_quantize(static_cast<const uint16_t*>(x), rows, cols,
                                             mode == PMN_NVFP4_ACT, rows_per_outer, outer_in, codes,
                                             scales, outer_out, hs(stream), mode == PMN_NVFP4_WEIGHT_2D));
}

size_t nvfp4_quantize_ws_size(void) { return pmn::nvfp4_weight_1pass_ws_bytes(); }

int nvfp4_quantize_ws(const void* x, int64_t rows, int64_t cols, int mode, int64_t rows_per_outer,
                      const float* outer_in, uint8_t* codes, uint8_t* scales, float* outer_out, void* ws,
                      size_t ws_bytes, pmn_stream_t stream)
{
    if (mode != PMN_NVFP4_WEIGHT && mode != PMN_NVFP4_ACT && mode != PMN_NVFP4_WEIGHT_2D) return PMN_EINVAL;
    if (rows < 0 || cols <= 0 || cols % 16 != 0 || rows_per_outer < 1 || rows % rows_per_outer != 0)
        return PMN_ESHAPE;
    if (mode == PMN_NVFP4_WEIGHT_2D && (rows % 16 != 0 || rows_per_outer % 16 != 0)) return PMN_ESHAPE;
    if (rows == 0) return PMN_OK;
    if (!x || !codes || !scales || !outer_out) return PMN_EINVAL;
    if (!ws || ws_bytes < nvfp4_quantize_ws_size()) return PMN_EWORKSPACE;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(outer_out, 4) || (outer_in && !aligned(outer_in, 4)) ||
        !aligned(ws, 16))
        return PMN_EALIGN;
    return status(pmn::launch_nvfp4_quantize(static_cast<const uint16_t*>(x), rows, cols,
                                             mode == PMN_NVFP4_ACT, rows_per_outer, outer_in, codes,
                                             scales, outer_out, hs(stream), mode == PMN_NVFP4_WEIGHT_2D, ws,
                                             ws_bytes));
}

int nvfp4_quantize_weights_bwd(const void* x, int64_t rows, int64_t cols, int64_t rows_per_outer, uint8_t* codes,
                               uint8_t* scales, float* outer_out, uint8_t* wt_codes, uint8_t* wt_e8m0, uint64_t seed,
                               uint32_t rng_stream, void* ws, size_t ws_bytes, pmn_stream_t stream)
{
    if (rows < 0 || cols <= 0 || cols % 16 != 0 || rows_per_outer < 1 || rows % rows_per_outer != 0 ||
        rows % 64 != 0)
        return PMN_ESHAPE;
    if (rows == 0) return PMN_OK;
    if (!x || !codes || !scales || !outer_out || !wt_codes || !wt_e8m0) return PMN_EINVAL;
    if (!ws || ws_bytes < nvfp4_quantize_ws_size()) return PMN_EWORKSPACE;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(outer_out, 4) || !aligned(wt_codes, 16) ||
        !aligned(wt_e8m0, 16) || !aligned(ws, 16))
        return PMN_EALIGN;
    return status(pmn::launch_nvfp4_quantize_weights_bwd(static_cast<const uint16_t*>(x), rows, cols, rows_per_outer,
                                                         codes, scales, outer_out, wt_codes, wt_e8m0, seed,
                                                         rng_stream, ws, ws_bytes, hs(stream)));
}

static int check_groups(int64_t M, const int64_t* offsets, int G, int64_t ld)
{
    if (M < 0 || G < 0 || (offsets == nullptr) != (G == 0)) return PMN_ESHAPE;
    if (ld % 32 != 0 || ld < pmn_padded_bound(M, G)) return PMN_ESHAPE;
    return PMN_OK;
}

int requant_transpose_sr_mxfp8(const uint8_t* codes, const uint8_t* scales, const float* outer,
                               int64_t src_rows, int64_t cols, int64_t rows_per_outer,
                               const int32_t* gather, int64_t M, const int64_t* offsets, int G,
                               int target, uint64_t seed, uint32_t rng_stream, uint8_t* out,
                               uint8_t* out_e8m0, int64_t ld_out, int64_t* padded_offsets,
                               pmn_stream_t stream)
{
    if (target != PMN_TARGET_E4M3 && target != PMN_TARGET_E2M1) return PMN_EINVAL;
    if (src_rows < 0 || cols <= 0 || cols % 16 != 0 || rows_per_outer < 1) return PMN_ESHAPE;
    if (!gather && M > src_rows) return PMN_ESHAPE;
    int st = check_groups(M, offsets, G, ld_out);
    if (st != PMN_OK) return st;
    if (M == 0 && !padded_offsets) return PMN_OK;
    if ((M > 0 && (!codes || !scales || !outer)) || !out || !out_e8m0) return PMN_EINVAL;
    if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(outer, 4)) return PMN_EALIGN;
    return status(pmn::launch_requant(codes, scales, outer, cols, rows_per_outer, gather, M, offsets, G,
                                      target, seed, rng_stream, out, out_e8m0, ld_out, false,
                                      padded_offsets, hs(stream)));
}

int mxfp8_quantize(const void* x, int64_t M, int64_t N, int layout, const int64_t* offsets, int G,
                   int rounding, uint64_t seed, uint32_t rng_stream, uint8_t* out,
                   uint8_t* out_e8m0, int64_t ld_out, int64_t* padded_offsets, pmn_stream_t stream)
{
    if ((layout != PMN_ROWWISE && layout != PMN_COLWISE) || (rounding != PMN_RNE && rounding != PMN_SR))
        return PMN_EINVAL;
    if (M < 0 || N <= 0 || N % 32 != 0) return PMN_ESHAPE;
    if (!x || !out || !out_e8m0) return M == 0 && layout == PMN_ROWWISE ? PMN_OK : PMN_EINVAL;
    if (!aligned(x, 16) || !aligned(out, 16)) return PMN_EALIGN;
    if (layout == PMN_ROWWISE)
        return status(pmn::launch_mxfp8_rows(static_cast<const uint16_t*>(x), M, N, rounding == PMN_SR, seed,
                                             rng_stream, out, out_e8m0, nullptr, 0, nullptr, 0, hs(stream)));
    int st = check_groups(M, offsets, G, ld_out);
    if (st != PMN_OK) return st;
    return status(pmn::launch_mxfp8_cols(static_cast<const uint16_t*>(x), M, N, offsets, G, rounding == PMN_SR,
                                         seed, rng_stream, out, out_e8m0, ld_out, false, padded_offsets,
                                         hs(stream)));
}

int rht32_s2f6_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint32_t sign_mask,
                        int8_t* codes, uint8_t* scales_e8m0, pmn_stream_t stream)
{
    if (dtype != PMN_DTYPE_BF16 && dtype != PMN_DTYPE_F32) return PMN_EINVAL;
    if (rows < 0 || cols <= 0 || cols % 32 != 0) return PMN_ESHAPE;
    if (rows == 0) return PMN_OK;
    if (!x || !codes || !scales_e8m0) return PMN_EINVAL;
    if (!aligned(x, 16) || !aligned(codes, 16)) return PMN_EALIGN;
    return status(pmn::launch_rht32_s2f6(x, dtype == PMN_DTYPE_F32, rows, cols, sign_mask, codes, scales_e8m0,
                                         hs(stream)));
}

int moe_grouped_gemm_fwd(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                         int64_t a_rows, int64_t a_rows_per_outer, const int32_t* gather,
                         const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                         int64_t b_rows_per_outer, const int64_t* offsets, int G, int64_t M,
                         int64_t N, int64_t K, int epilogue, uint32_t rht_sign_mask, void* out,
                         uint8_t* out_e8m0, void* out_aux, pmn_stream_t stream)
{
    if (epilogue < PMN_EPI_F32 || epilogue > PMN_EPI_RHT32_S2F6) return PMN_EINVAL;
    if (G < 1 || M < 0 || a_rows < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return PMN_ESHAPE;
    if (epilogue == PMN_EPI_SWIGLU && N % 64 != 0) return PMN_ESHAPE;   // F = N / 2 features, a multiple of 32
    if (a_rows_per_outer < 1 || b_rows_per_outer < 32 || b_rows_per_outer % 32 != 0) return PMN_ESHAPE;
    if (!gather && M > a_rows) return PMN_ESHAPE;
    if (!offsets || !b_codes || !b_scales || !b_outer) return PMN_EINVAL;
    // with no slots (M == 0) the row-sized buffers (activations, outputs) may be null
    if (M > 0 && (!a_codes || !a_scales || !a_outer || !out || (epilogue == PMN_EPI_RHT32_S2F6 && !out_e8m0)))
        return PMN_EINVAL;
    if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4) ||
        !aligned(out, 16) || (out_aux && !aligned(out_aux, 16)) ||
        (epilogue == PMN_EPI_RHT32_S2F6 && !aligned(out_e8m0, 8)))
        return PMN_EALIGN;
    if (M == 0) return PMN_OK;
    return status(pmn::launch_gemm_fwd(a_codes, a_scales, a_outer, a_rows_per_outer, gather, b_codes, b_scales,
                                       b_outer, b_rows_per_outer, offsets, G, M, N, K, epilogue, rht_sign_mask,
                                       out, out_e8m0, epilogue == PMN_EPI_SWIGLU ? out_aux : nullptr,
                                       hs(stream)));
}

size_t moe_grouped_gemm_bwd_workspace_size(int64_t M, int G, int64_t N, int64_t K, int flags)
{
    if (M < 0 || G < 1 || N <= 0 || K <= 0) return 0;
    return bwd_layout(M, G, N, K, (flags & PMN_BWD_FP4) != 0).total;
}

int moe_grouped_gemm_bwd(const void* dy, const uint8_t* a_codes, const uint8_t* a_scales,
                         const float* a_outer, int64_t a_rows, int64_t a_rows_per_outer,
                         const int32_t* gather, const uint8_t* b_codes, const uint8_t* b_scales,
                         const float* b_outer, int64_t b_rows_per_outer, const int64_t* offsets,
                         int G, int64_t M, int64_t N, int64_t K, int flags, int dy_rounding,
                         uint64_t seed, uint32_t rng_stream_a, uint32_t rng_stream_b,
                         uint32_t rng_stream_dy, float* da, float* db, void* workspace,
                         size_t workspace_bytes, pmn_stream_t stream)
{
    return pmn::grouped_gemm_bwd_run(dy, a_codes, a_scales, a_outer, a_rows, a_rows_per_outer, gather, b_codes,
                                     b_scales, b_outer, b_rows_per_outer, offsets, G, M, N, K, flags, dy_rounding,
                                     seed, rng_stream_a, rng_stream_b, rng_stream_dy, da, db, workspace,
                                     workspace_bytes, stream, nullptr);
}

int moe_grouped_gemm_bwd_swiglu(const float* da_act, const void* h13, const uint8_t* a_codes,
                                const uint8_t* a_scales, const float* a_outer, int64_t a_rows,
                                int64_t a_rows_per_outer, const int32_t* gather, const uint8_t* b_codes,
                                const uint8_t* b_scales, const float* b_outer, int64_t b_rows_per_outer,
                                const int64_t* offsets, int G, int64_t M, int64_t N, int64_t K, int flags,
                                uint64_t seed, uint32_t rng_stream_a, uint32_t rng_stream_b, float* dx, float* dw,
                                void* workspace, size_t workspace_bytes, pmn_stream_t stream)
{
    if ((flags & ~PMN_BWD_W_PREPARED) != 0) return PMN_EINVAL;
    return pmn::grouped_gemm_bwd_run(nullptr, a_codes, a_scales, a_outer, a_rows, a_rows_per_outer, gather, b_codes,
                                     b_scales, b_outer, b_rows_per_outer, offsets, G, M, N, K,
                                     PMN_BWD_DGRAD | PMN_BWD_WGRAD | flags, PMN_RNE, seed, rng_stream_a, rng_stream_b,
                                     0, dx, dw, workspace, workspace_bytes, stream, nullptr, true, da_act, h13);
}

size_t moe_grouped_gemm_fwd_mxfp8_workspace_size(int64_t M, int G, int64_t N, int64_t K)
{
    if (M < 0 || G < 1 || N <= 0 || K <= 0) return 0;
    return fwd_mx8_layout(M, G, N, K).total;
}

int moe_grouped_gemm_fwd_mxfp8(const void* x, int64_t x_rows, const int32_t* gather, const void* w,
                               const int64_t* offsets, int G, int64_t M, int64_t N, int64_t K, int epilogue,
                               uint32_t rht_sign_mask, void* out, uint8_t* out_e8m0, void* out_aux,
                               void* workspace, size_t workspace_bytes, pmn_stream_t stream)
{
    if (epilogue < PMN_EPI_F32 || epilogue > PMN_EPI_RHT32_S2F6) return PMN_EINVAL;
    if (G < 1 || M < 0 || x_rows < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return PMN_ESHAPE;
    if (epilogue == PMN_EPI_SWIGLU && N % 64 != 0) return PMN_ESHAPE;   // F = N / 2 features, a multiple of 32
    if (!gather && M > x_rows) return PMN_ESHAPE;
    if (!offsets || !w || (M > 0 && (!x || !out || (epilogue == PMN_EPI_RHT32_S2F6 && !out_e8m0))))
        return PMN_EINVAL;
    const FwdMx8Layout L = fwd_mx8_layout(M, G, N, K);
    if (!workspace || workspace_bytes < L.total) return PMN_EWORKSPACE;
    if (!aligned(workspace, 16) || !aligned(w, 16) || (x && !aligned(x, 16)) || !aligned(out, 16) ||
        (out_aux && !aligned(out_aux, 16)) || (out_e8m0 && !aligned(out_e8m0, 8)))
        return PMN_EALIGN;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const hipStream_t s = hs(stream);
    int64_t* po = reinterpret_cast<int64_t*>(ws + L.po);
    hipError_t e = pmn::launch_padded_offsets(offsets, G, M, po, s);
    if (e != hipSuccess) return PMN_ELAUNCH;
    // W row-wise (RNE), E8M0 k-block-major [K/32 x G*N]
    e = pmn::launch_mxfp8_rows(static_cast<const uint16_t*>(w), (int64_t)G * N, K, false, 0, 0, ws + L.wq,
                               ws + L.we, nullptr, 0, nullptr, (int64_t)G * N, s, nullptr, false, true);
    if (e != hipSuccess) return PMN_ELAUNCH;
    // X in slot order (row s = x[gather[s]]) at padded slot rows, E8M0 k-block-major at padded
    // slot columns
    e = pmn::launch_mxfp8_rows(static_cast<const uint16_t*>(x), M, K, false, 0, 0, ws + L.xq, ws + L.xe, offsets, G,
                               po, L.Pb, s, gather, false, true);
    if (e != hipSuccess) return PMN_ELAUNCH;
    e = pmn::launch_mxfp8_fwd(ws + L.wq, ws + L.we, ws + L.xq, ws + L.xe, offsets, po, L.Pb, G, M, N, K, epilogue,
                              rht_sign_mask, out, out_e8m0, out_aux, s);
    return e == hipSuccess ? PMN_OK : PMN_ELAUNCH;
}

int swiglu_bwd(const float* da, const void* h13, int64_t M, int64_t F, void* dh13, pmn_stream_t stream)
{
    if (M < 0 || F <= 0 || F % 8 != 0) return PMN_ESHAPE;
    if (M == 0) return PMN_OK;
    if (!da || !h13 || !dh13) return PMN_EINVAL;
    if (!aligned(da, 16) || !aligned(h13, 16) || !aligned(dh13, 16)) return PMN_EALIGN;
    return status(pmn::launch_swiglu_bwd(da, static_cast<const uint16_t*>(h13), M, F, static_cast<uint16_t*>(dh13),
                                         hs(stream)));
}

int moe_route_topk(const float* logits, int64_t T, int E, int k, int32_t* ids, float* gates,
                   int64_t* offsets, int32_t* gather_token, int32_t* slot_of, pmn_stream_t stream)
{
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > 16 || k > E) return PMN_ESHAPE;
    if (!offsets || (T > 0 && (!logits || !ids || !gates || !gather_token || !slot_of))) return PMN_EINVAL;
    return status(pmn::launch_route(logits, T, E, k, ids, gates, offsets, gather_token, slot_of, hs(stream)));
}

int pmn_check_indices(const int64_t* offsets, int G, int64_t M, const int32_t* gather, int64_t n_gather,
                      int64_t src_rows, uint32_t* result, pmn_stream_t stream)
{
    if (!result || (!offsets && !gather)) return PMN_EINVAL;
    if ((offsets && (G < 1 || M < 0)) || (gather && (n_gather < 0 || src_rows < 0))) return PMN_ESHAPE;
    if (!aligned(result, 4)) return PMN_EALIGN;
    return status(pmn::launch_check_indices(offsets, offsets ? G : 0, M, gather, gather ? n_gather : 0, src_rows,
                                            result, hs(stream)));
}

int moe_combine_s2f6(const int8_t* codes, const uint8_t* e8m0, int64_t M, int64_t H, uint32_t rht_sign_mask,
                     const int32_t* slot_of, const float* gates, int64_t T, int k, void* out,
                     pmn_stream_t stream)
{
    if (M < 0 || H < 0 || H % 32 != 0 || T < 0 || k < 1 || k > 64) return PMN_ESHAPE;
    if (T == 0 || H == 0) return PMN_OK;
    if (!slot_of || !gates || !out || (M > 0 && (!codes || !e8m0))) return PMN_EINVAL;
    if (!aligned(codes, 16) || !aligned(out, 16)) return PMN_EALIGN;
    return status(pmn::launch_combine_s2f6(codes, e8m0, M, H, rht_sign_mask, slot_of, gates, T, k,
                                           static_cast<uint16_t*>(out), hs(stream)));
}

}  // extern "C"
