// pmn_kernels.hpp -- launchers of the HIP kernels (internal to the library; the public
// interface is include/pmn.h). Every launcher only enqueues work on `stream` and returns
// hipGetLastError(); arguments are validated by the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmn.h"

namespace pmn {

// requant / column-quantizer target beyond the public PMN_TARGET_* values: E2M1 codes packed two
// per byte (slot 2j in the low nibble), the operand format of the FP4 backward GEMMs
constexpr int TARGET_E2M1_PACKED = 2;

// ws: NULL, or at least nvfp4_weight_1pass_ws_bytes() of device memory, which lets the weight
// mode (one candidate, computed outer scales) read x once when the device holds a whole group of
// rows in registers (cooperative launch); otherwise the group amax and the blocks take two reads.
hipError_t launch_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, bool four_six,
                                 int64_t rows_per_outer, const float* outer_in, uint8_t* codes,
                                 uint8_t* scales, float* outer_out, hipStream_t stream, bool square = false,
                                 void* ws = nullptr, size_t ws_bytes = 0);
size_t nvfp4_weight_1pass_ws_bytes();
// Weights (weight mode, computed outer scales) and the backward's W^T operand from them: wt E4M3
// [cols x rows] in the blocked layout below (rows % 64 == 0) and wte E8M0 [rows/32 x cols], the
// bytes of launch_requant(ungrouped, E4M3, SR with (seed, stream_id), k-block-major, blocked).
// One read of x when the device holds a tile of every matrix per CU, else the two steps.
hipError_t launch_nvfp4_quantize_weights_bwd(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_outer,
                                             uint8_t* codes, uint8_t* scales, float* outer_out, uint8_t* wt,
                                             uint8_t* wte, uint64_t seed, uint32_t stream_id, void* ws,
                                             size_t ws_bytes, hipStream_t stream);

// Row-wise MXFP8. With padded_offsets null the E8M0 scales are row-major [M x N/32]; otherwise
// they are k-block-major [N/32 x ld_e8m0] with slot s of group g at column
// padded_offsets[g] + s - offsets[g] (the layout the grouped dgrad GEMM streams). `blocked`
// (k-block-major only) writes the codes in the blocked layout below with slot s of group g at row
// padded_offsets[g] + s - offsets[g] (without padded_offsets: row s), in rows of N rounded up to
// 64 bytes (E4M3; the rounding bytes hold zero codes) or N/2 bytes (packed E2M1, N % 128 == 0);
// padding rows are not written.
hipError_t launch_mxfp8_rows(const uint16_t* x, int64_t M, int64_t N, bool sr, uint64_t seed,
                             uint32_t stream_id, uint8_t* out, uint8_t* out_e8m0,
                             const int64_t* offsets, int G, const int64_t* padded_offsets,
                             int64_t ld_e8m0, hipStream_t stream, const int32_t* gather = nullptr,
                             bool fp4 = false, bool blocked = false);

// Padded group offsets (each group rounded up to a multiple of `unit` slots: 32, or 64 for the
// blocked backward operands) into padded_offsets [G+1].
hipError_t launch_padded_offsets(const int64_t* offsets, int G, int64_t M, int64_t* padded_offsets,
                                 hipStream_t stream, int64_t unit = 32);

// The blocked operand layout of the backward GEMMs: a [R x C] code matrix (R % 16 == 0, C bytes,
// C % 64 == 0) is stored as 1 KB blocks of 16 rows x 64 bytes, block (rb, kb) at byte
// (rb * C/64 + kb) * 1024; inside a block row r occupies bytes 64 r .. 64 r + 63 and its 16-byte
// chunk c (bytes 16 c .. 16 c + 15 of the row's 64) sits at slot c ^ ((r / 4) % 4). Groups of
// slots are padded so that every GEMM stage (64 bytes of a row: 64 E4M3 codes or 128 packed E2M1
// codes) is one block column.
inline int64_t blocked_unit(bool fp4) { return fp4 ? 128 : 64; }

hipError_t launch_rht32_s2f6(const void* x, bool f32, int64_t rows, int64_t cols, uint32_t mask,
                             int8_t* codes, uint8_t* e8m0, hipStream_t stream);

hipError_t launch_requant(const uint8_t* codes, const uint8_t* scales, const float* outer,
                          int64_t cols, int64_t rows_per_outer, const int32_t* gather, int64_t M,
                          const int64_t* offsets, int G, int target, uint64_t seed,
                          uint32_t stream_id, uint8_t* out, uint8_t* out_e8m0, int64_t ld,
                          bool e8m0_kb_major, int64_t* padded_offsets, hipStream_t stream, bool blocked = false);

// dY [M x N] bf16 to MXFP8 (E4M3, round to nearest even) both ways in one read, in the blocked
// layouts of the backward's workspace: row-wise codes rq at padded rows ([Pb x N rounded to 64]
// in 1 KB blocks) with E8M0 re [N/32 x Pb], and column-wise codes cq ([N x Pb] in 1 KB blocks)
// with E8M0 ce [Pb/32 x N]; groups padded to 64 slots, po [G+1] their padded offsets (from
// launch_padded_offsets with unit 64, earlier on the stream). The same bytes as launch_mxfp8_rows
// and launch_mxfp8_cols with those layouts.
hipError_t launch_mxfp8_rows_cols(const uint16_t* x, int64_t M, int64_t N, const int64_t* offsets,
                                  const int64_t* po, int G, int64_t Pb, uint8_t* rq, uint8_t* re, uint8_t* cq,
                                  uint8_t* ce, hipStream_t stream);
// The same for dY = the SwiGLU backward's dh13 [M x 2F], formed from da [M x F] (fp32) and h13
// [M x 2F] (bf16) as launch_swiglu_bwd forms it, without writing it.
hipError_t launch_swiglu_bwd_mxfp8_rows_cols(const float* da, const uint16_t* h13, int64_t M, int64_t F,
                                             const int64_t* offsets, const int64_t* po, int G, int64_t Pb,
                                             uint8_t* rq, uint8_t* re, uint8_t* cq, uint8_t* ce, hipStream_t stream);

hipError_t launch_mxfp8_cols(const uint16_t* x, int64_t M, int64_t N, const int64_t* offsets,
                             int G, bool sr, uint64_t seed, uint32_t stream_id, uint8_t* out,
                             uint8_t* out_e8m0, int64_t ld, bool e8m0_kb_major,
                             int64_t* padded_offsets, hipStream_t stream, int target = 0, bool blocked = false);

hipError_t launch_gemm_fwd(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                           int64_t a_rpo, const int32_t* gather, const uint8_t* b_codes,
                           const uint8_t* b_scales, const float* b_outer, int64_t b_rpo,
                           const int64_t* offsets, int G, int64_t M, int64_t N, int64_t K,
                           int epilogue, uint32_t rht_mask, void* out, uint8_t* out_e8m0,
                           void* out_aux, hipStream_t stream);

// Grouped MXFP8 GEMMs. Code operands are in the blocked layout; all E8M0 operands are
// k-block-major: de [Nf/32 x Pb] (padded slot columns, po), wte [G*Nk/32 x Kf] (Nk = Nf rounded up
// to whole stages of 64 E4M3 or 128 E2M1 values), dte [Pb/32 x Nf], xte [Pb/32 x Kf]. The forward takes W8 [G*N rows x roundup(K, 64)] and X8 at padded slot rows.
hipError_t launch_mxfp8_dgrad(const uint8_t* dq, const uint8_t* de, const uint8_t* wt,
                              const uint8_t* wte, const int64_t* offsets, const int64_t* po,
                              int64_t Pb, int G, int64_t M, int64_t Nf, int64_t Kf, float* dx,
                              hipStream_t stream, bool fp4, int64_t Nk);
// o[g] = g * step for g = 0 .. G (device), one thread per entry
hipError_t launch_iota_offsets(int64_t* o, int G, int64_t step, hipStream_t stream);

hipError_t launch_mxfp8_fwd(const uint8_t* wq, const uint8_t* we, const uint8_t* xq, const uint8_t* xe,
                            const int64_t* offsets, const int64_t* po, int64_t Pb, int G, int64_t M, int64_t N,
                            int64_t K, int epilogue, uint32_t mask, void* out, uint8_t* out_e8m0, void* out_aux,
                            hipStream_t stream);

hipError_t launch_mxfp8_wgrad(const uint8_t* dt, const uint8_t* dte, const uint8_t* xt,
                              const uint8_t* xte, int64_t ld, const int64_t* po, int G,
                              int64_t Nf, int64_t Kf, float* dw, hipStream_t stream, bool fp4 = false);

hipError_t launch_swiglu_bwd(const float* da, const uint16_t* h13, int64_t M, int64_t F,
                             uint16_t* dh13, hipStream_t stream);

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int32_t* ids, float* gates,
                        int64_t* offsets, int32_t* gather_token, int32_t* slot_of, hipStream_t stream);

// Violations of the device index contract as a PMN_CHECK_* mask written to result[0].
hipError_t launch_check_indices(const int64_t* offsets, int G, int64_t M, const int32_t* gather, int64_t n,
                                int64_t src_rows, uint32_t* result, hipStream_t stream);

hipError_t launch_combine_s2f6(const int8_t* codes, const uint8_t* e8m0, int64_t M, int64_t H, uint32_t mask,
                               const int32_t* slot_of, const float* gates, int64_t T, int k, uint16_t* out,
                               hipStream_t stream);

// The whole moe_grouped_gemm_bwd call (argument checks, workspace layout, launches) on a given
// workspace. With workspace_needed non-null it only checks the arguments and stores the workspace
// bytes the sizes need (nothing is launched). With swiglu, dy is instead the SwiGLU backward of
// (swi_da [M x N/2] fp32, swi_h13 [M x N] bf16), formed inside the dY quantization (both
// gradients, E4M3, RNE only).
int grouped_gemm_bwd_run(const void* dy, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                         int64_t a_rows, int64_t a_rows_per_outer, const int32_t* gather, const uint8_t* b_codes,
                         const uint8_t* b_scales, const float* b_outer, int64_t b_rows_per_outer,
                         const int64_t* offsets, int G, int64_t M, int64_t N, int64_t K, int flags, int dy_rounding,
                         uint64_t seed, uint32_t rng_stream_a, uint32_t rng_stream_b, uint32_t rng_stream_dy,
                         float* da, float* db, void* workspace, size_t workspace_bytes, pmn_stream_t stream,
                         size_t* workspace_needed, bool swiglu = false, const float* swi_da = nullptr,
                         const void* swi_h13 = nullptr);

}  // namespace pmn
