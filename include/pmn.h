/*
 * pmn.h -- C ABI of the quantized MoE expert layer on AMD Instinct MI355X (gfx950).
 *
 * The hot path of an MoE expert layer trained with a 4-bit forward and an 8-bit backward:
 * NVFP4 quantization (FP4 E2M1 values, an E4M3 scale per 16 values, an fp32 outer scale per
 * token or per weight matrix, 4/6 scale choice for activations), the NVFP4 grouped expert GEMM,
 * the backward operand preparation (dequantize, transpose, stochastically re-quantize to MXFP8)
 * feeding MXFP8 dgrad/wgrad GEMMs, and the combine-side 32-point randomized Hadamard transform
 * with S2F6 block quantization.
 *
 * Pages cited (by title and section heading):
 *   [AREX] AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向传播
 *          贯穿预训练到最后一次 RL rollout", sections
 *            "更少的比特换更快的算术,量化误差是代价"   (formats and bits per value)
 *            "只把专家层的前向传播降到 4-bit"           (NVFP4 forward, MXFP8 backward)
 *            "转置打散分组,随机舍入保住期望值"           (blocks, transpose, SR requant)
 *            "计算提速后,NVLink 通信成了新瓶颈"          (dispatch in NVFP4, RHT + S2F6 combine)
 *            "配方的代价:预训练约 2% 的计算效率"         (4/6, outer scales per expert / token)
 *   [LHC]  lhc.media note "Le calcul en 4 bits dès le préentraînement d'Inkling 2 Small".
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host). The caller owns and allocates every
 *     buffer; no call allocates, frees or keeps a pointer after it returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream) and never
 *     synchronize the device. Outputs are valid once the stream reaches the call.
 *   - Arguments are checked on the host before any launch. On a bad argument the call returns
 *     a negative PMN_E* code, launches nothing and writes nothing. pmn_strerror() names it.
 *   - Results are deterministic: the same inputs, seed and RNG stream give the same bits,
 *     whatever the stream, launch order or launch configuration. Random bits are keyed by the
 *     element's index in the logical source matrix, never by thread or block id.
 *   - bf16 data is passed as `const void*` (raw 16-bit bf16 words).
 *   - Index arrays that live on the device are the caller's contract, because the host cannot
 *     read them without synchronizing: offsets non-decreasing from offsets[0] = 0 to
 *     offsets[G] = M, and gather values in [0, rows of the gathered matrix). Other values make
 *     the kernels read outside the operands (moe_combine_s2f6, whose slot ids come from the
 *     caller, skips ids outside [0, M) instead). pmn_check_indices (at the end) checks these
 *     rules on the device, for debugging a caller.
 *
 * Formats:
 *   NVFP4 matrix [R x C] (C % 16 == 0):
 *     codes  uint8 [R x C/2]  element 2j in the low nibble of byte j, 2j+1 in the high nibble;
 *                             nibble = sign bit 3 | magnitude index into {0,.5,1,1.5,2,3,4,6}
 *     scales uint8 [R x C/16] E4M3 (OCP E4M3FN) block scale of each 16 consecutive values
 *     outer  fp32  [R / rows_per_outer] second-level scale of each group of rows
 *     value(r, c) = fp4(code) * ( e4m3(scale) * outer[r / rows_per_outer] )
 *   MXFP8 matrix with blocks of 32 along its rows: E4M3 bytes + E8M0 bytes (2^(b-127)) per 32.
 *   S2F6: int8 code c, value c/64, plus an E8M0 scale per 32 values.
 *   Grouped, padded transposed layout (requant, column-wise MXFP8): a logical source of M slots
 *   split into G groups by offsets [G+1] becomes [cols x ld] where group g occupies columns
 *   [po_g, po_g + P_g), P_g = m_g rounded up to 32, po_g = sum_{h<g} P_h; columns of a group past
 *   m_g are zero; E8M0 scales are [cols x ld/32]. ld >= sum_g P_g is the caller's; when offsets
 *   are only on the device, pmn_padded_bound(M, G) is always enough. Columns past sum_g P_g are
 *   not written.
 */
#ifndef PMN_H
#define PMN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* pmn_stream_t; /* hipStream_t */

/* Status codes. */
#define PMN_OK          0
#define PMN_EINVAL     -1  /* null pointer, bad enum, bad seed/stream argument */
#define PMN_ESHAPE     -2  /* a size is negative, not a multiple of the block, or inconsistent */
#define PMN_EALIGN     -3  /* a pointer is not aligned as the call requires (16 bytes) */
#define PMN_EWORKSPACE -4  /* the workspace is missing or smaller than *_workspace_size() */
#define PMN_ELAUNCH    -5  /* the HIP runtime refused a launch (hipGetLastError after launch) */
#define PMN_ESCRATCH   -6  /* the sizes need more than the static scratch of moe_grouped_gemm_bwd_noalloc */

/* Text for a status code (static storage, never NULL). */
const char* pmn_strerror(int status);

/* ABI version: 100 * major + minor. */
int pmn_version(void);

/* Padded column count that is always enough for M slots in G groups: round32(M) + 32 * G. */
int64_t pmn_padded_bound(int64_t M, int G);

/* ------------------------------------------------------------------------------------------ */
/* NVFP4 quantization   [AREX] "转置打散分组,随机舍入保住期望值" (16-value blocks, E4M3 scales, */
/* the block max maps to the top of the grid) and "配方的代价:预训练约 2% 的计算效率" (4/6 for     */
/* activations only; outer scale per expert for weights, per token for activations).           */
/* ------------------------------------------------------------------------------------------ */

#define PMN_NVFP4_WEIGHT 0 /* one scale candidate (the block max maps to 6) */
#define PMN_NVFP4_ACT    1 /* 4/6: candidates 6 and 4, the smaller squared error is kept (ties: 6) */
#define PMN_NVFP4_WEIGHT_2D 2 /* 16 x 16 square blocks (the blocking the transpose section of [AREX]
                                 contrasts with the method): as WEIGHT with each block's amax taken
                                 over its 16 x 16 tile; the scale byte is stored per row segment
                                 (equal within a tile). rows and rows_per_outer multiples of 16. */

/*
 * x: bf16 [rows x cols], cols % 16 == 0, 16-byte aligned.
 * rows_per_outer: rows sharing one outer scale (1 = per token; N = one weight matrix of N rows);
 *   rows % rows_per_outer == 0.
 * outer_in: NULL, or fp32 [rows / rows_per_outer] outer scales to use instead of computing them.
 * Per group of rows: s_o = amax / 2688 (amax = max |x| over the group; 1 if amax == 0).
 * Per block of 16 and candidate c: t = (amax_b / c) / s_o; scale = E4M3(t) (RNE, saturating at
 *   448); d = scale * s_o; r = 1/d (0 if d == 0); code_i = FP4(x_i * r) (RNE, saturating at 6).
 * Outputs: codes [rows x cols/2], scales [rows x cols/16] (16-byte aligned), outer_out fp32
 *   [rows / rows_per_outer] (the outer scales used). For 4/6 the squared error of a candidate
 *   is accumulated as e = fma(delta_i, delta_i, e) over i = 0..15 with delta_i =
 *   fma(-fp4(code_i), d, x_i).
 */
int nvfp4_quantize(const void* x, int64_t rows, int64_t cols, int mode, int64_t rows_per_outer,
                   const float* outer_in, uint8_t* codes, uint8_t* scales, float* outer_out,
                   pmn_stream_t stream);

/*
 * The same quantization with a caller-provided workspace (device memory, 16-byte aligned, at
 * least nvfp4_quantize_ws_size() bytes; PMN_EWORKSPACE otherwise). Outputs are bit-identical to
 * nvfp4_quantize's. In the weight mode with outer_in == NULL, the per-group amax that must
 * precede every block ([AREX] "配方的代价:预训练约 2% 的计算效率": one outer scale per expert
 * matrix) is then taken without a second read of x: when a group has at most 7 * 512 * (compute
 * units) blocks of 16 (one expert matrix of 2048 x 7168 on MI355X), one cooperative launch of one
 * 512-thread workgroup per compute unit holds each group in registers while the workgroups
 * exchange their partial maxima through the workspace. Other modes and shapes take the two
 * reads, as nvfp4_quantize does, and so do calls on a capturing stream (a replayed graph would
 * not guarantee the co-residency) and calls whose cooperative launch the runtime refuses. The
 * workspace's contents need no initialization (the call clears what it uses, with a kernel on
 * the stream); calls that overlap in time must not share one workspace.
 */
size_t nvfp4_quantize_ws_size(void);
int nvfp4_quantize_ws(const void* x, int64_t rows, int64_t cols, int mode, int64_t rows_per_outer,
                      const float* outer_in, uint8_t* codes, uint8_t* scales, float* outer_out, void* ws,
                      size_t ws_bytes, pmn_stream_t stream);

/*
 * Weights for both passes ([AREX] "转置打散分组,随机舍入保住期望值": the backward multiplies by the
 * transposed weights, re-quantized from the NVFP4 ones by SR; the weights do not change between
 * a step's forward and backward): nvfp4_quantize_ws(x, rows, cols, PMN_NVFP4_WEIGHT,
 * rows_per_outer, NULL, codes, scales, outer_out) and, from the same codes, the W^T operand that
 * moe_grouped_gemm_bwd's dgrad would requantize for weights of G*N = rows rows:
 *   wt_codes  uint8 [cols x rows]   E4M3 codes of W^T, in the backward workspace's blocked layout
 *                                   (1 KB blocks of 16 rows x 64 bytes, see moe_grouped_gemm_bwd)
 *   wt_e8m0   uint8 [rows/32 x cols] E8M0 per 32 rows of W, k-block-major
 * i.e. the bytes of requant_transpose_sr_mxfp8(codes, scales, outer_out, rows, cols,
 * rows_per_outer, NULL, rows, NULL, 0, PMN_TARGET_E4M3, seed, rng_stream, ...) with ld = rows,
 * blocked. Pass them to moe_grouped_gemm_bwd with PMN_BWD_W_PREPARED as b_codes / b_scales; the
 * gradients then equal those of a call with the NVFP4 weights and rng_stream_b = rng_stream.
 * rows % 64 == 0, cols % 16 == 0, rows % rows_per_outer == 0 (PMN_ESHAPE); x, codes, wt_codes,
 * wt_e8m0 and the workspace 16-byte aligned (PMN_EALIGN). Workspace as nvfp4_quantize_ws.
 * When every matrix of rows_per_outer rows (a multiple of 64) splits into at most one tile per
 * compute unit (tiles of TH <= 512 rows, a multiple of 64, by TW columns, a multiple of 16, with
 * 49152 <= TH * TW <= 57344), x is read once and the codes are re-quantized while the matrix is on
 * chip;
 * otherwise (and on a capturing stream, or when the cooperative launch is refused) the call runs
 * the two steps. The results are the same.
 */
int nvfp4_quantize_weights_bwd(const void* x, int64_t rows, int64_t cols, int64_t rows_per_outer,
                               uint8_t* codes, uint8_t* scales, float* outer_out, uint8_t* wt_codes,
                               uint8_t* wt_e8m0, uint64_t seed, uint32_t rng_stream, void* ws,
                               size_t ws_bytes, pmn_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Backward operand preparation   [AREX] "转置打散分组,随机舍入保住期望值"; [LHC] (dequantize,   */
/* transpose in higher precision, re-quantize to MXFP8 with stochastic rounding; the           */
/* expectation of the re-quantized value is the forward value).                                */
/* ------------------------------------------------------------------------------------------ */

#define PMN_TARGET_E4M3 0 /* MXFP8 elements (one byte each) */
#define PMN_TARGET_E2M1 1 /* FP4 elements, one nibble per output byte (the pages' worked example) */

/*
 * Source: the NVFP4 matrix (codes, scales, outer, rows_per_outer) of src_rows x cols.
 * Slots: M logical rows; slot s reads source row gather[s] (gather: int32 [M], or NULL for
 *   slot s = row s, then M <= src_rows). Groups: offsets int64 [G+1] (device, offsets[0] = 0,
 *   offsets[G] = M), or NULL with G = 0 for one group of M slots.
 * For every output row c and 32-block of a group's slots:
 *   v = value(source(slot), c) computed as fp4(code) * RN(e4m3(scale) * outer) in fp32, 0 for
 *       padding; e = smallest e in [-127, 127] with max|v| <= Mx * 2^e (Mx = 448 for E4M3, 6 for
 *       E2M1), so no element saturates; y = v * 2^-e; code = SR(y): with lo <= |y| < hi its grid
 *       neighbours and f = (|y| - lo) / (hi - lo), round up iff r16 < floor(f * 2^16), where r16
 *       is the 16-bit slice (i & 7) of Philox4x32-10(key = seed, counter = (i / 8, rng_stream, 0))
 *       for i = slot * cols + c (low half for even i).
 * Outputs: out [cols x ld_out] (uint8 codes), out_e8m0 [cols x ld_out/32] (biased exponent
 *   e + 127), ld_out % 32 == 0, ld_out >= sum of padded group sizes; padded_offsets (nullable)
 *   int64 [G+1] (or [2] when G = 0) receives po_g.
 */
int requant_transpose_sr_mxfp8(const uint8_t* codes, const uint8_t* scales, const float* outer,
                               int64_t src_rows, int64_t cols, int64_t rows_per_outer,
                               const int32_t* gather, int64_t M, const int64_t* offsets, int G,
                               int target, uint64_t seed, uint32_t rng_stream, uint8_t* out,
                               uint8_t* out_e8m0, int64_t ld_out, int64_t* padded_offsets,
                               pmn_stream_t stream);

/*
 * MXFP8 quantization of a bf16 gradient x [M x N] (N % 32 == 0), [AREX]
 * "只把专家层的前向传播降到 4-bit" (gradients are computed with MXFP8 matmuls).
 * layout PMN_ROWWISE: blocks of 32 along each row -> out [M x N], out_e8m0 [M x N/32]
 *   (ld_out ignored).
 * layout PMN_COLWISE: the grouped, padded transposed layout -> out [N x ld_out],
 *   out_e8m0 [N x ld_out/32] (offsets/G as for the requant; padded_offsets as there).
 * Scale rule as the requant (Mx = 448); rounding PMN_RNE (default for gradients) or PMN_SR
 * (then r16 comes from index i = row * N + col of x, with seed and rng_stream).
 */
#define PMN_ROWWISE 0
#define PMN_COLWISE 1
#define PMN_RNE 0
#define PMN_SR  1
int mxfp8_quantize(const void* x, int64_t M, int64_t N, int layout, const int64_t* offsets, int G,
                   int rounding, uint64_t seed, uint32_t rng_stream, uint8_t* out,
                   uint8_t* out_e8m0, int64_t ld_out, int64_t* padded_offsets,
                   pmn_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Combine-side RHT + S2F6   [AREX] "计算提速后,NVLink 通信成了新瓶颈" (a 32-point randomized   */
/* Hadamard transform spreads outliers, is orthogonal and exactly invertible; then S2F6 block  */
/* quantization with one scale per 32 values: 16 -> 8.25 bits per value); [LHC].               */
/* ------------------------------------------------------------------------------------------ */

#define PMN_DTYPE_BF16 0
#define PMN_DTYPE_F32  1

/*
 * x: [rows x cols] bf16 or fp32 (cols % 32 == 0). For each aligned 32-chunk y of a row:
 *   y'_j = -y_j if bit j of sign_mask else y_j; z = H_32 y' (butterflies h = 1, 2, 4, 8, 16:
 *   (a, b) -> (a + b, a - b), fp32, no 1/sqrt(32)); e = smallest e with max|z| <= (127/64) 2^e;
 *   code_j = round-half-even(z_j * 2^(6 - e)) in [-127, 127].
 * Outputs: codes int8 [rows x cols], scales_e8m0 uint8 [rows x cols/32] (e + 127).
 * Decode: x = D H (code * 2^(e - 6)) / 32.
 */
int rht32_s2f6_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint32_t sign_mask,
                        int8_t* codes, uint8_t* scales_e8m0, pmn_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Grouped expert GEMMs   [AREX] "只把专家层的前向传播降到 4-bit" (NVFP4 expert forward with     */
/* dedicated kernels; MXFP8 backward) and "计算提速后,NVLink 通信成了新瓶颈" (RHT + quantization */
/* fused into the end of the w2 matmul).                                                       */
/* ------------------------------------------------------------------------------------------ */

#define PMN_EPI_F32        0 /* out fp32 [M x N] */
#define PMN_EPI_BF16       1 /* out bf16 [M x N] (round to nearest even) */
#define PMN_EPI_SWIGLU     2 /* N = 2F: rows 0..F-1 of each expert are w1, F..2F-1 are w3;
                                out bf16 [M x F] = silu(h1) * h3; out_aux (nullable) bf16 [M x N]
                                receives h1 | h3 for the backward */
#define PMN_EPI_RHT32_S2F6 3 /* out int8 [M x N] S2F6 codes, out_e8m0 [M x N/32], the transform
                                of rht32_s2f6_quantize applied to the fp32 result (no bf16 step) */

/*
 * Y[s, n] = (sum_k a(row_s, k) b(g*N + n, k)) * RN(a_outer(row_s) * b_outer(g*N + n)), where the
 * sum runs over exact products of dequantized values fp4 * e4m3 scale (fp32 accumulation), s is
 * a slot of group g (offsets, device int64 [G+1], offsets[G] = M) and row_s = gather[s] (or s).
 * A: NVFP4 [a_rows x K] with a_rows_per_outer; B: NVFP4 [G*N x K] with b_rows_per_outer.
 * K % 32 == 0, N % 32 == 0 (SWIGLU: N % 64 == 0, so that F = N/2 is a multiple of 32);
 * b_rows_per_outer % 32 == 0 (each aligned run of 32 weight rows shares
 * one outer scale; for SWIGLU, F % b_rows_per_outer == 0 keeps w1 and w3 apart). M is the number of
 * slots (host value); with M == 0 nothing is computed and a_*, out, out_e8m0 may be null.
 * Codes, out and out_aux 16-byte aligned, scales 4-byte aligned, out_e8m0 (RHT32_S2F6) 8-byte
 * aligned; PMN_EALIGN otherwise.
 */
int moe_grouped_gemm_fwd(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                         int64_t a_rows, int64_t a_rows_per_outer, const int32_t* gather,
                         const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                         int64_t b_rows_per_outer, const int64_t* offsets, int G, int64_t M,
                         int64_t N, int64_t K, int epilogue, uint32_t rht_sign_mask, void* out,
                         uint8_t* out_e8m0, void* out_aux, pmn_stream_t stream);

/*
 * Workspace bytes moe_grouped_gemm_fwd_mxfp8 needs for these sizes (host call).
 */
size_t moe_grouped_gemm_fwd_mxfp8_workspace_size(int64_t M, int G, int64_t N, int64_t K);

/*
 * MXFP8 forward of one grouped layer, for the layers that keep MXFP8 instead of NVFP4
 * ([AREX] "配方的代价:预训练约 2% 的计算效率": the last 16.6% of the layers):
 *   Y[s, n] = sum_k X8(row_s, k) W8(g*N + n, k)   (fp32 accumulation)
 * where X8 and W8 are the row-wise MXFP8 quantizations (E4M3 round to nearest even, one E8M0 per
 * 32 values along K, the smallest scale that does not saturate -- as mxfp8_quantize with
 * PMN_ROWWISE and PMN_RNE) of x bf16 [x_rows x K] and w bf16 [G*N x K], s a slot of group g
 * (offsets, device int64 [G+1]) and row_s = gather[s] (or s). The epilogues are those of
 * moe_grouped_gemm_fwd (SWIGLU: rows 0..F-1 of each expert are w1, F..2F-1 are w3). N % 32 == 0
 * (SWIGLU: N % 64 == 0), K % 32 == 0 (M == 0: only w is quantized; x, out, out_e8m0 may be null).
 * x, w, out, out_aux
 * and the workspace 16-byte aligned, out_e8m0 8-byte aligned
 * (PMN_EALIGN). Workspace (>= moe_grouped_gemm_fwd_mxfp8_workspace_size) holds, in order, each
 * part rounded up to 256 bytes: X8 codes [Pb x Kp] and E8M0 [K/32 x Pb], slot s of group g at
 * row / column padded_offsets[g] + s - offsets[g] (groups padded to 32 slots); W8 codes
 * [G*N x Kp] and E8M0 [K/32 x G*N]; padded offsets int64 [G+1] -- with Pb = pmn_padded_bound(M,
 * G) and Kp = K rounded up to a multiple of 64 (bytes K .. Kp-1 of a row hold zero codes). The
 * code parts are blocked as described for moe_grouped_gemm_bwd; rows of padding slots are left
 * unwritten.
 */
int moe_grouped_gemm_fwd_mxfp8(const void* x, int64_t x_rows, const int32_t* gather, const void* w,
                               const int64_t* offsets, int G, int64_t M, int64_t N, int64_t K, int epilogue,
                               uint32_t rht_sign_mask, void* out, uint8_t* out_e8m0, void* out_aux,
                               void* workspace, size_t workspace_bytes, pmn_stream_t stream);

#define PMN_BWD_DGRAD 1
#define PMN_BWD_WGRAD 2
#define PMN_BWD_FP4   4  /* with DGRAD and/or WGRAD: the FP4 backward variant (see below) */
#define PMN_BWD_W_PREPARED 8 /* b_codes / b_scales are nvfp4_quantize_weights_bwd's W^T operand */

/*
 * Workspace bytes moe_grouped_gemm_bwd needs for these sizes and flags (host call).
 */
size_t moe_grouped_gemm_bwd_workspace_size(int64_t M, int G, int64_t N, int64_t K, int flags);

/*
 * Backward of Y = A W^T for one grouped layer, from the saved NVFP4 operands ([AREX]: the
 * backward reuses the forward's quantized activations; both are requantized to MXFP8 by SR):
 *   dgrad (flags & PMN_BWD_DGRAD): da[s, k] = sum_n dY[s, n] W_g[n, k], with dY quantized
 *     row-wise to MXFP8 (dy_rounding) and W_g^T requantized (seed, rng_stream_b).
 *   wgrad (flags & PMN_BWD_WGRAD): db[g*N + n, k] = sum_{s in g} dY[s, n] A[row_s, k], with dY
 *     quantized column-wise per group and A^T requantized (seed, rng_stream_a), contraction over
 *     the zero-padded slot dimension.
 * dy: bf16 [M x N]; a_*: NVFP4 [a_rows x K] (+ gather); b_*: NVFP4 [G*N x K]; offsets device
 * int64 [G+1]. N % 32 == 0, K % 32 == 0. Outputs fp32: da [M x K], db [G*N x K].
 * dY quantized with SR uses rng_stream_dy (row-wise) and rng_stream_dy + 1 (column-wise).
 * M == 0 (no routed slots) is valid: dy, da and a_* may then be null, and db is set to zero.
 * Workspace (16-byte aligned, >= moe_grouped_gemm_bwd_workspace_size) holds, in order, each
 * part rounded up to 256 bytes: dY row-wise codes [Pb x Nk] and E8M0 [N/32 x Pb]; W^T codes
 * [K x G*Nk] and E8M0 [G*Nk/32 x K], expert g at columns g*Nk .. g*Nk + N - 1 (zero codes up to
 * the next expert); dY^T codes [N x Pb] and E8M0 [Pb/32 x N]; A^T codes [K x Pb] and E8M0
 * [Pb/32 x K]; padded offsets int64 [G+1]; the experts' row offsets g*N, int64 [G+1] (used when
 * Nk != N). Nk is N rounded up to a multiple of 64 (128 with PMN_BWD_FP4); codes of dY's row-wise
 * columns N .. Nk-1 are zero (E4M3) or unspecified E2M1 values whose scale the GEMM forces to
 * 2^-127 (FP4). Each group's slots are padded with zeros to
 * a multiple of U = 64 (padded_offsets[g] is group g's first padded slot) and Pb = roundup(M, U)
 * + U G. Slot s of group g is padded slot padded_offsets[g] + s - offsets[g]: the row of the
 * row-wise dY codes and the column of their E8M0. The E8M0 parts are k-block-major (entry
 * [b, r] is the scale of k-block b of row r). The code parts are blocked: a [R x C] part is a
 * grid of 1 KB blocks of 16 rows x 64 bytes, block (rb, kb) at byte (rb * C/64 + kb) * 1024,
 * row r of a block at its bytes 64 r .. 64 r + 63 with the row's 16-byte chunk c (bytes
 * 16 c .. 16 c + 15 of those 64) at position c ^ ((r / 4) % 4). Rows of padding slots in the
 * dY row-wise codes are left unwritten. The parts of a gradient not requested are still
 * reserved.
 * PMN_BWD_W_PREPARED (not with PMN_BWD_FP4; N % 64 == 0): b_codes and b_scales are the W^T codes
 * and E8M0 scales nvfp4_quantize_weights_bwd wrote for the G*N x K weights; b_outer and
 * b_rows_per_outer are not used, rng_stream_b neither, and the workspace's W^T parts are reserved
 * but not written.
 * PMN_BWD_FP4 ([AREX], closing section: FP4 in the backward pass is the next step; the transpose
 * section's worked example rounds onto the E2M1 grid by SR): every operand goes to MXFP4 instead
 * of MXFP8 -- E2M1 codes (W^T, A^T by SR; dY by dy_rounding) with one E8M0 per 32 values chosen
 * so that nothing saturates (amax <= 6 * 2^e) -- and dgrad / wgrad run on the block-scaled FP4
 * MFMA. Its workspace has the same parts and the same blocked layout, with U = 128 and code
 * parts of E2M1 codes packed two per byte (element 2j in the low nibble): rows of half the bytes.
 */
int moe_grouped_gemm_bwd(const void* dy, const uint8_t* a_codes, const uint8_t* a_scales,
                         const float* a_outer, int64_t a_rows, int64_t a_rows_per_outer,
                         const int32_t* gather, const uint8_t* b_codes, const uint8_t* b_scales,
                         const float* b_outer, int64_t b_rows_per_outer, const int64_t* offsets,
                         int G, int64_t M, int64_t N, int64_t K, int flags, int dy_rounding,
                         uint64_t seed, uint32_t rng_stream_a, uint32_t rng_stream_b,
                         uint32_t rng_stream_dy, float* da, float* db, void* workspace,
                         size_t workspace_bytes, pmn_stream_t stream);

/*
 * The w1||w3 backward of a SwiGLU layer with the SwiGLU backward folded into dY's quantization:
 * moe_grouped_gemm_bwd with both gradients (dgrad -> dx [M x K], wgrad -> dw [G*N x K]) and dY
 * rounded to nearest, where dY = dh13 [M x N] is not passed but formed from the gradient of the
 * SwiGLU output da_act (fp32 [M x F], F = N / 2) and the saved pre-activations h13 (bf16
 * [M x N], h1 in columns 0 .. F-1, h3 in F .. N-1) exactly as swiglu_bwd forms it, and never
 * written out. N % 64 == 0. The results and the workspace contents equal those of swiglu_bwd
 * followed by moe_grouped_gemm_bwd(PMN_BWD_DGRAD | PMN_BWD_WGRAD | flags, PMN_RNE), flags being 0
 * or PMN_BWD_W_PREPARED (PMN_EINVAL otherwise). The rounding of dY is fixed to RNE and there is no
 * FP4 variant; other configurations call the two separately.
 */
int moe_grouped_gemm_bwd_swiglu(const float* da_act, const void* h13, const uint8_t* a_codes,
                                const uint8_t* a_scales, const float* a_outer, int64_t a_rows,
                                int64_t a_rows_per_outer, const int32_t* gather, const uint8_t* b_codes,
                                const uint8_t* b_scales, const float* b_outer, int64_t b_rows_per_outer,
                                const int64_t* offsets, int G, int64_t M, int64_t N, int64_t K, int flags,
                                uint64_t seed, uint32_t rng_stream_a, uint32_t rng_stream_b, float* dx, float* dw,
                                void* workspace, size_t workspace_bytes, pmn_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): moe_grouped_gemm_bwd with its workspace taken from a static
 * device array of the library, PMN_NOALLOC_SCRATCH_BYTES per device, held by each device the
 * library runs on until the process ends. Arguments, results and errors are those of
 * moe_grouped_gemm_bwd without the workspace; sizes whose workspace
 * (moe_grouped_gemm_bwd_workspace_size) exceeds the array return PMN_ESCRATCH and launch nothing.
 * The call allocates and frees nothing. Every call on a device uses that device's one array, which
 * keeps the last call's contents (nothing in it needs to start at zero): calls that overlap on one
 * device (concurrent streams, several host threads) race and must be serialized by the caller.
 */
#define PMN_NOALLOC_SCRATCH_BYTES (256ull << 20)
size_t pmn_noalloc_scratch_bytes(void);
int moe_grouped_gemm_bwd_noalloc(const void* dy, const uint8_t* a_codes, const uint8_t* a_scales,
                                 const float* a_outer, int64_t a_rows, int64_t a_rows_per_outer,
                                 const int32_t* gather, const uint8_t* b_codes, const uint8_t* b_scales,
                                 const float* b_outer, int64_t b_rows_per_outer, const int64_t* offsets, int G,
                                 int64_t M, int64_t N, int64_t K, int flags, int dy_rounding, uint64_t seed,
                                 uint32_t rng_stream_a, uint32_t rng_stream_b, uint32_t rng_stream_dy, float* da,
                                 float* db, pmn_stream_t stream);

/*
 * SwiGLU backward (the layer's activation between w1/w3 and w2): da fp32 [M x F] and the saved
 * h13 bf16 [M x 2F] (h1 | h3) give dh13 bf16 [M x 2F]: dh1 = da h3 silu'(h1), dh3 = da silu(h1).
 */
int swiglu_bwd(const float* da, const void* h13, int64_t M, int64_t F, void* dh13,
               pmn_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Routing into expert groups   [AREX] "计算提速后,NVLink 通信成了新瓶颈" (the router picks each */
/* token's experts; tokens are dispatched to them and combined back).                          */
/* ------------------------------------------------------------------------------------------ */

/*
 * logits fp32 [T x E] (E <= 1024, 1 <= k <= min(E, 16)) -> ids int32 [T x k] (top-k by logit,
 * descending, equal logits: lower expert first), gates fp32 [T x k] (softmax probability of
 * each chosen expert, not renormalized), offsets int64 [E+1], gather_token int32 [T*k] (token
 * of each slot) and slot_of int32 [T*k] (slot of (t, j)); slots are ordered by (expert, token).
 */
int moe_route_topk(const float* logits, int64_t T, int E, int k, int32_t* ids, float* gates,
                   int64_t* offsets, int32_t* gather_token, int32_t* slot_of, pmn_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Combine, receiver side   [AREX] "计算提速后,NVLink 通信成了新瓶颈" (expert outputs return to  */
/* their tokens as RHT32 + S2F6 rows; the receiver inverts the transform exactly and weights   */
/* each of a token's k expert outputs by its gate).                                            */
/* ------------------------------------------------------------------------------------------ */

/*
 * codes int8 [M x H] and e8m0 uint8 [M x H/32]: the w2 outputs of M routed slots in the form
 * moe_grouped_gemm_fwd(PMN_EPI_RHT32_S2F6) and rht32_s2f6_quantize write, with the same
 * rht_sign_mask. slot_of int32 [T x k] names, for token t and its choice j, the slot that holds
 * its expert output (moe_route_topk's slot_of); gates fp32 [T x k] are the weights.
 *   out bf16 [T x H]:  out[t, :] = sum_j gates[t, j] * decode(slot_of[t, j]),
 *   decode(s) per 32-chunk:  D H (codes * 2^(e8m0 - 133)) / 32   (the exact inverse transform).
 * The sum is taken in fp32 on the scaled codes and transformed once (decode is linear); the
 * result is rounded once to bf16, nearest even. Values of slot_of outside [0, M) are not read
 * and add nothing (M = 0 gives zeros). H % 32 == 0 and 1 <= k <= 64 (PMN_ESHAPE); codes and out
 * 16-byte aligned (PMN_EALIGN). T = 0 launches nothing. All pointers are device pointers.
 */
int moe_combine_s2f6(const int8_t* codes, const uint8_t* e8m0, int64_t M, int64_t H, uint32_t rht_sign_mask,
                     const int32_t* slot_of, const float* gates, int64_t T, int k, void* out,
                     pmn_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Checking the device index contract (a debugging aid for callers; no other call runs it).   */
/* ------------------------------------------------------------------------------------------ */

#define PMN_CHECK_OFFSETS_START 1u  /* offsets[0] != 0 */
#define PMN_CHECK_OFFSETS_END   2u  /* offsets[G] != M */
#define PMN_CHECK_OFFSETS_ORDER 4u  /* offsets[g] > offsets[g + 1] for some g */
#define PMN_CHECK_OFFSETS_RANGE 8u  /* offsets[g] outside [0, M] for some g */
#define PMN_CHECK_GATHER_RANGE 16u  /* gather[i] outside [0, src_rows) for some i */

/*
 * The rules the grouped calls assume of their device index arrays (Conventions above), which they
 * cannot check without synchronizing: offsets int64 [G+1] and gather int32 [n_gather] (either may
 * be NULL, not both; G >= 1 and M >= 0 with offsets, n_gather >= 0 and src_rows >= 0 with gather),
 * src_rows being the rows of the matrix gather indexes. One small launch on `stream` writes to
 * result (device, uint32, 4-byte aligned) the OR of the PMN_CHECK_* bits of every violated rule,
 * 0 when all hold; the caller synchronizes the stream before reading it. Only offsets[0..G] and
 * gather[0..n_gather) are read, so the check itself is safe on any values.
 */
int pmn_check_indices(const int64_t* offsets, int G, int64_t M, const int32_t* gather, int64_t n_gather,
                      int64_t src_rows, uint32_t* result, pmn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PMN_H */
