/*
 * pmn_oracle.c -- plain, slow, obviously-correct CPU oracle for the quantized MoE expert layer.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. It shares no code, header, table or constant generator with the HIP
 * library; the two are written independently from the same reading of the pages.
 *
 * Pages cited (by title and section heading):
 *   [AREX]  AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit
 *           前向传播贯穿预训练到最后一次 RL rollout". Sections:
 *             S1 "更少的比特换更快的算术,量化误差是代价"  (fewer bits, faster math; error is the cost)
 *             S2 "只把专家层的前向传播降到 4-bit"          (only the expert-layer forward in 4-bit)
 *             S3 "转置打散分组,随机舍入保住期望值"          (transpose scatters groups; SR keeps E[.])
 *             S4 "计算提速后,NVLink 通信成了新瓶颈"         (dispatch / combine become the bottleneck)
 *             S5 "配方的代价:预训练约 2% 的计算效率"        (recipe details: 4/6, outer scales)
 *   [LHC]   lhc.media note "Le calcul en 4 bits dès le préentraînement d'Inkling 2 Small".
 *
 * Precision. Where a floating-point value decides an integer (a code, a scale byte, a 4/6
 * choice) the decision is taken in fp32 with one rounding per named operation, in the order
 * written here, because that is the precision the kernels decide in. Rounding onto a number
 * grid is done by the definition: find the two neighbouring grid values of |y| in exact
 * (double) arithmetic and pick one. GEMM accumulation is fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC (no FMA contraction,
 * so every a*b+c written below is two roundings; fmaf() is used where one rounding is meant).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads of the OpenMP loops below (for timing the oracle; no result depends on it). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------------------------ */
/* Scalars and bit views                                                                       */
/* ------------------------------------------------------------------------------------------ */

static float fbits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is the top half of an fp32 word; widening is exact. [AREX S1]: BF16 is 16 bits/value. */
float orc_bf16_to_f32(uint16_t h) { return fbits((uint32_t)h << 16); }

/* Round-to-nearest-even fp32 -> bf16 (finite inputs), used for bf16 outputs of the epilogues. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u; memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------------------------ */
/* Number grids                                                                                */
/* ------------------------------------------------------------------------------------------ */

/* FP4 E2M1 magnitudes, exactly the sixteen values listed in [AREX S3]: ±0, ±0.5, ±1, ±1.5,
 * ±2, ±3, ±4, ±6. Code = sign bit 3 | magnitude index 0..7. */
static const double FP4_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* E4M3 (OCP "E4M3FN": bias 7, no infinities, 0x7F/0xFF NaN) value of a byte. The pages name
 * the format as NVFP4's and MXFP8's element/scale type ([AREX S3]); the bit layout is the OCP
 * definition. */
double orc_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if ((c & 0x7F) == 0x7F) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

double orc_fp4_value(uint8_t nib)
{
    double v = FP4_GRID[nib & 7];
    return (nib & 8) ? -v : v;
}

/* E4M3 non-negative grid: index k (= code k) for k = 0..126, increasing. Filled once when the
 * library is loaded, before any parallel region can read it. */
static double E4M3_GRID[127];
__attribute__((constructor)) static void e4m3_grid_init(void)
{
    for (int k = 0; k < 127; k++) E4M3_GRID[k] = orc_e4m3_value((uint8_t)k);
}

enum { ORC_RNE = 0, ORC_SR = 1 };

/*
 * Round a magnitude a >= 0 onto a sorted grid g[0..n-1] (g[0] = 0).
 *   RNE: nearest neighbour, a tie goes to the even grid index (for these grids: the even
 *        mantissa / even code).
 *   SR:  with lo <= a < hi the neighbours and f = (a - lo)/(hi - lo), round up iff
 *        r16 < floor(f * 2^16); the probability of rounding up is f to within 2^-16, so the
 *        expectation is kept ([AREX S3]: 2.25 goes to 2 with p = 3/4 and to 3 with p = 1/4).
 * Magnitudes above the largest grid value saturate to it.
 * All differences below are exact in double for fp32 inputs and these grids.
 */
static int grid_round(double a, const double* g, int n, int mode, uint32_t r16)
{
    if (a >= g[n - 1]) return n - 1;
    int lo = 0, hi = n - 1;             /* invariant g[lo] <= a < g[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g[mid] <= a) lo = mid; else hi = mid;
    }
    double dlo = a - g[lo], dhi = g[hi] - a;
    if (mode == ORC_RNE) {
        if (dlo < dhi) return lo;
        if (dhi < dlo) return hi;
        return (lo % 2 == 0) ? lo : hi;
    }
    double f = dlo / (g[hi] - g[lo]);
    uint32_t f16 = (uint32_t)floor(f * 65536.0);
    return (r16 < f16) ? hi : lo;
}

/* fp32 -> E4M3 byte, RNE with saturation to ±448 (scale bytes, MXFP8 RTN elements). */
uint8_t orc_e4m3_encode(float y, int mode, uint32_t r16)
{
    int k = grid_round(fabs((double)y), E4M3_GRID, 127, mode, r16);
    return (uint8_t)(k | (signbit(y) ? 0x80 : 0));
}

/* fp32 -> FP4 nibble, RNE (or SR) with saturation to ±6; the sign is kept, so -0 exists. */
uint8_t orc_fp4_encode(float y, int mode, uint32_t r16)
{
    int k = grid_round(fabs((double)y), FP4_GRID, 8, mode, r16);
    return (uint8_t)(k | (signbit(y) ? 8 : 0));
}

/*
 * Power-of-two block scale for the E8M0-scaled formats (MXFP8 elements, requant targets, S2F6):
 * the smallest e in [-127, 127] with amax <= M * 2^e, so no element of the block saturates and
 * stochastic rounding stays unbiased ([AREX S3]: the backward pass must avoid bias).
 * Searched directly; the start e0 = E - 12 (amax = m * 2^E, m in [0.5, 1)) is never valid
 * because M < 2^9, so the first valid e found is the smallest.
 * amax == 0 gives e = -127 (byte 0).
 */
int orc_e8m0_exponent(float amax, double M)
{
    if (!(amax > 0.0f)) return -127;
    int E; frexp((double)amax, &E);
    int e = E - 12;
    if (e < -127) e = -127;
    while (e < 127 && !((double)amax <= ldexp(M, e))) e++;
    return e;
}

/* ------------------------------------------------------------------------------------------ */
/* Counter-based RNG: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As */
/* Easy as 1, 2, 3", SC'11), written from its published definition.                            */
/* ------------------------------------------------------------------------------------------ */

void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; round++) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * The 16 random bits that element i of a logical source matrix draws under (seed, stream):
 * key = (seed low word, seed high word); counter = (i/8 low word, i/8 high word, stream, 0);
 * element i uses 16-bit half (i & 1) (0 = low) of output word (i & 7) / 2.
 */
uint32_t orc_rand16(uint64_t seed, uint32_t stream, uint64_t i)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint64_t blk = i >> 3;
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), stream, 0u};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    uint32_t word = w[(i & 7) >> 1];
    return (i & 1) ? (word >> 16) : (word & 0xFFFFu);
}

/* ------------------------------------------------------------------------------------------ */
/* NVFP4 quantization  [AREX S3] block scaling, [AREX S5] 4/6 and outer scales                 */
/* ------------------------------------------------------------------------------------------ */

/*
 * Outer (second-level) fp32 scale of one group: s_o = A / 2688 with A = max|x| over the group
 * and 2688 = 6 * 448 (largest FP4 magnitude times largest E4M3 scale), so the largest block of
 * the group gets block scale 448 under the 6-candidate. A == 0 gives s_o = 1.
 * [AREX S5]: one outer scale per expert for weights, one per token for activations.
 */
float orc_outer_scale(float amax)
{
    if (!(amax > 0.0f)) return 1.0f;
    volatile float a = amax;
    return a / 2688.0f;
}

/*
 * One NVFP4 block (16 values x, fp32) under candidate c (6 or 4) and outer scale s_o:
 *   t  = RN(RN(a_b / c) / s_o)        a_b = max|x_i|
 *   sb = E4M3(t), RNE, saturating     ([AREX S3]: the block max maps to the top of the grid,
 *                                      e.g. max -54 with scale 9 is stored as -6)
 *   d  = RN(value(sb) * s_o)          effective scale of the block
 *   r  = 0 if d == 0, else min(RN(1/d), FLT_MAX)
 *   q_i = FP4(RN(x_i * r)), RNE, saturating to ±6
 * Returns sb and writes the 16 nibbles to q.
 */
static uint8_t nvfp4_block(const float* x, float s_o, float c, uint8_t* q, float* d_out)
{
    float ab = 0.0f;
    for (int i = 0; i < 16; i++) { float m = fabsf(x[i]); if (m > ab) ab = m; }
    volatile float t1 = ab / c;
    volatile float t = t1 / s_o;
    uint8_t sb = orc_e4m3_encode(t, ORC_RNE, 0);
    volatile float d = (float)orc_e4m3_value(sb) * s_o;
    float r = 0.0f;
    if (d != 0.0f) {
        volatile float inv = 1.0f / d;
        r = (inv > FLT_MAX) ? FLT_MAX : inv;
    }
    for (int i = 0; i < 16; i++) {
        volatile float y = x[i] * r;
        q[i] = orc_fp4_encode(y, ORC_RNE, 0);
    }
    *d_out = d;
    return sb;
}

/*
 * Squared dequantization error of a block for the 4/6 choice:
 *   delta_i = fma(-fp4(q_i), d, x_i)   (exact difference, one rounding)
 *   e <- fma(delta_i, delta_i, e)      for i = 0..15 in order, e starting at 0
 */
static float block_sq_error(const float* x, const uint8_t* q, float d)
{
    float e = 0.0f;
    for (int i = 0; i < 16; i++) {
        float delta = fmaf(-(float)orc_fp4_value(q[i]), d, x[i]);
        e = fmaf(delta, delta, e);
    }
    return e;
}

/*
 * NVFP4 quantization of a bf16 matrix x [rows x cols] (row-major, cols % 16 == 0).
 *   rows_per_outer: rows sharing one outer scale (1 = per token; N = one weight matrix).
 *   four_six:       if nonzero, each block tries candidates 6 and 4 and keeps the one whose
 *                   squared error is strictly smaller (ties keep 6). [AREX S5]: activations
 *                   choose between two scale factors; weights do not.
 *   outer_in:       if non-NULL, these outer scales are used instead of computed ones.
 * Outputs: codes [rows x cols/2] (element 2j in the low nibble of byte j, 2j+1 in the high),
 *          scales [rows x cols/16] E4M3 bytes, outer [rows / rows_per_outer] fp32,
 *          chose4 [rows x cols/16] (optional, 1 where candidate 4 was kept).
 */
void orc_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_outer,
                        int four_six, const float* outer_in, uint8_t* codes, uint8_t* scales,
                        float* outer_out, uint8_t* chose4)
{
    int64_t ngroups = rows / rows_per_outer;
    for (int64_t g = 0; g < ngroups; g++) {
        float s_o;
        if (outer_in) {
            s_o = outer_in[g];
        } else {
            float A = 0.0f;
            for (int64_t r = g * rows_per_outer; r < (g + 1) * rows_per_outer; r++)
                for (int64_t c = 0; c < cols; c++) {
                    float m = fabsf(orc_bf16_to_f32(x[r * cols + c]));
                    if (m > A) A = m;
                }
            s_o = orc_outer_scale(A);
        }
        outer_out[g] = s_o;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float s_o = outer_out[r / rows_per_outer];
        for (int64_t b = 0; b < cols / 16; b++) {
            float xb[16];
            for (int i = 0; i < 16; i++) xb[i] = orc_bf16_to_f32(x[r * cols + b * 16 + i]);
            uint8_t q6[16], q4[16];
            float d6, d4;
            uint8_t sb6 = nvfp4_block(xb, s_o, 6.0f, q6, &d6);
            uint8_t sb = sb6;
            const uint8_t* q = q6;
            int took4 = 0;
            if (four_six) {
                uint8_t sb4 = nvfp4_block(xb, s_o, 4.0f, q4, &d4);
                float e6 = block_sq_error(xb, q6, d6);
                float e4 = block_sq_error(xb, q4, d4);
                if (e4 < e6) { sb = sb4; q = q4; took4 = 1; }
            }
            scales[r * (cols / 16) + b] = sb;
            if (chose4) chose4[r * (cols / 16) + b] = (uint8_t)took4;
            for (int i = 0; i < 16; i += 2)
                codes[r * (cols / 2) + b * 8 + i / 2] = (uint8_t)(q[i] | (q[i + 1] << 4));
        }
    }
}

/*
 * NVFP4 with square 16 x 16 blocks ([AREX S3]: the blocking NVIDIA uses so that a tensor and its
 * transpose quantize bit-identically; the pages reject it because 256 values share one scale).
 * Tile (I, J) = rows 16I .. 16I+15, columns 16J .. 16J+15 has a_t = max|x| over its 256 values;
 * every row segment of the tile is quantized as a weight-mode block (candidate 6, no 4/6) whose
 * amax is a_t: t = RN(RN(a_t / 6) / s_o), sb = E4M3(t) RNE saturating, d = RN(value(sb) s_o),
 * r = RN(1/d), q = FP4(RN(x r)). Outer scale per group of rows_per_outer rows (a multiple of 16).
 * The scale is stored once per row segment ([rows x cols/16], the 1D layout, equal within a
 * tile), so the result is an ordinary NVFP4 matrix.
 */
void orc_nvfp4_quantize_2d(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_outer, uint8_t* codes,
                           uint8_t* scales, float* outer_out)
{
    for (int64_t g = 0; g < rows / rows_per_outer; g++) {
        float A = 0.0f;
        for (int64_t r = g * rows_per_outer; r < (g + 1) * rows_per_outer; r++)
            for (int64_t c = 0; c < cols; c++) {
                float m = fabsf(orc_bf16_to_f32(x[r * cols + c]));
                if (m > A) A = m;
            }
        outer_out[g] = orc_outer_scale(A);
    }
#pragma omp parallel for schedule(static)
    for (int64_t I = 0; I < rows / 16; I++)
        for (int64_t J = 0; J < cols / 16; J++) {
            float at = 0.0f;
            for (int64_t r = 16 * I; r < 16 * I + 16; r++)
                for (int64_t c = 16 * J; c < 16 * J + 16; c++) {
                    float m = fabsf(orc_bf16_to_f32(x[r * cols + c]));
                    if (m > at) at = m;
                }
            const float s_o = outer_out[(16 * I) / rows_per_outer];
            volatile float t1 = at / 6.0f;
            volatile float t = t1 / s_o;
            const uint8_t sb = orc_e4m3_encode(t, ORC_RNE, 0);
            volatile float d = (float)orc_e4m3_value(sb) * s_o;
            float rcp = 0.0f;
            if (d != 0.0f) {
                volatile float inv = 1.0f / d;
                rcp = (inv > FLT_MAX) ? FLT_MAX : inv;
            }
            for (int64_t r = 16 * I; r < 16 * I + 16; r++) {
                scales[r * (cols / 16) + J] = sb;
                for (int i = 0; i < 16; i += 2) {
                    volatile float y0 = orc_bf16_to_f32(x[r * cols + 16 * J + i]) * rcp;
                    volatile float y1 = orc_bf16_to_f32(x[r * cols + 16 * J + i + 1]) * rcp;
                    codes[r * (cols / 2) + 8 * J + i / 2] =
                        (uint8_t)(orc_fp4_encode(y0, ORC_RNE, 0) | (orc_fp4_encode(y1, ORC_RNE, 0) << 4));
                }
            }
        }
}

/* Effective scale of block (row r, block b) of an NVFP4 matrix: d = RN(value(sb) * s_o). */
static float nvfp4_block_scale(const uint8_t* scales, const float* outer, int64_t cols,
                               int64_t rows_per_outer, int64_t r, int64_t b)
{
    volatile float d = (float)orc_e4m3_value(scales[r * (cols / 16) + b]) * outer[r / rows_per_outer];
    return d;
}

static uint8_t nvfp4_nibble(const uint8_t* codes, int64_t cols, int64_t r, int64_t c)
{
    uint8_t byte = codes[r * (cols / 2) + c / 2];
    return (c & 1) ? (byte >> 4) : (byte & 15);
}

/* Dequantization to fp32 ([AREX S3]: the saved forward tensor goes back to high precision):
 * v = RN(fp4(q) * d) with d the block's effective scale. */
float orc_nvfp4_dequant_elem(const uint8_t* codes, const uint8_t* scales, const float* outer,
                             int64_t cols, int64_t rows_per_outer, int64_t r, int64_t c)
{
    float d = nvfp4_block_scale(scales, outer, cols, rows_per_outer, r, c / 16);
    volatile float v = (float)orc_fp4_value(nvfp4_nibble(codes, cols, r, c)) * d;
    return v;
}

void orc_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* outer,
                          int64_t rows, int64_t cols, int64_t rows_per_outer, float* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            out[r * cols + c] = orc_nvfp4_dequant_elem(codes, scales, outer, cols, rows_per_outer, r, c);
}

/* ------------------------------------------------------------------------------------------ */
/* Grouped, padded transposes: shared layout of the requant and column-wise MXFP8 outputs      */
/* ------------------------------------------------------------------------------------------ */

/*
 * A logical source matrix has M rows ("slots") split into G consecutive groups by offsets
 * [G+1] (offsets[0] = 0, offsets[G] = M). The transposed output has one row per source column
 * and, for group g, a column range of width P_g = m_g rounded up to 32 starting at
 * po_g = sum_{h<g} P_h; columns past m_g inside the range are zero padding. Blocks of 32 along
 * the output row never cross groups. With offsets == NULL there is one group of M rows.
 */
int64_t orc_padded_total(const int64_t* offsets, int G, int64_t M)
{
    if (!offsets) return (M + 31) / 32 * 32;
    int64_t p = 0;
    for (int g = 0; g < G; g++) p += (offsets[g + 1] - offsets[g] + 31) / 32 * 32;
    return p;
}

/* ------------------------------------------------------------------------------------------ */
/* Requantization: dequant -> transpose -> SR to MXFP8 (or E2M1)  [AREX S3], [LHC]             */
/* ------------------------------------------------------------------------------------------ */

enum { ORC_TARGET_E4M3 = 0, ORC_TARGET_E2M1 = 1 };

/*
 * Source: NVFP4 matrix (codes, scales, outer, rows_per_outer) of `src_rows` x `cols`.
 * Slots s = 0..M-1 read source row gather[s] (or row s when gather == NULL).
 * Output: out [cols x Ptot] codes (E4M3 bytes, or one E2M1 nibble per byte), out_e8m0
 * [cols x Ptot/32]. For each output row c and each 32-block of a group's slots:
 *   v_j  = dequant(source(slot), c), 0 for padding
 *   e    = smallest e with max|v| <= M * 2^e   (M = 448 for E4M3, 6 for E2M1)
 *   y_j  = RN(v_j * 2^-e)
 *   code = SR(y_j) with r16 = rand16(seed, stream, slot * cols + c)  (index in the gathered,
 *          unpadded source order, so the result does not depend on the launch layout)
 * Padding bytes are 0 and draw no random bits.
 */
void orc_requant_transpose_sr(const uint8_t* codes, const uint8_t* scales, const float* outer,
                              int64_t cols, int64_t rows_per_outer,
                              const int32_t* gather, const int64_t* offsets, int G, int64_t M,
                              int target, uint64_t seed, uint32_t stream,
                              uint8_t* out, uint8_t* out_e8m0)
{
    int64_t Ptot = orc_padded_total(offsets, G, M);
    int ng = offsets ? G : 1;
    double Mmax = (target == ORC_TARGET_E4M3) ? 448.0 : 6.0;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        int64_t po = 0;
        for (int g = 0; g < ng; g++) {
            int64_t s0 = offsets ? offsets[g] : 0, s1 = offsets ? offsets[g + 1] : M;
            int64_t P = (s1 - s0 + 31) / 32 * 32;
            for (int64_t jb = 0; jb < P; jb += 32) {
                float v[32];
                float amax = 0.0f;
                for (int j = 0; j < 32; j++) {
                    int64_t s = s0 + jb + j;
                    v[j] = 0.0f;
                    if (s < s1) {
                        int64_t r = gather ? gather[s] : s;
                        v[j] = orc_nvfp4_dequant_elem(codes, scales, outer, cols, rows_per_outer, r, c);
                    }
                    if (fabsf(v[j]) > amax) amax = fabsf(v[j]);
                }
                int e = orc_e8m0_exponent(amax, Mmax);
                out_e8m0[c * (Ptot / 32) + (po + jb) / 32] = (uint8_t)(e + 127);
                for (int j = 0; j < 32; j++) {
                    int64_t s = s0 + jb + j;
                    uint8_t code = 0;
                    if (s < s1) {
                        float y = ldexpf(v[j], -e);
                        uint32_t r16 = orc_rand16(seed, stream, (uint64_t)s * (uint64_t)cols + (uint64_t)c);
                        code = (target == ORC_TARGET_E4M3) ? orc_e4m3_encode(y, ORC_SR, r16)
                                                           : orc_fp4_encode(y, ORC_SR, r16);
                    }
                    out[c * Ptot + po + jb + j] = code;
                }
            }
            po += P;
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* MXFP8 quantization of gradients (E4M3 elements, E8M0 per 32)  [AREX S2], [AREX S3]          */
/* ------------------------------------------------------------------------------------------ */

/*
 * Row-wise: x bf16 [M x N], blocks of 32 along each row (N % 32 == 0).
 *   e = smallest e with max|x| <= Mx * 2^e (Mx = 448 for E4M3, 6 for E2M1); y = RN(x * 2^-e);
 *   code = E4M3(y) or E2M1(y) (one nibble per byte), RNE, or SR with
 *   r16 = rand16(seed, stream, row * N + col) when sr != 0.
 * The E2M1 target is the element format of an FP4 backward ([AREX], closing section: FP4 in the
 * backward pass is the next step; the transpose section's worked example rounds onto that grid).
 */
void orc_mx_quantize_rows(const uint16_t* x, int64_t M, int64_t N, int target, int sr, uint64_t seed,
                          uint32_t stream, uint8_t* out, uint8_t* out_e8m0)
{
    const double Mx = target == ORC_TARGET_E4M3 ? 448.0 : 6.0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; r++)
        for (int64_t b = 0; b < N / 32; b++) {
            float amax = 0.0f;
            for (int j = 0; j < 32; j++) {
                float m = fabsf(orc_bf16_to_f32(x[r * N + b * 32 + j]));
                if (m > amax) amax = m;
            }
            int e = orc_e8m0_exponent(amax, Mx);
            out_e8m0[r * (N / 32) + b] = (uint8_t)(e + 127);
            for (int j = 0; j < 32; j++) {
                int64_t c = b * 32 + j;
                float y = ldexpf(orc_bf16_to_f32(x[r * N + c]), -e);
                uint32_t r16 = sr ? orc_rand16(seed, stream, (uint64_t)r * (uint64_t)N + (uint64_t)c) : 0;
                out[r * N + c] = target == ORC_TARGET_E4M3 ? orc_e4m3_encode(y, sr ? ORC_SR : ORC_RNE, r16)
                                                           : orc_fp4_encode(y, sr ? ORC_SR : ORC_RNE, r16);
            }
        }
}

void orc_mxfp8_quantize_rows(const uint16_t* x, int64_t M, int64_t N, int sr, uint64_t seed,
                             uint32_t stream, uint8_t* out, uint8_t* out_e8m0)
{
    orc_mx_quantize_rows(x, M, N, ORC_TARGET_E4M3, sr, seed, stream, out, out_e8m0);
}

/*
 * Column-wise within groups: the transposed, padded layout described above, blocks of 32 along
 * the slots of one group, for x bf16 [M x N] -> out [N x Ptot], out_e8m0 [N x Ptot/32].
 */
void orc_mx_quantize_cols(const uint16_t* x, int64_t M, int64_t N, const int64_t* offsets,
                          int G, int target, int sr, uint64_t seed, uint32_t stream, uint8_t* out,
                          uint8_t* out_e8m0)
{
    const double Mx = target == ORC_TARGET_E4M3 ? 448.0 : 6.0;
    int64_t Ptot = orc_padded_total(offsets, G, M);
    int ng = offsets ? G : 1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        int64_t po = 0;
        for (int g = 0; g < ng; g++) {
            int64_t s0 = offsets ? offsets[g] : 0, s1 = offsets ? offsets[g + 1] : M;
            int64_t P = (s1 - s0 + 31) / 32 * 32;
            for (int64_t jb = 0; jb < P; jb += 32) {
                float v[32], amax = 0.0f;
                for (int j = 0; j < 32; j++) {
                    int64_t s = s0 + jb + j;
                    v[j] = (s < s1) ? orc_bf16_to_f32(x[s * N + n]) : 0.0f;
                    if (fabsf(v[j]) > amax) amax = fabsf(v[j]);
                }
                int e = orc_e8m0_exponent(amax, Mx);
                out_e8m0[n * (Ptot / 32) + (po + jb) / 32] = (uint8_t)(e + 127);
                for (int j = 0; j < 32; j++) {
                    int64_t s = s0 + jb + j;
                    uint8_t code = 0;
                    if (s < s1) {
                        float y = ldexpf(v[j], -e);
                        uint32_t r16 = sr ? orc_rand16(seed, stream, (uint64_t)s * (uint64_t)N + (uint64_t)n) : 0;
                        code = target == ORC_TARGET_E4M3 ? orc_e4m3_encode(y, sr ? ORC_SR : ORC_RNE, r16)
                                                         : orc_fp4_encode(y, sr ? ORC_SR : ORC_RNE, r16);
                    }
                    out[n * Ptot + po + jb + j] = code;
                }
            }
            po += P;
        }
    }
}

void orc_mxfp8_quantize_cols(const uint16_t* x, int64_t M, int64_t N, const int64_t* offsets,
                             int G, int sr, uint64_t seed, uint32_t stream, uint8_t* out,
                             uint8_t* out_e8m0)
{
    orc_mx_quantize_cols(x, M, N, offsets, G, ORC_TARGET_E4M3, sr, seed, stream, out, out_e8m0);
}

/* Value of an MX element: value(code) * 2^(e8m0 - 127), code E4M3 or E2M1 (one per byte). */
double orc_mx_value(uint8_t code, uint8_t e8m0, int target)
{
    return ldexp(target == ORC_TARGET_E4M3 ? orc_e4m3_value(code) : orc_fp4_value(code), (int)e8m0 - 127);
}
double orc_mxfp8_value(uint8_t code, uint8_t e8m0) { return orc_mx_value(code, e8m0, ORC_TARGET_E4M3); }

/* ------------------------------------------------------------------------------------------ */
/* 32-point randomized Hadamard transform + S2F6 block quantization  [AREX S4], [LHC]          */
/* ------------------------------------------------------------------------------------------ */

/*
 * Forward transform of one 32-chunk y (fp32), sign mask bit j flips element j:
 *   y'_j = -y_j if bit j of mask else y_j
 *   z = H_32 y' by butterflies h = 1, 2, 4, 8, 16: (a, b) -> (RN(a + b), RN(a - b)) over pairs
 *   (i, i + h) with (i & h) == 0. Unnormalized (no 1/sqrt(32)); H_32 H_32 = 32 I, so the exact
 *   inverse is D H z / 32 ([AREX S4]: an orthogonal transform that is inverted exactly).
 */
void orc_rht32(const float* y, uint32_t mask, float* z)
{
    float t[32];
    for (int j = 0; j < 32; j++) t[j] = ((mask >> j) & 1u) ? -y[j] : y[j];
    for (int h = 1; h < 32; h <<= 1)
        for (int i = 0; i < 32; i++)
            if ((i & h) == 0) {
                volatile float a = t[i], b = t[i + h];
                volatile float s = a + b, d = a - b;
                t[i] = s; t[i + h] = d;
            }
    for (int j = 0; j < 32; j++) z[j] = t[j];
}

/*
 * S2F6 block quantization of z (one 32-chunk): a signed fixed-point code c in [-127, 127] with
 * value c/64 ([AREX S4]: 2-bit signed integer + 6-bit fraction, range -128/64..127/64), and one
 * E8M0 scale per 32 values (8 + 8/32 = 8.25 bits per value, as [AREX S4] and [LHC] count):
 *   e = smallest e with max|z| <= (127/64) * 2^e;  c_j = RNE(z_j * 2^(6 - e)).
 */
void orc_s2f6_block(const float* z, int8_t* codes, uint8_t* e8m0)
{
    float amax = 0.0f;
    for (int j = 0; j < 32; j++) if (fabsf(z[j]) > amax) amax = fabsf(z[j]);
    int e = orc_e8m0_exponent(amax, 127.0 / 64.0);
    *e8m0 = (uint8_t)(e + 127);
    for (int j = 0; j < 32; j++) {
        double n = ldexp((double)z[j], 6 - e);      /* exact */
        double L = floor(n), f = n - L;
        if (f > 0.5 || (f == 0.5 && fmod(L, 2.0) != 0.0)) L += 1.0;
        if (L > 127.0) L = 127.0;
        if (L < -127.0) L = -127.0;
        codes[j] = (int8_t)L;
    }
}

/* Rows of fp32 y [rows x cols] (cols % 32 == 0) -> codes int8 [rows x cols], e8m0 [rows x cols/32]. */
void orc_rht32_s2f6_quantize(const float* y, int64_t rows, int64_t cols, uint32_t mask,
                             int8_t* codes, uint8_t* e8m0)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < cols / 32; b++) {
            float z[32];
            orc_rht32(y + r * cols + b * 32, mask, z);
            orc_s2f6_block(z, codes + r * cols + b * 32, e8m0 + r * (cols / 32) + b);
        }
}

/*
 * Plain block-scaled S2F6 without the transform (the ablation of [AREX S4]: outliers are what the
 * transform is there for): each aligned 32-chunk of y goes through the same block step,
 * codes c = RNE(y 2^(6 - e)), E8M0 by the smallest-e rule with M = 127/64.
 */
void orc_s2f6_quantize(const float* y, int64_t rows, int64_t cols, int8_t* codes, uint8_t* e8m0)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < cols / 32; b++)
            orc_s2f6_block(y + r * cols + b * 32, codes + r * cols + b * 32, e8m0 + r * (cols / 32) + b);
}

/* Decode (receiver side): z^ = c * 2^(e - 6); x^ = D H z^ / 32, in fp64. */
void orc_rht32_s2f6_decode(const int8_t* codes, const uint8_t* e8m0, int64_t rows, int64_t cols,
                           uint32_t mask, double* out)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < cols / 32; b++) {
            double t[32];
            int e = (int)e8m0[r * (cols / 32) + b] - 127;
            for (int j = 0; j < 32; j++) t[j] = ldexp((double)codes[r * cols + b * 32 + j], e - 6);
            for (int h = 1; h < 32; h <<= 1)
                for (int i = 0; i < 32; i++)
                    if ((i & h) == 0) { double a = t[i], c = t[i + h]; t[i] = a + c; t[i + h] = a - c; }
            for (int j = 0; j < 32; j++) {
                double v = t[j] / 32.0;
                out[r * cols + b * 32 + j] = ((mask >> j) & 1u) ? -v : v;
            }
        }
}

/*
 * Combine, receiver side ([AREX S4]: the w2 outputs travel back as RHT32 + S2F6 codes; the
 * receiver inverts the transform exactly and forms each token's output as the gate-weighted sum
 * of its routed slots' outputs). For token t and its k choices i: slot slot_of[t*k + i] with gate
 * gates[t*k + i];  out[t, :] = sum_i gates[t*k+i] * decode(row slot_of[t*k+i]), in fp64, decode
 * as orc_rht32_s2f6_decode (z^ = c * 2^(e - 127 - 6), x^ = D H z^ / 32).
 */
void orc_moe_combine_s2f6(const int8_t* codes, const uint8_t* e8m0, int64_t M, int64_t H, uint32_t mask,
                          const int32_t* slot_of, const float* gates, int64_t T, int k, double* out)
{
    (void)M;
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; t++) {
            for (int64_t c = 0; c < H; c++) out[t * H + c] = 0.0;
            for (int i = 0; i < k; i++) {
                const int64_t s = slot_of[t * k + i];
                orc_rht32_s2f6_decode(codes + s * H, e8m0 + s * (H / 32), 1, H, mask, row);
                const double g = (double)gates[t * k + i];
                for (int64_t c = 0; c < H; c++) out[t * H + c] += g * row[c];
            }
        }
        free(row);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Grouped GEMMs (fp64 accumulation)  [AREX S2]: expert forward in NVFP4, backward in MXFP8    */
/* ------------------------------------------------------------------------------------------ */

/*
 * NVFP4 grouped forward: slots s of group g (offsets) read activation row gather[s] (or s);
 * weights are [G*N x K] NVFP4 (group g = rows g*N .. g*N+N-1).
 *   acc = sum_k (fp4 * sb)_x[k] * (fp4 * sb)_w[n, k]   (every product exact; summed in fp64)
 *   Y[s, n] = fp32( acc * s_x(row) * s_w(row of w) )
 */
void orc_gemm_nvfp4_grouped(const uint8_t* xc, const uint8_t* xs, const float* xo, int64_t x_rpo,
                            const int32_t* gather, const uint8_t* wc, const uint8_t* ws,
                            const float* wo, int64_t w_rpo, const int64_t* offsets, int G,
                            int64_t N, int64_t K, float* Y)
{
    int64_t M = offsets[G];
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t s = 0; s < M; s++) {
        int g = 0;
        while (offsets[g + 1] <= s) g++;
        int64_t r = gather ? gather[s] : s;
        double* xv = (double*)malloc(sizeof(double) * (size_t)K);
        for (int64_t k = 0; k < K; k++)
            xv[k] = orc_fp4_value(nvfp4_nibble(xc, K, r, k)) * orc_e4m3_value(xs[r * (K / 16) + k / 16]);
        for (int64_t n = 0; n < N; n++) {
            int64_t wr = (int64_t)g * N + n;
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double wv = orc_fp4_value(nvfp4_nibble(wc, K, wr, k)) * orc_e4m3_value(ws[wr * (K / 16) + k / 16]);
                acc += xv[k] * wv;
            }
            Y[s * N + n] = (float)(acc * (double)xo[r / x_rpo] * (double)wo[wr / w_rpo]);
        }
        free(xv);
    }
}

/*
 * One output of the NVFP4 grouped forward (for sampled checks at full size).
 */
double orc_gemm_nvfp4_elem(const uint8_t* xc, const uint8_t* xs, const float* xo, int64_t x_rpo,
                           const int32_t* gather, const uint8_t* wc, const uint8_t* ws,
                           const float* wo, int64_t w_rpo, const int64_t* offsets, int G,
                           int64_t N, int64_t K, int64_t s, int64_t n)
{
    int g = 0;
    while (offsets[g + 1] <= s) g++;
    int64_t r = gather ? gather[s] : s;
    int64_t wr = (int64_t)g * N + n;
    double acc = 0.0;
    for (int64_t k = 0; k < K; k++) {
        double xv = orc_fp4_value(nvfp4_nibble(xc, K, r, k)) * orc_e4m3_value(xs[r * (K / 16) + k / 16]);
        double wv = orc_fp4_value(nvfp4_nibble(wc, K, wr, k)) * orc_e4m3_value(ws[wr * (K / 16) + k / 16]);
        acc += xv * wv;
    }
    return acc * (double)xo[r / x_rpo] * (double)wo[wr / w_rpo];
}

/*
 * MXFP8 "NT" product used by both backward GEMMs: D[m, n] = sum_k A[m, k] B[n, k] with
 * A = a_code * 2^(a_e8m0 - 127) per 32 along k (likewise B); rows of A and B have leading
 * dimensions lda / ldb bytes and scale leading dimensions lda/32, ldb/32.
 * Element (m, n) over k in [k0, k0 + kn) (k0, kn multiples of 32), fp64.
 */
double orc_mx_dot(const uint8_t* a, const uint8_t* ae, int64_t lda, const uint8_t* b, const uint8_t* be,
                  int64_t ldb, int64_t m, int64_t n, int64_t k0, int64_t kn, int target)
{
    double acc = 0.0;
    for (int64_t k = k0; k < k0 + kn; k++)
        acc += orc_mx_value(a[m * lda + k], ae[m * (lda / 32) + k / 32], target) *
               orc_mx_value(b[n * ldb + k], be[n * (ldb / 32) + k / 32], target);
    return acc;
}

double orc_mxfp8_dot(const uint8_t* a, const uint8_t* ae, int64_t lda, const uint8_t* b,
                     const uint8_t* be, int64_t ldb, int64_t m, int64_t n, int64_t k0, int64_t kn)
{
    return orc_mx_dot(a, ae, lda, b, be, ldb, m, n, k0, kn, ORC_TARGET_E4M3);
}

/*
 * MXFP8 forward of one grouped layer ([AREX S5]: the last 16.6% of the layers keep MXFP8 instead
 * of NVFP4): Y[s, n] = sum_k X[row(s), k] * W_g[n, k] for slot s of group g, with X quantized
 * row-wise (xq [x_rows x K], xe [x_rows x K/32]), row(s) = gather[s] or s, and W quantized
 * row-wise (wq [G*N x K], we [G*N x K/32], expert g in rows g*N .. g*N+N-1). fp64 output.
 */
void orc_gemm_mxfp8_fwd(const uint8_t* xq, const uint8_t* xe, const int32_t* gather, const uint8_t* wq,
                        const uint8_t* we, const int64_t* offsets, int G, int64_t N, int64_t K, double* Y)
{
    int64_t M = offsets[G];
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t s = 0; s < M; s++) {
        int g = 0;
        while (offsets[g + 1] <= s) g++;
        const int64_t r = gather ? (int64_t)gather[s] : s;
        for (int64_t n = 0; n < N; n++)
            Y[s * N + n] = orc_mxfp8_dot(xq, xe, K, wq, we, K, r, (int64_t)g * N + n, 0, K);
    }
}

/*
 * dgrad of one grouped layer: dX[s, k] = sum_n dY[s, n] * W_g[n, k], with dY quantized row-wise
 * (dq [M x N], de [M x N/32]) and W_g^T requantized (wt [K x G*N], wte [K x G*N/32]; group g's
 * columns g*N .. g*N+N-1).
 */
void orc_gemm_mx_dgrad(const uint8_t* dq, const uint8_t* de, const uint8_t* wt, const uint8_t* wte,
                       const int64_t* offsets, int G, int64_t N, int64_t K, int target, float* dX)
{
    int64_t M = offsets[G];
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t s = 0; s < M; s++) {
        int g = 0;
        while (offsets[g + 1] <= s) g++;
        for (int64_t k = 0; k < K; k++) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; n++)
                acc += orc_mx_value(dq[s * N + n], de[s * (N / 32) + n / 32], target) *
                       orc_mx_value(wt[k * (G * N) + g * N + n], wte[k * (G * N / 32) + (g * N + n) / 32], target);
            dX[s * K + k] = (float)acc;
        }
    }
}

void orc_gemm_mxfp8_dgrad(const uint8_t* dq, const uint8_t* de, const uint8_t* wt,
                          const uint8_t* wte, const int64_t* offsets, int G, int64_t N, int64_t K,
                          float* dX)
{
    orc_gemm_mx_dgrad(dq, de, wt, wte, offsets, G, N, K, ORC_TARGET_E4M3, dX);
}

/*
 * wgrad of one grouped layer: dW_g[n, k] = sum_{s in g} dY[s, n] X[s, k], from the column-wise
 * quantized dY^T (dt [N x Ptot]) and the requantized X^T (xt [K x Ptot]) in the padded grouped
 * layout (padding is zero and adds nothing).
 */
void orc_gemm_mx_wgrad(const uint8_t* dt, const uint8_t* dte, const uint8_t* xt, const uint8_t* xte,
                       const int64_t* offsets, int G, int64_t N, int64_t K, int target, float* dW)
{
    int64_t Ptot = orc_padded_total(offsets, G, offsets[G]);
#pragma omp parallel for schedule(dynamic, 1)
    for (int g = 0; g < G; g++) {
        int64_t po = 0;
        for (int h = 0; h < g; h++) po += (offsets[h + 1] - offsets[h] + 31) / 32 * 32;
        int64_t P = (offsets[g + 1] - offsets[g] + 31) / 32 * 32;
        for (int64_t n = 0; n < N; n++)
            for (int64_t k = 0; k < K; k++)
                dW[((int64_t)g * N + n) * K + k] =
                    (float)orc_mx_dot(dt, dte, Ptot, xt, xte, Ptot, n, k, po, P, target);
    }
}

void orc_gemm_mxfp8_wgrad(const uint8_t* dt, const uint8_t* dte, const uint8_t* xt,
                          const uint8_t* xte, const int64_t* offsets, int G, int64_t N, int64_t K,
                          float* dW)
{
    orc_gemm_mx_wgrad(dt, dte, xt, xte, offsets, G, N, K, ORC_TARGET_E4M3, dW);
}

/* ------------------------------------------------------------------------------------------ */
/* SwiGLU and its backward (the expert layer's shape: w1, w3 then w2), fp64                    */
/* ------------------------------------------------------------------------------------------ */

/* h13 [M x 2F] fp32 (h1 = columns 0..F-1, h3 = F..2F-1) -> a = silu(h1) * h3. */
void orc_swiglu(const float* h13, int64_t M, int64_t F, double* a)
{
    for (int64_t s = 0; s < M; s++)
        for (int64_t j = 0; j < F; j++) {
            double h1 = h13[s * 2 * F + j], h3 = h13[s * 2 * F + F + j];
            a[s * F + j] = h1 / (1.0 + exp(-h1)) * h3;
        }
}

/* da [M x F], h13 bf16 [M x 2F] -> dh13 [M x 2F]: dh1 = da h3 silu'(h1), dh3 = da silu(h1). */
void orc_swiglu_bwd(const float* da, const uint16_t* h13, int64_t M, int64_t F, double* dh13)
{
    for (int64_t s = 0; s < M; s++)
        for (int64_t j = 0; j < F; j++) {
            double h1 = orc_bf16_to_f32(h13[s * 2 * F + j]), h3 = orc_bf16_to_f32(h13[s * 2 * F + F + j]);
            double sg = 1.0 / (1.0 + exp(-h1));
            double d = da[s * F + j];
            dh13[s * 2 * F + j] = d * h3 * (sg * (1.0 + h1 * (1.0 - sg)));
            dh13[s * 2 * F + F + j] = d * h1 * sg;
        }
}

/* ------------------------------------------------------------------------------------------ */
/* Routing into expert groups  [AREX S4]: the router sends each token to its experts            */
/* ------------------------------------------------------------------------------------------ */

/*
 * logits [T x E] -> ids [T x k] (top-k by logit, descending; equal logits: lower expert first),
 * gates [T x k] = softmax probability of the chosen expert (not renormalized), and the grouped
 * order: slots sorted stably by (expert, token, rank) -> offsets [E+1], gather_token [T*k]
 * (token of each slot), slot_of [T*k] (slot of (t, j)).
 */
void orc_route_topk(const float* logits, int64_t T, int E, int k, int32_t* ids, float* gates,
                    int64_t* offsets, int32_t* gather_token, int32_t* slot_of)
{
    for (int64_t t = 0; t < T; t++) {
        const float* l = logits + t * E;
        double mx = -INFINITY;
        for (int e = 0; e < E; e++) if (l[e] > mx) mx = l[e];
        double z = 0.0;
        for (int e = 0; e < E; e++) z += exp((double)l[e] - mx);
        unsigned char* used = (unsigned char*)calloc((size_t)E, 1);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++)
                if (!used[e] && (best < 0 || l[e] > l[best])) best = e;
            used[best] = 1;
            ids[t * k + j] = best;
            gates[t * k + j] = (float)(exp((double)l[best] - mx) / z);
        }
        free(used);
    }
    for (int e = 0; e <= E; e++) offsets[e] = 0;
    for (int64_t i = 0; i < T * k; i++) offsets[ids[i] + 1]++;
    for (int e = 0; e < E; e++) offsets[e + 1] += offsets[e];
    int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
    for (int e = 0; e < E; e++) fill[e] = offsets[e];
    for (int64_t t = 0; t < T; t++)
        for (int j = 0; j < k; j++) {
            int e = ids[t * k + j];
            int64_t s = fill[e]++;
            gather_token[s] = (int32_t)t;
            slot_of[t * k + j] = (int32_t)s;
        }
    free(fill);
}

/* ------------------------------------------------------------------------------------------ */
/* Array forms of the scalar encoders (for exhaustive codec checks)                            */
/* ------------------------------------------------------------------------------------------ */

void orc_e4m3_encode_array(const float* y, int64_t n, int mode, const uint32_t* r16, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_encode(y[i], mode, r16 ? r16[i] : 0u);
}

void orc_fp4_encode_array(const float* y, int64_t n, int mode, const uint32_t* r16, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = orc_fp4_encode(y[i], mode, r16 ? r16[i] : 0u);
}

void orc_rand16_array(uint64_t seed, uint32_t stream, const uint64_t* idx, int64_t n, uint32_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = orc_rand16(seed, stream, idx[i]);
}

/*
 * The requantization of slots [s_begin, s_begin + count) of an ungrouped, ungathered source
 * (s_begin % 32 == 0), for checking windows of a large output one by one: the same computation
 * as orc_requant_transpose_sr, with the random bits of slot s drawn at index s * cols + c.
 * out [cols x round32(count)], out_e8m0 [cols x round32(count)/32].
 */
void orc_requant_window(const uint8_t* codes, const uint8_t* scales, const float* outer,
                        int64_t cols, int64_t rows_per_outer, int64_t s_begin, int64_t count,
                        int64_t M, int target, uint64_t seed, uint32_t stream, uint8_t* out,
                        uint8_t* out_e8m0)
{
    int64_t P = (count + 31) / 32 * 32;
    double Mmax = (target == ORC_TARGET_E4M3) ? 448.0 : 6.0;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++)
        for (int64_t jb = 0; jb < P; jb += 32) {
            float v[32], amax = 0.0f;
            for (int j = 0; j < 32; j++) {
                int64_t s = s_begin + jb + j;
                v[j] = (jb + j < count && s < M)
                           ? orc_nvfp4_dequant_elem(codes, scales, outer, cols, rows_per_outer, s, c) : 0.0f;
                if (fabsf(v[j]) > amax) amax = fabsf(v[j]);
            }
            int e = orc_e8m0_exponent(amax, Mmax);
            out_e8m0[c * (P / 32) + jb / 32] = (uint8_t)(e + 127);
            for (int j = 0; j < 32; j++) {
                int64_t s = s_begin + jb + j;
                uint8_t code = 0;
                if (jb + j < count && s < M) {
                    float y = ldexpf(v[j], -e);
                    uint32_t r16 = orc_rand16(seed, stream, (uint64_t)s * (uint64_t)cols + (uint64_t)c);
                    code = (target == ORC_TARGET_E4M3) ? orc_e4m3_encode(y, ORC_SR, r16) : orc_fp4_encode(y, ORC_SR, r16);
                }
                out[c * P + jb + j] = code;
            }
        }
}
