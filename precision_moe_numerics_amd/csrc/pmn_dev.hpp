// pmn_dev.hpp -- device helpers shared by the HIP kernels of the quantized MoE expert layer.
//
// Pages cited (by title and section heading):
//   [AREX] AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向传播
//          贯穿预训练到最后一次 RL rollout"; sections cited by heading below.
//
// Number formats used here (the pages name them; bit layouts are the OCP definitions):
//   FP4 E2M1 nibble: sign bit 3 | index into {0, .5, 1, 1.5, 2, 3, 4, 6}  ([AREX]
//     "转置打散分组,随机舍入保住期望值" lists exactly these sixteen values).
//   E4M3 byte (OCP E4M3FN): bias 7, max 448, subnormal step 2^-9.
//   E8M0 byte b: 2^(b - 127).
//
// gfx950 conversion instructions used, each checked on the device against the CPU oracle:
//   v_cvt_scalef32_pk_fp4_f32 with scale 1.0: round-to-nearest-even onto the FP4 grid,
//     saturating at 6, first operand in the low nibble (the scale only contributes its
//     power-of-two exponent, so it is kept at 1.0 and the block reciprocal is applied first).
//   v_cvt_scalef32_pk_f16_fp4 / _pk_f32_fp4 with scale 1.0: exact FP4 values.
//   v_cvt_pk_fp8_f32: round-to-nearest-even E4M3 for |x| <= 448 (NaN above: inputs are clamped).
//   v_cvt_sr_fp8_f32: stochastic E4M3 rounding that adds the top 20 bits of its random operand
//     to the 20 discarded mantissa bits; feeding (0xFFFF - r16) << 16 makes it round up exactly
//     when r16 < floor(f * 2^16), f being the position of |y| between its two grid neighbours.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pmn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

#define PMN_DEV __device__ __forceinline__

// ---- bf16 ---------------------------------------------------------------------------------

PMN_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
PMN_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
PMN_DEV uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 (a in the low half), round to nearest even: v_cvt_pk_bf16_f32.
PMN_DEV uint32_t bf16x2_bits(float a, float b)
{
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- E4M3 ---------------------------------------------------------------------------------

// Value of an E4M3 byte (finite codes).
// E4M3 (OCP, bias 7, no infinities) byte -> fp32 by the hardware converter: exact for every
// finite code, subnormals included; 0x7F / 0xFF (NaN) decode to NaN.
PMN_DEV float e4m3_value(uint32_t c)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// Non-negative t -> E4M3 byte, round to nearest even, saturating at 448.
PMN_DEV uint32_t e4m3_rne_sat(float t)
{
    t = fminf(t, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0, false) & 0xFFu;
}

// ---- correctly rounded quotients without a division sequence ------------------------------
//
// The activation quantizer needs RN(ab / 6), RN(q / s_o) and RN(1 / d) per 16-value block. The
// IEEE division sequence costs about ten instructions each; these replacements give the same
// bits on the domains where the quantizer uses them, which are finite and were checked
// exhaustively (the first two with IEEE fp32 arithmetic on the host, the third on the device).

// RN(a / 6) for every non-negative bf16 value a (widened to fp32): one product by RN(1/6) and one
// correction with the exact fma residual.
PMN_DEV float div6_rn(float a)
{
    const float y = 0x1.555556p-3f;   // RN(1/6)
    const float q = a * y;
    const float r = __builtin_fmaf(-q, 6.0f, a);
    return __builtin_fmaf(r, y, q);
}

// RN(q / s) given ys = RN(1 / s): one product and one fma correction. Exact whenever
// s = RN(A / 2688) >= 2^-96 for a bf16 amax A and q = RN(ab / 6) or ab / 4 for a bf16 block max
// ab <= A, except where the quotient is below 2^-11 (both results then encode as E4M3 zero).
PMN_DEV float div_rn(float q, float s, float ys)
{
    const float t = q * ys;
    const float r = __builtin_fmaf(-t, s, q);
    return __builtin_fmaf(r, ys, t);
}

// RN(1 / d) for every fp32 d in [2^-105, 2^126): the hardware reciprocal (within one ulp) and one
// Newton step with the exact fma residual.
PMN_DEV float recip_rn(float d)
{
    const float y = __builtin_amdgcn_rcpf(d);
    const float e = __builtin_fmaf(-d, y, 1.0f);
    return __builtin_fmaf(e, y, y);
}

// ---- FP4 ----------------------------------------------------------------------------------

// Two fp32 values -> one byte of two FP4 nibbles (a low, b high), placed at byte `sel` of old.
#define PMN_CVT_FP4(old, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// Byte `sel` of w (two FP4 nibbles) -> two fp32 values (low nibble first).
#define PMN_FP4_TO_F32(w, sel) __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((w), 1.0f, (sel))

// Byte `sel` of w -> two fp16 values (low nibble first).
#define PMN_FP4_TO_F16(w, sel) __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w), 1.0f, (sel))

// The 8 FP4 values of a code word (element 0 in the low nibble of byte 0) as fp32.
PMN_DEV void fp4x8_to_f32(uint32_t w, float (&q)[8])
{
    const f32x2 a = PMN_FP4_TO_F32(w, 0), b = PMN_FP4_TO_F32(w, 1);
    const f32x2 c = PMN_FP4_TO_F32(w, 2), d = PMN_FP4_TO_F32(w, 3);
    q[0] = a.x; q[1] = a.y; q[2] = b.x; q[3] = b.y;
    q[4] = c.x; q[5] = c.y; q[6] = d.x; q[7] = d.y;
}

// ---- E8M0 block exponent ----------------------------------------------------------------
//
// Smallest e in [-127, 127] with amax <= M * 2^e, for M = 448 (E4M3 elements), 6 (E2M1) and
// 127/64 (S2F6). With amax = m * 2^E (m in [1, 2)) and M = mM * 2^EM, e = E - EM + [m > mM].
// [AREX] "转置打散分组,随机舍入保住期望值": the backward must not be biased, so no element of a
// block may saturate; this rule guarantees that.
enum { E8M0_E4M3 = 0, E8M0_E2M1 = 1, E8M0_S2F6 = 2 };

template <int KIND>
PMN_DEV int e8m0_exponent(float amax)
{
    constexpr int EM = KIND == E8M0_E4M3 ? 8 : (KIND == E8M0_E2M1 ? 2 : 0);
    constexpr uint32_t MANT = KIND == E8M0_E4M3 ? 0x600000u : (KIND == E8M0_E2M1 ? 0x400000u : 0x7E0000u);
    uint32_t u = __float_as_uint(amax);
    if (u == 0u) return -127;
    int E;
    uint32_t m;
    uint32_t ef = u >> 23;
    if (ef != 0u) {
        E = (int)ef - 127;
        m = u & 0x7FFFFFu;
    } else {                              // fp32 subnormal: normalize
        int lz = __builtin_clz(u) - 8;    // u < 2^23
        E = -126 - lz;
        m = (u << lz) & 0x7FFFFFu;
    }
    int e = E - EM + (m > MANT ? 1 : 0);
    e = e < -127 ? -127 : e;
    e = e > 127 ? 127 : e;
    return e;
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) -------------------------------------
// Ten rounds on a four-word counter under a two-word key. A round multiplies words 0 and 2 by the
// two Philox multipliers; the new words 0 and 2 are the high halves of the products of words 2
// and 0, xor'ed with words 1 and 3 and the round key; the new words 1 and 3 are the low halves of
// those products; the key then advances by the two Weyl constants.
//
// The 8 random 16-bit values of elements 8*blk .. 8*blk+7 under (seed, stream), returned as
// four words: element 8*blk + j uses half (j & 1) of word j >> 1 (low half first). The counter is
// (blk lo, blk hi, stream, 0) and the key (seed lo, seed hi). The stream word, the zero word and
// the key are the same for every lane of a launch, so the first two rounds are written out to keep
// their products and xors on the scalar unit: round 0 costs one vector multiply, and each of the
// first two rounds two single vector xors.
PMN_DEV void rand16x8(uint64_t seed, uint32_t stream, uint64_t blk, uint32_t w[4])
{
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    // round 0 on (lo, hi, stream, 0)
    const uint64_t p0 = (uint64_t)0xD2511F53u * (uint32_t)blk;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * stream;
    // (readfirstlane keeps the lane-independent xor on the scalar unit)
    uint32_t c0 = __builtin_amdgcn_readfirstlane((uint32_t)(p1 >> 32) ^ k0) ^ (uint32_t)(blk >> 32);
    uint32_t c1 = (uint32_t)p1;
    uint32_t c2 = (uint32_t)(p0 >> 32) ^ k1;
    uint32_t c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
    // round 1: c1 is still lane-independent
    const uint64_t q0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t q1 = (uint64_t)0xCD9E8D57u * c2;
    w[0] = (uint32_t)(q1 >> 32) ^ (c1 ^ k0);
    w[1] = (uint32_t)q1;
    w[2] = __builtin_amdgcn_bitop3_b32((uint32_t)(q0 >> 32), c3, k1, 0x96);
    w[3] = (uint32_t)q0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
    // rounds 2 .. 9
#pragma unroll
    for (int r = 2; r < 10; r++) {
        const uint64_t m0 = (uint64_t)0xD2511F53u * w[0];
        const uint64_t m1 = (uint64_t)0xCD9E8D57u * w[2];
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(m1 >> 32), w[1], k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(m0 >> 32), w[3], k1, 0x96);
        w[1] = (uint32_t)m1;
        w[3] = (uint32_t)m0;
        w[0] = n0;
        w[2] = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// SR operand of the hardware converter for the element that owns 16-bit half `hi` of word w.
PMN_DEV uint32_t sr_operand(uint32_t w, int hi)
{
    uint32_t r16 = hi ? (w >> 16) : (w & 0xFFFFu);
    return (0xFFFFu - r16) << 16;
}

// y (|y| <= 448) -> E4M3 byte by stochastic rounding with the given SR operand.
PMN_DEV uint32_t e4m3_sr(float y, uint32_t rng)
{
    return (uint32_t)__builtin_amdgcn_cvt_sr_fp8_f32(y, (int)rng, 0, 0) & 0xFFu;
}

// E4M3 code of v / scale (scale a power of two) by stochastic rounding with the given SR operand,
// written into byte `sel` (0..3) of `word`.
PMN_DEV uint32_t e4m3_sr_scaled_into(uint32_t word, float v, uint32_t rng, float scale, int sel)
{
    switch (sel) {
    case 0: return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_fp8_f32((int)word, v, rng, scale, 0);
    case 1: return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_fp8_f32((int)word, v, rng, scale, 1);
    case 2: return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_fp8_f32((int)word, v, rng, scale, 2);
    default: return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_fp8_f32((int)word, v, rng, scale, 3);
    }
}

// Dequantize 8 consecutive NVFP4 values (one code word, one effective scale d) to fp32.
PMN_DEV void deq8(uint32_t cw, float d, float (&v)[8])
{
    float q[8];
    fp4x8_to_f32(cw, q);
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = q[i] * d;
}

// a + b for a per-lane a and a wavefront-uniform b: one 64-bit vector add. Written as asm so that
// the compiler keeps it an add instead of re-deriving each slot's counter with a 64-bit multiply.
PMN_DEV uint64_t add_uniform64(uint64_t a, uint64_t b)
{
    uint64_t r;
    asm("v_lshl_add_u64 %0, %1, 0, %2" : "=v"(r) : "v"(a), "s"(b));
    return r;
}

// y (|y| <= 448) -> E4M3 byte, round to nearest even.
PMN_DEV uint32_t e4m3_rne(float y)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFFu;
}

// y (|y| <= 6) -> FP4 nibble by stochastic rounding with 16 random bits (the E2M1 requant
// target, used for the pages' worked example): up iff r16 < floor(f * 2^16).
PMN_DEV uint32_t fp4_sr(float y, uint32_t r16)
{
    float a = fabsf(y);
    uint32_t base, scale_shift;
    if (a < 2.0f) { base = 0u; scale_shift = 17; }        // step 0.5: n = 2a
    else if (a < 4.0f) { base = 2u; scale_shift = 16; }   // step 1:   n = a, index = 2 + n
    else { base = 4u; scale_shift = 15; }                 // step 2:   n = a/2, index = 4 + n
    uint32_t N = (uint32_t)(a * __uint_as_float((127u + scale_shift) << 23));
    uint32_t L = N >> 16, f16 = N & 0xFFFFu;
    uint32_t idx = base + L + (r16 < f16 ? 1u : 0u);
    idx = idx > 7u ? 7u : idx;
    return idx | ((__float_as_uint(y) >> 28) & 8u);
}

// One block of 32 bf16 values (16 words) of row r, k-block kb -> 32 E4M3 codes (8 words, element
// 0 in the low byte) and the E8M0 exponent e (scale 2^e). SR draws the element index r * N + c.
template <bool SR>
PMN_DEV int mxfp8_block(const uint32_t (&w)[16], int64_t r, int64_t kb, int64_t N, uint64_t seed,
                        uint32_t stream_id, uint32_t (&o)[8])
{
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; j++) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
    const int e = e8m0_exponent<E8M0_E4M3>(amax);
    if (SR) {
        const uint64_t idx0 = (uint64_t)r * (uint64_t)N + (uint64_t)(kb * 32);   // multiple of 8
#pragma unroll
        for (int q = 0; q < 4; q++) {
            uint32_t rw[4];
            rand16x8(seed, stream_id, (idx0 >> 3) + q, rw);
            uint32_t lo = 0u, hi = 0u;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                uint32_t word = w[4 * q + j / 2];
                float v = (j & 1) ? bf16_hi(word) : bf16_lo(word);
                uint32_t c = e4m3_sr(__builtin_ldexpf(v, -e), sr_operand(rw[j >> 1], j & 1));
                if (j < 4) lo |= c << (8 * j); else hi |= c << (8 * (j - 4));
            }
            o[2 * q] = lo;
            o[2 * q + 1] = hi;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 8; q++) {
            float v0 = __builtin_ldexpf(bf16_lo(w[2 * q]), -e), v1 = __builtin_ldexpf(bf16_hi(w[2 * q]), -e);
            float v2 = __builtin_ldexpf(bf16_lo(w[2 * q + 1]), -e), v3 = __builtin_ldexpf(bf16_hi(w[2 * q + 1]), -e);
            int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
            o[q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, lo, true);
        }
    }
    return e;
}

// SwiGLU backward of one element, as bf16 bits: dh1 = g h3 silu'(h1), dh3 = g silu(h1), with
// silu'(h) = s (1 + h (1 - s)) and s = sigmoid(h)
PMN_DEV void swiglu_bwd_elem(float g, float h1, float h3, uint32_t& d1, uint32_t& d3)
{
    const float s = 1.0f / (1.0f + expf(-h1));
    d1 = f32_to_bf16_bits(g * h3 * (s * (1.0f + h1 * (1.0f - s))));
    d3 = f32_to_bf16_bits(g * h1 * s);
}

// ---- XCD-aware tile order for the GEMMs ----------------------------------------------------
//
// MI355X has 8 XCDs, each with its own L2; workgroup L of a 1-D grid runs on XCD L % 8, and the
// 32 CUs of an XCD run about 32 workgroups at a time. Tiles are grouped in "super-tiles" of
// SM row tiles x SN column tiles (SM * SN = 32): the j-th workgroup of XCD x takes position
// j % 32 of super-tile (j / 32) * 8 + x, so the workgroups an XCD runs together share SM A tiles
// and SN B tiles in its L2. Super-tiles are numbered row-major over a grid of
// ceil(rows / SM) x ceil(cols / SN); positions outside the tile grid return false.
struct TileXY {
    int64_t row, col, super_id;
};

PMN_DEV bool xcd_tile(int64_t L, int64_t row_tiles, int64_t col_tiles, int SM, int SN, TileXY& t)
{
    const int64_t x = L & 7, j = L >> 3;
    const int64_t s = (j >> 5) * 8 + x;
    const int p = (int)(j & 31);
    const int64_t scols = (col_tiles + SN - 1) / SN;
    const int64_t srow = s / scols, scol = s - srow * scols;
    t.super_id = s;
    t.row = srow * SM + p / SN;
    t.col = scol * SN + p % SN;
    return t.row < row_tiles && t.col < col_tiles;
}

// Grid size covering every super-tile of a rows x cols tile grid.
inline int64_t xcd_grid(int64_t row_tiles, int64_t col_tiles, int SM, int SN, int64_t batches = 1)
{
    const int64_t nsuper = ((row_tiles + SM - 1) / SM) * ((col_tiles + SN - 1) / SN) * batches;
    return 8 * 32 * ((nsuper + 7) / 8);
}

// SM x SN with SM * SN = 32 that wastes the fewest positions on a rows x cols tile grid.
inline void xcd_shape(int64_t row_tiles, int64_t col_tiles, int& SM, int& SN)
{
    const int cand[2][2] = {{8, 4}, {4, 8}};
    int64_t best = -1;
    for (auto& c : cand) {
        const int64_t n = ((row_tiles + c[0] - 1) / c[0]) * ((col_tiles + c[1] - 1) / c[1]);
        if (best < 0 || n < best) { best = n; SM = c[0]; SN = c[1]; }
    }
}

// ---- wave reductions ------------------------------------------------------------------------

PMN_DEV float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// ---- ragged groups --------------------------------------------------------------------------

// Unit t of the concatenation of per-group unit lists, where group g (slots offsets[g] ..
// offsets[g+1]) holds ceil(size / unit) units: its group, its index inside the group and the
// group's slot range. Wavefront-parallel (lane l reads group 64c + l, a prefix sum over the lanes
// and a ballot pick the group), so the cost does not grow with the group index. Every lane of
// the wavefront must call it; the result is wavefront-uniform. g = -1 when t is past the end.
struct GroupUnit {
    int g;
    int64_t index;      // unit index inside the group
    int64_t s0, s1;     // the group's slots
};

PMN_DEV GroupUnit locate_group_unit(const int64_t* offsets, int G, int64_t t, int64_t unit)
{
    const int lane = threadIdx.x & 63;
    int64_t before = 0;   // units of the groups of earlier chunks
    for (int c0 = 0; c0 < G; c0 += 64) {
        const int gl = c0 + lane;
        const int64_t a = gl < G ? offsets[gl] : 0, b = gl < G ? offsets[gl + 1] : 0;
        const int64_t n = (b - a + unit - 1) / unit;
        int64_t cum = n;   // inclusive prefix over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t y = __shfl_up(cum, d, 64);
            if (lane >= d) cum += y;
        }
        const uint64_t hit = __ballot(before + cum > t);
        if (hit) {
            const int lg = __builtin_ctzll(hit);
            GroupUnit r;
            r.g = c0 + lg;
            r.index = t - (before + __shfl(cum, lg, 64) - __shfl(n, lg, 64));
            r.s0 = __shfl(a, lg, 64);
            r.s1 = __shfl(b, lg, 64);
            return r;
        }
        before += __shfl(cum, 63, 64);
    }
    return GroupUnit{-1, 0, 0, 0};
}

// ---- GEMM epilogues shared by the forward GEMMs -------------------------------------------

// silu(h) = h * sigmoid(h) with the hardware exp2 and reciprocal (each within about 1 ulp in
// fp32); the product silu(h1) * h3 is rounded to bf16 afterwards, which dwarfs that error. For
// h -> -inf the reciprocal of +inf is 0 and the result is -0.
PMN_DEV float silu(float h)
{
    const float e = __builtin_amdgcn_exp2f(-h * 1.44269504088896341f);
    return h * __builtin_amdgcn_rcpf(1.0f + e);
}

// RHT32 + S2F6 on one 32 x 32 accumulator block whose 32 rows (n) are one aligned chunk:
// lane l holds column m = l % 32 and rows i = (v/4)*8 + (l/32)*4 + v%4. The 32 codes of slot m
// go to out_row_chunk (the epilogue's LDS tile), its E8M0 byte to e8m0_ptr. Butterfly stages
// h = 1, 2, 4, 8, 16 in that order: h = 1, 2, 8, 16 pair registers of one lane, h = 4 pairs the
// two lane halves.
PMN_DEV void rht_block_store(f32x16 z, uint32_t mask, int lane, int8_t* out_row_chunk, uint8_t* e8m0_ptr)
{
    const int hh = lane >> 5;
    float t[16];
#pragma unroll
    for (int v = 0; v < 16; v++) {
        const int i = (v >> 2) * 8 + hh * 4 + (v & 3);
        t[v] = __uint_as_float(__float_as_uint(z[v]) ^ (((mask >> i) & 1u) << 31));
    }
    // h = 1 (v ^ 1), h = 2 (v ^ 2)
#pragma unroll
    for (int hb = 1; hb <= 2; hb <<= 1) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            if ((v & hb) == 0) {
                float a = t[v], b = t[v + hb];
                t[v] = a + b;
                t[v + hb] = a - b;
            }
        }
    }
    // h = 4: across lane halves (lane l pairs with l ^ 32; the lower lane holds the first element
    // of each pair). v_permlane32_swap exchanges the upper lane half of its first register with
    // the lower lane half of its second. For registers (p, q) one swap gives A = [p_lo, q_lo] and
    // B = [p_hi, q_hi], so every lane holds both elements of one pair; A + B and A - B hold p's
    // results in their lower lanes and q's in their upper lanes, and a second swap of (A + B,
    // A - B) puts p's and q's results back in place.
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
        const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[v]), __float_as_uint(t[v + 1]), false, false);
        const float A = __uint_as_float(s1[0]), B = __uint_as_float(s1[1]);
        const float X = A + B, Y = A - B;
        const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(X), __float_as_uint(Y), false, false);
        t[v] = __uint_as_float(s2[0]);
        t[v + 1] = __uint_as_float(s2[1]);
    }
    // h = 8 (v ^ 4), h = 16 (v ^ 8)
#pragma unroll
    for (int hb = 4; hb <= 8; hb <<= 1) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            if ((v & hb) == 0) {
                float a = t[v], b = t[v + hb];
                t[v] = a + b;
                t[v + hb] = a - b;
            }
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; v++) amax = fmaxf(amax, fabsf(t[v]));
    {
        // max with the partner lane: the swap of (amax, amax) gives both lane halves' values to
        // every lane
        const auto m = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(m[0]), __uint_as_float(m[1]));
    }
    const int e = e8m0_exponent<E8M0_S2F6>(amax);
    // code c = RNE(t * 2^(6 - e)), |c| <= 127: the scaling is exact, and adding 1.5 * 2^23 (where
    // the float spacing is 1) rounds to the nearest even integer; the sum's low byte is c in two's
    // complement. Four such bytes pack with three byte permutes.
#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint32_t c[4];
#pragma unroll
        for (int j = 0; j < 4; j++) c[j] = __float_as_uint(__builtin_ldexpf(t[4 * q + j], 6 - e) + 12582912.0f);
        const uint32_t lo = __builtin_amdgcn_perm(c[1], c[0], 0x0c0c0400u);   // bytes c0, c1, 0, 0
        const uint32_t hi = __builtin_amdgcn_perm(c[3], c[2], 0x0c0c0400u);   // bytes c2, c3, 0, 0
        *reinterpret_cast<uint32_t*>(out_row_chunk + q * 8 + hh * 4) = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    if (hh == 0) *e8m0_ptr = (uint8_t)(e + 127);
}

// ---- shared by the ring-buffered GEMMs -----------------------------------------------------
// Asynchronous global -> LDS copies. The LDS destination of lane l is m0 + 16 l (dwordx4) or
// m0 + 4 l (dword), m0 being wavefront-uniform. They are issued from inline assembly so that the
// compiler does not make every later LDS read wait for all of them; the kernel waits itself.
PMN_DEV void dma16(const void* src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(src) : "memory", "m0");
}
PMN_DEV void dma4(const void* src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(src) : "memory", "m0");
}
// 2 bytes per lane; lane l's bytes land in the low half of the LDS dword at m0 + 4 l
PMN_DEV void dma2(const void* src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_ushort %1, off" ::"s"(lds_base), "v"(src) : "memory", "m0");
}
// Wait for this wavefront's LDS reads and until at most N of its loads are outstanding, then
// barrier: afterwards the stage those loads waited for is visible to the workgroup and every
// wavefront has finished reading the stages it read before.
template <int N>
PMN_DEV void wait_loads_and_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// Forward GEMMs with the SwiGLU epilogue (256 x 256 tiles of 4 wavefronts, 2 along weight rows):
// the expert-local weight row (within its 2F rows) that tile row t of feature tile nt holds.
// Blocks i of wavefront wr = t / 128 hold w1 (i = 0, 1) and w3 (i = 2, 3) rows of the same 64
// features, so an accumulator lane holds h1 and h3 of one feature in blocks i and i + 2
PMN_DEV int64_t swiglu_a_row(int t, int64_t nt, int64_t F)
{
    return ((t >> 6) & 1) * F + nt * 128 + (t >> 7) * 64 + ((t >> 5) & 1) * 32 + (t & 31);
}
// The same for an F that need not be a multiple of 128 (a multiple of 32): a 32-row run past the
// expert's F features re-reads the first run of the same matrix (w1 or w3); its outputs are never
// stored.
PMN_DEV int64_t swiglu_a_row_clamped(int t, int64_t nt, int64_t F)
{
    const int64_t f = nt * 128 + (t >> 7) * 64 + ((t >> 5) & 1) * 32 + (t & 31);
    return ((t >> 6) & 1) * F + (f < F ? f : (int64_t)(t & 31));
}

}  // namespace pmn
