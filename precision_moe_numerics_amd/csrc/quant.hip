// quant.hip -- NVFP4 quantization, MXFP8 row-wise gradient quantization and the standalone
// RHT32 + S2F6 combine quantizer.
//
// Pages cited (by title and section heading):
//   [AREX] AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向传播
//          贯穿预训练到最后一次 RL rollout".
//
// All three kernels stream HBM once: each element is read once and its codes written once; the
// per-token outer scale is reduced across a wavefront while the row sits in registers.
#include "pmn_dev.hpp"
#include "pmn_kernels.hpp"

namespace pmn {

// ------------------------------------------------------------------------------------------
// NVFP4 block quantization  [AREX] "转置打散分组,随机舍入保住期望值": 16 consecutive values share
// an E4M3 scale chosen so that the block max lands on the top of the FP4 grid.
// [AREX] "配方的代价:预训练约 2% 的计算效率": activations pick the better of two scale factors
// (here: the block max mapped to 6 or to 4, the smaller squared error wins, ties keep 6).
// ------------------------------------------------------------------------------------------

struct Block16 {
    float x[16];
};

PMN_DEV void load_block(const uint4* p, Block16& b)
{
    uint4 lo = p[0], hi = p[1];
    uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        b.x[2 * i] = bf16_lo(w[i]);
        b.x[2 * i + 1] = bf16_hi(w[i]);
    }
}

PMN_DEV float block_absmax(const Block16& b)
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) m = fmaxf(m, fabsf(b.x[i]));
    return m;
}

// One candidate: scale byte, 16 nibbles (2 words) and the effective scale d. FAST (rows whose
// outer scale s_o >= 2^-96, with ys = RN(1 / s_o)) forms the same correctly rounded quotients
// without division sequences (div6_rn, div_rn, recip_rn: d then lies in [2^-105, 2^126)).
template <int CAND, bool FAST = false>
PMN_DEV void quant_candidate(const Block16& b, float ab, float s_o, uint32_t& sb, uint32_t& w0,
                             uint32_t& w1, float& d, float ys = 0.0f)
{
    float t;
    if (FAST) t = div_rn(CAND == 4 ? ab * 0.25f : div6_rn(ab), s_o, ys);
    else t = (ab / (float)CAND) / s_o;
    sb = e4m3_rne_sat(t);
    d = e4m3_value(sb) * s_o;
    float r;
    if (FAST) r = (d != 0.0f) ? recip_rn(d) : 0.0f;
    else r = (d != 0.0f) ? fminf(1.0f / d, 3.402823466e38f) : 0.0f;
    w0 = 0u;
    w1 = 0u;
    w0 = PMN_CVT_FP4(w0, b.x[0] * r, b.x[1] * r, 0);
    w0 = PMN_CVT_FP4(w0, b.x[2] * r, b.x[3] * r, 1);
    w0 = PMN_CVT_FP4(w0, b.x[4] * r, b.x[5] * r, 2);
    w0 = PMN_CVT_FP4(w0, b.x[6] * r, b.x[7] * r, 3);
    w1 = PMN_CVT_FP4(w1, b.x[8] * r, b.x[9] * r, 0);
    w1 = PMN_CVT_FP4(w1, b.x[10] * r, b.x[11] * r, 1);
    w1 = PMN_CVT_FP4(w1, b.x[12] * r, b.x[13] * r, 2);
    w1 = PMN_CVT_FP4(w1, b.x[14] * r, b.x[15] * r, 3);
}

// Squared error e = fma(delta_i, delta_i, e) over i = 0..15, delta_i = fma(-q_i, d, x_i).
PMN_DEV float candidate_error(const Block16& b, uint32_t w0, uint32_t w1, float d)
{
    float q[16];
    float (&q0)[8] = *reinterpret_cast<float(*)[8]>(&q[0]);
    float (&q1)[8] = *reinterpret_cast<float(*)[8]>(&q[8]);
    fp4x8_to_f32(w0, q0);
    fp4x8_to_f32(w1, q1);
    float e = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float delta = __builtin_fmaf(-q[i], d, b.x[i]);
        e = __builtin_fmaf(delta, delta, e);
    }
    return e;
}

// ab: the block's max |x| (block_absmax(b)).
template <bool FOUR_SIX, bool FAST = false>
PMN_DEV void quant_block_ab(const Block16& b, float ab, float s_o, uint32_t& sb, uint2& q, float ys = 0.0f)
{
    uint32_t sb6, a0, a1;
    float d6;
    quant_candidate<6, FAST>(b, ab, s_o, sb6, a0, a1, d6, ys);
    sb = sb6;
    q = make_uint2(a0, a1);
    if (FOUR_SIX) {
        uint32_t sb4, c0, c1;
        float d4;
        quant_candidate<4, FAST>(b, ab, s_o, sb4, c0, c1, d4, ys);
        float e6 = candidate_error(b, a0, a1, d6);
        float e4 = candidate_error(b, c0, c1, d4);
        if (e4 < e6) {
            sb = sb4;
            q = make_uint2(c0, c1);
        }
    }
}

template <bool FOUR_SIX>
PMN_DEV void quant_block(const Block16& b, float s_o, uint32_t& sb, uint2& q)
{
    quant_block_ab<FOUR_SIX>(b, block_absmax(b), s_o, sb, q);
}

PMN_DEV float outer_from_amax(float amax) { return amax > 0.0f ? amax / 2688.0f : 1.0f; }

// One wavefront per row; the row stays in registers (NBL blocks of 16 per lane) while its
// amax is reduced, then every block is quantized. Rows of up to 64 * 16 * NBL values.
template <int NBL, bool FOUR_SIX>
__global__ __launch_bounds__(256) void k_nvfp4_rows(const uint16_t* __restrict__ x, int64_t rows,
                                                    int64_t cols, uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales,
                                                    float* __restrict__ outer_out)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int nb = (int)(cols >> 4);
    const uint4* xr = reinterpret_cast<const uint4*>(x + r * cols);
    Block16 blk[NBL];
    float ab[NBL];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NBL; j++) {
        int b = lane + 64 * j;
        ab[j] = 0.0f;
        if (b < nb) {
            load_block(xr + 2 * b, blk[j]);
            ab[j] = block_absmax(blk[j]);
            amax = fmaxf(amax, ab[j]);
        }
    }
    amax = wave_max(amax);
    const float s_o = outer_from_amax(amax);
    if (lane == 0) outer_out[r] = s_o;
    uint2* cr = reinterpret_cast<uint2*>(codes + r * (cols >> 1));
    uint8_t* sr = scales + r * nb;
    // the row's quotients take the division-free path when its outer scale allows (uniform per row)
    const bool fast = s_o >= 0x1p-96f;
    const float ys = fast ? 1.0f / s_o : 0.0f;
#pragma unroll
    for (int j = 0; j < NBL; j++) {
        int b = lane + 64 * j;
        if (b < nb) {
            uint32_t sb;
            uint2 q;
            if (fast) quant_block_ab<FOUR_SIX, true>(blk[j], ab[j], s_o, sb, q, ys);
            else quant_block_ab<FOUR_SIX, false>(blk[j], ab[j], s_o, sb, q);
            cr[b] = q;
            sr[b] = (uint8_t)sb;
        }
    }
}

// Rows of 129 .. 512 blocks (up to 8192 values): the 4 wavefronts of a workgroup share one row,
// lane l of wavefront w holding blocks 256 j + 64 w + l (j < NBL), so each lane keeps at most
// NBL blocks in registers (more wavefronts fit per SIMD) and every load instruction reads 2 KB
// of contiguous row. The row amax is combined across the wavefronts through LDS.
template <int NBL, bool FOUR_SIX>
__global__ __launch_bounds__(256) void k_nvfp4_row_split(const uint16_t* __restrict__ x, int64_t rows,
                                                         int64_t cols, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales,
                                                         float* __restrict__ outer_out)
{
    __shared__ float wmax[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t r = blockIdx.x;
    const int nb = (int)(cols >> 4);
    const uint4* xr = reinterpret_cast<const uint4*>(x + r * cols);
    Block16 blk[NBL];
    float ab[NBL];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NBL; j++) {
        const int b = 256 * j + 64 * w + lane;
        ab[j] = 0.0f;
        if (b < nb) {
            load_block(xr + 2 * b, blk[j]);
            ab[j] = block_absmax(blk[j]);
            amax = fmaxf(amax, ab[j]);
        }
    }
    amax = wave_max(amax);
    if (lane == 0) wmax[w] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s_o = outer_from_amax(amax);
    if (threadIdx.x == 0) outer_out[r] = s_o;
    uint2* cr = reinterpret_cast<uint2*>(codes + r * (cols >> 1));
    uint8_t* sr = scales + r * nb;
    const bool fast = s_o >= 0x1p-96f;   // uniform per row, as in k_nvfp4_rows
    const float ys = fast ? 1.0f / s_o : 0.0f;
#pragma unroll
    for (int j = 0; j < NBL; j++) {
        const int b = 256 * j + 64 * w + lane;
        if (b < nb) {
            uint32_t sb;
            uint2 q;
            if (fast) quant_block_ab<FOUR_SIX, true>(blk[j], ab[j], s_o, sb, q, ys);
            else quant_block_ab<FOUR_SIX, false>(blk[j], ab[j], s_o, sb, q);
            cr[b] = q;
            sr[b] = (uint8_t)sb;
        }
    }
}

// One thread per block of 16 with the outer scales already known (weights after the group
// amax pass, caller-provided outer scales, or rows too long for k_nvfp4_rows).
template <bool FOUR_SIX>
__global__ __launch_bounds__(256) void k_nvfp4_given(const uint16_t* __restrict__ x, int64_t rows,
                                                     int64_t cols, int64_t rows_per_outer,
                                                     const float* __restrict__ outer,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales)
{
    const int64_t nb = cols >> 4;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * nb) return;
    const int64_t r = i / nb;
    Block16 blk;
    load_block(reinterpret_cast<const uint4*>(x) + 2 * i, blk);
    uint32_t sb;
    uint2 q;
    quant_block<FOUR_SIX>(blk, outer[r / rows_per_outer], sb, q);
    reinterpret_cast<uint2*>(codes)[i] = q;
    scales[i] = (uint8_t)sb;
}

// 16 x 16 square blocks ([AREX] "转置打散分组,随机舍入保住期望值": the blocking NVIDIA uses so that
// a tensor and its transpose quantize bit-identically). A wavefront takes a band of 16 rows x 4
// tiles; lane l holds row l % 16 of tile l / 16 (16 values) and the tile amax is a 4-step
// butterfly max over the tile's 16 lanes. Each row segment is then a weight-mode block whose amax
// is the tile's; the scale byte is stored per row segment (equal within the tile).
__global__ __launch_bounds__(256) void k_nvfp4_2d(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                  int64_t rows_per_outer, const float* __restrict__ outer,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t tiles_c = cols >> 4;
    const int64_t strips = (tiles_c + 3) >> 2;
    const int64_t band = wave / strips;
    if (band >= (rows >> 4)) return;                     // wavefront-uniform
    const int64_t J = (wave - band * strips) * 4 + (lane >> 4);
    const int64_t r = band * 16 + (lane & 15);
    const bool ok = J < tiles_c;
    Block16 blk;
    float am = 0.0f;
    if (ok) {
        load_block(reinterpret_cast<const uint4*>(x + r * cols + J * 16), blk);
        am = block_absmax(blk);
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) am = fmaxf(am, __shfl_xor(am, m, 64));
    if (ok) {
        uint32_t sb, w0, w1;
        float d;
        quant_candidate<6>(blk, am, outer[r / rows_per_outer], sb, w0, w1, d);
        reinterpret_cast<uint2*>(codes + r * (cols >> 1))[J] = make_uint2(w0, w1);
        scales[r * tiles_c + J] = (uint8_t)sb;
    }
}

// Group amax: max |x| over each group of rows_per_outer rows, as fp32 bits folded with an
// integer atomic max (order-independent and exact, so the result is deterministic). At most
// AMAX_BLOCKS workgroups per group, each looping over the group with 16 independent 16-byte
// loads per thread per step (indices past the group end re-read its last chunk, which leaves a
// max unchanged), reduce in LDS and issue one atomic, so no address sees many atomics.
constexpr int AMAX_CHUNKS_PER_THREAD = 16;
constexpr int AMAX_BLOCKS = 32;

__global__ __launch_bounds__(256) void k_group_amax(const uint16_t* __restrict__ x, int64_t group_elems,
                                                    uint32_t* __restrict__ amax_bits)
{
    __shared__ float wmax[4];
    const int64_t g = blockIdx.y;
    const uint4* xg = reinterpret_cast<const uint4*>(x + g * group_elems);
    const int64_t n16 = group_elems >> 3;
    const int64_t step = (int64_t)gridDim.x * 256 * AMAX_CHUNKS_PER_THREAD;
    float m = 0.0f;
    for (int64_t base = (int64_t)blockIdx.x * 256 * AMAX_CHUNKS_PER_THREAD + threadIdx.x; base < n16; base += step) {
        uint4 v[AMAX_CHUNKS_PER_THREAD];
#pragma unroll
        for (int u = 0; u < AMAX_CHUNKS_PER_THREAD; u++) {
            const int64_t i = base + u * 256;
            // nontemporal: a pure streaming read (measured faster than cached loads here)
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xg) + (i < n16 ? i : n16 - 1));
            v[u] = make_uint4(t.x, t.y, t.z, t.w);
        }
#pragma unroll
        for (int u = 0; u < AMAX_CHUNKS_PER_THREAD; u++) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int q = 0; q < 4; q++) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[q])), fabsf(bf16_hi(w[q]))));
        }
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        atomicMax(amax_bits + g, __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ void k_outer_from_amax(float* outer, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) outer[i] = outer_from_amax(outer[i]);   // outer[i] holds the amax bits
}

__global__ void k_copy_f32(const float* __restrict__ a, float* __restrict__ b, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) b[i] = a[i];
}

// ------------------------------------------------------------------------------------------
// Weights in one read. The per-(expert, matrix) outer scale needs the whole matrix's amax before
// any block, and the Infinity Cache does not serve a second pass faster than HBM. Here the whole
// chip holds one matrix at a time: one 512-thread workgroup per CU (a cooperative launch, so all
// are resident together), thread t of T taking blocks t, t + T, .. (W1P_NBT of them).
//
// Round m: matrix m + 1 (copied into the LDS during the previous round) moves into registers,
// the copies of matrix m + 2 are issued, matrix m + 1's partial amax is published, matrix m's
// amax is gathered from every workgroup's word, and matrix m (in registers since the previous
// round) is quantized while matrix m + 2 arrives. The copies go global -> LDS without registers
// (each lane's 16 bytes land at its own LDS position), so the kernel waits for them with exact
// counts: loads into registers would make the compiler wait for every outstanding load wherever
// stores are pending too.
//
// A workgroup's partial amax is a max of |bf16| values, so it is one of them: a word is
// (m + 1) << 16 | its 16 bits, published in slot m % 4 of an array in the workspace (a workgroup
// can be at most three rounds ahead of the slowest, so four slots never overwrite a word still
// awaited). The words are cleared before the launch. Codes, scales and outer scales are those of
// k_nvfp4_given.
// ------------------------------------------------------------------------------------------
constexpr int W1P_THREADS = 512;
constexpr int W1P_WAVES = W1P_THREADS / 64;
constexpr int W1P_NBT = 7;          // blocks per thread per matrix
constexpr int W1P_MAX_WG = 512;     // workspace sized for up to this many workgroups
constexpr int64_t W1P_MAX_G = 65535;
constexpr int W1P_SPIN_LIMIT = 1 << 22;

typedef uint32_t w1p_u32x4 __attribute__((ext_vector_type(4)));
struct RawBlock16 {
    w1p_u32x4 lo, hi;
};

PMN_DEV Block16 unpack_block(const RawBlock16& r)
{
    Block16 b;
    const uint32_t w[8] = {r.lo[0], r.lo[1], r.lo[2], r.lo[3], r.hi[0], r.hi[1], r.hi[2], r.hi[3]};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        b.x[2 * i] = bf16_lo(w[i]);
        b.x[2 * i + 1] = bf16_hi(w[i]);
    }
    return b;
}

template <int N>
PMN_DEV void w1p_wait_loads()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The backward's operand from the same read (RQ). [AREX] "转置打散分组,随机舍入保住期望值": the
// backward multiplies by the transposed weights, whose blocks run along the other axis, so the
// NVFP4 weights are dequantized, transposed and re-quantized to MXFP8 (E8M0 per 32 values, SR).
// Weights do not change between a step's forward and backward, so the RQ kernel produces that
// operand while each matrix is on chip. Its workgroups own rectangular tiles instead of
// interleaved blocks: tile (band, q) is rows band * TH .. and columns q * TW .. of every matrix
// (TH a multiple of 64, TW of 16, one tile per workgroup), thread t holding blocks t + 512 k of
// the tile in row-major order. After quantizing matrix m a workgroup stages the tile's codes and
// scales in the LDS; thread pairs then take 8 columns x 32 rows (16 rows per lane, the pair's
// maxima meet by one exchange), dequantize, reduce the per-column amax and convert by SR (one
// Philox4x32-10 call per 8 columns of a row, keyed by the element's index in the [rows x cols]
// source) into one 16-byte chunk per column of the backward's blocked W^T layout. The bytes are
// those of requant_transpose_sr_mxfp8 on the quantized weights (ungrouped, E4M3, blocked).
constexpr int W1R_STG_CODES = 32768;   // TH * (TW / 2 + 8) bytes with TH <= 512, TH * TW <= 57344
constexpr int W1R_STG_SCALES = 3584;   // TH * TW / 16
constexpr int W1R_TH_MAX = 512;
constexpr int W1R_TILE_MIN = 6 * 64 * 128;   // six wavefronts of requant lanes, 128 values each

struct W1PArgs {
    const uint16_t* x;
    int64_t G;              // matrices (rows_per_outer rows each)
    int64_t group_blocks;   // 16-value blocks per matrix
    float* outer_out;
    uint8_t* codes;
    uint8_t* scales;
    uint32_t* words;
    uint32_t* flags;
    // RQ: the matrix shape, the tile and the W^T outputs
    int64_t R, C;
    int TH, TW;
    uint8_t* wt;            // E4M3 [C x G*R], blocked (1 KB blocks of 16 rows x 64 bytes)
    uint8_t* wte;           // E8M0 [G*R/32 x C]
    uint64_t seed;
    uint32_t stream_id;
};

template <bool RQ>
__global__ __launch_bounds__(W1P_THREADS, 1) void k_nvfp4_weight_1pass(W1PArgs a)
{
    // landing area of the copies: wavefront w, copy c (block c / 2, half c % 2) at [w][c]
    __shared__ __attribute__((aligned(1024))) uint8_t sdata[W1P_WAVES][2 * W1P_NBT][1024];
    __shared__ __attribute__((aligned(16))) uint8_t stg_c[RQ ? W1R_STG_CODES : 16];   // RQ: staged codes
    __shared__ uint8_t stg_s[RQ ? W1R_STG_SCALES : 16];                               // RQ: staged scales
    __shared__ uint32_t swords[W1P_WAVES][64];
    __shared__ float red_a[W1P_WAVES];
    __shared__ uint32_t red_w[2][W1P_WAVES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nwg = gridDim.x;
    const int64_t G = a.G, group_blocks = a.group_blocks;
    const uint32_t lds_data = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)&sdata[wave][0][0]);
    const uint32_t lds_words = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)&swords[wave][0]);
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x);

    // block k of this thread: its index within the matrix and whether it exists (a thread past
    // the last block re-reads an existing one, which changes no max and is not quantized)
    int bidx[W1P_NBT];   // fewer than 2^31 blocks per matrix (one matrix fits on chip)
    bool bok[W1P_NBT];
    const int bpr = RQ ? a.TW >> 4 : 0;                  // RQ: blocks per tile row
    const int pitch = RQ ? (a.TW >> 1) + 8 : 0;          // RQ: staged code bytes per tile row
    const int64_t row0 = RQ ? (int64_t)(blockIdx.x / (int)(a.C / a.TW)) * a.TH : 0;
    const int64_t col0 = RQ ? (int64_t)(blockIdx.x % (int)(a.C / a.TW)) * a.TW : 0;
#pragma unroll
    for (int k = 0; k < W1P_NBT; k++) {
        if (RQ) {
            const int beta = tid + W1P_THREADS * k, nblk = (a.TH * a.TW) >> 4;
            bok[k] = beta < nblk;
            const int b = bok[k] ? beta : 0;
            bidx[k] = (int)(((row0 + b / bpr) * a.C + col0) / 16 + b % bpr);
        } else {
            const int64_t blk = (int64_t)blockIdx.x * W1P_THREADS + tid + (int64_t)k * nwg * W1P_THREADS;
            bok[k] = blk < group_blocks;
            bidx[k] = (int)(bok[k] ? blk : group_blocks - 1);
        }
    }

    // matrix m into the landing area: 14 copies per lane
    auto copy_in = [&](int64_t m) {
#pragma unroll
        for (int k = 0; k < W1P_NBT; k++) {
            const uint8_t* src = xb + 32 * (m * group_blocks + bidx[k]);
            dma16(src, lds_data + (2 * k) * 1024);
            dma16(src + 16, lds_data + (2 * k + 1) * 1024);
        }
    };
    // the landed copies into registers (the caller has waited for them)
    auto read_in = [&](RawBlock16 (&b)[W1P_NBT]) {
#pragma unroll
        for (int k = 0; k < W1P_NBT; k++) {
            b[k].lo = *reinterpret_cast<const w1p_u32x4*>(&sdata[wave][2 * k][16 * lane]);
            b[k].hi = *reinterpret_cast<const w1p_u32x4*>(&sdata[wave][2 * k + 1][16 * lane]);
        }
        // every lane's reads are done before its next copies land on the same bytes
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    // publish this workgroup's max |x| of matrix m (a bf16 value: its upper 16 bits)
    auto arrive = [&](int64_t m, const RawBlock16 (&b)[W1P_NBT]) {
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k < W1P_NBT; k++) v = fmaxf(v, block_absmax(unpack_block(b[k])));
        v = wave_max(v);
        if (lane == 0) red_a[wave] = v;
        __syncthreads();
        if (tid == 0) {
            float r = red_a[0];
#pragma unroll
            for (int w = 1; w < W1P_WAVES; w++) r = fmaxf(r, red_a[w]);
            const uint32_t word = ((uint32_t)(m + 1) << 16) | (__float_as_uint(r) >> 16);
            __hip_atomic_store(a.words + (m & 3) * W1P_MAX_WG + blockIdx.x, word, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    // thread u < nwg reads workgroup u's word of matrix m into the LDS (every lane issues one
    // copy, so that each wavefront's count of outstanding copies is fixed)
    auto word_in = [&](int64_t m) {
        dma4(a.words + (m & 3) * W1P_MAX_WG + (tid < nwg ? tid : 0), lds_words);
    };
    // matrix m's amax from the landed words; a word not yet published is read again (boundedly)
    auto gather = [&](int64_t m) -> float {
        uint32_t bits = 0;
        if (tid < nwg) {
            uint32_t word = swords[wave][lane];
            const uint32_t tag = (uint32_t)(m + 1);
            const uint32_t* wp = a.words + (m & 3) * W1P_MAX_WG + tid;
            for (int spin = 0; (word >> 16) != tag; spin++) {
                if (spin == W1P_SPIN_LIMIT) {
                    // never expected with every workgroup resident; the outputs are then wrong
                    // and flags[0] says so, but no wavefront waits forever
                    atomicOr(a.flags, 1u);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
                word = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            bits = word & 0xffffu;
        }
        // max |bf16| bits = bits of the max (non-negative values order as their bit patterns)
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) bits = max(bits, (uint32_t)__shfl_xor((int)bits, d, 64));
        if (lane == 0) red_w[m & 1][wave] = bits;
        __syncthreads();
        uint32_t r = red_w[m & 1][0];
#pragma unroll
        for (int w = 1; w < W1P_WAVES; w++) r = max(r, red_w[m & 1][w]);
        return __uint_as_float(r << 16);
    };
    auto quantize = [&](int64_t m, const RawBlock16 (&b)[W1P_NBT], float s_o) {
        const bool fast = s_o >= 0x1p-96f;   // uniform per matrix, as in k_nvfp4_rows
        const float ys = fast ? 1.0f / s_o : 0.0f;
#pragma unroll
        for (int k = 0; k < W1P_NBT; k++) {
            if (bok[k]) {
                const Block16 v = unpack_block(b[k]);
                uint32_t sb;
                uint2 q;
                if (fast) quant_block_ab<false, true>(v, block_absmax(v), s_o, sb, q, ys);
                else quant_block_ab<false, false>(v, block_absmax(v), s_o, sb, q);
                const int64_t i = m * group_blocks + bidx[k];
                reinterpret_cast<uint2*>(a.codes)[i] = q;
                a.scales[i] = (uint8_t)sb;
                if (RQ) {
                    // (the laundered sizes keep these offsets from being hoisted out of the
                    // matrix loop, where they would hold registers for the whole kernel)
                    int bp = bpr, pt = pitch;
                    asm volatile("" : "+s"(bp), "+s"(pt));
                    const int beta = tid + W1P_THREADS * k;
                    const int r = beta / bp, c = beta - r * bp;
                    *reinterpret_cast<uint2*>(&stg_c[r * pt + 8 * c]) = q;
                    stg_s[r * bp + c] = (uint8_t)sb;
                }
            }
        }
    };
    // RQ: matrix m's tile, staged by quantize, to E4M3 codes of W^T by SR
    auto requant = [&](int64_t m, float s_o) {
        __syncthreads();   // every thread's codes and scales are staged
        // (sizes laundered as in quantize: every address below is formed inside this call)
        int pt = pitch, bp = bpr, cpr = a.TW >> 3;        // cpr: column octets per tile row
        asm volatile("" : "+s"(pt), "+s"(bp), "+s"(cpr));
        const int p = tid >> 1, h = tid & 1;
        if (p >= cpr * (a.TH >> 5)) return;
        const int rb = p / cpr, co = p - rb * cpr;
        const int r0 = 32 * rb + 16 * h;                  // the lane's first tile row
        const uint8_t* cb = &stg_c[r0 * pt + 4 * co];
        const uint8_t* sbp = &stg_s[r0 * bp + (co >> 1)];
        // pass 1: per-column amax over the lane's 16 rows (codes and scales read from the LDS in
        // both passes, so that neither pass keeps them in registers)
        float amax[8];
#pragma unroll
        for (int c = 0; c < 8; c++) amax[c] = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            float v0[8], v1[8];
            deq8(*reinterpret_cast<const uint32_t*>(cb + j * pt), e4m3_value(sbp[j * bp]) * s_o, v0);
            deq8(*reinterpret_cast<const uint32_t*>(cb + (j + 1) * pt), e4m3_value(sbp[(j + 1) * bp]) * s_o, v1);
#pragma unroll
            for (int c = 0; c < 8; c++) amax[c] = fmaxf(fmaxf(amax[c], fabsf(v0[c])), fabsf(v1[c]));
        }
        // the other 16 rows of the 32-row block sit in the partner lane
        float escale[8];   // 2^e: the scaled converter divides by it exactly
        uint32_t elo = 0u, ehi = 0u;
#pragma unroll
        for (int c = 0; c < 8; c++) {
            amax[c] = fmaxf(amax[c], __shfl_xor(amax[c], 1, 64));
            const int e = e8m0_exponent<E8M0_E4M3>(amax[c]);
            escale[c] = __builtin_ldexpf(1.0f, e);
            if (c < 4) elo |= (uint32_t)(e + 127) << (8 * c);
            else ehi |= (uint32_t)(e + 127) << (8 * (c - 4));
        }
        const int64_t n0 = m * a.R + row0 + r0;           // W row (W^T column) of the lane's first row
        const int64_t k0 = col0 + 8 * co;                 // first W column (W^T row)
        if (h == 0) *reinterpret_cast<uint2*>(a.wte + (n0 >> 5) * a.C + k0) = make_uint2(elo, ehi);
        asm volatile("" ::: "memory");   // pass 2 reads the LDS again
        // pass 2: element (n, k) of the [G*R x C] source draws from Philox block (n * C + k) / 8;
        // consecutive rows are C / 8 blocks apart. (The laundered key makes the scalar unit
        // derive the round keys here rather than hold them for the whole kernel.)
        uint32_t seed_lo = (uint32_t)a.seed, seed_hi = (uint32_t)(a.seed >> 32), sid = a.stream_id;
        asm volatile("" : "+s"(seed_lo), "+s"(seed_hi), "+s"(sid));
        const uint64_t seed = ((uint64_t)seed_hi << 32) | seed_lo;
        uint64_t ctr = ((uint64_t)n0 * (uint64_t)a.C + (uint64_t)k0) >> 3;
        const uint64_t cstep = (uint64_t)a.C >> 3;
        uint32_t o[8][4];
#pragma unroll
        for (int c = 0; c < 8; c++)
#pragma unroll
            for (int q = 0; q < 4; q++) o[c][q] = __builtin_nondeterministic_value(o[c][q]);   // every byte is written below
#pragma unroll
        for (int j = 0; j < 16; j++) {
            float v[8];
            deq8(*reinterpret_cast<const uint32_t*>(cb + j * pt), e4m3_value(sbp[j * bp]) * s_o, v);
            uint32_t rw[4];
            rand16x8(seed, sid, ctr, rw);
            ctr = add_uniform64(ctr, cstep);
#pragma unroll
            for (int c = 0; c < 8; c++)
                o[c][j >> 2] = e4m3_sr_scaled_into(o[c][j >> 2], v[c], sr_operand(rw[c >> 1], c & 1), escale[c], j & 3);
        }
        // the lane's 16 slots of column k are one 16-byte chunk of W^T row k
        const int64_t ldb = (G * a.R) >> 6;               // 64-slot block columns of W^T
#pragma unroll
        for (int c = 0; c < 8; c++) {
            const int64_t k = k0 + c;
            const int r16 = (int)(k & 15);
            const int pos = (int)((n0 & 63) >> 4) ^ ((r16 >> 2) & 3);
            *reinterpret_cast<uint4*>(a.wt + ((k >> 4) * ldb + (n0 >> 6)) * 1024 + 64 * r16 + 16 * pos) =
                make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]);
        }
    };
    // round m: cur holds matrix m (published); matrix m + 1 sits in the landing area
    auto round = [&](int64_t m, RawBlock16 (&cur)[W1P_NBT], RawBlock16 (&nx)[W1P_NBT]) {
        word_in(m);
        const bool more1 = m + 1 < G, more2 = m + 2 < G;
        if (more1) {
            w1p_wait_loads<1>();                       // all but the word: matrix m + 1 has landed
            read_in(nx);
        }
        if (more2) copy_in(m + 2);
        if (more1) arrive(m + 1, nx);
        // younger than the word: matrix m + 2's copies (and wavefront 0's publishing store)
        if (more2) w1p_wait_loads<2 * W1P_NBT>();
        else w1p_wait_loads<0>();
        const float s_o = outer_from_amax(gather(m));
        if (blockIdx.x == 0 && tid == 0) a.outer_out[m] = s_o;
        quantize(m, cur, s_o);
        if (RQ) requant(m, s_o);
    };
    RawBlock16 b0[W1P_NBT], b1[W1P_NBT];
    copy_in(0);
    w1p_wait_loads<0>();
    read_in(b0);
    if (G > 1) copy_in(1);
    arrive(0, b0);
    for (int64_t m = 0; m < G; m += 2) {
        round(m, b0, b1);
        if (m + 1 < G) round(m + 1, b1, b0);
    }
    // flags[0] bit 1: the W^T operand came from this kernel (bit 0: a wait was abandoned)
    if (RQ && blockIdx.x == 0 && tid == 0) atomicOr(a.flags, 2u);
}

size_t nvfp4_weight_1pass_ws_bytes() { return (size_t)4 * W1P_MAX_WG * 4 + 256; }

// RQ tile of an R x C matrix for at most ncu workgroups: TH a multiple of 64 dividing R (at most
// W1R_TH_MAX), TW a multiple of 16 dividing C, TH * TW <= the blocks a workgroup holds; the most
// tiles, then the widest. False if none exists, or if the tile gives the requant fewer than six
// wavefronts of thread pairs (TH * TW < W1R_TILE_MIN): the two steps are then faster (the 32-expert
// layer's 1536 x 4096 and 4096 x 1536 matrices, tiles of 24576 values, measured 0.61 + 0.34 ms
// fused against 0.49 ms of one-read quantization plus the backward's cheaper requants).
static bool w1r_tile(int64_t R, int64_t C, int ncu, int& TH, int& TW)
{
    int64_t best = 0;
    for (int64_t th = 64; th <= W1R_TH_MAX && th <= R; th += 64) {
        if (R % th != 0) continue;
        for (int64_t tw = 16; tw <= C; tw += 16) {
            if (C % tw != 0 || th * tw > (int64_t)W1P_NBT * W1P_THREADS * 16) continue;
            const int64_t tiles = (R / th) * (C / tw);
            if (tiles > ncu || tiles < best || (tiles == best && tw <= TW)) continue;
            best = tiles;
            TH = (int)th;
            TW = (int)tw;
        }
    }
    return best > 0 && (int64_t)TH * TW >= W1R_TILE_MIN;
}

// The one-read path, if the device and the shape allow it; hipErrorNotSupported otherwise (the
// caller then takes the two passes). wt != nullptr: also the backward's W^T operand (RQ), which
// needs rows_per_outer % 64 == 0 and a tile (w1r_tile).
static hipError_t launch_nvfp4_weight_1pass(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_outer,
                                            uint8_t* codes, uint8_t* scales, float* outer_out, void* ws,
                                            size_t ws_bytes, hipStream_t stream, uint8_t* wt = nullptr,
                                            uint8_t* wte = nullptr, uint64_t seed = 0, uint32_t stream_id = 0)
{
    if (ws == nullptr || ws_bytes < nvfp4_weight_1pass_ws_bytes()) return hipErrorNotSupported;
    // a captured graph would replay the launch without the co-residency a cooperative launch
    // guarantees, so a capturing stream takes the two reads
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
        return hipErrorNotSupported;
    const bool rq = wt != nullptr;
    const void* kern = rq ? (const void*)k_nvfp4_weight_1pass<true> : (const void*)k_nvfp4_weight_1pass<false>;
    int dev = 0, ncu = 0, coop = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, W1P_THREADS, 0) != hipSuccess)
        return hipErrorNotSupported;
    if (!coop || per_cu < 1 || ncu < 1 || ncu > W1P_MAX_WG) return hipErrorNotSupported;
    W1PArgs a{};
    a.x = x;
    a.G = rows / rows_per_outer;
    a.group_blocks = rows_per_outer * (cols / 16);
    a.outer_out = outer_out;
    a.codes = codes;
    a.scales = scales;
    a.words = static_cast<uint32_t*>(ws);
    a.flags = a.words + 4 * W1P_MAX_WG;
    int nwg = ncu;
    if (a.G > W1P_MAX_G) return hipErrorNotSupported;
    if (rq) {
        if (rows_per_outer % 64 != 0 || !w1r_tile(rows_per_outer, cols, ncu, a.TH, a.TW)) return hipErrorNotSupported;
        a.R = rows_per_outer;
        a.C = cols;
        a.wt = wt;
        a.wte = wte;
        a.seed = seed;
        a.stream_id = stream_id;
        nwg = (int)((a.R / a.TH) * (a.C / a.TW));
    } else if (a.group_blocks > (int64_t)W1P_NBT * ncu * W1P_THREADS) {
        return hipErrorNotSupported;
    }
    const int64_t nfill = (int64_t)(nvfp4_weight_1pass_ws_bytes() / 4);
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((nfill + 255) / 256)), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ws), nfill, 0u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    void* args[] = {(void*)&a};
    e = hipLaunchCooperativeKernel(kern, dim3((unsigned)nwg), dim3(W1P_THREADS), args, 0, stream);
    if (e != hipSuccess) {
        // a runtime that refuses the cooperative launch: the two reads instead
        (void)hipGetLastError();
        return hipErrorNotSupported;
    }
    return hipSuccess;
}

hipError_t launch_nvfp4_quantize_weights_bwd(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_outer,
                                             uint8_t* codes, uint8_t* scales, float* outer_out, uint8_t* wt,
                                             uint8_t* wte, uint64_t seed, uint32_t stream_id, void* ws,
                                             size_t ws_bytes, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    hipError_t e = launch_nvfp4_weight_1pass(x, rows, cols, rows_per_outer, codes, scales, outer_out, ws, ws_bytes,
                                             stream, wt, wte, seed, stream_id);
    if (e != hipErrorNotSupported) return e;
    e = launch_nvfp4_quantize(x, rows, cols, false, rows_per_outer, nullptr, codes, scales, outer_out, stream, false,
                              ws, ws_bytes);
    if (e != hipSuccess) return e;
    return launch_requant(codes, scales, outer_out, cols, rows_per_outer, nullptr, rows, nullptr, 0, PMN_TARGET_E4M3,
                          seed, stream_id, wt, wte, rows, true, nullptr, stream, true);
}

hipError_t launch_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, bool four_six,
                                 int64_t rows_per_outer, const float* outer_in, uint8_t* codes,
                                 uint8_t* scales, float* outer_out, hipStream_t stream, bool square,
                                 void* ws, size_t ws_bytes)
{
    if (rows == 0) return hipSuccess;
    if (!four_six && !square && outer_in == nullptr && ws != nullptr) {
        const hipError_t e = launch_nvfp4_weight_1pass(x, rows, cols, rows_per_outer, codes, scales, outer_out, ws,
                                                       ws_bytes, stream);
        if (e != hipErrorNotSupported) return e;
    }
    const int64_t nb = cols / 16;
    const int64_t ngroups = rows / rows_per_outer;
    if (!square && outer_in == nullptr && rows_per_outer == 1 && nb > 128 && nb <= 512) {
        if (four_six)
            hipLaunchKernelGGL((k_nvfp4_row_split<2, true>), dim3((unsigned)rows), dim3(256), 0, stream, x, rows, cols,
                               codes, scales, outer_out);
        else
            hipLaunchKernelGGL((k_nvfp4_row_split<2, false>), dim3((unsigned)rows), dim3(256), 0, stream, x, rows, cols,
                               codes, scales, outer_out);
        return hipGetLastError();
    }
    if (!square && outer_in == nullptr && rows_per_outer == 1 && nb <= 64 * 8) {
        const int64_t grid = (rows + 3) / 4;
        int nbl = nb <= 64 ? 1 : (nb <= 128 ? 2 : (nb <= 256 ? 4 : 8));
#define PMN_ROWS(N)                                                                                       \
    if (four_six) hipLaunchKernelGGL((k_nvfp4_rows<N, true>), dim3(grid), dim3(256), 0, stream, x, rows, cols, codes, scales, outer_out); \
    else hipLaunchKernelGGL((k_nvfp4_rows<N, false>), dim3(grid), dim3(256), 0, stream, x, rows, cols, codes, scales, outer_out);
        switch (nbl) {
        case 1: PMN_ROWS(1) break;
        case 2: PMN_ROWS(2) break;
        case 4: PMN_ROWS(4) break;
        default: PMN_ROWS(8) break;
        }
#undef PMN_ROWS
        return hipGetLastError();
    }
    if (outer_in != nullptr) {
        hipLaunchKernelGGL(k_copy_f32, dim3((ngroups + 255) / 256), dim3(256), 0, stream, outer_in, outer_out, ngroups);
    } else {
        uint32_t* amax = reinterpret_cast<uint32_t*>(outer_out);
        hipLaunchKernelGGL(k_fill_u32, dim3((ngroups + 255) / 256), dim3(256), 0, stream, amax, ngroups, 0u);
        const int64_t group_elems = rows_per_outer * cols;
        const int64_t per_block = 256 * AMAX_CHUNKS_PER_THREAD;
        int64_t gx = (group_elems / 8 + per_block - 1) / per_block;
        gx = gx > AMAX_BLOCKS ? AMAX_BLOCKS : gx;
        hipLaunchKernelGGL(k_group_amax, dim3((unsigned)gx, (unsigned)ngroups), dim3(256), 0, stream, x, group_elems, amax);
        hipLaunchKernelGGL(k_outer_from_amax, dim3((ngroups + 255) / 256), dim3(256), 0, stream, outer_out, ngroups);
    }
    if (square) {
        const int64_t waves = (rows / 16) * ((nb + 3) / 4);
        hipLaunchKernelGGL(k_nvfp4_2d, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, x, rows, cols,
                           rows_per_outer, outer_out, codes, scales);
        return hipGetLastError();
    }
    const int64_t nblocks = rows * nb;
    const int64_t grid = (nblocks + 255) / 256;
    if (four_six)
        hipLaunchKernelGGL((k_nvfp4_given<true>), dim3(grid), dim3(256), 0, stream, x, rows, cols, rows_per_outer, outer_out, codes, scales);
    else
        hipLaunchKernelGGL((k_nvfp4_given<false>), dim3(grid), dim3(256), 0, stream, x, rows, cols, rows_per_outer, outer_out, codes, scales);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// MXFP8 row-wise quantization  [AREX] "只把专家层的前向传播降到 4-bit" (gradients go through
// MXFP8 matmuls) and "配方的代价:预训练约 2% 的计算效率" (the last layers' forward stays in
// MXFP8). One thread per block of 32: e from the block amax, y = x * 2^-e, E4M3 by
// round-to-nearest-even or by stochastic rounding. Row r reads source row gather[r] (or r).
// E8M0 layouts: row-major [M x N/32] (ld_e8m0 == 0); k-block-major [N/32 x ld_e8m0] with
// column r (pad_off == nullptr, ld_e8m0 > 0); or k-block-major at the padded slot column
// pad_off[g] + r - offsets[g] of r's group g.
// ------------------------------------------------------------------------------------------

// The same block to E2M1 (the FP4 backward): E8M0 by the smallest scale with amax <= 6 * 2^e,
// codes packed two per byte (element 2j in the low nibble) into 4 words, RNE or SR.
template <bool SR>
PMN_DEV int mxfp4_block(const uint32_t (&w)[16], int64_t r, int64_t kb, int64_t N, uint64_t seed,
                        uint32_t stream_id, uint32_t (&o)[4])
{
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; j++) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
    const int e = e8m0_exponent<E8M0_E2M1>(amax);
    const uint64_t idx0 = (uint64_t)r * (uint64_t)N + (uint64_t)(kb * 32);   // multiple of 8
#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint32_t rw[4] = {0u, 0u, 0u, 0u};
        if (SR) rand16x8(seed, stream_id, (idx0 >> 3) + q, rw);
        uint32_t word = 0u;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t src = w[4 * q + j / 2];
            const float y = __builtin_ldexpf((j & 1) ? bf16_hi(src) : bf16_lo(src), -e);
            const uint32_t c = SR ? fp4_sr(y, (j & 1) ? (rw[j >> 1] >> 16) : (rw[j >> 1] & 0xFFFFu))
                                  : ((uint32_t)PMN_CVT_FP4(0u, y, 0.0f, 0) & 0xFu);
            word |= c << (4 * j);
        }
        o[q] = word;
    }
    return e;
}

PMN_DEV void load_block32(const uint16_t* x, int64_t word16, uint32_t (&w)[16])
{
    const uint4* p = reinterpret_cast<const uint4*>(x) + 4 * word16;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint4 v = p[q];
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
    }
}

PMN_DEV void store_block32(uint8_t* out, int64_t block, const uint32_t (&o)[8])
{
    uint4* po = reinterpret_cast<uint4*>(out) + 2 * block;
    po[0] = make_uint4(o[0], o[1], o[2], o[3]);
    po[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// Row-major E8M0 [M x N/32]: one thread per block, in row order.
template <bool SR>
__global__ __launch_bounds__(256) void k_mxfp8_rows(const uint16_t* __restrict__ x, int64_t M,
                                                    int64_t N, uint64_t seed, uint32_t stream_id,
                                                    uint8_t* __restrict__ out,
                                                    uint8_t* __restrict__ out_e8m0,
                                                    const int32_t* __restrict__ gather)
{
    const int64_t nb = N >> 5;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * nb) return;
    const int64_t r = i / nb, kb = i - r * nb;
    uint32_t w[16], o[8];
    load_block32(x, (gather ? (int64_t)gather[r] : r) * nb + kb, w);
    const int e = mxfp8_block<SR>(w, r, kb, N, seed, stream_id, o);
    out_e8m0[i] = (uint8_t)(e + 127);
    store_block32(out, i, o);
}

// k-block-major E8M0 [N/32 x ld_e8m0]: a workgroup takes 64 rows x 4 k-blocks (four threads
// read 256 contiguous bytes of a row), and the scale bytes go through LDS so that each k-block's
// 64 rows are written as one contiguous run. Column of row r: r (pad_off == nullptr), else
// pad_off[g] + r - offsets[g] for r's group g. FP4: E2M1 codes packed two per byte, [M x N/2].
// BLK: the codes go to that same padded position as a row of the blocked GEMM operand layout
// (1 KB blocks of 16 rows x 64 bytes, chunk c of row r at slot c ^ ((r / 4) % 4)).
template <bool SR, bool FP4 = false, bool BLK = false>
__global__ __launch_bounds__(256) void k_mxfp8_rows_kbm(const uint16_t* __restrict__ x, int64_t M,
                                                        int64_t N, uint64_t seed, uint32_t stream_id,
                                                        uint8_t* __restrict__ out,
                                                        uint8_t* __restrict__ out_e8m0,
                                                        const int64_t* __restrict__ offsets, int G,
                                                        const int64_t* __restrict__ pad_off, int64_t ld_e8m0,
                                                        const int32_t* __restrict__ gather)
{
    __shared__ uint8_t se[4][64];
    __shared__ int64_t pcol[64];
    const int64_t nb = N >> 5;
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * 64, kb0 = (int64_t)blockIdx.y * 4;
    // padded position of slot r: pad_off[g] + r - offsets[g] for its group g (the largest g with
    // offsets[g] <= r; empty groups are skipped)
    auto padded_col = [&](int64_t r) {
        if (pad_off == nullptr) return r;
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
        }
        return pad_off[lo] + (r - offsets[lo]);
    };
    const int64_t r = r0 + (t >> 2), kb = kb0 + (t & 3);
    const bool live = r < M && kb < nb;
    uint32_t w[16];
    if (live) load_block32(x, (gather ? (int64_t)gather[r] : r) * nb + kb, w);
    // the workgroup's 64 rows look their padded positions up once, while the loads are in flight
    if (t < 64) pcol[t] = r0 + t < M ? padded_col(r0 + t) : 0;
    __syncthreads();
    {
        if (live) {
            int e;
            if (FP4) {
                uint32_t o[4];
                e = mxfp4_block<SR>(w, r, kb, N, seed, stream_id, o);
                if (BLK) {
                    // k-block kb = chunk kb % 4 of 64-byte column kb / 4
                    // rows are whole 64-byte columns (N rounded up to 128 values); with N not a
                    // multiple of 128 the last column's chunks past N are not written (the GEMM
                    // gives those k-blocks the scale 2^-127 on both operands, and every E2M1 code
                    // is finite)
                    const int64_t pr = pcol[t >> 2];
                    const int r16 = (int)(pr & 15), x = (r16 >> 2) & 3, c = (int)(kb & 3);
                    *reinterpret_cast<uint4*>(out + ((pr >> 4) * ((N + 127) >> 7) + (kb >> 2)) * 1024 + r16 * 64 +
                                              ((c ^ x) << 4)) = make_uint4(o[0], o[1], o[2], o[3]);
                } else {
                    reinterpret_cast<uint4*>(out)[r * nb + kb] = make_uint4(o[0], o[1], o[2], o[3]);
                }
            } else {
                uint32_t o[8];
                e = mxfp8_block<SR>(w, r, kb, N, seed, stream_id, o);
                if (BLK) {
                    // k-block kb = chunks 2 (kb % 2) and 2 (kb % 2) + 1 of 64-byte column kb / 2; rows
                    // are whole columns (N rounded up to 64 bytes), and with an odd k-block count the
                    // last column's second half holds zero codes
                    const int64_t pr = pcol[t >> 2];
                    const int r16 = (int)(pr & 15), x = (r16 >> 2) & 3, c = 2 * (int)(kb & 1);
                    uint8_t* blk = out + ((pr >> 4) * ((N + 63) >> 6) + (kb >> 1)) * 1024 + r16 * 64;
                    *reinterpret_cast<uint4*>(blk + ((c ^ x) << 4)) = make_uint4(o[0], o[1], o[2], o[3]);
                    *reinterpret_cast<uint4*>(blk + (((c + 1) ^ x) << 4)) = make_uint4(o[4], o[5], o[6], o[7]);
                    if ((nb & 1) && kb == nb - 1) {
                        *reinterpret_cast<uint4*>(blk + (((c + 2) ^ x) << 4)) = make_uint4(0u, 0u, 0u, 0u);
                        *reinterpret_cast<uint4*>(blk + (((c + 3) ^ x) << 4)) = make_uint4(0u, 0u, 0u, 0u);
                    }
                } else {
                    store_block32(out, r * nb + kb, o);
                }
            }
            se[t & 3][t >> 2] = (uint8_t)(e + 127);
        }
    }
    __syncthreads();
    const int64_t re = r0 + (t & 63), kbe = kb0 + (t >> 6);
    if (re < M && kbe < nb) out_e8m0[kbe * ld_e8m0 + pcol[t & 63]] = se[t >> 6][t & 63];
}

hipError_t launch_mxfp8_rows(const uint16_t* x, int64_t M, int64_t N, bool sr, uint64_t seed,
                             uint32_t stream_id, uint8_t* out, uint8_t* out_e8m0,
                             const int64_t* offsets, int G, const int64_t* padded_offsets,
                             int64_t ld_e8m0, hipStream_t stream, const int32_t* gather, bool fp4,
                             bool blocked)
{
    const int64_t nb = N / 32;
    if (M * nb == 0) return hipSuccess;
    if ((fp4 || blocked) && padded_offsets == nullptr && ld_e8m0 == 0) return hipErrorInvalidValue;   // k-block-major only
    if (padded_offsets == nullptr && ld_e8m0 == 0) {
        const int64_t grid = (M * nb + 255) / 256;
        if (sr)
            hipLaunchKernelGGL((k_mxfp8_rows<true>), dim3(grid), dim3(256), 0, stream, x, M, N, seed, stream_id, out,
                               out_e8m0, gather);
        else
            hipLaunchKernelGGL((k_mxfp8_rows<false>), dim3(grid), dim3(256), 0, stream, x, M, N, seed, stream_id, out,
                               out_e8m0, gather);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((M + 63) / 64), (unsigned)((nb + 3) / 4));
    if (fp4 && blocked) {
        if (sr)
            hipLaunchKernelGGL((k_mxfp8_rows_kbm<true, true, true>), grid, dim3(256), 0, stream, x, M, N, seed,
                               stream_id, out, out_e8m0, offsets, G, padded_offsets, ld_e8m0, gather);
        else
            hipLaunchKernelGGL((k_mxfp8_rows_kbm<false, true, true>), grid, dim3(256), 0, stream, x, M, N, seed,
                               stream_id, out, out_e8m0, offsets, G, padded_offsets, ld_e8m0, gather);
        return hipGetLastError();
    }
    if (fp4) {
        if (sr)
            hipLaunchKernelGGL((k_mxfp8_rows_kbm<true, true>), grid, dim3(256), 0, stream, x, M, N, seed, stream_id,
                               out, out_e8m0, offsets, G, padded_offsets, ld_e8m0, gather);
        else
            hipLaunchKernelGGL((k_mxfp8_rows_kbm<false, true>), grid, dim3(256), 0, stream, x, M, N, seed, stream_id,
                               out, out_e8m0, offsets, G, padded_offsets, ld_e8m0, gather);
        return hipGetLastError();
    }
    if (blocked) {
        if (sr)
            hipLaunchKernelGGL((k_mxfp8_rows_kbm<true, false, true>), grid, dim3(256), 0, stream, x, M, N, seed,
                               stream_id, out, out_e8m0, offsets, G, padded_offsets, ld_e8m0, gather);
        else
            hipLaunchKernelGGL((k_mxfp8_rows_kbm<false, false, true>), grid, dim3(256), 0, stream, x, M, N, seed,
                               stream_id, out, out_e8m0, offsets, G, padded_offsets, ld_e8m0, gather);
        return hipGetLastError();
    }
    if (sr)
        hipLaunchKernelGGL((k_mxfp8_rows_kbm<true>), grid, dim3(256), 0, stream, x, M, N, seed, stream_id, out,
                           out_e8m0, offsets, G, padded_offsets, ld_e8m0, gather);
    else
        hipLaunchKernelGGL((k_mxfp8_rows_kbm<false>), grid, dim3(256), 0, stream, x, M, N, seed, stream_id, out,
                           out_e8m0, offsets, G, padded_offsets, ld_e8m0, gather);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// RHT32 + S2F6  [AREX] "计算提速后,NVLink 通信成了新瓶颈": a 32-point randomized Hadamard
// transform (orthogonal, exactly invertible) spreads outliers, then S2F6 codes (2-bit signed
// integer part, 6-bit fraction: -128/64 .. 127/64) with one scale per 32 values.
// One thread per 32-chunk: the whole butterfly network runs in registers.
// ------------------------------------------------------------------------------------------

PMN_DEV void rht32_s2f6_chunk(float (&t)[32], uint32_t mask, uint32_t (&o)[8], uint32_t& e8m0)
{
#pragma unroll
    for (int j = 0; j < 32; j++) t[j] = __uint_as_float(__float_as_uint(t[j]) ^ (((mask >> j) & 1u) << 31));
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 32; i++) {
            if ((i & h) == 0) {
                float a = t[i], b = t[i + h];
                t[i] = a + b;
                t[i + h] = a - b;
            }
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(t[j]));
    const int e = e8m0_exponent<E8M0_S2F6>(amax);
    e8m0 = (uint32_t)(e + 127);
#pragma unroll
    for (int q = 0; q < 8; q++) {
        uint32_t w = 0u;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            int c = (int)__builtin_rintf(__builtin_ldexpf(t[4 * q + j], 6 - e));
            w |= ((uint32_t)c & 0xFFu) << (8 * j);
        }
        o[q] = w;
    }
}

template <bool F32>
__global__ __launch_bounds__(256) void k_rht32_s2f6(const void* __restrict__ x, int64_t rows,
                                                    int64_t cols, uint32_t mask,
                                                    int8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ e8m0)
{
    const int64_t n = rows * (cols >> 5);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float t[32];
    if (F32) {
        const float4* p = reinterpret_cast<const float4*>(x) + 8 * i;
#pragma unroll
        for (int q = 0; q < 8; q++) {
            float4 v = p[q];
            t[4 * q] = v.x; t[4 * q + 1] = v.y; t[4 * q + 2] = v.z; t[4 * q + 3] = v.w;
        }
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(x) + 4 * i;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            uint4 v = p[q];
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                t[8 * q + 2 * j] = bf16_lo(w[j]);
                t[8 * q + 2 * j + 1] = bf16_hi(w[j]);
            }
        }
    }
    uint32_t o[8], e;
    rht32_s2f6_chunk(t, mask, o, e);
    uint4* po = reinterpret_cast<uint4*>(codes) + 2 * i;
    po[0] = make_uint4(o[0], o[1], o[2], o[3]);
    po[1] = make_uint4(o[4], o[5], o[6], o[7]);
    e8m0[i] = (uint8_t)e;
}

hipError_t launch_rht32_s2f6(const void* x, bool f32, int64_t rows, int64_t cols, uint32_t mask,
                             int8_t* codes, uint8_t* e8m0, hipStream_t stream)
{
    const int64_t n = rows * (cols / 32);
    if (n == 0) return hipSuccess;
    const int64_t grid = (n + 255) / 256;
    if (f32)
        hipLaunchKernelGGL((k_rht32_s2f6<true>), dim3(grid), dim3(256), 0, stream, x, rows, cols, mask, codes, e8m0);
    else
        hipLaunchKernelGGL((k_rht32_s2f6<false>), dim3(grid), dim3(256), 0, stream, x, rows, cols, mask, codes, e8m0);
    return hipGetLastError();
}

}  // namespace pmn
