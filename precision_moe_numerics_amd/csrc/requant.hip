// requant.hip -- backward operand preparation: dequantize the saved NVFP4 tensor, transpose it
// and re-quantize it to MXFP8 with stochastic rounding; and the column-wise (transposed,
// grouped) MXFP8 quantization of bf16 gradients, which shares the same output layout.
//
// Pages cited (by title and section heading):
//   [AREX] AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向传播
//          贯穿预训练到最后一次 RL rollout", section "转置打散分组,随机舍入保住期望值": the backward
//          needs the forward tensors transposed; blocks then run the other way, so the saved
//          tensor is dequantized to high precision, transposed and re-quantized with stochastic
//          rounding, keeping the expectation equal to the forward value; MXFP8 is the chosen
//          re-quantization precision.
//
// Work split. A wavefront owns one 32-slot block of the padded output (one E8M0 scale per
// output row) and 64 groups of 8 consecutive source columns; each lane owns 8 columns. The 8
// columns of a lane are 8 consecutive element indices of one source row, which is exactly one
// Philox4x32-10 call (16 random bits per element), so every random bit is drawn once. Pass 1
// reduces the per-column amax over the 32 slots with the codes kept in registers; pass 2
// converts and writes 16 bytes per column every 16 slots.
#include "pmn_dev.hpp"
#include "pmn_kernels.hpp"

namespace pmn {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct GroupBlock {
    int64_t s0;   // first slot of the block
    int valid;    // slots of the block that exist (the rest is zero padding)
    bool live;    // the block lies inside the padded output
};

// Map padded block pb (32 output columns) to its slots: walk the groups, each padded to a
// multiple of `unit` (32, or 64 / 128 for the blocked GEMM operands, whose last blocks of a group
// can then be all padding: valid = 0).
PMN_DEV GroupBlock find_block(int64_t pb, const int64_t* offsets, int G, int64_t M, int64_t unit)
{
    GroupBlock r;
    const int64_t col = pb * 32;
    if (offsets == nullptr) {
        r.s0 = col;
        r.live = col < M;
        int64_t v = M - col;
        r.valid = (int)(v > 32 ? 32 : (v < 0 ? 0 : v));
        return r;
    }
    int64_t po = 0;
    for (int g = 0; g < G; g++) {
        int64_t a = offsets[g], b = offsets[g + 1];
        int64_t P = (b - a + unit - 1) & ~(unit - 1);
        if (col < po + P) {
            r.s0 = a + (col - po);
            int64_t v = (b < M ? b : M) - r.s0;     // never past the last slot
            v = v < 0 ? 0 : v;
            r.valid = (int)(v > 32 ? 32 : v);
            r.live = true;
            return r;
        }
        po += P;
    }
    r.s0 = 0;
    r.valid = 0;
    r.live = false;
    return r;
}

// po[0] = 0, po[g + 1] = sum over h <= g of the group sizes rounded up to `unit`: one wavefront,
// an inclusive prefix sum over 64 groups at a time
__global__ void k_padded_offsets(const int64_t* offsets, int G, int64_t M, int64_t* po, int64_t unit)
{
    const int lane = threadIdx.x;
    if (blockIdx.x != 0 || lane >= 64) return;
    if (offsets == nullptr) {
        if (lane == 0) {
            po[0] = 0;
            po[1] = (M + unit - 1) & ~(unit - 1);
        }
        return;
    }
    if (lane == 0) po[0] = 0;
    int64_t base = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + lane;
        const int64_t P = g < G ? (offsets[g + 1] - offsets[g] + unit - 1) & ~(unit - 1) : 0;
        int64_t cum = P;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t y = __shfl_up(cum, d, 64);
            if (lane >= d) cum += y;
        }
        if (g < G) po[g + 1] = base + cum;
        base += __shfl(cum, 63, 64);
    }
}

__global__ void k_iota_offsets(int64_t* o, int G, int64_t step)
{
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g <= G) o[g] = (int64_t)g * step;
}

hipError_t launch_iota_offsets(int64_t* o, int G, int64_t step, hipStream_t stream)
{
    hipLaunchKernelGGL(k_iota_offsets, dim3((unsigned)((G + 1 + 255) / 256)), dim3(256), 0, stream, o, G, step);
    return hipGetLastError();
}

enum { SRC_NVFP4 = 0, SRC_BF16 = 1 };

struct TransposeArgs {
    // source
    const uint8_t* codes;     // NVFP4 codes [src_rows x cols/2]    (SRC_NVFP4)
    const uint8_t* scales;    // E4M3 [src_rows x cols/16]
    const float* outer;       // [src_rows / rows_per_outer]
    int64_t rows_per_outer;
    const uint16_t* x;        // bf16 [M x cols]                    (SRC_BF16)
    int64_t cols;
    const int32_t* gather;    // slot -> source row (nullable)
    int64_t M;
    const int64_t* offsets;   // [G+1] (nullable)
    int G;
    uint64_t seed;
    uint32_t stream_id;
    uint8_t* out;             // [cols x ld]
    uint8_t* out_e8m0;        // [cols x ld/32], or k-block-major [ld/32 x cols] when e8m0_kb_major
    int64_t ld;
    bool e8m0_kb_major;
    // codes in 1 KB blocks of 16 rows x 64 bytes (the GEMM operand layout) and groups padded to
    // `unit` slots (64 for E4M3, 128 for packed E2M1: one 64-byte block column) instead of 32
    bool blocked;
    int64_t unit;
};

// E4M3 codes of a / scale and b / scale (scale a power of two), round to nearest even, written
// into the low (hi = false) or high 16 bits of `word`.
PMN_DEV uint32_t e4m3_rne_pair_scaled_into(uint32_t word, float a, float b, float scale, bool hi)
{
    typedef short v2i16 __attribute__((ext_vector_type(2)));
    const v2i16 old = __builtin_bit_cast(v2i16, word);
    const v2i16 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, scale, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, scale, false);
    return __builtin_bit_cast(uint32_t, r);
}

// p, a wavefront-uniform pointer, pinned to scalar registers: a load from p + (32-bit lane offset)
// then takes the scalar-base addressing form and needs no per-lane 64-bit address arithmetic.
typedef const __attribute__((address_space(1))) uint8_t gbyte;   // global memory
PMN_DEV gbyte* uniform_ptr(const uint8_t* p)
{
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return reinterpret_cast<gbyte*>(((uint64_t)hi << 32) | lo);
}

PMN_DEV void bf8(uint4 w, float (&v)[8])
{
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// Output tile of a workgroup: 512 output rows (source columns) x 128 padded slots (4 blocks),
// assembled in LDS so that global stores write whole 128-byte row segments (or whole 1 KB
// blocks). Rows are 128 bytes (8 chunks of 16); chunk p of row r sits at position
// p ^ ((r / 8) % 8) ^ (4 ((r / 2) % 2)), so the transposed writes (lane l -> rows 8l .. 8l+7), the
// row-wise reads (2 rows x 8 chunks per quarter-wavefront) and the block reads (4 rows x 4
// chunks) all spread over the LDS banks.
constexpr int TQ_ROWS = 512;
constexpr int TQ_RS = 128;

PMN_DEV int tile_chunk(int row, int chunk)
{
    return row * TQ_RS + ((chunk ^ ((row >> 3) & 7) ^ (((row >> 1) & 1) << 2)) << 4);
}

// SRC: SRC_NVFP4 or SRC_BF16. ROUND: 0 = RNE, 1 = SR. TARGET: 0 = E4M3, 1 = E2M1 (one code per
// byte, SR only), 2 = E2M1 packed two per byte (slot 2j in the low nibble): out [cols x ld/2].
template <int SRC, int ROUND, int TARGET>
__global__ __launch_bounds__(256, 2) void k_transpose_quant(TransposeArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[TQ_ROWS * TQ_RS];
    __shared__ uint8_t tile_e[TQ_ROWS * 4];
    __shared__ int block_live[4];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wavefront-uniform
    const int64_t pb = (int64_t)blockIdx.x * 4 + w;
    const int64_t cg = (int64_t)blockIdx.y * 64 + lane;   // column group of 8
    const int64_t c0 = cg * 8;
    const GroupBlock blk = find_block(pb, a.offsets, a.G, a.M, a.unit);
    if (lane == 0) block_live[w] = blk.live ? 1 : 0;
    const bool active = blk.live && c0 < a.cols;
    // lane j (mod 32) fetches slot j's source row and outer scale with one vector load each;
    // readlane later hands every slot's values to the whole wavefront, so every lane of a live
    // block computes them, whatever its columns
    // a block that is all padding (valid = 0) re-reads slot 0; all its values become +0
    const int last = blk.valid - 1;
    const int64_t rs0 = blk.valid > 0 ? blk.s0 : 0;
    const int lastc = blk.valid > 0 ? last : 0;
    int rl = 0;
    float ol = 0.0f;
    if (SRC == SRC_NVFP4 && blk.live) {
        const int jl = lane & 31;
        const int64_t sl = rs0 + (jl < lastc ? jl : lastc);
        rl = a.gather ? a.gather[sl] : (int)sl;
        // rl is a 32-bit row index, so a 32-bit division serves whenever the divisor fits
        ol = a.outer[a.rows_per_outer <= 0x7FFFFFFF ? (int64_t)((uint32_t)rl / (uint32_t)a.rows_per_outer)
                                                    : (int64_t)rl / a.rows_per_outer];
    }

    if (active) {
        // ---- pass 1: every load of the 32 slots is issued before any is used (slots past the
        // group's end re-read its last slot and get a zero scale), then per-column amax
        uint32_t cw[32];      // NVFP4: code words
        float dsc[32];        // NVFP4: effective block scale per slot
        uint4 xw[32];         // BF16: raw values
        if (SRC == SRC_NVFP4) {
            uint32_t sbyte[32];
            float so[32];
            // row bases are wavefront-uniform (scalar registers); each lane adds a 32-bit offset.
            // The loads are nontemporal: the source is read once (measured 4% faster than cached
            // loads on the 8192 x 7168 workload and on the layer's X^T)
            const uint32_t coff = (uint32_t)(c0 >> 1), soff = (uint32_t)(c0 >> 4);
#pragma unroll
            for (int j = 0; j < 32; j++) {
                const int64_t r = __builtin_amdgcn_readlane(rl, j);
                so[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ol), j));
                gbyte* crow = uniform_ptr(a.codes + r * (a.cols >> 1));
                gbyte* srow = uniform_ptr(a.scales + r * (a.cols >> 4));
                cw[j] = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(crow + coff));
                sbyte[j] = __builtin_nontemporal_load(srow + soff);
            }
            // slots past the group's end become +0 (code word 0, scale 0), so they need no branch:
            // a wavefront-uniform mask clears both
#pragma unroll
            for (int j = 0; j < 32; j++) {
                const uint32_t keep = j <= last ? 0xFFFFFFFFu : 0u;
                dsc[j] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, e4m3_value(sbyte[j]) * so[j]) & keep);
                cw[j] &= keep;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 32; j++) {
                const uint4 v = *reinterpret_cast<const uint4*>(a.x + (rs0 + (j < lastc ? j : lastc)) * a.cols + c0);
                xw[j] = j <= last ? v : make_uint4(0u, 0u, 0u, 0u);
            }
        }
        float amax[8];
#pragma unroll
        for (int c = 0; c < 8; c++) amax[c] = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; j += 2) {
            float v0[8], v1[8];
            if (SRC == SRC_NVFP4) {
                deq8(cw[j], dsc[j], v0);
                deq8(cw[j + 1], dsc[j + 1], v1);
            } else {
                bf8(xw[j], v0);
                bf8(xw[j + 1], v1);
            }
            // one running maximum per column, two slots per step (one three-input max)
#pragma unroll
            for (int c = 0; c < 8; c++) amax[c] = fmaxf(fmaxf(amax[c], fabsf(v0[c])), fabsf(v1[c]));
        }
        int e[8];
        float escale[8];   // 2^e: the scaled converter divides by it exactly
#pragma unroll
        for (int c = 0; c < 8; c++) {
            e[c] = TARGET == 0 ? e8m0_exponent<E8M0_E4M3>(amax[c]) : e8m0_exponent<E8M0_E2M1>(amax[c]);
            escale[c] = __builtin_ldexpf(1.0f, e[c]);
            tile_e[(lane * 8 + c) * 4 + w] = (uint8_t)(e[c] + 127);
        }

        // ---- pass 2: convert 16 slots at a time (4 words per column) into the LDS tile
        // Philox counter of slot s0 + j: (s * cols + c0) / 8 = ctr0 + j * cols / 8 (cols and c0 are
        // multiples of 8), so consecutive slots add a wavefront-uniform step
        const uint64_t ctr0 = ((uint64_t)blk.s0 * (uint64_t)a.cols + (uint64_t)c0) >> 3;
        const uint64_t cstep = (uint64_t)a.cols >> 3;
#pragma unroll
        for (int half = 0; half < 2; half++) {
            uint32_t o[8][4];
#pragma unroll
            for (int c = 0; c < 8; c++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    // the E4M3 target writes all four bytes of every word below, so the words need
                    // no initial value; the packed E2M1 targets OR nibbles into zero
                    if (TARGET == 0) o[c][q] = __builtin_nondeterministic_value(o[c][q]);
                    else o[c][q] = 0u;
                }
            if (TARGET == 0) {
                // E4M3 target: every slot runs (padding slots are +0 and convert to 0 whatever the
                // random bits). The scaled converters compute the conversion of v / 2^e exactly and
                // write their bytes straight into the packed word: SR one value at a time, RNE two
                // slots of a column at a time.
#pragma unroll
                for (int jj = 0; jj < 16; jj += 2) {
                    float v[2][8];
#pragma unroll
                    for (int u = 0; u < 2; u++) {
                        const int j = half * 16 + jj + u;
                        // recompute the values instead of keeping the amax pass's 256 values alive
                        // (the empty asm hides that they are equal)
                        if (SRC == SRC_NVFP4) {
                            uint32_t cwj = cw[j];
                            asm volatile("" : "+v"(cwj));
                            deq8(cwj, dsc[j], v[u]);
                        } else {
                            uint4 xj = xw[j];
                            asm volatile("" : "+v"(xj.x), "+v"(xj.y), "+v"(xj.z), "+v"(xj.w));
                            bf8(xj, v[u]);
                        }
                    }
                    if (ROUND == 1) {
#pragma unroll
                        for (int u = 0; u < 2; u++) {
                            uint32_t rw[4];
                            rand16x8(a.seed, a.stream_id, add_uniform64(ctr0, (uint64_t)(half * 16 + jj + u) * cstep), rw);
#pragma unroll
                            for (int c = 0; c < 8; c++)
                                o[c][jj >> 2] = e4m3_sr_scaled_into(o[c][jj >> 2], v[u][c], sr_operand(rw[c >> 1], c & 1),
                                                                    escale[c], (jj + u) & 3);
                        }
                    } else {
#pragma unroll
                        for (int c = 0; c < 8; c++) o[c][jj >> 2] = e4m3_rne_pair_scaled_into(o[c][jj >> 2], v[0][c], v[1][c], escale[c], (jj & 2) != 0);
                    }
                }
            } else {
                // E2M1 target (the pages' worked example and the FP4 backward): SR (or RNE, packed
                // target only) onto the FP4 grid
#pragma unroll
                for (int jj = 0; jj < 16; jj++) {
                    const int j = half * 16 + jj;
                    if (j < blk.valid) {
                        float v[8];
                        if (SRC == SRC_NVFP4) {
                            uint32_t cwj = cw[j];
                            asm volatile("" : "+v"(cwj));   // recompute rather than keep the amax pass's values
                            deq8(cwj, dsc[j], v);
                        } else {
                            uint4 xj = xw[j];
                            asm volatile("" : "+v"(xj.x), "+v"(xj.y), "+v"(xj.z), "+v"(xj.w));
                            bf8(xj, v);
                        }
                        uint32_t rw[4] = {0u, 0u, 0u, 0u};
                        if (ROUND == 1)
                            rand16x8(a.seed, a.stream_id, add_uniform64(ctr0, (uint64_t)j * cstep), rw);
#pragma unroll
                        for (int c = 0; c < 8; c++) {
                            const float y = __builtin_ldexpf(v[c], -e[c]);
                            const uint32_t word = rw[c >> 1];
                            const uint32_t code = (TARGET == 2 && ROUND == 0)
                                                      ? ((uint32_t)PMN_CVT_FP4(0u, y, 0.0f, 0) & 0xFu)
                                                      : fp4_sr(y, (c & 1) ? (word >> 16) : (word & 0xFFFFu));
                            if (TARGET == 1) o[c][jj >> 2] |= code << (8 * (jj & 3));
                            else o[c][jj >> 3] |= code << (4 * (jj & 7));
                        }
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < 8; c++) {
                const int row = lane * 8 + c;
                if (TARGET == 2)   // 16 slots = 8 bytes: half h of chunk w
                    *reinterpret_cast<uint2*>(tile + tile_chunk(row, w) + 8 * half) = make_uint2(o[c][0], o[c][1]);
                else
                    *reinterpret_cast<uint4*>(tile + tile_chunk(row, w * 2 + half)) =
                        make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]);
            }
        }
    }
    __syncthreads();

    // ---- store: 512 rows x 8 chunks of 16 bytes; a chunk is written if its column exists and its
    // 32-slot block lies inside the padded output.
    const int64_t col_base = (int64_t)blockIdx.y * 512;
    if (TARGET == 2 && a.blocked) {
        // 1 KB blocks of 16 output rows x 64 bytes: this tile's 128 slots are one block column
        const int64_t nkb = a.ld >> 7;
#pragma unroll 4
        for (int k = 0; k < 8; k++) {
            const int q = k * 256 + threadIdx.x;
            const int b = q >> 6, t = q & 63;
            const int r16 = t >> 2;
            const int c = (t & 3) ^ ((r16 >> 2) & 3);
            const int row = b * 16 + r16;
            const int64_t col = col_base + row;
            if (col < a.cols && block_live[c]) {
                const uint4 v = *reinterpret_cast<const uint4*>(tile + tile_chunk(row, c));
                *reinterpret_cast<uint4*>(a.out + (((col_base >> 4) + b) * nkb + (int64_t)blockIdx.x) * 1024 + t * 16) = v;
            }
        }
    } else if (TARGET == 2) {
        // packed: 512 rows x 4 chunks of 16 bytes (one 32-slot block each)
#pragma unroll 4
        for (int k = 0; k < 8; k++) {
            const int q = k * 256 + threadIdx.x;
            const int row = q >> 2, chunk = q & 3;
            const int64_t col = col_base + row;
            if (col < a.cols && block_live[chunk]) {
                const uint4 v = *reinterpret_cast<const uint4*>(tile + tile_chunk(row, chunk));
                *reinterpret_cast<uint4*>(a.out + col * (a.ld >> 1) + (int64_t)blockIdx.x * 64 + chunk * 16) = v;
            }
        }
    } else if (a.blocked) {
        // 1 KB blocks of 16 output rows x 64 bytes (32 row blocks x 2 k-blocks of this tile), one
        // per 64 threads. Block (rb, kb) of the output sits at (rb * ld/64 + kb) * 1024 and holds
        // row r (0..15) at bytes 64 r .. 64 r + 63 with its 16-byte chunk c at slot c ^ ((r / 4) % 4):
        // exactly the LDS image the GEMM reads, so the GEMM copies whole blocks.
        const int64_t nkb = a.ld >> 6;
#pragma unroll 4
        for (int k = 0; k < 16; k++) {
            const int q = k * 256 + threadIdx.x;
            const int b = q >> 6, t = q & 63;
            const int rb = b >> 1, kb = b & 1;
            const int r16 = t >> 2;
            const int c = (t & 3) ^ ((r16 >> 2) & 3);
            const int row = rb * 16 + r16;
            const int64_t col = col_base + row;
            if (col < a.cols && block_live[kb * 2 + (c >> 1)]) {
                const uint4 v = *reinterpret_cast<const uint4*>(tile + tile_chunk(row, kb * 4 + c));
                *reinterpret_cast<uint4*>(a.out + (((col_base >> 4) + rb) * nkb + (int64_t)blockIdx.x * 2 + kb) * 1024 +
                                          t * 16) = v;
            }
        }
    } else {
#pragma unroll 4
        for (int k = 0; k < 16; k++) {
            const int q = k * 256 + threadIdx.x;
            const int row = q >> 3, chunk = q & 7;
            const int64_t col = col_base + row;
            if (col < a.cols && block_live[chunk >> 1]) {
                const uint4 v = *reinterpret_cast<const uint4*>(tile + tile_chunk(row, chunk));
                *reinterpret_cast<uint4*>(a.out + col * a.ld + (int64_t)blockIdx.x * 128 + chunk * 16) = v;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 2; k++) {
        const int row = k * 256 + threadIdx.x;
        const int64_t col = col_base + row;
        if (col < a.cols) {
#pragma unroll
            for (int b = 0; b < 4; b++)
                if (block_live[b]) {
                    const int64_t kb = (int64_t)blockIdx.x * 4 + b;
                    a.out_e8m0[a.e8m0_kb_major ? kb * a.cols + col : col * (a.ld >> 5) + kb] = tile_e[row * 4 + b];
                }
        }
    }
}

hipError_t launch_padded_offsets(const int64_t* offsets, int G, int64_t M, int64_t* padded_offsets,
                                 hipStream_t stream, int64_t unit)
{
    hipLaunchKernelGGL(k_padded_offsets, dim3(1), dim3(64), 0, stream, offsets, G, M, padded_offsets, unit);
    return hipGetLastError();
}

static hipError_t launch_transpose(const TransposeArgs& a, int src, int round, int target,
                                   int64_t* padded_offsets, hipStream_t stream)
{
    if (padded_offsets)
        hipLaunchKernelGGL(k_padded_offsets, dim3(1), dim3(64), 0, stream, a.offsets, a.G, a.M, padded_offsets,
                           a.unit);
    const int64_t nblk = a.ld / 32;
    if (nblk == 0 || a.cols == 0) return hipGetLastError();
    dim3 grid((unsigned)((nblk + 3) / 4), (unsigned)((a.cols / 8 + 63) / 64));
    if (src == SRC_NVFP4) {
        if (target == 0) {
            if (round == 1) hipLaunchKernelGGL((k_transpose_quant<SRC_NVFP4, 1, 0>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((k_transpose_quant<SRC_NVFP4, 0, 0>), grid, dim3(256), 0, stream, a);
        } else if (target == 1) {
            hipLaunchKernelGGL((k_transpose_quant<SRC_NVFP4, 1, 1>), grid, dim3(256), 0, stream, a);
        } else {
            hipLaunchKernelGGL((k_transpose_quant<SRC_NVFP4, 1, 2>), grid, dim3(256), 0, stream, a);
        }
    } else if (target == 2) {
        if (round == 1) hipLaunchKernelGGL((k_transpose_quant<SRC_BF16, 1, 2>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((k_transpose_quant<SRC_BF16, 0, 2>), grid, dim3(256), 0, stream, a);
    } else {
        if (round == 1) hipLaunchKernelGGL((k_transpose_quant<SRC_BF16, 1, 0>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((k_transpose_quant<SRC_BF16, 0, 0>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_requant(const uint8_t* codes, const uint8_t* scales, const float* outer,
                          int64_t cols, int64_t rows_per_outer, const int32_t* gather, int64_t M,
                          const int64_t* offsets, int G, int target, uint64_t seed,
                          uint32_t stream_id, uint8_t* out, uint8_t* out_e8m0, int64_t ld,
                          bool e8m0_kb_major, int64_t* padded_offsets, hipStream_t stream, bool blocked)
{
    TransposeArgs a{};
    a.e8m0_kb_major = e8m0_kb_major;
    a.blocked = blocked && (target == PMN_TARGET_E4M3 || target == TARGET_E2M1_PACKED);
    a.unit = a.blocked ? (target == PMN_TARGET_E4M3 ? 64 : 128) : 32;
    a.codes = codes; a.scales = scales; a.outer = outer; a.rows_per_outer = rows_per_outer;
    a.x = nullptr; a.cols = cols; a.gather = gather; a.M = M; a.offsets = offsets; a.G = G;
    a.seed = seed; a.stream_id = stream_id; a.out = out; a.out_e8m0 = out_e8m0; a.ld = ld;
    return launch_transpose(a, SRC_NVFP4, 1, target, padded_offsets, stream);
}

// ------------------------------------------------------------------------------------------
// dY to MXFP8 both ways in one read (the backward's gradient operands, E4M3 by round to nearest
// even): the row-wise codes that dgrad takes and the column-wise codes (per 32 slots of a group)
// that wgrad takes, each in the blocked GEMM operand layout, with the same bytes as
// k_mxfp8_rows_kbm<false, false, true> and k_transpose_quant<SRC_BF16, 0, 0> write separately.
// A workgroup takes one 64-slot unit of the padded slot space (groups are padded to 64 slots, so
// the unit lies in one group) and 256 columns: the 64 x 256 bf16 tile is read once into the LDS;
// then each thread quantizes two row blocks (32 columns of one slot) and one column pair (two
// columns over 32 slots). Padding slots read as zero.
//
// SWI: dY is the SwiGLU backward's dh13 = [dh1 | dh3] (N = 2F), formed on the fly from
// da [M x F] (fp32) and h13 [M x 2F] (bf16) exactly as k_swiglu_bwd forms it; the workgroup's
// 256 features give a dh1 tile and a dh3 tile, both quantized both ways.
// ------------------------------------------------------------------------------------------
constexpr int RC_COLS = 256;
constexpr int RC_PITCH = RC_COLS * 2 + 16;   // bytes per tile row: 16-byte row reads of 16 rows cover all banks

// The 64-slot unit at padded slot p0 (a multiple of 64): its first slot s0 and how many of its
// slots exist (nv), from the groups' 64-slot padded offsets po [G+1] by one binary search (the
// largest g with po[g] <= p0 is the group holding p0; empty groups have po[g] == po[g+1]). False
// past the last group's padding.
PMN_DEV bool unit_of(int64_t p0, const int64_t* __restrict__ offsets, const int64_t* __restrict__ po, int G,
                     int64_t M, int64_t& s0, int64_t& nv)
{
    if (offsets == nullptr) {
        s0 = p0;
        nv = M - p0 < 64 ? M - p0 : 64;
        return p0 < M;
    }
    if (p0 >= po[G]) return false;
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (po[mid] <= p0) lo = mid; else hi = mid - 1;
    }
    s0 = offsets[lo] + (p0 - po[lo]);
    const int64_t end = offsets[lo + 1] < M ? offsets[lo + 1] : M;
    nv = end - s0 < 0 ? 0 : (end - s0 < 64 ? end - s0 : 64);
    return true;
}

template <bool SWI>
__global__ __launch_bounds__(256) void k_mxfp8_rows_cols(const uint16_t* __restrict__ x, const float* __restrict__ da,
                                                        int64_t M, int64_t N, const int64_t* __restrict__ offsets,
                                                        const int64_t* __restrict__ po, int G, int64_t Pb,
                                                        uint8_t* __restrict__ rq, uint8_t* __restrict__ re,
                                                        uint8_t* __restrict__ cq, uint8_t* __restrict__ ce)
{
    constexpr int NT = SWI ? 2 : 1;   // tiles per workgroup
    __shared__ __attribute__((aligned(16))) uint8_t tile[NT][64 * RC_PITCH];
    const int t = threadIdx.x;
    const int64_t p0 = (int64_t)blockIdx.x * 64;          // first padded slot of the unit
    const int64_t c0 = (int64_t)blockIdx.y * RC_COLS;     // first column (SWI: first feature)
    const int64_t W = SWI ? N / 2 : N;                    // columns the grid spans (SWI: F)
    // slots of the unit that exist: s0 .. s0 + nv - 1
    int64_t s0 = 0, nv = 0;
    if (!unit_of(p0, offsets, po, G, M, s0, nv)) return;   // workgroup-uniform
    // ---- the tile(s): 8 chunks of 8 columns per thread (row t / 32 + 8 i, chunk t % 32)
    if (SWI) {
        const uint16_t* h13 = x;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int row = (t >> 5) + 8 * i;
            const int64_t f = c0 + (t & 31) * 8;
            uint32_t o1[4] = {0u, 0u, 0u, 0u}, o3[4] = {0u, 0u, 0u, 0u};
            if (row < nv && f < W) {
                const int64_t s = s0 + row;
                // nontemporal: dA and h13 are read once
                const f32x4 g0v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(da + s * W + f));
                const f32x4 g1v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(da + s * W + f + 4));
                const u32x4 w1v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(h13 + s * N + f));
                const u32x4 w3v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(h13 + s * N + W + f));
                const float4 g0 = make_float4(g0v[0], g0v[1], g0v[2], g0v[3]);
                const float4 g1 = make_float4(g1v[0], g1v[1], g1v[2], g1v[3]);
                const uint4 w1 = make_uint4(w1v[0], w1v[1], w1v[2], w1v[3]);
                const uint4 w3 = make_uint4(w3v[0], w3v[1], w3v[2], w3v[3]);
                const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                const uint32_t a1[4] = {w1.x, w1.y, w1.z, w1.w}, a3[4] = {w3.x, w3.y, w3.z, w3.w};
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    uint32_t r1[2], r3[2];
#pragma unroll
                    for (int u = 0; u < 2; u++)
                        swiglu_bwd_elem(g[2 * q + u], u ? bf16_hi(a1[q]) : bf16_lo(a1[q]),
                                        u ? bf16_hi(a3[q]) : bf16_lo(a3[q]), r1[u], r3[u]);
                    o1[q] = r1[0] | (r1[1] << 16);
                    o3[q] = r3[0] | (r3[1] << 16);
                }
            }
            *reinterpret_cast<uint4*>(tile[0] + row * RC_PITCH + (t & 31) * 16) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
            *reinterpret_cast<uint4*>(tile[NT - 1] + row * RC_PITCH + (t & 31) * 16) = make_uint4(o3[0], o3[1], o3[2], o3[3]);
        }
    } else {
        uint4 v[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int row = (t >> 5) + 8 * i;
            const int64_t col = c0 + (t & 31) * 8;
            if (row < nv && col < N) {   // nontemporal: dY is read once
                const u32x4 t4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (s0 + row) * N + col));
                v[i] = make_uint4(t4[0], t4[1], t4[2], t4[3]);
            } else {
                v[i] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; i++)
            *reinterpret_cast<uint4*>(tile[0] + ((t >> 5) + 8 * i) * RC_PITCH + (t & 31) * 16) = v[i];
    }
    __syncthreads();
    const int64_t nb = N >> 5;

#pragma unroll
    for (int h = 0; h < NT; h++) {
        const uint8_t* tl = tile[h];
        const int64_t cb = c0 + h * W;   // the tile's first column of dY

        // ---- row-wise: unit u = t + 256 i is slot row u % 64, k-block u / 64 of the tile
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int u = t + 256 * i;
            const int row = u & 63, kbl = u >> 6;
            const int64_t kb = (cb >> 5) + kbl;
            if (row < nv && c0 + 32 * kbl < W) {
                uint32_t w[16];
                const uint4* src = reinterpret_cast<const uint4*>(tl + row * RC_PITCH + kbl * 64);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const uint4 a4 = src[q];
                    w[4 * q] = a4.x; w[4 * q + 1] = a4.y; w[4 * q + 2] = a4.z; w[4 * q + 3] = a4.w;
                }
                uint32_t o[8];
                const int e = mxfp8_block<false>(w, 0, kb, N, 0, 0, o);
                // padded row pr: k-block kb = chunks 2 (kb % 2), 2 (kb % 2) + 1 of 64-byte column
                // kb / 2 of its 1 KB block (16 rows x 64 bytes, chunk c of row r16 at slot
                // c ^ ((r16 / 4) % 4)); with an odd k-block count the last column's second half
                // holds zero codes
                const int64_t pr = p0 + row;
                const int r16 = (int)(pr & 15), xs = (r16 >> 2) & 3, c = 2 * (int)(kb & 1);
                uint8_t* b = rq + ((pr >> 4) * ((N + 63) >> 6) + (kb >> 1)) * 1024 + r16 * 64;
                *reinterpret_cast<uint4*>(b + ((c ^ xs) << 4)) = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4*>(b + (((c + 1) ^ xs) << 4)) = make_uint4(o[4], o[5], o[6], o[7]);
                if ((nb & 1) && kb == nb - 1) {
                    *reinterpret_cast<uint4*>(b + (((c + 2) ^ xs) << 4)) = make_uint4(0u, 0u, 0u, 0u);
                    *reinterpret_cast<uint4*>(b + (((c + 3) ^ xs) << 4)) = make_uint4(0u, 0u, 0u, 0u);
                }
                re[kb * Pb + pr] = (uint8_t)(e + 127);
            }
        }

        // ---- column-wise: thread t takes columns 2 (t % 128) and 2 (t % 128) + 1 over slots
        // 32 (t / 128) .. + 31 of the unit (padding slots are +0)
        const int cp = t & 127, sb = t >> 7;
        if (c0 + 2 * cp < W) {
            const int64_t col = cb + 2 * cp;
            uint32_t pw[32];
#pragma unroll
            for (int j = 0; j < 32; j++) pw[j] = *reinterpret_cast<const uint32_t*>(tl + (sb * 32 + j) * RC_PITCH + cp * 4);
            float amax0 = 0.0f, amax1 = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; j++) {
                amax0 = fmaxf(amax0, fabsf(bf16_lo(pw[j])));
                amax1 = fmaxf(amax1, fabsf(bf16_hi(pw[j])));
            }
            const int e0 = e8m0_exponent<E8M0_E4M3>(amax0), e1 = e8m0_exponent<E8M0_E4M3>(amax1);
            const float s0 = __builtin_ldexpf(1.0f, e0), s1 = __builtin_ldexpf(1.0f, e1);
            uint32_t o0[8], o1[8];
#pragma unroll
            for (int q = 0; q < 8; q++) {
                // slots 4q .. 4q + 3 of each column into one word (slot 4q in the low byte)
                o0[q] = e4m3_rne_pair_scaled_into(0u, bf16_lo(pw[4 * q]), bf16_lo(pw[4 * q + 1]), s0, false);
                o0[q] = e4m3_rne_pair_scaled_into(o0[q], bf16_lo(pw[4 * q + 2]), bf16_lo(pw[4 * q + 3]), s0, true);
                o1[q] = e4m3_rne_pair_scaled_into(0u, bf16_hi(pw[4 * q]), bf16_hi(pw[4 * q + 1]), s1, false);
                o1[q] = e4m3_rne_pair_scaled_into(o1[q], bf16_hi(pw[4 * q + 2]), bf16_hi(pw[4 * q + 3]), s1, true);
            }
            // output row c (one per column): 1 KB blocks of 16 rows x 64 bytes, the unit's 64
            // slots one block column; this 32-slot block is chunks 2 sb and 2 sb + 1 of the row
            const int64_t kbo = p0 >> 6, nkb = Pb >> 6;
#pragma unroll
            for (int hc = 0; hc < 2; hc++) {
                const int64_t c = col + hc;
                const uint32_t* o = hc ? o1 : o0;
                const int r16 = (int)(c & 15), xs = (r16 >> 2) & 3;
                uint8_t* b = cq + ((c >> 4) * nkb + kbo) * 1024 + r16 * 64;
                *reinterpret_cast<uint4*>(b + (((2 * sb) ^ xs) << 4)) = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4*>(b + (((2 * sb + 1) ^ xs) << 4)) = make_uint4(o[4], o[5], o[6], o[7]);
            }
            // E8M0 k-block-major: [Pb/32 x N], 32-slot block (p0 / 32 + sb) at row kb
            uint8_t* eo = ce + (p0 / 32 + sb) * N + col;
            eo[0] = (uint8_t)(e0 + 127);
            eo[1] = (uint8_t)(e1 + 127);
        }
    }
}

hipError_t launch_mxfp8_rows_cols(const uint16_t* x, int64_t M, int64_t N, const int64_t* offsets,
                                  const int64_t* po, int G, int64_t Pb, uint8_t* rq, uint8_t* re, uint8_t* cq,
                                  uint8_t* ce, hipStream_t stream)
{
    if (M == 0 || N == 0 || Pb == 0) return hipSuccess;
    const dim3 grid((unsigned)(Pb / 64), (unsigned)((N + RC_COLS - 1) / RC_COLS));
    hipLaunchKernelGGL(k_mxfp8_rows_cols<false>, grid, dim3(256), 0, stream, x, nullptr, M, N, offsets, po, G, Pb,
                       rq, re, cq, ce);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd_mxfp8_rows_cols(const float* da, const uint16_t* h13, int64_t M, int64_t F,
                                             const int64_t* offsets, const int64_t* po, int G, int64_t Pb,
                                             uint8_t* rq, uint8_t* re, uint8_t* cq, uint8_t* ce, hipStream_t stream)
{
    if (M == 0 || F == 0 || Pb == 0) return hipSuccess;
    const dim3 grid((unsigned)(Pb / 64), (unsigned)((F + RC_COLS - 1) / RC_COLS));
    hipLaunchKernelGGL(k_mxfp8_rows_cols<true>, grid, dim3(256), 0, stream, h13, da, M, 2 * F, offsets, po, G, Pb,
                       rq, re, cq, ce);
    return hipGetLastError();
}

hipError_t launch_mxfp8_cols(const uint16_t* x, int64_t M, int64_t N, const int64_t* offsets,
                             int G, bool sr, uint64_t seed, uint32_t stream_id, uint8_t* out,
                             uint8_t* out_e8m0, int64_t ld, bool e8m0_kb_major,
                             int64_t* padded_offsets, hipStream_t stream, int target, bool blocked)
{
    TransposeArgs a{};
    a.e8m0_kb_major = e8m0_kb_major;
    a.blocked = blocked && (target == PMN_TARGET_E4M3 || target == TARGET_E2M1_PACKED);
    a.unit = a.blocked ? (target == PMN_TARGET_E4M3 ? 64 : 128) : 32;
    a.codes = nullptr; a.scales = nullptr; a.outer = nullptr; a.rows_per_outer = 1;
    a.x = x; a.cols = N; a.gather = nullptr; a.M = M; a.offsets = offsets; a.G = G;
    a.seed = seed; a.stream_id = stream_id; a.out = out; a.out_e8m0 = out_e8m0; a.ld = ld;
    return launch_transpose(a, SRC_BF16, sr ? 1 : 0, target, padded_offsets, stream);
}

}  // namespace pmn
