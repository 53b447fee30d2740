// gemm_fwd.hip -- NVFP4 grouped expert GEMM (forward) with bf16/fp32, SwiGLU and RHT32 + S2F6
// epilogues.
//
// Pages cited (by title and section heading):
//   [AREX] AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向传播
//          贯穿预训练到最后一次 RL rollout":
//            "只把专家层的前向传播降到 4-bit" -- the expert layers' forward runs in NVFP4 with
//              dedicated kernels;
//            "计算提速后,NVLink 通信成了新瓶颈" -- the RHT and the S2F6 quantization are fused
//              into the end of the w2 matmul, so the combine payload leaves the GEMM at 8.25
//              bits per value.
//
// Arithmetic. Every NVFP4 value is fp4 * e4m3 (the outer scales are applied in the epilogue).
// That product has at most 6 significant bits and lies in [2^-10, 2688], so it is exact in
// fp16; products of two such values are exact in fp32. The kernel dequantizes FP4 codes with
// the gfx950 FP4->fp16 converter and one packed fp16 multiply by the block scale, then runs
// v_mfma_f32_32x32x16_f16 with fp32 accumulation. gfx950's block-scaled MFMA only takes E8M0
// scales per 32 values, which cannot carry an E4M3 scale per 16, so the exact path is the fp16
// one.
//
// Tiling. A workgroup of 8 wavefronts computes a 256 (weight rows n) x 256 (slots m) tile of
// D = W X^T, i.e. Y^T, as 2 x 4 wavefront tiles of 128 x 64 (4 x 2 MFMA blocks), two wavefronts
// per SIMD. K advances in stages of 64: each thread owns one weight row or one (gathered)
// activation row, fetches its 32 code bytes and 4 scale bytes two stages ahead into registers,
// and dequantizes them into 128 bytes of fp16 in LDS (rows padded to 144 bytes, so fragment
// reads are bank-conflict free) between the MFMAs of the current stage; two LDS stages
// alternate with one barrier per stage.
// Groups (experts) are ragged: workgroup y walks the device offsets to find its (expert,
// slot tile), so no host synchronization is needed.
#include "pmn_dev.hpp"
#include "pmn_kernels.hpp"

namespace pmn {

namespace fwd {
constexpr int BT = 256;                       // rows per operand tile
constexpr int BK = 64;                        // K per stage
constexpr int ROWB = 144;                     // LDS bytes per row: 64 fp16 + 16 pad
constexpr int TILEB = BT * ROWB;              // one operand tile
constexpr int STAGEB = 2 * TILEB;             // weights + activations
constexpr int LDSB = 2 * STAGEB;              // two stages
constexpr int THREADS = 512;                  // 8 wavefronts: 2 along weight rows x 4 along slots
static_assert(THREADS == 2 * BT, "one staging thread per row of each operand tile");
// Epilogue: the LDS holds output tiles of 256 slots x 256 bytes (row pitch 272, so the
// transposed fragment writes of 32 slots fall on 16 distinct bank groups), written out as whole
// row segments.
constexpr int OPITCH = 272;
constexpr int OTILE = BT * OPITCH;
static_assert(2 * OTILE + BT * 8 <= LDSB, "two output tiles and the E8M0 tile fit in the LDS");
}  // namespace fwd

struct FwdArgs {
    const uint8_t* a_codes;   // activations NVFP4 [a_rows x K]
    const uint8_t* a_scales;
    const float* a_outer;
    int64_t a_rpo;
    const int32_t* gather;
    const uint8_t* b_codes;   // weights NVFP4 [G*N x K]
    const uint8_t* b_scales;
    const float* b_outer;
    int64_t b_rpo;
    const int64_t* offsets;
    int G;
    int64_t N, K;
    uint32_t rht_mask;
    void* out;
    uint8_t* out_e8m0;
    void* out_aux;
    int64_t mtiles, ntiles;   // slot-tile bound and weight tiles
    int SM, SN;               // super-tile shape
};

// Dequantize block blk (16 FP4 values, two code words, one E4M3 scale byte) of one row's stage
// to 16 fp16 values written as 2 x 16 bytes to LDS.
struct RawStage {
    uint4 c0, c1;   // 32 code bytes = 64 FP4 values
    uint32_t s;     // 4 E4M3 block scales
};

template <int BLK>
PMN_DEV void dequant_block_to_lds(const RawStage& r, uint8_t* dst)
{
    const uint32_t w0 = BLK == 0 ? r.c0.x : BLK == 1 ? r.c0.z : BLK == 2 ? r.c1.x : r.c1.z;
    const uint32_t w1 = BLK == 0 ? r.c0.y : BLK == 1 ? r.c0.w : BLK == 2 ? r.c1.y : r.c1.w;
    // E4M3 (OCP, bias 7) byte -> fp32 by the hardware converter (exact, subnormals included)
    const _Float16 s = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.s, BLK);
    const f16x2 ss = {s, s};
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint32_t word = h ? w1 : w0;
        f16x2 p0 = PMN_FP4_TO_F16(word, 0) * ss;
        f16x2 p1 = PMN_FP4_TO_F16(word, 1) * ss;
        f16x2 p2 = PMN_FP4_TO_F16(word, 2) * ss;
        f16x2 p3 = PMN_FP4_TO_F16(word, 3) * ss;
        uint4 v;
        __builtin_memcpy(&v.x, &p0, 4);
        __builtin_memcpy(&v.y, &p1, 4);
        __builtin_memcpy(&v.z, &p2, 4);
        __builtin_memcpy(&v.w, &p3, 4);
        *reinterpret_cast<uint4*>(dst + 16 * (2 * BLK + h)) = v;
    }
}

template <int EPI>
__global__ __launch_bounds__(fwd::THREADS, 1) void k_nvfp4_grouped_gemm(FwdArgs p)
{
    using namespace fwd;
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDSB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave >> 2, wm = wave & 3;    // 2 wavefronts along weight rows, 4 along slots

    // ---- which (expert, slot tile, weight tile): XCD-aware order over slot tiles x weight tiles
    TileXY tile;
    if (!xcd_tile(blockIdx.x, p.mtiles, p.ntiles, p.SM, p.SN, tile)) return;
    const GroupUnit u = locate_group_unit(p.offsets, p.G, tile.row, BT);
    if (u.g < 0) return;
    const int g = u.g;
    const int64_t m0 = u.s0 + u.index * BT;
    const int64_t mvalid = u.s1 - m0 < BT ? u.s1 - m0 : BT;
    const int64_t N = p.N, K = p.K;
    const int64_t n0 = tile.col * (EPI == PMN_EPI_SWIGLU ? BT / 2 : BT);

    // ---- staging: threads 0..255 stage weight row t, threads 256..511 activation row t - 256
    const bool stage_w = tid < BT;                  // wavefront-uniform
    const int srow = tid & (BT - 1);
    const uint8_t* sc_codes;
    const uint8_t* sc_scales;
    bool svalid = true;
    if (stage_w) {
        int64_t wrow;
        if (EPI == PMN_EPI_SWIGLU) {
            const int F = (int)(N >> 1);
            const int twn = srow >> 7, trb = (srow & 127) >> 5, tr = srow & 31;
            wrow = (int64_t)g * N + (trb < 2 ? 0 : F) + n0 + twn * 64 + (trb & 1) * 32 + tr;
        } else {
            wrow = (int64_t)g * N + n0 + srow;
        }
        sc_codes = p.b_codes + wrow * (K >> 1);
        sc_scales = p.b_scales + wrow * (K >> 4);
    } else {
        svalid = srow < mvalid;
        const int64_t xrow = svalid ? (p.gather ? (int64_t)p.gather[m0 + srow] : m0 + srow) : 0;
        sc_codes = p.a_codes + xrow * (K >> 1);
        sc_scales = p.a_scales + xrow * (K >> 4);
    }
    uint8_t* const lds_row = lds + (stage_w ? 0 : TILEB) + srow * ROWB;

    // Raw stages are fetched into registers two iterations ahead of their dequantization: three
    // register sets rotate over an unrolled-by-3 loop. Fetches past the last stage re-read it, so
    // every iteration issues the same loads and the compiler's load counting stays exact.
    // A slot row past the tile's end reads activation row 0 instead: its products land only in
    // output columns that are never stored, so the loaded values need no masking (masking them
    // here would make every fetch wait for its data at once).
    auto load_raw = [&](int kt, RawStage& r) {
        const uint4* pc = reinterpret_cast<const uint4*>(sc_codes + (int64_t)kt * (BK / 2));
        r.c0 = pc[0];
        r.c1 = pc[1];
        r.s = *reinterpret_cast<const uint32_t*>(sc_scales + (int64_t)kt * (BK / 16));
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int KT = (int)(K / BK);
    const int lrow = lane & 31, lk = (lane >> 5) * 16;
    // one iteration: MFMAs on LDS stage kt % 2 while stage kt + 1 (registers `nxt`) is
    // dequantized into the other LDS stage, one 16-value block per k-substep, and stage kt + 3 is
    // fetched into `fut` (whose stage kt was dequantized in the previous iteration)
    // The last iteration dequantizes a repeated stage into the LDS stage nobody reads again, so
    // the body has no conditional work and the compiler's wait counts stay exact.
    auto step = [&](int kt, const RawStage& nxt, RawStage& fut) {
        const int buf = kt & 1;
        load_raw(kt + 3 < KT ? kt + 3 : KT - 1, fut);
        uint8_t* const dst = lds_row + (buf ^ 1) * STAGEB;
        const uint8_t* wb = lds + buf * STAGEB + (wn * 128 + lrow) * ROWB + lk;
        const uint8_t* xb = lds + buf * STAGEB + TILEB + (wm * 64 + lrow) * ROWB + lk;
        // fragments of k-substep ks + 1 are read while the MFMAs of ks run
        f16x8 af[2][4], bf[2][2];
        auto read_frags = [&](int ks, f16x8 (&a)[4], f16x8 (&b)[2]) {
#pragma unroll
            for (int i = 0; i < 4; i++) a[i] = *reinterpret_cast<const f16x8*>(wb + i * 32 * ROWB + ks * 32);
#pragma unroll
            for (int j = 0; j < 2; j++) b[j] = *reinterpret_cast<const f16x8*>(xb + j * 32 * ROWB + ks * 32);
        };
        read_frags(0, af[0], bf[0]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ks++) {
            if (ks + 1 < BK / 16) read_frags(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks & 1][i], bf[ks & 1][j], acc[i][j], 0, 0, 0);
            if (ks == 0) dequant_block_to_lds<0>(nxt, dst);
            if (ks == 1) dequant_block_to_lds<1>(nxt, dst);
            if (ks == 2) dequant_block_to_lds<2>(nxt, dst);
            if (ks == 3) dequant_block_to_lds<3>(nxt, dst);
        }
        __syncthreads();
    };

    RawStage r0, r1, r2;
    load_raw(0, r0);
    load_raw(KT > 1 ? 1 : 0, r1);
    load_raw(KT > 2 ? 2 : KT - 1, r2);
    dequant_block_to_lds<0>(r0, lds_row);
    dequant_block_to_lds<1>(r0, lds_row);
    dequant_block_to_lds<2>(r0, lds_row);
    dequant_block_to_lds<3>(r0, lds_row);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 < KT; kt += 3) {
        step(kt, r1, r0);
        step(kt + 1, r2, r1);
        step(kt + 2, r0, r2);
    }
    if (kt < KT) step(kt, r1, r0);
    if (kt + 1 < KT) step(kt + 1, r2, r1);

    // ---- epilogue: lane holds slot m = (wm*64 + j*32 + lane%32), weight rows of block i
    const int hh = lane >> 5;
    // copy rows [0, mvalid) of an output tile (256 bytes per slot) to dst + (m0 + row) * pitch
    auto store_tile = [&](const uint8_t* src, uint8_t* dst, int64_t pitch) {
#pragma unroll
        for (int k = 0; k < (BT * 16) / THREADS; k++) {
            const int q = k * THREADS + tid;
            const int row = q >> 4, c = q & 15;
            if (row < mvalid)
                *reinterpret_cast<uint4*>(dst + (m0 + row) * pitch + c * 16) =
                    *reinterpret_cast<const uint4*>(src + row * OPITCH + c * 16);
        }
    };
    if (EPI == PMN_EPI_SWIGLU || EPI == PMN_EPI_RHT32_S2F6) {
        __syncthreads();   // every fragment read of the main loop is done: the LDS holds output tiles
        uint8_t* const t0 = lds;
        uint8_t* const t1 = lds + OTILE;
        uint8_t* const te = lds + 2 * OTILE;
        float sxs[2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t ml = wm * 64 + j * 32 + (lane & 31);
            const bool mok = ml < mvalid;
            const int64_t m = m0 + ml;
            const int64_t xr = mok ? (p.gather ? (int64_t)p.gather[m] : m) : 0;
            sxs[j] = mok ? p.a_outer[xr / p.a_rpo] : 0.0f;
        }
        if (EPI == PMN_EPI_SWIGLU) {
            // tile 0: A = silu(h1) h3 (128 features), tile 1: h1; then tile 0 again: h3
            const int64_t F = N >> 1;
            const bool aux = p.out_aux != nullptr;
#pragma unroll
            for (int phase = 0; phase < 2; phase++) {
                if (phase == 1 && !aux) break;
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int ml = wm * 64 + j * 32 + (lane & 31);
#pragma unroll
                    for (int i = 0; i < 2; i++) {
                        const int64_t jbase = n0 + wn * 64 + i * 32;       // A column of row 0 of block
                        const float s1 = sxs[j] * p.b_outer[((int64_t)g * N + jbase) / p.b_rpo];
                        const float s3 = sxs[j] * p.b_outer[((int64_t)g * N + F + jbase) / p.b_rpo];
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            uint32_t ab[4], b1[4], b3[4];
#pragma unroll
                            for (int u = 0; u < 4; u++) {
                                const float h1 = acc[i][j][4 * q + u] * s1;
                                const float h3 = acc[i + 2][j][4 * q + u] * s3;
                                ab[u] = f32_to_bf16_bits(silu(h1) * h3);
                                b1[u] = f32_to_bf16_bits(h1);
                                b3[u] = f32_to_bf16_bits(h3);
                            }
                            const int off = ml * OPITCH + 2 * (wn * 64 + i * 32 + q * 8 + hh * 4);
                            if (phase == 0) {
                                *reinterpret_cast<uint2*>(t0 + off) = make_uint2(ab[0] | (ab[1] << 16), ab[2] | (ab[3] << 16));
                                if (aux) *reinterpret_cast<uint2*>(t1 + off) = make_uint2(b1[0] | (b1[1] << 16), b1[2] | (b1[3] << 16));
                            } else {
                                *reinterpret_cast<uint2*>(t0 + off) = make_uint2(b3[0] | (b3[1] << 16), b3[2] | (b3[3] << 16));
                            }
                        }
                    }
                }
                __syncthreads();
                uint8_t* const H = reinterpret_cast<uint8_t*>(p.out_aux);
                if (phase == 0) {
                    store_tile(t0, reinterpret_cast<uint8_t*>(p.out) + n0 * 2, F * 2);
                    if (aux) store_tile(t1, H + n0 * 2, N * 2);
                } else {
                    store_tile(t0, H + (F + n0) * 2, N * 2);
                }
                if (phase == 0 && aux) __syncthreads();   // tile 0 is rewritten with h3
            }
        } else {
            // RHT32 + S2F6: codes into tile 0 (256 columns of int8), E8M0 into the E8M0 tile
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int ml = wm * 64 + j * 32 + (lane & 31);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int nl = wn * 128 + i * 32;                  // tile column of row 0 of block
                    const float s = sxs[j] * p.b_outer[((int64_t)g * N + n0 + nl) / p.b_rpo];
                    f32x16 z;
#pragma unroll
                    for (int v = 0; v < 16; v++) z[v] = acc[i][j][v] * s;
                    rht_block_store(z, p.rht_mask, lane, reinterpret_cast<int8_t*>(t0 + ml * OPITCH + nl),
                                    te + ml * 8 + (nl >> 5));
                }
            }
            __syncthreads();
            store_tile(t0, reinterpret_cast<uint8_t*>(p.out) + n0, N);
            if (tid < mvalid)
                *reinterpret_cast<uint2*>(p.out_e8m0 + (m0 + tid) * (N >> 5) + (n0 >> 5)) =
                    *reinterpret_cast<const uint2*>(te + tid * 8);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int64_t ml = wm * 64 + j * 32 + (lane & 31);
        const bool mok = ml < mvalid;
        const int64_t m = m0 + ml;
        const int64_t xr = mok ? (p.gather ? (int64_t)p.gather[m] : m) : 0;
        const float sx = mok ? p.a_outer[xr / p.a_rpo] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t nb = n0 + wn * 128 + i * 32;           // first weight row of block
            const float s = sx * p.b_outer[((int64_t)g * N + nb) / p.b_rpo];
            if (mok) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int64_t col = nb + q * 8 + hh * 4;
                    float y0 = acc[i][j][4 * q] * s, y1 = acc[i][j][4 * q + 1] * s;
                    float y2 = acc[i][j][4 * q + 2] * s, y3 = acc[i][j][4 * q + 3] * s;
                    if (EPI == PMN_EPI_F32) {
                        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + m * N + col) = make_float4(y0, y1, y2, y3);
                    } else {
                        uint2 v = make_uint2(f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16),
                                             f32_to_bf16_bits(y2) | (f32_to_bf16_bits(y3) << 16));
                        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + m * N + col) = v;
                    }
                }
            }
        }
    }
}

hipError_t launch_gemm_fwd(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                           int64_t a_rpo, const int32_t* gather, const uint8_t* b_codes,
                           const uint8_t* b_scales, const float* b_outer, int64_t b_rpo,
                           const int64_t* offsets, int G, int64_t M, int64_t N, int64_t K,
                           int epilogue, uint32_t rht_mask, void* out, uint8_t* out_e8m0,
                           void* out_aux, hipStream_t stream)
{
    if (M == 0 || G == 0) return hipSuccess;
    const int64_t mtiles = (M + fwd::BT - 1) / fwd::BT + G;   // bound on sum of ceil(m_g / 256)
    const int64_t ntiles = N / fwd::BT;   // SWIGLU: each tile covers 128 w1 and 128 w3 rows
    int SM, SN;
    xcd_shape(mtiles, ntiles, SM, SN);
    FwdArgs p{a_codes, a_scales, a_outer, a_rpo, gather, b_codes, b_scales, b_outer, b_rpo,
              offsets, G, N, K, rht_mask, out, out_e8m0, out_aux, mtiles, ntiles, SM, SN};
    dim3 grid((unsigned)xcd_grid(mtiles, ntiles, SM, SN));
    switch (epilogue) {
    case PMN_EPI_F32: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_F32>), grid, dim3(fwd::THREADS), 0, stream, p); break;
    case PMN_EPI_BF16: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_BF16>), grid, dim3(fwd::THREADS), 0, stream, p); break;
    case PMN_EPI_SWIGLU: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_SWIGLU>), grid, dim3(fwd::THREADS), 0, stream, p); break;
    default: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_RHT32_S2F6>), grid, dim3(fwd::THREADS), 0, stream, p); break;
    }
    return hipGetLastError();
}

}  // namespace pmn
