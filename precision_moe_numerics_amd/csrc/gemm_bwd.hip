// gemm_bwd.hip -- MXFP8 grouped GEMMs of the expert-layer backward (dgrad, wgrad) and the
// SwiGLU backward.
//
// Pages cited (by title and section heading):
//   [AREX] AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向传播
//          贯穿预训练到最后一次 RL rollout":
//            "只把专家层的前向传播降到 4-bit" -- the backward pass runs in MXFP8;
//            "转置打散分组,随机舍入保住期望值" -- weights and activations are re-quantized to
//              MXFP8 with stochastic rounding and the gradients use MXFP8 matmuls.
//
// Both GEMMs are D[r, c] = sum_k A[r, k] B[c, k] over E4M3 operands with one E8M0 scale per 32
// consecutive k, which is exactly the operand format of gfx950's block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3). Its lane layout, measured on the device:
// lane l supplies row l % 32; with h = l / 32 its bytes 0..15 are k = 16h .. 16h+15 and bytes
// 16..31 are k = 32+16h .. 32+16h+15 of the 64-k step, and its scale operand is the E8M0 scale
// of k-block h of that row (k-block b of the step = k in [32b, 32b+32)).
//
// Tiling: 256 x 256 output tile per workgroup of 8 wavefronts (128 x 64 each, 4 x 2 MFMA
// blocks, two wavefronts per SIMD to hide latency), K stages of 64 bytes (one MFMA k-step)
// staged through LDS (rows padded to 80 bytes), two stages.
#include "pmn_dev.hpp"
#include "pmn_kernels.hpp"

namespace pmn {

namespace bwd {
constexpr int BT = 256;
constexpr int BK = 64;                  // k per stage (bytes per row) = one MFMA k-step
constexpr int ROWB = 80;                // 64 + 16 pad: 16 consecutive rows hit 16 distinct 16-byte bank groups
constexpr int TILEB = BT * ROWB;        // one operand's codes
constexpr int SCB = BT * 4;             // one operand's scale bytes per row (2 used: 2 blocks of 32)
constexpr int STAGEB = 2 * TILEB + 2 * SCB;
constexpr int LDSB = 2 * STAGEB;
constexpr int THREADS = 512;            // 8 wavefronts: 2 along output rows x 4 along columns
static_assert(THREADS == 2 * BT, "one staging thread per row of each operand tile");
}  // namespace bwd

enum { MODE_DGRAD = 0, MODE_WGRAD = 1 };

struct Mx8Args {
    // dgrad: A = dY row-wise [M x Nf] (lda = Nf), B = W^T [Kf x G*Nf] (ldb = G*Nf, group g at
    //        column g*Nf), contraction Nf, output dX [M x Kf].
    // wgrad: A = dY^T [Nf x ld] , B = X^T [Kf x ld], contraction over the padded slots of group
    //        g (columns po[g] .. po[g+1]), output dW [G*Nf x Kf].
    const uint8_t* a;
    const uint8_t* ae;
    int64_t lda;
    const uint8_t* b;
    const uint8_t* be;
    int64_t ldb;
    const int64_t* offsets;
    const int64_t* po;        // padded offsets (wgrad)
    int G;
    int64_t Nf, Kf;
    float* out;
    int64_t rtiles, ctiles;   // tile grid (dgrad: slot-tile bound x Kf/256; wgrad: Nf/256 x Kf/256)
    int SM, SN;
};

template <int MODE>
__global__ __launch_bounds__(bwd::THREADS, 1) void k_mxfp8_grouped_gemm(Mx8Args p)
{
    using namespace bwd;
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDSB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave >> 2, wc = wave & 3;    // 2 wavefronts along output rows, 4 along columns

    int g = -1;
    int64_t r0 = 0, rvalid = BT, c0 = 0, kbeg = 0, klen = 0;
    const uint8_t *abase, *aebase, *bbase, *bebase;
    int64_t ldo;
    float* obase;
    TileXY tile;
    int64_t L = blockIdx.x, batch = 0;
    if (MODE == MODE_WGRAD) {
        // super-tiles of expert g are numbered after those of experts 0 .. g-1
        const int64_t nsuper = ((p.rtiles + p.SM - 1) / p.SM) * ((p.ctiles + p.SN - 1) / p.SN);
        const int64_t s = ((L >> 3) >> 5) * 8 + (L & 7);
        batch = s / nsuper;
        if (batch >= p.G) return;
        const int64_t s_in = s - batch * nsuper;
        const int64_t j = ((s_in >> 3) << 5) + ((L >> 3) & 31);
        L = (j << 3) | (s_in & 7);
    }
    if (!xcd_tile(L, p.rtiles, p.ctiles, p.SM, p.SN, tile)) return;
    if (MODE == MODE_DGRAD) {
        int64_t t = tile.row, cum = 0;
        for (int gg = 0; gg < p.G; gg++) {
            const int64_t s0 = p.offsets[gg], s1 = p.offsets[gg + 1];
            const int64_t tiles = (s1 - s0 + BT - 1) / BT;
            if (t < cum + tiles) {
                g = gg;
                r0 = s0 + (t - cum) * BT;
                rvalid = s1 - r0 < BT ? s1 - r0 : BT;
                break;
            }
            cum += tiles;
        }
        if (g < 0) return;
        c0 = tile.col * BT;
        kbeg = 0;
        klen = p.Nf;
        abase = p.a; aebase = p.ae;
        bbase = p.b + (int64_t)g * p.Nf; bebase = p.be + (int64_t)g * (p.Nf / 32);
        ldo = p.Kf;
        obase = p.out;
    } else {
        g = (int)batch;
        r0 = tile.row * BT;
        rvalid = BT;
        c0 = tile.col * BT;
        kbeg = p.po[g];
        klen = p.po[g + 1] - kbeg;
        abase = p.a + kbeg; aebase = p.ae + kbeg / 32;
        bbase = p.b + kbeg; bebase = p.be + kbeg / 32;
        ldo = p.Kf;
        obase = p.out + (int64_t)g * p.Nf * p.Kf;
    }

    // Staging: per stage each operand tile is 256 rows x 64 bytes = 1024 chunks of 16 bytes.
    // Threads 0..255 stage A and threads 256..511 stage B (wavefront-uniform); thread t stages
    // chunks q = 256 k + (t % 256) (row q / 4, part q % 4), so 4 lanes cover one row segment,
    // plus the 2 scale bytes of row t % 256. Loads are branch-free: a chunk outside the tile
    // reads a valid address and is replaced by zeros (scale 127).
    const bool stage_a = tid < BT;
    const int st = tid & (BT - 1);
    const int prow = st >> 2, part = st & 3;
    const uint8_t* srow[4];
    bool srow_ok[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int row = k * 64 + prow;
        srow_ok[k] = stage_a ? row < rvalid : true;
        srow[k] = stage_a ? abase + (r0 + (srow_ok[k] ? row : 0)) * p.lda + part * 16
                          : bbase + (c0 + row) * p.ldb + part * 16;
    }
    const bool scrow_ok = stage_a ? st < rvalid : true;
    const uint8_t* sep = stage_a ? aebase + (r0 + (scrow_ok ? st : 0)) * (p.lda / 32)
                                 : bebase + (c0 + st) * (p.ldb / 32);
    const int64_t kblocks = klen / 32;
    uint8_t* const lds_tile = lds + (stage_a ? 0 : TILEB);
    uint32_t* const lds_sc = reinterpret_cast<uint32_t*>(lds + 2 * TILEB + (stage_a ? 0 : SCB));

    uint4 sv[4];
    uint32_t ss;
    auto load_stage = [&](int kt) {
        const int64_t k0 = (int64_t)kt * BK;
        const bool kok = k0 + part * 16 < klen;
        const int64_t koff = kok ? k0 : 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint4 v = *reinterpret_cast<const uint4*>(srow[k] + koff);
            sv[k] = (kok && srow_ok[k]) ? v : make_uint4(0u, 0u, 0u, 0u);
        }
        uint32_t sc = 0u;
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int64_t kb = k0 / 32 + q;
            const bool ok = kb < kblocks;
            const uint32_t x = sep[ok ? kb : 0];
            sc |= ((ok && scrow_ok) ? x : 127u) << (8 * q);
        }
        ss = sc;
    };
    auto store_stage = [&](int buf) {
        uint8_t* base = lds_tile + buf * STAGEB;
#pragma unroll
        for (int k = 0; k < 4; k++) *reinterpret_cast<uint4*>(base + (k * 64 + prow) * ROWB + part * 16) = sv[k];
        lds_sc[buf * (STAGEB / 4) + st] = ss;
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int KT = (int)((klen + BK - 1) / BK);
    if (KT > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();
    const int lrow = lane & 31, hh = lane >> 5;
    for (int kt = 0; kt < KT; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load_stage(kt + 1);
        const uint8_t* base = lds + buf * STAGEB;
        const uint32_t* sca = reinterpret_cast<const uint32_t*>(base + 2 * TILEB);
        const uint32_t* scb = reinterpret_cast<const uint32_t*>(base + 2 * TILEB + SCB);
#pragma unroll
        for (int ks = 0; ks < BK / 64; ks++) {
            i32x8 af[4], bf[2];
            int sa[4], sb[2];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int row = wr * 128 + i * 32 + lrow;
                const uint8_t* src = base + row * ROWB + ks * 64 + hh * 16;
                uint4 lo = *reinterpret_cast<const uint4*>(src);
                uint4 hi = *reinterpret_cast<const uint4*>(src + 32);
                af[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                sa[i] = (int)((sca[row] >> (8 * (2 * ks + hh))) & 0xFFu);
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int row = wc * 64 + j * 32 + lrow;
                const uint8_t* src = base + TILEB + row * ROWB + ks * 64 + hh * 16;
                uint4 lo = *reinterpret_cast<const uint4*>(src);
                uint4 hi = *reinterpret_cast<const uint4*>(src + 32);
                bf[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                sb[j] = (int)((scb[row] >> (8 * (2 * ks + hh))) & 0xFFu);
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
        }
        // keep the next stage's LDS writes (which wait for its global loads) after the MFMAs
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < KT) store_stage(buf ^ 1);
        __syncthreads();
    }

    // epilogue: block (i, j): lane holds column c = c0 + wc*64 + j*32 + lane%32 and rows
    // r = r0 + wr*128 + i*32 + (v/4)*8 + hh*4 + v%4
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = c0 + wc * 64 + j * 32 + lrow;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t rl = wr * 128 + i * 32 + (v >> 2) * 8 + hh * 4 + (v & 3);
                if (rl < rvalid) obase[(r0 + rl) * ldo + col] = acc[i][j][v];
            }
        }
}

hipError_t launch_mxfp8_dgrad(const uint8_t* dq, const uint8_t* de, const uint8_t* wt,
                              const uint8_t* wte, const int64_t* offsets, int G, int64_t M,
                              int64_t Nf, int64_t Kf, float* dx, hipStream_t stream)
{
    if (M == 0 || G == 0) return hipSuccess;
    const int64_t rt = (M + bwd::BT - 1) / bwd::BT + G, ct = Kf / bwd::BT;
    int SM, SN;
    xcd_shape(rt, ct, SM, SN);
    Mx8Args p{dq, de, Nf, wt, wte, (int64_t)G * Nf, offsets, nullptr, G, Nf, Kf, dx, rt, ct, SM, SN};
    dim3 grid((unsigned)xcd_grid(rt, ct, SM, SN));
    hipLaunchKernelGGL((k_mxfp8_grouped_gemm<MODE_DGRAD>), grid, dim3(bwd::THREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mxfp8_wgrad(const uint8_t* dt, const uint8_t* dte, const uint8_t* xt,
                              const uint8_t* xte, int64_t ld, const int64_t* po, int G,
                              int64_t Nf, int64_t Kf, float* dw, hipStream_t stream)
{
    if (G == 0) return hipSuccess;
    const int64_t rt = Nf / bwd::BT, ct = Kf / bwd::BT;
    int SM, SN;
    xcd_shape(rt, ct, SM, SN);
    Mx8Args p{dt, dte, ld, xt, xte, ld, nullptr, po, G, Nf, Kf, dw, rt, ct, SM, SN};
    dim3 grid((unsigned)xcd_grid(rt, ct, SM, SN, G));
    hipLaunchKernelGGL((k_mxfp8_grouped_gemm<MODE_WGRAD>), grid, dim3(bwd::THREADS), 0, stream, p);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// SwiGLU backward (elementwise): dh1 = da * h3 * silu'(h1), dh3 = da * silu(h1),
// silu'(h) = s (1 + h (1 - s)), s = sigmoid(h). Eight elements per thread.
// ------------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_swiglu_bwd(const float* __restrict__ da, const uint16_t* __restrict__ h13,
                                                    int64_t M, int64_t F, uint16_t* __restrict__ dh13)
{
    const int64_t per_row = F / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * per_row) return;
    const int64_t m = i / per_row, j0 = (i - m * per_row) * 8;
    const float4* pd = reinterpret_cast<const float4*>(da + m * F + j0);
    float4 d0 = pd[0], d1 = pd[1];
    float d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    uint4 w1 = *reinterpret_cast<const uint4*>(h13 + m * 2 * F + j0);
    uint4 w3 = *reinterpret_cast<const uint4*>(h13 + m * 2 * F + F + j0);
    uint32_t a1[4] = {w1.x, w1.y, w1.z, w1.w}, a3[4] = {w3.x, w3.y, w3.z, w3.w};
    uint32_t o1[4], o3[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint32_t r1[2], r3[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            float h1 = u ? bf16_hi(a1[q]) : bf16_lo(a1[q]);
            float h3 = u ? bf16_hi(a3[q]) : bf16_lo(a3[q]);
            float s = 1.0f / (1.0f + expf(-h1));
            float g = d[2 * q + u];
            r1[u] = f32_to_bf16_bits(g * h3 * (s * (1.0f + h1 * (1.0f - s))));
            r3[u] = f32_to_bf16_bits(g * h1 * s);
        }
        o1[q] = r1[0] | (r1[1] << 16);
        o3[q] = r3[0] | (r3[1] << 16);
    }
    *reinterpret_cast<uint4*>(dh13 + m * 2 * F + j0) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
    *reinterpret_cast<uint4*>(dh13 + m * 2 * F + F + j0) = make_uint4(o3[0], o3[1], o3[2], o3[3]);
}

hipError_t launch_swiglu_bwd(const float* da, const uint16_t* h13, int64_t M, int64_t F,
                             uint16_t* dh13, hipStream_t stream)
{
    const int64_t n = M * (F / 8);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_swiglu_bwd, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, da, h13, M, F, dh13);
    return hipGetLastError();
}

}  // namespace pmn
