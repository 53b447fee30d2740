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
// blocks, two wavefronts per SIMD). Operands stream through a ring of 4 LDS stages of 64 k
// (one MFMA k-step) filled by global_load_lds (global -> LDS without registers), so three
// stages are in flight while one is multiplied. Every wavefront issues the same 5 loads per
// stage (4 x 1 KB of codes, 1 x 128 B of scales), so "stage kt has landed" is the per-wave
// condition vmcnt <= 5 x (stages issued after kt), followed by a barrier.
//
// LDS stage: A codes [256 rows x 64 B], B codes [256 x 64 B], A scales [2 k-blocks x 256 rows],
// B scales [2 x 256]. Chunk c (16 B) of row r sits at slot c ^ ((r / 4) % 4): the 16 rows a
// quarter-wavefront reads cover all 16 bank groups (the load side applies the same permutation
// when it picks which chunk each lane fetches). Scales are streamed from k-block-major arrays, so
// one k-block of 256 rows is 256 contiguous bytes.
#include "pmn_dev.hpp"
#include "pmn_kernels.hpp"

namespace pmn {

namespace bwd {
constexpr int BT = 256;
constexpr int BK = 64;                  // k per stage (bytes per row) = one MFMA k-step
constexpr int NSTAGE = 4;
constexpr int TILEB = BT * BK;          // one operand's codes per stage
constexpr int SCB = 2 * BT;             // one operand's scales per stage
constexpr int STAGEB = 2 * TILEB + 2 * SCB;
constexpr int LDSB = NSTAGE * STAGEB;
constexpr int THREADS = 512;            // 8 wavefronts: 2 along output rows x 4 along columns
constexpr int LOADS_PER_STAGE = 5;      // per wavefront
static_assert(THREADS == 512 && BT == 256 && BK == 64, "the load assignment below assumes these sizes");
}  // namespace bwd

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
template <int N>
PMN_DEV void wait_loads_and_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

enum { MODE_DGRAD = 0, MODE_WGRAD = 1 };

struct Mx8Args {
    // dgrad: A = dY row-wise codes [M x Nf] (lda = Nf) with scales de [Nf/32 x Pb] at padded slot
    //        columns; B = W^T codes [Kf x G*Nf] (ldb = G*Nf, group g at column g*Nf) with scales
    //        [G*Nf/32 x Kf]; contraction Nf, output dX [M x Kf].
    // wgrad: A = dY^T [Nf x Pb], B = X^T [Kf x Pb] (lda = ldb = Pb), scales [Pb/32 x Nf] and
    //        [Pb/32 x Kf]; contraction over the padded slots of group g (po[g] .. po[g+1]),
    //        output dW [G*Nf x Kf].
    const uint8_t* a;
    const uint8_t* ae;
    int64_t lda;
    const uint8_t* b;
    const uint8_t* be;
    int64_t ldb;
    const int64_t* offsets;
    const int64_t* po;
    int64_t Pb;
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
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDSB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave >> 2, wc = wave & 3;    // 2 wavefronts along output rows, 4 along columns

    int g = -1;
    int64_t r0 = 0, rvalid = BT, c0 = 0, klen = 0;
    const uint8_t *acode, *bcode, *asc, *bsc;
    int64_t asld, bsld, asrows = BT;
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
    c0 = tile.col * BT;
    if (MODE == MODE_DGRAD) {
        int64_t t = tile.row, cum = 0, p0 = 0;
        for (int gg = 0; gg < p.G; gg++) {
            const int64_t s0 = p.offsets[gg], s1 = p.offsets[gg + 1];
            const int64_t tiles = (s1 - s0 + BT - 1) / BT;
            if (t < cum + tiles) {
                g = gg;
                r0 = s0 + (t - cum) * BT;
                p0 = p.po[gg] + (t - cum) * BT;
                rvalid = s1 - r0 < BT ? s1 - r0 : BT;
                break;
            }
            cum += tiles;
        }
        if (g < 0) return;
        klen = p.Nf;
        acode = p.a + r0 * p.lda;
        asc = p.ae + p0;
        asld = p.Pb;
        asrows = p.Pb - p0;                      // scale columns of this tile inside the array
        bcode = p.b + c0 * p.ldb + (int64_t)g * p.Nf;
        bsc = p.be + (int64_t)g * (p.Nf / 32) * p.Kf + c0;
        bsld = p.Kf;
        obase = p.out + r0 * p.Kf;
    } else {
        g = (int)batch;
        r0 = tile.row * BT;
        const int64_t kbeg = p.po[g];
        klen = p.po[g + 1] - kbeg;
        acode = p.a + r0 * p.lda + kbeg;
        asc = p.ae + (kbeg / 32) * p.Nf + r0;
        asld = p.Nf;
        bcode = p.b + c0 * p.ldb + kbeg;
        bsc = p.be + (kbeg / 32) * p.Kf + c0;
        bsld = p.Kf;
        obase = p.out + (int64_t)g * p.Nf * p.Kf + r0 * p.Kf;
    }

    // Load assignment. Wavefronts 0-3 load A, 4-7 load B. Codes: wavefront w issues the 1 KB
    // pieces 4 (w % 4) .. 4 (w % 4) + 3 of its operand (16 rows each); lane l of a piece lands at
    // row 16 n + l / 4, slot l % 4, and so fetches chunk (l % 4) ^ ((l / 16) % 4). Rows outside the
    // tile (dgrad's last tile of a group) fetch row 0 instead: their outputs are never stored.
    // Scales: wavefront w covers k-block (w / 2) % 2 of the stage, rows 128 (w % 2) .. +127, four
    // per lane over lanes 0-31.
    const int op = wave >> 2;
    const uint8_t* cbase = op ? bcode : acode;
    const int64_t cld = op ? p.ldb : p.lda;
    const int64_t crows = op ? (int64_t)BT : rvalid;
    const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
    const uint8_t* cptr[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int row = ((wave & 3) * 4 + i) * 16 + (lane >> 2);
        cptr[i] = cbase + (int64_t)(row < crows ? row : 0) * cld + chunk * 16;
    }
    const int kbsel = (wave >> 1) & 1;
    const int srow = ((wave & 1) * 32 + lane) * 4;
    const uint8_t* sbase = op ? bsc : asc;
    const int64_t sld = op ? bsld : asld;
    const int64_t srows = op ? (int64_t)BT : asrows;
    const uint8_t* sptr = sbase + (srow < srows ? srow : 0);
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);   // LDS offset
    const uint32_t cdst = lds0 + op * TILEB + (wave & 3) * 4096;
    const uint32_t sdst = lds0 + 2 * TILEB + op * SCB + kbsel * 256 + (wave & 1) * 128;

    const int64_t kblocks = klen / 32;
    const int KT = (int)((klen + BK - 1) / BK);
    const bool half_tail = (klen & (BK - 1)) != 0;   // last stage holds one k-block (wgrad)
    const int tail_back = chunk >= 2 ? 32 : 0;        // that stage's missing chunks re-read valid k

    auto issue = [&](int kt) {
        const int64_t k0 = (int64_t)kt * BK;
        const int64_t kc = (half_tail && kt == KT - 1) ? k0 - tail_back : k0;
        const uint32_t so = (uint32_t)(kt % NSTAGE) * STAGEB;
#pragma unroll
        for (int i = 0; i < 4; i++) dma16(cptr[i] + kc, cdst + so + i * 1024);
        int64_t kb = (k0 >> 5) + kbsel;
        kb = kb < kblocks ? kb : kblocks - 1;
        const uint32_t sd = sdst + so;
        if (lane < 32) dma4(sptr + kb * sld, sd);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    if (KT > 0) issue(0);
    if (KT > 1) issue(1);
    if (KT > 2) issue(2);
    const int lrow = lane & 31, hh = lane >> 5;
    const int swz = (lrow >> 2) & 3;
    const int off_lo = ((hh ^ swz) << 4), off_hi = (((2 + hh) ^ swz) << 4);
    for (int kt = 0; kt < KT; kt++) {
        // stage kt has landed once at most 5 x (stages issued after it) loads are outstanding
        const int later = KT - 1 - kt;
        if (later >= 2) wait_loads_and_barrier<2 * LOADS_PER_STAGE>();
        else if (later == 1) wait_loads_and_barrier<LOADS_PER_STAGE>();
        else wait_loads_and_barrier<0>();
        // the barrier also ends every wavefront's reads of stage kt - 1, whose slot is refilled here
        if (kt + 3 < KT) issue(kt + 3);

        const uint8_t* base = lds + (kt % NSTAGE) * STAGEB;
        const uint8_t* sca = base + 2 * TILEB + hh * BT;
        const uint8_t* scb = base + 2 * TILEB + SCB + hh * BT;
        const bool tail = half_tail && kt == KT - 1;
        i32x8 af[4], bf[2];
        int sa[4], sb[2];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = wr * 128 + i * 32 + lrow;
            const uint4 lo = *reinterpret_cast<const uint4*>(base + row * BK + off_lo);
            uint4 hi = *reinterpret_cast<const uint4*>(base + row * BK + off_hi);
            int sc = sca[row];
            if (tail) {
                hi = make_uint4(0u, 0u, 0u, 0u);
                sc = hh ? 127 : sc;
            }
            af[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            sa[i] = sc;
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int row = wc * 64 + j * 32 + lrow;
            const uint4 lo = *reinterpret_cast<const uint4*>(base + TILEB + row * BK + off_lo);
            uint4 hi = *reinterpret_cast<const uint4*>(base + TILEB + row * BK + off_hi);
            int sc = scb[row];
            if (tail) {
                hi = make_uint4(0u, 0u, 0u, 0u);
                sc = hh ? 127 : sc;
            }
            bf[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            sb[j] = sc;
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
    }

    // epilogue: block (i, j): lane holds column c = c0 + wc*64 + j*32 + lane%32 and tile rows
    // wr*128 + i*32 + (v/4)*8 + hh*4 + v%4
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = c0 + wc * 64 + j * 32 + lrow;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t rl = wr * 128 + i * 32 + (v >> 2) * 8 + hh * 4 + (v & 3);
                if (rl < rvalid) obase[rl * p.Kf + col] = acc[i][j][v];
            }
        }
}

hipError_t launch_mxfp8_dgrad(const uint8_t* dq, const uint8_t* de, const uint8_t* wt,
                              const uint8_t* wte, const int64_t* offsets, const int64_t* po,
                              int64_t Pb, int G, int64_t M, int64_t Nf, int64_t Kf, float* dx,
                              hipStream_t stream)
{
    if (M == 0 || G == 0) return hipSuccess;
    const int64_t rt = (M + bwd::BT - 1) / bwd::BT + G, ct = Kf / bwd::BT;
    int SM, SN;
    xcd_shape(rt, ct, SM, SN);
    Mx8Args p{dq, de, Nf, wt, wte, (int64_t)G * Nf, offsets, po, Pb, G, Nf, Kf, dx, rt, ct, SM, SN};
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
    Mx8Args p{dt, dte, ld, xt, xte, ld, nullptr, po, ld, G, Nf, Kf, dw, rt, ct, SM, SN};
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
