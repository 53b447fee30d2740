// gemm_bwd.hip -- MXFP8 grouped GEMMs: the expert-layer backward (dgrad, wgrad), the MXFP8
// forward of the layers that keep MXFP8, and the SwiGLU backward.
//
// Pages cited (by title and section heading):
//   [AREX] AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向传播
//          贯穿预训练到最后一次 RL rollout":
//            "只把专家层的前向传播降到 4-bit" -- the backward pass runs in MXFP8;
//            "转置打散分组,随机舍入保住期望值" -- weights and activations are re-quantized to
//              MXFP8 with stochastic rounding and the gradients use MXFP8 matmuls;
//            "配方的代价:预训练约 2% 的计算效率" -- the last 16.6% of the layers compute their
//              forward in MXFP8 rather than NVFP4.
//
// All three are D[r, c] = sum_k A[r, k] B[c, k] over E4M3 operands with one E8M0 scale per 32
// consecutive k, which is exactly the operand format of gfx950's block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3). Its lane layout, measured on the device:
// lane l supplies row l % 32; with h = l / 32 its bytes 0..15 are k = 16h .. 16h+15 and bytes
// 16..31 are k = 32+16h .. 32+16h+15 of the 64-k step, and its scale operand is the E8M0 scale
// of k-block h of that row (k-block b of the step = k in [32b, 32b+32)).
//
// Tiling: 256 x 256 output tile per workgroup of 4 wavefronts, one per SIMD, each computing a
// 128 x 128 quarter (4 x 4 MFMA blocks, accumulators in AGPRs). Operands stream through a ring
// of 4 LDS stages of 64 k (one MFMA k-step) filled by global_load_lds (global -> LDS without
// registers). A wavefront reads the fragments of stage kt + 1 from LDS while the MFMAs of stage
// kt run from registers, so the matrix cores never wait for LDS after a barrier; three further
// stages are in flight. Every wavefront issues the same 9 loads per stage (8 x 1 KB of codes,
// 1 x 256 B of scales), so "stage s has landed" is the per-wave condition vmcnt <= 9 x (stages
// issued after s), followed by a barrier.
//
// LDS stage: A codes [256 rows x 64 B], B codes [256 x 64 B], A scales [2 k-blocks x 256 rows],
// B scales [2 x 256]. Chunk c (16 B) of row r sits at slot c ^ ((r / 4) % 4): the 16 rows a
// quarter-wavefront reads cover all 16 bank groups. The operands arrive in that order: the
// quantizers write them in 1 KB blocks of 16 rows x 64 bytes with the same permutation (the
// blocked layout), so every copy moves one whole contiguous block. Scales are streamed from
// k-block-major arrays, so one k-block of 256 rows is 256 contiguous bytes.
#include <type_traits>

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
constexpr int THREADS = 256;            // 4 wavefronts: 2 along output rows x 2 along columns
constexpr int LOADS_PER_STAGE = 9;      // per wavefront
static_assert(THREADS == 256 && BT == 256 && BK == 64 && NSTAGE == 4, "the load schedule below assumes these");
}  // namespace bwd

enum { MODE_DGRAD = 0, MODE_WGRAD = 1, MODE_FWD = 2 };

struct Mx8Args {
    // dgrad: A = dY row-wise codes [M x Nf] (lda = Nf) with scales de [Nf/32 x Pb] at padded slot
    //        columns; B = W^T codes [Kf x G*Nf] (ldb = G*Nf, group g at column g*Nf) with scales
    //        [G*Nf/32 x Kf]; contraction Nf, output dX [M x Kf].
    // wgrad: A = dY^T [Nf x Pb], B = X^T [Kf x Pb] (lda = ldb = Pb), scales [Pb/32 x Nf] and
    //        [Pb/32 x Kf]; contraction over the padded slots of group g (po[g] .. po[g+1]),
    //        output dW [G*Nf x Kf].
    // fwd:   computes Y^T = W X^T so that a lane holds one slot and 16 output features. A = W
    //        codes [G*Kf x Nf] (lda = Nf; expert g in rows g*Kf ..) with scales [Nf/32 x G*Kf];
    //        B = X in slot order [M x Nf] (ldb = Nf) with scales [Nf/32 x Pb] at padded slot
    //        columns; contraction Nf, output Y [M x Kf] through the epilogue. With the SwiGLU
    //        epilogue (Kf = 2F) a tile's 256 A rows are 128 features of w1 and the same 128 of w3,
    //        arranged so that blocks i and i + 2 of a wavefront pair h1 and h3.
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
    int64_t rtiles, ctiles;   // tile grid (dgrad: slot-tile bound x Kf/256; wgrad: Nf/256 x Kf/256;
                              // fwd: Kf/256 x slot-tile bound)
    int SM, SN;
    // fwd epilogue outputs: Y (fp32 / bf16 / A of SwiGLU / S2F6 codes), E8M0 of the codes, h13
    void* yout;
    uint8_t* ye8m0;
    void* yaux;
    uint32_t mask;
    // dgrad: B columns per expert (Nf rounded up to whole stages, so that every expert's columns
    // start on a block column)
    int64_t gstride;
};

// MFMA operands of one k-step for a wavefront's 128 x 128 quarter
struct Mx8Frags {
    i32x8 a[4], b[4];
    int sa[4], sb[4];
};
// FP4 (E2M1) operands of one 64-byte stage = two k-steps of 64 values: an E2M1 operand of the
// block-scaled MFMA is 4 registers (the upper half of the 8-register operand is left undefined)
struct Mx4Frags {
    i32x8 a[4], b[4], a2[4], b2[4];
    int sa[4], sb[4], sa2[4], sb2[4];
};
template <bool FP4> struct FragsOf { typedef Mx8Frags type; };
template <> struct FragsOf<true> { typedef Mx4Frags type; };

PMN_DEV i32x8 lo4(uint4 x)
{
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 v = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
    return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

// FP4: the operands are E2M1 codes packed two per byte (k even in the low nibble), lda / ldb in
// bytes; a stage is still 64 bytes per row, now 128 values = 4 k-blocks = two MFMA k-steps, and
// each loading wavefront streams two scale lines per stage.
template <int MODE, int EPI = PMN_EPI_F32, bool FP4 = false>
__global__ __launch_bounds__(bwd::THREADS, 1) void k_mxfp8_grouped_gemm(Mx8Args p)
{
    using namespace bwd;
    static_assert(!(FP4 && MODE == MODE_FWD), "the FP4 operand format is used by the backward only");
    constexpr int SCBk = FP4 ? 4 * BT : SCB;        // one operand's scales per stage
    constexpr int STAGEBk = 2 * TILEB + 2 * SCBk;
    constexpr int LDSBk = NSTAGE * STAGEBk;
    constexpr int LPS = FP4 ? LOADS_PER_STAGE + 1 : LOADS_PER_STAGE;
    constexpr int KS = FP4 ? 2 * BK : BK;           // values (k) per stage
    typedef typename FragsOf<FP4>::type Frags;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDSBk];
    // An AGPR operand marks the kernel as using AGPRs, so the compiler keeps the 256 accumulator
    // registers in AGPRs (MFMA accumulator form) instead of arch VGPRs.
    asm volatile("; agpr in use %0" ::"a"(0));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave >> 1, wc = wave & 1;    // 2 wavefronts along output rows, 2 along columns

    int g = -1;
    int64_t r0 = 0, rvalid = BT, c0 = 0, klen = 0, cvalid = BT;
    // operands in the blocked layout: acode / bcode point at block column 0 of the tile's k range,
    // arb0 / brb0 are the tile's first row blocks
    const uint8_t *acode, *bcode, *asc, *bsc;
    int64_t arb0 = 0, brb0 = 0;
    int64_t asld, bsld, asrows = BT, bsrows = BT;
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
    if (MODE == MODE_FWD) {
        const GroupUnit u = locate_group_unit(p.offsets, p.G, tile.col, BT);
        if (u.g < 0) return;
        g = u.g;
        c0 = u.s0 + u.index * BT;                // first slot of the tile
        const int64_t p0 = p.po[g] + u.index * BT;
        cvalid = u.s1 - c0 < BT ? u.s1 - c0 : BT;
        klen = p.Nf;
        r0 = tile.row * BT;                      // first feature row (plain order)
        if (EPI != PMN_EPI_SWIGLU) {
            // the last feature tile of an N that is not a multiple of 256: rows past it re-read
            // the tile's first block (their outputs are not stored)
            rvalid = p.Kf - r0 < BT ? p.Kf - r0 : BT;
            asrows = rvalid;
        }
        const int64_t wrow0 = (int64_t)g * p.Kf + (EPI == PMN_EPI_SWIGLU ? 0 : r0);
        acode = p.a;
        arb0 = wrow0 >> 4;                       // (the SwiGLU tile maps each piece itself)
        asc = p.ae + wrow0;
        asld = (int64_t)p.G * p.Kf;
        bcode = p.b;
        brb0 = p0 >> 4;                          // slot rows sit at their padded positions
        bsc = p.be + p0;
        bsld = p.Pb;
        bsrows = p.Pb - p0;
        obase = nullptr;
    } else if (MODE == MODE_DGRAD) {
        const GroupUnit u = locate_group_unit(p.offsets, p.G, tile.row, BT);
        if (u.g < 0) return;
        g = u.g;
        r0 = u.s0 + u.index * BT;
        const int64_t p0 = p.po[g] + u.index * BT;
        rvalid = u.s1 - r0 < BT ? u.s1 - r0 : BT;
        klen = p.Nf;
        acode = p.a;
        arb0 = p0 >> 4;                          // slot rows sit at their padded positions
        asc = p.ae + p0;
        asld = p.Pb;
        asrows = p.Pb - p0;                      // scale columns of this tile inside the array
        bcode = p.b + (int64_t)g * ((FP4 ? p.gstride / 2 : p.gstride) >> 6) * 1024;   // expert g's columns
        brb0 = c0 >> 4;
        bsc = p.be + (int64_t)g * (p.gstride / 32) * p.Kf + c0;
        bsld = p.Kf;
        // the last column tile of a K that is not a multiple of 256
        cvalid = p.Kf - c0 < BT ? p.Kf - c0 : BT;
        bsrows = cvalid;
        obase = p.out + r0 * p.Kf;
    } else {
        g = (int)batch;
        r0 = tile.row * BT;
        const int64_t kbeg = p.po[g];
        klen = p.po[g + 1] - kbeg;
        const int64_t kbyte = FP4 ? kbeg / 2 : kbeg;   // first code byte of the group in a row
        acode = p.a + (kbyte >> 6) * 1024;
        arb0 = r0 >> 4;
        asc = p.ae + (kbeg / 32) * p.Nf + r0;
        asld = p.Nf;
        bcode = p.b + (kbyte >> 6) * 1024;
        brb0 = c0 >> 4;
        bsc = p.be + (kbeg / 32) * p.Kf + c0;
        bsld = p.Kf;
        // the last row / column tiles of an N / K that is not a multiple of 256
        rvalid = p.Nf - r0 < BT ? p.Nf - r0 : BT;
        asrows = rvalid;
        cvalid = p.Kf - c0 < BT ? p.Kf - c0 : BT;
        bsrows = cvalid;
        obase = p.out + (int64_t)g * p.Nf * p.Kf + r0 * p.Kf;
    }

    // Load schedule. Wavefronts 0-1 load A, 2-3 load B. Codes: wavefront w issues the 1 KB
    // pieces 8 (w % 2) .. 8 (w % 2) + 7 of its operand (16 rows each). A piece of a stage is one
    // block of the blocked operand layout, copied whole (lane l moves its bytes 16 l .. 16 l + 15),
    // so it lands in the order the fragment reads expect. Pieces past the tile's valid rows (the
    // last tile of a group) re-read the tile's first block: their outputs are never stored.
    // Scales: wavefront w loads k-block w % 2 of the stage, rows 4 l .. 4 l + 3 in lane l.
    const int op = wave >> 1, half = wave & 1;
    const uint8_t* cbase = op ? bcode : acode;
    const int64_t crb0 = op ? brb0 : arb0;
    const int64_t cld = ((op ? p.ldb : p.lda) >> 6) * 1024;   // bytes per row block (ld / 64 blocks)
    const int crows = (int)(op ? cvalid : rvalid);
    const uint8_t* sbase = op ? bsc : asc;
    const int64_t sld = op ? bsld : asld;
    const int64_t srows = op ? bsrows : asrows;
    // the forward's SwiGLU tile takes its A rows (w1 and w3 features) through swiglu_a_row
    const bool remap = MODE == MODE_FWD && EPI == PMN_EPI_SWIGLU && op == 0;
    const int64_t Fh = p.Kf >> 1;
    const uint8_t* sptr = sbase + (remap ? swiglu_a_row_clamped(4 * lane, tile.row, Fh) : (4 * lane < srows ? 4 * lane : 0));
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);   // LDS offset
    const uint32_t cdst = lds0 + op * TILEB + half * 8192;
    const uint32_t sdst = lds0 + 2 * TILEB + op * SCBk + half * (FP4 ? 2 : 1) * BT;

    const int64_t kblocks = klen / 32;
    const int KT = (int)((klen + KS - 1) / KS);
    // last stage holds one k-block (the forward with K = 32 mod 64; the other half of its block
    // column holds zero codes)
    const bool half_tail = (klen & (BK - 1)) != 0;

    // Steps v = 0 .. KV-1 walk the stages; when KT is odd a leading step (v = 0) re-reads stage 0
    // with every scale forced to 2^-127 on both operands, so it adds nothing and the step count
    // is even. Step v multiplies stage v - pre and uses LDS slot v % NSTAGE.
    const int pre = KT & 1;
    const int KV = KT + pre;
    auto stage_of = [&](int v) { const int st = v - pre; return st < 0 ? 0 : (st < KT ? st : KT - 1); };
    // the loads of step v: 8 code pieces and one scale line
    struct IssueAt {
        int64_t kc, kb, kb2;
        uint32_t so;
    };
    auto issue_at = [&](int v) {
        const int kt = stage_of(v);
        IssueAt r;
        // stage kt of a piece is block column kt; this lane's 16 bytes of it
        r.kc = (int64_t)kt * 1024 + lane * 16;
        if (FP4) {
            // FP4: k-blocks 4 kt .. 4 kt + 3 (every k length is a multiple of 128)
            r.kb = 4 * (int64_t)kt + 2 * half;
            r.kb2 = r.kb + 1 < kblocks ? r.kb + 1 : kblocks - 1;
            r.kb = r.kb < kblocks ? r.kb : kblocks - 1;
        } else {
            r.kb = 2 * (int64_t)kt + half;
            r.kb = r.kb < kblocks ? r.kb : kblocks - 1;
            r.kb2 = 0;
        }
        r.so = (uint32_t)(v % NSTAGE) * STAGEBk;
        return r;
    };
    auto issue_piece = [&](const IssueAt& r, int i) {
        // row block of piece pb = half * 8 + i: the SwiGLU tile's A rows come from w1 and w3 in
        // 32-row runs, so each 16-row piece is still one block
        const int pb = half * 8 + i;
        const int64_t rb = remap ? (((int64_t)g * p.Kf + swiglu_a_row_clamped(16 * pb, tile.row, Fh)) >> 4)
                                 : crb0 + (16 * pb < crows ? pb : 0);
        dma16(cbase + rb * cld + r.kc, cdst + r.so + i * 1024);
    };
    auto issue_scales = [&](const IssueAt& r) { dma4(sptr + r.kb * sld, sdst + r.so); };
    auto issue_scales2 = [&](const IssueAt& r) { dma4(sptr + r.kb2 * sld, sdst + r.so + BT); };
    auto issue = [&](int v) {
        const IssueAt r = issue_at(v);
#pragma unroll
        for (int i = 0; i < 8; i++) issue_piece(r, i);
        issue_scales(r);
        if (FP4) issue_scales2(r);
    };

    const int lrow = lane & 31, hh = lane >> 5;
    const int swz = (lrow >> 2) & 3;
    const int off_lo = ((hh ^ swz) << 4), off_hi = (((2 + hh) ^ swz) << 4);
    // Fragments of step v: lane l supplies row l % 32 of each 32-row block with bytes 0..15 =
    // k 16h .. 16h+15 and bytes 16..31 = k 32+16h .. (h = l / 32), and the scale of k-block h.
    // A half-full last stage (the forward with K = 32 mod 64) holds zero codes in k-block 1, and
    // both operands also give it the E8M0 scale 2^-127; the whole leading step is scaled by
    // 2^-254 the same way, so its products vanish in fp32.
    auto frag_mask = [&](int v) {
        const int kt = v - pre;
        return (kt < 0 || (half_tail && kt == KT - 1 && hh)) ? 0 : 0xFF;
    };
    // FP4: k-step s of stage kt uses k-block 4 kt + 2 s + hh
    auto frag_mask4 = [&](int v, int s) {
        const int kt = v - pre;
        return (kt < 0 || 4 * (int64_t)kt + 2 * s + hh >= kblocks) ? 0 : 0xFF;
    };
    // (the scale mask is applied when the MFMA is issued, one step after the read: applying it at
    // the read would make the wavefront wait for the LDS byte right away)
    auto read_frag = [&](const uint8_t* base, int opb, int row, i32x8& f, int& sc) {
        const uint4 lo = *reinterpret_cast<const uint4*>(base + opb * TILEB + row * BK + off_lo);
        const uint4 hi = *reinterpret_cast<const uint4*>(base + opb * TILEB + row * BK + off_hi);
        sc = (int)base[2 * TILEB + opb * SCBk + hh * BT + row];
        f = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    // FP4: chunk hh is k-block hh of k-step 0 and chunk 2 + hh is k-block hh of k-step 1
    auto read_frag4 = [&](const uint8_t* base, int opb, int row, i32x8& f0, i32x8& f1, int& s0, int& s1) {
        f0 = lo4(*reinterpret_cast<const uint4*>(base + opb * TILEB + row * BK + off_lo));
        f1 = lo4(*reinterpret_cast<const uint4*>(base + opb * TILEB + row * BK + off_hi));
        s0 = (int)base[2 * TILEB + opb * SCBk + hh * BT + row];
        s1 = (int)base[2 * TILEB + opb * SCBk + (2 + hh) * BT + row];
    };
    auto read_a = [&](const uint8_t* base, int i, Frags& f) {
        if constexpr (FP4) read_frag4(base, 0, wr * 128 + i * 32 + lrow, f.a[i], f.a2[i], f.sa[i], f.sa2[i]);
        else read_frag(base, 0, wr * 128 + i * 32 + lrow, f.a[i], f.sa[i]);
    };
    auto read_b = [&](const uint8_t* base, int j, Frags& f) {
        if constexpr (FP4) read_frag4(base, 1, wc * 128 + j * 32 + lrow, f.b[j], f.b2[j], f.sb[j], f.sb2[j]);
        else read_frag(base, 1, wc * 128 + j * 32 + lrow, f.b[j], f.sb[j]);
    };
    auto read_frags = [&](int v, Frags& f) {
        const uint8_t* base = lds + (v % NSTAGE) * STAGEBk;
#pragma unroll
        for (int i = 0; i < 4; i++) read_a(base, i, f);
#pragma unroll
        for (int j = 0; j < 4; j++) read_b(base, j, f);
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    // One step: once slot v + 1 has landed (and every wavefront is done reading slot v, which is
    // refilled), read its fragments while the MFMAs of step v (already in registers) run. With
    // one wavefront per SIMD the wavefront itself must keep the matrix core fed, so each of the
    // 16 MFMAs is followed by one piece of the next step's work (a load or a fragment read) and
    // the compiler may not regroup them. Every step is identical: the refill loads step
    // min(v + 4, KV - 1) (near the end this re-loads the last stage, into a free slot or over
    // identical bytes) and the fragment read re-reads the last step once past it, so each step
    // waits for exactly two younger slots and no value is live only on some paths.
    auto step = [&](int v, const Frags& cur, Frags& nxt) {
        wait_loads_and_barrier<2 * LPS>();
        const IssueAt r = issue_at(v + NSTAGE < KV ? v + NSTAGE : KV - 1);
        const int vr = v + 1 < KV ? v + 1 : v;
        const uint8_t* rbase = lds + (vr % NSTAGE) * STAGEBk;
        if constexpr (FP4) {
            // k-step 0 of all 16 blocks, then k-step 1: an accumulator's two MFMAs are 16 apart
            const int m0 = frag_mask4(v, 0), m1 = frag_mask4(v, 1);
            int sa[4], sb[4], sa2[4], sb2[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                sa[i] = cur.sa[i] & m0;
                sb[i] = cur.sb[i] & m0;
                sa2[i] = cur.sa2[i] & m1;
                sb2[i] = cur.sb2[i] & m1;
            }
#pragma unroll
            for (int q = 0; q < 32; q++) {
                const int i = (q >> 2) & 3, j = q & 3;
                if (q < 16)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.a[i], cur.b[j], acc[i][j], 4, 4, 0,
                                                                               sa[i], 0, sb[j]);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.a2[i], cur.b2[j], acc[i][j], 4, 4,
                                                                               0, sa2[i], 0, sb2[j]);
                if (q < 8) issue_piece(r, q);
                if (q == 8) issue_scales(r);
                if (q == 9) issue_scales2(r);
                if (q >= 16 && q < 20) read_a(rbase, q - 16, nxt);
                if (q >= 20 && q < 24) read_b(rbase, q - 20, nxt);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            const int smask = frag_mask(v);
            int sa[4], sb[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                sa[i] = cur.sa[i] & smask;
                sb[i] = cur.sb[i] & smask;
            }
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int i = q >> 2, j = q & 3;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0,
                                                                           sa[i], 0, sb[j]);
                if (q < 8) issue_piece(r, q);
                if (q == 8) issue_scales(r);
                if (q >= 8 && q < 12) read_frag(rbase, 0, wr * 128 + (q - 8) * 32 + lrow, nxt.a[q - 8], nxt.sa[q - 8]);
                if (q >= 12) read_frag(rbase, 1, wc * 128 + (q - 12) * 32 + lrow, nxt.b[q - 12], nxt.sb[q - 12]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if (KT > 0) {
#pragma unroll
        for (int v = 0; v < NSTAGE; v++) issue(v < KV ? v : KV - 1);
        Frags f0, f1;
        wait_loads_and_barrier<3 * LPS>();
        read_frags(0, f0);
        for (int v = 0; v < KV; v += 2) {
            step(v, f0, f1);
            step(v + 1, f1, f0);
        }
        // no LDS copy may still be in flight when the workgroup's LDS is released
        wait_loads_and_barrier<0>();
    }

    if (MODE == MODE_FWD) {
        // Y^T tile: block (i, j) of this wavefront holds, in lane l, slot c0 + wc*128 + j*32 + l%32
        // and the 16 feature rows wr*128 + i*32 + (v/4)*8 + (l/32)*4 + v%4 of the tile.
        const int64_t Nout = p.Kf;
        if (EPI == PMN_EPI_F32 || EPI == PMN_EPI_BF16) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int sl = wc * 128 + j * 32 + lrow;
                if (sl < cvalid) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        if (r0 + wr * 128 + i * 32 >= Nout) continue;   // past the expert's N
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const int64_t n = r0 + wr * 128 + i * 32 + q * 8 + hh * 4;
                            const int64_t o = (c0 + sl) * Nout + n;
                            if (EPI == PMN_EPI_F32) {
                                *reinterpret_cast<float4*>(static_cast<float*>(p.yout) + o) =
                                    make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                                acc[i][j][4 * q + 3]);
                            } else {
                                const uint32_t lo = bf16x2_bits(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                                const uint32_t hi = bf16x2_bits(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.yout) + o) = make_uint2(lo, hi);
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
        // SwiGLU and RHT32 + S2F6 stage a 256-slot output tile of 256 bytes per slot in LDS and
        // write whole 16-byte pieces of each slot's row
        constexpr int OPITCH = 272;                 // bytes per slot row: conflict-free 8-byte writes
        uint8_t* const t0 = lds;
        uint8_t* const te = lds + BT * OPITCH;      // E8M0 tile: 8 bytes per slot
        // piece c (16 bytes) of a slot's row is stored if pvalid(c): it lies inside the expert's N
        auto store_tile = [&](uint8_t* dst, int64_t pitch, auto pvalid) {
#pragma unroll
            for (int k = 0; k < (BT * 16) / THREADS; k++) {
                const int q = k * THREADS + tid;
                const int row = q >> 4, c = q & 15;
                if (row < cvalid && pvalid(c))
                    *reinterpret_cast<uint4*>(dst + (c0 + row) * pitch + c * 16) =
                        *reinterpret_cast<const uint4*>(t0 + row * OPITCH + c * 16);
            }
        };
        if (EPI == PMN_EPI_SWIGLU) {
            // blocks i = 0, 1 hold h1 and i + 2 the matching h3 of features n0 + wr*64 + i*32 + ..
            const int64_t F = Nout >> 1, n0 = tile.row * 128;
            uint8_t* const A = static_cast<uint8_t*>(p.yout);
            uint8_t* const Hs = static_cast<uint8_t*>(p.yaux);
#pragma unroll
            for (int phase = 0; phase < 3; phase++) {
                if (phase > 0 && !Hs) break;
                if (phase > 0) __syncthreads();     // the previous phase's tile has been stored
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int sl = wc * 128 + j * 32 + lrow;
#pragma unroll
                    for (int i = 0; i < 2; i++) {
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            float o[4];
#pragma unroll
                            for (int u = 0; u < 4; u++) {
                                const float h1 = acc[i][j][4 * q + u], h3 = acc[i + 2][j][4 * q + u];
                                o[u] = phase == 0 ? silu(h1) * h3 : (phase == 1 ? h1 : h3);
                            }
                            const int off = sl * OPITCH + 2 * (wr * 64 + i * 32 + q * 8 + hh * 4);
                            *reinterpret_cast<uint2*>(t0 + off) = make_uint2(bf16x2_bits(o[0], o[1]), bf16x2_bits(o[2], o[3]));
                        }
                        // one block pair at a time: the accumulators stay in AGPRs until used
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                __syncthreads();
                auto fvalid = [&](int c) { return n0 + c * 8 < F; };   // 8 features per piece
                if (phase == 0) store_tile(A + n0 * 2, F * 2, fvalid);
                else if (phase == 1) store_tile(Hs + n0 * 2, Nout * 2, fvalid);
                else store_tile(Hs + (F + n0) * 2, Nout * 2, fvalid);
            }
        } else {
            // RHT32 + S2F6: each block's 32 feature rows are one aligned chunk of the slot's row
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int sl = wc * 128 + j * 32 + lrow;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int nl = wr * 128 + i * 32;
                    rht_block_store(acc[i][j], p.mask, lane, reinterpret_cast<int8_t*>(t0 + sl * OPITCH + nl),
                                    te + sl * 8 + (nl >> 5));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __syncthreads();
            store_tile(static_cast<uint8_t*>(p.yout) + r0, Nout, [&](int c) { return r0 + c * 16 < Nout; });
            if (tid < cvalid) {
                // the tile's 8 chunk scales; an N that is not a multiple of 256 has fewer in its
                // last tile, and its rows of scales are then not 8-byte aligned
                uint8_t* const d = p.ye8m0 + (c0 + tid) * (Nout >> 5) + (r0 >> 5);
                if ((Nout & 255) == 0) {
                    *reinterpret_cast<uint2*>(d) = *reinterpret_cast<const uint2*>(te + tid * 8);
                } else {
                    const int64_t nc = (Nout - r0) >> 5;
#pragma unroll
                    for (int c = 0; c < 8; c++)
                        if (c < nc) d[c] = te[tid * 8 + c];
                }
            }
        }
        return;
    }

    // epilogue: block (i, j): lane holds column c = c0 + wc*128 + j*32 + lane%32 and tile rows
    // wr*128 + i*32 + (v/4)*8 + hh*4 + v%4. Stores are nontemporal: the fp32 gradients are not
    // read again by this pass, and streaming them past the caches measured faster. A whole tile
    // (every tile of the pages' shapes but the last slot tile of each expert in dgrad) stores
    // without per-value checks.
    auto store_blocks = [&](auto masked) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int64_t col = c0 + wc * 128 + j * 32 + lrow;
                const bool cok = col < p.Kf;        // a K that is not a multiple of 256
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int64_t rl = wr * 128 + i * 32 + (v >> 2) * 8 + hh * 4 + (v & 3);
                    if (!decltype(masked)::value || (cok && rl < rvalid))
                        __builtin_nontemporal_store(acc[i][j][v], obase + rl * p.Kf + col);
                }
                // one block at a time: keeps the accumulators in AGPRs until they are stored
                __builtin_amdgcn_sched_barrier(0);
            }
    };
    if (rvalid == BT && cvalid == BT)
        store_blocks(std::integral_constant<bool, false>());
    else
        store_blocks(std::integral_constant<bool, true>());
}

hipError_t launch_mxfp8_dgrad(const uint8_t* dq, const uint8_t* de, const uint8_t* wt,
                              const uint8_t* wte, const int64_t* offsets, const int64_t* po,
                              int64_t Pb, int G, int64_t M, int64_t Nf, int64_t Kf, float* dx,
                              hipStream_t stream, bool fp4, int64_t Nk)
{
    if (M == 0 || G == 0) return hipSuccess;
    const int64_t rt = (M + bwd::BT - 1) / bwd::BT + G, ct = (Kf + bwd::BT - 1) / bwd::BT;
    int SM, SN;
    xcd_shape(rt, ct, SM, SN);
    const int64_t bpv = fp4 ? 2 : 1;   // values per byte
    // dY rows and each expert's W^T columns are Nk (Nf rounded up to whole stages) wide
    Mx8Args p{dq, de, Nk / bpv, wt, wte, (int64_t)G * Nk / bpv, offsets, po, Pb, G, Nf, Kf, dx, rt, ct, SM, SN,
              nullptr, nullptr, nullptr, 0u, Nk};
    dim3 grid((unsigned)xcd_grid(rt, ct, SM, SN));
    if (fp4)
        hipLaunchKernelGGL((k_mxfp8_grouped_gemm<MODE_DGRAD, PMN_EPI_F32, true>), grid, dim3(bwd::THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((k_mxfp8_grouped_gemm<MODE_DGRAD>), grid, dim3(bwd::THREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mxfp8_fwd(const uint8_t* wq, const uint8_t* we, const uint8_t* xq, const uint8_t* xe,
                            const int64_t* offsets, const int64_t* po, int64_t Pb, int G, int64_t M, int64_t N,
                            int64_t K, int epilogue, uint32_t mask, void* out, uint8_t* out_e8m0, void* out_aux,
                            hipStream_t stream)
{
    if (M == 0 || G == 0) return hipSuccess;
    // a feature tile is 256 rows of one expert (SwiGLU: 128 features of w1 and the same of w3)
    const int64_t rt = epilogue == PMN_EPI_SWIGLU ? (N / 2 + 127) / 128 : (N + bwd::BT - 1) / bwd::BT;
    const int64_t ct = (M + bwd::BT - 1) / bwd::BT + G;
    int SM, SN;
    xcd_shape(rt, ct, SM, SN);
    const int64_t Kp = (K + 63) & ~(int64_t)63;   // blocked rows: K rounded up to whole 64-byte blocks
    Mx8Args p{wq, we, Kp, xq, xe, Kp, offsets, po, Pb, G, K, N, nullptr, rt, ct, SM, SN, out, out_e8m0, out_aux, mask};
    dim3 grid((unsigned)xcd_grid(rt, ct, SM, SN));
    switch (epilogue) {
    case PMN_EPI_F32:
        hipLaunchKernelGGL((k_mxfp8_grouped_gemm<MODE_FWD, PMN_EPI_F32>), grid, dim3(bwd::THREADS), 0, stream, p);
        break;
    case PMN_EPI_BF16:
        hipLaunchKernelGGL((k_mxfp8_grouped_gemm<MODE_FWD, PMN_EPI_BF16>), grid, dim3(bwd::THREADS), 0, stream, p);
        break;
    case PMN_EPI_SWIGLU:
        hipLaunchKernelGGL((k_mxfp8_grouped_gemm<MODE_FWD, PMN_EPI_SWIGLU>), grid, dim3(bwd::THREADS), 0, stream, p);
        break;
    default:
        hipLaunchKernelGGL((k_mxfp8_grouped_gemm<MODE_FWD, PMN_EPI_RHT32_S2F6>), grid, dim3(bwd::THREADS), 0, stream,
                           p);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_mxfp8_wgrad(const uint8_t* dt, const uint8_t* dte, const uint8_t* xt,
                              const uint8_t* xte, int64_t ld, const int64_t* po, int G,
                              int64_t Nf, int64_t Kf, float* dw, hipStream_t stream, bool fp4)
{
    if (G == 0) return hipSuccess;
    const int64_t rt = (Nf + bwd::BT - 1) / bwd::BT, ct = (Kf + bwd::BT - 1) / bwd::BT;
    int SM, SN;
    xcd_shape(rt, ct, SM, SN);
    const int64_t ldb = fp4 ? ld / 2 : ld;   // code bytes per row
    Mx8Args p{dt, dte, ldb, xt, xte, ldb, nullptr, po, ld, G, Nf, Kf, dw, rt, ct, SM, SN, nullptr, nullptr, nullptr, 0u};
    dim3 grid((unsigned)xcd_grid(rt, ct, SM, SN, G));
    if (fp4)
        hipLaunchKernelGGL((k_mxfp8_grouped_gemm<MODE_WGRAD, PMN_EPI_F32, true>), grid, dim3(bwd::THREADS), 0, stream, p);
    else
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
        for (int u = 0; u < 2; u++)
            swiglu_bwd_elem(d[2 * q + u], u ? bf16_hi(a1[q]) : bf16_lo(a1[q]), u ? bf16_hi(a3[q]) : bf16_lo(a3[q]),
                            r1[u], r3[u]);
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
