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
// Tiling. A workgroup of 4 wavefronts (one per SIMD) computes a 256 (weight rows n) x 256
// (slots m) tile of D = W X^T, i.e. Y^T; each wavefront computes a 128 x 128 quarter (4 x 4 MFMA
// blocks, accumulators in AGPRs). A stage is 128 k: 64 code bytes plus 8 E4M3 scale bytes per
// row. Stages stream into a ring of 3 LDS slots with global_load_lds (global -> LDS without
// registers), so the LDS holds FP4 codes rather than fp16 values: a fragment read moves a quarter
// of the bytes of an fp16 fragment. Each wavefront dequantizes its own fragments in registers,
// half a fragment after each MFMA, one substep (16 k) ahead of the MFMAs that use it.
//
// Fragment k order. Within a stage, lane half h (lanes 32h .. 32h+31) takes the 64 values
// 64h .. 64h+63 of its row: substep s (0..7) feeds the MFMA the values 64h + 8s .. 64h + 8s + 7,
// i.e. dword s of the lane's 32 code bytes, scaled by its block scale s / 2. Both operands use
// the same order, so every MFMA multiplies matching k; only the fp32 summation order differs
// from a k-sequential one.
//
// Code layout in a stage slot: the weight rows, then the slot rows, then their scale bytes (8 per
// row). Row r of an operand's region holds its 64 code bytes at 64 r, 16-byte chunk c at position
// c ^ ((r / 4) % 4), so the 16 rows a quarter-wavefront reads cover all 16 bank groups. Each copy
// lane fetches the chunk its destination position needs, so plain row-major codes arrive permuted.
//
// Groups (experts) are ragged: a workgroup finds its (expert, slot tile) from the device offsets
// with one wavefront-parallel search, so no host synchronization is needed. An expert's last
// unit of at most 128 slots runs as 512 weight rows x 128 slots (two weight tiles), so fewer
// MFMAs fall on padded slots.
#include <type_traits>

#include "pmn_dev.hpp"
#include "pmn_kernels.hpp"

namespace pmn {

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

namespace fwd {
constexpr int BT = 256;
constexpr int KS = 128;                       // k per stage
constexpr int NSTAGE = 3;
constexpr int ROWS_MAX = 640;                 // weight + slot rows of a stage (the 512 x 128 shape)
// Per row and stage: 64 code bytes, then the 8 E4M3 scale bytes, copied as two 4-byte words
// (8 LDS bytes) or, when K = 32 mod 64 leaves rows of scales only 2-byte aligned (SC2), as four
// 2-byte pieces that each land in the low half of a 4-byte LDS word (16 LDS bytes).
constexpr int srow_bytes(bool sc2) { return sc2 ? 16 : 8; }
constexpr int stage_bytes(bool sc2) { return ROWS_MAX * (64 + srow_bytes(sc2)); }
constexpr int lds_bytes(bool sc2) { return NSTAGE * stage_bytes(sc2); }
constexpr int THREADS = 256;
constexpr int OPITCH = 272;
static_assert(BT * OPITCH + BT * 8 <= lds_bytes(false), "the epilogue's output tile and E8M0 tile fit in the ring");
static_assert(lds_bytes(true) <= 160 * 1024, "the 2-byte scale layout fits the LDS");
}  // namespace fwd

// One workgroup tile. SHAPE false: 256 weight rows x 256 slots, wavefront w computes weight rows
// (w / 2) * 128 .. and slots (w % 2) * 128 ... SHAPE true (the last unit of an expert's slots
// when it holds at most 128 of them): 512 weight rows (weight tiles nt0 and nt0 + 1) x 128 slots,
// wavefront w computes weight rows w * 128 .. and all 128 slots. Each wavefront's work (a
// 128 x 128 quarter) and inner loop are the same in both. SC2: scales copied as 2-byte pieces
// (K = 32 mod 64).
//
// Edges. N (weight rows per expert; 2F for SwiGLU) need only be a multiple of 32 (64 for
// SwiGLU): weight rows past the expert's last re-read one of its first 32 rows, and the outputs
// of those rows are never stored. K need only be a multiple of 32: the last stage may hold 32,
// 64 or 96 valid k; its other 32-k chunks re-read the stage's first chunk and their block scales
// are forced to zero, so they add nothing.
template <int EPI, bool SHAPE, bool SC2>
PMN_DEV void nvfp4_gemm_tile(const FwdArgs& p, uint8_t* lds, int g, int64_t m0, int mvalid, int64_t nt0)
{
    using namespace fwd;
    constexpr int SROW = srow_bytes(SC2);                    // LDS bytes of a row's scales per stage
    constexpr int STAGEB = stage_bytes(SC2);
    constexpr int RW = SHAPE ? 512 : 256, RX = SHAPE ? 128 : 256;   // weight and slot rows
    constexpr int XOFF = RW * 64, SOFF = (RW + RX) * 64, XSOFF = SOFF + RW * SROW;   // stage layout
    constexpr int RL = SC2 ? 16 : 32;                        // rows per scale line
    constexpr int NLW = 128 / RL;                            // scale lines of 128 rows
    constexpr int NP = SHAPE ? 10 : 8, NL = SHAPE ? NLW + 32 / RL : NLW;   // code pieces, scale lines per wavefront
    constexpr int LPS = NP + NL;                             // copies per wavefront per stage
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t N = p.N, K = p.K;
    const int64_t cbytes = K >> 1, sbytes = K >> 4;
    const int KT = (int)((K + KS - 1) / KS);
    const int tailv = (int)(K % KS);             // valid k of the last stage (0: a full stage)

    // ---- copy schedule. Code piece = 16 rows (lane l: row l / 4, position l % 4), scale line =
    // 32 rows (lane l: row l / 2, dword l % 2) or, with SC2, 16 rows (lane l: row l / 4, 2-byte
    // piece l % 4). SHAPE false: wavefronts 0-1 copy weight rows, 2-3 slot rows, 128 rows each
    // (8 pieces, NLW lines). SHAPE true: wavefront w copies weight rows 128 w .. (8 pieces, NLW
    // lines) and slot rows 32 w .. (2 pieces, 32 / RL lines).
    // A slot row past the tile's valid slots reads the tile's first slot: its products land only
    // in output columns that are never stored.
    auto piece_op = [&](int i) { return SHAPE ? (i < 8 ? 0 : 1) : (wave >> 1); };
    auto piece_row = [&](int i) { return SHAPE ? (i < 8 ? wave * 128 + 16 * i : wave * 32 + 16 * (i - 8)) : (wave & 1) * 128 + 16 * i; };
    auto line_op = [&](int i) { return SHAPE ? (i < NLW ? 0 : 1) : (wave >> 1); };
    auto line_row = [&](int i) { return SHAPE ? (i < NLW ? wave * 128 + RL * i : wave * 32 + RL * (i - NLW)) : (wave & 1) * 128 + RL * i; };
    auto row_of = [&](int op, int t) -> int64_t {
        if (op == 0) {
            const int64_t nt = nt0 + (t >> 8);
            const int tt = t & 255;
            int64_t r;
            if (EPI == PMN_EPI_SWIGLU) {
                r = swiglu_a_row_clamped(tt, nt, N >> 1);
            } else {
                r = nt * BT + tt;
                r = r < N ? r : (int64_t)(tt & 31);
            }
            return (int64_t)g * N + r;
        }
        const int64_t m = m0 + (t < mvalid ? t : 0);
        return p.gather ? (int64_t)p.gather[m] : m;
    };
    const int csrc = (lane & 3) ^ ((lane >> 4) & 3);   // source chunk for this lane's position
    // in the last stage only its first tailv / 32 chunks and tailv / 16 scales of a row exist: the
    // other lanes re-read the stage's first chunk or scales (their values are scaled by zero below)
    const int64_t cadj = tailv && csrc >= tailv / 32 ? -16 * csrc : 0;
    const int sidx = SC2 ? (lane & 3) : (lane & 1);   // this lane's scale piece of a row
    const int64_t sadj = tailv && sidx >= tailv / (SC2 ? 32 : 64) ? -(SC2 ? 2 : 4) * sidx : 0;
    const uint8_t* cp[NP];
    const uint8_t* sp[NL];
    uint32_t cd[NP], sd[NL];                     // LDS offsets within a stage slot
#pragma unroll
    for (int i = 0; i < NP; i++) {
        const int op = piece_op(i), r = piece_row(i);
        cp[i] = (op ? p.a_codes : p.b_codes) + row_of(op, r + (lane >> 2)) * cbytes + csrc * 16;
        cd[i] = (op ? XOFF : 0) + r * 64;
    }
#pragma unroll
    for (int i = 0; i < NL; i++) {
        const int op = line_op(i), r = line_row(i);
        sp[i] = (op ? p.a_scales : p.b_scales) + row_of(op, r + lane / (64 / RL)) * sbytes + sidx * (SC2 ? 2 : 4);
        sd[i] = (op ? XSOFF : SOFF) + r * SROW;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);
    // stage v of the copy stream: stages past the last re-load it (into a free slot or over
    // identical bytes), so every stage issues the same copies
    auto stage_src = [&](int v, int64_t& co, int64_t& so) {
        const int kt = v < KT ? v : KT - 1;
        const bool tail = tailv && kt == KT - 1;
        co = (int64_t)kt * 64 + (tail ? cadj : 0);
        so = (int64_t)kt * 8 + (tail ? sadj : 0);
    };
    auto issue_piece = [&](int v, int i) {
        int64_t co, so;
        stage_src(v, co, so);
        dma16(cp[i] + co, lds0 + (uint32_t)(v % NSTAGE) * STAGEB + cd[i]);
    };
    auto issue_line = [&](int v, int i) {
        int64_t co, so;
        stage_src(v, co, so);
        if (SC2) dma2(sp[i] + so, lds0 + (uint32_t)(v % NSTAGE) * STAGEB + sd[i]);
        else dma4(sp[i] + so, lds0 + (uint32_t)(v % NSTAGE) * STAGEB + sd[i]);
    };

    // ---- fragments: 4 weight blocks (f = 0..3) and 4 slot blocks (f = 4..7) per wavefront
    const int wrow0 = SHAPE ? wave * 128 : (wave >> 1) * 128;   // first weight row of the wavefront
    const int xrow0 = SHAPE ? 0 : (wave & 1) * 128;             // first slot row
    const int lrow = lane & 31, hh = lane >> 5;
    const int swz = (lrow >> 2) & 3;
    const int offA = ((2 * hh) ^ swz) << 4, offB = ((2 * hh + 1) ^ swz) << 4;
    uint4 rawA[8], rawB[8];       // code bytes 0..15 (substeps 0-3) and 16..31 (4-7) of the lane's half
    uint32_t scA[8], scB[8];      // the lane's 4 block scales, read with each half
    auto read_half = [&](int v, int f, bool second) {
        const uint8_t* base = lds + (v % NSTAGE) * STAGEB;
        const int row = f < 4 ? wrow0 + f * 32 + lrow : xrow0 + (f - 4) * 32 + lrow;
        const uint4 c = *reinterpret_cast<const uint4*>(base + (f < 4 ? 0 : XOFF) + row * 64 + (second ? offB : offA));
        uint32_t sc;
        if (SC2) {
            // the lane half's two 2-byte pieces sit in the low halves of two LDS words
            const uint2 t = *reinterpret_cast<const uint2*>(base + (f < 4 ? SOFF : XSOFF) + row * 16 + hh * 8);
            sc = __builtin_amdgcn_perm(t.y, t.x, 0x05040100u);
        } else {
            sc = *reinterpret_cast<const uint32_t*>(base + (f < 4 ? SOFF : XSOFF) + row * 8 + hh * 4);
        }
        if (second) { rawB[f] = c; scB[f] = sc; } else { rawA[f] = c; scA[f] = sc; }
    };
    // in the last stage, the scales of blocks past its tailv valid k are forced to zero: lane half
    // hh holds blocks 4 hh .. 4 hh + 3
    const int tcnt = tailv / 16 - 4 * hh;
    const uint32_t tmask = tcnt >= 4 ? 0xFFFFFFFFu : (tcnt <= 0 ? 0u : (1u << (8 * tcnt)) - 1u);
    auto smask = [&](int kt) -> uint32_t { return (tailv && kt >= KT - 1) ? tmask : 0xFFFFFFFFu; };

    f16x8 fa[2][4], fb[2][4];
    // Dequantize half `part` (values 4 part .. 4 part + 3) of fragment f of substep s (of stage
    // kt) into buffer b. The two block scales of a code half convert together (E4M3 -> fp16 is
    // exact); substep s takes scale s / 2. TAIL: the stage may be the last, partly filled one.
    auto convert = [&](int kt, int s, int f, int b, int part, auto tail) {
        const uint4 c = s < 4 ? rawA[f] : rawB[f];
        const uint32_t w = (s & 3) == 0 ? c.x : (s & 3) == 1 ? c.y : (s & 3) == 2 ? c.z : c.w;
        uint32_t sc = s < 4 ? scA[f] : scB[f];
        if (decltype(tail)::value) sc &= smask(kt);
        const f16x2 sp2 = s < 4 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false)
                                : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, true);
        const _Float16 sv = ((s >> 1) & 1) ? sp2[1] : sp2[0];
        const f16x2 ss = {sv, sv};
        const f16x2 p0 = (part ? PMN_FP4_TO_F16(w, 2) : PMN_FP4_TO_F16(w, 0)) * ss;
        const f16x2 p1 = (part ? PMN_FP4_TO_F16(w, 3) : PMN_FP4_TO_F16(w, 1)) * ss;
        f16x8& d = f < 4 ? fa[b][f] : fb[b][f - 4];
        d[4 * part] = p0[0];
        d[4 * part + 1] = p0[1];
        d[4 * part + 2] = p1[0];
        d[4 * part + 3] = p1[1];
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    // One stage kt: 8 substeps of 16 MFMAs. Each MFMA is followed by one piece of side work, in
    // an order the compiler may not regroup:
    //   every MFMA q of substep s: dequantize half q % 2 of fragment q / 2 of substep s + 1 (for
    //     s = 7: of the next stage's substep 0), so the VALU work is spread evenly;
    //   substep 0, MFMAs 8-15: read the second halves (code bytes 16..31) of this stage;
    //   substep 4, MFMA 8: wait until the next stage has landed and barrier (every wavefront is
    //     then done reading this stage's slot), then MFMAs 8-15 copy code pieces 0-7 of stage
    //     kt + 3 into this slot; substep 5, MFMAs 8-11: scale lines 0-3 (SC2: and substep 7,
    //     MFMAs 8-11, lines 4-7); substep 6, MFMAs 12-14: the 512 x 128 shape's further two pieces
    //     and one line (SC2: substep 7, MFMAs 12-13, its two further lines);
    //   substep 5, MFMAs 12-15 and substep 6, MFMAs 8-11: read the first halves of stage kt + 1.
    auto stage = [&](int kt, auto tail) {
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const int b = s & 1;
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int i = q >> 2, j = q & 3;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[b][i], fb[b][j], acc[i][j], 0, 0, 0);
                if (s < 7) convert(kt, s + 1, q >> 1, b ^ 1, q & 1, tail);
                else convert(kt + 1, 0, q >> 1, b ^ 1, q & 1, tail);
                if (s == 0 && q >= 8) read_half(kt, q - 8, true);
                if (s == 4 && q == 8) wait_loads_and_barrier<LPS>();
                if (s == 4 && q >= 8) issue_piece(kt + NSTAGE, q - 8);
                if (s == 5 && q >= 8 && q < 12) issue_line(kt + NSTAGE, q - 8);
                if (SC2 && s == 7 && q >= 8 && q < 12) issue_line(kt + NSTAGE, q - 4);
                if (SHAPE && s == 6 && q >= 12 && q < 14) issue_piece(kt + NSTAGE, q - 4);
                if (SHAPE && !SC2 && s == 6 && q == 14) issue_line(kt + NSTAGE, 4);
                if (SHAPE && SC2 && s == 7 && q >= 12 && q < 14) issue_line(kt + NSTAGE, q - 4);
                if (s == 5 && q >= 12) read_half(kt + 1, q - 12, false);
                if (s == 6 && q >= 8 && q < 12) read_half(kt + 1, q - 4, false);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    typedef std::integral_constant<bool, false> Full;
    typedef std::integral_constant<bool, true> Tail;

    // prologue: stages 0..2 in flight, stage 0's halves read and its substep 0 dequantized
#pragma unroll
    for (int v = 0; v < NSTAGE; v++) {
#pragma unroll
        for (int i = 0; i < NP; i++) issue_piece(v, i);
#pragma unroll
        for (int i = 0; i < NL; i++) issue_line(v, i);
    }
    wait_loads_and_barrier<(NSTAGE - 1) * LPS>();
#pragma unroll
    for (int f = 0; f < 8; f++) read_half(0, f, false);
#pragma unroll
    for (int f = 0; f < 8; f++) {
        convert(0, 0, f, 0, 0, Tail());
        convert(0, 0, f, 0, 1, Tail());
    }
    // the last two stages dequantize values of the last stage, which may be partly filled
    int kt = 0;
    for (; kt + 2 < KT; kt++) stage(kt, Full());
    for (; kt < KT; kt++) stage(kt, Tail());
    // no copy may still be in flight when the LDS is reused or released
    wait_loads_and_barrier<0>();

    // ---- epilogue. Block (i, j) of this wavefront holds, in lane l, slot m0 + xrow0 + j*32 + l%32
    // and the 16 rows wr*128 + i*32 + (v/4)*8 + (l/32)*4 + v%4 of weight tile nt (wr = the
    // wavefront's 128-row half of that tile). The staged outputs (SwiGLU, RHT32 + S2F6) of weight
    // tile nt0 + rg sit in staging rows rg * 128 + slot (SHAPE true) or slot (SHAPE false).
    const int64_t nt = SHAPE ? nt0 + (wave >> 1) : nt0;
    const int wr = SHAPE ? (wave & 1) : (wave >> 1);
    const int srow0 = SHAPE ? (wave >> 1) * 128 : xrow0;        // staging row of slot xrow0
    float sx[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int ml = xrow0 + j * 32 + lrow;
        const bool mok = ml < mvalid;
        const int64_t m = m0 + ml;
        const int64_t xr = mok ? (p.gather ? (int64_t)p.gather[m] : m) : 0;
        sx[j] = mok ? p.a_outer[xr / p.a_rpo] : 0.0f;
    }
    if (EPI == PMN_EPI_F32 || EPI == PMN_EPI_BF16) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t nb = nt * BT + wr * 128 + i * 32;       // first weight row of block i
            const bool nok = nb < N;                              // inside the expert's rows
            const float sw = nok ? p.b_outer[((int64_t)g * N + nb) / p.b_rpo] : 0.0f;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int ml = xrow0 + j * 32 + lrow;
                if (nok && ml < mvalid) {
                    const float s = sx[j] * sw;
                    const int64_t m = m0 + ml;
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const int64_t col = nb + q * 8 + hh * 4;
                        const float y0 = acc[i][j][4 * q] * s, y1 = acc[i][j][4 * q + 1] * s;
                        const float y2 = acc[i][j][4 * q + 2] * s, y3 = acc[i][j][4 * q + 3] * s;
                        if (EPI == PMN_EPI_F32) {
                            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + m * N + col) = make_float4(y0, y1, y2, y3);
                        } else {
                            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + m * N + col) =
                                make_uint2(bf16x2_bits(y0, y1), bf16x2_bits(y2, y3));
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        return;
    }
    // SwiGLU and RHT32 + S2F6 stage 256 rows of 256 bytes (one per slot of a weight tile) in the
    // LDS and write whole 16-byte pieces of each slot's row. Staging row r holds slot r of weight
    // tile nt0 (SHAPE false) or slot r % 128 of weight tile nt0 + r / 128 (SHAPE true).
    uint8_t* const t0 = lds;
    uint8_t* const te = lds + BT * OPITCH;       // E8M0 tile: 8 bytes per staging row
    auto staged = [&](int r, int& slot, int64_t& ntr) {
        slot = SHAPE ? (r & 127) : r;
        ntr = SHAPE ? nt0 + (r >> 7) : nt0;
    };
    // dst(ntr) = the output row base of weight tile ntr for slot 0, rows pitch bytes apart; piece c
    // (16 bytes) of a staged row is stored if cvalid(ntr, c) (it lies inside the expert's N)
    auto store_tile = [&](auto dst, int64_t pitch, auto cvalid) {
#pragma unroll
        for (int k = 0; k < (BT * 16) / THREADS; k++) {
            const int qq = k * THREADS + tid;
            const int r = qq >> 4, c = qq & 15;
            int slot;
            int64_t ntr;
            staged(r, slot, ntr);
            if (slot < mvalid && cvalid(ntr, c))
                *reinterpret_cast<uint4*>(dst(ntr) + (m0 + slot) * pitch + c * 16) =
                    *reinterpret_cast<const uint4*>(t0 + r * OPITCH + c * 16);
        }
    };
    if (EPI == PMN_EPI_SWIGLU) {
        // blocks i = 0, 1 hold h1 and i + 2 the matching h3 of features nt*128 + wr*64 + i*32 + ..
        const int64_t F = N >> 1;
        uint8_t* const A = static_cast<uint8_t*>(p.out);
        uint8_t* const Hs = static_cast<uint8_t*>(p.out_aux);
        float s1[2], s3[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            // features past F (an F that is not a multiple of 128) get scale 0: their values are
            // finite zeros and never stored
            const int64_t f0 = nt * 128 + wr * 64 + i * 32;
            s1[i] = f0 < F ? p.b_outer[((int64_t)g * N + f0) / p.b_rpo] : 0.0f;
            s3[i] = f0 < F ? p.b_outer[((int64_t)g * N + F + f0) / p.b_rpo] : 0.0f;
        }
        auto fvalid = [&](int64_t ntr, int c) { return ntr * 128 + c * 8 < F; };   // 8 features per piece
#pragma unroll
        for (int phase = 0; phase < 3; phase++) {
            if (phase > 0 && !Hs) break;
            if (phase > 0) __syncthreads();     // the previous phase's tile has been stored
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int sl = srow0 + j * 32 + lrow;
#pragma unroll
                for (int i = 0; i < 2; i++) {
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        float o[4];
#pragma unroll
                        for (int v = 0; v < 4; v++) {
                            const float h1 = acc[i][j][4 * q + v] * (sx[j] * s1[i]);
                            const float h3 = acc[i + 2][j][4 * q + v] * (sx[j] * s3[i]);
                            o[v] = phase == 0 ? silu(h1) * h3 : (phase == 1 ? h1 : h3);
                        }
                        const int off = sl * OPITCH + 2 * (wr * 64 + i * 32 + q * 8 + hh * 4);
                        *reinterpret_cast<uint2*>(t0 + off) = make_uint2(bf16x2_bits(o[0], o[1]), bf16x2_bits(o[2], o[3]));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __syncthreads();
            if (phase == 0) store_tile([&](int64_t ntr) { return A + ntr * 128 * 2; }, F * 2, fvalid);
            else if (phase == 1) store_tile([&](int64_t ntr) { return Hs + ntr * 128 * 2; }, N * 2, fvalid);
            else store_tile([&](int64_t ntr) { return Hs + (F + ntr * 128) * 2; }, N * 2, fvalid);
        }
    } else {
        // RHT32 + S2F6: each block's 32 weight rows are one aligned chunk of the slot's row
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int nl = wr * 128 + i * 32;
            // rows past the expert's N get scale 0 (finite zeros, never stored)
            const float sw = nt * BT + nl < N ? p.b_outer[((int64_t)g * N + nt * BT + nl) / p.b_rpo] : 0.0f;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int sl = srow0 + j * 32 + lrow;
                f32x16 z;
#pragma unroll
                for (int v = 0; v < 16; v++) z[v] = acc[i][j][v] * (sx[j] * sw);
                rht_block_store(z, p.rht_mask, lane, reinterpret_cast<int8_t*>(t0 + sl * OPITCH + nl),
                                te + sl * 8 + (nl >> 5));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();
        store_tile([&](int64_t ntr) { return static_cast<uint8_t*>(p.out) + ntr * BT; }, N,
                   [&](int64_t ntr, int c) { return ntr * BT + c * 16 < N; });
        {
            int slot;
            int64_t ntr;
            staged(tid, slot, ntr);
            if (slot < mvalid) {
                // the tile's 8 chunk scales; an N that is not a multiple of 256 has fewer in its last
                // tile, and its rows of scales are then not 8-byte aligned
                uint8_t* const d = p.out_e8m0 + (m0 + slot) * (N >> 5) + ((ntr * BT) >> 5);
                const int64_t nc = (N >> 5) - ntr * 8;
                if ((N & 255) == 0) {
                    *reinterpret_cast<uint2*>(d) = *reinterpret_cast<const uint2*>(te + tid * 8);
                } else {
#pragma unroll
                    for (int c = 0; c < 8; c++)
                        if (c < nc) d[c] = te[tid * 8 + c];
                }
            }
        }
    }
}

template <int EPI, bool SC2>
__global__ __launch_bounds__(fwd::THREADS, 1) void k_nvfp4_grouped_gemm(FwdArgs p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[fwd::lds_bytes(SC2)];
    asm volatile("; agpr in use %0" ::"a"(0));   // keep the accumulators in AGPRs
    TileXY tile;
    if (!xcd_tile(blockIdx.x, p.mtiles, p.ntiles, p.SM, p.SN, tile)) return;
    const GroupUnit u = locate_group_unit(p.offsets, p.G, tile.row, fwd::BT);
    if (u.g < 0) return;
    const int64_t m0 = u.s0 + u.index * fwd::BT;
    const int mvalid = (int)(u.s1 - m0 < fwd::BT ? u.s1 - m0 : fwd::BT);
    // a unit of at most 128 slots is computed as 512 weight rows x 128 slots by the workgroup of
    // the even weight tile of each pair (the odd one has nothing to do); an unpaired last weight
    // tile keeps the 256 x 256 shape
    if (mvalid <= 128 && (tile.col & 1)) return;
    if (mvalid <= 128 && tile.col + 1 < p.ntiles)
        nvfp4_gemm_tile<EPI, true, SC2>(p, lds, u.g, m0, mvalid, tile.col);
    else
        nvfp4_gemm_tile<EPI, false, SC2>(p, lds, u.g, m0, mvalid, tile.col);
}

hipError_t launch_gemm_fwd(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                           int64_t a_rpo, const int32_t* gather, const uint8_t* b_codes,
                           const uint8_t* b_scales, const float* b_outer, int64_t b_rpo,
                           const int64_t* offsets, int G, int64_t M, int64_t N, int64_t K,
                           int epilogue, uint32_t rht_mask, void* out, uint8_t* out_e8m0,
                           void* out_aux, hipStream_t stream)
{
    if (M == 0 || G == 0) return hipSuccess;
    const int64_t mtiles = (M + fwd::BT - 1) / fwd::BT + G;
    // a weight tile is 256 rows of one expert (SwiGLU: 128 features of w1 and the same of w3)
    const int64_t ntiles = epilogue == PMN_EPI_SWIGLU ? (N / 2 + 127) / 128 : (N + fwd::BT - 1) / fwd::BT;
    int SM, SN;
    xcd_shape(mtiles, ntiles, SM, SN);
    FwdArgs p{a_codes, a_scales, a_outer, a_rpo, gather, b_codes, b_scales, b_outer, b_rpo,
              offsets, G, N, K, rht_mask, out, out_e8m0, out_aux, mtiles, ntiles, SM, SN};
    dim3 grid((unsigned)xcd_grid(mtiles, ntiles, SM, SN));
    const dim3 blk(fwd::THREADS);
    if (K % 64 == 0) {
        switch (epilogue) {
        case PMN_EPI_F32: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_F32, false>), grid, blk, 0, stream, p); break;
        case PMN_EPI_BF16: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_BF16, false>), grid, blk, 0, stream, p); break;
        case PMN_EPI_SWIGLU: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_SWIGLU, false>), grid, blk, 0, stream, p); break;
        default: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_RHT32_S2F6, false>), grid, blk, 0, stream, p); break;
        }
    } else {
        switch (epilogue) {
        case PMN_EPI_F32: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_F32, true>), grid, blk, 0, stream, p); break;
        case PMN_EPI_BF16: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_BF16, true>), grid, blk, 0, stream, p); break;
        case PMN_EPI_SWIGLU: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_SWIGLU, true>), grid, blk, 0, stream, p); break;
        default: hipLaunchKernelGGL((k_nvfp4_grouped_gemm<PMN_EPI_RHT32_S2F6, true>), grid, blk, 0, stream, p); break;
        }
    }
    return hipGetLastError();
}

}  // namespace pmn
