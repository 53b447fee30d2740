// combine.hip -- receiver side of the combine: a token's routed slots send their w2 outputs back
// as RHT32 + S2F6 rows (int8 codes, one E8M0 per 32 values); the token's output is the
// gate-weighted sum of their decoded rows, stored as bf16.
//
// Pages cited: AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向
// 传播贯穿预训练到最后一次 RL rollout", section "计算提速后,NVLink 通信成了新瓶颈": the combine
// brings expert outputs back to each token in the 8-bit RHT form, and the receiver undoes the
// orthogonal transform exactly; the gates are the router's softmax weights.
//
// Decoding one 32-chunk is x^ = D H z^ / 32 with z^_j = c_j 2^(e - 127 - 6): linear in the codes.
// So the sum over a token's k slots is taken on the scaled codes first and the Walsh-Hadamard
// butterflies run once per chunk instead of once per slot:
//     out = D H ( sum_i  g_i 2^(e_i - 138) c_i )
// c_i are integers (|c| <= 127) and g_i 2^(e_i - 138) is exact (a power-of-two scaling), so the
// only roundings are one fma per slot and value, one per butterfly stage (five) and the final
// bf16 rounding.
//
// Work split: one lane per (token, 32-chunk). A wave reads, for each slot, 64 consecutive chunks
// of one source row (2 KB) plus their 64 E8M0 bytes, and writes 64 consecutive bf16 chunks
// (4 KB). The kernel is HBM-bound: per token and slot H + H/32 bytes are read, 2H written.
#include "pmn_dev.hpp"
#include "pmn_kernels.hpp"

namespace pmn {

namespace cmb {
constexpr int THREADS = 256;
constexpr int KB = 8;  // slots loaded per batch
}  // namespace cmb

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 (a in the low half), round to nearest even: v_cvt_pk_bf16_f32.
PMN_DEV uint32_t bf16x2_bits(float a, float b)
{
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// acc[j] += gs * c_j for the 32 int8 codes held in two 16-byte words.
PMN_DEV void accumulate_codes(const uint4 (&w)[2], float gs, float (&acc)[32])
{
    const uint32_t d[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
    for (int q = 0; q < 8; q++)
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const float c = (float)(int32_t)((int8_t)(d[q] >> (8 * b)));
            acc[4 * q + b] = __builtin_fmaf(c, gs, acc[4 * q + b]);
        }
}

// acc += sum over N slots of gate * 2^(e - 138) * codes. A slot outside [0, M) reads row 0 with
// gate 0 (the caller guarantees M >= 1), which adds exactly nothing: c * 0 = +-0 and acc + +-0 = acc.
template <int N>
PMN_DEV void accumulate_slots(const int8_t* __restrict__ codes, const uint8_t* __restrict__ e8m0, uint32_t Mu,
                              uint32_t H, uint32_t CH, uint32_t b, const int32_t* so, const float* gt,
                              float (&acc)[32])
{
    uint32_t s[N];
    float g[N];
#pragma unroll
    for (int j = 0; j < N; j++) {
        s[j] = (uint32_t)so[j];
        g[j] = gt[j];
    }
#pragma unroll
    for (int j = 0; j < N; j++) {
        const bool ok = s[j] < Mu;
        g[j] = ok ? g[j] : 0.0f;
        s[j] = ok ? s[j] : 0u;
    }
    uint4 w[N][2];
    uint32_t e[N];
#pragma unroll
    for (int j = 0; j < N; j++) {
        const uint4* p = reinterpret_cast<const uint4*>(codes + ((uint64_t)s[j] * H + 32u * b));
        w[j][0] = p[0];
        w[j][1] = p[1];
        e[j] = e8m0[(uint64_t)s[j] * CH + b];
    }
#pragma unroll
    for (int j = 0; j < N; j++) {
        // gate times 2^(e - 138): exact (for e < 12 the factor is a subnormal float)
        const float gs = __builtin_ldexpf(g[j], (int)e[j] - 138);
        accumulate_codes(w[j], gs, acc);
    }
}

__global__ __launch_bounds__(cmb::THREADS) void k_combine_s2f6(const int8_t* __restrict__ codes,
                                                               const uint8_t* __restrict__ e8m0, int64_t M,
                                                               int64_t H, uint32_t mask,
                                                               const int32_t* __restrict__ slot_of,
                                                               const float* __restrict__ gates, int64_t T, int k,
                                                               uint16_t* __restrict__ out)
{
    const int64_t CH = H >> 5;
    const int64_t lane = (int64_t)blockIdx.x * cmb::THREADS + threadIdx.x;
    if (lane >= T * CH) return;
    const int64_t t = lane / CH;
    const uint32_t b = (uint32_t)(lane - t * CH);

    float acc[32];
#pragma unroll
    for (int j = 0; j < 32; j++) acc[j] = 0.0f;

    if (M > 0) {
        // slot values are int32, so every valid one is below min(M, 2^31); negative ones wrap above
        const uint32_t Mu = (uint32_t)min(M, (int64_t)0x80000000LL);
        const int32_t* so = slot_of + t * k;
        const float* gt = gates + t * k;
        int i = 0;
        for (; i + cmb::KB <= k; i += cmb::KB)
            accumulate_slots<cmb::KB>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, so + i, gt + i, acc);
        switch (k - i) {
        case 1: accumulate_slots<1>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, so + i, gt + i, acc); break;
        case 2: accumulate_slots<2>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, so + i, gt + i, acc); break;
        case 3: accumulate_slots<3>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, so + i, gt + i, acc); break;
        case 4: accumulate_slots<4>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, so + i, gt + i, acc); break;
        case 5: accumulate_slots<5>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, so + i, gt + i, acc); break;
        case 6: accumulate_slots<6>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, so + i, gt + i, acc); break;
        case 7: accumulate_slots<7>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, so + i, gt + i, acc); break;
        default: break;
        }
    }

    // H: butterflies in stages of 1, 2, 4, 8, 16 (Sylvester order, H[i][j] = (-1)^popcount(i & j))
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
        for (int i = 0; i < 32; i++)
            if ((i & h) == 0) {
                const float x = acc[i], y = acc[i + h];
                acc[i] = x + y;
                acc[i + h] = x - y;
            }

    // D: value j changes sign where bit j of the mask is set; then bf16, round to nearest even
    uint32_t o[16];
#pragma unroll
    for (int q = 0; q < 16; q++) {
        // RNE commutes with negation, so the sign bits go onto the rounded values
        const uint32_t sg = (((mask >> (2 * q)) & 1u) << 15) | (((mask >> (2 * q + 1)) & 1u) << 31);
        o[q] = bf16x2_bits(acc[2 * q], acc[2 * q + 1]) ^ sg;
    }
    uint4* po = reinterpret_cast<uint4*>(out + t * H + 32 * b);
#pragma unroll
    for (int q = 0; q < 4; q++) po[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

hipError_t launch_combine_s2f6(const int8_t* codes, const uint8_t* e8m0, int64_t M, int64_t H, uint32_t mask,
                               const int32_t* slot_of, const float* gates, int64_t T, int k, uint16_t* out,
                               hipStream_t stream)
{
    const int64_t n = T * (H / 32);
    if (n == 0) return hipSuccess;
    const int64_t grid = (n + cmb::THREADS - 1) / cmb::THREADS;
    hipLaunchKernelGGL(k_combine_s2f6, dim3((uint32_t)grid), dim3(cmb::THREADS), 0, stream, codes, e8m0, M, H, mask,
                       slot_of, gates, T, k, out);
    return hipGetLastError();
}

}  // namespace pmn
