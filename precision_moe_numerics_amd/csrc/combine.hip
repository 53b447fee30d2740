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
// Work split: two lanes per (token, 32-chunk); the even lane holds values 0..15, the odd lane
// 16..31. For each slot a wave then reads 1 KB of one source row with one 16-byte load per lane,
// contiguous across the wave, plus the chunks' E8M0 bytes; butterfly stages 1..8 stay inside a
// lane and stage 16 pairs the two lanes through a DPP swap. Code loads are nontemporal: each
// byte is read once, and streaming them past the caches measured faster. The kernel is
// HBM-bound: per token and slot H + H/32 bytes are read, 2H bytes are written.
#include "pmn_dev.hpp"
#include "pmn_kernels.hpp"

namespace pmn {

namespace cmb {
constexpr int THREADS = 256;
constexpr int KB = 8;  // slots loaded per batch
}  // namespace cmb


// acc[j] += gs * c_j for 16 int8 codes held in one 16-byte word.
PMN_DEV void accumulate_codes16(const uint4 w, float gs, float (&acc)[16])
{
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const float c = (float)(int32_t)((int8_t)(d[q] >> (8 * b)));
            acc[4 * q + b] = __builtin_fmaf(c, gs, acc[4 * q + b]);
        }
}

// acc += sum over N slots of gate * 2^(e - 138) * codes, for this lane's half chunk. A slot
// outside [0, M) reads row 0 with gate 0 (the caller guarantees M >= 1), which adds exactly
// nothing: c * 0 = +-0 and acc + +-0 = acc.
template <int N>
PMN_DEV void accumulate_slots(const int8_t* __restrict__ codes, const uint8_t* __restrict__ e8m0, uint32_t Mu,
                              uint32_t H, uint32_t CH, uint32_t b, uint32_t half, const int32_t* so,
                              const float* gt, float (&acc)[16])
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
    uint4 w[N];
    uint32_t e[N];
#pragma unroll
    for (int j = 0; j < N; j++) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + ((uint64_t)s[j] * H + 32u * b + 16u * half)));
        w[j] = make_uint4(v.x, v.y, v.z, v.w);
        e[j] = e8m0[(uint64_t)s[j] * CH + b];
    }
#pragma unroll
    for (int j = 0; j < N; j++) {
        // gate times 2^(e - 138): exact (for e < 12 the factor is a subnormal float)
        const float gs = __builtin_ldexpf(g[j], (int)e[j] - 138);
        accumulate_codes16(w[j], gs, acc);
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
    const int64_t pair = ((int64_t)blockIdx.x * cmb::THREADS + threadIdx.x) >> 1;
    const uint32_t half = threadIdx.x & 1u;
    if (pair >= T * CH) return;
    const int64_t t = pair / CH;
    const uint32_t b = (uint32_t)(pair - t * CH);

    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; j++) acc[j] = 0.0f;

    if (M > 0) {
        const uint32_t Mu = (uint32_t)min(M, (int64_t)0x80000000LL);
        const int32_t* so = slot_of + t * k;
        const float* gt = gates + t * k;
        int i = 0;
        for (; i + cmb::KB <= k; i += cmb::KB)
            accumulate_slots<cmb::KB>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, half, so + i, gt + i, acc);
        switch (k - i) {
        case 1: accumulate_slots<1>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, half, so + i, gt + i, acc); break;
        case 2: accumulate_slots<2>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, half, so + i, gt + i, acc); break;
        case 3: accumulate_slots<3>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, half, so + i, gt + i, acc); break;
        case 4: accumulate_slots<4>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, half, so + i, gt + i, acc); break;
        case 5: accumulate_slots<5>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, half, so + i, gt + i, acc); break;
        case 6: accumulate_slots<6>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, half, so + i, gt + i, acc); break;
        case 7: accumulate_slots<7>(codes, e8m0, Mu, (uint32_t)H, (uint32_t)CH, b, half, so + i, gt + i, acc); break;
        default: break;
        }
    }

#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; i++)
            if ((i & h) == 0) {
                const float x = acc[i], y = acc[i + h];
                acc[i] = x + y;
                acc[i + h] = x - y;
            }
    // stage 16 across the lane pair: with x = value i (even lane) and y = value i + 16 (odd lane),
    // the even lane keeps x + y and the odd lane x - y, each computed as other + (+-1) * own
    const float sg = half ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float other = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[i]), 0xB1, 0xF, 0xF, false));
        acc[i] = __builtin_fmaf(sg, acc[i], other);
    }
    const uint32_t m = mask >> (16 * half);
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 8; q++) {
        const uint32_t sgn = (((m >> (2 * q)) & 1u) << 15) | (((m >> (2 * q + 1)) & 1u) << 31);
        o[q] = bf16x2_bits(acc[2 * q], acc[2 * q + 1]) ^ sgn;
    }
    uint4* po = reinterpret_cast<uint4*>(out + t * H + 32 * b + 16 * half);
    po[0] = make_uint4(o[0], o[1], o[2], o[3]);
    po[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

hipError_t launch_combine_s2f6(const int8_t* codes, const uint8_t* e8m0, int64_t M, int64_t H, uint32_t mask,
                               const int32_t* slot_of, const float* gates, int64_t T, int k, uint16_t* out,
                               hipStream_t stream)
{
    const int64_t n = 2 * T * (H / 32);
    if (n == 0) return hipSuccess;
    const int64_t grid = (n + cmb::THREADS - 1) / cmb::THREADS;
    hipLaunchKernelGGL(k_combine_s2f6, dim3((uint32_t)grid), dim3(cmb::THREADS), 0, stream, codes, e8m0, M, H, mask,
                       slot_of, gates, T, k, out);
    return hipGetLastError();
}

}  // namespace pmn
