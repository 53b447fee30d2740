// probe.hip -- measurement kernels: the HBM roof for a given read:write mix and the matrix-core
// ceilings of the MFMA instructions the grouped GEMMs issue. They compute nothing of the layer;
// the benchmark runs them in the same process as the kernels it rates, so every fraction of a
// measured roof is taken against a roof measured on the same chip, clock and run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pmn_dev.hpp"
#include "pmn_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// One wavefront streams units of `rv` 1 KB read rows and `wv` 1 KB write rows: each 16-byte
// load or store instruction covers 64 consecutive vectors (one contiguous KB). NT_LOAD / NT_STORE
// choose nontemporal or ordinary accesses. The stored value depends on every loaded vector so
// that no load can be dropped.
template <bool NT_LOAD, bool NT_STORE>
__global__ __launch_bounds__(256) void k_stream_mix(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                    int64_t units, int rv, int wv)
{
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    auto ld = [](const u32x4* p) { return NT_LOAD ? __builtin_nontemporal_load(p) : *p; };
    for (int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); u < units; u += nwaves) {
        const u32x4* s = src + u * rv * 64 + lane;
        u32x4 acc = {(uint32_t)lane, (uint32_t)u, 0u, 0u};
        int r = 0;
        for (; r + 8 <= rv; r += 8) {
            u32x4 v[8];
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = ld(s + (r + i) * 64);
            acc ^= ((v[0] ^ v[1]) ^ (v[2] ^ v[3])) ^ ((v[4] ^ v[5]) ^ (v[6] ^ v[7]));
        }
        for (; r < rv; r++) acc ^= ld(s + r * 64);
        u32x4* d = dst + u * wv * 64 + lane;
        for (int w = 0; w < wv; w++) {
            u32x4 v = acc;
            v.x += (uint32_t)w;
            if (NT_STORE)
                __builtin_nontemporal_store(v, d + w * 64);
            else
                d[w * 64] = v;
        }
    }
}

// Independent accumulator chains per wavefront, constant operands, no memory traffic in the loop.
// KIND: 0 fp16 32x32x16, 1 fp16 16x16x32, 2 E4M3 block-scaled 32x32x64, 3 E4M3 block-scaled
// 16x16x128, 4 E2M1 block-scaled 32x32x64.
template <int KIND>
__global__ __launch_bounds__(512) void k_mfma_probe(float* __restrict__ sink, int iters)
{
    const int lane = threadIdx.x & 63;
    f32x16 acc[8];
    f32x4 acc4[16];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < 16; i++) acc4[i] = f32x4{};
    f16x8 a, b;
    i32x8 ia, ib;
#pragma unroll
    for (int v = 0; v < 8; v++) {
        a[v] = (_Float16)(lane * 0.001f + v);
        b[v] = (_Float16)(v * 0.5f);
        ia[v] = lane * 0x01030507 + v * 0x11111111;
        ib[v] = v * 0x07050301 + 0x22222222;
    }
    for (int it = 0; it < iters; it++) {
        if (KIND == 0 || KIND == 2 || KIND == 4) {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                if (KIND == 0) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
                if (KIND == 2)
                    acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ia, ib, acc[i], 0, 0, 0, 127, 0, 127);
                if (KIND == 4)
                    acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ia, ib, acc[i], 4, 4, 0, 127, 0, 127);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; i++) {
                if (KIND == 1) acc4[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc4[i], 0, 0, 0);
                if (KIND == 3)
                    acc4[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ia, ib, acc4[i], 0, 0, 0, 127, 0, 127);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) s += acc[i][v];
#pragma unroll
    for (int i = 0; i < 16; i++)
#pragma unroll
        for (int v = 0; v < 4; v++) s += acc4[i][v];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The forward GEMM's inner loop without its memory traffic: one wavefront per SIMD computes a
// 128 x 128 tile with fp16 MFMAs while it dequantizes the operand fragments of the next k-step
// from FP4 codes (one FP4 -> fp16 conversion and one packed multiply by the block scale per two
// values of each operand, the same vector work per flop for either instruction), interleaved with
// the MFMAs. KIND 0: v_mfma_f32_32x32x16_f16 on 4 x 4 blocks, two 16-k substeps per iteration,
// every MFMA followed by half a fragment of the next substep (double-buffered fragments). KIND 1:
// v_mfma_f32_16x16x32_f16 on 8 x 8 blocks, one 32-k substep per half iteration; each row of 8
// MFMAs carries the next B fragment of that row (double-buffered) and the next A fragment
// (written once the row's MFMAs are issued).
__device__ __forceinline__ void dequant_half(f16x8& r, uint32_t w, _Float16 s, int part)
{
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 ss = {s, s};
    const f16x2 p0 = (part ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)
                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)) * ss;
    const f16x2 p1 = (part ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)
                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)) * ss;
    r[4 * part] = p0[0];
    r[4 * part + 1] = p0[1];
    r[4 * part + 2] = p1[0];
    r[4 * part + 3] = p1[1];
}

template <int KIND>
__global__ __launch_bounds__(256, 1) void k_mfma_dequant_probe(float* __restrict__ sink, int iters)
{
    const int lane = threadIdx.x & 63;
    uint32_t raw[16];   // FP4 code words (magnitudes only, so the values stay small)
#pragma unroll
    for (int f = 0; f < 16; f++) raw[f] = (lane * 0x9E3779B1u + f * 0x85EBCA77u + 7u) & 0x77777777u;
    const _Float16 sc = (_Float16)(1.0f + (lane & 7) * 0.125f);
    float t = 0.0f;
    if (KIND == 0) {
        f32x16 acc[4][4];
        f16x8 fa[2][4], fb[2][4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int j = 0; j < 4; j++) acc[i][j] = f32x16{};
            dequant_half(fa[0][i], raw[i], sc, 0);
            dequant_half(fa[0][i], raw[i], sc, 1);
            dequant_half(fb[0][i], raw[4 + i], sc, 0);
            dequant_half(fb[0][i], raw[4 + i], sc, 1);
        }
        for (int it = 0; it < iters; it++) {
#pragma unroll
            for (int b = 0; b < 2; b++) {
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int i = q >> 2, j = q & 3, f = q >> 1;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[b][i], fb[b][j], acc[i][j], 0, 0, 0);
                    const uint32_t w = raw[f + 8 * b] ^ (uint32_t)it;
                    if (f < 4) dequant_half(fa[b ^ 1][f], w, sc, q & 1);
                    else dequant_half(fb[b ^ 1][f - 4], w, sc, q & 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) t += acc[i][j][v];
    } else {
        f32x4 acc[8][8];
        f16x8 fa[8], fb[2][8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
#pragma unroll
            for (int j = 0; j < 8; j++) acc[i][j] = f32x4{};
            dequant_half(fa[i], raw[i], sc, 0);
            dequant_half(fa[i], raw[i], sc, 1);
            dequant_half(fb[0][i], raw[8 + i], sc, 0);
            dequant_half(fb[0][i], raw[8 + i], sc, 1);
        }
        auto substep = [&](int it, auto bc) {
            constexpr int b = decltype(bc)::value;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                f16x8 na = fa[i];
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[b][j], acc[i][j], 0, 0, 0);
                    if (j == 1 || j == 3) dequant_half(fb[b ^ 1][i], raw[8 + i] ^ (uint32_t)it, sc, j == 3);
                    if (j == 5 || j == 7) dequant_half(na, raw[i] ^ (uint32_t)it, sc, j == 7);
                    __builtin_amdgcn_sched_barrier(0);
                }
                fa[i] = na;
            }
        };
        for (int it = 0; it < iters; it += 2) {
            substep(it, std::integral_constant<int, 0>());
            substep(it + 1, std::integral_constant<int, 1>());
        }
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < 8; j++)
#pragma unroll
                for (int v = 0; v < 4; v++) t += acc[i][j][v];
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = t;
}

// FLOPs one wavefront does per loop iteration of k_mfma_probe<KIND> (kinds 5 and 6: of
// k_mfma_dequant_probe, 32 k of a 128 x 128 tile per iteration).
double mfma_flops_per_iter(int kind)
{
    switch (kind) {
    case 0: return 8.0 * 2 * 32 * 32 * 16;
    case 1: return 16.0 * 2 * 16 * 16 * 32;
    case 2: return 8.0 * 2 * 32 * 32 * 64;
    case 3: return 16.0 * 2 * 16 * 16 * 128;
    case 5:
    case 6: return 2.0 * 128 * 128 * 32;
    default: return 8.0 * 2 * 32 * 32 * 64;
    }
}

// Counts the fp32 values d with bit patterns in [first, last] for which the quantizer's reciprocal
// recip_rn(d) differs from the IEEE quotient 1.0f / d.
__global__ __launch_bounds__(256) void k_recip_check(uint32_t first, uint32_t last,
                                                     unsigned long long* __restrict__ mismatches)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    unsigned long long bad = 0;
    for (uint64_t u = (uint64_t)first + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u <= last; u += stride) {
        const float d = __uint_as_float((uint32_t)u);
        const float ieee = 1.0f / d;
        bad += __float_as_uint(pmn::recip_rn(d)) != __float_as_uint(ieee) ? 1u : 0u;
    }
    if (bad) atomicAdd(mismatches, bad);
}

}  // namespace

extern "C" {

int pmn_probe_stream(const void* src, void* dst, int64_t units, int read_kb, int write_kb, int grid, int hints,
                     pmn_stream_t stream)
{
    if (hints < 0 || hints > 3) return PMN_EINVAL;
    if (units < 0 || read_kb < 0 || write_kb < 0 || read_kb + write_kb == 0 || grid < 1) return PMN_ESHAPE;
    if (units == 0) return PMN_OK;
    if ((read_kb > 0 && !src) || (write_kb > 0 && !dst)) return PMN_EINVAL;
    if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15)) return PMN_EALIGN;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const u32x4* a = static_cast<const u32x4*>(src);
    u32x4* b = static_cast<u32x4*>(dst);
    switch (hints) {
    case 0: hipLaunchKernelGGL((k_stream_mix<false, false>), dim3(grid), dim3(256), 0, s, a, b, units, read_kb, write_kb); break;
    case 1: hipLaunchKernelGGL((k_stream_mix<true, false>), dim3(grid), dim3(256), 0, s, a, b, units, read_kb, write_kb); break;
    case 2: hipLaunchKernelGGL((k_stream_mix<false, true>), dim3(grid), dim3(256), 0, s, a, b, units, read_kb, write_kb); break;
    default: hipLaunchKernelGGL((k_stream_mix<true, true>), dim3(grid), dim3(256), 0, s, a, b, units, read_kb, write_kb); break;
    }
    return hipGetLastError() == hipSuccess ? PMN_OK : PMN_ELAUNCH;
}

size_t pmn_probe_mfma_sink_floats(int waves_per_simd, int workgroups)
{
    return (size_t)workgroups * 256 * (size_t)waves_per_simd;
}

int pmn_probe_mfma(int kind, int waves_per_simd, int workgroups, int iters, float* sink, double* flops,
                   pmn_stream_t stream)
{
    if (kind < 0 || kind > 6 || !sink || !flops) return PMN_EINVAL;
    if (waves_per_simd < 1 || waves_per_simd > 2 || workgroups < 1 || iters < 1) return PMN_ESHAPE;
    if (kind >= 5 && (waves_per_simd != 1 || iters % 2 != 0)) return PMN_ESHAPE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 g(workgroups), b(256 * waves_per_simd);
    switch (kind) {
    case 0: hipLaunchKernelGGL(k_mfma_probe<0>, g, b, 0, s, sink, iters); break;
    case 1: hipLaunchKernelGGL(k_mfma_probe<1>, g, b, 0, s, sink, iters); break;
    case 2: hipLaunchKernelGGL(k_mfma_probe<2>, g, b, 0, s, sink, iters); break;
    case 3: hipLaunchKernelGGL(k_mfma_probe<3>, g, b, 0, s, sink, iters); break;
    case 4: hipLaunchKernelGGL(k_mfma_probe<4>, g, b, 0, s, sink, iters); break;
    case 5: hipLaunchKernelGGL(k_mfma_dequant_probe<0>, g, b, 0, s, sink, iters); break;
    default: hipLaunchKernelGGL(k_mfma_dequant_probe<1>, g, b, 0, s, sink, iters); break;
    }
    *flops = mfma_flops_per_iter(kind) * iters * 4.0 * waves_per_simd * workgroups;
    return hipGetLastError() == hipSuccess ? PMN_OK : PMN_ELAUNCH;
}

int pmn_probe_recip_check(uint32_t first_bits, uint32_t last_bits, unsigned long long* mismatches,
                          pmn_stream_t stream)
{
    if (!mismatches) return PMN_EINVAL;
    if (first_bits > last_bits) return PMN_ESHAPE;
    hipLaunchKernelGGL(k_recip_check, dim3(8192), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), first_bits,
                       last_bits, mismatches);
    return hipGetLastError() == hipSuccess ? PMN_OK : PMN_ELAUNCH;
}

}  // extern "C"
