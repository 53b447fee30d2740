// noalloc.hip -- moe_grouped_gemm_bwd_noalloc: the grouped backward with its workspace in a static
// device array of the library, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives once per device for the life of the process. In host code its name stands in for
// a host symbol, not a device address, so the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that pointer is handed to the kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pmn.h"
#include "pmn_kernels.hpp"

__device__ __align__(256) uint8_t scratch[PMN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up on the first call per device.
int scratch_of_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PMN_ELAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return PMN_EINVAL;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) return PMN_ELAUNCH;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return PMN_OK;
}

}  // namespace

extern "C" {

size_t pmn_noalloc_scratch_bytes(void) { return (size_t)PMN_NOALLOC_SCRATCH_BYTES; }

int moe_grouped_gemm_bwd_noalloc(const void* dy, const uint8_t* a_codes, const uint8_t* a_scales,
                                 const float* a_outer, int64_t a_rows, int64_t a_rows_per_outer,
                                 const int32_t* gather, const uint8_t* b_codes, const uint8_t* b_scales,
                                 const float* b_outer, int64_t b_rows_per_outer, const int64_t* offsets, int G,
                                 int64_t M, int64_t N, int64_t K, int flags, int dy_rounding, uint64_t seed,
                                 uint32_t rng_stream_a, uint32_t rng_stream_b, uint32_t rng_stream_dy, float* da,
                                 float* db, pmn_stream_t stream)
{
    size_t need = 0;
    int st = pmn::grouped_gemm_bwd_run(dy, a_codes, a_scales, a_outer, a_rows, a_rows_per_outer, gather, b_codes,
                                       b_scales, b_outer, b_rows_per_outer, offsets, G, M, N, K, flags, dy_rounding,
                                       seed, rng_stream_a, rng_stream_b, rng_stream_dy, da, db, nullptr, 0, stream,
                                       &need);
    if (st != PMN_OK) return st;
    if (need > (size_t)PMN_NOALLOC_SCRATCH_BYTES) return PMN_ESCRATCH;
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != PMN_OK) return st;
    return pmn::grouped_gemm_bwd_run(dy, a_codes, a_scales, a_outer, a_rows, a_rows_per_outer, gather, b_codes,
                                     b_scales, b_outer, b_rows_per_outer, offsets, G, M, N, K, flags, dy_rounding,
                                     seed, rng_stream_a, rng_stream_b, rng_stream_dy, da, db, ws,
                                     (size_t)PMN_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

}  // extern "C"
