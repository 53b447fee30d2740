// route.hip -- top-k routing of tokens to experts and the stable grouping of routed slots.
//
// Pages cited: AREX Feed article "Thinking Machines 发文详解 Inkling 2 Small 训练:原生 4-bit 前向
// 传播贯穿预训练到最后一次 RL rollout", section "计算提速后,NVLink 通信成了新瓶颈" (the router
// decides where each token goes; each token is routed to 8 of 384 experts per the model
// description at the top of the article). Top-k of the softmax equals top-k of the logits, so the
// selection compares logits and the softmax only produces the gates.
//
// Grouping is deterministic: per-expert counts use integer atomics (order-independent), and
// each expert's slots are placed by one workgroup scanning the flat (token, rank) order with a
// block prefix sum, so slot order within an expert is token order.
#include "pmn_dev.hpp"
#include "pmn_kernels.hpp"

namespace pmn {

constexpr int ROUTE_KMAX = 16;

__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int64_t T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ gates)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const float* l = logits + t * E;
    float mx = -INFINITY;
    for (int e = 0; e < E; e++) mx = fmaxf(mx, l[e]);
    float z = 0.0f;
    for (int e = 0; e < E; e++) z += expf(l[e] - mx);
    float bv[ROUTE_KMAX];
    int bi[ROUTE_KMAX];
    int cnt = 0;
    for (int e = 0; e < E; e++) {
        const float v = l[e];
        // position: after every kept value >= v (equal logits keep the lower expert first)
        int pos = cnt;
        while (pos > 0 && bv[pos - 1] < v) pos--;
        if (pos >= k) continue;
        int last = cnt < k ? cnt : k - 1;
        for (int q = last; q > pos; q--) {
            bv[q] = bv[q - 1];
            bi[q] = bi[q - 1];
        }
        bv[pos] = v;
        bi[pos] = e;
        if (cnt < k) cnt++;
    }
    for (int j = 0; j < k; j++) {
        ids[t * k + j] = bi[j];
        gates[t * k + j] = expf(bv[j] - mx) / z;
    }
}

__global__ void k_zero_i64(int64_t* p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void k_route_count(const int32_t* __restrict__ ids, int64_t n, int64_t* offsets)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) atomicAdd(reinterpret_cast<unsigned long long*>(offsets + ids[i] + 1), 1ull);
}

__global__ void k_route_scan(int64_t* offsets, int E)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    for (int e = 0; e < E; e++) offsets[e + 1] += offsets[e];
}

__global__ __launch_bounds__(256) void k_route_scatter(const int32_t* __restrict__ ids, int64_t n, int k,
                                                       const int64_t* __restrict__ offsets,
                                                       int32_t* __restrict__ gather_token,
                                                       int32_t* __restrict__ slot_of)
{
    __shared__ int wave_cnt[4];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t running = offsets[e];
    for (int64_t base = 0; base < n; base += 256) {
        const int64_t i = base + tid;
        const bool hit = i < n && ids[i] == e;
        const unsigned long long bal = __ballot(hit);
        const int below = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wave_cnt[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < 4; w++) {
            if (w < wave) before += wave_cnt[w];
            total += wave_cnt[w];
        }
        if (hit) {
            const int64_t s = running + before + below;
            gather_token[s] = (int32_t)(i / k);
            slot_of[i] = (int32_t)s;
        }
        running += total;
        __syncthreads();
    }
}

// The device index contract of the grouped calls, checked by one workgroup (for debugging a
// caller; nothing on the hot path runs it): each violated rule sets its PMN_CHECK_* bit, and the
// mask is written to *result, 0 when every rule holds. Reads offsets[0..G] and gather[0..n) only.
__global__ __launch_bounds__(1024) void k_check_indices(const int64_t* __restrict__ offsets, int G, int64_t M,
                                                        const int32_t* __restrict__ gather, int64_t n,
                                                        int64_t src_rows, uint32_t* __restrict__ result)
{
    __shared__ uint32_t bad;
    if (threadIdx.x == 0) bad = 0u;
    __syncthreads();
    uint32_t b = 0u;
    if (offsets) {
        for (int64_t g = threadIdx.x; g <= G; g += blockDim.x) {
            const int64_t o = offsets[g];
            if (g == 0 && o != 0) b |= PMN_CHECK_OFFSETS_START;
            if (g == G && o != M) b |= PMN_CHECK_OFFSETS_END;
            if (o < 0 || o > M) b |= PMN_CHECK_OFFSETS_RANGE;
            if (g > 0 && offsets[g - 1] > o) b |= PMN_CHECK_OFFSETS_ORDER;
        }
    }
    if (gather) {
        for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
            const int64_t r = gather[i];
            if (r < 0 || r >= src_rows) b |= PMN_CHECK_GATHER_RANGE;
        }
    }
    if (b) atomicOr(&bad, b);
    __syncthreads();
    if (threadIdx.x == 0) result[0] = bad;
}

hipError_t launch_check_indices(const int64_t* offsets, int G, int64_t M, const int32_t* gather, int64_t n,
                                int64_t src_rows, uint32_t* result, hipStream_t stream)
{
    hipLaunchKernelGGL(k_check_indices, dim3(1), dim3(1024), 0, stream, offsets, G, M, gather, n, src_rows, result);
    return hipGetLastError();
}

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int32_t* ids, float* gates,
                        int64_t* offsets, int32_t* gather_token, int32_t* slot_of, hipStream_t stream)
{
    const int64_t n = T * k;
    hipLaunchKernelGGL(k_zero_i64, dim3((unsigned)((E + 1 + 255) / 256)), dim3(256), 0, stream, offsets, (int64_t)E + 1);
    if (T > 0) {
        hipLaunchKernelGGL(k_route_topk, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream, logits, T, E, k, ids, gates);
        hipLaunchKernelGGL(k_route_count, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, ids, n, offsets);
    }
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(64), 0, stream, offsets, E);
    if (T > 0)
        hipLaunchKernelGGL(k_route_scatter, dim3((unsigned)E), dim3(256), 0, stream, ids, n, k, offsets, gather_token, slot_of);
    return hipGetLastError();
}

}  // namespace pmn
