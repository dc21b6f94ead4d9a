// Segment pre-pass: packed-sample bounds from position_ids.
//
// The attention mask is driven by position_ids, never by a 4D mask
// (Transformers guide "Ulysses sequence parallelism", "Configuration",
// sp_attn_implementation item; blog "Ulysses Sequence Parallelism: Training
// with Million-Token Contexts", "Loss aggregation" paragraph on
// position_ids).  A sample starts at token 0 and wherever position_ids is 0.
// For every token i this pass writes
//     kstart[i] = index of the first token of i's sample,
//     kend[i]   = one past the last token of i's sample,
// so that query i may see key j iff kstart[i] <= j <= i (equivalently
// j <= i < kend[j]).  Both arrays are non-decreasing, so the bounds of any
// tile of consecutive tokens are read from its end points.
//
// Two launches over chunks of kChunk tokens: the first records, per chunk,
// its last and first sample start; the second scans each chunk (a max-scan
// forwards for kstart, a min-scan backwards for kend) seeded with the
// nearest starts of the other chunks.  O(N) work, a few microseconds.
#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kItems = 8;
constexpr int kChunk = kThreads * kItems;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ bool is_start(const int64_t *pos, int32_t i) {
    return i == 0 || pos[i] == 0;
}

// agg[2c] = last start in chunk c (or -1), agg[2c+1] = first start in chunk c (or N).
__global__ __launch_bounds__(kThreads) void k_segment_chunks(const int64_t *__restrict__ pos,
                                                             int32_t *__restrict__ agg, int32_t N) {
    __shared__ int32_t smax[kWaves], smin[kWaves];
    const int32_t c0 = blockIdx.x * kChunk;
    int32_t mx = -1, mn = N;
    for (int k = 0; k < kItems; ++k) {
        const int32_t i = c0 + k * kThreads + threadIdx.x;
        if (i < N && is_start(pos, i)) {
            mx = max(mx, i);
            mn = min(mn, i);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mx = max(mx, __shfl_xor(mx, o));
        mn = min(mn, __shfl_xor(mn, o));
    }
    if ((threadIdx.x & 63) == 0) {
        smax[threadIdx.x >> 6] = mx;
        smin[threadIdx.x >> 6] = mn;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kWaves; ++w) {
            mx = max(mx, smax[w]);
            mn = min(mn, smin[w]);
        }
        agg[2 * blockIdx.x] = max(mx, smax[0]);
        agg[2 * blockIdx.x + 1] = min(mn, smin[0]);
    }
}

// Inclusive scan of one value per thread across the workgroup.
template <bool MAX>
__device__ int32_t block_scan(int32_t x, int32_t *wtot) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x, o);
        if (lane >= o) x = MAX ? max(x, y) : min(x, y);
    }
    if (lane == 63) wtot[wid] = x;
    __syncthreads();
    int32_t pre = MAX ? INT32_MIN : INT32_MAX;
    for (int w = 0; w < wid; ++w) pre = MAX ? max(pre, wtot[w]) : min(pre, wtot[w]);
    __syncthreads();
    return MAX ? max(pre, x) : min(pre, x);
}

__global__ __launch_bounds__(kThreads) void k_segment_scan(const int64_t *__restrict__ pos,
                                                           const int32_t *__restrict__ agg,
                                                           int32_t *__restrict__ kstart,
                                                           int32_t *__restrict__ kend, int32_t N,
                                                           int n_chunks) {
    __shared__ int32_t wtot[kWaves];
    __shared__ int32_t carry[2];
    const int c = blockIdx.x;
    const int32_t c0 = c * kChunk;
    const int tid = threadIdx.x;
    if (tid < 64) {   // nearest starts before and after this chunk
        int32_t lo = -1, hi = N;
        for (int b = tid; b < n_chunks; b += 64) {
            if (b < c) lo = max(lo, agg[2 * b]);
            if (b > c) hi = min(hi, agg[2 * b + 1]);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            lo = max(lo, __shfl_xor(lo, o));
            hi = min(hi, __shfl_xor(hi, o));
        }
        if (tid == 0) {
            carry[0] = lo;
            carry[1] = hi;
        }
    }
    __syncthreads();

    // Forward: kstart[i] = max{ s <= i : s starts a sample }.
    {
        int32_t v[kItems];
        int32_t run = carry[0];
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int32_t i = c0 + tid * kItems + k;
            if (i < N && is_start(pos, i)) run = i;
            v[k] = run;
        }
        const int32_t incl = block_scan<true>(run, wtot);
        int32_t excl = __shfl_up(incl, 1);
        if ((tid & 63) == 0) {
            excl = carry[0];
            for (int w = 0; w < (tid >> 6); ++w) excl = max(excl, wtot[w]);
        }
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int32_t i = c0 + tid * kItems + k;
            if (i < N) kstart[i] = max(excl, v[k]);
        }
    }
    __syncthreads();
    // Backward: kend[i] = min{ s > i : s starts a sample } (or N).
    {
        int32_t v[kItems];
        int32_t run = carry[1];
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int32_t i = c0 + kChunk - 1 - (tid * kItems + k);
            if (i + 1 < N && i + 1 < c0 + kChunk && is_start(pos, i + 1)) run = i + 1;
            v[k] = run;
        }
        const int32_t incl = block_scan<false>(run, wtot);
        int32_t excl = __shfl_up(incl, 1);
        if ((tid & 63) == 0) {
            excl = carry[1];
            for (int w = 0; w < (tid >> 6); ++w) excl = min(excl, wtot[w]);
        }
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int32_t i = c0 + kChunk - 1 - (tid * kItems + k);
            if (i < N) kend[i] = min(excl, v[k]);
        }
    }
}

}  // namespace

size_t segments_scratch_ints(int64_t N) { return 2 * (size_t)((N + kChunk - 1) / kChunk); }

hipError_t launch_segments(const int64_t *pos, int32_t *kstart, int32_t *kend, int32_t *agg,
                           int64_t N, hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    const int n_chunks = (int)((N + kChunk - 1) / kChunk);
    {
        KernelTimer timer("segment_chunks", stream);
        hipLaunchKernelGGL(k_segment_chunks, dim3(n_chunks), dim3(kThreads), 0, stream, pos, agg,
                           (int32_t)N);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    KernelTimer timer("segment_scan", stream);
    hipLaunchKernelGGL(k_segment_scan, dim3(n_chunks), dim3(kThreads), 0, stream, pos,
                       (const int32_t *)agg, kstart, kend, (int32_t)N, n_chunks);
    return hipGetLastError();
}
