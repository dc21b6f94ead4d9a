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
// One workgroup scans the whole sequence in chunks (a max-scan forwards for
// kstart, a min-scan backwards for kend).  O(N) work; a few microseconds per
// 10^5 tokens, negligible next to the O(N^2) attention.
#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kItems = 8;
constexpr int kWaves = kThreads / 64;

template <bool MAX>
__device__ __forceinline__ int32_t comb(int32_t a, int32_t b) {
    return MAX ? max(a, b) : min(a, b);
}

// Inclusive scan of one value per thread across the workgroup.
template <bool MAX>
__device__ int32_t block_scan(int32_t x, int32_t *wtot) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x, o);
        if (lane >= o) x = comb<MAX>(x, y);
    }
    if (lane == 63) wtot[wid] = x;
    __syncthreads();
    int32_t pre = MAX ? INT32_MIN : INT32_MAX;
    for (int w = 0; w < wid; ++w) pre = comb<MAX>(pre, wtot[w]);
    __syncthreads();
    return comb<MAX>(pre, x);
}

__global__ __launch_bounds__(kThreads) void k_segments(const int64_t *__restrict__ pos,
                                                       int32_t *__restrict__ kstart,
                                                       int32_t *__restrict__ kend, int32_t N) {
    __shared__ int32_t wtot[kWaves];
    __shared__ int32_t carry_s;
    const int tid = threadIdx.x;

    // Forward: kstart[i] = max{ s <= i : s == 0 or pos[s] == 0 }.
    int32_t carry = 0;
    for (int32_t c0 = 0; c0 < N; c0 += kThreads * kItems) {
        int32_t v[kItems];
        int32_t run = INT32_MIN;
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int32_t i = c0 + tid * kItems + k;
            const int32_t s = (i < N && (i == 0 || pos[i] == 0)) ? i : INT32_MIN;
            run = max(run, s);
            v[k] = run;
        }
        const int32_t incl = block_scan<true>(run, wtot);
        int32_t excl = __shfl_up(incl, 1);
        if ((tid & 63) == 0) excl = INT32_MIN;
        if ((tid & 63) == 0 && tid > 0) {
            int32_t pre = INT32_MIN;
            for (int w = 0; w < (tid >> 6); ++w) pre = max(pre, wtot[w]);
            excl = pre;
        }
        excl = max(excl, carry);
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int32_t i = c0 + tid * kItems + k;
            if (i < N) kstart[i] = max(excl, v[k]);
        }
        if (tid == kThreads - 1) carry_s = max(carry, incl);
        __syncthreads();
        carry = carry_s;
        __syncthreads();
    }

    // Backward: kend[i] = min{ s > i : pos[s] == 0 } (or N).
    carry = N;
    for (int32_t c1 = N; c1 > 0; c1 -= kThreads * kItems) {
        int32_t v[kItems];
        int32_t run = INT32_MAX;
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int32_t i = c1 - 1 - (tid * kItems + k);
            int32_t f = INT32_MAX;
            if (i >= 0) f = (i + 1 < N && pos[i + 1] == 0) ? i + 1 : N;
            run = min(run, f);
            v[k] = run;
        }
        const int32_t incl = block_scan<false>(run, wtot);
        int32_t excl = __shfl_up(incl, 1);
        if ((tid & 63) == 0) excl = INT32_MAX;
        if ((tid & 63) == 0 && tid > 0) {
            int32_t pre = INT32_MAX;
            for (int w = 0; w < (tid >> 6); ++w) pre = min(pre, wtot[w]);
            excl = pre;
        }
        excl = min(excl, carry);
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int32_t i = c1 - 1 - (tid * kItems + k);
            if (i >= 0) kend[i] = min(excl, v[k]);
        }
        if (tid == kThreads - 1) carry_s = min(carry, incl);
        __syncthreads();
        carry = carry_s;
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_segments(const int64_t *pos, int32_t *kstart, int32_t *kend, int64_t N,
                           hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    KernelTimer timer("segments", stream);
    hipLaunchKernelGGL(k_segments, dim3(1), dim3(kThreads), 0, stream, pos, kstart, kend,
                       (int32_t)N);
    return hipGetLastError();
}
