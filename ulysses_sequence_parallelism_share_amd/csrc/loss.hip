// Token-weighted loss across sequence-parallel ranks (Accelerate guide
// "Sequence parallelism in accelerate", "ALST/Ulysses SP backend
// configuration", the loss-aggregation loop; blog "Ulysses Sequence
// Parallelism: Training with Million-Token Contexts", "Loss aggregation").
//
// Each rank's loss is the mean over its valid tokens (label != ignore
// index).  The ranks' losses are combined weighted by their valid-token
// counts, ranks with no valid token are skipped (their NaN mean would
// otherwise poison the sum), and the total is divided by max(T, 1) where T
// is the number of valid tokens over all ranks.  On one GPU the all_gather
// of the per-rank (loss, count) pairs becomes a read of a [P] buffer.
//
// k_loss_rank: one workgroup of 1024 threads per rank, fp64 sum and int64
// count; each thread keeps 8 independent loads of labels and losses in
// flight (the pass is bound by load latency, not bandwidth), and the
// per-thread sums meet in a fixed reduction tree, so the result is
// deterministic.
// k_loss_finish: combines the P pairs and writes the per-token gradient
// 1/max(T,1) on valid tokens.
#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 256;
constexpr int kRankThreads = 1024;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kRankThreads) void k_loss_rank(const float *__restrict__ token_loss,
                                                            const int64_t *__restrict__ labels,
                                                            int64_t T, int64_t ignore_index,
                                                            float *__restrict__ rank_loss,
                                                            int64_t *__restrict__ good) {
    __shared__ double ssum[kRankThreads / 64];
    __shared__ long long scnt[kRankThreads / 64];
    const int r = blockIdx.x;
    const float *tl = token_loss + (size_t)r * T;
    const int64_t *lb = labels + (size_t)r * T;
    double sum = 0.0;
    long long cnt = 0;
    for (int64_t base = threadIdx.x; base < T; base += (int64_t)kRankThreads * kUnroll) {
        int64_t lv[kUnroll];
        float tv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kRankThreads;
            lv[u] = i < T ? lb[i] : ignore_index;
            tv[u] = i < T ? tl[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (lv[u] != ignore_index) {
                sum += (double)tv[u];
                ++cnt;
            }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        sum += __shfl_xor(sum, m);
        cnt += __shfl_xor(cnt, m);
    }
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        ssum[wid] = sum;
        scnt[wid] = cnt;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0;
        long long c = 0;
        for (int w = 0; w < kRankThreads / 64; ++w) {
            s += ssum[w];
            c += scnt[w];
        }
        rank_loss[r] = c > 0 ? (float)(s / (double)c) : __builtin_nanf("");
        good[r] = c;
    }
}

__global__ __launch_bounds__(kThreads) void k_loss_finish(const int64_t *__restrict__ labels,
                                                          int64_t N, int64_t ignore_index,
                                                          int P,
                                                          const float *__restrict__ rank_loss,
                                                          const int64_t *__restrict__ good,
                                                          float *__restrict__ loss,
                                                          float *__restrict__ d_token_loss) {
    long long T = 0;
    for (int r = 0; r < P; ++r) T += good[r];
    const long long denom = T > 1 ? T : 1;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        double total = 0.0;
        for (int r = 0; r < P; ++r)
            if (good[r] > 0) total += (double)rank_loss[r] * (double)good[r];
        *loss = (float)(total / (double)denom);
    }
    if (d_token_loss == nullptr) return;
    const float gval = 1.0f / (float)denom;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < N;
         i += (int64_t)gridDim.x * kThreads)
        d_token_loss[i] = labels[i] != ignore_index ? gval : 0.0f;
}

}  // namespace

hipError_t launch_weighted_loss(const float *token_loss, const int64_t *labels, int P, int64_t N,
                                int64_t ignore_index, float *loss, float *rank_loss,
                                int64_t *good, float *d_token_loss, hipStream_t stream) {
    const int64_t T = N / P;
    {
        KernelTimer timer("loss_rank", stream);
        hipLaunchKernelGGL(k_loss_rank, dim3((unsigned)P), dim3(kRankThreads), 0, stream, token_loss,
                       labels, T, ignore_index, rank_loss, good);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t blocks = d_token_loss ? (N + kThreads - 1) / kThreads : 1;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    KernelTimer timer("loss_finish", stream);
    hipLaunchKernelGGL(k_loss_finish, dim3((unsigned)blocks), dim3(kThreads), 0, stream, labels, N,
                       ignore_index, P, rank_loss, good, loss, d_token_loss);
    return hipGetLastError();
}
