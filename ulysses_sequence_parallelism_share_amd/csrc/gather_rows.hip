// Virtual-row gather for grouped-query attention.
//
// For KV head kh the g = hq/hkv query heads sharing it are handled as
// "virtual rows" v = t*g + (h - kh*g).  When g does not divide 32, the
// dK/dV kernel's row blocks do not start at token boundaries, so this pass
// copies each KV head's rows into a contiguous [n_kv][rows_pad][D] buffer
// (zero rows past N*g) that it streams with a constant stride.  One 16-byte
// vector per thread; HBM-bound.
#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void k_gather_rows(const bf16 *__restrict__ src,
                                                          int64_t src_stride,
                                                          bf16 *__restrict__ dst, int M,
                                                          int rows_pad, int g, FastDiv fg,
                                                          int64_t total) {
    constexpr int VPR = D / 8;   // 16-byte vectors per row
    const int64_t x = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (x >= total) return;
    const int64_t row = x / VPR;               // kh * rows_pad + v
    const int c = (int)(x % VPR);
    const int kh = (int)(row / rows_pad);
    const int v = (int)(row - (int64_t)kh * rows_pad);
    u32x4 val = {0u, 0u, 0u, 0u};
    if (v < M) {
        const int t = (int)fdiv((uint32_t)v, fg);
        val = *(const u32x4 *)(src + (size_t)t * src_stride + (kh * g + (v - t * g)) * D + c * 8);
    }
    *(u32x4 *)(dst + row * D + c * 8) = val;
}

}  // namespace

// src: token t, head h at src[t * src_stride + h * D] (bf16, n_kv * g heads);
// dst: [n_kv][rows_pad][D] bf16.
hipError_t launch_gather_rows(const void *src, int64_t src_stride, void *dst, int64_t N, int n_kv,
                              int g, int D, int64_t rows_pad, hipStream_t stream) {
    const int64_t total = (int64_t)n_kv * rows_pad * (D / 8);
    if (total == 0) return hipSuccess;
    const FastDiv fg = make_fastdiv((uint32_t)g);
    const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads);
    KernelTimer timer("gather_rows", stream);
    if (D == 128)
        hipLaunchKernelGGL(k_gather_rows<128>, dim3(blocks), dim3(kThreads), 0, stream,
                           (const bf16 *)src, src_stride, (bf16 *)dst, (int)(N * g),
                           (int)rows_pad, g, fg, total);
    else
        hipLaunchKernelGGL(k_gather_rows<64>, dim3(blocks), dim3(kThreads), 0, stream,
                           (const bf16 *)src, src_stride, (bf16 *)dst, (int)(N * g),
                           (int)rows_pad, g, fg, total);
    return hipGetLastError();
}
