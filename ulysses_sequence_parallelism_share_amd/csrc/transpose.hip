// Transposed operand copies for the attention kernels.
//
// Products that contract over tokens (P.V in the forward; dO^T.P, Q^T.dS
// and dS.K in the backward) need their token-axis operand with tokens
// contiguous per feature column.  The inputs are token-major ([N][H][d]),
// so one streaming pass writes, per KV head, a [d][rows] copy.  Rows are
// "virtual rows": row v of KV head kh is token v / g, query head
// kh*g + v % g (g = query heads per KV head; g = 1 for K and V).  Inside
// each group of 16 positions the order is permuted (perm16) so that the
// 8 rows a lane feeds one MFMA slot are contiguous (see common.h).
// Positions past the last row are written as zeros up to `rows_pad`.
// Optionally the same rows are also written row-major in virtual-row order,
// [n_kv][rows_pad][D] (zero rows past the end), for kernels that stream
// row tiles of one KV head's virtual rows.
#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;

template <int D>
__global__ __launch_bounds__(kThreads) void k_transpose_rows(const bf16 *__restrict__ src,
                                                             bf16 *__restrict__ dst,
                                                             bf16 *__restrict__ dst_rows, int M,
                                                             int rows_pad, int heads_src, int g,
                                                             FastDiv fg) {
    __shared__ bf16 tile[kRows][D + 8];
    const int kh = blockIdx.y;
    const int v0 = blockIdx.x * kRows;
    constexpr int VPR = D / 8;  // 16-byte vectors per row
#pragma unroll
    for (int i = 0; i < kRows * VPR / kThreads; ++i) {
        const int x = threadIdx.x + i * kThreads;
        const int r = x / VPR, c = x % VPR;
        const int v = v0 + r;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (v < M) {
            const int t = (int)fdiv((uint32_t)v, fg);
            const int hh = kh * g + (v - t * g);
            val = *(const u32x4 *)(src + ((size_t)t * heads_src + hh) * D + c * 8);
        }
        *(u32x4 *)&tile[r][c * 8] = val;
        if (dst_rows) *(u32x4 *)(dst_rows + ((size_t)kh * rows_pad + v0 + r) * D + c * 8) = val;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRows * VPR / kThreads; ++i) {
        const int x = threadIdx.x + i * kThreads;
        const int e = x / (kRows / 8), c = x % (kRows / 8);
        bf16x8 w;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = c * 8 + u;                     // output position in the tile
            const int r = (p & ~15) | perm16(p & 15);    // source row (perm16 is an involution)
            w[u] = tile[r][e];
        }
        *(bf16x8 *)(dst + ((size_t)kh * D + e) * rows_pad + v0 + c * 8) = w;
    }
}

}  // namespace

// src: [N][heads_src][D] bf16; dst: [n_kv][D][rows_pad] bf16 with rows_pad a
// multiple of 64 and >= N * g; dst_rows: NULL or [n_kv][rows_pad][D] bf16.
hipError_t launch_transpose_rows(const void *src, void *dst, void *dst_rows, int64_t N,
                                 int heads_src, int n_kv, int g, int D, int64_t rows_pad,
                                 hipStream_t stream) {
    const int M = (int)(N * g);
    const dim3 grid((unsigned)(rows_pad / kRows), (unsigned)n_kv);
    if (grid.x == 0) return hipSuccess;
    const FastDiv fg = make_fastdiv((uint32_t)g);
    KernelTimer timer("transpose_rows", stream);
    if (D == 128)
        hipLaunchKernelGGL(k_transpose_rows<128>, grid, dim3(kThreads), 0, stream,
                           (const bf16 *)src, (bf16 *)dst, (bf16 *)dst_rows, M, (int)rows_pad,
                           heads_src, g, fg);
    else
        hipLaunchKernelGGL(k_transpose_rows<64>, grid, dim3(kThreads), 0, stream,
                           (const bf16 *)src, (bf16 *)dst, (bf16 *)dst_rows, M, (int)rows_pad,
                           heads_src, g, fg);
    return hipGetLastError();
}
