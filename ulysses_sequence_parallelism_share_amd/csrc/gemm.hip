// bf16 matrix products with fp32 accumulation for the fused linear
// cross-entropy:  C[m][n] (=, +=) sum_k A(m, k) B(n, k).
//
// Each operand is either k-contiguous (element (r, k) at p[r * ld + k]) or
// row-contiguous (element (r, k) at p[k * ld + r]); the three products of
// the cross-entropy use all combinations they need:
//   logits = X W^T   A = X  (k-contig)  B = W  (k-contig)
//   dX     = G W     A = G  (k-contig)  B = W  (row-contig: k = vocab)
//   dW    += G^T X   A = G  (row-contig: k = token)  B = X (row-contig)
// A workgroup of 8 waves computes a 256 x 256 tile, each wave 128 x 64 as
// 4 x 2 MFMA 32x32x16 blocks, over k-steps of 64 staged through a
// double-buffered, XOR-swizzled LDS ring by direct global->LDS loads (the
// products are bound by moving operand tiles into LDS, so the tile is as
// large as the LDS allows: 2 x 64 KiB, one workgroup and two waves per SIMD
// per CU; every fragment read feeds 2 or 4 MFMAs).  A
// k-contiguous operand is read 16 bytes per lane; a row-contiguous one with
// the transposing LDS read that yields the same k-slots per lane.  Rows
// past an operand's end read its last row (the caller keeps the k-range
// padded with zeros in the other operand, so they add nothing); output rows
// past m_store are not written.  Tiles are ordered so that the workgroups on
// one XCD (blockIdx % 8) sweep all row tiles of one column tile together,
// sharing that B tile in their L2.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tile.h"

namespace {

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

constexpr int GT = 256;      // tile rows and columns
constexpr int GK = 64;       // k per step
constexpr int kThreads = 512;
constexpr int kWaves = 8;

template <bool KC>
struct OperandTile {
    // k-contiguous: [256 rows][64 k]; row-contiguous: two [64 k][128 rows]
    // halves (a swizzled tile row holds at most 256 bytes)
    using T = typename std::conditional<KC, SwzTile<GT, GK / 8>, SwzTile<GK, GT / 16>>::type;
    static constexpr int kParts = KC ? 1 : 2;
    static constexpr int kBytes = kParts * T::kBytes;
    static constexpr int kRows = KC ? GT : GK;
    static constexpr int kCh = KC ? GK / 8 : GT / 16;
};

template <bool KC>
__device__ __forceinline__ bf16x8 operand(const char *tile, int r0, int s, int lane) {
    using T = typename OperandTile<KC>::T;
    if constexpr (KC)
        return *(const bf16x8 *)(tile + T::off(r0 + (lane & 31), 2 * s + (lane >> 5)));
    else
        return read_tr8k<T>(tile + (r0 >> 7) * T::kBytes, 16 * s, r0 & 127, lane);
}

// OUT: 0 = store fp32, 1 = add into fp32, 2 = store bf16
template <bool AK, bool BK, int OUT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(const bf16 *__restrict__ A, int64_t lda,
                                                      int a_rows, const bf16 *__restrict__ B,
                                                      int64_t ldb, int b_rows, int k_steps,
                                                      void *__restrict__ C, int64_t ldc,
                                                      int m_store, int m_tiles, int n_tiles) {
    using TA = OperandTile<AK>;
    using TB = OperandTile<BK>;
    constexpr int kStage = TA::kBytes + TB::kBytes;
    __shared__ __attribute__((aligned(1024))) char smem[2 * kStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // XCD-aware tile order: linear tile L = xcd * per + (blockIdx / 8)
    const int per = gridDim.x / 8;
    const int L = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (L >= m_tiles * n_tiles) return;
    const int tm = L % m_tiles, tn = L / m_tiles;
    const int m0 = tm * GT, n0 = tn * GT;
    const int wm = wave >> 2, wn = wave & 3;   // wave tile rows wm*128, columns wn*64

    RowStager<TA::kRows, TA::kCh, kWaves> sa;
    RowStager<TB::kRows, TB::kCh, kWaves> sb;
    sa.init(wave, lane, (uint32_t)(lda * 2), 0, 0);
    sb.init(wave, lane, (uint32_t)(ldb * 2), 0, 0);
    // base and valid rows of k-step ks
    using PA = typename TA::T;
    using PB = typename TB::T;
    auto stage = [&](int ks, int buf) {
        char *base = smem + buf * kStage;
        const int k0 = ks * GK;
        if constexpr (AK) {
            sa.issue(base, wave, lane, A + (size_t)m0 * lda + k0, a_rows - m0);
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p)
                sa.issue(base + p * PA::kBytes, wave, lane, A + (size_t)k0 * lda + m0 + 128 * p, GK);
        }
        if constexpr (BK) {
            sb.issue(base + TA::kBytes, wave, lane, B + (size_t)n0 * ldb + k0, b_rows - n0);
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p)
                sb.issue(base + TA::kBytes + p * PB::kBytes, wave, lane,
                         B + (size_t)k0 * ldb + n0 + 128 * p, b_rows - k0);
        }
    };
    stage(0, 0);

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int ks = 0; ks < k_steps; ++ks) {
        wait_async();
        __syncthreads();
        if (ks + 1 < k_steps) stage(ks + 1, (ks + 1) & 1);
        const char *ta = smem + (ks & 1) * kStage;
        const char *tb = ta + TA::kBytes;
        bf16x8 a[GK / 16][4], b[GK / 16][2];
#pragma unroll
        for (int s = 0; s < GK / 16; ++s) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a[s][i] = operand<AK>(ta, wm * 128 + 32 * i, s, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j) b[s][j] = operand<BK>(tb, wn * 64 + 32 * j, s, lane);
        }
#pragma unroll
        for (int s = 0; s < GK / 16; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[s][i], b[s][j], acc[i][j]);
        // The fragments of k16 step s+1 are read while step s multiplies
        // (sched_group_barrier pins that interleave; left alone the compiler
        // waits for each step's reads before its MFMAs).
        {
            constexpr int RD = (AK ? 1 : 2) * 4 + (BK ? 1 : 2) * 2;   // LDS reads per k16 step
            __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
#pragma unroll
            for (int s = 0; s + 1 < GK / 16; ++s) {
                static_for<0, 8>([&](auto m) {
                    constexpr int M = decltype(m)::value;
                    constexpr int nr = RD * (M + 1) / 8 - RD * M / 8;
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
                });
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
    }

    // lane = column n, register r = row acc_row(r, half)
    const int half = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 128 + 32 * i + acc_row(r, half);
                if (m >= m_store) continue;
                const size_t o = (size_t)m * ldc + n;
                if constexpr (OUT == 0)
                    ((float *)C)[o] = acc[i][j][r];
                else if constexpr (OUT == 1)
                    ((float *)C)[o] += acc[i][j][r];
                else
                    ((bf16 *)C)[o] = (bf16)acc[i][j][r];
            }
        }
}

template <bool AK, bool BK, int OUT>
hipError_t gemm_launch(const char *name, const void *A, int64_t lda, int a_rows, const void *B,
                       int64_t ldb, int b_rows, int64_t K, void *C, int64_t ldc, int m_store,
                       int64_t M, int64_t N, hipStream_t stream) {
    const int m_tiles = (int)((M + GT - 1) / GT), n_tiles = (int)((N + GT - 1) / GT);
    const int64_t tiles = (int64_t)m_tiles * n_tiles;
    if (tiles == 0 || K == 0) return hipSuccess;
    const unsigned grid = (unsigned)((tiles + 7) / 8 * 8);
    KernelTimer timer(name, stream);
    hipLaunchKernelGGL((k_gemm<AK, BK, OUT>), dim3(grid), dim3(kThreads), 0, stream,
                       (const bf16 *)A, lda, a_rows, (const bf16 *)B, ldb, b_rows, (int)(K / GK),
                       C, ldc, m_store, m_tiles, n_tiles);
    return hipGetLastError();
}

}  // namespace

// logits[m][n] = sum_k X[m][k] W[n][k]; M rows (tile-padded buffer rows),
// N columns, K % 64 == 0.  x_rows / w_rows: valid operand rows.
hipError_t launch_gemm_logits(const void *x, int x_rows, const void *w, int w_rows, int64_t K,
                              float *logits, int64_t ldl, int64_t M, int64_t N,
                              hipStream_t stream) {
    return gemm_launch<true, true, 0>("lce_gemm_logits", x, K, x_rows, w, K, w_rows, K, logits,
                                      ldl, (int)M, M, N, stream);
}

// dX[m][n] = sum_v G[m][v] W[v][n]; G [M][ldg] (k = vocab, Kv % 64 == 0,
// zero past the vocabulary), W [w_rows][N]; rows >= m_store not written.
hipError_t launch_gemm_dx(const void *g, int64_t ldg, int g_rows, const void *w, int w_rows,
                          int64_t Kv, void *dx, bool dx_f32, int64_t N, int m_store, int64_t M,
                          hipStream_t stream) {
    if (dx_f32)
        return gemm_launch<true, false, 0>("lce_gemm_dx", g, ldg, g_rows, w, N, w_rows, Kv, dx, N,
                                           m_store, M, N, stream);
    return gemm_launch<true, false, 2>("lce_gemm_dx", g, ldg, g_rows, w, N, w_rows, Kv, dx, N,
                                       m_store, M, N, stream);
}

// dW[m][n] (+)= sum_t G[t][m] X[t][n] (stored for the first chunk, added for
// the others); G [Kt][ldg] (Kt % 64 == 0, zero rows past the chunk's
// tokens), X [x_rows][N]; rows >= m_store not written.
hipError_t launch_gemm_dw(const void *g, int64_t ldg, const void *x, int x_rows, int64_t Kt,
                          float *dw, int64_t N, int m_store, int64_t M, bool accumulate,
                          hipStream_t stream) {
    if (accumulate)
        return gemm_launch<false, false, 1>("lce_gemm_dw", g, ldg, (int)Kt, x, N, x_rows, Kt, dw,
                                            N, m_store, M, N, stream);
    return gemm_launch<false, false, 0>("lce_gemm_dw", g, ldg, (int)Kt, x, N, x_rows, Kt, dw, N,
                                        m_store, M, N, stream);
}
