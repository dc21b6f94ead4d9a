// Sequence-sharded <-> head-sharded relayout: the two all-to-alls of a
// Ulysses attention layer, emulated on one GPU over all rank buffers
// (Transformers guide "Ulysses sequence parallelism", introduction and
// figure; blog "Ulysses Sequence Parallelism: Training with Million-Token
// Contexts", "How Ulysses works", steps 1, 3 and 5).
//
// Rank p's chunk [p][t] of the sequence-sharded buffer is global token
// n = p*N/P + t, so the buffer is simply token-major: [N][G][H][d].  The
// exchange is then a transpose of the (token, rank-column) axes with
// "pieces" of (H/P)*d contiguous elements as the unit:
//     seq  side: piece (n, g, q) at ((n*G + g)*H + q*H/P) * d
//     head side: piece (q, g, n) at ((q*G + g)*N + n) * (H/P)*d
// Both sides touch whole pieces (>= 16 bytes, normally 256 B - 1 KiB), so
// every access is a run of full 16-byte vectors.  The data are streamed
// once, with non-temporal loads and stores (HBM-bound; no reuse).
#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;   // 16-byte vectors in flight per thread

// One workgroup covers `rows_per_block` consecutive tokens.  Within it the
// flat index j enumerates (token, group g, rank column q, vector w) with w
// fastest, so consecutive lanes move consecutive 16-byte vectors of a piece
// and consecutive pieces of the sequence-side row.
template <bool TO_HEAD>
__global__ __launch_bounds__(kThreads) void k_relayout(const u32x4 *__restrict__ src,
                                                       u32x4 *__restrict__ dst, uint32_t N,
                                                       uint32_t rows_per_block, FastDiv fR,
                                                       FastDiv fQW, FastDiv fW, uint32_t G,
                                                       int rank, uint32_t HW) {
    const uint32_t n0 = blockIdx.x * rows_per_block;
    const uint32_t nrows = min(rows_per_block, N - n0);
    const uint32_t cnt = nrows * fR.d;
    const uint32_t W = fW.d;
    for (uint32_t base = threadIdx.x; base < cnt; base += kThreads * kUnroll) {
        u32x4 val[kUnroll];
        size_t doff[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t j = base + u * kThreads;
            const bool ok = j < cnt;
            j = ok ? j : 0;
            const uint32_t nl = fdiv(j, fR);
            uint32_t rem = j - nl * fR.d;
            const uint32_t g = fdiv(rem, fQW);
            rem -= g * fQW.d;
            const uint32_t q = fdiv(rem, fW);
            const uint32_t w = rem - q * W;
            const uint32_t n = n0 + nl;
            const uint32_t qq = rank < 0 ? q : (uint32_t)rank;
            const size_t seq_off = ((size_t)n * G + g) * HW + (size_t)qq * W + w;
            const size_t head_off =
                (rank < 0 ? (((size_t)qq * G + g) * N + n) : ((size_t)g * N + n)) * W + w;
            const size_t soff = TO_HEAD ? seq_off : head_off;
            doff[u] = ok ? (TO_HEAD ? head_off : seq_off) : ~(size_t)0;
            if (ok) val[u] = __builtin_nontemporal_load(src + soff);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (doff[u] != ~(size_t)0) __builtin_nontemporal_store(val[u], dst + doff[u]);
    }
}

}  // namespace

hipError_t launch_relayout(bool to_head, const void *src, void *dst, int P, int64_t N, int G,
                           int H, int d, int rank, hipStream_t stream) {
    const uint32_t hl = (uint32_t)(H / P);
    const uint32_t W = hl * (uint32_t)d / 8;               // 16-byte vectors per piece
    const uint32_t nq = rank < 0 ? (uint32_t)P : 1u;        // pieces per (token, group)
    const uint32_t R = (uint32_t)G * nq * W;                // vectors per token
    const uint32_t HW = (uint32_t)H * (uint32_t)d / 8;      // vectors per (token, group) row
    // About 2048 vectors (32 KiB) per workgroup: many small workgroups keep
    // more of the chip streaming than fewer large ones (measured 74 % of HBM
    // against 66 % with 8192).
    uint32_t rows = 2048u / R;
    if (rows < 1) rows = 1;
    const uint32_t blocks = (uint32_t)((N + rows - 1) / rows);
    if (blocks == 0) return hipSuccess;
    const FastDiv fR = make_fastdiv(R), fQW = make_fastdiv(nq * W), fW = make_fastdiv(W);
    KernelTimer timer(to_head ? "relayout_seq_to_head" : "relayout_head_to_seq", stream);
    if (to_head)
        hipLaunchKernelGGL(k_relayout<true>, dim3(blocks), dim3(kThreads), 0, stream,
                           (const u32x4 *)src, (u32x4 *)dst, (uint32_t)N, rows, fR, fQW, fW,
                           (uint32_t)G, rank, HW);
    else
        hipLaunchKernelGGL(k_relayout<false>, dim3(blocks), dim3(kThreads), 0, stream,
                           (const u32x4 *)src, (u32x4 *)dst, (uint32_t)N, rows, fR, fQW, fW,
                           (uint32_t)G, rank, HW);
    return hipGetLastError();
}
