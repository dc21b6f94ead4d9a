// The all-to-all of K/V-like tensors when a model has fewer KV heads than
// sequence-parallel ranks.
//
// The pages require the attention heads to be divisible by sp_size
// (Transformers guide "Ulysses sequence parallelism", "Configuration") and
// are silent on grouped-query models whose KV heads are fewer than the
// ranks.  Query head h uses KV head h / (Hq / n_kv), so rank q's query
// heads [q Hq/P, (q+1) Hq/P) all use KV head (q n_kv) / P; the seq->head
// exchange therefore sends each KV head to the P / n_kv ranks that use it,
// and the head->seq exchange of the gradients sums those copies (it is the
// adjoint of the copy).  With n_kv >= P both reduce to the plain exchange.
//
// Layouts (token-major exchange buffers, as in relayout.hip):
//   x_seq  [P][N/P][G][n_kv][d]  (token n = p N/P + t)
//   x_head [P][G][N][hl][d], hl = max(n_kv / P, 1); rank q holds KV heads
//          [(q n_kv)/P, (q n_kv)/P + hl)
// One thread moves one 16-byte chunk (8 bf16); the copy reads each chunk
// once and writes it to every rank that holds its head.  The gradient sum
// runs in fp32 in ascending rank order and is rounded once to the output type.
#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 256;

// grid.y = group g; x = chunk over [n][j][c] of the heads read (all H heads
// for every rank, or the hl heads of one rank).  Each chunk is read once and
// written to every rank that holds its head: the one owner when n_kv >= P,
// else the R = P / n_kv consecutive ranks [j R, (j+1) R).
__global__ __launch_bounds__(kThreads) void k_kv_seq_to_head(
    const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int N, int G, int H, int P, int hl,
    int V, FastDiv f_row, int rank, int64_t chunks) {
    const int64_t x = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (x >= chunks) return;
    const int g = blockIdx.y;
    const uint32_t n = fdiv((uint32_t)x, f_row);
    const uint32_t jc = (uint32_t)x - n * f_row.d;                 // head * V + c, heads read
    const uint32_t jl = jc / (uint32_t)V, c = jc - jl * (uint32_t)V;
    const int h0 = rank < 0 ? 0 : (int)(((int64_t)rank * H) / P);
    const int j = h0 + (int)jl;                                      // KV head
    const u32x4 val = __builtin_nontemporal_load(src + ((int64_t)n * G + g) * H * V + (int64_t)j * V + c);
    if (rank >= 0) {
        __builtin_nontemporal_store(val, dst + (((int64_t)g * N + n) * hl + jl) * V + c);
    } else if (H >= P) {
        const int q = j / hl, i = j - q * hl;
        __builtin_nontemporal_store(val, dst + ((((int64_t)q * G + g) * N + n) * hl + i) * V + c);
    } else {
        const int R = P / H;
        for (int r = 0; r < R; ++r)
            __builtin_nontemporal_store(val, dst + (((int64_t)(j * R + r) * G + g) * N + n) * V + c);
    }
}

// dst rank block y = pi (token chunk of rank p_first + pi);
// x = chunk over [t][g][j][c] of that block.  Input element type: bf16
// (F32 = false) or fp32; 8 elements per chunk.
template <bool F32>
__global__ __launch_bounds__(kThreads) void k_kv_head_to_seq_sum(
    const void *__restrict__ src, void *__restrict__ dst, int N, int T, int G, int H, int P,
    int hl, int V, FastDiv f_v, FastDiv f_h, FastDiv f_g, int p_first, int64_t chunks) {
    const int64_t x = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (x >= chunks) return;
    const int pi = blockIdx.y, p = p_first + pi;
    const uint32_t r0 = fdiv((uint32_t)x, f_v);
    const int c = (int)((uint32_t)x - r0 * (uint32_t)V);
    const uint32_t r1 = fdiv(r0, f_h);
    const int j = (int)(r0 - r1 * (uint32_t)H);
    const uint32_t t = fdiv(r1, f_g);
    const int g = (int)(r1 - t * (uint32_t)G);
    const int64_t n = (int64_t)p * T + t;
    // ranks holding head j: the one block owner (n_kv >= P) or the P/n_kv copies
    int q0, nq, i;
    if (H >= P) {
        q0 = j / hl;
        nq = 1;
        i = j - q0 * hl;
    } else {
        nq = P / H;
        q0 = j * nq;
        i = 0;
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int q = q0; q < q0 + nq; ++q) {                 // ascending rank order
        const int64_t off = ((((int64_t)q * G + g) * N + n) * hl + i) * V + c;   // in chunks
        if constexpr (F32) {
            const f32x4 *s = (const f32x4 *)src + 2 * off;
            const f32x4 a = s[0], b = s[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += a[e];
                acc[4 + e] += b[e];
            }
        } else {
            const bf16x8 a = *((const bf16x8 *)src + off);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (float)a[e];
        }
    }
    const int64_t doff = ((int64_t)pi * T + t) * G * H * V + ((int64_t)g * H + j) * V + c;
    if constexpr (F32) {
        f32x4 *d = (f32x4 *)dst + 2 * doff;
        d[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
        d[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)acc[e];
        *((bf16x8 *)dst + doff) = o;
    }
}

}  // namespace

hipError_t launch_kv_seq_to_head(const void *x_seq, void *x_head, int P, int64_t N, int G, int H,
                                 int d, int rank, hipStream_t stream) {
    const int hl = H >= P ? H / P : 1;
    const int V = d / 8;
    const int heads_read = rank < 0 ? H : hl;
    const int64_t chunks = N * heads_read * V;
    const dim3 grid((unsigned)((chunks + kThreads - 1) / kThreads), (unsigned)G);
    KernelTimer timer("relayout_kv_seq_to_head", stream);
    hipLaunchKernelGGL(k_kv_seq_to_head, grid, dim3(kThreads), 0, stream, (const u32x4 *)x_seq,
                       (u32x4 *)x_head, (int)N, G, H, P, hl, V,
                       make_fastdiv((uint32_t)(heads_read * V)), rank, chunks);
    return hipGetLastError();
}

hipError_t launch_kv_head_to_seq_sum(const void *x_head, void *x_seq, int P, int64_t N, int G,
                                     int H, int d, bool f32, int rank, hipStream_t stream) {
    const int hl = H >= P ? H / P : 1;
    const int V = d / 8;
    const int T = (int)(N / P);
    const int64_t chunks = (int64_t)T * G * H * V;
    const int np = rank < 0 ? P : 1;
    const dim3 grid((unsigned)((chunks + kThreads - 1) / kThreads), (unsigned)np);
    const FastDiv fv = make_fastdiv((uint32_t)V), fh = make_fastdiv((uint32_t)H),
                  fg = make_fastdiv((uint32_t)G);
    KernelTimer timer("relayout_kv_head_to_seq_sum", stream);
    if (f32)
        hipLaunchKernelGGL(k_kv_head_to_seq_sum<true>, grid, dim3(kThreads), 0, stream, x_head,
                           x_seq, (int)N, T, G, H, P, hl, V, fv, fh, fg, rank < 0 ? 0 : rank,
                           chunks);
    else
        hipLaunchKernelGGL(k_kv_head_to_seq_sum<false>, grid, dim3(kThreads), 0, stream, x_head,
                           x_seq, (int)N, T, G, H, P, hl, V, fv, fh, fg, rank < 0 ? 0 : rank,
                           chunks);
    return hipGetLastError();
}
