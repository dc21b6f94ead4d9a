// Per-token cross-entropy from hidden states and an LM-head matrix, with
// its gradients, never holding more than one chunk of logits.
//
// The model computes a per-token loss from shift_labels before the
// token-weighted aggregation (Accelerate guide "Sequence parallelism in
// accelerate", "ALST/Ulysses SP backend configuration", the loss loop and
// the note after it; blog "Ulysses Sequence Parallelism: Training with
// Million-Token Contexts", "Loss aggregation"); for long sequences the
// pages recommend a fused logit-loss that never materialises the full
// logits tensor.  For tokens t, vocabulary entries v:
//     lse_t  = log sum_v exp(x_t . w_v),  loss_t = lse_t - x_t . w_{y_t}
//     G_tv   = g_t (softmax_v - [v == y_t]),  dX = G W,  dW = G^T X
// (ignored tokens: no loss, no gradient).  Tokens are processed in chunks:
// logits of the chunk (one GEMM), a row pass (log-sum-exp, loss and G in
// bf16), then dX of the chunk and dW (= for the first chunk, += after) G^T X
// (two GEMMs).  Only the chunk's logits (fp32) and G (bf16) live in the
// workspace.
#include "common.h"
#include "launch.h"

hipError_t launch_gemm_logits(const void *x, int x_rows, const void *w, int w_rows, int64_t K,
                              float *logits, int64_t ldl, int64_t M, int64_t N,
                              hipStream_t stream);
hipError_t launch_gemm_dx(const void *g, int64_t ldg, int g_rows, const void *w, int w_rows,
                          int64_t Kv, void *dx, bool dx_f32, int64_t N, int m_store, int64_t M,
                          hipStream_t stream);
hipError_t launch_gemm_dw(const void *g, int64_t ldg, const void *x, int x_rows, int64_t Kt,
                          float *dw, int64_t N, int m_store, int64_t M, bool accumulate,
                          hipStream_t stream);

namespace {

// The row pass reads each logits row twice.  A persistent grid of one
// 1024-thread workgroup per CU keeps only 256 rows in flight (128 MiB at the
// Llama-3 vocabulary), which the 256 MiB last-level cache holds, so the
// second read of a row is served from it: 0.75 ms against 1.04 ms for one
// 256-thread workgroup per row (4096 x 128256 logits).
constexpr int kThreads = 1024;
constexpr int kRowGrid = 256;
constexpr int kUnroll = 4;   // 16-byte loads in flight per thread

// Block-wide log-sum-exp in the log2 domain: each thread brings a running
// max m and a sum s of 2^(x - m); pairs combine as
// (max(m1, m2), s1 2^(m1 - m) + s2 2^(m2 - m)).
__device__ __forceinline__ void lse_combine(float &m, float &s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;   // both empty
    s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
    m = mn;
}

__device__ __forceinline__ void block_lse(float &m, float &s, float2 *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lse_combine(m, s, __shfl_xor(m, o), __shfl_xor(s, o));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = make_float2(m, s);
    __syncthreads();
    m = red[0].x;
    s = red[0].y;
    for (int i = 1; i < kThreads / 64; ++i) lse_combine(m, s, red[i].x, red[i].y);
}

// A workgroup walks token rows row = blockIdx.x, + gridDim.x, ... of the
// chunk's n_rows (rows at or past n_tok only clear their G row, so the dW
// product's padded k-range adds nothing).  Labels outside [0, V) other than
// ignore_index give a NaN loss and no gradient.  A row is read twice: once
// for its log-sum-exp (running max and rescaled sum, kUnroll 16-byte pieces
// per thread and step), once for G.
__global__ __launch_bounds__(kThreads) void k_lce_rows(
    const float *__restrict__ logits, int64_t ldl, int V, int v_pad,
    const int64_t *__restrict__ labels, int64_t ignore_index, const float *__restrict__ g,
    int n_tok, int n_rows, float *__restrict__ token_loss, float *__restrict__ lse_out,
    bf16 *__restrict__ G, int64_t ldg) {
    __shared__ float2 red[kThreads / 64];
    const int n4 = v_pad / 4;   // v_pad is a multiple of 256
    for (int row = blockIdx.x; row < n_rows; row += gridDim.x) {
        __syncthreads();   // red[] of the previous row has been read
        if (row >= n_tok) {
            if (G) {
                bf16x4 z;
#pragma unroll
                for (int e = 0; e < 4; ++e) z[e] = (bf16)0.f;
                for (int c = threadIdx.x; c < n4; c += kThreads)
                    *((bf16x4 *)(G + (size_t)row * ldg) + c) = z;
            }
            continue;
        }
        const float *l = logits + (size_t)row * ldl;
        float m = -INFINITY, sum = 0.f;   // log2 domain
        for (int c0 = threadIdx.x; c0 < n4; c0 += kThreads * kUnroll) {
            f32x4 x[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int c = c0 + u * kThreads;
                if (c < n4) x[u] = *((const f32x4 *)l + c);
            }
            float y[kUnroll][4], cm = -INFINITY;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = c0 + u * kThreads;
                    y[u][e] = (c < n4 && 4 * c + e < V) ? x[u][e] * SP_LOG2E : -INFINITY;
                    cm = fmaxf(cm, y[u][e]);
                }
            if (cm == -INFINITY) continue;   // past the vocabulary
            const float mn = fmaxf(m, cm);
            sum *= fast_exp2(m - mn);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) sum += fast_exp2(y[u][e] - mn);
            m = mn;
        }
        block_lse(m, sum, red);
        const float lse = (m + __log2f(sum)) * SP_LN2;
        const int64_t y = labels[row];
        const bool ignored = y == ignore_index;
        const bool in_range = y >= 0 && y < V;
        const bool valid = !ignored && in_range;
        if (threadIdx.x == 0) {
            lse_out[row] = lse;
            token_loss[row] = valid ? lse - l[y] : (ignored ? 0.f : NAN);
        }
        if (!G) continue;
        const float gt = valid ? g[row] : 0.f;
        const float sh = lse * SP_LOG2E;
        bf16x4 *gr = (bf16x4 *)(G + (size_t)row * ldg);
        for (int c0 = threadIdx.x; c0 < n4; c0 += kThreads * kUnroll) {
            f32x4 x[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int c = c0 + u * kThreads;
                if (c < n4) x[u] = *((const f32x4 *)l + c);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int c = c0 + u * kThreads;
                if (c >= n4) break;
                bf16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = 4 * c + e;
                    float p = 0.f;
                    if (v < V) p = gt * (fast_exp2(fmaf(x[u][e], SP_LOG2E, -sh)) - (v == y ? 1.f : 0.f));
                    o[e] = (bf16)p;
                }
                gr[c] = o;
            }
        }
    }
}

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

size_t lce_workspace_layout(int64_t vocab, int64_t chunk, void *base, LceWorkspace *ws) {
    const int64_t v_pad = round_up(vocab, 256);   // the GEMM's tile width
    const size_t logits_bytes = (size_t)chunk * v_pad * 4;
    const size_t g_bytes = (size_t)round_up(chunk, 64) * v_pad * 2;
    const size_t a = (logits_bytes + 255) & ~(size_t)255;
    if (ws) {
        ws->logits = base ? (float *)base : nullptr;
        ws->g = base ? (char *)base + a : nullptr;
        ws->v_pad = v_pad;
    }
    return a + ((g_bytes + 255) & ~(size_t)255);
}

hipError_t launch_linear_ce(const void *x, const void *w, const int64_t *labels,
                            int64_t ignore_index, const float *g, int64_t N, int64_t V, int64_t K,
                            bool dx_f32, float *token_loss, float *lse, void *dx, float *dw,
                            int64_t chunk, const LceWorkspace &ws, hipStream_t stream) {
    hipError_t e;
    const int64_t v_pad = ws.v_pad;
    for (int64_t t0 = 0; t0 < N; t0 += chunk) {
        const int nt = (int)(N - t0 < chunk ? N - t0 : chunk);
        const bf16 *xc = (const bf16 *)x + (size_t)t0 * K;
        if ((e = launch_gemm_logits(xc, nt, w, (int)V, K, ws.logits, v_pad, nt, V, stream)) != hipSuccess)
            return e;
        {
            const int rows = g ? (int)round_up(nt, 64) : nt;
            KernelTimer timer("lce_rows", stream);
            hipLaunchKernelGGL(k_lce_rows, dim3((unsigned)(rows < kRowGrid ? rows : kRowGrid)),
                               dim3(kThreads), 0, stream, ws.logits, v_pad, (int)V, (int)v_pad,
                               labels + t0, ignore_index, g ? g + t0 : nullptr, nt, rows,
                               token_loss + t0, lse + t0,
                               g ? (bf16 *)ws.g : nullptr, v_pad);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (!g) continue;
        void *dxc = (char *)dx + (size_t)t0 * K * (dx_f32 ? 4 : 2);
        if ((e = launch_gemm_dx(ws.g, v_pad, nt, w, (int)V, round_up(V, 64), dxc, dx_f32, K, nt,
                                nt, stream)) != hipSuccess)
            return e;
        if ((e = launch_gemm_dw(ws.g, v_pad, xc, nt, round_up(nt, 64), dw, K, (int)V, V, t0 > 0,
                                stream)) != hipSuccess)
            return e;
    }
    return hipSuccess;
}
