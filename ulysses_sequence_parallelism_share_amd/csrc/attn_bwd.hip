// Causal attention backward for one rank's heads (blog "Ulysses Sequence
// Parallelism: Training with Million-Token Contexts", "How Ulysses works",
// step 4, run in reverse; the mask is the same position_ids-derived one as
// in the forward).
//
// With P rebuilt from the forward's log-sum-exp (P = 2^(s*scale*log2e -
// lse*log2e)), the gradients are
//     dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q.
// Two kernels share that recurrence without atomics, so the result is
// deterministic:
//  * k_attn_bwd_dkdv - a workgroup owns 128 keys of one KV head (4 waves x
//    32); K and V stay in registers as B operands, and the wave walks the
//    virtual query rows that can see its keys (t in [j0, segment end)) in
//    tiles of 32.  S = Q K^T and dP = dO V^T come out with one key per lane,
//    so P and dS feed dV^T += dO^T P and dK^T += Q^T dS directly (dO^T and
//    Q^T are pre-transposed copies in perm16 row order).  The GQA sum over
//    the query heads of a KV head falls out of the virtual-row walk.
//  * k_attn_bwd_dq - a workgroup owns 128 virtual query rows (like the
//    forward); Q and dO stay in registers, K, V and K^T tiles stream through
//    LDS, and dQ^T += K^T dS^T accumulates per lane.
#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 256;
constexpr int BK = 128;  // keys per dK/dV workgroup
constexpr int BQ = 32;   // virtual query rows per dK/dV tile
constexpr int BM = 128;  // virtual query rows per dQ workgroup
constexpr int BN = 64;   // keys per dQ tile

// ---------------------------------------------------------------------------
// D = rowsum(dO * O): one group of D/8 lanes per (token, head) row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void k_bwd_delta(const bf16 *__restrict__ o,
                                                        const bf16 *__restrict__ d_o,
                                                        float *__restrict__ delta, int N,
                                                        int hq) {
    constexpr int LPR = D / 8;
    const int64_t row = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / LPR;
    const int c = threadIdx.x % LPR;
    const bool ok = row < (int64_t)N * hq;
    float acc = 0.f;
    if (ok) {
        const bf16x8 a = *(const bf16x8 *)(o + row * D + c * 8);
        const bf16x8 b = *(const bf16x8 *)(d_o + row * D + c * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += (float)a[i] * (float)b[i];
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (ok && c == 0) {
        const int t = (int)(row / hq), h = (int)(row % hq);
        delta[(size_t)h * N + t] = acc;
    }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
struct DkdvTiles {
    bf16 q[BQ][D + 8];
    bf16 dO[BQ][D + 8];
    bf16 qt[D][BQ + 8];
    bf16 dot[D][BQ + 8];
    float lse2[BQ];
    float delta[BQ];
};

template <int D>
__global__ __launch_bounds__(kThreads) void k_attn_bwd_dkdv(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ d_o, const bf16 *__restrict__ qt, const bf16 *__restrict__ dot,
    const float *__restrict__ lse, const float *__restrict__ delta,
    const int32_t *__restrict__ kend, void *__restrict__ dk, void *__restrict__ dv, int N,
    int Mpad, int hq, int hkv, int g, FastDiv fg, float scale_log2, float scale, int out_f32) {
    __shared__ DkdvTiles<D> sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;
    const int kh = blockIdx.x % hkv;
    const int j0 = (blockIdx.x / hkv) * BK;
    const int M = N * g;
    const int key = j0 + wave * 32 + col;
    const bool key_ok = key < N;
    const int my_kend = kend[key_ok ? key : N - 1];
    const int kw0 = j0 + wave * 32;                     // this wave's first key
    const int kw1 = min(kw0 + 31, N - 1);               // and last (if kw0 < N)
    const bool wave_has_keys = kw0 < N;
    const int kend_w0 = wave_has_keys ? kend[kw0] : 0;
    const int kend_w1 = wave_has_keys ? kend[kw1] : 0;
    const int kend_max = kend[min(j0 + BK, N) - 1];

    bf16x8 kf[D / 16], vf[D / 16];
    {
        const size_t off = ((size_t)(key_ok ? key : 0) * hkv + kh) * D + half * 8;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            bf16x8 a = *(const bf16x8 *)(k + off + 16 * st);
            bf16x8 b = *(const bf16x8 *)(v + off + 16 * st);
            if (!key_ok) {
#pragma unroll
                for (int i = 0; i < 8; ++i) a[i] = b[i] = (bf16)0.f;
            }
            kf[st] = a;
            vf[st] = b;
        }
    }
    f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkacc[i][r] = dvacc[i][r] = 0.f;

    constexpr int RV = BQ * D / 8 / kThreads;  // 16-byte vectors per thread per row tile
    const int vq_hi = kend_max * g;            // rows [j0*g, kend_max*g) can see these keys
    for (int vq0 = j0 * g; vq0 < vq_hi; vq0 += BQ) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RV; ++i) {
            const int x = tid + i * kThreads;
            const int r = x / (D / 8), c = x % (D / 8);
            const int vv = vq0 + r;
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (vv < M) {
                const int t = (int)fdiv((uint32_t)vv, fg);
                const size_t off = ((size_t)t * hq + kh * g + (vv - t * g)) * D + c * 8;
                a = *(const u32x4 *)(q + off);
                b = *(const u32x4 *)(d_o + off);
            }
            *(u32x4 *)&sm.q[r][c * 8] = a;
            *(u32x4 *)&sm.dO[r][c * 8] = b;
        }
#pragma unroll
        for (int i = 0; i < RV; ++i) {
            const int x = tid + i * kThreads;
            const int e = x / (BQ / 8), c = x % (BQ / 8);
            const size_t off = ((size_t)kh * D + e) * Mpad + vq0 + c * 8;
            *(u32x4 *)&sm.qt[e][c * 8] = *(const u32x4 *)(qt + off);
            *(u32x4 *)&sm.dot[e][c * 8] = *(const u32x4 *)(dot + off);
        }
        if (tid < BQ) {
            const int vv = vq0 + tid;
            float l2 = INFINITY, dl = 0.f;
            if (vv < M) {
                const int t = (int)fdiv((uint32_t)vv, fg);
                const size_t idx = (size_t)(kh * g + (vv - t * g)) * N + t;
                l2 = lse[idx] * SP_LOG2E;
                dl = delta[idx];
            }
            sm.lse2[tid] = l2;
            sm.delta[tid] = dl;
        }
        __syncthreads();

        const int tq_first = (int)fdiv((uint32_t)vq0, fg);
        const int tq_last = (int)fdiv((uint32_t)(min(vq0 + BQ, M) - 1), fg);
        // every pair masked: all rows before the wave's keys, or past their samples
        const bool skip = !wave_has_keys || tq_last < kw0 || tq_first >= kend_w1;
        if (skip) continue;
        const bool full = (kw1 <= tq_first) && (tq_last < kend_w0);

        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const bf16x8 a = *(const bf16x8 *)&sm.q[col][16 * st + 8 * half];
            s = mfma32(a, kf[st], s);
        }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const bf16x8 a = *(const bf16x8 *)&sm.dO[col][16 * st + 8 * half];
            dp = mfma32(a, vf[st], dp);
        }

        bf16x8 pf[2], dsf[2];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const f32x4 l2 = *(const f32x4 *)&sm.lse2[rg * 8 + half * 4];
            const f32x4 dl = *(const f32x4 *)&sm.delta[rg * 8 + half * 4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rg * 4 + i;
                float p = fast_exp2(s[r] * scale_log2 - l2[i]);
                if (!full) {
                    const int tq = (int)fdiv((uint32_t)(vq0 + acc_row(r, half)), fg);
                    if (!(key <= tq && tq < my_kend)) p = 0.f;
                }
                const float ds = p * (dp[r] - dl[i]);
                pf[r >> 3][r & 7] = (bf16)p;
                dsf[r >> 3][r & 7] = (bf16)ds;
            }
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const bf16x8 a = *(const bf16x8 *)&sm.dot[db * 32 + col][s2 * 16 + half * 8];
                dvacc[db] = mfma32(a, pf[s2], dvacc[db]);
                const bf16x8 b = *(const bf16x8 *)&sm.qt[db * 32 + col][s2 * 16 + half * 8];
                dkacc[db] = mfma32(b, dsf[s2], dkacc[db]);
            }
    }

    if (!key_ok) return;
    const size_t base = ((size_t)key * hkv + kh) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int e = db * 32 + rg * 8 + half * 4;
            if (out_f32) {
                f32x4 a, b;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] = dkacc[db][rg * 4 + i] * scale;
                    b[i] = dvacc[db][rg * 4 + i];
                }
                *(f32x4 *)((float *)dk + base + e) = a;
                *(f32x4 *)((float *)dv + base + e) = b;
            } else {
                bf16x4 a, b;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] = (bf16)(dkacc[db][rg * 4 + i] * scale);
                    b[i] = (bf16)dvacc[db][rg * 4 + i];
                }
                *(bf16x4 *)((bf16 *)dk + base + e) = a;
                *(bf16x4 *)((bf16 *)dv + base + e) = b;
            }
        }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
struct DqTiles {
    bf16 k[BN][D + 8];
    bf16 v[BN][D + 8];
    bf16 kt[D][BN + 8];
};

template <int D>
__global__ __launch_bounds__(kThreads) void k_attn_bwd_dq(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ d_o, const bf16 *__restrict__ kt, const float *__restrict__ lse,
    const float *__restrict__ delta, const int32_t *__restrict__ kstart, void *__restrict__ dq,
    int N, int Npad, int hq, int hkv, int g, FastDiv fg, float scale_log2, float scale,
    int n_row_tiles, int out_f32) {
    __shared__ DqTiles<D> sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;
    const int kh = blockIdx.x % hkv;
    const int tile = n_row_tiles - 1 - blockIdx.x / hkv;
    const int M = N * g;
    const int v0 = tile * BM;
    const int vrow = v0 + wave * 32 + col;
    const bool row_ok = vrow < M;
    const int vr = row_ok ? vrow : M - 1;
    const int t = (int)fdiv((uint32_t)vr, fg);
    const int h = kh * g + (vr - t * g);
    const int t_first = (int)fdiv((uint32_t)v0, fg);
    const int t_last = (int)fdiv((uint32_t)(min(v0 + BM, M) - 1), fg);
    const int key_lo = kstart[t_first];
    const int ks_max = kstart[t_last];
    const int my_ks = kstart[t];
    const float l2 = lse[(size_t)h * N + t] * SP_LOG2E;
    const float dl = delta[(size_t)h * N + t];

    bf16x8 qf[D / 16], dof[D / 16];
    {
        const size_t off = ((size_t)t * hq + h) * D + half * 8;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            qf[s] = *(const bf16x8 *)(q + off + 16 * s);
            dof[s] = *(const bf16x8 *)(d_o + off + 16 * s);
        }
    }
    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[i][r] = 0.f;

    constexpr int KV = BN * D / 8 / kThreads;
    const int jt0 = key_lo / BN, jt1 = t_last / BN;
    for (int jt = jt0; jt <= jt1; ++jt) {
        const int j0 = jt * BN;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KV; ++i) {
            const int x = tid + i * kThreads;
            const int r = x / (D / 8), c = x % (D / 8);
            const int j = j0 + r;
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (j < N) {
                const size_t off = ((size_t)j * hkv + kh) * D + c * 8;
                a = *(const u32x4 *)(k + off);
                b = *(const u32x4 *)(v + off);
            }
            *(u32x4 *)&sm.k[r][c * 8] = a;
            *(u32x4 *)&sm.v[r][c * 8] = b;
        }
#pragma unroll
        for (int i = 0; i < KV; ++i) {
            const int x = tid + i * kThreads;
            const int e = x / (BN / 8), c = x % (BN / 8);
            *(u32x4 *)&sm.kt[e][c * 8] =
                *(const u32x4 *)(kt + ((size_t)kh * D + e) * Npad + j0 + c * 8);
        }
        __syncthreads();
        const bool full = (j0 + BN - 1 <= t_first) && (j0 >= ks_max);

        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.f;
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
                const bf16x8 a = *(const bf16x8 *)&sm.k[kb * 32 + col][16 * st + 8 * half];
                s[kb] = mfma32(a, qf[st], s[kb]);
            }
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
                const bf16x8 a = *(const bf16x8 *)&sm.v[kb * 32 + col][16 * st + 8 * half];
                dp[kb] = mfma32(a, dof[st], dp[kb]);
            }
        }
        bf16x8 dsf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(s[kb][r] * scale_log2 - l2);
                if (!full) {
                    const int key = j0 + kb * 32 + acc_row(r, half);
                    if (key < my_ks || key > t) p = 0.f;
                }
                dsf[kb][r >> 3][r & 7] = (bf16)(p * (dp[kb][r] - dl));
            }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const bf16x8 a =
                        *(const bf16x8 *)&sm.kt[db * 32 + col][kb * 32 + s2 * 16 + half * 8];
                    dqacc[db] = mfma32(a, dsf[kb][s2], dqacc[db]);
                }
    }

    if (!row_ok) return;
    const size_t base = ((size_t)t * hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int e = db * 32 + rg * 8 + half * 4;
            if (out_f32) {
                f32x4 a;
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = dqacc[db][rg * 4 + i] * scale;
                *(f32x4 *)((float *)dq + base + e) = a;
            } else {
                bf16x4 a;
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = (bf16)(dqacc[db][rg * 4 + i] * scale);
                *(bf16x4 *)((bf16 *)dq + base + e) = a;
            }
        }
}

template <int D>
hipError_t bwd_launch(const void *q, const void *k, const void *v, const void *o,
                      const void *d_o, const float *lse, int64_t N, int hq, int hkv, float scale,
                      bool grad_f32, void *dq, void *dk, void *dv, const AttnWorkspace &ws,
                      hipStream_t stream) {
    const int g = hq / hkv;
    const int64_t M = N * g;
    const int64_t Npad = (N + 63) / 64 * 64;
    const int64_t Mpad = (M + 63) / 64 * 64;
    const FastDiv fg = make_fastdiv((uint32_t)g);
    const float scale_log2 = scale * SP_LOG2E;
    hipError_t e;

    const int64_t delta_threads = N * hq * (D / 8);
    {
        KernelTimer timer("bwd_delta", stream);
        hipLaunchKernelGGL(k_bwd_delta<D>, dim3((unsigned)((delta_threads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, (const bf16 *)o, (const bf16 *)d_o, ws.delta,
                       (int)N, hq);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_transpose_rows(q, ws.qt, N, hq, hkv, g, D, Mpad, stream)) != hipSuccess) return e;
    if ((e = launch_transpose_rows(d_o, ws.dot, N, hq, hkv, g, D, Mpad, stream)) != hipSuccess) return e;
    if ((e = launch_transpose_rows(k, ws.kvt, N, hkv, hkv, 1, D, Npad, stream)) != hipSuccess) return e;

    const int n_key_tiles = (int)((N + BK - 1) / BK);
    {
        KernelTimer timer("attn_bwd_dkdv", stream);
        hipLaunchKernelGGL(k_attn_bwd_dkdv<D>, dim3((unsigned)(n_key_tiles * hkv)), dim3(kThreads), 0,
                       stream, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v,
                       (const bf16 *)d_o, (const bf16 *)ws.qt, (const bf16 *)ws.dot, lse,
                       (const float *)ws.delta, (const int32_t *)ws.kend, dk, dv, (int)N,
                       (int)Mpad, hq, hkv, g, fg, scale_log2, scale, (int)grad_f32);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const int n_row_tiles = (int)((M + BM - 1) / BM);
    KernelTimer timer("attn_bwd_dq", stream);
    hipLaunchKernelGGL(k_attn_bwd_dq<D>, dim3((unsigned)(n_row_tiles * hkv)), dim3(kThreads), 0,
                       stream, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v,
                       (const bf16 *)d_o, (const bf16 *)ws.kvt, lse, (const float *)ws.delta,
                       (const int32_t *)ws.kstart, dq, (int)N, (int)Npad, hq, hkv, g, fg,
                       scale_log2, scale, n_row_tiles, (int)grad_f32);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                           const void *d_o, const float *lse, const int64_t *pos, int64_t N,
                           int hq, int hkv, int d, float scale, bool grad_f32, void *dq,
                           void *dk, void *dv, const AttnWorkspace &ws, hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    hipError_t e = launch_segments(pos, ws.kstart, ws.kend, N, stream);
    if (e != hipSuccess) return e;
    if (d == 128)
        return bwd_launch<128>(q, k, v, o, d_o, lse, N, hq, hkv, scale, grad_f32, dq, dk, dv, ws,
                               stream);
    return bwd_launch<64>(q, k, v, o, d_o, lse, N, hq, hkv, scale, grad_f32, dq, dk, dv, ws,
                          stream);
}
