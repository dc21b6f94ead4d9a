// Causal attention forward for one rank's heads over the full sequence
// (blog "Ulysses Sequence Parallelism: Training with Million-Token
// Contexts", "How Ulysses works", step 4: each GPU runs standard attention
// for its heads over all positions).  Masking comes from position_ids
// through the segment bounds (Transformers guide "Ulysses sequence
// parallelism", "Configuration": position_ids replace the 4D mask and
// packed samples must not attend across their boundaries).
//
// Design (gfx950, 64-wide waves, MFMA 32x32x16 bf16):
//  * GQA rows are folded together: for KV head kh the g = hq/hkv query heads
//    that share it form "virtual rows" v = t*g + (h - kh*g).  A workgroup
//    owns 256 consecutive virtual rows (8 waves x 32), so every K/V tile it
//    stages in LDS serves all g heads and 256 rows (the tile loads cost a
//    sixth of the kernel's time with 128 rows), and the causal bound of the
//    tile spans only 256/g tokens.
//  * Each wave computes S^T = K Q^T (keys x queries), so a lane owns one
//    query column: the row max and row sum of the softmax are per-lane
//    register reductions plus one exchange with lane l^32.
//  * The probabilities leave the S^T accumulators directly as the B operand
//    of O^T += V^T P^T, and the per-row rescale of O is a per-lane multiply.
//    The V^T operand comes from V^T tiles ([d][keys], 16-byte reads like the
//    K tiles) of a transposed copy of V that a pre-pass writes with the keys
//    of every group of 16 in the accumulators' order: lane half h holds keys
//    4h..4h+3 and 8+4h..8+4h+3 of each group in its 8 k-slots.
//  * fp32 online softmax in the log2 domain (scale * log2(e) folded into one
//    FMA per score, exponentials with v_exp_f32); the running max is
//    updated lazily (only when it grows by more than 2^8), so the O
//    accumulators are rarely rescaled.
//  * One workgroup of 8 waves per CU (2 waves per SIMD).
//  * K and V^T tiles are double-buffered in LDS (XOR-swizzled, bank-conflict
//    free) and filled by direct global->LDS loads issued one tile ahead, so
//    the loads overlap the MFMA and softmax work of the current tile without
//    occupying registers.
//  * Tiles inside every row's segment and below every row's diagonal skip
//    the mask; the key range of a workgroup is [kstart(first row), last row].
//  * Workgroups are launched last row tile first.  For one sequence that is
//    longest-first; with packed samples the last tiles belong to the last
//    sample, not necessarily the longest, but a dispatch simulation over 256
//    CUs puts this order within 0.2 % of a perfect balance.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tile.h"

namespace {

constexpr int BM = 256;  // virtual query rows per workgroup (8 waves x 32)
constexpr int BN = 64;   // keys per tile
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

template <int D>
struct FwdSmem {
    using K = SwzTile<BN, D / 8>;   // keys x features
    using VT = SwzTile<D, BN / 8>;  // features x keys (permuted within groups of 16)
    static constexpr int kStage = K::kBytes + VT::kBytes;
};

// Position p (0..15) of a group of 16 keys in the transposed copy holds key
// kperm(p): lane half h of an MFMA operand reads positions 8h..8h+7, which
// must be the keys its accumulator registers hold (rows 4h+{0..3} and
// 8+4h+{0..3} of each 16-row group).
__device__ __forceinline__ int kperm(int p) { return (p & 3) + ((p >> 2) & 1) * 8 + (p >> 3) * 4; }

// V [N][hkv][d] (token stride kv_st) -> vt [hkv][d][Npad], keys permuted
// within groups of 16, zero past N.  A workgroup transposes 64 keys of one
// KV head through LDS.
template <int D>
__global__ __launch_bounds__(256) void k_v_transpose(const bf16 *__restrict__ v, bf16 *__restrict__ vt,
                                                     int N, int64_t Npad, int64_t kv_st) {
    __shared__ bf16 tile[64][D + 8];   // +8: rows 16 bytes apart in bank order
    const int kh = blockIdx.y, j0 = blockIdx.x * 64;
    constexpr int CPR = D / 8;         // 16-byte chunks per key row
#pragma unroll
    for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
        const int r = i / CPR, c = i % CPR;
        bf16x8 x;
        if (j0 + r < N) {
            x = *(const bf16x8 *)(v + (size_t)(j0 + r) * kv_st + (size_t)kh * D + c * 8);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (bf16)0.f;
        }
        *(bf16x8 *)&tile[r][c * 8] = x;
    }
    __syncthreads();
#pragma unroll
    for (int i = threadIdx.x; i < D * 8; i += 256) {   // output chunk: feature f, keys 8c..8c+7
        const int f = i / 8, c = i % 8;
        bf16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int p = 8 * c + e;
            x[e] = tile[(p & ~15) + kperm(p & 15)][f];
        }
        *(bf16x8 *)(vt + ((size_t)kh * D + f) * Npad + j0 + 8 * c) = x;
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void k_attn_fwd(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ vt,
    int64_t vt_n, const int32_t *__restrict__ kstart, bf16 *__restrict__ o,
    float *__restrict__ lse, int N, int hq, int hkv, int g, FastDiv fg, float scale_log2,
    int n_row_tiles, int64_t q_st, int64_t kv_st, int64_t o_st) {
    using S = FwdSmem<D>;
    __shared__ __attribute__((aligned(1024))) char smem[2 * S::kStage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    const int jt0 = key_lo / BN, jt1 = t_last / BN;
    // Keys past the end are read from the last key: finite values, always masked.
    RowStager<BN, D / 8, kWaves> stager;
    stager.init(wave, lane, (uint32_t)(kv_st * 2), 0, 0);
    RowStager<D, BN / 8, kWaves> stager_vt;   // D feature rows of the V^T tile
    stager_vt.init(wave, lane, (uint32_t)(vt_n * 2), 0, 0);
    const bf16 *vt_head = vt + (size_t)kh * D * vt_n;
    auto stage = [&](int jt, int buf) {
        char *base = smem + buf * S::kStage;
        const int j0 = jt * BN;
        const size_t roff = (size_t)j0 * kv_st + kh * D;
        stager.issue(base, wave, lane, k + roff, N - j0);
        stager_vt.issue(base + S::K::kBytes, wave, lane, vt_head + j0, D);
    };
    stage(jt0, 0);

    // This lane's query row as the B operand of S^T = K Q^T.
    bf16x8 qf[D / 16];
    {
        const bf16 *qrow = q + (size_t)t * q_st + h * D + half * 8;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qf[s] = *(const bf16x8 *)(qrow + 16 * s);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    float m_run = -1e30f, l_run = 0.f;

    // One key tile; `masked` selects the code that evaluates the mask.  The
    // LDS slot of tile jt is (jt - jt0) & 1; `slot` passes it as a constant
    // where the caller knows it (0 or 1), or -1 to compute it.
    auto tile_step = [&](int jt, auto masked, auto slot) {
        const int j0 = jt * BN;
        wait_async();
        __syncthreads();
        const int sl = decltype(slot)::value >= 0 ? decltype(slot)::value : ((jt - jt0) & 1);
        if (jt < jt1) stage(jt + 1, sl ^ 1);
        const char *ks = smem + sl * S::kStage;
        const char *vs = ks + S::K::kBytes;

        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
                const bf16x8 a = *(const bf16x8 *)(ks + S::K::off(kb * 32 + col, 2 * st + half));
                s[kb] = mfma32(a, qf[st], s[kb]);
            }
        }

        // Row max of the raw scores (masked scores set to -inf), then in the
        // log2 domain; lanes l and l^32 hold the two halves of one row.
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (decltype(masked)::value) {
                    const int key = j0 + kb * 32 + acc_row(r, half);
                    s[kb][r] = (key >= my_ks && key <= t) ? s[kb][r] : -INFINITY;
                }
                mx = fmaxf(mx, s[kb][r]);
            }
        mx = wave_max_pair(mx) * scale_log2;
        // Lazy rescaling: the reference max only moves when a row's max
        // exceeds it by more than 2^8, so the O accumulators are rescaled
        // rarely; probabilities stay below 256, exact after the final
        // division by the row sum.
        if (__any(mx > m_run + 8.f)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < D / 32; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        }

        bf16x8 pf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[kb][r], scale_log2, -m_run));
                l_run += p;
                pf[kb][r >> 3][r & 7] = (bf16)p;
            }

#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const bf16x8 a = *(const bf16x8 *)(vs + S::VT::off(db * 32 + col, kb * 4 + 2 * s2 + half));
                    oacc[db] = mfma32(a, pf[kb][s2], oacc[db]);
                }
    };

    // Tiles [fa, fb] lie inside every row's segment and below every row's
    // diagonal and skip the mask; the tiles before and after evaluate it.
    // Separate loops keep the mask code out of the unmasked tiles entirely.
    const int fa = max(jt0, (ks_max + BN - 1) / BN);
    const int fb = min(jt1, t_first >= BN - 1 ? (t_first - (BN - 1)) / BN : -1);
    using dyn = std::integral_constant<int, -1>;
    using s0 = std::integral_constant<int, 0>;
    using s1 = std::integral_constant<int, 1>;
    int jt = jt0;
    for (; jt <= jt1 && jt < fa; ++jt) tile_step(jt, std::true_type{}, dyn{});
    // Unmasked tiles in pairs, so that each tile's LDS slot is a constant and
    // its fragment reads take the slot offset as an immediate.
    if (jt <= fb && ((jt - jt0) & 1)) tile_step(jt++, std::false_type{}, s1{});
    for (; jt + 1 <= fb; jt += 2) {
        tile_step(jt, std::false_type{}, s0{});
        tile_step(jt + 1, std::false_type{}, s1{});
    }
    if (jt <= fb) tile_step(jt++, std::false_type{}, s0{});
    for (; jt <= jt1; ++jt) tile_step(jt, std::true_type{}, dyn{});

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    if (row_ok) {
        bf16 *orow = o + (size_t)t * o_st + h * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                bf16x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (bf16)(oacc[db][rg * 4 + i] * inv);
                *(bf16x4 *)(orow + db * 32 + rg * 8 + half * 4) = w;
            }
        if (half == 0) lse[(size_t)h * N + t] = (m_run + log2f(l_tot)) * SP_LN2;
    }
}

}  // namespace

hipError_t launch_attn_fwd(const void *q, const void *k, const void *v, const int64_t *pos,
                           int64_t N, int hq, int hkv, int d, float scale, void *o, float *lse,
                           const AttnStrides &st, const AttnWorkspace &ws, hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    hipError_t e = launch_segments(pos, ws.kstart, ws.kend, ws.seg_agg, N, stream);
    if (e != hipSuccess) return e;
    const int g = hq / hkv;
    const int M = (int)(N * g);
    const int n_row_tiles = (M + BM - 1) / BM;
    const FastDiv fg = make_fastdiv((uint32_t)g);
    const float scale_log2 = scale * SP_LOG2E;
    const int64_t n_pad = (N + BN - 1) / BN * BN;
    {
        const dim3 tgrid((unsigned)(n_pad / 64), (unsigned)hkv);
        KernelTimer timer("attn_fwd_v_transpose", stream);
        if (d == 128)
            hipLaunchKernelGGL(k_v_transpose<128>, tgrid, dim3(256), 0, stream, (const bf16 *)v,
                               (bf16 *)ws.vt, (int)N, n_pad, st.k);
        else
            hipLaunchKernelGGL(k_v_transpose<64>, tgrid, dim3(256), 0, stream, (const bf16 *)v,
                               (bf16 *)ws.vt, (int)N, n_pad, st.k);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const dim3 grid((unsigned)(n_row_tiles * hkv));
    KernelTimer timer("attn_fwd", stream);
    if (d == 128)
        hipLaunchKernelGGL(k_attn_fwd<128>, grid, dim3(kThreads), 0, stream, (const bf16 *)q,
                           (const bf16 *)k, (const bf16 *)ws.vt, n_pad, ws.kstart, (bf16 *)o,
                           lse, (int)N, hq, hkv, g, fg, scale_log2, n_row_tiles, st.q, st.k,
                           st.o);
    else
        hipLaunchKernelGGL(k_attn_fwd<64>, grid, dim3(kThreads), 0, stream, (const bf16 *)q,
                           (const bf16 *)k, (const bf16 *)ws.vt, n_pad, ws.kstart, (bf16 *)o,
                           lse, (int)N, hq, hkv, g, fg, scale_log2, n_row_tiles, st.q, st.k,
                           st.o);
    return hipGetLastError();
}
