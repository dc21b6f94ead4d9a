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
//  * k_attn_bwd_dkdv - a workgroup owns 128 keys of one KV head (4 pairs of
//    waves x 32 keys); K and V stay in registers as B operands, and the
//    pairs walk the virtual query rows that can see their keys (t in
//    [j0, segment end)) in tiles of 64, from the segment end down.
//    S = Q K^T and dP = dO V^T come out with one key per lane, so P and dS
//    feed dV^T += dO^T P and dK^T += Q^T dS directly; the dO^T and Q^T operands are transposing LDS
//    reads of the same Q and dO tiles.  The GQA sum over the query heads of
//    a KV head falls out of the virtual-row walk.
//  * k_attn_bwd_dq - a workgroup owns 256 virtual query rows (like the
//    forward); Q and dO stay in registers, K and V tiles stream through LDS,
//    and dQ^T += K^T dS^T accumulates per lane (K^T by transposing reads).
// Both stream their tiles through LDS rings filled by direct global->LDS
// loads issued ahead.  A pre-pass writes the row statistics lse * log2e and
// D per block of 32 virtual rows (32 of each, contiguous), so a row tile's
// statistics are one load and each role reads only the half it needs.
// Small grids run both kernels' work in one launch (k_attn_bwd_fused); the
// kernel bodies live in attn_bwd_dkdv.inc and attn_bwd_dq.inc, included by
// the standalone kernels and by the fused one.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tile.h"

namespace {

constexpr int kThreads = 256;
constexpr int BK = 128;  // keys per dK/dV workgroup
constexpr int TQ = 64;   // virtual query rows per dK/dV tile
constexpr int RB = TQ / 32;   // its blocks of 32 rows (one MFMA row block each)
constexpr int BM = 256;  // virtual query rows per dQ workgroup (8 waves x 32)
constexpr int kDqThreads = 512;
constexpr int BN = 128;  // keys per dQ tile

// ---------------------------------------------------------------------------
// Row statistics of virtual row v < Mpad of KV head kh, in blocks of 32 rows:
// with R = kh * Mpad + v, b = R / 32 and j = R % 32,
//     rowstat[64 b + j] = lse * log2e,   rowstat[64 b + 32 + j] = rowsum(dO * O).
// Rows past M get (+inf, 0), so their probabilities are exactly 0.  One group
// of D/8 lanes per row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void k_bwd_rowstats(const bf16 *__restrict__ o,
                                                           const bf16 *__restrict__ d_o,
                                                           const float *__restrict__ lse,
                                                           float *__restrict__ rowstat, int N,
                                                           int hq, int hkv, int g, FastDiv fg,
                                                           int Mpad, int64_t o_st, int64_t do_st) {
    constexpr int LPR = D / 8;
    const int64_t row = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / LPR;  // kh*Mpad + v
    const int c = threadIdx.x % LPR;
    const bool in_grid = row < (int64_t)hkv * Mpad;
    const int kh = in_grid ? (int)(row / Mpad) : 0;
    const int v = in_grid ? (int)(row - (int64_t)kh * Mpad) : 0;
    const bool ok = in_grid && v < N * g;
    float acc = 0.f;
    int t = 0, h = 0;
    if (ok) {
        t = (int)fdiv((uint32_t)v, fg);
        h = kh * g + (v - t * g);
        const bf16x8 a = *(const bf16x8 *)(o + (size_t)t * o_st + h * D + c * 8);
        const bf16x8 b = *(const bf16x8 *)(d_o + (size_t)t * do_st + h * D + c * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += (float)a[i] * (float)b[i];
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (in_grid && c == 0) {
        float *blk = rowstat + (row & ~(int64_t)31) * 2 + (row & 31);
        blk[0] = ok ? lse[(size_t)h * N + t] * SP_LOG2E : INFINITY;
        blk[32] = ok ? acc : 0.f;
    }
}

// ---------------------------------------------------------------------------
// dK, dV
//
// A workgroup owns BK = 128 keys of one KV head, split over 4 wave pairs of
// 32 keys; 8 waves, two per SIMD.  Wave "A" of a pair holds K
// and accumulates dV: S = Q K^T, P, then dV^T += dO^T P.  Wave "B" holds V
// and accumulates dK: dP = dO V^T, then, with P from A, dS = P * (dP - D)
// and dK^T += Q^T dS.  A hands P to B through LDS in bf16, lane for lane in
// the accumulator layout both waves share (S and dP are both [rows x keys]
// products).  Every Q / dO fragment read from LDS feeds one MFMA (two key
// blocks per wave would halve that traffic but need more registers than
// two waves per SIMD leave).  A query tile holds TQ = 64 rows (two row
// blocks of 32), so the per-tile costs (barrier, load waits, ring and slot
// bookkeeping) are paid once per 32 MFMAs of a wave; that size leaves LDS for
// a ring of 3 tiles: B's, A's (one ahead) and one in flight.
// ---------------------------------------------------------------------------
// Where the query rows (Q and dO) of the dK/dV kernel's KV head come from:
// virtual row v of KV head kh at byte offset
// kh * head_bytes + (v >> gshift) * tok_bytes + (v & (2^gshift - 1)) * d * 2;
// `rows` rows exist.
struct RowSource {
    int64_t q_head_bytes, do_head_bytes;
    uint32_t q_tok_bytes, do_tok_bytes;
    int gshift, rows;
};

constexpr int kDkdvStages = 3;   // LDS ring of query tiles
constexpr int kDkdvAhead = 2;    // tiles staged ahead of the tile B works on

template <int D>
struct DkdvSmem {
    static constexpr int kWaves = 8, kPairs = 4;
    using R = SwzTile<TQ, D / 8>;    // Q or dO rows of the tile
    static_assert(TQ * 8 % (kWaves * 16) == 0, "statistics split into 16-byte loads per wave");
    static constexpr int kStatLanes = TQ * 8 / (kWaves * 16);   // 16-byte stat loads per wave
    static constexpr int kQ = 0, kDO = R::kBytes, kStat = 2 * R::kBytes;
    static constexpr int kStage = kStat + TQ * 8;   // per 32-row block: lse2 of 32 rows, then D
    // P handed from A to B: [2 slots][pair][row block][2 halves][64 lanes] x
    // 16 bytes (a 16-byte lane stride keeps the exchange bank-conflict free)
    static constexpr int kP = kDkdvStages * kStage;
    static constexpr int kPSlot = kPairs * RB * 2 * 64 * 16;
    static constexpr int kBytes = kP + 2 * kPSlot;
    // direct loads per wave per tile: its share of the Q and dO rows, plus statistics
    __device__ static constexpr int loads(int wave) {
        int n = 0;
        for (int i = wave; i < R::kInstr; i += kWaves) ++n;
        return 2 * n + 1;
    }
};

// Wait until at most `pending` (0..2) tiles of this wave's direct loads are
// still in flight; PER is how many loads the wave issues per tile.
template <int PER>
__device__ __forceinline__ void wait_tiles(int pending) {
    // vmcnt(n) is encoded as 0x0F70 | n only for n < 16 (its high bits sit
    // elsewhere in the immediate)
    static_assert(2 * PER < 16, "vmcnt range of this encoding");
    if (pending == 0)
        __builtin_amdgcn_s_waitcnt(0x0F70);
    else if (pending == 1)
        __builtin_amdgcn_s_waitcnt(0x0F70 | PER);
    else
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * PER));
}

template <int D>
__global__ __launch_bounds__(512, 1) void k_attn_bwd_dkdv(
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, const bf16 *__restrict__ q_rows,
    const bf16 *__restrict__ do_rows, RowSource rs, const float *__restrict__ rowstat,
    const int32_t *__restrict__ kend, void *__restrict__ dk, void *__restrict__ dv, int N,
    int Mpad, int hkv, int g, FastDiv fg, float scale_log2, float scale, int out_f32,
    int64_t kv_st, int64_t dk_st, int64_t dv_st) {
    __shared__ __attribute__((aligned(1024))) char smem[DkdvSmem<D>::kBytes];
#define BWD_BLOCK blockIdx.x
#include "attn_bwd_dkdv.inc"
#undef BWD_BLOCK
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
struct DqSmem {
    using R = SwzTile<BN, D / 8>;    // K or V rows
    static constexpr int kK = 0, kV = R::kBytes;
    static constexpr int kStage = 2 * R::kBytes;
};

template <int D>
__global__ __launch_bounds__(kDqThreads, 1) void k_attn_bwd_dq(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ d_o, const float *__restrict__ rowstat,
    const int32_t *__restrict__ kstart, void *__restrict__ dq, int N, int Mpad, int hq, int hkv,
    int g, FastDiv fg,
    float scale_log2, float scale, int n_row_tiles, int out_f32, int64_t q_st, int64_t kv_st,
    int64_t do_st, int64_t dq_st) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * DqSmem<D>::kStage];
#define BWD_BLOCK blockIdx.x
#include "attn_bwd_dq.inc"
#undef BWD_BLOCK
}

// ---------------------------------------------------------------------------
// Both backward kernels in one launch, for grids too small to fill the chip
// several times over.  The dK/dV work of a key tile grows with the rows that
// see it, so in a short grid the workgroups of a long sample's first key
// tiles run long after the rest have finished, and a separate dQ launch
// cannot start until they have; here workgroups [0, n_dkdv) do the dK/dV
// work and the rest the dQ work, which fills the CUs the long dK/dV
// workgroups leave idle.  The two parts share no data (both read the row
// statistics), so the results are the separate kernels' bit for bit.
// (Large grids keep the separate kernels: there the gain is nil and the
// combined kernel's dK/dV part schedules slightly worse.)
// ---------------------------------------------------------------------------
template <int D>
constexpr int fused_smem_bytes() {
    return DkdvSmem<D>::kBytes > 2 * DqSmem<D>::kStage ? DkdvSmem<D>::kBytes
                                                       : 2 * DqSmem<D>::kStage;
}
static_assert(kDqThreads == 512, "both parts of the fused backward run 512 threads");

// at most this many dK/dV workgroups (two per CU of a 256-CU MI355X) take the
// fused launch
constexpr int kFuseMaxDkdvBlocks = 512;

template <int D>
__global__ __launch_bounds__(512, 1) void k_attn_bwd_fused(
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, const bf16 *__restrict__ q_rows,
    const bf16 *__restrict__ do_rows, RowSource rs, const float *__restrict__ rowstat,
    const int32_t *__restrict__ kend, void *__restrict__ dk, void *__restrict__ dv, int N,
    int Mpad, int hkv, int g, FastDiv fg, float scale_log2, float scale, int out_f32,
    int64_t kv_st, int64_t dk_st, int64_t dv_st, int n_dkdv, const bf16 *__restrict__ q,
    const bf16 *__restrict__ d_o, const int32_t *__restrict__ kstart, void *__restrict__ dq,
    int hq, int n_row_tiles, int64_t q_st, int64_t do_st, int64_t dq_st) {
    __shared__ __attribute__((aligned(1024))) char smem[fused_smem_bytes<D>()];
    if ((int)blockIdx.x < n_dkdv) {
#define BWD_BLOCK blockIdx.x
#include "attn_bwd_dkdv.inc"
#undef BWD_BLOCK
    } else {
#define BWD_BLOCK (blockIdx.x - (unsigned)n_dkdv)
#include "attn_bwd_dq.inc"
#undef BWD_BLOCK
    }
}

template <int D>
hipError_t bwd_launch(const void *q, const void *k, const void *v, const void *o,
                      const void *d_o, const float *lse, int64_t N, int hq, int hkv, float scale,
                      bool grad_f32, void *dq, void *dk, void *dv, const AttnStrides &st,
                      const AttnWorkspace &ws, hipStream_t stream) {
    const int g = hq / hkv;
    const int64_t M = N * g;
    const int64_t Mpad = (M + 63) / 64 * 64;
    const FastDiv fg = make_fastdiv((uint32_t)g);
    const float scale_log2 = scale * SP_LOG2E;
    hipError_t e;

    {
        const int64_t threads = (int64_t)hkv * Mpad * (D / 8);
        KernelTimer timer("bwd_rowstats", stream);
        hipLaunchKernelGGL(k_bwd_rowstats<D>, dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, (const bf16 *)o, (const bf16 *)d_o, lse,
                           ws.rowstat, (int)N, hq, hkv, g, fg, (int)Mpad, st.o, st.d_o);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // Query rows of a KV head: read in place when g divides 32, else gathered
    // into row-major virtual-row copies first.
    RowSource rs;
    const bf16 *q_rows, *do_rows;
    if (attn_rows_direct(hq, hkv)) {
        int gshift = 0;
        while ((1 << gshift) < g) ++gshift;
        q_rows = (const bf16 *)q;
        do_rows = (const bf16 *)d_o;
        rs = {(int64_t)g * D * 2, (int64_t)g * D * 2, (uint32_t)(st.q * 2), (uint32_t)(st.d_o * 2),
              gshift, (int)M};
    } else {
        if ((e = launch_gather_rows(q, st.q, ws.qv, N, hkv, g, D, Mpad, stream)) != hipSuccess) return e;
        if ((e = launch_gather_rows(d_o, st.d_o, ws.dov, N, hkv, g, D, Mpad, stream)) != hipSuccess) return e;
        q_rows = (const bf16 *)ws.qv;
        do_rows = (const bf16 *)ws.dov;
        rs = {Mpad * D * 2, Mpad * D * 2, (uint32_t)(D * 2), (uint32_t)(D * 2), 0, (int)Mpad};
    }

    const int n_key_tiles = (int)((N + BK - 1) / BK);
    const int n_row_tiles = (int)((M + BM - 1) / BM);
    const int n_dkdv = n_key_tiles * hkv;
    if (n_dkdv <= kFuseMaxDkdvBlocks) {
        KernelTimer timer("attn_bwd_fused", stream);
        hipLaunchKernelGGL((k_attn_bwd_fused<D>), dim3((unsigned)(n_dkdv + n_row_tiles * hkv)),
                           dim3(512), 0, stream, (const bf16 *)k, (const bf16 *)v, q_rows, do_rows,
                           rs, (const float *)ws.rowstat, (const int32_t *)ws.kend, dk, dv, (int)N,
                           (int)Mpad, hkv, g, fg, scale_log2, scale, (int)grad_f32, st.k, st.dk,
                           st.dv, n_dkdv, (const bf16 *)q, (const bf16 *)d_o,
                           (const int32_t *)ws.kstart, dq, hq, n_row_tiles, st.q, st.d_o, st.dq);
        return hipGetLastError();
    }
    {
        KernelTimer timer("attn_bwd_dkdv", stream);
        hipLaunchKernelGGL((k_attn_bwd_dkdv<D>), dim3((unsigned)n_dkdv),
                           dim3(512), 0, stream, (const bf16 *)k, (const bf16 *)v,
                           q_rows, do_rows, rs, (const float *)ws.rowstat,
                           (const int32_t *)ws.kend, dk, dv, (int)N, (int)Mpad, hkv, g, fg,
                           scale_log2, scale, (int)grad_f32, st.k, st.dk, st.dv);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;

    KernelTimer timer("attn_bwd_dq", stream);
    hipLaunchKernelGGL(k_attn_bwd_dq<D>, dim3((unsigned)(n_row_tiles * hkv)), dim3(kDqThreads), 0,
                       stream, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v,
                       (const bf16 *)d_o, (const float *)ws.rowstat, (const int32_t *)ws.kstart,
                       dq, (int)N, (int)Mpad, hq, hkv, g, fg, scale_log2, scale, n_row_tiles,
                       (int)grad_f32, st.q, st.k, st.d_o, st.dq);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                           const void *d_o, const float *lse, const int64_t *pos, int64_t N,
                           int hq, int hkv, int d, float scale, bool grad_f32, void *dq,
                           void *dk, void *dv, const AttnStrides &st, const AttnWorkspace &ws,
                           hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    hipError_t e = launch_segments(pos, ws.kstart, ws.kend, ws.seg_agg, N, stream);
    if (e != hipSuccess) return e;
    if (d == 128)
        return bwd_launch<128>(q, k, v, o, d_o, lse, N, hq, hkv, scale, grad_f32, dq, dk, dv, st,
                               ws, stream);
    return bwd_launch<64>(q, k, v, o, d_o, lse, N, hq, hkv, scale, grad_f32, dq, dk, dv, st, ws,
                          stream);
}
