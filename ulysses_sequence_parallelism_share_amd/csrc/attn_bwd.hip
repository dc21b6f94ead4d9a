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
    using S = DkdvSmem<D>;
    constexpr int W = S::kWaves, PAIRS = S::kPairs;
    __shared__ __attribute__((aligned(1024))) char smem[S::kBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave % PAIRS;
    const bool role_a = wave < PAIRS;
    const int col = lane & 31, half = lane >> 5;
    const int kh = blockIdx.x % hkv;
    const int j0 = (blockIdx.x / hkv) * BK;
    const int M = N * g;
    const int kw0 = j0 + pair * 32;               // the pair's first key
    const int kw1 = min(kw0 + 31, N - 1);         // and last (if kw0 < N)
    const bool pair_has_keys = kw0 < N;
    const int kend_w0 = pair_has_keys ? kend[kw0] : 0;
    const int kend_max = kend[min(j0 + BK, N) - 1];
    const int key = kw0 + col;                    // this lane's key
    const int my_kend = kend[key < N ? key : N - 1];

    // Rows [j0*g, kend_max*g) can see these keys; j0*g is a multiple of TQ.
    const int vq_lo = j0 * g;
    const int n_it = (kend_max * g - vq_lo + TQ - 1) / TQ;
    // Tiles are walked from the end of the range down to the diagonal: key
    // tiles of one sample share that end, so workgroups running side by side
    // read the same Q and dO rows at about the same time and share them in L2.
    auto tile_row = [&](int it) { return vq_lo + (n_it - 1 - it) * TQ; };
    // Virtual row v of KV head kh lies at byte offset kh * head_bytes +
    // (v >> gshift) * tok_bytes + (v & (2^gshift - 1)) * D * 2 of q_rows /
    // do_rows (`RowSource`); tiles start at multiples of 32 rows, hence at
    // token boundaries.  Rows past the end are read from the last row: finite
    // data, and their statistics make P exactly 0.
    RowStager<TQ, D / 8, W, false> stager_q, stager_do;
    stager_q.init(wave, lane, rs.q_tok_bytes, D * 2, rs.gshift);
    stager_do.init(wave, lane, rs.do_tok_bytes, D * 2, rs.gshift);
    const char *q_head = (const char *)q_rows + (size_t)kh * rs.q_head_bytes;
    const char *do_head = (const char *)do_rows + (size_t)kh * rs.do_head_bytes;
    auto stage = [&](int it, int buf) {
        char *base = smem + buf * S::kStage;
        const int vq0 = tile_row(it);
        const size_t tok0 = (size_t)(vq0 >> rs.gshift);
        stager_q.issue(base + S::kQ, wave, lane, q_head + tok0 * rs.q_tok_bytes, rs.rows - vq0);
        stager_do.issue(base + S::kDO, wave, lane, do_head + tok0 * rs.do_tok_bytes, rs.rows - vq0);
        if (lane < S::kStatLanes)   // every wave: its 16-byte pieces of the rows' statistics
            dma16((const void *)((const char *)(rowstat + ((size_t)kh * Mpad + vq0) * 2) +
                                 (wave * S::kStatLanes + lane) * 16),
                  (lds_byte *)(base + S::kStat + wave * S::kStatLanes * 16));
    };
    for (int i = 0; i < kDkdvAhead && i < n_it; ++i) stage(i, i);

    // This wave's B operand (K for A, V for B), lane = key.
    bf16x8 kv[D / 16];
    {
        const bf16 *src = role_a ? k : v;
        const bool ok = key < N;
        const size_t off = (size_t)(ok ? key : 0) * kv_st + kh * D + half * 8;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            bf16x8 a = *(const bf16x8 *)(src + off + 16 * st);
            if (!ok) {
#pragma unroll
                for (int i = 0; i < 8; ++i) a[i] = (bf16)0.f;
            }
            kv[st] = a;
        }
    }
    f32x16 acc[D / 32];   // dV^T (A) or dK^T (B): lane = key, registers = features
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    // A runs one tile ahead of B: in iteration `it`, A turns tile it+1 into P
    // (double-buffered exchange slot) and dV, while B turns tile it and A's P
    // of the previous iteration into dS and dK.  One barrier per iteration;
    // the two roles share no data inside an iteration.  Both roles run the
    // same MFMA code (only the operand tiles and the middle step differ), so
    // each accumulator is updated in place.
    const int rows1 = role_a ? S::kQ : S::kDO;     // rows of the first product (lane = key)
    const int rows2 = role_a ? S::kDO : S::kQ;     // rows read transposed for the second
    // Per-lane offsets of the transposing reads of a row tile (k-row base 0;
    // a k-row base of 16 adds 16 * stride, folded into the read's immediate).
    int tr_off[D / 32][2];
    {
        using R = typename S::R;
        const int G = lane >> 4, j = lane & 15;
        const int row = 4 * (G >> 1) + (j >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int m = db * 32 + 16 * (G & 1) + 4 * (j & 3);
            tr_off[db][0] = R::off(row, m >> 3) + (m & 7) * 2;
            tr_off[db][1] = R::off(row + 8, m >> 3) + (m & 7) * 2;
        }
    }
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    auto tr_read = [&](const char *tile, int db, int kb) {   // kb: k-row base, multiple of 16
        const char *p0 = tile + tr_off[db][0] + kb * S::R::kStride;
        const char *p1 = tile + tr_off[db][1] + kb * S::R::kStride;
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds_byte *)p0);
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds_byte *)p1);
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        return __builtin_bit_cast(bf16x8, v);
    };

    constexpr int PER_A = S::loads(0), PER_B = S::loads(W - 1);
    auto wait_for = [&](int pending) {   // this wave's loads per tile decide the count
        if (PER_A == PER_B || wave < S::R::kInstr % W || S::R::kInstr % W == 0)
            wait_tiles<PER_A>(pending);
        else
            wait_tiles<PER_B>(pending);
    };
    if (n_it > 0) wait_for(min(kDkdvAhead - 1, n_it - 1));   // tile 0
    int slot_a = 0, slot_st = kDkdvAhead - 1;   // ring slots of tile it+1 and of the next stage
    auto advance = [](int x) { return x + 1 == kDkdvStages ? 0 : x + 1; };
    // Iteration -1 runs A on tile 0 only; iteration it runs A on it+1, B on it.
    for (int it = -1; it < n_it; ++it) {
        if (it >= 0) wait_for(max(0, min(kDkdvAhead - 2, n_it - 2 - it)));   // tile it+1 for A
        __syncthreads();
        if (it >= 0 && it + kDkdvAhead < n_it) {
            slot_st = advance(slot_st);
            stage(it + kDkdvAhead, slot_st);
        }
        const int slot_b = slot_a == 0 ? kDkdvStages - 1 : slot_a - 1;
        const int t = role_a ? it + 1 : it;
        const int slot = role_a ? slot_a : slot_b;
        slot_a = advance(slot_a);
        if (t < 0 || t >= n_it) continue;
        const char *base = smem + slot * S::kStage;
        const int vq0 = tile_row(t);
        const float *stat = (const float *)(base + S::kStat);   // per row block: lse2 of 32 rows, then D
        // P slot: [pair][row block][2 halves][64 lanes]
        bf16x8 *ps = (bf16x8 *)(smem + S::kP + (t & 1) * S::kPSlot) + pair * RB * 128 + lane;

        // First product: S = Q K^T (A) or dP = dO V^T (B); lane = key.
        f32x16 x[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) x[rb][r] = 0.f;
        // The row fragments are read PF ahead of the MFMA that takes them
        // (sched_group_barrier pins that order: the compiler would otherwise
        // wait for each read right before its MFMA).
        {
            constexpr int NFR = (D / 16) * RB, PF = 6;
            bf16x8 fa[NFR];
#pragma unroll
            for (int f = 0; f < NFR; ++f)
                fa[f] = *(const bf16x8 *)(base + rows1 + S::R::off((f % RB) * 32 + col, 2 * (f / RB) + half));
#pragma unroll
            for (int f = 0; f < NFR; ++f) x[f % RB] = mfma32(fa[f], kv[f / RB], x[f % RB]);
            __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
            for (int f = 0; f < NFR - PF; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
        }

        // rows of accumulator register r: rg*8 + half*4 + i (r = rg*4 + i)
        bf16x8 opnd[RB][2];
        if (role_a) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int vb = vq0 + rb * 32;
                const float *l2s = stat + rb * 64;
                const int tq_first = (int)fdiv((uint32_t)min(vb, M - 1), fg);
                const int tq_last = (int)fdiv((uint32_t)(min(vb + 32, M) - 1), fg);
                // A pair whose pairs are all masked still runs (its P is exactly
                // 0); that happens only on the diagonal and at sample ends.
                const bool full = pair_has_keys && vb < M && (kw1 <= tq_first) && (tq_last < kend_w0);
                auto softmax = [&](auto masked) {
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int q0 = rg * 8 + half * 4;
                        const f32x4 l2 = *(const f32x4 *)(l2s + q0);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = rg * 4 + i;
                            int tq = 0;
                            if constexpr (decltype(masked)::value)
                                tq = (int)fdiv((uint32_t)(vb + q0 + i), fg);
                            float p = fast_exp2(fmaf(x[rb][r], scale_log2, -l2[i]));
                            if constexpr (decltype(masked)::value)
                                p = (key <= tq && tq < my_kend) ? p : 0.f;
                            opnd[rb][r >> 3][r & 7] = (bf16)p;
                        }
                    }
                };
                if (full)
                    softmax(std::false_type{});
                else
                    softmax(std::true_type{});
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                ps[rb * 128] = opnd[rb][0];
                ps[rb * 128 + 64] = opnd[rb][1];
            }
        } else {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const bf16x8 pb[2] = {ps[rb * 128], ps[rb * 128 + 64]};
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int q0 = rg * 8 + half * 4;
                    const f32x4 dl = *(const f32x4 *)(stat + rb * 64 + 32 + q0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = rg * 4 + i;
                        const float p = (float)pb[r >> 3][r & 7];
                        opnd[rb][r >> 3][r & 7] = (bf16)(p * (x[rb][r] - dl[i]));
                    }
                }
            }
        }

        // Second product: dV^T += dO^T P (A) or dK^T += Q^T dS (B).
        // Transposed fragments f = s2 * D/32 + db, read PF2 ahead; each
        // accumulator still sums its k-rows in ascending order.
        {
            constexpr int NF2 = (D / 32) * 2 * RB, PF2 = 4;
            bf16x8 fb[NF2];
#pragma unroll
            for (int f = 0; f < NF2; ++f) fb[f] = tr_read(base + rows2, f % (D / 32), 16 * (f / (D / 32)));
#pragma unroll
            for (int f = 0; f < NF2; ++f) {
                const int db = f % (D / 32), s2 = f / (D / 32);
                acc[db] = mfma32(fb[f], opnd[s2 >> 1][s2 & 1], acc[db]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF2, 1);
#pragma unroll
            for (int f = 0; f < NF2 - PF2; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, PF2, 1);
        }
    }

    if (key >= N) return;
    void *out = role_a ? dv : dk;
    const float mul = role_a ? 1.f : scale;
    const size_t obase = (size_t)key * (role_a ? dv_st : dk_st) + kh * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int e = db * 32 + rg * 8 + half * 4;
            if (out_f32) {
                f32x4 a;
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = acc[db][rg * 4 + i] * mul;
                *(f32x4 *)((float *)out + obase + e) = a;
            } else {
                bf16x4 a;
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = (bf16)(acc[db][rg * 4 + i] * mul);
                *(bf16x4 *)((bf16 *)out + obase + e) = a;
            }
        }
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
    using S = DqSmem<D>;
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
    RowStager<BN, D / 8, kDqThreads / 64> stager;
    stager.init(wave, lane, (uint32_t)(kv_st * 2), 0, 0);
    auto stage = [&](int jt, int buf) {
        char *base = smem + buf * S::kStage;
        const int j0 = jt * BN;
        const size_t roff = (size_t)j0 * kv_st + kh * D;
        stager.issue(base + S::kK, wave, lane, k + roff, N - j0);
        stager.issue(base + S::kV, wave, lane, v + roff, N - j0);
    };
    stage(jt0, 0);

    const float *blk = rowstat + ((size_t)kh * Mpad + (vr & ~31)) * 2 + (vr & 31);
    const float l2 = blk[0], dl = blk[32];
    bf16x8 qf[D / 16], dof[D / 16];
    {
        const bf16 *qrow = q + (size_t)t * q_st + h * D + half * 8;
        const bf16 *dorow = d_o + (size_t)t * do_st + h * D + half * 8;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            qf[s] = *(const bf16x8 *)(qrow + 16 * s);
            dof[s] = *(const bf16x8 *)(dorow + 16 * s);
        }
    }
    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[i][r] = 0.f;

    // One key tile; `masked` selects the code that evaluates the mask.
    auto tile_step = [&](int jt, auto masked) {
        const int j0 = jt * BN;
        wait_async();
        __syncthreads();
        if (jt < jt1) stage(jt + 1, (jt + 1 - jt0) & 1);
        const char *base = smem + ((jt - jt0) & 1) * S::kStage;

        // One 32-key block at a time: S^T and dP^T, then dS^T, then its part
        // of dQ^T (keeps the score registers of one block live; unrolled by
        // two, which the register budget still holds without spilling).
#pragma unroll 2
        for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
                const int off = S::R::off(kb * 32 + col, 2 * st + half);
                s = mfma32(*(const bf16x8 *)(base + S::kK + off), qf[st], s);
                dp = mfma32(*(const bf16x8 *)(base + S::kV + off), dof[st], dp);
            }
            bf16x8 dsf[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(fmaf(s[r], scale_log2, -l2));
                if constexpr (decltype(masked)::value) {
                    const int key = j0 + kb * 32 + acc_row(r, half);
                    p = (key >= my_ks && key <= t) ? p : 0.f;
                }
                dsf[r >> 3][r & 7] = (bf16)(p * (dp[r] - dl));
            }
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const bf16x8 a = read_tr8<typename S::R>(base + S::kK, kb * 32 + 16 * s2, db * 32, lane);
                    dqacc[db] = mfma32(a, dsf[s2], dqacc[db]);
                }
        }
    };

    // Tiles [fa, fb] lie inside every row's segment and below every row's
    // diagonal and skip the mask (separate loops keep the mask code out of
    // them entirely).
    const int fa = max(jt0, (ks_max + BN - 1) / BN);
    const int fb = min(jt1, t_first >= BN - 1 ? (t_first - (BN - 1)) / BN : -1);
    int jt = jt0;
    for (; jt <= jt1 && jt < fa; ++jt) tile_step(jt, std::true_type{});
    for (; jt <= fb; ++jt) tile_step(jt, std::false_type{});
    for (; jt <= jt1; ++jt) tile_step(jt, std::true_type{});

    if (!row_ok) return;
    const size_t obase = (size_t)t * dq_st + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int e = db * 32 + rg * 8 + half * 4;
            if (out_f32) {
                f32x4 a;
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = dqacc[db][rg * 4 + i] * scale;
                *(f32x4 *)((float *)dq + obase + e) = a;
            } else {
                bf16x4 a;
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = (bf16)(dqacc[db][rg * 4 + i] * scale);
                *(bf16x4 *)((bf16 *)dq + obase + e) = a;
            }
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

    {
        const int n_key_tiles = (int)((N + BK - 1) / BK);
        KernelTimer timer("attn_bwd_dkdv", stream);
        hipLaunchKernelGGL((k_attn_bwd_dkdv<D>), dim3((unsigned)(n_key_tiles * hkv)),
                           dim3(512), 0, stream, (const bf16 *)k, (const bf16 *)v,
                           q_rows, do_rows, rs, (const float *)ws.rowstat,
                           (const int32_t *)ws.kend, dk, dv, (int)N, (int)Mpad, hkv, g, fg,
                           scale_log2, scale, (int)grad_f32, st.k, st.dk, st.dv);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const int n_row_tiles = (int)((M + BM - 1) / BM);
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
