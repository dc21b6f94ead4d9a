// C ABI of the library: argument checks, workspace layout and launches.
// Every check runs on the host before anything is enqueued, so an invalid
// call returns an error without touching the device (and works on a host
// without a GPU).  The rules follow the pages' problem statement: the
// sequence is padded to a multiple of sp_size and the head count must be
// divisible by sp_size (Transformers guide "Ulysses sequence parallelism",
// "Configuration"); masking comes from position_ids only.
#include <math.h>

#include <initializer_list>
#include <mutex>

#include "../../include/ulysses_sp.h"
#include "launch.h"

namespace {

inline bool misaligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

constexpr int64_t kMaxRows = (int64_t)1 << 30;  // token and virtual-row indices stay in int32

// a0 * a1 * ... < lim, for non-negative factors, without overflow (the
// running product stays below lim < 2^63 before each multiply, so it fits
// in 128 bits)
inline bool prod_below(std::initializer_list<int64_t> factors, int64_t lim) {
    __int128 p = 1;
    for (int64_t f : factors) {
        p *= f;
        if (p >= lim) return false;
    }
    return true;
}

sp_status check_relayout(const void *src, const void *dst, int P, int64_t N, int G, int H, int d,
                         int rank) {
    if (P < 1 || N < 0 || G < 1 || H < 1 || d < 1) return SP_E_SHAPE;
    if (N % P != 0 || H % P != 0) return SP_E_NOT_DIVISIBLE;
    if (rank < -1 || rank >= P) return SP_E_RANK;
    const int64_t piece = (int64_t)(H / P) * d;
    if (piece % 8 != 0) return SP_E_SHAPE;
    // a token's G*H*d/8 16-byte vectors are indexed in 24 bits
    if (N >= kMaxRows || !prod_below({G, H, d}, (int64_t)1 << 27)) return SP_E_SHAPE;
    if (N == 0) return SP_OK;
    if (src == nullptr || dst == nullptr) return SP_E_NULL;
    if (misaligned(src, 16) || misaligned(dst, 16)) return SP_E_ALIGN;
    return SP_OK;
}

// K/V exchange: n_kv and sp_size must divide one another; 16-byte chunks.
sp_status check_kv_relayout(const void *src, const void *dst, int P, int64_t N, int G, int H,
                            int d, int rank) {
    if (P < 1 || N < 0 || G < 1 || H < 1 || d < 1) return SP_E_SHAPE;
    if (N % P != 0) return SP_E_NOT_DIVISIBLE;
    if ((H >= P && H % P != 0) || (H < P && P % H != 0)) return SP_E_NOT_DIVISIBLE;
    if (rank < -1 || rank >= P) return SP_E_RANK;
    if (d % 8 != 0) return SP_E_SHAPE;
    const int64_t hl = H >= P ? H / P : 1;
    const int64_t lim = (int64_t)1 << 31;   // 16-byte chunk indices in 31 bits
    if (!prod_below({N, hl, d / 8}, lim) || !prod_below({N, H, d / 8}, lim) ||
        !prod_below({N / P, G, H, d / 8}, lim) || (int64_t)P * G > 65535)
        return SP_E_SHAPE;
    if (N == 0) return SP_OK;
    if (src == nullptr || dst == nullptr) return SP_E_NULL;
    if (misaligned(src, 16) || misaligned(dst, 16)) return SP_E_ALIGN;
    return SP_OK;
}

sp_status check_attn_shape(int64_t N, int hq, int hkv, int d, float scale) {
    if (N < 0 || hq < 1 || hkv < 1) return SP_E_SHAPE;
    if (d != 64 && d != 128) return SP_E_SHAPE;
    if (hq % hkv != 0) return SP_E_NOT_DIVISIBLE;
    if (!prod_below({N, hq}, kMaxRows)) return SP_E_SHAPE;
    // Tile rows are addressed by 32-bit byte offsets from the tile base; the
    // longest span is the forward's V^T tile: head_dim rows of the transposed
    // copy, (n_tokens rounded up to 64) keys each.
    if ((int64_t)d * ((N + 63) / 64 * 64) * 2 > ((int64_t)1 << 32)) return SP_E_SHAPE;
    if (!(scale >= 0.f) || isinf(scale)) return SP_E_SHAPE;
    return SP_OK;
}

// A token stride (in elements) must cover the token's heads, keep 16-byte
// vectors aligned and keep a tile's row offsets within 32 bits.
constexpr int64_t kMaxStride = (int64_t)1 << 24;
inline bool bad_stride(int64_t stride, int heads, int d) {
    return stride < (int64_t)heads * d || stride % 8 != 0 || stride > kMaxStride;
}

// The cross-entropy's dX product stages 256-token rows of the bf16 softmax
// gradient G ([chunk][vocab rounded up to 256]) with 32-bit byte offsets from
// the tile base: 255 * v_pad * 2 + 127 must stay below 2^32, which holds for
// v_pad <= 8421376 (a multiple of 256), so the vocabulary is limited to that.
constexpr int64_t kMaxLceVocab = 8421376;

// The loss kernels index tokens with 64-bit integers; the grid arithmetic
// adds a workgroup's worth to the count, so counts stay below 2^48.
constexpr int64_t kMaxLossTokens = (int64_t)1 << 48;

inline int64_t pad64(int64_t x) { return (x + 63) / 64 * 64; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t attn_workspace_layout(int64_t N, int hq, int hkv, int d, void *base, AttnWorkspace *ws,
                             bool with_vt) {
    const int g = hq / hkv;
    const int64_t Mpad = pad64(N * g);
    size_t off = 0;
    char *b = (char *)base;
    auto take = [&](size_t bytes) {
        char *p = b ? b + off : nullptr;
        off += align256(bytes);
        return (void *)p;
    };
    AttnWorkspace w;
    w.kstart = (int32_t *)take(4 * (size_t)N);
    w.kend = (int32_t *)take(4 * (size_t)N);
    w.seg_agg = (int32_t *)take(4 * segments_scratch_ints(N));
    const bool gather = !attn_rows_direct(hq, hkv);
    w.qv = gather ? take(2 * (size_t)hkv * d * Mpad) : nullptr;
    w.dov = gather ? take(2 * (size_t)hkv * d * Mpad) : nullptr;
    w.rowstat = (float *)take(8 * (size_t)hkv * Mpad);
    w.vt = with_vt ? take(2 * (size_t)hkv * d * pad64(N)) : nullptr;
    if (ws) *ws = w;
    return off;
}

// ---------------------------------------------------------------------------
// Fixed device scratch for sp_attn_bwd_noalloc: the backward's workspace
// (segment bounds, row statistics, gathered rows) taken from this array
// instead of a caller buffer.  Every GPU the library runs on holds its own
// copy at its own address for the life of the process.  In host code the
// array's name is only a stand-in for the symbol, so its device address is
// looked up once per device with hipGetSymbolAddress and kept; kernels get
// that address.  No part of the scratch needs to start at zero (the segment
// pass, the row-statistics pass and the row gather write everything the
// later kernels read), and calls that overlap on one GPU share, and race on,
// the array.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on its first use).
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

// Checks and launches of the backward, shared by the workspace and the
// scratch entry points.  With `workspace` NULL and use_scratch set, the
// workspace comes from the device's scratch array.
sp_status attn_bwd_checked(const void *q, int64_t q_stride, const void *k, const void *v,
                           int64_t kv_stride, const void *o, int64_t o_stride, const void *d_o,
                           int64_t do_stride, const float *lse, const int64_t *position_ids,
                           int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                           float softmax_scale, int grad_dtype, void *dq, int64_t dq_stride,
                           void *dk, int64_t dk_stride, void *dv, int64_t dv_stride,
                           void *workspace, size_t workspace_bytes, bool use_scratch,
                           hipStream_t stream) {
    sp_status st = check_attn_shape(n_tokens, n_q_heads, n_kv_heads, head_dim, softmax_scale);
    if (st != SP_OK) return st;
    if (grad_dtype != SP_DTYPE_BF16 && grad_dtype != SP_DTYPE_F32) return SP_E_DTYPE;
    if (bad_stride(q_stride, n_q_heads, head_dim) || bad_stride(kv_stride, n_kv_heads, head_dim) ||
        bad_stride(o_stride, n_q_heads, head_dim) || bad_stride(do_stride, n_q_heads, head_dim) ||
        bad_stride(dq_stride, n_q_heads, head_dim) || bad_stride(dk_stride, n_kv_heads, head_dim) ||
        bad_stride(dv_stride, n_kv_heads, head_dim))
        return SP_E_SHAPE;
    // the scratch must hold the backward's part of the workspace (checked
    // before anything touches the device)
    const size_t need = attn_workspace_layout(n_tokens, n_q_heads, n_kv_heads, head_dim, nullptr,
                                              nullptr, !use_scratch);
    if (use_scratch && need > kNoAllocScratchBytes) return SP_E_SCRATCH;
    if (n_tokens == 0) return SP_OK;
    if (!q || !k || !v || !o || !d_o || !lse || !position_ids || !dq || !dk || !dv) return SP_E_NULL;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(d_o, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) ||
        misaligned(position_ids, 8) || misaligned(lse, 4))
        return SP_E_ALIGN;
    if (use_scratch) {
        if (scratch_address(&workspace) != hipSuccess) return SP_E_HIP;
    } else {
        if (!workspace || workspace_bytes < need) return SP_E_WORKSPACE;
        if (misaligned(workspace, 16)) return SP_E_ALIGN;
    }
    AttnWorkspace ws;
    attn_workspace_layout(n_tokens, n_q_heads, n_kv_heads, head_dim, workspace, &ws, !use_scratch);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
    const AttnStrides strides{q_stride, kv_stride, o_stride, do_stride, dq_stride, dk_stride, dv_stride};
    return launch_attn_bwd(q, k, v, o, d_o, lse, position_ids, n_tokens, n_q_heads, n_kv_heads,
                           head_dim, scale, grad_dtype == SP_DTYPE_F32, dq, dk, dv, strides, ws,
                           stream) == hipSuccess ? SP_OK : SP_E_HIP;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

const char *sp_status_string(int status) {
    switch (status) {
        case SP_OK: return "ok";
        case SP_E_NULL: return "a required pointer is NULL";
        case SP_E_SHAPE: return "a size is negative or unsupported";
        case SP_E_NOT_DIVISIBLE: return "n_tokens or n_heads not divisible by sp_size, or query heads not divisible by KV heads";
        case SP_E_ALIGN: return "a pointer is not suitably aligned";
        case SP_E_RANK: return "rank outside [-1, sp_size)";
        case SP_E_WORKSPACE: return "workspace missing or too small";
        case SP_E_HIP: return "a HIP launch failed";
        case SP_E_DTYPE: return "unknown element type";
        case SP_E_SCRATCH: return "the call needs more scratch than the library's fixed device array holds";
        default: return "unknown status";
    }
}

int sp_abi_version(void) { return 1; }

sp_status ulysses_seq_to_head(const void *x_seq, void *x_head, int sp_size, int64_t n_tokens,
                              int n_groups, int n_heads, int head_dim, int rank,
                              hipStream_t stream) {
    sp_status st = check_relayout(x_seq, x_head, sp_size, n_tokens, n_groups, n_heads, head_dim, rank);
    if (st != SP_OK || n_tokens == 0) return st;
    return launch_relayout(true, x_seq, x_head, sp_size, n_tokens, n_groups, n_heads, head_dim,
                           rank, stream) == hipSuccess ? SP_OK : SP_E_HIP;
}

sp_status ulysses_head_to_seq(const void *x_head, void *x_seq, int sp_size, int64_t n_tokens,
                              int n_groups, int n_heads, int head_dim, int rank,
                              hipStream_t stream) {
    sp_status st = check_relayout(x_head, x_seq, sp_size, n_tokens, n_groups, n_heads, head_dim, rank);
    if (st != SP_OK || n_tokens == 0) return st;
    return launch_relayout(false, x_head, x_seq, sp_size, n_tokens, n_groups, n_heads, head_dim,
                           rank, stream) == hipSuccess ? SP_OK : SP_E_HIP;
}

sp_status ulysses_seq_to_head_kv(const void *x_seq, void *x_head, int sp_size, int64_t n_tokens,
                                 int n_groups, int n_kv_heads, int head_dim, int rank,
                                 hipStream_t stream) {
    sp_status st = check_kv_relayout(x_seq, x_head, sp_size, n_tokens, n_groups, n_kv_heads,
                                     head_dim, rank);
    if (st != SP_OK || n_tokens == 0) return st;
    return launch_kv_seq_to_head(x_seq, x_head, sp_size, n_tokens, n_groups, n_kv_heads, head_dim,
                                 rank, stream) == hipSuccess ? SP_OK : SP_E_HIP;
}

sp_status ulysses_head_to_seq_kv_grad(const void *x_head, void *x_seq, int sp_size,
                                      int64_t n_tokens, int n_groups, int n_kv_heads,
                                      int head_dim, int dtype, int rank, hipStream_t stream) {
    if (dtype != SP_DTYPE_BF16 && dtype != SP_DTYPE_F32) return SP_E_DTYPE;
    sp_status st = check_kv_relayout(x_head, x_seq, sp_size, n_tokens, n_groups, n_kv_heads,
                                     head_dim, rank);
    if (st != SP_OK || n_tokens == 0) return st;
    return launch_kv_head_to_seq_sum(x_head, x_seq, sp_size, n_tokens, n_groups, n_kv_heads,
                                     head_dim, dtype == SP_DTYPE_F32, rank, stream) == hipSuccess
               ? SP_OK : SP_E_HIP;
}

size_t sp_attn_workspace_bytes(int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim) {
    if (check_attn_shape(n_tokens, n_q_heads, n_kv_heads, head_dim, 0.f) != SP_OK) return 0;
    return attn_workspace_layout(n_tokens, n_q_heads, n_kv_heads, head_dim, nullptr, nullptr);
}

sp_status sp_attn_fwd_strided(const void *q, int64_t q_stride, const void *k, const void *v,
                              int64_t kv_stride, const int64_t *position_ids, int64_t n_tokens,
                              int n_q_heads, int n_kv_heads, int head_dim, float softmax_scale,
                              void *o, int64_t o_stride, float *lse, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    sp_status st = check_attn_shape(n_tokens, n_q_heads, n_kv_heads, head_dim, softmax_scale);
    if (st != SP_OK) return st;
    if (bad_stride(q_stride, n_q_heads, head_dim) || bad_stride(kv_stride, n_kv_heads, head_dim) ||
        bad_stride(o_stride, n_q_heads, head_dim))
        return SP_E_SHAPE;
    if (n_tokens == 0) return SP_OK;
    if (!q || !k || !v || !position_ids || !o || !lse) return SP_E_NULL;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(position_ids, 8) || misaligned(lse, 4))
        return SP_E_ALIGN;
    const size_t need = attn_workspace_layout(n_tokens, n_q_heads, n_kv_heads, head_dim, nullptr, nullptr);
    if (!workspace || workspace_bytes < need) return SP_E_WORKSPACE;
    if (misaligned(workspace, 16)) return SP_E_ALIGN;
    AttnWorkspace ws;
    attn_workspace_layout(n_tokens, n_q_heads, n_kv_heads, head_dim, workspace, &ws);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
    const AttnStrides strides{q_stride, kv_stride, o_stride, 0, 0, 0, 0};
    return launch_attn_fwd(q, k, v, position_ids, n_tokens, n_q_heads, n_kv_heads, head_dim,
                           scale, o, lse, strides, ws, stream) == hipSuccess ? SP_OK : SP_E_HIP;
}

sp_status sp_attn_fwd(const void *q, const void *k, const void *v, const int64_t *position_ids,
                      int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                      float softmax_scale, void *o, float *lse, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    const int64_t sq = (int64_t)n_q_heads * head_dim, skv = (int64_t)n_kv_heads * head_dim;
    return sp_attn_fwd_strided(q, sq, k, v, skv, position_ids, n_tokens, n_q_heads, n_kv_heads,
                               head_dim, softmax_scale, o, sq, lse, workspace, workspace_bytes,
                               stream);
}

sp_status sp_attn_bwd_strided(const void *q, int64_t q_stride, const void *k, const void *v,
                              int64_t kv_stride, const void *o, int64_t o_stride, const void *d_o,
                              int64_t do_stride, const float *lse, const int64_t *position_ids,
                              int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                              float softmax_scale, int grad_dtype, void *dq, int64_t dq_stride,
                              void *dk, int64_t dk_stride, void *dv, int64_t dv_stride,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return attn_bwd_checked(q, q_stride, k, v, kv_stride, o, o_stride, d_o, do_stride, lse,
                            position_ids, n_tokens, n_q_heads, n_kv_heads, head_dim,
                            softmax_scale, grad_dtype, dq, dq_stride, dk, dk_stride, dv, dv_stride,
                            workspace, workspace_bytes, false, stream);
}

sp_status sp_attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *d_o,
                      const float *lse, const int64_t *position_ids, int64_t n_tokens,
                      int n_q_heads, int n_kv_heads, int head_dim, float softmax_scale,
                      int grad_dtype, void *dq, void *dk, void *dv, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    const int64_t sq = (int64_t)n_q_heads * head_dim, skv = (int64_t)n_kv_heads * head_dim;
    return sp_attn_bwd_strided(q, sq, k, v, skv, o, sq, d_o, sq, lse, position_ids, n_tokens,
                               n_q_heads, n_kv_heads, head_dim, softmax_scale, grad_dtype, dq, sq,
                               dk, skv, dv, skv, workspace, workspace_bytes, stream);
}

sp_status sp_attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                              const void *d_o, const float *lse, const int64_t *position_ids,
                              int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                              float softmax_scale, int grad_dtype, void *dq, void *dk, void *dv,
                              hipStream_t stream) {
    const int64_t sq = (int64_t)n_q_heads * head_dim, skv = (int64_t)n_kv_heads * head_dim;
    return attn_bwd_checked(q, sq, k, v, skv, o, sq, d_o, sq, lse, position_ids, n_tokens,
                            n_q_heads, n_kv_heads, head_dim, softmax_scale, grad_dtype, dq, sq,
                            dk, skv, dv, skv, nullptr, 0, true, stream);
}

size_t sp_linear_ce_workspace_bytes(int64_t vocab, int64_t chunk_tokens) {
    if (vocab < 1 || vocab > kMaxLceVocab || chunk_tokens < 64 || chunk_tokens % 64 != 0 ||
        chunk_tokens >= ((int64_t)1 << 24))
        return 0;
    return lce_workspace_layout(vocab, chunk_tokens, nullptr, nullptr);
}

sp_status sp_linear_ce(const void *x, const void *w, const int64_t *labels, int64_t ignore_index,
                       const float *d_token_loss, int64_t n_tokens, int64_t vocab, int64_t hidden,
                       int grad_dtype, float *token_loss, float *lse, void *dx, float *dw,
                       int64_t chunk_tokens, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    if (n_tokens < 0 || vocab < 1 || vocab > kMaxLceVocab || hidden < 256 ||
        hidden % 256 != 0 || hidden > 65536 || n_tokens >= ((int64_t)1 << 31))
        return SP_E_SHAPE;
    if (chunk_tokens < 64 || chunk_tokens % 64 != 0 || chunk_tokens >= ((int64_t)1 << 24))
        return SP_E_SHAPE;
    if ((size_t)vocab * hidden >= ((size_t)1 << 40)) return SP_E_SHAPE;
    if (grad_dtype != SP_DTYPE_BF16 && grad_dtype != SP_DTYPE_F32) return SP_E_DTYPE;
    if (n_tokens == 0) return SP_OK;
    if (!x || !w || !labels || !token_loss || !lse) return SP_E_NULL;
    if (d_token_loss && (!dx || !dw)) return SP_E_NULL;
    if (misaligned(x, 16) || misaligned(w, 16) || misaligned(labels, 8) ||
        misaligned(token_loss, 4) || misaligned(lse, 4) || misaligned(d_token_loss, 4) ||
        misaligned(dx, 16) || misaligned(dw, 16))
        return SP_E_ALIGN;
    const size_t need = lce_workspace_layout(vocab, chunk_tokens, nullptr, nullptr);
    if (!workspace || workspace_bytes < need) return SP_E_WORKSPACE;
    if (misaligned(workspace, 256)) return SP_E_ALIGN;
    LceWorkspace ws;
    lce_workspace_layout(vocab, chunk_tokens, workspace, &ws);
    return launch_linear_ce(x, w, labels, ignore_index, d_token_loss, n_tokens, vocab, hidden,
                            grad_dtype == SP_DTYPE_F32, token_loss, lse, dx, dw, chunk_tokens, ws,
                            stream) == hipSuccess ? SP_OK : SP_E_HIP;
}

sp_status sp_weighted_loss(const float *token_loss, const int64_t *shift_labels, int sp_size,
                           int64_t n_tokens, int64_t ignore_index, float *loss, float *rank_loss,
                           int64_t *good_tokens, float *d_token_loss, hipStream_t stream) {
    if (sp_size < 1 || n_tokens < 0 || n_tokens >= kMaxLossTokens) return SP_E_SHAPE;
    if (n_tokens % sp_size != 0) return SP_E_NOT_DIVISIBLE;
    if (!loss || !rank_loss || !good_tokens) return SP_E_NULL;
    if (n_tokens > 0 && (!token_loss || !shift_labels)) return SP_E_NULL;
    if (misaligned(token_loss, 4) || misaligned(shift_labels, 8) || misaligned(loss, 4) ||
        misaligned(rank_loss, 4) || misaligned(good_tokens, 8) || misaligned(d_token_loss, 4))
        return SP_E_ALIGN;
    return launch_weighted_loss(token_loss, shift_labels, sp_size, n_tokens, ignore_index, loss,
                                rank_loss, good_tokens, d_token_loss, stream) == hipSuccess
               ? SP_OK : SP_E_HIP;
}

}  // extern "C"
#pragma GCC visibility pop
