// Host-side launchers of the gfx950 kernels (internal to the library).  All
// arguments have been validated by the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// RAII: brackets one kernel launch with HIP events on its stream when the
// library's timing mode is on (sp_timing_enable); otherwise does nothing.
class KernelTimer {
  public:
    KernelTimer(const char *name, hipStream_t s);
    ~KernelTimer();
    KernelTimer(const KernelTimer &) = delete;
    KernelTimer &operator=(const KernelTimer &) = delete;

  private:
    const char *name_;
    hipStream_t s_;
    hipEvent_t a_, b_;
};

hipError_t launch_relayout(bool to_head, const void *src, void *dst, int P, int64_t N, int G,
                           int H, int d, int rank, hipStream_t stream);

hipError_t launch_kv_seq_to_head(const void *x_seq, void *x_head, int P, int64_t N, int G, int H,
                                 int d, int rank, hipStream_t stream);
hipError_t launch_kv_head_to_seq_sum(const void *x_head, void *x_seq, int P, int64_t N, int G,
                                     int H, int d, bool f32, int rank, hipStream_t stream);

hipError_t launch_gather_rows(const void *src, int64_t src_stride, void *dst, int64_t N, int n_kv,
                              int g, int D, int64_t rows_pad, hipStream_t stream);

// Scratch ints the segment pre-pass needs for N tokens (per-chunk aggregates).
size_t segments_scratch_ints(int64_t N);
hipError_t launch_segments(const int64_t *pos, int32_t *kstart, int32_t *kend, int32_t *agg,
                           int64_t N, hipStream_t stream);

// Token strides (in elements) of the attention tensors: element (t, h, e)
// of q lies at q[t * q + h * d + e], and so on.  k and v share one stride.
struct AttnStrides {
    int64_t q, k, o, d_o, dq, dk, dv;
};

// Workspace layout shared by the forward and backward calls.
struct AttnWorkspace {
    int32_t *kstart;   // [N]
    int32_t *kend;     // [N]
    int32_t *seg_agg;  // segment pre-pass chunk aggregates
    void *qv;          // bwd, groups not dividing 32: Q in virtual-row order  [hkv][Mpad][d]
    void *dov;         // bwd, groups not dividing 32: dO in virtual-row order [hkv][Mpad][d]
    float *rowstat;    // bwd: lse*log2e and rowsum(dO*O) per 32-row block [hkv][Mpad/32][2][32]
    void *vt;          // fwd: V transposed, keys permuted within groups of 16 [hkv][d][Npad]
};

// Lays the workspace out from `base` (nullptr: sizes only) and returns its
// size; with_vt = false leaves out the forward's transposed V (vt = nullptr),
// which the backward does not use.
size_t attn_workspace_layout(int64_t N, int hq, int hkv, int d, void *base, AttnWorkspace *ws,
                             bool with_vt = true);

// The dK/dV kernel reads query rows of one KV head straight from q and dO
// when its g = hq/hkv query heads per token are a power of two dividing 32
// (then every block of 32 rows, and so every tile, starts at a token
// boundary); otherwise they are
// gathered into the workspace first.
inline bool attn_rows_direct(int hq, int hkv) { return 32 % (hq / hkv) == 0; }

hipError_t launch_attn_fwd(const void *q, const void *k, const void *v, const int64_t *pos,
                           int64_t N, int hq, int hkv, int d, float scale, void *o, float *lse,
                           const AttnStrides &st, const AttnWorkspace &ws, hipStream_t stream);

hipError_t launch_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                           const void *d_o, const float *lse, const int64_t *pos, int64_t N,
                           int hq, int hkv, int d, float scale, bool grad_f32, void *dq,
                           void *dk, void *dv, const AttnStrides &st, const AttnWorkspace &ws,
                           hipStream_t stream);

// Workspace of the fused linear cross-entropy: one chunk of fp32 logits and
// of the bf16 softmax gradient, both [rows][v_pad] with v_pad = vocab rounded
// up to 256.
struct LceWorkspace {
    float *logits;
    void *g;
    int64_t v_pad;
};

size_t lce_workspace_layout(int64_t vocab, int64_t chunk, void *base, LceWorkspace *ws);

hipError_t launch_linear_ce(const void *x, const void *w, const int64_t *labels,
                            int64_t ignore_index, const float *g, int64_t N, int64_t V, int64_t K,
                            bool dx_f32, float *token_loss, float *lse, void *dx, float *dw,
                            int64_t chunk, const LceWorkspace &ws, hipStream_t stream);

hipError_t launch_weighted_loss(const float *token_loss, const int64_t *labels, int P, int64_t N,
                                int64_t ignore_index, float *loss, float *rank_loss,
                                int64_t *good, float *d_token_loss, hipStream_t stream);
