/*
 * ulysses_sp.h - C ABI of the MI355X (gfx950) library for one rank's share of
 * a Ulysses sequence-parallel attention layer.
 *
 * Sources for what each call computes (page titles and sections):
 *  [T] Transformers guide "Ulysses sequence parallelism": introduction and its
 *      two-GPU figure; section "Configuration" (heads divisible by sp_size,
 *      sequences padded to a multiple of sp_size, position_ids instead of a
 *      4D mask, FlashAttention correct on packed samples).
 *  [A] Accelerate guide "Sequence parallelism in accelerate": section
 *      "ALST/Ulysses SP backend configuration" (sp_attn_implementation item;
 *      the loss-aggregation loop with shift_labels and ignore index -100).
 *  [B] Blog "Ulysses Sequence Parallelism: Training with Million-Token
 *      Contexts": "How Ulysses works" steps 1-6 (contiguous token chunks, the
 *      two all-to-alls, heads independent); "Loss aggregation".
 *
 * Conventions for every call
 *  - All pointers are device pointers unless stated otherwise.  The caller
 *    allocates and owns every buffer, including the workspace; the library
 *    never allocates, frees, copies host<->device or synchronises, and keeps
 *    no state between calls (apart from the opt-in timing records at the end).
 *  - Work is enqueued on `stream` (NULL = the default stream) and runs
 *    asynchronously; results are valid once the stream has reached that point.
 *  - Every argument is checked on the host before anything is enqueued.  On an
 *    error nothing is launched and outputs are left untouched.  SP_E_HIP
 *    reports a failed launch (outputs are then undefined).
 *  - bf16 tensors are 16-bit bfloat16 values; element sizes are as stated.
 *  - Pointer alignment: bf16 tensors and the workspace 16 bytes; int64
 *    tensors 8 bytes; fp32 tensors 4 bytes (else SP_E_ALIGN).
 *  - Calls that race on overlapping output buffers on concurrent streams are
 *    the caller's responsibility.
 */
#ifndef ULYSSES_SP_H
#define ULYSSES_SP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sp_status {
    SP_OK = 0,
    SP_E_NULL = 1,           /* a required pointer is NULL */
    SP_E_SHAPE = 2,          /* a size is negative or unsupported */
    SP_E_NOT_DIVISIBLE = 3,  /* n_tokens % sp_size, n_heads % sp_size or hq % hkv != 0 */
    SP_E_ALIGN = 4,          /* a pointer breaks the alignment rule above */
    SP_E_RANK = 5,           /* rank outside [-1, sp_size) */
    SP_E_WORKSPACE = 6,      /* workspace NULL or smaller than sp_attn_workspace_bytes() */
    SP_E_HIP = 7,            /* a HIP launch failed */
    SP_E_DTYPE = 8,          /* unknown sp_dtype */
    SP_E_SCRATCH = 9         /* sp_attn_bwd_noalloc: more scratch than its fixed array holds */
} sp_status;

typedef enum sp_dtype {
    SP_DTYPE_BF16 = 0,
    SP_DTYPE_F32 = 1
} sp_dtype;

/* Short English description of a status code (static storage; never NULL). */
const char *sp_status_string(int status);

/* Version of this ABI (incremented on any signature change). */
int sp_abi_version(void);

/*
 * ulysses_seq_to_head - the first all-to-all of [T]'s figure and [B] step 3,
 * emulated on one GPU over all sp_size rank buffers.
 *
 * Rank p holds the contiguous token chunk [p*N/P, (p+1)*N/P) for all heads
 * ([B] step 1).  After the exchange rank q holds all N tokens for the head
 * block [q*H/P, (q+1)*H/P) ([T] figure: GPU 0 gets heads 0..H/2):
 *     x_head[q][g][p*N/P + t][hl][e] = x_seq[p][t][g][q*H/P + hl][e]
 *
 *   x_seq    [sp_size][n_tokens/sp_size][n_groups][n_heads][head_dim]  bf16 (read)
 *   x_head   rank == -1: [sp_size][n_groups][n_tokens][n_heads/sp_size][head_dim]
 *            rank ==  r: [n_groups][n_tokens][n_heads/sp_size][head_dim]
 *            (rank r's share only)                                      bf16 (written)
 *   n_heads  GLOBAL head count of this tensor family (Hq for Q, Hkv for K/V);
 *   n_groups number of same-shaped tensors fused per token (3 for QKV when
 *            Hq == Hkv; 1 for Q, O, dO; 2 for K/V).
 * Bits are moved verbatim (NaN payloads, -0 and subnormals preserved).
 * Errors: SP_E_NOT_DIVISIBLE if n_tokens or n_heads is not a multiple of
 * sp_size ([T] "Configuration"); SP_E_SHAPE if (n_heads/sp_size)*head_dim is
 * not a multiple of 8 elements (16 bytes), or a size is < 0 / sp_size < 1;
 * SP_E_RANK; SP_E_NULL; SP_E_ALIGN.  n_tokens == 0 is a no-op.
 * x_seq and x_head must not overlap.
 */
sp_status ulysses_seq_to_head(const void *x_seq, void *x_head, int sp_size, int64_t n_tokens,
                              int n_groups, int n_heads, int head_dim, int rank,
                              hipStream_t stream);

/*
 * ulysses_head_to_seq - the second all-to-all ([T] figure, [B] step 5): the
 * exact inverse permutation of ulysses_seq_to_head, same arguments and
 * layouts with source and destination swapped.  With rank == r only rank
 * r's head columns [r*H/P, (r+1)*H/P) of x_seq are written; every other byte
 * of x_seq is left untouched.
 */
sp_status ulysses_head_to_seq(const void *x_head, void *x_seq, int sp_size, int64_t n_tokens,
                              int n_groups, int n_heads, int head_dim, int rank,
                              hipStream_t stream);

/*
 * ulysses_seq_to_head_kv - the seq->head exchange of a K/V-like tensor with
 * n_kv_heads KV heads, also when there are fewer KV heads than ranks.
 *
 * The pages ask for head counts divisible by sp_size ([T] "Configuration")
 * and do not treat grouped-query models with fewer KV heads than ranks.
 * Query head h uses KV head h / (Hq / n_kv_heads), so rank q's query heads
 * all use KV head (q * n_kv_heads) / sp_size; with n_kv_heads < sp_size
 * (sp_size a multiple of n_kv_heads) each KV head is copied to the
 * sp_size / n_kv_heads ranks that use it.  With n_kv_heads >= sp_size
 * (n_kv_heads a multiple of sp_size) this is ulysses_seq_to_head.
 *
 *   x_seq   [sp_size][n_tokens/sp_size][n_groups][n_kv_heads][head_dim]  (read)
 *   x_head  rank == -1: [sp_size][n_groups][n_tokens][hl][head_dim]
 *           rank ==  r: [n_groups][n_tokens][hl][head_dim]   (written)
 *   with hl = max(n_kv_heads / sp_size, 1); rank q holds KV heads
 *   [(q*n_kv_heads)/sp_size, ... + hl).  Elements are 16-bit and moved
 *   verbatim.  head_dim must be a multiple of 8 (SP_E_SHAPE); n_kv_heads and
 *   sp_size must divide one another and n_tokens % sp_size == 0
 *   (SP_E_NOT_DIVISIBLE); pointers 16-byte aligned.  SP_E_SHAPE also when
 *   n_tokens * n_kv_heads * head_dim / 8 reaches 2^31 or sp_size * n_groups
 *   exceeds 65535.
 */
sp_status ulysses_seq_to_head_kv(const void *x_seq, void *x_head, int sp_size, int64_t n_tokens,
                                 int n_groups, int n_kv_heads, int head_dim, int rank,
                                 hipStream_t stream);

/*
 * ulysses_head_to_seq_kv_grad - the head->seq exchange of K/V gradients:
 * the adjoint of ulysses_seq_to_head_kv.  Every rank that received a copy
 * of a KV head contributes its gradient and the copies are summed:
 *   x_seq[p][t][g][j][e] = sum over ranks q holding head j (ascending q) of
 *                          x_head[q][g][p*N/P + t][j - (q*n_kv)/P][e]
 * in fp32, rounded once to the element type.
 *
 *   x_head  [sp_size][n_groups][n_tokens][hl][head_dim]  (read; all ranks)
 *   x_seq   rank == -1: [sp_size][n_tokens/sp_size][n_groups][n_kv_heads][head_dim]
 *           rank ==  r: rank r's tokens only, [n_tokens/sp_size][n_groups][n_kv_heads][head_dim]
 *   dtype   SP_DTYPE_BF16 or SP_DTYPE_F32: element type of both buffers
 *           (else SP_E_DTYPE)
 * Other errors as for ulysses_seq_to_head_kv.  Deterministic.
 */
sp_status ulysses_head_to_seq_kv_grad(const void *x_head, void *x_seq, int sp_size,
                                      int64_t n_tokens, int n_groups, int n_kv_heads,
                                      int head_dim, int dtype, int rank, hipStream_t stream);

/*
 * sp_attn_workspace_bytes - size of the device workspace sp_attn_fwd and
 * sp_attn_bwd need for these sizes (the same buffer serves both calls; its
 * contents need no initialisation and are not preserved).  Returns 0 for
 * invalid sizes.
 */
size_t sp_attn_workspace_bytes(int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim);

/*
 * sp_attn_fwd - exact causal attention of one rank's heads over the full
 * sequence ([B] step 4; heads independent, same section).
 *
 * Masking comes from position_ids alone, never from a 4D mask ([T]
 * "Configuration"; [A] sp_attn_implementation item): a packed sample starts
 * at token 0 and at every token whose position_id is 0; query i attends to
 * key j iff both lie in the same sample and j <= i.  Query head h uses KV
 * head h / (n_q_heads / n_kv_heads).
 *
 *   q             [n_tokens][n_q_heads][head_dim]   bf16 (read)
 *   k, v          [n_tokens][n_kv_heads][head_dim]  bf16 (read)
 *   position_ids  [n_tokens]                        int64 (read; any values
 *                 are accepted, the rule above defines the mask)
 *   softmax_scale > 0: used as given; 0: 1/sqrt(head_dim)
 *   o             [n_tokens][n_q_heads][head_dim]   bf16 (written)
 *   lse           [n_q_heads][n_tokens]             fp32 (written):
 *                 natural-log log-sum-exp of the scaled scores of each row
 *                 (consumed by sp_attn_bwd)
 *   workspace     >= sp_attn_workspace_bytes(...) bytes of device memory
 * n_q_heads and n_kv_heads are the LOCAL (per-rank) head counts.
 * head_dim must be 64 or 128 (else SP_E_SHAPE); n_q_heads % n_kv_heads != 0
 * gives SP_E_NOT_DIVISIBLE.  Size limits (else SP_E_SHAPE): n_tokens *
 * n_q_heads < 2^30, and head_dim * (n_tokens rounded up to 64) * 2 <= 2^32,
 * i.e. at most 16,777,216 tokens at head_dim 128 (33,554,432 at 64); the
 * same limits apply to sp_attn_bwd.  n_tokens == 0 is a no-op.
 * Arithmetic: bf16 MFMA products with fp32 accumulation and an fp32 online
 * softmax; probabilities are rounded to bf16 before the product with V.
 */
sp_status sp_attn_fwd(const void *q, const void *k, const void *v, const int64_t *position_ids,
                      int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                      float softmax_scale, void *o, float *lse,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sp_attn_bwd - gradients of sp_attn_fwd for an upstream gradient d_o.
 *
 * With P the attention probabilities (rebuilt from q, k and lse):
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_e dO_ie O_ie,  dS = P * (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q;
 * dK and dV of a KV head sum over the query heads that share it.
 *
 *   q, k, v, position_ids, softmax_scale: as passed to sp_attn_fwd
 *   o, lse        outputs of sp_attn_fwd for those inputs (read)
 *   d_o           [n_tokens][n_q_heads][head_dim]   bf16 (read)
 *   grad_dtype    SP_DTYPE_F32 or SP_DTYPE_BF16: element type of dq, dk, dv
 *   dq            [n_tokens][n_q_heads][head_dim]   (written)
 *   dk, dv        [n_tokens][n_kv_heads][head_dim]  (written)
 *   workspace     as for sp_attn_fwd
 * Errors as for sp_attn_fwd, plus SP_E_DTYPE.  Results are deterministic
 * (no atomics): repeated calls give identical bits.
 */
sp_status sp_attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *d_o,
                      const float *lse, const int64_t *position_ids,
                      int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                      float softmax_scale, int grad_dtype, void *dq, void *dk, void *dv,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sp_attn_bwd_noalloc - sp_attn_bwd without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  It allocates nothing:
 * the workspace comes from a fixed device array of 32 MiB inside the library
 * (one per GPU, held until the process ends; its device address is looked up
 * on the first call on each device).
 *
 * Arguments, layouts, arithmetic and results are those of sp_attn_bwd, bit
 * for bit.  The backward's part of the workspace must fit the array: with
 * M = n_tokens * (n_q_heads / n_kv_heads) rounded up to 64, about
 * 8 * n_tokens + 8 * n_kv_heads * M bytes (plus 4 * n_kv_heads * head_dim * M
 * when n_q_heads / n_kv_heads does not divide 32), e.g. 20 MiB for 524288
 * tokens with 4 query heads and 1 KV head; a larger call returns SP_E_SCRATCH
 * before anything touches the device.  Every call on one GPU uses that GPU's
 * array (nothing in it needs to start at zero): calls that overlap on one GPU,
 * on different streams or from different threads, race and give undefined
 * results.  The current HIP device must be the one `stream` belongs to.
 */
sp_status sp_attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                              const void *d_o, const float *lse, const int64_t *position_ids,
                              int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                              float softmax_scale, int grad_dtype, void *dq, void *dk, void *dv,
                              hipStream_t stream);

/*
 * sp_attn_fwd_strided, sp_attn_bwd_strided - sp_attn_fwd and sp_attn_bwd on
 * tensors whose tokens lie a given stride apart: element (t, h, e) of q is
 * at q[t * q_stride + h * head_dim + e], and likewise for k and v
 * (kv_stride, shared), o, d_o, dq, dk and dv.  Strides are in elements (of
 * the tensor's own type), at least heads * head_dim, multiples of 8 and at
 * most 2^24; otherwise SP_E_SHAPE.  Everything else (arguments, layouts of
 * lse and position_ids, errors, arithmetic, determinism) is as for the
 * unstrided calls, which are these calls with the packed strides
 * (n_q_heads * head_dim, n_kv_heads * head_dim); results are bit-identical
 * to theirs on the same values.
 *
 * Purpose: the seq->head exchange ([T] two-GPU figure; [B] "How Ulysses
 * works", steps 1-3) gives rank r the heads [r*H/P, (r+1)*H/P) of every
 * token.  Where the gathered tokens sit in one buffer [N][G][H][d] (the
 * exchange buffer laid out token-major), rank r's q, k and v are that
 * buffer at head offset r*H/P (plus g*H*d for the g-th tensor of a fused
 * group) with stride G*H*d, so attention can read them, and write o and the
 * gradients back, in place of separate relayout passes.
 */
sp_status sp_attn_fwd_strided(const void *q, int64_t q_stride, const void *k, const void *v,
                              int64_t kv_stride, const int64_t *position_ids, int64_t n_tokens,
                              int n_q_heads, int n_kv_heads, int head_dim, float softmax_scale,
                              void *o, int64_t o_stride, float *lse, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);
sp_status sp_attn_bwd_strided(const void *q, int64_t q_stride, const void *k, const void *v,
                              int64_t kv_stride, const void *o, int64_t o_stride, const void *d_o,
                              int64_t do_stride, const float *lse, const int64_t *position_ids,
                              int64_t n_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                              float softmax_scale, int grad_dtype, void *dq, int64_t dq_stride,
                              void *dk, int64_t dk_stride, void *dv, int64_t dv_stride,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sp_linear_ce_workspace_bytes - workspace sp_linear_ce needs for this
 * vocabulary size and token chunk (0 for invalid sizes, including a vocab
 * above 8421376).
 */
size_t sp_linear_ce_workspace_bytes(int64_t vocab, int64_t chunk_tokens);

/*
 * sp_linear_ce - per-token cross-entropy of the logits x w^T against labels,
 * and its gradients, without holding the logits of more than one chunk of
 * tokens: the fused logit-loss the pages recommend for long sequences ([A]
 * "ALST/Ulysses SP backend configuration", the note after the loss loop;
 * [B] "Loss aggregation").  Its token losses feed sp_weighted_loss.
 *
 *   x            [n_tokens][hidden] bf16 (read): hidden states of this
 *                rank's tokens
 *   w            [vocab][hidden] bf16 (read): LM-head matrix
 *   labels       [n_tokens] int64 (read): target ids (shift_labels);
 *                ignore_index marks tokens without a loss; any other value
 *                outside [0, vocab) gives a NaN loss and no gradient
 *   d_token_loss [n_tokens] fp32 (read) or NULL: upstream gradient g of the
 *                token losses.  For the token-weighted loss it is
 *                sp_weighted_loss's d_token_loss (1/T on valid tokens), which
 *                depends only on the labels.  NULL: forward only.
 *   token_loss   [n_tokens] fp32 (written): lse_t - x_t.w_{y_t} (0 if ignored)
 *   lse          [n_tokens] fp32 (written): log sum_v exp(x_t.w_v)
 *   dx           [n_tokens][hidden] (written if d_token_loss): G w, with
 *                G_tv = g_t (softmax_v - [v == y_t]); fp32 or bf16 by grad_dtype
 *   dw           [vocab][hidden] fp32 (written if d_token_loss): G^T x
 *   chunk_tokens tokens per chunk: a positive multiple of 64; the workspace
 *                holds that many rows of fp32 logits and bf16 G
 *   workspace    >= sp_linear_ce_workspace_bytes(vocab, chunk_tokens) bytes,
 *                256-byte aligned
 * hidden must be a positive multiple of 256 (<= 65536) and vocab at most
 * 8421376 (the 256-token tiles of G are addressed with 32-bit byte offsets:
 * 255 rows of vocab rounded up to 256 bf16 values), else SP_E_SHAPE.
 * Arithmetic: bf16 MFMA products with fp32 accumulation; fp32 log-sum-exp;
 * G rounded to bf16 for the two gradient products.  Deterministic.
 */
sp_status sp_linear_ce(const void *x, const void *w, const int64_t *labels, int64_t ignore_index,
                       const float *d_token_loss, int64_t n_tokens, int64_t vocab, int64_t hidden,
                       int grad_dtype, float *token_loss, float *lse, void *dx, float *dw,
                       int64_t chunk_tokens, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * sp_weighted_loss - token-weighted aggregation of per-rank losses ([A]
 * "ALST/Ulysses SP backend configuration", the loss loop; [B] "Loss
 * aggregation"), for all sp_size ranks at once.
 *
 *   token_loss    [sp_size][n_tokens/sp_size]  fp32 (read): per-token loss;
 *                 rank r owns tokens [r*N/P, (r+1)*N/P)
 *   shift_labels  [sp_size][n_tokens/sp_size]  int64 (read): a token is
 *                 valid iff its label != ignore_index (the pages use -100)
 *   loss          [1]        fp32 (written): sum over ranks with good_r > 0 of
 *                 rank_loss_r * good_r, divided by max(sum_r good_r, 1)
 *   rank_loss     [sp_size]  fp32 (written): mean loss over rank r's valid
 *                 tokens; NaN for a rank with none (such a rank is skipped
 *                 in `loss`, so its NaN never reaches it)
 *   good_tokens   [sp_size]  int64 (written): valid-token count per rank
 *   d_token_loss  [sp_size][n_tokens/sp_size]  fp32 (written; may be NULL):
 *                 d loss / d token_loss = 1/max(T,1) on valid tokens, else 0
 * Errors: SP_E_NOT_DIVISIBLE if n_tokens % sp_size; SP_E_SHAPE if sp_size < 1
 * or n_tokens is negative or at least 2^48; SP_E_NULL; SP_E_ALIGN.  With n_tokens == 0 the outputs are
 * loss 0, rank_loss NaN and good_tokens 0.
 */
sp_status sp_weighted_loss(const float *token_loss, const int64_t *shift_labels, int sp_size,
                           int64_t n_tokens, int64_t ignore_index, float *loss, float *rank_loss,
                           int64_t *good_tokens, float *d_token_loss, hipStream_t stream);

/*
 * Per-kernel timing (a profiling aid, not part of the computation).
 *
 * sp_timing_enable(1) makes every later kernel launch of this library record
 * a pair of HIP events around itself on its own stream (and drops earlier
 * records); sp_timing_enable(0) stops recording.  Returns the previous
 * setting.  This is the only process-wide state of the library.
 *
 * sp_timing_collect waits for the recorded events, aggregates them per
 * kernel name into `out` (up to max_entries entries), clears the records and
 * returns the number of distinct kernels, or -1 if an event could not be
 * read.  With out == NULL it only returns the count and keeps the records.
 * `out` is host memory.
 */
typedef struct sp_kernel_time {
    char name[48];
    int64_t launches;
    double total_ms;
    double min_ms;
    double max_ms;
} sp_kernel_time;

int sp_timing_enable(int on);
int sp_timing_collect(sp_kernel_time *out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_SP_H */
