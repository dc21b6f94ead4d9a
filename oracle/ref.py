"""CPU oracle for one rank's share of a Ulysses attention layer (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and never imports it; the library never falls back to it.

Every function is the plain definition of what the step computes, written
out in float64 with no blocking beyond what is stated:

* relayout - index arithmetic of the all-to-all that swaps sequence sharding
  for head sharding (Transformers guide "Ulysses sequence parallelism",
  introduction and its two-GPU figure; blog "Ulysses Sequence Parallelism:
  Training with Million-Token Contexts", "How Ulysses works", steps 1, 3, 5).
  For fewer KV heads than ranks (on which the pages are silent) the exchange
  copies each KV head to the ranks whose query heads use it, and the
  gradient exchange sums the copies (its adjoint).
* mask - causal attention within each packed sample, with sample boundaries
  read from position_ids rather than a 4D mask (Transformers guide,
  "Configuration", the sp_attn_implementation item; Accelerate guide
  "Sequence parallelism in accelerate", "ALST/Ulysses SP backend
  configuration", the sp_attn_implementation item; blog, "Loss aggregation"
  paragraph on position_ids).
* attention forward/backward - standard softmax attention for each local
  head (blog, "How Ulysses works", step 4; heads independent, same section).
* weighted loss - the token-weighted aggregation of per-rank losses
  (Accelerate guide, "ALST/Ulysses SP backend configuration", the loss
  aggregation loop; blog, "Loss aggregation").

Readings taken where the pages are silent (the pages give no formulas for
these): a sample starts at index 0 and wherever position_ids is 0; causality
is by sequence index within a sample; softmax scale defaults to 1/sqrt(d);
LSE uses the natural log; query head h uses KV head h // (hq/hkv); rank r
holds tokens [r*N/P, (r+1)*N/P) and heads [r*H/P, (r+1)*H/P); a rank's loss is
the mean over its valid tokens.

Parity pins: see tests/test_oracle.py (brute force, closed forms,
invariants, finite differences).  Every function here is pinned there.
"""
from __future__ import annotations

import math

import numpy as np

IGNORE_INDEX = -100


# ---------------------------------------------------------------------------
# bf16 <-> float64
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening: put the 16 bits in the top half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Relayout: the all-to-all as a permutation of bits
# ---------------------------------------------------------------------------

def seq_to_head(x_seq: np.ndarray, rank: int = -1) -> np.ndarray:
    """Sequence-sharded [P][N/P][G][H][d] -> head-sharded layout.

    Rank p holds tokens [p*N/P, (p+1)*N/P) for all H heads; after the
    exchange rank q holds all N tokens for heads [q*H/P, (q+1)*H/P):
        out[q][g][p*N/P + t][hl][e] = x_seq[p][t][g][q*H/P + hl][e]
    rank == -1 returns all ranks, [P][G][N][H/P][d]; rank == r returns rank
    r's share, [G][N][H/P][d].  Bits are moved verbatim.
    """
    P, T, G, H, d = x_seq.shape
    if H % P:
        raise ValueError("heads not divisible by sp_size")
    hl = H // P
    v = x_seq.reshape(P, T, G, P, hl, d)          # [p][t][g][q][hl][e]
    out = v.transpose(3, 2, 0, 1, 4, 5)           # [q][g][p][t][hl][e]
    out = np.ascontiguousarray(out).reshape(P, G, P * T, hl, d)
    return out if rank < 0 else np.ascontiguousarray(out[rank])


def head_to_seq(x_head: np.ndarray, sp_size: int, rank: int = -1,
                out: np.ndarray | None = None) -> np.ndarray:
    """Inverse of seq_to_head.  rank == r takes rank r's share [G][N][H/P][d]
    and writes only head columns [r*H/P, (r+1)*H/P) of ``out`` (created as
    zeros if not given)."""
    P = sp_size
    if rank < 0:
        _, G, N, hl, d = x_head.shape
        T = N // P
        v = x_head.reshape(P, G, P, T, hl, d)     # [q][g][p][t][hl][e]
        return np.ascontiguousarray(v.transpose(2, 3, 1, 0, 4, 5)).reshape(P, T, G, P * hl, d)
    G, N, hl, d = x_head.shape
    T = N // P
    if out is None:
        out = np.zeros((P, T, G, P * hl, d), dtype=x_head.dtype)
    v = x_head.reshape(G, P, T, hl, d)            # [g][p][t][hl][e]
    out[:, :, :, rank * hl:(rank + 1) * hl, :] = v.transpose(1, 2, 0, 3, 4)
    return out


def kv_head_start(n_kv: int, sp_size: int, rank: int) -> int:
    """First KV head rank ``rank`` holds.  With n_kv >= sp_size it holds the
    block [r*n_kv/P, (r+1)*n_kv/P); with fewer KV heads than ranks (P a
    multiple of n_kv) it holds the single KV head its query heads use: query
    heads [r*Hq/P, (r+1)*Hq/P) all map to KV head r // (P/n_kv) when query
    head h uses KV head h // (Hq/n_kv).  Both are (r*n_kv) // P."""
    return (rank * n_kv) // sp_size


def seq_to_head_kv(x_seq: np.ndarray, rank: int = -1) -> np.ndarray:
    """The seq->head exchange of K/V-like tensors, also for fewer KV heads than
    ranks (then each KV head is sent to the P/n_kv ranks that use it):
        out[q][g][p*N/P + t][i][e] = x_seq[p][t][g][kv_head_start(q) + i][e]
    for i < hl = max(n_kv/P, 1).  x_seq is [P][N/P][G][n_kv][d]; rank == -1
    returns [P][G][N][hl][d], rank == r rank r's [G][N][hl][d].  Bits are
    moved verbatim."""
    P, T, G, H, d = x_seq.shape
    if (H >= P and H % P) or (H < P and P % H):
        raise ValueError("KV heads and sp_size must divide one another")
    hl = max(H // P, 1)
    out = np.empty((P, G, P * T, hl, d), dtype=x_seq.dtype)
    for q in range(P):
        h0 = kv_head_start(H, P, q)
        part = x_seq[:, :, :, h0:h0 + hl, :]                     # [p][t][g][i][e]
        out[q] = part.transpose(2, 0, 1, 3, 4).reshape(G, P * T, hl, d)
    return out if rank < 0 else np.ascontiguousarray(out[rank])


def _bf16_bits_round(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite input)."""
    b = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def head_to_seq_kv_sum(x_head: np.ndarray, n_kv: int, rank: int = -1,
                       bf16_bits: bool = False) -> np.ndarray:
    """The head->seq exchange of K/V gradients: the adjoint of seq_to_head_kv.
    Every rank that received a copy of KV head j contributes its gradient, and
    the copies are summed:
        out[p][t][g][j][e] = sum over ranks q holding head j, ascending q, of
                             x_head[q][g][p*N/P + t][j - kv_head_start(q)][e].
    x_head is [P][G][N][hl][d].  The sum runs in float32 for float32 and bf16
    input (bf16_bits=True: uint16 bit patterns, widened exactly, the float32
    sum rounded once to bf16, nearest-even) and in float64 for float64 input.
    rank == r returns only rank r's tokens, [N/P][G][n_kv][d]."""
    P, G, N, hl, d = x_head.shape
    T = N // P
    if bf16_bits:
        xs = (x_head.astype(np.uint32) << 16).view(np.float32)
        acc_t = np.float32
    else:
        xs = x_head
        acc_t = np.float64 if x_head.dtype == np.float64 else np.float32
    acc = np.zeros((P, T, G, n_kv, d), dtype=acc_t)
    for q in range(P):                                          # ascending rank order
        h0 = kv_head_start(n_kv, P, q)
        part = xs[q].reshape(G, P, T, hl, d).transpose(1, 2, 0, 3, 4).astype(acc_t)
        acc[:, :, :, h0:h0 + hl, :] += part
    out = _bf16_bits_round(acc) if bf16_bits else acc.astype(x_head.dtype)
    return out if rank < 0 else np.ascontiguousarray(out[rank])


def gather_share(x_seq: np.ndarray, rank: int, g0: int = 0, g1: int | None = None) -> np.ndarray:
    """Rank ``rank``'s head block of groups [g0, g1) as a token-major
    [N][G'][H/P][d] array (the layout attention consumes)."""
    P, T, G, H, d = x_seq.shape
    g1 = G if g1 is None else g1
    hl = H // P
    s = x_seq[:, :, g0:g1, rank * hl:(rank + 1) * hl, :]
    return np.ascontiguousarray(s).reshape(P * T, g1 - g0, hl, d)


# ---------------------------------------------------------------------------
# Segments and the mask
# ---------------------------------------------------------------------------

def segment_ids(position_ids: np.ndarray) -> np.ndarray:
    """A new sample starts at token 0 and at every token whose position_id is 0."""
    pos = np.asarray(position_ids)
    start = (pos == 0)
    if start.size:
        start[0] = True
    return np.cumsum(start) - 1


def segment_first(position_ids: np.ndarray) -> np.ndarray:
    """Index of the first token of each token's sample (from the segment ids)."""
    seg = segment_ids(position_ids)
    n = seg.size
    firsts = np.flatnonzero(np.r_[True, seg[1:] != seg[:-1]]) if n else np.zeros(0, np.int64)
    return firsts[seg] if n else np.zeros(0, np.int64)


def allowed(seg: np.ndarray, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Explicit boolean mask block: query i may see key j iff they lie in the
    same sample and j <= i."""
    rows = np.asarray(rows)[:, None]
    cols = np.asarray(cols)[None, :]
    return (seg[rows] == seg[cols]) & (cols <= rows)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _as_f64(x):
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float64)


def _scale(d, softmax_scale):
    return 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)


def _row_blocks(n, seg, first, block_rows):
    """Yield (rows, cols): a block of consecutive query rows and the key span
    [first token of the block's first sample, last row].  Keys outside it are
    masked for every row of the block, so they contribute exact zeros."""
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        c0 = int(first[r0])
        yield np.arange(r0, r1), np.arange(c0, r1)


def _probs(qh, kh, seg, rows, cols, scale):
    """Row softmax of scale*q k^T over the explicit mask: returns P, m, l."""
    S = scale * (qh[rows] @ kh[cols].T)
    S[~allowed(seg, rows, cols)] = -np.inf
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return E / l, m[:, 0], l[:, 0]


def attn_fwd(q, k, v, position_ids, softmax_scale=None, block_rows=256):
    """O = softmax(scale q k^T + mask) v and LSE = log sum exp(scale q k) over
    allowed keys, per local query head.

    q: [N][hq][d], k, v: [N][hkv][d] (bf16 bits or floats).  Returns
    o [N][hq][d] and lse [hq][N], float64."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    N, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    scale = _scale(d, softmax_scale)
    seg = segment_ids(position_ids)
    first = segment_first(position_ids)
    o = np.zeros((N, hq, d))
    lse = np.zeros((hq, N))
    for h in range(hq):
        kv = h // grp
        qh, kh, vh = q[:, h], k[:, kv], v[:, kv]
        for rows, cols in _row_blocks(N, seg, first, block_rows):
            P, m, l = _probs(qh, kh, seg, rows, cols, scale)
            o[rows, h] = P @ vh[cols]
            lse[h, rows] = m + np.log(l)
    return o, lse


def attn_bwd(q, k, v, do, position_ids, softmax_scale=None, block_rows=256, o=None):
    """Gradients of sum(dO * O) with respect to q, k, v (float64).

    With P the attention probabilities: dV = P^T dO, dP = dO v^T,
    D_i = sum_j P_ij dP_ij, dS = P * (dP - D), dQ = scale dS k,
    dK = scale dS^T q; dK/dV of a KV head sum over the query heads that
    share it.

    ``o`` (optional, [N][hq][d], bf16 bits or floats): a stored forward output
    to form D from instead, D_i = sum_e dO_ie o_ie, the way a backward that is
    handed the layer's output computes it.  With the exact output this is the
    same D (sum_j P_ij dP_ij = dO_i . sum_j P_ij v_j); with a rounded one it is
    the gradient such a backward reaches."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    o = None if o is None else _as_f64(o)
    N, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    scale = _scale(d, softmax_scale)
    seg = segment_ids(position_ids)
    first = segment_first(position_ids)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        kv = h // grp
        qh, kh, vh, doh = q[:, h], k[:, kv], v[:, kv], do[:, h]
        for rows, cols in _row_blocks(N, seg, first, block_rows):
            P, _, _ = _probs(qh, kh, seg, rows, cols, scale)
            dv[cols, kv] += P.T @ doh[rows]
            dP = doh[rows] @ vh[cols].T
            if o is None:
                D = (P * dP).sum(axis=1, keepdims=True)
            else:
                D = (doh[rows] * o[rows, h]).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[rows, h] = scale * (dS @ kh[cols])
            dk[cols, kv] += scale * (dS.T @ qh[rows])
    return dq, dk, dv


def attn_rows(q, k, v, do, position_ids, rows, softmax_scale=None, chunk=64):
    """O, LSE and dQ for selected query rows only (each row's full softmax
    over all its allowed keys).  Returns o [R][hq][d], lse [hq][R],
    dq [R][hq][d] (dq is None when do is None)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    do = None if do is None else _as_f64(do)
    N, hq, d = q.shape
    grp = hq // k.shape[1]
    scale = _scale(d, softmax_scale)
    seg = segment_ids(position_ids)
    first = segment_first(position_ids)
    rows = np.asarray(rows, dtype=np.int64)
    R = rows.size
    o = np.zeros((R, hq, d))
    lse = np.zeros((hq, R))
    dq = None if do is None else np.zeros((R, hq, d))
    for c0 in range(0, R, chunk):
        sel = np.arange(c0, min(R, c0 + chunk))
        rr = rows[sel]
        cols = np.arange(int(first[rr].min()), int(rr.max()) + 1)
        for h in range(hq):
            kv = h // grp
            P, m, l = _probs(q[:, h], k[:, kv], seg, rr, cols, scale)
            o[sel, h] = P @ v[cols, kv]
            lse[h, sel] = m + np.log(l)
            if do is not None:
                dP = do[rr, h] @ v[cols, kv].T
                D = (P * dP).sum(axis=1, keepdims=True)
                dq[sel, h] = scale * ((P * (dP - D)) @ k[cols, kv])
    return o, lse, dq


def attn_key_cols(q, k, v, do, position_ids, cols, softmax_scale=None):
    """dK and dV for selected key columns only.  Key j receives gradient from
    the query rows i >= j of its own sample; every such row's full softmax
    (over all its allowed keys) is recomputed.  Returns dk, dv [C][hkv][d]."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    N, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    scale = _scale(d, softmax_scale)
    seg = segment_ids(position_ids)
    first = segment_first(position_ids)
    cols = np.asarray(cols, dtype=np.int64)
    dk = np.zeros((cols.size, hkv, d))
    dv = np.zeros((cols.size, hkv, d))
    for s in np.unique(seg[cols]):
        sel = np.flatnonzero(seg[cols] == s)
        cc = cols[sel]
        last = int(np.flatnonzero(seg == s)[-1])
        rows = np.arange(int(cc.min()), last + 1)       # rows that can see any of cc
        span = np.arange(int(first[rows[0]]), last + 1)  # all keys those rows see
        for h in range(hq):
            kv = h // grp
            for r0 in range(0, rows.size, 128):
                rr = rows[r0:r0 + 128]
                P, _, _ = _probs(q[:, h], k[:, kv], seg, rr, span, scale)
                dP = do[rr, h] @ v[span, kv].T
                D = (P * dP).sum(axis=1, keepdims=True)
                dS = P * (dP - D)
                pos_c = cc - span[0]
                dv[sel, kv] += P[:, pos_c].T @ do[rr, h]
                dk[sel, kv] += scale * (dS[:, pos_c].T @ q[rr, h])
    return dk, dv


def attn_row_stats(q, k, v, do, position_ids, r0, r1, softmax_scale=None, block_rows=256):
    """Per-row statistics of the query rows [r0, r1): the natural-log LSE of
    each row's softmax, its output O and D_i = sum_e dO_ie O_ie (which equals
    sum_j P_ij dP_ij, the row term of dS = P * (dP - D)).  Each row gets its
    full softmax over all of its allowed keys, in blocks of consecutive rows
    with the explicit mask over the block's key span.

    Returns lse [hq][R], o [R][hq][d] and D [hq][R] (float64, R = r1 - r0)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    N, hq, d = q.shape
    grp = hq // k.shape[1]
    scale = _scale(d, softmax_scale)
    seg = segment_ids(position_ids)
    first = segment_first(position_ids)
    R = r1 - r0
    lse = np.zeros((hq, R))
    o = np.zeros((R, hq, d))
    D = np.zeros((hq, R))
    for b0 in range(r0, r1, block_rows):
        b1 = min(r1, b0 + block_rows)
        rows = np.arange(b0, b1)
        cols = np.arange(int(first[b0]), b1)
        for h in range(hq):
            kv = h // grp
            P, m, l = _probs(q[:, h], k[:, kv], seg, rows, cols, scale)
            ob = P @ v[cols, kv]
            o[b0 - r0:b1 - r0, h] = ob
            lse[h, b0 - r0:b1 - r0] = m + np.log(l)
            D[h, b0 - r0:b1 - r0] = (do[rows, h] * ob).sum(axis=1)
    return lse, o, D


def attn_key_cols_from_stats(q, k, v, do, position_ids, cols, lse, D, softmax_scale=None,
                             block_rows=1024):
    """dK and dV of selected key columns from given row statistics.

    Key j of KV head kh receives gradient from the query rows i >= j of its own
    sample and every query head h sharing kh:
        P_ij = exp(scale q_ih . k_j - LSE_hi),  dP_ij = dO_ih . v_j,
        dV_j = sum_(h,i) P_ij dO_ih,  dK_j = scale sum_(h,i) P_ij (dP_ij - D_hi) q_ih.
    ``lse`` and ``D`` are [hq][N] arrays (natural-log LSE and D = rowsum(dO * O)
    of every query row); only the rows that see a requested column are read.
    The rows are walked in blocks with the explicit mask of (rows x cols); each
    column costs O(L d) for the L rows after it.  Returns dk, dv [C][hkv][d]."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    N, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    scale = _scale(d, softmax_scale)
    seg = segment_ids(position_ids)
    cols = np.asarray(cols, dtype=np.int64)
    dk = np.zeros((cols.size, hkv, d))
    dv = np.zeros((cols.size, hkv, d))
    for s in np.unique(seg[cols]):
        sel = np.flatnonzero(seg[cols] == s)
        cc = cols[sel]
        last = int(np.flatnonzero(seg == s)[-1])
        for b0 in range(int(cc.min()), last + 1, block_rows):
            rows = np.arange(b0, min(last + 1, b0 + block_rows))
            mask = allowed(seg, rows, cc)
            for h in range(hq):
                kv = h // grp
                S = scale * (q[rows, h] @ k[cc, kv].T)
                S[~mask] = -np.inf
                P = np.exp(S - lse[h, rows][:, None])
                dP = do[rows, h] @ v[cc, kv].T
                dS = P * (dP - D[h, rows][:, None])
                dv[sel, kv] += P.T @ do[rows, h]
                dk[sel, kv] += scale * (dS.T @ q[rows, h])
    return dk, dv


# ---------------------------------------------------------------------------
# Token-weighted loss across ranks
# ---------------------------------------------------------------------------

def weighted_loss(token_loss, shift_labels, ignore_index=IGNORE_INDEX):
    """Token-weighted mean of per-rank losses, following the pages' loop:
    good_r = #valid tokens of rank r; rank r's loss = mean of its valid token
    losses (NaN if it has none); total = sum over ranks with good_r > 0 of
    loss_r * good_r; loss = total / max(sum_r good_r, 1).

    Returns loss, rank_loss [P], good [P] (int64) and d loss / d token_loss
    [P][N/P] (1/max(T,1) on valid tokens, 0 elsewhere).  float64."""
    tl = np.asarray(token_loss, dtype=np.float64)
    lab = np.asarray(shift_labels)
    P = tl.shape[0]
    valid = lab != ignore_index
    good = valid.sum(axis=1).astype(np.int64)
    rank_loss = np.full(P, np.nan)
    for r in range(P):
        if good[r] > 0:
            rank_loss[r] = tl[r][valid[r]].sum() / good[r]
    total = 0.0
    for r in range(P):
        if good[r] > 0:                      # a rank with no valid tokens is skipped: NaN*0 = NaN
            total = total + rank_loss[r] * good[r]
    T = int(good.sum())
    loss = total / max(T, 1)
    dtl = np.where(valid, 1.0 / max(T, 1), 0.0)
    return float(loss), rank_loss, good, dtl


# ---------------------------------------------------------------------------
# Per-token cross-entropy from hidden states (the loss the model computes
# from shift_labels before the aggregation above; the Accelerate guide,
# "ALST/Ulysses SP backend configuration", and the blog, "Loss aggregation",
# recommend computing it with a fused logit-loss that never holds the full
# logits tensor).  Written here as its plain definition.
# ---------------------------------------------------------------------------

def linear_cross_entropy(x, w, labels, g=None, ignore_index=IGNORE_INDEX):
    """Token losses of logits = x w^T against labels, and their gradients.

    x [N][K] hidden states, w [V][K] LM-head matrix (float64 or bf16 bit
    patterns as uint16), labels [N] int64 (ignore_index: no loss), g [N]
    upstream gradient of the token losses (None: forward only).
        lse_t  = log sum_v exp(logit_tv)
        loss_t = lse_t - logit_{t, labels_t}       (0 where ignored)
        G_tv   = g_t (softmax_v(logit_t) - [v == labels_t])   (0 rows where ignored)
        dx = G w,   dw = G^T x
    Returns token_loss [N], lse [N] and, with g, dx [N][K], dw [V][K] (float64)."""
    x, w = _as_f64(x), _as_f64(w)
    labels = np.asarray(labels)
    logits = x @ w.T
    m = logits.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True)))[:, 0]
    valid = labels != ignore_index
    idx = np.where(valid, labels, 0).astype(np.int64)
    target = logits[np.arange(len(labels)), idx]
    token_loss = np.where(valid, lse - target, 0.0)
    if g is None:
        return token_loss, lse
    G = np.exp(logits - lse[:, None])
    G[np.arange(len(labels)), idx] -= 1.0
    G *= (np.asarray(g, dtype=np.float64) * valid)[:, None]
    return token_loss, lse, G @ w, G.T @ x


def linear_ce_vocab_rows(x, w, labels, g, vrows, ignore_index=IGNORE_INDEX, chunk=256):
    """dw of linear_cross_entropy for selected vocabulary rows only:
        dw_v = sum_t G_tv x_t,  G_tv = g_t (softmax_v(logit_t) - [v == labels_t])
    over the valid tokens.  Every token's log-sum-exp comes from its full row of
    logits (one pass over the vocabulary, tokens taken `chunk` at a time); only the
    requested columns of G are formed.  Returns lse [N] and dw [R][K] (float64)."""
    x, w = _as_f64(x), _as_f64(w)
    labels = np.asarray(labels)
    g = np.asarray(g, dtype=np.float64)
    vrows = np.asarray(vrows, dtype=np.int64)
    N = x.shape[0]
    lse = np.zeros(N)
    dw = np.zeros((vrows.size, x.shape[1]))
    for t0 in range(0, N, chunk):
        t1 = min(N, t0 + chunk)
        logits = x[t0:t1] @ w.T
        m = logits.max(axis=1, keepdims=True)
        lse_c = (m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True)))[:, 0]
        lse[t0:t1] = lse_c
        lab = labels[t0:t1]
        valid = lab != ignore_index
        G = np.exp(logits[:, vrows] - lse_c[:, None])
        G -= (lab[:, None] == vrows[None, :])
        G *= (g[t0:t1] * valid)[:, None]
        dw += G.T @ x[t0:t1]
    return lse, dw
