"""torch-tensor wrappers of the C entry points (same names as the C ABI).

Each wrapper checks dtype, shape, device and contiguity, allocates outputs
with torch (device memory and streams are the only torch services used),
passes raw pointers and the current HIP stream, and raises SPError on a
non-zero status.  All work runs in the library's HIP kernels.
"""
from __future__ import annotations

import torch

from . import _lib

_BF16 = torch.bfloat16


def _stream():
    return ctypes_ptr(torch.cuda.current_stream().cuda_stream)


def ctypes_ptr(x) -> int | None:
    return int(x) if x else None


def _ptr(t: torch.Tensor | None):
    return None if t is None else (t.data_ptr() or None)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


# ---------------------------------------------------------------------------
# Relayout
# ---------------------------------------------------------------------------

def ulysses_seq_to_head(x_seq: torch.Tensor, rank: int = -1, out: torch.Tensor | None = None):
    """[P][N/P][G][H][d] -> [P][G][N][H/P][d] (rank -1) or [G][N][H/P][d] (rank r)."""
    if x_seq.dim() != 5:
        raise ValueError("x_seq must be [P][N/P][G][H][d]")
    P, T, G, H, d = x_seq.shape
    _need(x_seq, "x_seq", _BF16)
    shape = (P, G, P * T, H // P, d) if rank < 0 else (G, P * T, H // P, d)
    if out is None:
        out = torch.empty(shape, dtype=_BF16, device=x_seq.device)
    _need(out, "out", _BF16, shape)
    _lib.check("ulysses_seq_to_head", _lib.call(
        "ulysses_seq_to_head", _ptr(x_seq), _ptr(out), P, P * T, G, H, d, rank, _stream()))
    return out


def ulysses_head_to_seq(x_head: torch.Tensor, sp_size: int, rank: int = -1,
                        out: torch.Tensor | None = None):
    """Inverse of ulysses_seq_to_head.  With rank r only that rank's head
    columns of `out` are written (pass `out` to keep the other columns)."""
    P = sp_size
    if rank < 0:
        if x_head.dim() != 5:
            raise ValueError("x_head must be [P][G][N][H/P][d]")
        _, G, N, hl, d = x_head.shape
    else:
        if x_head.dim() != 4:
            raise ValueError("x_head must be [G][N][H/P][d]")
        G, N, hl, d = x_head.shape
    _need(x_head, "x_head", _BF16)
    shape = (P, N // P, G, hl * P, d)
    if out is None:
        out = (torch.empty if rank < 0 else torch.zeros)(shape, dtype=_BF16, device=x_head.device)
    _need(out, "out", _BF16, shape)
    _lib.check("ulysses_head_to_seq", _lib.call(
        "ulysses_head_to_seq", _ptr(x_head), _ptr(out), P, N, G, hl * P, d, rank, _stream()))
    return out


def ulysses_seq_to_head_kv(x_seq: torch.Tensor, rank: int = -1, out: torch.Tensor | None = None):
    """K/V exchange, also for fewer KV heads than ranks: [P][N/P][G][n_kv][d] ->
    [P][G][N][hl][d] (rank -1) or [G][N][hl][d] (rank r), hl = max(n_kv/P, 1)."""
    if x_seq.dim() != 5:
        raise ValueError("x_seq must be [P][N/P][G][n_kv][d]")
    P, T, G, H, d = x_seq.shape
    _need(x_seq, "x_seq", _BF16)
    hl = max(H // P, 1)
    shape = (P, G, P * T, hl, d) if rank < 0 else (G, P * T, hl, d)
    if out is None:
        out = torch.empty(shape, dtype=_BF16, device=x_seq.device)
    _need(out, "out", _BF16, shape)
    _lib.check("ulysses_seq_to_head_kv", _lib.call(
        "ulysses_seq_to_head_kv", _ptr(x_seq), _ptr(out), P, P * T, G, H, d, rank, _stream()))
    return out


def ulysses_head_to_seq_kv_grad(x_head: torch.Tensor, n_kv_heads: int, rank: int = -1,
                                out: torch.Tensor | None = None):
    """Adjoint of ulysses_seq_to_head_kv (copies of a KV head summed in fp32):
    [P][G][N][hl][d] -> [P][N/P][G][n_kv][d] (rank -1) or rank r's [N/P][G][n_kv][d].
    bf16 or fp32."""
    if x_head.dim() != 5:
        raise ValueError("x_head must be [P][G][N][hl][d]")
    P, G, N, hl, d = x_head.shape
    dt = x_head.dtype
    if dt == torch.float32:
        code = _lib.SP_DTYPE_F32
    elif dt == _BF16:
        code = _lib.SP_DTYPE_BF16
    else:
        raise TypeError("x_head must be bfloat16 or float32")
    _need(x_head, "x_head", dt)
    shape = (P, N // P, G, n_kv_heads, d) if rank < 0 else (N // P, G, n_kv_heads, d)
    if out is None:
        out = torch.empty(shape, dtype=dt, device=x_head.device)
    _need(out, "out", dt, shape)
    _lib.check("ulysses_head_to_seq_kv_grad", _lib.call(
        "ulysses_head_to_seq_kv_grad", _ptr(x_head), _ptr(out), P, N, G, n_kv_heads, d, code, rank,
        _stream()))
    return out


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def sp_attn_workspace_bytes(n_tokens: int, n_q_heads: int, n_kv_heads: int, head_dim: int) -> int:
    return int(_lib.call("sp_attn_workspace_bytes", n_tokens, n_q_heads, n_kv_heads, head_dim))


def workspace(n_tokens: int, n_q_heads: int, n_kv_heads: int, head_dim: int, device="cuda"):
    nbytes = sp_attn_workspace_bytes(n_tokens, n_q_heads, n_kv_heads, head_dim)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def sp_attn_fwd(q, k, v, position_ids, softmax_scale: float = 0.0, o=None, lse=None, ws=None):
    """q [N][hq][d], k/v [N][hkv][d] bf16; position_ids [N] int64.
    Returns (o [N][hq][d] bf16, lse [hq][N] fp32)."""
    N, hq, d = q.shape
    hkv = k.shape[1]
    _need(q, "q", _BF16)
    _need(k, "k", _BF16, (N, hkv, d))
    _need(v, "v", _BF16, (N, hkv, d))
    _need(position_ids, "position_ids", torch.int64, (N,))
    if o is None:
        o = torch.empty((N, hq, d), dtype=_BF16, device=q.device)
    if lse is None:
        lse = torch.empty((hq, N), dtype=torch.float32, device=q.device)
    _need(o, "o", _BF16, (N, hq, d))
    _need(lse, "lse", torch.float32, (hq, N))
    if ws is None:
        ws = workspace(N, hq, hkv, d, q.device)
    _lib.check("sp_attn_fwd", _lib.call(
        "sp_attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(position_ids), N, hq, hkv, d,
        float(softmax_scale), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return o, lse


def sp_attn_bwd(q, k, v, o, d_o, lse, position_ids, softmax_scale: float = 0.0,
                grad_dtype=torch.float32, dq=None, dk=None, dv=None, ws=None):
    """Gradients (dq [N][hq][d], dk/dv [N][hkv][d]) in grad_dtype (fp32 or bf16)."""
    N, hq, d = q.shape
    hkv = k.shape[1]
    for t, name, shp in ((q, "q", None), (k, "k", (N, hkv, d)), (v, "v", (N, hkv, d)),
                         (o, "o", (N, hq, d)), (d_o, "d_o", (N, hq, d))):
        _need(t, name, _BF16, shp)
    _need(lse, "lse", torch.float32, (hq, N))
    _need(position_ids, "position_ids", torch.int64, (N,))
    if grad_dtype == torch.float32:
        code = _lib.SP_DTYPE_F32
    elif grad_dtype == torch.bfloat16:
        code = _lib.SP_DTYPE_BF16
    else:
        raise TypeError("grad_dtype must be torch.float32 or torch.bfloat16")
    if dq is None:
        dq = torch.empty((N, hq, d), dtype=grad_dtype, device=q.device)
    if dk is None:
        dk = torch.empty((N, hkv, d), dtype=grad_dtype, device=q.device)
    if dv is None:
        dv = torch.empty((N, hkv, d), dtype=grad_dtype, device=q.device)
    _need(dq, "dq", grad_dtype, (N, hq, d))
    _need(dk, "dk", grad_dtype, (N, hkv, d))
    _need(dv, "dv", grad_dtype, (N, hkv, d))
    if ws is None:
        ws = workspace(N, hq, hkv, d, q.device)
    _lib.check("sp_attn_bwd", _lib.call(
        "sp_attn_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
        _ptr(position_ids), N, hq, hkv, d, float(softmax_scale), code, _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(ws), ws.numel(), _stream()))
    return dq, dk, dv


def sp_attn_bwd_noalloc(q, k, v, o, d_o, lse, position_ids, softmax_scale: float = 0.0,
                        grad_dtype=torch.float32, dq=None, dk=None, dv=None):
    """sp_attn_bwd with the library's fixed device scratch instead of a workspace
    (the C call allocates nothing; pass dq, dk, dv to keep this wrapper from
    allocating its outputs)."""
    N, hq, d = q.shape
    hkv = k.shape[1]
    for t, name, shp in ((q, "q", None), (k, "k", (N, hkv, d)), (v, "v", (N, hkv, d)),
                         (o, "o", (N, hq, d)), (d_o, "d_o", (N, hq, d))):
        _need(t, name, _BF16, shp)
    _need(lse, "lse", torch.float32, (hq, N))
    _need(position_ids, "position_ids", torch.int64, (N,))
    if grad_dtype == torch.float32:
        code = _lib.SP_DTYPE_F32
    elif grad_dtype == torch.bfloat16:
        code = _lib.SP_DTYPE_BF16
    else:
        raise TypeError("grad_dtype must be torch.float32 or torch.bfloat16")
    if dq is None:
        dq = torch.empty((N, hq, d), dtype=grad_dtype, device=q.device)
    if dk is None:
        dk = torch.empty((N, hkv, d), dtype=grad_dtype, device=q.device)
    if dv is None:
        dv = torch.empty((N, hkv, d), dtype=grad_dtype, device=q.device)
    _need(dq, "dq", grad_dtype, (N, hq, d))
    _need(dk, "dk", grad_dtype, (N, hkv, d))
    _need(dv, "dv", grad_dtype, (N, hkv, d))
    _lib.check("sp_attn_bwd_noalloc", _lib.call(
        "sp_attn_bwd_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
        _ptr(position_ids), N, hq, hkv, d, float(softmax_scale), code, _ptr(dq), _ptr(dk),
        _ptr(dv), _stream()))
    return dq, dk, dv


def _need_rows(t: torch.Tensor, name: str, dtype, shape) -> int:
    """A [N][h][d] view whose heads and elements are packed (strides (s, d, 1));
    returns the token stride s."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
        raise ValueError(f"{name}: heads and elements of a token must be packed")
    return t.stride(0)


def sp_attn_fwd_strided(q, k, v, position_ids, softmax_scale: float = 0.0, o=None, lse=None,
                        ws=None):
    """sp_attn_fwd on [N][h][d] views with any token stride (e.g. one rank's
    heads of a [N][G][H][d] exchange buffer); k and v share one stride.
    `o` may be such a view too.  Returns (o, lse)."""
    N, hq, d = q.shape
    hkv = k.shape[1]
    sq = _need_rows(q, "q", _BF16, (N, hq, d))
    sk = _need_rows(k, "k", _BF16, (N, hkv, d))
    if _need_rows(v, "v", _BF16, (N, hkv, d)) != sk:
        raise ValueError("k and v must share one token stride")
    _need(position_ids, "position_ids", torch.int64, (N,))
    if o is None:
        o = torch.empty((N, hq, d), dtype=_BF16, device=q.device)
    so = _need_rows(o, "o", _BF16, (N, hq, d))
    if lse is None:
        lse = torch.empty((hq, N), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (hq, N))
    if ws is None:
        ws = workspace(N, hq, hkv, d, q.device)
    _lib.check("sp_attn_fwd_strided", _lib.call(
        "sp_attn_fwd_strided", _ptr(q), sq, _ptr(k), _ptr(v), sk, _ptr(position_ids), N, hq, hkv,
        d, float(softmax_scale), _ptr(o), so, _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return o, lse


def sp_attn_bwd_strided(q, k, v, o, d_o, lse, position_ids, softmax_scale: float = 0.0,
                        grad_dtype=torch.float32, dq=None, dk=None, dv=None, ws=None):
    """sp_attn_bwd on [N][h][d] views with any token stride (see
    sp_attn_fwd_strided); dq, dk, dv may be such views too."""
    N, hq, d = q.shape
    hkv = k.shape[1]
    sq = _need_rows(q, "q", _BF16, (N, hq, d))
    sk = _need_rows(k, "k", _BF16, (N, hkv, d))
    if _need_rows(v, "v", _BF16, (N, hkv, d)) != sk:
        raise ValueError("k and v must share one token stride")
    so = _need_rows(o, "o", _BF16, (N, hq, d))
    sdo = _need_rows(d_o, "d_o", _BF16, (N, hq, d))
    _need(lse, "lse", torch.float32, (hq, N))
    _need(position_ids, "position_ids", torch.int64, (N,))
    if grad_dtype == torch.float32:
        code = _lib.SP_DTYPE_F32
    elif grad_dtype == torch.bfloat16:
        code = _lib.SP_DTYPE_BF16
    else:
        raise TypeError("grad_dtype must be torch.float32 or torch.bfloat16")
    if dq is None:
        dq = torch.empty((N, hq, d), dtype=grad_dtype, device=q.device)
    if dk is None:
        dk = torch.empty((N, hkv, d), dtype=grad_dtype, device=q.device)
    if dv is None:
        dv = torch.empty((N, hkv, d), dtype=grad_dtype, device=q.device)
    sdq = _need_rows(dq, "dq", grad_dtype, (N, hq, d))
    sdk = _need_rows(dk, "dk", grad_dtype, (N, hkv, d))
    sdv = _need_rows(dv, "dv", grad_dtype, (N, hkv, d))
    if ws is None:
        ws = workspace(N, hq, hkv, d, q.device)
    _lib.check("sp_attn_bwd_strided", _lib.call(
        "sp_attn_bwd_strided", _ptr(q), sq, _ptr(k), _ptr(v), sk, _ptr(o), so, _ptr(d_o), sdo,
        _ptr(lse), _ptr(position_ids), N, hq, hkv, d, float(softmax_scale), code, _ptr(dq), sdq,
        _ptr(dk), sdk, _ptr(dv), sdv, _ptr(ws), ws.numel(), _stream()))
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Loss
# ---------------------------------------------------------------------------

def sp_linear_ce(x, w, labels, d_token_loss=None, ignore_index: int = -100,
                 grad_dtype=torch.float32, chunk_tokens: int = 4096, out=None, ws=None):
    """Per-token cross-entropy of x w^T (x [N][K] bf16, w [V][K] bf16, labels [N]
    int64) without holding more than one chunk of logits.  Returns (token_loss,
    lse) and, with d_token_loss [N] fp32, also (dx, dw fp32)."""
    N, K = x.shape
    V = w.shape[0]
    _need(x, "x", _BF16)
    _need(w, "w", _BF16, (V, K))
    _need(labels, "labels", torch.int64, (N,))
    if d_token_loss is not None:
        _need(d_token_loss, "d_token_loss", torch.float32, (N,))
    if grad_dtype == torch.float32:
        code = _lib.SP_DTYPE_F32
    elif grad_dtype == torch.bfloat16:
        code = _lib.SP_DTYPE_BF16
    else:
        raise TypeError("grad_dtype must be torch.float32 or torch.bfloat16")
    dev = x.device
    if out is None:
        out = (torch.empty(N, dtype=torch.float32, device=dev),
               torch.empty(N, dtype=torch.float32, device=dev),
               torch.empty((N, K), dtype=grad_dtype, device=dev) if d_token_loss is not None else None,
               torch.empty((V, K), dtype=torch.float32, device=dev) if d_token_loss is not None else None)
    tl, lse, dx, dw = out
    _need(tl, "token_loss", torch.float32, (N,))
    _need(lse, "lse", torch.float32, (N,))
    if d_token_loss is not None:
        _need(dx, "dx", grad_dtype, (N, K))
        _need(dw, "dw", torch.float32, (V, K))
    if ws is None:
        nb = int(_lib.call("sp_linear_ce_workspace_bytes", V, chunk_tokens))
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _lib.check("sp_linear_ce", _lib.call(
        "sp_linear_ce", _ptr(x), _ptr(w), _ptr(labels), ignore_index, _ptr(d_token_loss), N, V, K,
        code, _ptr(tl), _ptr(lse), _ptr(dx), _ptr(dw), chunk_tokens, _ptr(ws), ws.numel(),
        _stream()))
    return (tl, lse) if d_token_loss is None else (tl, lse, dx, dw)


def sp_weighted_loss(token_loss, shift_labels, ignore_index: int = -100, with_grad: bool = True,
                     out=None):
    """token_loss fp32 [P][N/P], shift_labels int64 [P][N/P] ->
    (loss [1] fp32, rank_loss [P] fp32, good_tokens [P] int64, d_token_loss or None)."""
    if token_loss.dim() != 2:
        raise ValueError("token_loss must be [P][N/P]")
    P, T = token_loss.shape
    _need(token_loss, "token_loss", torch.float32)
    _need(shift_labels, "shift_labels", torch.int64, (P, T))
    dev = token_loss.device
    if out is None:
        out = (torch.empty(1, dtype=torch.float32, device=dev),
               torch.empty(P, dtype=torch.float32, device=dev),
               torch.empty(P, dtype=torch.int64, device=dev),
               torch.empty((P, T), dtype=torch.float32, device=dev) if with_grad else None)
    loss, rank_loss, good, dtl = out
    _lib.check("sp_weighted_loss", _lib.call(
        "sp_weighted_loss", _ptr(token_loss), _ptr(shift_labels), P, P * T, int(ignore_index),
        _ptr(loss), _ptr(rank_loss), _ptr(good), _ptr(dtl), _stream()))
    return loss, rank_loss, good, dtl


# ---------------------------------------------------------------------------
# Per-kernel timing (profiling aid)
# ---------------------------------------------------------------------------

def sp_timing_enable(on: bool = True) -> bool:
    return bool(_lib.call("sp_timing_enable", 1 if on else 0))


def sp_timing_collect() -> dict:
    """{kernel name: {"launches", "total_ms", "avg_ms", "min_ms", "max_ms"}} of the
    launches recorded since timing was enabled (or last collected)."""
    import ctypes
    n = _lib.call("sp_timing_collect", None, 0)
    if n < 0:
        raise RuntimeError("sp_timing_collect: events could not be read")
    buf = (_lib.KernelTime * max(n, 1))()
    n = _lib.call("sp_timing_collect", ctypes.cast(buf, ctypes.c_void_p), n)
    out = {}
    for i in range(max(n, 0)):
        r = buf[i]
        out[r.name.decode()] = {"launches": r.launches, "total_ms": r.total_ms,
                                "avg_ms": r.total_ms / max(r.launches, 1),
                                "min_ms": r.min_ms, "max_ms": r.max_ms}
    return out
