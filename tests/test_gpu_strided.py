"""Strided attention (sp_attn_fwd_strided / sp_attn_bwd_strided) on the GPU.

The strided calls run the same arithmetic as the packed ones, so on the same
values they must return identical bits, and must not touch the rest of the
buffers they write into.  The zero-copy layer reads every rank's heads
straight out of the token-major exchange buffer (rank r's heads of
[N][G][H][d] are a strided view) and writes O and the gradients back into
it; it must match the relayout path bit for bit and the oracle within the
gates."""
import zlib

import numpy as np
import pytest

from oracle import ref
from synth import configs, gen

from helpers import f64_of, gate, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

SENTINEL = -7.25   # exactly representable in bf16 and fp32


def _ops():
    from ulysses_sequence_parallelism_share_amd import ops
    return ops


CASES = [  # name, N, hq, hkv, d, sample lengths, padding heads around the view
    ("gqa4-d128", 781, 4, 1, 128, [100, 1, 300, 380], 3),
    ("gqa2-d64-two-kv", 600, 4, 2, 64, [300, 300], 1),
    ("gqa3-gathered-rows", 211, 3, 1, 128, [100, 111], 2),
    ("gqa3-two-kv-gathered", 190, 6, 2, 64, [190], 2),
    ("mha-d128", 257, 2, 2, 128, [1, 256], 5),
    ("gqa8", 300, 8, 1, 128, [150, 150], 1),
]


def _padded(torch, x, pad, lead=1):
    """x [N][h][d] placed at heads [lead, lead+h) of a sentinel-filled [N][h+pad][d]
    buffer; returns (buffer, view)."""
    N, h, d = x.shape
    buf = torch.full((N, h + pad, d), SENTINEL, dtype=x.dtype, device=x.device)
    view = buf[:, lead:lead + h]
    view.copy_(x)
    return buf, view


def _untouched(torch, buf, lead, h):
    mask = torch.ones(buf.shape[1], dtype=torch.bool, device=buf.device)
    mask[lead:lead + h] = False
    rest = buf[:, mask]
    return bool((rest == SENTINEL).all())


@pytest.mark.parametrize("name,N,hq,hkv,d,lens,pad", CASES, ids=[c[0] for c in CASES])
def test_strided_matches_packed(name, N, hq, hkv, d, lens, pad):
    import torch
    ops = _ops()
    assert sum(lens) == N
    say(f"strided {name}: N={N} hq={hq} hkv={hkv} d={d} pad={pad}")
    seed = zlib.crc32(name.encode()) % 1000
    q, k, v, do = (to_dev_bf16(gen.normal_bf16((seed, i), shp)) for i, shp in
                   ((1, (N, hq, d)), (2, (N, hkv, d)), (3, (N, hkv, d)), (4, (N, hq, d))))
    pos = to_dev(gen.position_ids_from_lengths(lens))
    o, lse = ops.sp_attn_fwd(q, k, v, pos)
    g32 = ops.sp_attn_bwd(q, k, v, o, do, lse, pos)
    g16 = ops.sp_attn_bwd(q, k, v, o, do, lse, pos, grad_dtype=torch.bfloat16)

    lead = 1
    _, qs = _padded(torch, q, pad, lead)
    _, dos = _padded(torch, do, pad, lead)
    kvbuf = torch.full((N, 2, hkv + pad, d), SENTINEL, dtype=torch.bfloat16, device="cuda")
    ks, vs = kvbuf[:, 0, lead:lead + hkv], kvbuf[:, 1, lead:lead + hkv]
    ks.copy_(k)
    vs.copy_(v)
    obuf = torch.full((N, hq + pad, d), SENTINEL, dtype=torch.bfloat16, device="cuda")
    os_ = obuf[:, lead:lead + hq]
    o2, lse2 = ops.sp_attn_fwd_strided(qs, ks, vs, pos, o=os_)
    assert torch.equal(os_.view(torch.int16), o.view(torch.int16)), "O differs from packed"
    assert torch.equal(lse2, lse), "LSE differs from packed"
    assert _untouched(torch, obuf, lead, hq), "O write left its view"
    for dt, ref_g in ((torch.float32, g32), (torch.bfloat16, g16)):
        dqbuf = torch.full((N, hq + pad, d), SENTINEL, dtype=dt, device="cuda")
        dkvbuf = torch.full((N, 2, hkv + pad, d), SENTINEL, dtype=dt, device="cuda")
        dqs = dqbuf[:, lead:lead + hq]
        dks, dvs = dkvbuf[:, 0, lead:lead + hkv], dkvbuf[:, 1, lead:lead + hkv]
        ops.sp_attn_bwd_strided(qs, ks, vs, os_, dos, lse2, pos, grad_dtype=dt, dq=dqs, dk=dks,
                                dv=dvs)
        for nm, got, want in (("dQ", dqs, ref_g[0]), ("dK", dks, ref_g[1]), ("dV", dvs, ref_g[2])):
            assert torch.equal(got, want), f"{nm} ({dt}) differs from packed"
        assert _untouched(torch, dqbuf, lead, hq)
        assert _untouched(torch, dkvbuf[:, 0], lead, hkv) and _untouched(torch, dkvbuf[:, 1], lead, hkv)


def test_zero_copy_full_layer_tiny_sp4():
    """sp_size 4, N=1024, 8 heads, d=64: every rank's attention reads its 2 heads of
    q, k and v straight from the fused QKV exchange buffer [N][3][H][d] and writes O
    and the gradients into [N][1][H][d] / [N][3][H][d] buffers; identical bits to the
    relayout path, and the oracle's unsharded 8-head attention within the gates."""
    import torch
    ops = _ops()
    w = configs.WORKLOADS[1]
    P, N, d, H = w.sp_size, w.n_tokens, w.head_dim, w.Hq
    hl = H // P
    inp = configs.exchange_inputs(w)
    pos = inp["pos"]
    posd = to_dev(pos)
    say(f"zero-copy full layer P={P} N={N} H={H} d={d}")
    qkv_seq = to_dev_bf16(inp["qkv_seq"])                     # [P][N/P][3][H][d]
    do_seq = to_dev_bf16(inp["do_seq"])                       # [P][N/P][1][H][d]
    X = qkv_seq.view(N, 3, H, d)
    dO = do_seq.view(N, 1, H, d)
    # relayout path
    qkv_h = ops.ulysses_seq_to_head(qkv_seq)
    do_h = ops.ulysses_seq_to_head(do_seq)
    o_h = torch.empty((P, 1, N, hl, d), dtype=torch.bfloat16, device="cuda")
    g_h = torch.empty((P, 3, N, hl, d), dtype=torch.bfloat16, device="cuda")
    for r in range(P):
        qr, kr, vr = qkv_h[r, 0], qkv_h[r, 1], qkv_h[r, 2]
        o, lse = ops.sp_attn_fwd(qr, kr, vr, posd, o=o_h[r, 0])
        ops.sp_attn_bwd(qr, kr, vr, o, do_h[r, 0], lse, posd, grad_dtype=torch.bfloat16,
                        dq=g_h[r, 0], dk=g_h[r, 1], dv=g_h[r, 2])
    o_seq = ops.ulysses_head_to_seq(o_h, P)
    g_seq = ops.ulysses_head_to_seq(g_h, P)
    # zero-copy path
    O = torch.empty((N, 1, H, d), dtype=torch.bfloat16, device="cuda")
    G = torch.empty((N, 3, H, d), dtype=torch.bfloat16, device="cuda")
    G32 = torch.empty((N, 3, H, d), dtype=torch.float32, device="cuda")
    for r in range(P):
        sl = slice(r * hl, (r + 1) * hl)
        q, k, v = X[:, 0, sl], X[:, 1, sl], X[:, 2, sl]
        o, lse = ops.sp_attn_fwd_strided(q, k, v, posd, o=O[:, 0, sl])
        ops.sp_attn_bwd_strided(q, k, v, o, dO[:, 0, sl], lse, posd, grad_dtype=torch.bfloat16,
                                dq=G[:, 0, sl], dk=G[:, 1, sl], dv=G[:, 2, sl])
        ops.sp_attn_bwd_strided(q, k, v, o, dO[:, 0, sl], lse, posd, grad_dtype=torch.float32,
                                dq=G32[:, 0, sl], dk=G32[:, 1, sl], dv=G32[:, 2, sl])
    assert torch.equal(O.view(torch.int16).flatten(), o_seq.view(torch.int16).flatten())
    assert torch.equal(G.view(torch.int16).flatten(), g_seq.view(torch.int16).flatten())
    full = inp["qkv_seq"].reshape(N, 3, H, d)
    o_ref, _ = ref.attn_fwd(full[:, 0], full[:, 1], full[:, 2], pos)
    dq_r, dk_r, dv_r = ref.attn_bwd(full[:, 0], full[:, 1], full[:, 2],
                                    inp["do_seq"].reshape(N, H, d), pos)
    gate("O (zero-copy)", f64_of(O[:, 0]), o_ref)
    g = G32.cpu().numpy().astype(np.float64)
    gate("dQ (zero-copy)", g[:, 0], dq_r)
    gate("dK (zero-copy)", g[:, 1], dk_r)
    gate("dV (zero-copy)", g[:, 2], dv_r)


@pytest.mark.slow
def test_zero_copy_500k_share_matches_relayout_path():
    """The 500K-token share in the benchmark's shapes: rank 0's attention read in place
    from the Q [N][1][32][d] and KV [N][2][8][d] exchange buffers gives the same bits as
    attention on the relayouted copies."""
    import torch
    ops = _ops()
    w = configs.WORKLOADS[5]
    N, hq, hkv, d = w.n_tokens, w.hq, w.hkv, w.head_dim
    say(f"zero-copy 500K share: N={N} hq={hq} hkv={hkv}")
    inp = configs.exchange_inputs(w)
    posd = to_dev(inp["pos"])
    q_seq = to_dev_bf16(inp["q_seq"])
    kv_seq = to_dev_bf16(inp["kv_seq"])
    do_seq = to_dev_bf16(inp["do_seq"])
    Hq, Hkv = q_seq.shape[3], kv_seq.shape[3]
    qh = ops.ulysses_seq_to_head(q_seq, rank=0)[0]
    kvh = ops.ulysses_seq_to_head(kv_seq, rank=0)
    doh = ops.ulysses_seq_to_head(do_seq, rank=0)[0]
    ws = ops.workspace(N, hq, hkv, d)
    o, lse = ops.sp_attn_fwd(qh, kvh[0], kvh[1], posd, ws=ws)
    dq, dk, dv = ops.sp_attn_bwd(qh, kvh[0], kvh[1], o, doh, lse, posd,
                                 grad_dtype=torch.bfloat16, ws=ws)
    Q = q_seq.view(N, 1, Hq, d)[:, 0, :hq]
    KV = kv_seq.view(N, 2, Hkv, d)
    DO = do_seq.view(N, 1, Hq, d)[:, 0, :hq]
    O = torch.empty((N, 1, Hq, d), dtype=torch.bfloat16, device="cuda")
    o2, lse2 = ops.sp_attn_fwd_strided(Q, KV[:, 0, :hkv], KV[:, 1, :hkv], posd, o=O[:, 0, :hq],
                                       ws=ws)
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16))
    assert torch.equal(lse2, lse)
    GQ = torch.empty((N, 1, Hq, d), dtype=torch.bfloat16, device="cuda")
    GKV = torch.empty((N, 2, Hkv, d), dtype=torch.bfloat16, device="cuda")
    ops.sp_attn_bwd_strided(Q, KV[:, 0, :hkv], KV[:, 1, :hkv], o2, DO, lse2, posd,
                            grad_dtype=torch.bfloat16, dq=GQ[:, 0, :hq], dk=GKV[:, 0, :hkv],
                            dv=GKV[:, 1, :hkv], ws=ws)
    assert torch.equal(GQ[:, 0, :hq].view(torch.int16), dq.view(torch.int16))
    assert torch.equal(GKV[:, 0, :hkv].view(torch.int16), dk.view(torch.int16))
    assert torch.equal(GKV[:, 1, :hkv].view(torch.int16), dv.view(torch.int16))
