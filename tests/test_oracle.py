"""Pins for the CPU oracle: brute force on tiny inputs, closed forms, invariants,
finite differences and the pages' own statements.  CPU only."""
import math
import os

import numpy as np
import pytest

from oracle import ref
from synth import configs, gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _read_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------------------
# Relayout
# ---------------------------------------------------------------------------

def _tagged(P, T, G, H, d):
    """Each element's value encodes (p, t, g, h, e) so its destination can be read back."""
    p, t, g, h, e = np.meshgrid(np.arange(P), np.arange(T), np.arange(G), np.arange(H),
                                np.arange(d), indexing="ij")
    return (((((p * T + t) * G + g) * H + h) * d) + e).astype(np.int64), (p * T + t), g, h, e


def test_two_gpu_figure_layouts():
    """The figure: GPU i first holds tokens [i N/2, (i+1) N/2) for all heads; after the
    exchange it holds all N tokens for heads [i H/2, (i+1) H/2); the second exchange
    returns the first layout."""
    P, T, G, H, d = 2, 5, 1, 6, 3
    N = P * T
    x, tok, grp, head, e = _tagged(P, T, G, H, d)
    sym = {"0": 0, "N/2": N // 2, "N": N, "H/2": H // 2, "H": H}
    rows = _read_golden("two_gpu_figure.txt")
    h2 = ref.seq_to_head(x)
    back = ref.head_to_seq(h2, P)
    for phase, gpu, trange, hrange in rows:
        gpu = int(gpu)
        t0, t1 = (sym[s] for s in trange.split(":"))
        h0, h1 = (sym[s] for s in hrange.split(":"))
        if phase in ("seq_sharded", "back_to_seq"):
            arr = x if phase == "seq_sharded" else back
            held_tok = tok[gpu] if phase == "seq_sharded" else tok[gpu]
            assert np.array_equal(arr[gpu], x[gpu])
            assert held_tok.min() == t0 and held_tok.max() == t1 - 1
        else:
            share = h2[gpu]                        # [G][N][H/P][d]
            n_idx = np.arange(N)[None, :, None, None]
            hl = np.arange(H // P)[None, None, :, None]
            ee = np.arange(d)[None, None, None, :]
            gg = np.arange(G)[:, None, None, None]
            # decode each element back into (token, head) and check the ranges
            dec_e = share % d
            dec_h = (share // d) % H
            dec_g = (share // (d * H)) % G
            dec_tok = share // (d * H * G)
            assert np.array_equal(dec_e, np.broadcast_to(ee, share.shape))
            assert np.array_equal(dec_g, np.broadcast_to(gg, share.shape))
            assert np.array_equal(dec_tok, np.broadcast_to(n_idx, share.shape))
            assert np.array_equal(dec_h, np.broadcast_to(h0 + hl, share.shape))
            assert dec_tok.min() == t0 and dec_tok.max() == t1 - 1
            assert dec_h.min() == h0 and dec_h.max() == h1 - 1


@pytest.mark.parametrize("P,T,G,H,d", [(1, 4, 3, 2, 2), (2, 3, 1, 4, 2), (3, 2, 2, 6, 4),
                                       (4, 3, 3, 8, 2), (8, 2, 2, 16, 1)])
def test_relayout_places_every_element(P, T, G, H, d):
    """After seq->head, rank q holds global token p*T+t, group g, head q*H/P+hl at
    [q][g][p*T+t][hl]; every source element appears exactly once."""
    x, tok, grp, head, e = _tagged(P, T, G, H, d)
    out = ref.seq_to_head(x)
    hl = H // P
    assert out.shape == (P, G, P * T, hl, d)
    for q in range(P):
        for g in range(G):
            for n in range(P * T):
                for j in range(hl):
                    expect = (((n * G + g) * H + q * hl + j) * d) + np.arange(d)
                    assert np.array_equal(out[q, g, n, j], expect)
    assert np.array_equal(np.sort(out.ravel()), np.sort(x.ravel()))


def test_relayout_p1_is_textbook_transpose():
    x = gen.raw_bits_u16((99, 1), (1, 7, 3, 5, 4))
    out = ref.seq_to_head(x)
    assert np.array_equal(out[0], np.transpose(x[0], (1, 0, 2, 3)))


@pytest.mark.parametrize("P,T,G,H,d", [(2, 3, 3, 4, 8), (4, 5, 1, 8, 16), (8, 2, 2, 8, 8)])
def test_relayout_roundtrip_and_rank_slices_bitexact(P, T, G, H, d):
    x = gen.raw_bits_u16((99, P), (P, T, G, H, d))   # includes NaN payloads, -0, subnormals
    h = ref.seq_to_head(x)
    assert np.array_equal(ref.head_to_seq(h, P), x)
    y = np.zeros_like(x)
    for r in range(P):
        s = ref.seq_to_head(x, rank=r)
        assert np.array_equal(s, h[r])
        ref.head_to_seq(s, P, rank=r, out=y)
    assert np.array_equal(y, x)
    # a single rank's write touches only its own head columns
    z = np.zeros_like(x)
    ref.head_to_seq(h[1 % P], P, rank=1 % P, out=z)
    hl = H // P
    mask = np.zeros(H, bool)
    mask[(1 % P) * hl:((1 % P) + 1) * hl] = True
    assert np.array_equal(z[..., mask, :], x[..., mask, :])
    assert not z[..., ~mask, :].any()


def test_head_divisibility_golden():
    for H_s, *accepted in _read_golden("head_divisibility.txt"):
        H = int(H_s.rstrip(":"))
        acc = {int(a) for a in accepted}
        for P in range(1, H + 1):
            x = np.zeros((P, 1, 1, H, 1), np.uint16)
            if P in acc:
                ref.seq_to_head(x)
            else:
                with pytest.raises(ValueError):
                    ref.seq_to_head(x)


# ---------------------------------------------------------------------------
# K/V relayout with fewer KV heads than ranks (replicate forward, sum backward)
# ---------------------------------------------------------------------------

KV_SHAPES = [  # P, T, G, n_kv, d
    (4, 3, 2, 2, 8),     # 2 ranks per KV head
    (8, 2, 1, 1, 4),     # every rank holds the single KV head
    (4, 3, 2, 8, 4),     # more KV heads than ranks: the plain exchange
    (6, 2, 2, 3, 8),     # 2 ranks per KV head, odd counts
]


@pytest.mark.parametrize("P,T,G,H,d", KV_SHAPES)
def test_kv_relayout_brute_force(P, T, G, H, d):
    """Loops over every output element; rank q's first KV head is q*H//P, which is
    the KV head of its query heads under the consecutive GQA grouping."""
    x = _rand(11, (P, T, G, H, d))
    y = ref.seq_to_head_kv(x)
    hl = max(H // P, 1)
    Hq = 2 * max(H, P)                       # any query-head count divisible by both
    for q in range(P):
        q_heads = range(q * Hq // P, (q + 1) * Hq // P)
        kv_of_q = {h // (Hq // H) for h in q_heads}
        assert min(kv_of_q) == q * H // P and len(kv_of_q) == hl
        for g in range(G):
            for n in range(P * T):
                for i in range(hl):
                    assert np.array_equal(y[q, g, n, i], x[n // T, n % T, g, q * H // P + i])
    z = ref.head_to_seq_kv_sum(y.astype(np.float64), H)
    for p in range(P):
        for t in range(T):
            for g in range(G):
                for j in range(H):
                    want = sum(y[q, g, p * T + t, j - q * H // P] for q in range(P)
                               if q * H // P <= j < q * H // P + hl)
                    assert np.allclose(z[p, t, g, j], want, rtol=0, atol=1e-15)
    assert np.array_equal(ref.seq_to_head_kv(x, rank=1), y[1])
    assert np.array_equal(ref.head_to_seq_kv_sum(y, H, rank=P - 1), ref.head_to_seq_kv_sum(y, H)[P - 1])


def test_kv_relayout_is_plain_exchange_when_heads_cover_ranks():
    x = gen.normal_bf16((3, 1), (4, 5, 2, 8, 16))
    y = ref.seq_to_head_kv(x)
    assert np.array_equal(y, ref.seq_to_head(x))
    assert np.array_equal(ref.head_to_seq_kv_sum(y, 8, bf16_bits=True), x)   # one copy each


def test_kv_replication_equals_repeated_heads():
    """Sending KV head j to P/n_kv ranks is the plain exchange of the tensor whose
    heads are repeated P/n_kv times."""
    P, H = 8, 2
    x = gen.normal_bf16((3, 2), (P, 4, 2, H, 16))
    assert np.array_equal(ref.seq_to_head_kv(x), ref.seq_to_head(np.repeat(x, P // H, axis=3)))


def test_kv_gradient_sum_is_the_adjoint():
    """<s2h(x), y> == <x, h2s_sum(y)>: the summed gradient exchange is the adjoint of
    the replicating exchange (exact here: small integers in float64)."""
    rng = np.random.default_rng(5)
    for P, T, G, H, d in KV_SHAPES:
        x = rng.integers(-8, 9, (P, T, G, H, d)).astype(np.float64)
        y = rng.integers(-8, 9, (P, G, P * T, max(H // P, 1), d)).astype(np.float64)
        assert np.sum(ref.seq_to_head_kv(x) * y) == np.sum(x * ref.head_to_seq_kv_sum(y, H))


def test_kv_gradient_sum_bf16_rounding():
    """bf16 copies are summed in float32 in ascending rank order and rounded once,
    to nearest even: 1 + 2^-8 is a tie and rounds to 1; 1 + 2^-8 + 2^-8 = 1 + 2^-7
    is exact; -(1 + 3*2^-9) rounds to -(1 + 2^-7)."""
    def bits(v):
        return (np.array(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for vals, want in (([1.0, 2.0 ** -8], 1.0), ([1.0, 2.0 ** -8, 2.0 ** -8], 1.0 + 2.0 ** -7),
                       ([-1.0, -3 * 2.0 ** -9], -(1.0 + 2.0 ** -7))):
        P = len(vals)
        y = np.stack([np.full((1, P, 1, 8), bits(v), np.uint16) for v in vals])   # [P][G][N][1][d]
        z = ref.head_to_seq_kv_sum(y, 1, bf16_bits=True)
        assert np.all(z == bits(want)), (vals, want)


def test_gqa_layer_with_kv_replication_matches_unsharded():
    """8 query heads, 2 KV heads, sp_size 4: each rank gets 2 query heads through the
    plain exchange and its one KV head through the replicating exchange; its attention
    equals the unsharded GQA attention on its heads, and the summed dK/dV equal the
    unsharded ones."""
    P, N, Hq, H, d = 4, 48, 8, 2, 8
    T = N // P
    pos = gen.position_ids_from_lengths([20, 1, 27])
    q_seq = _rand(21, (P, T, 1, Hq, d))
    kv_seq = _rand(22, (P, T, 2, H, d))
    do_seq = _rand(23, (P, T, 1, Hq, d))
    qh = ref.seq_to_head(q_seq)
    kvh = ref.seq_to_head_kv(kv_seq)                      # [P][2][N][1][d]
    doh = ref.seq_to_head(do_seq)
    q_full, do_full = q_seq.reshape(N, Hq, d), do_seq.reshape(N, Hq, d)
    k_full, v_full = kv_seq.reshape(N, 2, H, d)[:, 0], kv_seq.reshape(N, 2, H, d)[:, 1]
    o_ref, _ = ref.attn_fwd(q_full, k_full, v_full, pos)
    dq_ref, dk_ref, dv_ref = ref.attn_bwd(q_full, k_full, v_full, do_full, pos)
    dkv_h = np.empty((P, 2, N, 1, d))
    hl = Hq // P
    for r in range(P):
        o, _ = ref.attn_fwd(qh[r, 0], kvh[r, 0], kvh[r, 1], pos)
        assert np.allclose(o, o_ref[:, r * hl:(r + 1) * hl], rtol=0, atol=1e-12)
        dq, dk, dv = ref.attn_bwd(qh[r, 0], kvh[r, 0], kvh[r, 1], doh[r, 0], pos)
        assert np.allclose(dq, dq_ref[:, r * hl:(r + 1) * hl], rtol=0, atol=1e-12)
        dkv_h[r, 0], dkv_h[r, 1] = dk, dv
    dkv_seq = ref.head_to_seq_kv_sum(dkv_h, H).reshape(N, 2, H, d)
    assert np.allclose(dkv_seq[:, 0], dk_ref, rtol=0, atol=1e-12)
    assert np.allclose(dkv_seq[:, 1], dv_ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Mask
# ---------------------------------------------------------------------------

def _brute_allowed(pos):
    """Query i sees key j iff j <= i and no sample starts in (j, i]."""
    n = len(pos)
    out = np.zeros((n, n), bool)
    for i in range(n):
        for j in range(i + 1):
            ok = True
            for s in range(j + 1, i + 1):
                if pos[s] == 0:
                    ok = False
                    break
            out[i, j] = ok
    return out


@pytest.mark.parametrize("pos", [
    list(range(10)),
    [0, 1, 2, 0, 1, 0, 0, 1, 2, 3, 4],
    [0] * 7,
    [5, 6, 7, 0, 1, 2, 3],          # first token always starts a sample
    [0, 1, 2, 3, 0, 1],             # truncated last sample
    [0, 2, 9, 0, 3, 1, 0],          # non-consecutive positions: only zeros start samples
])
def test_mask_brute_force(pos):
    pos = np.array(pos, np.int64)
    seg = ref.segment_ids(pos)
    n = len(pos)
    got = ref.allowed(seg, np.arange(n), np.arange(n))
    assert np.array_equal(got, _brute_allowed(pos))
    first = ref.segment_first(pos)
    for i in range(n):
        assert first[i] == min(j for j in range(n) if _brute_allowed(pos)[i, j])


# ---------------------------------------------------------------------------
# Attention forward
# ---------------------------------------------------------------------------

def _brute_fwd(q, k, v, pos, scale):
    """Pure-Python loops: per head and row, softmax over keys allowed by the brute mask."""
    N, hq, d = q.shape
    grp = hq // k.shape[1]
    A = _brute_allowed(pos)
    o = np.zeros_like(q)
    lse = np.zeros((hq, N))
    for h in range(hq):
        kv = h // grp
        for i in range(N):
            s = {}
            for j in range(N):
                if A[i, j]:
                    s[j] = scale * sum(q[i, h, e] * k[j, kv, e] for e in range(d))
            m = max(s.values())
            w = {j: math.exp(x - m) for j, x in s.items()}
            tot = sum(w.values())
            for e in range(d):
                o[i, h, e] = sum(w[j] * v[j, kv, e] for j in w) / tot
            lse[h, i] = m + math.log(tot)
    return o, lse


@pytest.mark.parametrize("N,hq,hkv,d,pos_kind", [(24, 2, 1, 4, "packed"), (17, 3, 3, 8, "single"),
                                                 (32, 4, 2, 5, "packed")])
def test_fwd_brute_force(N, hq, hkv, d, pos_kind):
    q, k, v = _rand(1, (N, hq, d)), _rand(2, (N, hkv, d)), _rand(3, (N, hkv, d))
    if pos_kind == "packed":
        pos = gen.position_ids_from_lengths([5, 1, 9, N - 15])
    else:
        pos = np.arange(N)
    scale = 0.37
    o, lse = ref.attn_fwd(q, k, v, pos, softmax_scale=scale, block_rows=5)
    ob, lb = _brute_fwd(q, k, v, pos, scale)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-12, atol=1e-13)


def test_fwd_rows_sum_to_one_and_default_scale():
    N, hq, hkv, d = 40, 4, 2, 16
    q, k = _rand(4, (N, hq, d)), _rand(5, (N, hkv, d))
    pos = gen.position_ids_from_lengths([13, 20, 7])
    o, _ = ref.attn_fwd(q, k, np.ones((N, hkv, d)), pos)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)
    # default scale is 1/sqrt(d)
    v = _rand(6, (N, hkv, d))
    a, la = ref.attn_fwd(q, k, v, pos)
    b, lb = ref.attn_fwd(q, k, v, pos, softmax_scale=1 / math.sqrt(d))
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_fwd_zero_scale_is_uniform_mean():
    """scale 0: every allowed key weighs the same, O_i is the mean of V over [start, i]."""
    N, d = 23, 3
    q, k, v = _rand(7, (N, 1, d)), _rand(8, (N, 1, d)), _rand(9, (N, 1, d))
    pos = gen.position_ids_from_lengths([4, 11, 8])
    o, lse = ref.attn_fwd(q, k, v, pos, softmax_scale=0.0)
    first = [0] * 4 + [4] * 11 + [15] * 8
    for i in range(N):
        np.testing.assert_allclose(o[i, 0], v[first[i]:i + 1, 0].mean(axis=0), rtol=1e-12)
        assert abs(lse[0, i] - math.log(i - first[i] + 1)) < 1e-12


def test_fwd_segment_start_rows_and_all_zero_positions():
    N, hq, hkv, d = 30, 4, 2, 8
    q, k, v = _rand(10, (N, hq, d)), _rand(11, (N, hkv, d)), _rand(12, (N, hkv, d))
    lens = [6, 1, 10, 13]
    pos = gen.position_ids_from_lengths(lens)
    scale = 0.5
    o, lse = ref.attn_fwd(q, k, v, pos, softmax_scale=scale)
    starts = np.cumsum([0] + lens[:-1])
    for i in starts:
        for h in range(hq):
            kv = h // 2
            assert np.array_equal(o[i, h], v[i, kv])
            assert abs(lse[h, i] - scale * np.dot(q[i, h], k[i, kv])) < 1e-12
    o0, _ = ref.attn_fwd(q, k, v, np.zeros(N, np.int64))
    for h in range(hq):
        assert np.array_equal(o0[:, h], v[:, h // 2])


def test_fwd_constant_key_is_cumulative_mean():
    N, d = 26, 4
    q = _rand(13, (N, 2, d))
    k = np.tile(_rand(14, (1, 1, d)), (N, 1, 1))
    v = _rand(15, (N, 1, d))
    pos = gen.position_ids_from_lengths([9, 17])
    o, lse = ref.attn_fwd(q, k, v, pos, softmax_scale=0.3)
    for i in range(N):
        s = 0 if i < 9 else 9
        for h in range(2):
            np.testing.assert_allclose(o[i, h], v[s:i + 1, 0].mean(axis=0), rtol=1e-12)
            expect = 0.3 * np.dot(q[i, h], k[0, 0]) + math.log(i - s + 1)
            assert abs(lse[h, i] - expect) < 1e-12


def test_fwd_packed_equals_separate_and_chunking():
    lens = [37, 5, 64, 1, 50]
    N, hq, hkv, d = sum(lens), 4, 1, 16
    q, k, v = _rand(16, (N, hq, d)), _rand(17, (N, hkv, d)), _rand(18, (N, hkv, d))
    pos = gen.position_ids_from_lengths(lens)
    o, lse = ref.attn_fwd(q, k, v, pos, block_rows=16)
    o_full, lse_full = ref.attn_fwd(q, k, v, pos, block_rows=N)
    np.testing.assert_allclose(o, o_full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_full, rtol=1e-12, atol=1e-14)
    s = 0
    for L in lens:
        sl = slice(s, s + L)
        os_, ls_ = ref.attn_fwd(q[sl], k[sl], v[sl], np.arange(L), block_rows=7)
        np.testing.assert_allclose(o[sl], os_, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[:, sl], ls_, rtol=1e-12, atol=1e-14)
        s += L
    # a boundary-blind mask (one sample) must differ: the SDPA failure mode on packed rows
    o_blind, _ = ref.attn_fwd(q, k, v, np.arange(N))
    assert np.abs(o_blind[37:] - o[37:]).max() > 1e-3


def test_full_layer_sp_equivalence():
    """seq->head, attention on each rank's heads, head->seq == attention over all heads
    on the unsharded sequence (heads are independent)."""
    P, T, H, d = 4, 8, 8, 8
    N = P * T
    qkv = gen.normal_bf16((77, 1), (P, T, 3, H, d))
    pos = gen.position_ids_from_lengths([11, 21])
    h2 = ref.seq_to_head(qkv)                       # [P][3][N][H/P][d]
    outs = []
    for r in range(P):
        o, _ = ref.attn_fwd(h2[r, 0], h2[r, 1], h2[r, 2], pos)
        outs.append(o)
    # head->seq of the float outputs: reuse the permutation on float arrays
    o_head = np.stack(outs)[:, None]                # [P][1][N][H/P][d]
    o_seq = ref.head_to_seq(o_head, P)              # [P][T][1][H][d]
    full = qkv.reshape(N, 3, H, d)
    o_ref, _ = ref.attn_fwd(full[:, 0], full[:, 1], full[:, 2], pos)
    np.testing.assert_allclose(o_seq.reshape(N, H, d), o_ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Attention backward
# ---------------------------------------------------------------------------

def test_bwd_finite_differences():
    N, hq, hkv, d = 14, 4, 2, 3
    q, k, v, do = _rand(20, (N, hq, d)), _rand(21, (N, hkv, d)), _rand(22, (N, hkv, d)), _rand(23, (N, hq, d))
    pos = gen.position_ids_from_lengths([6, 1, 7])
    scale = 0.8
    dq, dk, dv = ref.attn_bwd(q, k, v, do, pos, softmax_scale=scale, block_rows=4)

    def f(q_, k_, v_):
        o, _ = ref.attn_fwd(q_, k_, v_, pos, softmax_scale=scale)
        return float((o * do).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (f(**{kk + "_": vv for kk, vv in args_p.items()})
                        - f(**{kk + "_": vv for kk, vv in args_m.items()})) / (2 * eps)
        err = np.abs(num - g).max() / np.abs(g).max()
        assert err < 1e-7, (name, err)


def test_bwd_with_given_output():
    """D formed from a given output: the exact output gives the exact backward; an output
    off by delta_i moves D_i by dO_i . delta_i and dQ_i by -scale (dO_i . delta_i) sum_j P_ij k_j."""
    lens = [9, 1, 14]
    N, hq, hkv, d = sum(lens), 4, 2, 6
    q, k, v, do = _rand(60, (N, hq, d)), _rand(61, (N, hkv, d)), _rand(62, (N, hkv, d)), _rand(63, (N, hq, d))
    pos = gen.position_ids_from_lengths(lens)
    o, _ = ref.attn_fwd(q, k, v, pos, softmax_scale=0.6)
    want = ref.attn_bwd(q, k, v, do, pos, softmax_scale=0.6)
    got = ref.attn_bwd(q, k, v, do, pos, softmax_scale=0.6, o=o, block_rows=5)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)
    delta = np.zeros_like(o)
    delta[12, 1] = _rand(64, (d,))
    dq2, _, _ = ref.attn_bwd(q, k, v, do, pos, softmax_scale=0.6, o=o + delta)
    # row 12 (sample 3, keys 10..12), head 1 uses KV head 0: sum_j P_ij k_j is the output
    # of attention with v replaced by k
    ok, _ = ref.attn_fwd(q, k, k, pos, softmax_scale=0.6)
    shift = -0.6 * float(do[12, 1] @ delta[12, 1]) * ok[12, 1]
    np.testing.assert_allclose(dq2[12, 1] - want[0][12, 1], shift, rtol=1e-10, atol=1e-13)
    others = np.ones(N, bool)
    others[12] = False
    np.testing.assert_allclose(dq2[others], want[0][others], rtol=1e-12, atol=1e-14)


def test_bwd_gqa_equals_replicated_sum():
    N, hq, hkv, d = 33, 6, 2, 8
    grp = hq // hkv
    q, k, v, do = _rand(24, (N, hq, d)), _rand(25, (N, hkv, d)), _rand(26, (N, hkv, d)), _rand(27, (N, hq, d))
    pos = gen.position_ids_from_lengths([20, 13])
    dq, dk, dv = ref.attn_bwd(q, k, v, do, pos)
    kr, vr = np.repeat(k, grp, axis=1), np.repeat(v, grp, axis=1)
    dq2, dk2, dv2 = ref.attn_bwd(q, kr, vr, do, pos)
    np.testing.assert_allclose(dq, dq2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(N, hkv, grp, d).sum(2), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(N, hkv, grp, d).sum(2), rtol=1e-11, atol=1e-13)


def test_bwd_special_cases_and_segment_sums():
    N, hq, hkv, d = 40, 4, 1, 8
    q, k, v, do = _rand(28, (N, hq, d)), _rand(29, (N, hkv, d)), _rand(30, (N, hkv, d)), _rand(31, (N, hq, d))
    lens = [12, 1, 27]
    pos = gen.position_ids_from_lengths(lens)
    dq, dk, dv = ref.attn_bwd(q, k, v, do, pos, block_rows=9)
    starts = np.cumsum([0] + lens[:-1])
    assert not dq[starts].any()                          # a sample's first row sees only itself
    s = 0
    for L in lens:                                       # per sample: sum_j dV_j = sum_i dO_i, sum_j dK_j = 0
        np.testing.assert_allclose(dv[s:s + L, 0].sum(0), do[s:s + L].sum((0, 1)), rtol=1e-11, atol=1e-12)
        assert np.abs(dk[s:s + L, 0].sum(0)).max() < 1e-12
        s += L
    z = np.zeros(N, np.int64)
    dq0, dk0, dv0 = ref.attn_bwd(q, k, v, do, z)
    assert not dq0.any() and not dk0.any()
    np.testing.assert_allclose(dv0[:, 0], do.sum(1), rtol=1e-13)


def test_sampled_rows_and_cols_match_full():
    lens = [70, 3, 100, 37]
    N, hq, hkv, d = sum(lens), 4, 2, 16
    q, k, v, do = (gen.normal_bf16((55, s), sh) for s, sh in
                   ((1, (N, hq, d)), (2, (N, hkv, d)), (3, (N, hkv, d)), (4, (N, hq, d))))
    pos = gen.position_ids_from_lengths(lens)
    o, lse = ref.attn_fwd(q, k, v, pos, block_rows=32)
    dq, dk, dv = ref.attn_bwd(q, k, v, do, pos, block_rows=32)
    rows = np.array([0, 1, 69, 70, 71, 72, 73, 100, 172, 173, 200, N - 1])
    o_s, lse_s, dq_s = ref.attn_rows(q, k, v, do, pos, rows, chunk=5)
    np.testing.assert_allclose(o_s, o[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_s, lse[:, rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq_s, dq[rows], rtol=1e-11, atol=1e-12)
    cols = np.array([0, 5, 69, 70, 72, 73, 150, 172, 173, 190, N - 1])
    dk_s, dv_s = ref.attn_key_cols(q, k, v, do, pos, cols)
    np.testing.assert_allclose(dk_s, dk[cols], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv_s, dv[cols], rtol=1e-11, atol=1e-12)


def test_row_stats_match_forward_and_closed_forms():
    """LSE and O of attn_row_stats equal the (brute-force pinned) forward on any row
    range; D has closed forms: with every V row equal to c, O_i = c and D_i = dO_i . c;
    with scale 0, O_i is the mean of V over [start, i] and D_i = dO_i . that mean."""
    lens = [45, 1, 80, 30]
    N, hq, hkv, d = sum(lens), 4, 2, 16
    q, k, v, do = (_rand(40 + i, sh) for i, sh in
                   enumerate(((N, hq, d), (N, hkv, d), (N, hkv, d), (N, hq, d))))
    pos = gen.position_ids_from_lengths(lens)
    o, lse = ref.attn_fwd(q, k, v, pos, softmax_scale=0.4)
    for r0, r1, blk in ((0, N, 256), (3, 130, 7), (46, 47, 1), (100, N, 64)):
        l_s, o_s, D_s = ref.attn_row_stats(q, k, v, do, pos, r0, r1, softmax_scale=0.4, block_rows=blk)
        np.testing.assert_allclose(l_s, lse[:, r0:r1], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(o_s, o[r0:r1], rtol=1e-12, atol=1e-13)
        assert D_s.shape == (hq, r1 - r0)
    c = _rand(50, (d,))
    vc = np.tile(c, (N, hkv, 1))
    _, o_c, D_c = ref.attn_row_stats(q, k, vc, do, pos, 0, N, block_rows=33)
    np.testing.assert_allclose(o_c, np.broadcast_to(c, o_c.shape), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(D_c, (do @ c).T, rtol=1e-11, atol=1e-12)
    _, _, D_0 = ref.attn_row_stats(q, k, v, do, pos, 0, N, softmax_scale=0.0, block_rows=17)
    first = ref.segment_first(pos)
    for i in (0, 44, 45, 46, 47, 100, N - 1):
        for h in range(hq):
            mean = v[first[i]:i + 1, h // 2].mean(axis=0)
            assert abs(D_0[h, i] - float(do[i, h] @ mean)) < 1e-12


@pytest.mark.parametrize("lens,hq,hkv", [([70, 3, 100, 37], 4, 2), ([1, 64, 1, 130], 3, 1),
                                         ([211], 2, 2)])
def test_key_cols_from_stats_match_full_backward(lens, hq, hkv):
    """dK/dV of chosen key columns, from all-row statistics, equal the full backward's
    (itself pinned by finite differences) at those columns, with GQA and packing."""
    N, d = sum(lens), 8
    q, k, v, do = (gen.normal_bf16((61, s), sh) for s, sh in
                   ((1, (N, hq, d)), (2, (N, hkv, d)), (3, (N, hkv, d)), (4, (N, hq, d))))
    pos = gen.position_ids_from_lengths(lens)
    _, dk, dv = ref.attn_bwd(q, k, v, do, pos, softmax_scale=0.7, block_rows=32)
    lse, _, D = ref.attn_row_stats(q, k, v, do, pos, 0, N, softmax_scale=0.7, block_rows=40)
    cols = np.arange(N)
    dk_s, dv_s = ref.attn_key_cols_from_stats(q, k, v, do, pos, cols, lse, D, softmax_scale=0.7,
                                              block_rows=13)
    np.testing.assert_allclose(dk_s, dk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv_s, dv, rtol=1e-10, atol=1e-12)
    some = np.array(sorted({0, N - 1, N // 2, lens[0] - 1, min(N - 1, lens[0])}))
    dk_p, dv_p = ref.attn_key_cols_from_stats(q, k, v, do, pos, some, lse, D, softmax_scale=0.7)
    np.testing.assert_allclose(dk_p, dk[some], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv_p, dv[some], rtol=1e-10, atol=1e-12)
    # a wrong D (one row's value moved) must change some key's dK
    D_bad = D.copy()
    D_bad[0, N - 1] += 1.0
    dk_b, _ = ref.attn_key_cols_from_stats(q, k, v, do, pos, cols, lse, D_bad, softmax_scale=0.7)
    assert np.abs(dk_b - dk).max() > 1e-6


def test_bf16_widening_all_patterns_against_torch():
    """bf16_to_f64 over all 65536 bit patterns equals torch's bf16 -> float64
    conversion (NaN compared by class: both NaN), plus hand-worked values."""
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):          # signalling-NaN patterns widen to NaN
        ours = ref.bf16_to_f64(bits)
    theirs = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan_o, nan_t = np.isnan(ours), np.isnan(theirs)
    assert np.array_equal(nan_o, nan_t) and nan_o.sum() == 2 * 127
    assert np.array_equal(ours[~nan_o], theirs[~nan_t])
    assert np.array_equal(np.signbit(ours[~nan_o]), np.signbit(theirs[~nan_t]))   # -0 stays -0
    hand = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
            0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x7F80: math.inf, 0xFF80: -math.inf,
            0x3E80: 0.25, 0x4049: 3.140625}
    for b, val in hand.items():
        assert ref.bf16_to_f64(np.array([b], np.uint16))[0] == val
    assert ref.bf16_to_f64(np.array([0x8000], np.uint16))[0] == 0.0
    assert np.signbit(ref.bf16_to_f64(np.array([0x8000], np.uint16))[0])


@pytest.mark.parametrize("P,T,G,H,d,r,g0,g1", [(2, 3, 3, 4, 2, 1, 0, 3), (4, 2, 3, 8, 3, 2, 1, 3),
                                               (8, 2, 1, 8, 2, 0, 0, 1), (3, 4, 2, 6, 1, 2, 1, 2)])
def test_gather_share_is_rank_slice_of_relayout(P, T, G, H, d, r, g0, g1):
    """gather_share(x, r, g0, g1) equals rank r's seq->head share, groups [g0, g1),
    moved to token-major [N][G'][H/P][d]; checked by element tags against brute-force
    index loops too."""
    x, tok, grp, head, e = _tagged(P, T, G, H, d)
    got = ref.gather_share(x, r, g0, g1)
    want = np.ascontiguousarray(ref.seq_to_head(x, rank=r)[g0:g1].transpose(1, 0, 2, 3))
    assert got.shape == (P * T, g1 - g0, H // P, d)
    assert np.array_equal(got, want)
    hl = H // P
    for n in range(P * T):
        for gi in range(g1 - g0):
            for j in range(hl):
                for ee in range(d):
                    assert got[n, gi, j, ee] == (((n * G + g0 + gi) * H + r * hl + j) * d) + ee


# ---------------------------------------------------------------------------
# Token-weighted loss
# ---------------------------------------------------------------------------

def test_loss_worked_example_prompt_only_rank():
    """Rank 0 holds only prompt tokens (all -100); rank 1 has 3 valid tokens with losses
    1, 2, 3: rank losses (NaN, 2), total 2*3 = 6 over 3 tokens -> 2.0."""
    tl = np.array([[9.0, 9.0, 9.0, 9.0], [1.0, 100.0, 2.0, 3.0]])
    lab = np.array([[-100] * 4, [5, -100, 7, 8]])
    loss, rl, good, dtl = ref.weighted_loss(tl, lab)
    assert loss == 2.0
    assert np.isnan(rl[0]) and rl[1] == 2.0
    assert list(good) == [0, 3]
    assert np.array_equal(dtl, np.array([[0, 0, 0, 0], [1 / 3, 0, 1 / 3, 1 / 3]]))


@pytest.mark.parametrize("P", [1, 2, 8])
def test_loss_closed_form(P):
    rng = np.random.default_rng(P)
    tl = rng.uniform(0, 12, (P, 64))
    lab = rng.integers(0, 1000, (P, 64))
    lab[rng.random((P, 64)) < 0.3] = -100
    loss, rl, good, dtl = ref.weighted_loss(tl, lab)
    valid = lab != -100
    T = valid.sum()
    assert abs(loss - tl[valid].sum() / T) < 1e-12 * abs(loss)
    # P == 1 reduces to the plain masked mean; per-rank loss is that rank's masked mean
    for r in range(P):
        assert abs(rl[r] - tl[r][valid[r]].mean()) < 1e-12
    np.testing.assert_array_equal(dtl, np.where(valid, 1.0 / T, 0.0))


def test_loss_zero_rank_and_all_masked():
    w = configs.Workload(3, "t", 8, 1024, 1, 1, 8, prompt_frac=0.15)
    inp = configs.loss_inputs(w)
    lab = inp["shift_labels"].copy()
    lab[0] = -100                                   # rank 0 fully masked
    loss, rl, good, dtl = ref.weighted_loss(inp["token_loss"], lab)
    valid = lab != -100
    assert good[0] == 0 and np.isnan(rl[0]) and np.isfinite(loss)
    assert abs(loss - inp["token_loss"][valid].astype(np.float64).sum() / valid.sum()) < 1e-12 * loss
    loss0, rl0, good0, dtl0 = ref.weighted_loss(inp["token_loss"], np.full_like(lab, -100))
    assert loss0 == 0.0 and not good0.any() and not dtl0.any() and np.isnan(rl0).all()


# ---------------------------------------------------------------------------
# Generator
# ---------------------------------------------------------------------------

def test_generator_lengths_and_positions():
    assert configs.WORKLOADS[2].lengths() == [6945, 2521, 1351, 2804, 3690, 6766, 3978, 1218, 3084, 411]
    assert configs.WORKLOADS[5].lengths() == [186631, 217417, 37964, 82276]
    assert configs.WORKLOADS[2].allowed_pairs() == 75345846
    assert configs.WORKLOADS[5].allowed_pairs() == 45156205905
    pos = configs.WORKLOADS[2].position_ids()
    assert pos.size == 32768 and (pos == 0).sum() == 10 and pos[6945] == 0 and pos[6944] == 6944


def test_generator_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0]   # ties go to even
    ours = gen.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert list(ours[:3]) == [0x3F80, 0x3F82, 0xBF80]


def test_generator_is_deterministic_and_chunked():
    a = gen.normal_bf16((1, 1), (gen.CHUNK + 5,))
    b = gen.normal_bf16((1, 1), (gen.CHUNK + 5,))
    assert np.array_equal(a, b)
    tail = gen.f32_to_bf16_bits(np.random.default_rng([1, 1, 1]).standard_normal(5, dtype=np.float32))
    assert np.array_equal(a[gen.CHUNK:], tail)


# ---------------------------------------------------------------------------
# Per-token cross-entropy from hidden states (fused-logit-loss definition)
# ---------------------------------------------------------------------------

def _lce_case(seed, N=6, K=5, V=9, ignore=(1,)):
    r = np.random.default_rng(seed)
    x, w = r.standard_normal((N, K)), r.standard_normal((V, K))
    lab = r.integers(0, V, N)
    for i in ignore:
        lab[i] = -100
    return x, w, lab, r.standard_normal(N)


def test_lce_matches_library_log_softmax():
    from scipy.special import log_softmax, logsumexp
    x, w, lab, _ = _lce_case(1)
    tl, lse = ref.linear_cross_entropy(x, w, lab)
    logits = x @ w.T
    assert np.allclose(lse, logsumexp(logits, axis=1), rtol=0, atol=1e-12)
    ls = log_softmax(logits, axis=1)
    for t, y in enumerate(lab):
        assert tl[t] == 0.0 if y == -100 else abs(tl[t] + ls[t, y]) < 1e-12


def test_lce_gradients_finite_differences():
    x, w, lab, g = _lce_case(2)
    _, _, dx, dw = ref.linear_cross_entropy(x, w, lab, g)
    f = lambda xx, ww: float(np.dot(g, ref.linear_cross_entropy(xx, ww, lab)[0]))
    h = 1e-6
    for arr, grad, which in ((x, dx, 0), (w, dw, 1)):
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[i] += h
            m[i] -= h
            num[i] = (f(p, w) - f(m, w)) / (2 * h) if which == 0 else (f(x, p) - f(x, m)) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7), which


def test_lce_closed_forms():
    """w = 0: every logit is 0, loss = ln V, dx = 0, dw_v = sum_t g_t (1/V - [y_t = v]) x_t.
    One vocabulary entry: loss 0 and zero gradients."""
    x, _, lab, g = _lce_case(3, V=7)
    V = 7
    tl, lse, dx, dw = ref.linear_cross_entropy(x, np.zeros((V, x.shape[1])), lab, g)
    valid = lab != -100
    assert np.allclose(tl, np.where(valid, math.log(V), 0.0), rtol=0, atol=1e-14)
    assert np.allclose(lse, math.log(V), rtol=0, atol=1e-14)
    assert np.all(dx == 0)
    want = np.zeros_like(dw)
    for t in range(len(lab)):
        if valid[t]:
            want += g[t] * (1.0 / V) * x[t]
            want[lab[t]] -= g[t] * x[t]
    assert np.allclose(dw, want, rtol=0, atol=1e-13)
    x1, w1, lab1, g1 = _lce_case(4, V=1, ignore=())
    lab1[:] = 0
    tl1, _, dx1, dw1 = ref.linear_cross_entropy(x1, w1, lab1, g1)
    assert np.allclose(tl1, 0, atol=1e-14) and np.allclose(dx1, 0, atol=1e-14) and np.allclose(dw1, 0, atol=1e-14)


def test_lce_shift_invariance_and_ignored_tokens():
    """Adding one vector to every row of w shifts all logits of a token equally: the
    losses and dx do not change.  Ignored tokens have no loss and no gradient; all
    ignored gives zeros."""
    x, w, lab, g = _lce_case(5)
    tl, lse, dx, dw = ref.linear_cross_entropy(x, w, lab, g)
    c = np.random.default_rng(6).standard_normal(w.shape[1])
    tl2, _, dx2, _ = ref.linear_cross_entropy(x, w + c, lab, g)
    assert np.allclose(tl, tl2, rtol=0, atol=1e-12) and np.allclose(dx, dx2, rtol=0, atol=1e-12)
    assert tl[1] == 0 and np.all(dx[1] == 0)
    x0 = x.copy()
    x0[1] += 100.0                                     # an ignored token's values do not matter
    _, _, dx0, dw0 = ref.linear_cross_entropy(x0, w, lab, g)
    assert np.allclose(dw0, dw, rtol=0, atol=1e-12)
    lab_all = np.full_like(lab, -100)
    tla, _, dxa, dwa = ref.linear_cross_entropy(x, w, lab_all, g)
    assert np.all(tla == 0) and np.all(dxa == 0) and np.all(dwa == 0)


def test_lce_vocab_rows_match_full():
    """dw of selected vocabulary rows (and every token's lse) equal the full oracle's,
    including label rows (the one-hot term), with token chunks that do not divide N."""
    x, w, lab, g = _lce_case(7, N=11, K=6, V=13, ignore=(2, 5))
    tl, lse, dx, dw = ref.linear_cross_entropy(x, w, lab, g)
    rows = np.array(sorted({0, 12, int(lab[0]), int(lab[3]), 7}))
    lse_s, dw_s = ref.linear_ce_vocab_rows(x, w, lab, g, rows, chunk=4)
    np.testing.assert_allclose(lse_s, lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dw_s, dw[rows], rtol=1e-12, atol=1e-13)
    _, dw_all = ref.linear_ce_vocab_rows(x, w, lab, g, np.arange(13), chunk=3)
    np.testing.assert_allclose(dw_all, dw, rtol=1e-12, atol=1e-13)

