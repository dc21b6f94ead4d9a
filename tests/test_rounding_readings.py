"""The arithmetic behind two tolerance readings, on the CPU: the fp64 oracle's
quantities with only the GPU path's bf16 roundings applied (O stored in bf16 and
D formed from it, P handed over in bf16, dS rounded to bf16 before its product).

* Peaked softmax (softmax_scale 1 at head_dim 128): dP - D cancels on nearly
  one-hot rows, so the rounding of O alone moves dQ by about 5e-3 relative L2,
  and all the roundings together by more than 5e-3 against the exact gradient;
  the GPU cases are therefore gated against the backward given the bf16 O.
* Wide query groups (16 query heads per KV head): dK sums 16 heads, and these
  roundings alone put its max abs error above 2e-2 while relative L2 stays near
  2.5e-3 and max abs near 0.3 % of the largest value.
"""
import zlib

import numpy as np

from oracle import ref
from synth import gen


def _bf(x):
    return ref.bf16_to_f64(gen.f32_to_bf16_bits(np.asarray(x, np.float32)))


def _inputs(seed, N, hq, hkv, d):
    return tuple(ref.bf16_to_f64(gen.normal_bf16((seed, s), sh)) for s, sh in
                 ((1, (N, hq, d)), (2, (N, hkv, d)), (3, (N, hkv, d)), (4, (N, hq, d))))


def _rounded_backward(q, k, v, do, pos, scale, round_o=True, round_p=True, round_ds=True):
    """dQ, dK from the textbook backward with the chosen bf16 roundings."""
    N, hq, d = q.shape
    g = hq // k.shape[1]
    o, lse = ref.attn_fwd(q, k, v, pos, softmax_scale=scale)
    ob = _bf(o) if round_o else o
    seg = ref.segment_ids(pos)
    allowed = ref.allowed(seg, np.arange(N), np.arange(N))
    dq, dk = np.zeros_like(q), np.zeros_like(k)
    for h in range(hq):
        kh = h // g
        S = scale * (q[:, h] @ k[:, kh].T)
        P = np.where(allowed, np.exp(np.where(allowed, S, 0.0) - lse[h][:, None]), 0.0)
        if round_p:
            P = _bf(P)
        D = (do[:, h] * ob[:, h]).sum(1)
        dS = P * (do[:, h] @ v[:, kh].T - D[:, None])
        if round_ds:
            dS = _bf(dS)
        dq[:, h] = scale * dS @ k[:, kh]
        dk[:, kh] += scale * dS.T @ q[:, h]
    return dq, dk


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_peaked_softmax_rounding_exceeds_the_relative_gate_on_dq():
    # the peaked GPU case: 2000 tokens, 4 query heads, 1 KV head, d 128, scale 1; a
    # 700-token sample whose ids start at 5000, then a 1300-token one from 0
    name, N, hq, hkv, d, scale = "peaked-softmax-scale1", 2000, 4, 1, 128, 1.0
    q, k, v, do = _inputs(zlib.crc32(name.encode()) % 1000 + 1000, N, hq, hkv, d)
    pos = np.concatenate([np.arange(5000, 5000 + 700), np.arange(N - 700)]).astype(np.int64)
    dq_r, _, _ = ref.attn_bwd(q, k, v, do, pos, softmax_scale=scale)
    dq_o, _ = _rounded_backward(q, k, v, do, pos, scale, round_p=False, round_ds=False)
    dq_all, _ = _rounded_backward(q, k, v, do, pos, scale)
    assert 3e-3 < _rel(dq_o, dq_r) < 5e-3        # O's rounding alone: about 4.8e-3
    assert 5e-3 < _rel(dq_all, dq_r) < 1e-2      # all roundings: past the 5e-3 gate


def test_wide_group_rounding_exceeds_the_absolute_gate_on_dk():
    name, N, hq, hkv, d, lens = "gqa16-d64", 150, 16, 1, 64, [100, 50]
    q, k, v, do = _inputs(zlib.crc32(name.encode()) % 1000, N, hq, hkv, d)
    pos = gen.position_ids_from_lengths(lens)
    _, dk_r, _ = ref.attn_bwd(q, k, v, do, pos)
    _, dk = _rounded_backward(q, k, v, do, pos, 1.0 / np.sqrt(d))
    err = np.abs(dk - dk_r).max()
    assert err > 2e-2                            # past the absolute gate
    assert err < 0.01 * np.abs(dk_r).max()       # within 1 % of the largest value
    assert _rel(dk, dk_r) < 5e-3
