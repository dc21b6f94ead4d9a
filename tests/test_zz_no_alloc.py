"""The allocation-free backward (sp_attn_bwd_noalloc, for callers that cannot
allocate device memory) against the workspace backward it varies: bit-identical
gradients on consecutive calls of different sizes (the fixed device scratch keeps
the previous call's contents), within the oracle gates, and the scratch limit."""
import numpy as np
import pytest

from oracle import ref
from synth import gen

from helpers import f64_of, gate, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


CALLS = [  # N, hq, hkv, d, sample lengths: a larger call, then smaller ones
    (5000, 4, 1, 128, [3000, 1, 1999]),
    (1000, 6, 2, 64, [400, 600]),          # 3 query heads per KV head: gathered rows in scratch
    (300, 2, 2, 128, [300]),
]


def _case(seed, N, hq, hkv, d, lens):
    import torch
    from ulysses_sequence_parallelism_share_amd import ops
    q, k, v, do = (gen.normal_bf16((seed, s), sh) for s, sh in
                   ((1, (N, hq, d)), (2, (N, hkv, d)), (3, (N, hkv, d)), (4, (N, hq, d))))
    pos = gen.position_ids_from_lengths(lens)
    qd, kd, vd, dod = (to_dev_bf16(a) for a in (q, k, v, do))
    posd = to_dev(pos)
    o, lse = ops.sp_attn_fwd(qd, kd, vd, posd)
    return (q, k, v, do, pos), (qd, kd, vd, o, dod, lse, posd)


def test_noalloc_backward_matches_workspace_backward():
    import torch
    from ulysses_sequence_parallelism_share_amd import ops
    for i, (N, hq, hkv, d, lens) in enumerate(CALLS):
        say(f"noalloc call {i}: N={N} hq={hq} hkv={hkv} d={d}")
        host, dev = _case(90 + i, N, hq, hkv, d, lens)
        for gdt in (torch.float32, torch.bfloat16):
            want = ops.sp_attn_bwd(*dev, grad_dtype=gdt)
            got = ops.sp_attn_bwd_noalloc(*dev, grad_dtype=gdt)
            torch.cuda.synchronize()
            for nm, a, b in zip(("dQ", "dK", "dV"), got, want):
                assert torch.equal(a.view(torch.int16) if gdt == torch.bfloat16 else a.view(torch.int32),
                                   b.view(torch.int16) if gdt == torch.bfloat16 else b.view(torch.int32)), nm
        dq, dk, dv = ops.sp_attn_bwd_noalloc(*dev)
        q, k, v, do, pos = host
        dq_r, dk_r, dv_r = ref.attn_bwd(q, k, v, do, pos)
        gate("dQ (noalloc)", f64_of(dq), dq_r)
        gate("dK (noalloc)", f64_of(dk), dk_r)
        gate("dV (noalloc)", f64_of(dv), dv_r)


def test_noalloc_backward_rejects_oversize_and_runs_the_500k_share_shape():
    import torch
    from ulysses_sequence_parallelism_share_amd import _lib, ops
    N, hq, hkv, d = 1 << 20, 8, 1, 64
    say("noalloc oversize call (must be refused before any launch)")
    q = torch.zeros((N, hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((N, hkv, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((hq, N), dtype=torch.float32, device="cuda")
    pos = torch.zeros(N, dtype=torch.int64, device="cuda")
    with pytest.raises(_lib.SPError) as ei:
        ops.sp_attn_bwd_noalloc(q, k, k, q, q, lse, pos)
    assert ei.value.status == _lib.SP_E_SCRATCH
    del q, k, lse, pos
    # the 500K-token rank share's backward (N=524288, 4 query / 1 KV head, d=128) fits
    # the scratch: bit-identical to the workspace backward on a packed input
    N, hq, hkv, d = 524288, 4, 1, 128
    say(f"noalloc 500K-share shape: N={N}")
    g = torch.Generator(device="cuda").manual_seed(7)
    mk = lambda *s: torch.randn(*s, device="cuda", generator=g).to(torch.bfloat16)
    q, k, v, do = mk(N, hq, d), mk(N, hkv, d), mk(N, hkv, d), mk(N, hq, d)
    pos = to_dev(gen.position_ids_from_lengths([186631, 217417, 37964, 82276]))
    o, lse = ops.sp_attn_fwd(q, k, v, pos)
    want = ops.sp_attn_bwd(q, k, v, o, do, lse, pos, grad_dtype=torch.bfloat16)
    got = ops.sp_attn_bwd_noalloc(q, k, v, o, do, lse, pos, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
