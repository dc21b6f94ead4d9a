"""Calls on two streams at once: every entry point enqueues on the stream it is
given and keeps no state between calls (each call has its own workspace), so two
independent problems run concurrently on two streams give, bit for bit, what they
give one after the other on the default stream."""
import pytest

from synth import gen

from helpers import say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _problem(seed, N, hq, hkv, d, lens):
    import torch
    from ulysses_sequence_parallelism_share_amd import ops
    q, k, v, do = (to_dev_bf16(gen.normal_bf16((seed, s), sh)) for s, sh in
                   ((1, (N, hq, d)), (2, (N, hkv, d)), (3, (N, hkv, d)), (4, (N, hq, d))))
    pos = to_dev(gen.position_ids_from_lengths(lens))
    x = to_dev_bf16(gen.raw_bits_u16((seed, 5), (4, 96, 2, 8, 64)))
    bufs = dict(
        ws=ops.workspace(N, hq, hkv, d),
        o=torch.empty((N, hq, d), dtype=torch.bfloat16, device="cuda"),
        lse=torch.empty((hq, N), dtype=torch.float32, device="cuda"),
        dq=torch.empty((N, hq, d), dtype=torch.float32, device="cuda"),
        dk=torch.empty((N, hkv, d), dtype=torch.float32, device="cuda"),
        dv=torch.empty((N, hkv, d), dtype=torch.float32, device="cuda"),
        xh=torch.empty((4, 2, 384, 2, 64), dtype=torch.bfloat16, device="cuda"),
        xs=torch.empty((4, 96, 2, 8, 64), dtype=torch.bfloat16, device="cuda"))

    def run():
        b = bufs
        ops.sp_attn_fwd(q, k, v, pos, o=b["o"], lse=b["lse"], ws=b["ws"])
        ops.sp_attn_bwd(q, k, v, b["o"], do, b["lse"], pos, dq=b["dq"], dk=b["dk"], dv=b["dv"],
                        ws=b["ws"])
        ops.ulysses_seq_to_head(x, out=b["xh"])
        ops.ulysses_head_to_seq(b["xh"], 4, out=b["xs"])

    outs = [bufs[n] for n in ("o", "lse", "dq", "dk", "dv", "xh", "xs")]
    return run, outs, x


def test_two_streams_match_sequential():
    import torch
    say("two streams: attention fwd/bwd and relayout round trip, 2 x 6 rounds")
    p1 = _problem(301, 3000, 4, 1, 128, [1200, 1800])
    p2 = _problem(302, 2048, 8, 2, 64, [100, 1948])
    want = []
    for run, outs, _ in (p1, p2):
        run()
        torch.cuda.synchronize()
        want.append([t.clone() for t in outs])
        for t in outs:
            t.zero_()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(6):
        with torch.cuda.stream(s1):
            p1[0]()
        with torch.cuda.stream(s2):
            p2[0]()
    torch.cuda.synchronize()
    for (run, outs, x), w in zip((p1, p2), want):
        for got, ref in zip(outs, w):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))
        assert torch.equal(outs[-1].view(torch.int16), x.view(torch.int16))
