"""The attention path, the loss and the fused cross-entropy under HIP graph capture:
every launch of the library is a kernel (no memset or copy nodes), so a captured
step replays to the eager results bit for bit, replay after replay, with the
program's own eager work and synchronisations in between."""
import numpy as np
import pytest

from synth import configs, gen

from helpers import say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    import torch
    from ulysses_sequence_parallelism_share_amd import ops
    N, hq, hkv, d = 1500, 4, 2, 128
    lens = [700, 1, 799]
    say(f"graph capture: N={N} hq={hq} hkv={hkv} d={d}")
    q, k, v, do = (to_dev_bf16(gen.normal_bf16((41, i), s)) for i, s in
                   ((1, (N, hq, d)), (2, (N, hkv, d)), (3, (N, hkv, d)), (4, (N, hq, d))))
    pos = to_dev(gen.position_ids_from_lengths(lens))
    li = configs.loss_inputs(configs.Workload(3, "t", 4, 1024, 4, 1, 128, prompt_frac=0.1))
    tl, lab = to_dev(li["token_loss"]), to_dev(li["shift_labels"])
    ws = ops.workspace(N, hq, hkv, d)
    o = torch.empty((N, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, N), dtype=torch.float32, device="cuda")
    dq = torch.empty((N, hq, d), dtype=torch.float32, device="cuda")
    dk = torch.empty((N, hkv, d), dtype=torch.float32, device="cuda")
    dv = torch.empty((N, hkv, d), dtype=torch.float32, device="cuda")
    ce = configs.lce_inputs(configs.LCE_WORKLOADS[11])
    cx, cw = to_dev_bf16(ce["x"]), to_dev_bf16(ce["w"])
    clab, cg = to_dev(ce["labels"]), to_dev(ce["g"])
    cn, ck = cx.shape
    cout = (torch.empty(cn, dtype=torch.float32, device="cuda"),
            torch.empty(cn, dtype=torch.float32, device="cuda"),
            torch.empty((cn, ck), dtype=torch.float32, device="cuda"),
            torch.empty((cw.shape[0], ck), dtype=torch.float32, device="cuda"))
    cws = torch.empty(ops._lib.call("sp_linear_ce_workspace_bytes", cw.shape[0], 128),
                      dtype=torch.uint8, device="cuda")
    lout = (torch.empty(1, dtype=torch.float32, device="cuda"),
            torch.empty(4, dtype=torch.float32, device="cuda"),
            torch.empty(4, dtype=torch.int64, device="cuda"),
            torch.empty((4, 256), dtype=torch.float32, device="cuda"))

    def step():
        ops.sp_attn_fwd(q, k, v, pos, o=o, lse=lse, ws=ws)
        ops.sp_attn_bwd(q, k, v, o, do, lse, pos, dq=dq, dk=dk, dv=dv, ws=ws)
        ops.sp_weighted_loss(tl, lab, out=lout)
        ops.sp_linear_ce(cx, cw, clab, cg, chunk_tokens=128, out=cout, ws=cws)

    outs = (o, lse, dq, dk, dv, *lout, *cout)
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in outs:                                # eager work between replays
            t.fill_(-3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(outs, want)):
            assert torch.equal(t, w), (rep, i)
    say("  4 replays bit-identical to eager")
