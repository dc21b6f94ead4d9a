#!/usr/bin/env python3
"""Benchmark of one rank's share of a Ulysses attention layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
seq->head relayout of Q and K/V for rank 0, segment bounds from position_ids,
causal attention forward, head->seq of O, seq->head of dO, attention backward,
head->seq of dQ and dK/dV, and the token-weighted loss over all ranks.
Default workload: the 500K-token rank share at sp_size 8 (N=524288, 4 query
heads, 1 KV head, d=128, 4 packed samples).

Prints ONE JSON line.  `value` is attention fwd+bwd TFLOP/s over the whole
step (algorithmic FLOPs 14*d*A*hq, A = allowed causal pairs per head).
"""
from __future__ import annotations

import argparse
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBPS = 8000.0
METRIC = "causal attn fwd+bwd TFLOP/s per rank-share (%MFMA peak); relayout GB/s (%HBM)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=5, choices=[2, 3, 5])
    ap.add_argument("--relayout-reps", type=int, default=10,
                    help="timed round trips of the relayout-bound workload and of the K/V exchange (0: skip)")
    ap.add_argument("--cpu-tokens", type=int, default=20480,
                    help="tokens of the oracle's CPU-baseline sample (0: skip)")
    ap.add_argument("--other-configs", type=int, default=3,
                    help="timed fwd+bwd repetitions on the 32768- and 131072-token rank shares "
                         "(0: skip)")
    ap.add_argument("--lce-steps", type=int, default=3,
                    help="timed calls of the fused cross-entropy workload (0: skip)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="print a text summary of a rocprofv3 --stats kernel table and exit")
    ap.add_argument("--summarize-counters", metavar="COUNTER_CSV",
                    help="print the MFMA/LDS counter summary of one rocprofv3 --pmc run of "
                         "COUNTER_PASS and exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM-traffic summary of two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, then WRITE_SIZE) and exit")
    ap.add_argument("--relayout-profile", action="store_true",
                    help="run only the relayout dispatches of RELAYOUT_PLAN (for rocprofv3) and exit")
    ap.add_argument("--summarize-relayout", nargs=3, metavar=("TRACE_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="print per-dispatch time and HBM bytes of the --relayout-profile run "
                         "from a rocprofv3 kernel trace and two --pmc runs, and exit")
    return ap.parse_args()


def to_dev_bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _host_info():
    """Host cores, affinity, CPU model and BLAS threads of the process."""
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        import threadpoolctl
        blas = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        blas = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu_count": os.cpu_count(), "affinity": aff, "cpu_model": model,
            "blas_threads": int(blas)}


def _gate(name, got, ref_, rel_tol=5e-3, abs_tol=2e-2):
    got = np.asarray(got, np.float64)
    d = got - ref_
    rel = float(np.linalg.norm(d) / np.linalg.norm(ref_))
    mx = float(np.abs(d).max())
    return {"relL2": rel, "maxabs": mx, "pass": bool(np.isfinite(got).all() and rel <= rel_tol
                                                     and mx <= abs_tol)}


def cpu_baseline(w, tokens, dev):
    """The oracle (fp64 numpy) timed on the host on a bounded sample of the workload,
    and the in-job parity check on that sample.

    Attention: the first `tokens` tokens of the workload's first packed sample (one
    causal sample, the workload's heads and head_dim), fwd + bwd; the GPU path runs on
    the same inputs (fp32 gradients) and every output element is compared with the
    oracle's under the gates (relative L2 <= 5e-3, max abs <= 2e-2).  Also timed, each
    checked against the GPU: the seq->head relayout of a slice of the relayout-bound
    buffer (bit-exact) and the token-weighted loss of the long-sequence workload."""
    import torch
    from oracle import ref
    from synth import configs, gen
    from ulysses_sequence_parallelism_share_amd import ops
    host = _host_info()
    L = min(tokens, w.lengths()[0])
    q = gen.normal_bf16((w.cfg, 1), (L, w.hq, w.head_dim))
    k = gen.normal_bf16((w.cfg, 2), (L, w.hkv, w.head_dim))
    v = gen.normal_bf16((w.cfg, 3), (L, w.hkv, w.head_dim))
    do = gen.normal_bf16((w.cfg, 4), (L, w.hq, w.head_dim))
    pos = np.arange(L, dtype=np.int64)
    t0 = time.perf_counter()
    o_r, lse_r = ref.attn_fwd(q, k, v, pos)
    t1 = time.perf_counter()
    dq_r, dk_r, dv_r = ref.attn_bwd(q, k, v, do, pos)
    t2 = time.perf_counter()
    # the GPU path on the same sample
    qd, kd, vd, dod = (to_dev_bf16(a, dev) for a in (q, k, v, do))
    posd = torch.from_numpy(pos).to(dev)
    o, lse = ops.sp_attn_fwd(qd, kd, vd, posd)
    dq, dk, dv = ops.sp_attn_bwd(qd, kd, vd, o, dod, lse, posd)
    f64 = lambda t: (ref.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
                     if t.dtype == torch.bfloat16 else t.double().cpu().numpy())
    parity = {"sample": f"first {L} tokens of the workload's first packed sample, all heads",
              "O": _gate("O", f64(o), o_r), "dQ": _gate("dQ", f64(dq), dq_r),
              "dK": _gate("dK", f64(dk), dk_r), "dV": _gate("dV", f64(dv), dv_r),
              "lse_maxabs": float(np.abs(f64(lse) - lse_r).max())}
    del qd, kd, vd, dod, o, lse, dq, dk, dv
    # relayout: a slice of the relayout-bound buffer (P=8, 1024 tokens per rank)
    w4 = configs.WORKLOADS[4]
    xs = gen.normal_bf16((w4.cfg, 1), (w4.sp_size, 1024, w4.relayout_groups, w4.relayout_heads,
                                       w4.head_dim))
    t3 = time.perf_counter()
    h_r = ref.seq_to_head(xs)
    t4 = time.perf_counter()
    h_g = ops.ulysses_seq_to_head(to_dev_bf16(xs, dev))
    parity["relayout_bit_exact"] = bool(np.array_equal(
        h_g.view(torch.int16).cpu().numpy().view(np.uint16), h_r))
    # token-weighted loss of the long-sequence workload (N=131072 over 8 ranks, 10 % prompt)
    li = configs.loss_inputs(configs.WORKLOADS[3])
    t5 = time.perf_counter()
    l_r, _, good_r, _ = ref.weighted_loss(li["token_loss"], li["shift_labels"])
    t6 = time.perf_counter()
    l_g, _, good_g, _ = ops.sp_weighted_loss(torch.from_numpy(li["token_loss"]).to(dev),
                                              torch.from_numpy(li["shift_labels"]).to(dev))
    parity["loss_counts_exact"] = bool(np.array_equal(good_g.cpu().numpy(), good_r))
    parity["loss_relerr"] = abs(float(l_g.cpu()[0]) - l_r) / abs(l_r)
    parity["pass"] = bool(all(parity[n]["pass"] for n in ("O", "dQ", "dK", "dV"))
                          and parity["lse_maxabs"] <= 1e-3 and parity["relayout_bit_exact"]
                          and parity["loss_counts_exact"] and parity["loss_relerr"] <= 1e-5)
    A = L * (L + 1) // 2
    flops = 14.0 * w.head_dim * A * w.hq
    dt = t2 - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host["blas_threads"],
            "kind": "oracle", "seconds": dt,
            "sample": f"fp64 oracle attn_fwd+attn_bwd on one causal sample of {L} tokens "
                      f"(the first {L} tokens of the workload's first packed sample), "
                      f"hq={w.hq}, hkv={w.hkv}, d={w.head_dim}; {flops:.3e} algorithmic FLOP",
            "host": host,
            "extrapolated_full_workload_s": 14.0 * w.head_dim * w.allowed_pairs() * w.hq / (flops / dt),
            "phases_s": {"attn_fwd": t1 - t0, "attn_bwd": t2 - t1, "relayout": t4 - t3,
                         "loss": t6 - t5},
            "relayout_GB/s": 2 * xs.nbytes / (t4 - t3) / 1e9,
            "relayout_sample": f"seq->head of [8][1024][3][32][128] bf16 ({xs.nbytes} bytes)",
            "loss_sample": "token-weighted loss over 8 ranks x 16384 tokens"}, parity


def attention_config(dev, cfg, reps):
    """Attention fwd+bwd (bf16 gradients) on a rank-share workload without relayouts:
    average ms per fwd+bwd pair of calls and TFLOP/s of 14 d A hq."""
    import torch
    from synth import configs
    from ulysses_sequence_parallelism_share_amd import ops
    w = configs.WORKLOADS[cfg]
    inp = configs.rank_share_inputs(w)
    q, k, v, do = (to_dev_bf16(inp[n], dev) for n in ("q", "k", "v", "do"))
    pos = torch.from_numpy(inp["pos"]).to(dev)
    N, hq, hkv, d = w.n_tokens, w.hq, w.hkv, w.head_dim
    ws = ops.workspace(N, hq, hkv, d, dev)
    o = torch.empty((N, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((hq, N), dtype=torch.float32, device=dev)
    g = [torch.empty((N, h, d), dtype=torch.bfloat16, device=dev) for h in (hq, hkv, hkv)]

    def one():
        ops.sp_attn_fwd(q, k, v, pos, o=o, lse=lse, ws=ws)
        ops.sp_attn_bwd(q, k, v, o, do, lse, pos, grad_dtype=torch.bfloat16, dq=g[0], dk=g[1],
                        dv=g[2], ws=ws)

    one()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        one()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flop = 14.0 * d * w.allowed_pairs() * hq
    return {"workload": w.name, "sample_lengths": w.lengths(), "ms_fwd_bwd": ms,
            "TFLOP/s": flop / ms / 1e9, "frac_mfma": flop / ms / 1e9 / PEAK_BF16_TFLOPS}

# ---------------------------------------------------------------------------
# HBM traffic of the attention kernels, from rocprofv3 counters.
#
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one --pmc run each) are scaled
# by what the same counter reads for a plain device copy of known size in the
# same run (the relayout-bound workload's copy_ of 6 GiB), so that the figure
# is in bytes of HBM traffic.  The summary records a hash of the sources each
# kernel is built from; the bench reports the traffic only while it matches.
# ---------------------------------------------------------------------------
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_500k_share_hbm_traffic.txt")
KERNEL_SYMBOL = {"attn_fwd": "k_attn_fwd", "attn_bwd_dkdv": "k_attn_bwd_dkdv",
                 "attn_bwd_dq": "k_attn_bwd_dq"}
KERNEL_SOURCES = {"attn_fwd": ("attn_fwd.hip",),
                  "attn_bwd_dkdv": ("attn_bwd.hip", "attn_bwd_dkdv.inc"),
                  "attn_bwd_dq": ("attn_bwd.hip", "attn_bwd_dq.inc")}


def sources_hash(kernel):
    import hashlib
    csrc = os.path.join(ROOT, "ulysses_sequence_parallelism_share_amd", "csrc")
    h = hashlib.sha256()
    files = [os.path.join(csrc, n) for n in (*KERNEL_SOURCES[kernel], "common.h", "tile.h",
                                             "launch.h")]
    for f in (*files,
              os.path.join(ROOT, "ulysses_sequence_parallelism_share_amd", "build.py")):
        with open(f) as fh:
            text = fh.read()
        # code only: comments and layout do not change the kernel
        if f.endswith(".py"):
            text = re.sub(r"#[^\n]*", "", text)
        else:
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_counter_csv(path, counter):
    """Per-dispatch values of one counter: list of (kernel_name, KiB)."""
    import csv
    acc = {}
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            key = int(row["Dispatch_Id"])
            name, val = acc.get(key, (row["Kernel_Name"], 0.0))
            acc[key] = (name, val + float(row["Counter_Value"]))
    return [acc[k] for k in sorted(acc)]


def summarize_traffic(fetch_csv, write_csv):
    from synth import configs
    w = configs.WORKLOADS[4]
    copy_bytes = 2 * w.n_tokens * w.relayout_groups * w.relayout_heads * w.head_dim
    out = ["# HBM traffic per dispatch from rocprofv3 counters, 500K-token rank share",
           "# (N=524288, hq=4, hkv=1, d=128, 4 packed samples)",
           "# commands (GPU, from /tmp with TMPDIR=/tmp; REPO = the repository root):",
           "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d REPO/gpurun_out/pmc_fetch -o run "
           "-- python3 REPO/bench.py --steps 1 --warmup 0 --relayout-reps 1 --cpu-tokens 0 --other-configs 0",
           "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d REPO/gpurun_out/pmc_write -o run "
           "-- python3 REPO/bench.py --steps 1 --warmup 0 --relayout-reps 1 --cpu-tokens 0 --other-configs 0",
           "#   python3 REPO/bench.py --summarize-traffic "
           "REPO/gpurun_out/pmc_fetch/run_counter_collection.csv "
           "REPO/gpurun_out/pmc_write/run_counter_collection.csv",
           f"# calibration: the largest dispatch whose name holds 'copy' is the plain copy of "
           f"{copy_bytes} bytes (read {copy_bytes} + write {copy_bytes})"]
    factors = {}
    per_kernel = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = read_counter_csv(path, counter)
        copies = [v for n, v in rows if "copy" in n.lower()]
        if not copies:
            raise SystemExit(f"{path}: no copy dispatch to calibrate {counter} against")
        cal = max(copies)
        factors[counter] = copy_bytes / (cal * 1024.0)
        out.append(f"# {counter}: copy reads {cal:.1f} KiB -> factor {factors[counter]:.4f} "
                   "(bytes per counted byte)")
        for kernel, sym in KERNEL_SYMBOL.items():
            # demangled "...::k_name<...>(" or, where the profiler leaves it mangled, "<len>k_nameI"
            pat = re.compile(r"(^|[\s:\d])" + sym + r"([<(]|I[LZN])")
            vals = [v for n, v in rows if pat.search(n)]
            if vals:
                per_kernel.setdefault(kernel, {})[counter] = (sum(vals) / len(vals), len(vals))
    out.append("# per dispatch: counter KiB as read; traffic_bytes = fetch*1024*f_fetch + "
               "write*1024*f_write")
    for kernel, c in per_kernel.items():
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        fk, nd = c["FETCH_SIZE"]
        wk, _ = c["WRITE_SIZE"]
        tb = fk * 1024 * factors["FETCH_SIZE"] + wk * 1024 * factors["WRITE_SIZE"]
        out.append(f"kernel={kernel} dispatches={nd} fetch_kib={fk:.1f} write_kib={wk:.1f} "
                   f"traffic_bytes={tb:.0f} sources={sources_hash(kernel)}")
    return "\n".join(out)


def load_traffic(kernel):
    """Traffic bytes per launch of `kernel` from the committed summary, or None when the
    summary is absent or was taken from other sources than the current ones."""
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    for ln in lines:
        if not ln.startswith("kernel="):
            continue
        kv = dict(tok.split("=", 1) for tok in ln.split())
        if kv["kernel"] == kernel and kv["sources"] == sources_hash(kernel):
            return float(kv["traffic_bytes"])
    return None


COUNTER_PASS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES "
                "GRBM_GUI_ACTIVE SQ_INSTS_LDS SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT")
N_XCD, N_SIMD = 8, 1024        # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_counters(csv_path):
    """MFMA and LDS figures of the attention kernels from one rocprofv3 --pmc run of
    COUNTER_PASS: bf16 MFMA FLOP (MOPS x 512) against the kernel's executed FLOP, the
    clock the kernel ran at (GRBM_GUI_ACTIVE is summed over the 8 XCDs), MFMA busy
    cycles per SIMD-cycle (the profiler's MfmaUtil) and LDS bank conflicts."""
    import csv
    from synth import configs
    w = configs.WORKLOADS[5]
    A, hq, d = w.allowed_pairs(), w.hq, w.head_dim
    executed = {"attn_fwd": 4 * d * A * hq, "attn_bwd_dkdv": 8 * d * A * hq,
                "attn_bwd_dq": 6 * d * A * hq}
    disp = {}
    with open(csv_path, newline="") as fh:
        for r in csv.DictReader(fh):
            e = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "c": {},
                                                         "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = ["# MFMA and LDS counters per dispatch, 500K-token rank share (N=524288, hq=4, hkv=1,",
           "# d=128, 4 packed samples)",
           "# commands (GPU, from /tmp with TMPDIR=/tmp; REPO = the repository root):",
           f"#   rocprofv3 --pmc {COUNTER_PASS} --output-format csv -d REPO/gpurun_out/pmc_sq -o run "
           "-- python3 REPO/bench.py --steps 1 --warmup 0 --relayout-reps 1 --cpu-tokens 0 --other-configs 0 "
           "--lce-steps 1",
           "#   python3 REPO/bench.py --summarize-counters REPO/gpurun_out/pmc_sq/run_counter_collection.csv",
           "# mfma_flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (executed_flop: 4/8/6 d A hq for fwd/dK,dV/dQ;",
           "# 2 n V K for each cross-entropy product, 4096 x 128256 x 4096, the bench's --lce-steps call);",
           "# clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES /",
           "# (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs), the share of SIMD-cycles with the matrix unit busy at",
           "# the clock the kernel ran at; tflops_at_clock_peak = 1024 FLOP x 1024 SIMDs x clock;",
           "# lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE. Averages over the dispatches."]
    # the fused cross-entropy's three products on the Llama-3-8B LM head (one call)
    lw = configs.LCE_WORKLOADS[13]
    gemm_flop = 2 * lw.n_tokens * lw.vocab * lw.hidden
    kinds = [(k, s, None) for k, s in KERNEL_SYMBOL.items()] + [
        ("lce_gemm_logits", "k_gemm<true, true,", gemm_flop),
        ("lce_gemm_dx", "k_gemm<true, false,", gemm_flop),
        ("lce_gemm_dw", "k_gemm<false, false,", gemm_flop)]
    for kernel, sym, fixed_flop in kinds:
        if fixed_flop is None:
            pat = re.compile(r"(^|[\s:\d])" + sym + r"([<(]|I[LZN])")
            rows = [e for e in disp.values() if pat.search(e["name"])]
        else:
            rows = [e for e in disp.values() if sym in e["name"]]
        if not rows:
            continue
        executed[kernel] = executed.get(kernel, fixed_flop)
        n = len(rows)
        avg = lambda f: sum(f(e) for e in rows) / n
        ms = avg(lambda e: e["ns"]) / 1e6
        gui = avg(lambda e: e["c"]["GRBM_GUI_ACTIVE"]) / N_XCD
        flop = avg(lambda e: e["c"]["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512
        busy = avg(lambda e: e["c"]["SQ_VALU_MFMA_BUSY_CYCLES"]) / (gui * N_SIMD)
        clk = gui / (ms * 1e-3) / 1e9
        idx = avg(lambda e: e["c"]["SQ_LDS_IDX_ACTIVE"])
        conf = avg(lambda e: e["c"]["SQ_LDS_BANK_CONFLICT"]) / idx if idx else 0.0
        out.append(f"kernel={kernel} dispatches={n} avg_ms={ms:.2f} clock_ghz={clk:.3f} "
                   f"mfma_flop={flop:.4e} executed_flop={executed[kernel]:.4e} "
                   f"tflops={flop / ms / 1e9:.1f} tflops_at_clock_peak={1024 * N_SIMD * clk / 1e3:.1f} "
                   f"mfma_busy={busy:.3f} lds_insts={avg(lambda e: e['c']['SQ_INSTS_LDS']):.4e} "
                   f"lds_conflict={conf:.4f}")
    return "\n".join(out)


def summarize_trace(stats_csv):
    import csv
    rows = []
    with open(stats_csv, newline="") as fh:
        for r in csv.DictReader(fh):
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                         float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    out = [f"{'kernel':<44}{'calls':>7}{'total_us':>15}{'avg_us':>13}{'pct':>9}"]
    for n, c, t, a, p in rows:
        out.append(f"{n[:42]:<44}{c:>7}{t:>15.1f}{a:>13.1f}{p:>8.2f}%")
    return "\n".join(out)


# ---------------------------------------------------------------------------
# Relayout dispatches under the profiler.  --relayout-profile launches, in this
# order: a plain device copy of the relayout-bound buffer (the counters'
# calibration), then two round trips of the relayout-bound workload (P=8,
# N=262144, 32 heads, fused QKV), then two steps' worth of the 500K share's
# rank-0 relayouts.  Every entry is one k_relayout dispatch; bytes are the
# algorithmic read + write of that call.
# ---------------------------------------------------------------------------
def relayout_plan():
    from synth import configs
    w4, w5 = configs.WORKLOADS[4], configs.WORKLOADS[5]
    full = w4.n_tokens * w4.relayout_groups * w4.relayout_heads * w4.head_dim * 2   # bytes
    N, hq, hkv, d = w5.n_tokens, w5.hq, w5.hkv, w5.head_dim
    q_share, kv_share = N * hq * d * 2, 2 * N * hkv * d * 2
    plan = []
    for _ in range(2):
        plan += [("relayout-bound seq->head (all ranks)", "seq_to_head", 2 * full),
                 ("relayout-bound head->seq (all ranks)", "head_to_seq", 2 * full)]
    for _ in range(2):
        plan += [("500k step: Q seq->head (rank 0)", "seq_to_head", 2 * q_share),
                 ("500k step: K/V seq->head (rank 0)", "seq_to_head", 2 * kv_share),
                 ("500k step: O head->seq (rank 0)", "head_to_seq", 2 * q_share),
                 ("500k step: dO seq->head (rank 0)", "seq_to_head", 2 * q_share),
                 ("500k step: dQ head->seq (rank 0)", "head_to_seq", 2 * q_share),
                 ("500k step: dK/dV head->seq (rank 0)", "head_to_seq", 2 * kv_share)]
    return plan, full


def relayout_profile(dev):
    import torch
    from synth import configs
    from ulysses_sequence_parallelism_share_amd import ops
    w4, w5 = configs.WORKLOADS[4], configs.WORKLOADS[5]
    x = to_dev_bf16(configs.relayout_inputs(w4), dev)
    h = torch.empty((w4.sp_size, w4.relayout_groups, w4.n_tokens, w4.relayout_heads // w4.sp_size,
                     w4.head_dim), dtype=torch.bfloat16, device=dev)
    back = torch.empty_like(x)
    back.copy_(x)                                   # the calibration copy
    torch.cuda.synchronize()
    for _ in range(2):
        ops.ulysses_seq_to_head(x, out=h)
        ops.ulysses_head_to_seq(h, w4.sp_size, out=back)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))
    del x, h, back
    torch.cuda.empty_cache()
    P, N, hq, hkv, d = w5.sp_size, w5.n_tokens, w5.hq, w5.hkv, w5.head_dim
    inp = configs.exchange_inputs(w5)
    q_seq, kv_seq, do_seq = (to_dev_bf16(inp.pop(n), dev) for n in ("q_seq", "kv_seq", "do_seq"))
    qh = torch.empty((1, N, hq, d), dtype=torch.bfloat16, device=dev)
    kvh = torch.empty((2, N, hkv, d), dtype=torch.bfloat16, device=dev)
    doh = torch.empty_like(qh)
    o_seq, dq_seq, dkv_seq = (torch.zeros_like(t) for t in (q_seq, q_seq, kv_seq))
    torch.cuda.synchronize()
    for _ in range(2):
        ops.ulysses_seq_to_head(q_seq, rank=0, out=qh)
        ops.ulysses_seq_to_head(kv_seq, rank=0, out=kvh)
        ops.ulysses_head_to_seq(qh, P, rank=0, out=o_seq)
        ops.ulysses_seq_to_head(do_seq, rank=0, out=doh)
        ops.ulysses_head_to_seq(doh, P, rank=0, out=dq_seq)
        ops.ulysses_head_to_seq(kvh, P, rank=0, out=dkv_seq)
    torch.cuda.synchronize()
    log(f"[bench] relayout profile: {len(relayout_plan()[0])} relayout dispatches done")


def _relayout_rows(path, value_col=None, counter=None):
    """(dispatch_id, kernel name, value) of a rocprofv3 csv, ascending dispatch id; value is
    the duration in ns (kernel trace) or the counter summed over its instances (KiB)."""
    import csv
    acc = {}
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if counter is not None and r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            if counter is None:
                acc[key] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            else:
                name, v = acc.get(key, (r["Kernel_Name"], 0.0))
                acc[key] = (name, v + float(r["Counter_Value"]))
    return [(k, *acc[k]) for k in sorted(acc)]


def summarize_relayout(trace_csv, fetch_csv, write_csv):
    plan, full = relayout_plan()
    is_rel = re.compile(r"(^|[\s:\d])k_relayout([<(]|I[LZN])")
    trace = [r for r in _relayout_rows(trace_csv) if is_rel.search(r[1])]
    counts = {}
    for c, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _relayout_rows(path, counter=c)
        copies = [v for _, n, v in rows if "copy" in n.lower()]
        rel = [v for _, n, v in rows if is_rel.search(n)]
        counts[c] = (max(copies) if copies else None, rel)
    if len(trace) != len(plan) or any(len(v[1]) != len(plan) for v in counts.values()):
        raise SystemExit(f"expected {len(plan)} k_relayout dispatches, found {len(trace)} traced, "
                         f"{[len(v[1]) for v in counts.values()]} counted")
    out = ["# k_relayout per dispatch: kernel-trace duration and HBM bytes from rocprofv3 counters",
           "# workloads: relayout-bound (P=8, N=262144, 32 heads, d=128, fused QKV [8][32768][3][32][128]",
           "# bf16, 6 GiB each way) and the 500K-token rank share's rank-0 relayouts (N=524288,",
           "# Q/dO/O/dQ: 32 global heads -> 4, K/V and dK/dV: 8 global KV heads -> 1, d=128)",
           "# commands (GPU, from /tmp with TMPDIR=/tmp; REPO = the repository root):",
           "#   rocprofv3 --kernel-trace --output-format csv -d REPO/gpurun_out/rl_trace -o run "
           "-- python3 REPO/bench.py --relayout-profile",
           "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d REPO/gpurun_out/rl_fetch -o run "
           "-- python3 REPO/bench.py --relayout-profile",
           "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d REPO/gpurun_out/rl_write -o run "
           "-- python3 REPO/bench.py --relayout-profile",
           "#   python3 REPO/bench.py --summarize-relayout REPO/gpurun_out/rl_trace/run_kernel_trace.csv "
           "REPO/gpurun_out/rl_fetch/run_counter_collection.csv REPO/gpurun_out/rl_write/run_counter_collection.csv"]
    half = full          # a plain copy of the relayout-bound buffer reads and writes `full` bytes
    fc, wc = counts["FETCH_SIZE"][0], counts["WRITE_SIZE"][0]
    f_fetch = half / (fc * 1024) if fc else None
    f_write = half / (wc * 1024) if wc else None
    out.append(f"# calibration copy ({half} bytes each way): FETCH_SIZE {fc} KiB -> factor "
               f"{f_fetch}, WRITE_SIZE {wc} KiB -> factor {f_write}")
    out.append("# read_bytes/write_bytes = counter KiB x 1024 x factor; algorithmic = read once + write once")
    out.append(f"{'dispatch':<40}{'algo_GB':>9}{'ms':>9}{'GB/s':>9}{'%HBM':>7}"
               f"{'fetch_KiB':>14}{'write_KiB':>14}{'read_GB':>9}{'write_GB':>9}{'counted/algo':>13}")
    for i, (label, _, nbytes) in enumerate(plan):
        ns = trace[i][2]
        fk, wk = counts["FETCH_SIZE"][1][i], counts["WRITE_SIZE"][1][i]
        rb = fk * 1024 * (f_fetch or 1.0)
        wb = wk * 1024 * (f_write or 1.0)
        gbs = nbytes / ns
        out.append(f"{label:<40}{nbytes / 1e9:>9.3f}{ns / 1e6:>9.3f}{gbs:>9.1f}"
                   f"{100 * gbs / PEAK_HBM_GBPS:>6.1f}%{fk:>14.1f}{wk:>14.1f}{rb / 1e9:>9.3f}"
                   f"{wb / 1e9:>9.3f}{(rb + wb) / nbytes:>13.3f}")
    return "\n".join(out)


def relayout_bound(dev, reps):
    """The relayout-bound workload: P=8, N=262144, 32 heads, d=128, fused QKV (G=3),
    seq->head of all ranks then head->seq back, checked bit-exact on the device."""
    import torch
    from synth import configs
    from ulysses_sequence_parallelism_share_amd import ops
    w = configs.WORKLOADS[4]
    x = to_dev_bf16(configs.relayout_inputs(w), dev)
    h = torch.empty((w.sp_size, w.relayout_groups, w.n_tokens, w.relayout_heads // w.sp_size,
                     w.head_dim), dtype=torch.bfloat16, device=dev)
    back = torch.empty_like(x)
    for _ in range(2):
        ops.ulysses_seq_to_head(x, out=h)
        ops.ulysses_head_to_seq(h, w.sp_size, out=back)
    torch.cuda.synchronize()
    ops.sp_timing_enable(True)
    for _ in range(reps):
        ops.ulysses_seq_to_head(x, out=h)
        ops.ulysses_head_to_seq(h, w.sp_size, out=back)
    torch.cuda.synchronize()
    kt = ops.sp_timing_collect()
    ops.sp_timing_enable(False)
    exact = bool(torch.equal(back.view(torch.int16), x.view(torch.int16)))
    nbytes = 2 * x.numel() * 2                      # read once + write once
    # reference: a plain device-to-device copy of the same buffer (torch copy_)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    back.copy_(x)
    torch.cuda.synchronize()
    s0.record()
    for _ in range(reps):
        back.copy_(x)
    s1.record()
    torch.cuda.synchronize()
    copy_ms = s0.elapsed_time(s1) / reps
    out = {"workload": w.name, "bytes_per_direction": nbytes, "bit_exact_roundtrip": exact,
           "plain_copy": {"avg_ms": copy_ms, "GB/s": nbytes / copy_ms / 1e6}}
    for key, name in (("seq_to_head", "relayout_seq_to_head"), ("head_to_seq", "relayout_head_to_seq")):
        ms = kt[name]["avg_ms"]
        out[key] = {"avg_ms": ms, "GB/s": nbytes / ms / 1e6, "frac_hbm": nbytes / ms / 1e6 / PEAK_HBM_GBPS,
                    "frac_plain_copy": copy_ms / ms}
    del x, h, back
    torch.cuda.empty_cache()
    return out


def kv_exchange_bench(dev, reps):
    """The K/V exchange for fewer KV heads than ranks: 8 KV heads (Llama-3-8B) at
    sp_size 16, K and V together (G=2), N=65536 tokens, d=128: seq->head copies every
    KV head to the 2 ranks that use it, head->seq sums the two gradient copies (bf16).
    Algorithmic bytes: the sequence side once, the head side once (2x as large)."""
    import torch
    from synth import gen
    from ulysses_sequence_parallelism_share_amd import ops
    P, N, G, H, d = 16, 65536, 2, 8, 128
    x = to_dev_bf16(gen.normal_bf16((71, 1), (P, N // P, G, H, d)), dev)
    h = ops.ulysses_seq_to_head_kv(x)                       # [P][G][N][1][d]
    back = ops.ulysses_head_to_seq_kv_grad(h, H)
    torch.cuda.synchronize()
    ops.sp_timing_enable(True)
    for _ in range(reps):
        ops.ulysses_seq_to_head_kv(x, out=h)
        ops.ulysses_head_to_seq_kv_grad(h, H, out=back)
    torch.cuda.synchronize()
    kt = ops.sp_timing_collect()
    ops.sp_timing_enable(False)
    # each KV head reaches 2 ranks, so the summed gradient is exactly twice the input
    doubled = bool(torch.equal(back.float(), 2 * x.float()))
    nbytes = (x.numel() + h.numel()) * 2
    out = {"workload": f"kv-exchange-p{P}-n{N}-kv{H}-g{G}-d{d}", "bytes_per_direction": nbytes,
           "grad_is_sum_of_copies": doubled}
    for key, name in (("seq_to_head", "relayout_kv_seq_to_head"),
                      ("head_to_seq_sum", "relayout_kv_head_to_seq_sum")):
        ms = kt[name]["avg_ms"]
        out[key] = {"avg_ms": ms, "GB/s": nbytes / ms / 1e6, "frac_hbm": nbytes / ms / 1e6 / PEAK_HBM_GBPS}
    del x, h, back
    torch.cuda.empty_cache()
    return out


def linear_ce_bench(dev, steps):
    """The fused per-token cross-entropy on the Llama-3-8B-shaped LM head: 4096 tokens
    (one chunk), hidden 4096, vocabulary 128256, forward and both gradients per call;
    algorithmic FLOP 6*N*V*K (three products)."""
    import torch
    from synth import configs
    from ulysses_sequence_parallelism_share_amd import ops
    w = configs.LCE_WORKLOADS[13]
    inp = configs.lce_inputs(w)
    x, mat = to_dev_bf16(inp["x"], dev), to_dev_bf16(inp["w"], dev)
    lab = torch.from_numpy(inp["labels"]).to(dev)
    g = torch.from_numpy(inp["g"]).to(dev)
    N, K, V = w.n_tokens, w.hidden, w.vocab
    out = ops.sp_linear_ce(x, mat, lab, g, chunk_tokens=N)
    nb = int(ops._lib.call("sp_linear_ce_workspace_bytes", V, N))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    ops.sp_linear_ce(x, mat, lab, g, chunk_tokens=N, out=out, ws=ws)
    torch.cuda.synchronize()
    ops.sp_timing_enable(True)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        ops.sp_linear_ce(x, mat, lab, g, chunk_tokens=N, out=out, ws=ws)
    t1.record()
    torch.cuda.synchronize()
    kt = ops.sp_timing_collect()
    ops.sp_timing_enable(False)
    ms = t0.elapsed_time(t1) / steps
    gemm_flop = 2.0 * N * V * K
    kernels = {k: v["avg_ms"] for k, v in kt.items()}
    dom = max(("lce_gemm_logits", "lce_gemm_dx", "lce_gemm_dw"), key=lambda n: kernels[n])
    tf = gemm_flop / kernels[dom] / 1e9
    res = {"workload": w.name, "ms_per_call": ms, "TFLOP/s": 3 * gemm_flop / ms / 1e9,
           "frac_mfma": 3 * gemm_flop / ms / 1e9 / PEAK_BF16_TFLOPS, "kernels_ms": kernels,
           "roofline": {"kernel": dom, "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                        "algorithmic_flop_per_launch": gemm_flop}}
    del x, mat, out, ws
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.summarize_relayout:
        print(summarize_relayout(*args.summarize_relayout))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the all-to-all is emulated on one device); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import configs
    from ulysses_sequence_parallelism_share_amd import ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.relayout_profile:
        relayout_profile(dev)
        return
    w = configs.WORKLOADS[args.workload]
    P, N, hq, hkv, d = w.sp_size, w.n_tokens, w.hq, w.hkv, w.head_dim
    lengths = w.lengths()
    A = w.allowed_pairs()
    fwd_flop = 4.0 * d * A * hq
    bwd_flop = 10.0 * d * A * hq
    log(f"[bench] workload {w.name}: lengths {lengths}, A={A}")

    t0 = time.time()
    relayout_in_step = args.workload == 5
    if relayout_in_step:
        inp = configs.exchange_inputs(w)
        q_seq = to_dev_bf16(inp.pop("q_seq"), dev)
        kv_seq = to_dev_bf16(inp.pop("kv_seq"), dev)
        do_seq = to_dev_bf16(inp.pop("do_seq"), dev)
        qh = torch.empty((1, N, hq, d), dtype=torch.bfloat16, device=dev)
        kvh = torch.empty((2, N, hkv, d), dtype=torch.bfloat16, device=dev)
        doh = torch.empty((1, N, hq, d), dtype=torch.bfloat16, device=dev)
        o_seq = torch.zeros_like(q_seq)
        dq_seq = torch.zeros_like(q_seq)
        dkv_seq = torch.zeros_like(kv_seq)
    else:
        inp = configs.rank_share_inputs(w)
        qh = to_dev_bf16(inp.pop("q"), dev)[None]
        kvh = torch.stack([to_dev_bf16(inp.pop("k"), dev), to_dev_bf16(inp.pop("v"), dev)])
        doh = to_dev_bf16(inp.pop("do"), dev)[None]
        q_seq = kv_seq = do_seq = o_seq = dq_seq = dkv_seq = None
    pos = torch.from_numpy(inp["pos"]).to(dev)
    lw = configs.Workload(w.cfg, w.name, P, N, hq, hkv, d, prompt_frac=0.1)
    li = configs.loss_inputs(lw)
    token_loss = torch.from_numpy(li["token_loss"]).to(dev)
    labels = torch.from_numpy(li["shift_labels"]).to(dev)
    o = torch.empty((N, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((hq, N), dtype=torch.float32, device=dev)
    dq = torch.empty((1, N, hq, d), dtype=torch.bfloat16, device=dev)
    dkv = torch.empty((2, N, hkv, d), dtype=torch.bfloat16, device=dev)
    ws = ops.workspace(N, hq, hkv, d, dev)
    loss_out = (torch.empty(1, dtype=torch.float32, device=dev),
                torch.empty(P, dtype=torch.float32, device=dev),
                torch.empty(P, dtype=torch.int64, device=dev),
                torch.empty((P, N // P), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")

    cpu = parity = None
    if args.cpu_tokens > 0:
        # the oracle on a bounded sample, and the in-job parity check on it, before timing
        t1 = time.time()
        cpu, parity = cpu_baseline(w, args.cpu_tokens, dev)
        log(f"[bench] cpu baseline and parity check done in {time.time() - t1:.1f}s "
            f"(parity {'pass' if parity['pass'] else 'FAIL'})")

    relayout_bytes = 0

    def step():
        nonlocal relayout_bytes
        nb = 0
        if relayout_in_step:
            ops.ulysses_seq_to_head(q_seq, rank=0, out=qh)
            ops.ulysses_seq_to_head(kv_seq, rank=0, out=kvh)
            nb += 2 * 2 * (qh.numel() + kvh.numel())
        ops.sp_attn_fwd(qh[0], kvh[0], kvh[1], pos, o=o, lse=lse, ws=ws)
        if relayout_in_step:
            ops.ulysses_head_to_seq(o[None], P, rank=0, out=o_seq)
            ops.ulysses_seq_to_head(do_seq, rank=0, out=doh)
            nb += 2 * 2 * (o.numel() + doh.numel())
        ops.sp_attn_bwd(qh[0], kvh[0], kvh[1], o, doh[0], lse, pos, grad_dtype=torch.bfloat16,
                        dq=dq[0], dk=dkv[0], dv=dkv[1], ws=ws)
        if relayout_in_step:
            ops.ulysses_head_to_seq(dq, P, rank=0, out=dq_seq)
            ops.ulysses_head_to_seq(dkv, P, rank=0, out=dkv_seq)
            nb += 2 * 2 * (dq.numel() + dkv.numel())
        ops.sp_weighted_loss(token_loss, labels, out=loss_out)
        relayout_bytes = nb

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")
    ops.sp_timing_enable(True)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    kt = ops.sp_timing_collect()
    ops.sp_timing_enable(False)
    log(f"[bench] {args.steps} timed steps: {ms_per_step:.3f} ms/step")

    per_step = {k: v["total_ms"] / args.steps for k, v in kt.items()}
    fwd_ms = kt["attn_fwd"]["avg_ms"]
    # small grids run the backward as one fused launch (attn_bwd_fused)
    fused = "attn_bwd_fused" in kt
    dkdv_ms = None if fused else kt["attn_bwd_dkdv"]["avg_ms"]
    dq_ms = None if fused else kt["attn_bwd_dq"]["avg_ms"]
    bwd_ms = kt["attn_bwd_fused"]["avg_ms"] if fused else dkdv_ms + dq_ms
    attn_kernel_ms = sum(per_step.get(n, 0.0) for n in
                         ("segment_chunks", "segment_scan", "gather_rows", "attn_fwd_v_transpose",
                          "attn_fwd", "bwd_rowstats", "attn_bwd_dkdv", "attn_bwd_dq",
                          "attn_bwd_fused"))
    # algorithmic FLOP per launch (credited: 4 d A hq forward, 10 d A hq backward, of
    # which 8 in the dK/dV kernel and 2 in dQ, whose S and dP recomputes are extra)
    algo = ({"attn_fwd": fwd_flop, "attn_bwd_fused": bwd_flop} if fused else
            {"attn_fwd": fwd_flop, "attn_bwd_dkdv": 0.8 * bwd_flop, "attn_bwd_dq": 0.2 * bwd_flop})
    executed = {"attn_fwd": fwd_flop, "attn_bwd_dkdv": 0.8 * bwd_flop, "attn_bwd_dq": 0.6 * bwd_flop,
                "attn_bwd_fused": 1.4 * bwd_flop}
    dom = max(algo, key=lambda n: kt[n]["avg_ms"])
    dom_tflops = algo[dom] / kt[dom]["avg_ms"] / 1e9
    roofline = {"kernel": dom, "bound": "mfma", "achieved": dom_tflops, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": dom_tflops / PEAK_BF16_TFLOPS,
                "traffic": load_traffic(dom) if args.workload == 5 and dom in KERNEL_SOURCES else None,
                "avg_ms": kt[dom]["avg_ms"], "algorithmic_flop_per_launch": algo[dom]}
    value = (fwd_flop + bwd_flop) / ms_per_step / 1e9
    attention = {
        "fwd_flop": fwd_flop, "bwd_flop": bwd_flop,
        "attn_fwd_ms": fwd_ms, "attn_bwd_dkdv_ms": dkdv_ms, "attn_bwd_dq_ms": dq_ms,
        "attn_bwd_ms": bwd_ms, "bwd_fused_launch": fused,
        "fwd_kernel_tflops": fwd_flop / fwd_ms / 1e9,
        "bwd_kernels_tflops": bwd_flop / bwd_ms / 1e9,
        "attention_calls_ms": attn_kernel_ms,
        "tflops_attention_kernels": (fwd_flop + bwd_flop) / attn_kernel_ms / 1e9,
        "frac_mfma_attention_kernels": (fwd_flop + bwd_flop) / attn_kernel_ms / 1e9 / PEAK_BF16_TFLOPS,
        "frac_mfma_step": value / PEAK_BF16_TFLOPS,
    }
    # every attention kernel against its roofline: matrix kernels in TFLOP/s of
    # their algorithmic (and executed) FLOP, the pre-passes in GB/s of the bytes
    # they must move
    Mpad = (N * (hq // hkv) + 63) // 64 * 64
    hbm_bytes = {"attn_fwd_v_transpose": 2 * N * hkv * d * 2,
                 "bwd_rowstats": N * hq * d * 2 * 2 + N * hq * 4 + 8 * hkv * Mpad}
    kernel_rooflines = {}
    for n, f in algo.items():
        ms = kt[n]["avg_ms"]
        kernel_rooflines[n] = {"bound": "mfma", "avg_ms": ms, "achieved": f / ms / 1e9,
                               "executed_tflops": executed[n] / ms / 1e9, "unit": "TFLOP/s",
                               "peak": PEAK_BF16_TFLOPS, "frac": f / ms / 1e9 / PEAK_BF16_TFLOPS}
    for n, b in hbm_bytes.items():
        if n in kt:
            ms = kt[n]["avg_ms"]
            kernel_rooflines[n] = {"bound": "hbm", "avg_ms": ms, "achieved": b / ms / 1e6,
                                   "unit": "GB/s", "peak": PEAK_HBM_GBPS,
                                   "frac": b / ms / 1e6 / PEAK_HBM_GBPS}
    zero_copy = None
    if relayout_in_step:
        # The same step with attention reading rank 0's heads in place from the
        # exchange buffers and writing O and the gradients back (no relayouts).
        Hq, Hkv = q_seq.shape[3], kv_seq.shape[3]
        Qv = q_seq.view(N, 1, Hq, d)[:, 0, :hq]
        KVv = kv_seq.view(N, 2, Hkv, d)
        DOv = do_seq.view(N, 1, Hq, d)[:, 0, :hq]
        Ov = o_seq.view(N, 1, Hq, d)[:, 0, :hq]
        DQv = dq_seq.view(N, 1, Hq, d)[:, 0, :hq]
        DKVv = dkv_seq.view(N, 2, Hkv, d)

        def zc_step():
            o_, lse_ = ops.sp_attn_fwd_strided(Qv, KVv[:, 0, :hkv], KVv[:, 1, :hkv], pos, o=Ov,
                                               lse=lse, ws=ws)
            ops.sp_attn_bwd_strided(Qv, KVv[:, 0, :hkv], KVv[:, 1, :hkv], Ov, DOv, lse, pos,
                                    grad_dtype=torch.bfloat16, dq=DQv, dk=DKVv[:, 0, :hkv],
                                    dv=DKVv[:, 1, :hkv], ws=ws)
            ops.sp_weighted_loss(token_loss, labels, out=loss_out)

        zc_step()
        torch.cuda.synchronize()
        z0, z1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        z0.record()
        for _ in range(args.steps):
            zc_step()
        z1.record()
        torch.cuda.synchronize()
        zc_ms = z0.elapsed_time(z1) / args.steps
        zero_copy = {"ms_per_step": zc_ms, "TFLOP/s": (fwd_flop + bwd_flop) / zc_ms / 1e9,
                     "note": "attention on strided views of the exchange buffers, no relayouts"}
        log(f"[bench] zero-copy step: {zc_ms:.3f} ms/step")

    relayout = None
    if relayout_in_step:
        rl_ms = per_step.get("relayout_seq_to_head", 0.0) + per_step.get("relayout_head_to_seq", 0.0)
        relayout = {"step_bytes": relayout_bytes, "step_ms": rl_ms,
                    "step_GB/s": relayout_bytes / rl_ms / 1e6,
                    "step_frac_hbm": relayout_bytes / rl_ms / 1e6 / PEAK_HBM_GBPS}
    del q_seq, kv_seq, do_seq, o_seq, dq_seq, dkv_seq
    torch.cuda.empty_cache()

    relayout_bound_out = None
    if args.relayout_reps > 0:
        t1 = time.time()
        relayout_bound_out = relayout_bound(dev, args.relayout_reps)
        log(f"[bench] relayout-bound workload done in {time.time() - t1:.1f}s")

    kv_ex = None
    if args.relayout_reps > 0:
        t1 = time.time()
        kv_ex = kv_exchange_bench(dev, args.relayout_reps)
        log(f"[bench] K/V exchange done in {time.time() - t1:.1f}s")

    lce = None
    if args.lce_steps > 0:
        t1 = time.time()
        lce = linear_ce_bench(dev, args.lce_steps)
        log(f"[bench] linear cross-entropy: {lce['ms_per_call']:.2f} ms/call "
            f"({time.time() - t1:.1f}s)")

    other = None
    if args.other_configs > 0 and args.workload == 5:
        other = {}
        for cfg in (2, 3):
            t1 = time.time()
            other[str(cfg)] = attention_config(dev, cfg, args.other_configs)
            log(f"[bench] config {cfg}: {other[str(cfg)]['TFLOP/s']:.0f} TFLOP/s "
                f"({time.time() - t1:.1f}s)")

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "n_tokens": N, "sp_size": P, "hq": hq, "hkv": hkv,
                   "head_dim": d, "sample_lengths": lengths, "allowed_pairs_per_head": A,
                   "grad_dtype": "bf16", "parallelism": "one rank's share (Ulysses sp_size "
                   f"{P}) on 1 GPU; all-to-all emulated on device"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "other_configs": other,
        "attention": attention,
        "relayout_step": relayout,
        "zero_copy_step": zero_copy,
        "linear_ce": lce,
        "relayout_bound": relayout_bound_out,
        "kv_exchange": kv_ex,
        "kernels_ms_per_step": per_step,
        "kernel_rooflines": kernel_rooflines,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
