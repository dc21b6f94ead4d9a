"""Host logic of bench.py, on the CPU: the HBM-traffic summary built from rocprofv3 counter
files (calibration against the plain copy, kernel-name matching, per-dispatch averages),
the source-hash guard on the committed summary, the kernel-trace table, and the refusal
to run on more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _counter_csv(path, counter, rows):
    """rows: (dispatch_id, kernel_name, values per counter instance)."""
    with open(path, "w") as fh:
        fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for did, name, vals in rows:
            for v in vals:
                fh.write(f'{did},"{name}",{counter},{v}\n')


def test_traffic_summary_calibrates_against_the_copy(tmp_path):
    from synth import configs
    w = configs.WORKLOADS[4]
    copy_bytes = 2 * w.n_tokens * w.relayout_groups * w.relayout_heads * w.head_dim
    # FETCH_SIZE reads half the copied bytes, WRITE_SIZE all of them (split over 2 instances)
    f_copy = copy_bytes / 2 / 1024
    w_copy = copy_bytes / 1024
    dkdv = "void (anonymous namespace)::k_attn_bwd_dkdv<128>(bf16 const*, ...)"
    mangled_fwd = "_ZN12_GLOBAL__N_110k_attn_fwdILi128EEEvPKDF16bS2_"
    decoy = "k_attn_bwd_dkdv_helper(int)"          # must not count as the dK/dV kernel
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [
        (1, "__amd_rocclr_copyBuffer", [f_copy / 2, f_copy / 2]),
        (2, dkdv, [100.0, 200.0]),                 # 300 KiB
        (3, dkdv, [250.0, 250.0]),                 # 500 KiB -> average 400
        (4, mangled_fwd, [64.0]),
        (5, decoy, [1e9]),
    ])
    _counter_csv(write, "WRITE_SIZE", [
        (1, "__amd_rocclr_copyBuffer", [w_copy]),
        (2, dkdv, [10.0]),
        (3, dkdv, [30.0]),                         # average 20
        (4, mangled_fwd, [8.0]),
        (5, decoy, [1e9]),
    ])
    text = bench.summarize_traffic(str(fetch), str(write))
    assert "FETCH_SIZE: copy reads" in text and "factor 2.0000" in text
    assert "WRITE_SIZE: copy reads" in text and "factor 1.0000" in text
    lines = {ln.split()[0]: dict(t.split("=", 1) for t in ln.split())
             for ln in text.splitlines() if ln.startswith("kernel=")}
    d = lines["kernel=attn_bwd_dkdv"]
    assert d["dispatches"] == "2"
    assert float(d["traffic_bytes"]) == pytest.approx(400 * 1024 * 2 + 20 * 1024)
    assert d["sources"] == bench.sources_hash("attn_bwd_dkdv")
    f = lines["kernel=attn_fwd"]
    assert float(f["traffic_bytes"]) == pytest.approx(64 * 1024 * 2 + 8 * 1024)
    assert "kernel=attn_bwd_dq" not in lines


def test_counter_summary_formulas(tmp_path):
    """MFMA FLOP = MOPS x 512; the clock and the busy share use GRBM_GUI_ACTIVE per XCD
    (the profiler sums it over the 8 XCDs); several counter instances of one dispatch are
    summed; dispatches are averaged; other kernels are ignored."""
    from synth import configs
    w = configs.WORKLOADS[5]
    fwd = "void (anonymous namespace)::k_attn_fwd<128>(bf16 const*, ...)"
    path = tmp_path / "sq.csv"
    ms = 2.0                                            # 2 ms per dispatch
    gui_per_xcd = 3.6e6                                 # 1.8 GHz over 2 ms
    busy = 0.5 * gui_per_xcd * 1024                     # half of the SIMD-cycles
    with open(path, "w") as fh:
        fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
        for did in (7, 9):
            rows = [("GRBM_GUI_ACTIVE", [gui_per_xcd] * 8),
                    ("SQ_INSTS_VALU_MFMA_MOPS_BF16", [1e9, 1e9]),
                    ("SQ_VALU_MFMA_BUSY_CYCLES", [busy / 4] * 4),
                    ("SQ_INSTS_LDS", [5.0]), ("SQ_LDS_IDX_ACTIVE", [100.0]),
                    ("SQ_LDS_BANK_CONFLICT", [10.0 if did == 7 else 30.0])]
            for name, vals in rows:
                for v in vals:
                    fh.write(f'{did},"{fwd}",{name},{v},1000,{1000 + int(ms * 1e6)}\n')
        fh.write('8,"k_relayout<true>(...)",SQ_INSTS_LDS,1e12,0,1\n')
    text = bench.summarize_counters(str(path))
    lines = {ln.split()[0]: dict(t.split("=", 1) for t in ln.split())
             for ln in text.splitlines() if ln.startswith("kernel=")}
    assert list(lines) == ["kernel=attn_fwd"]
    f = lines["kernel=attn_fwd"]
    assert f["dispatches"] == "2"
    assert float(f["avg_ms"]) == pytest.approx(ms)
    assert float(f["clock_ghz"]) == pytest.approx(1.8)
    assert float(f["mfma_flop"]) == pytest.approx(2e9 * 512, rel=1e-4)
    assert float(f["mfma_busy"]) == pytest.approx(0.5)
    assert float(f["tflops_at_clock_peak"]) == pytest.approx(1024 * 1024 * 1.8 / 1e3, rel=1e-3)
    assert float(f["lds_conflict"]) == pytest.approx(0.2)
    A = w.allowed_pairs()
    assert float(f["executed_flop"]) == pytest.approx(4 * w.head_dim * A * w.hq, rel=1e-4)


def test_traffic_summary_needs_a_copy(tmp_path):
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [(1, "k_attn_fwd<128>(x)", [1.0])])
    _counter_csv(write, "WRITE_SIZE", [(1, "k_attn_fwd<128>(x)", [1.0])])
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(fetch), str(write))


def test_load_traffic_checks_the_source_hash(tmp_path, monkeypatch):
    good = bench.sources_hash("attn_bwd_dkdv")
    path = tmp_path / "traffic.txt"
    path.write_text("# header\n"
                    f"kernel=attn_bwd_dkdv dispatches=3 fetch_kib=1 write_kib=1 traffic_bytes=12345 sources={good}\n"
                    "kernel=attn_fwd dispatches=3 fetch_kib=1 write_kib=1 traffic_bytes=999 sources=0000000000000000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.load_traffic("attn_bwd_dkdv") == 12345.0
    assert bench.load_traffic("attn_fwd") is None          # taken from other sources
    assert bench.load_traffic("attn_bwd_dq") is None       # absent
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.load_traffic("attn_bwd_dkdv") is None


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    import shutil
    pkg = os.path.join(bench.ROOT, "ulysses_sequence_parallelism_share_amd")
    copy = tmp_path / "ulysses_sequence_parallelism_share_amd"
    shutil.copytree(os.path.join(pkg, "csrc"), copy / "csrc")
    shutil.copy(os.path.join(pkg, "build.py"), copy / "build.py")
    names = ("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq")
    base = {n: bench.sources_hash(n) for n in names}
    assert len(set(base.values())) == 3 and all(len(h) == 16 for h in base.values())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert {n: bench.sources_hash(n) for n in names} == base
    # comments and layout: no change
    body = copy / "csrc" / "attn_bwd_dq.inc"
    body.write_text("// a comment\n" + body.read_text().replace(";", ";  /* x */"))
    assert {n: bench.sources_hash(n) for n in names} == base
    # code: the kernels built from that file change, the others do not
    body.write_text(body.read_text() + "\nint extra_symbol;\n")
    now = {n: bench.sources_hash(n) for n in names}
    assert now["attn_bwd_dq"] != base["attn_bwd_dq"]
    assert now["attn_bwd_dkdv"] == base["attn_bwd_dkdv"] and now["attn_fwd"] == base["attn_fwd"]


def test_trace_summary_table(tmp_path):
    p = tmp_path / "stats.csv"
    p.write_text("Name,Calls,TotalDurationNs,AverageNs,Percentage\n"
                 '"void k_attn_fwd<128>(...)",3,300000,100000,75.0\n'
                 '"k_loss_rank(...)",3,100000,33333.3,25.0\n')
    text = bench.summarize_trace(str(p)).splitlines()
    assert text[0].split() == ["kernel", "calls", "total_us", "avg_us", "pct"]
    assert text[1].split()[-4:] == ["3", "300.0", "100.0", "75.00%"]
    assert len(text) == 3


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
