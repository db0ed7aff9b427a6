"""Host-side logic of bench.py: the one-GPU guard, the algorithmic byte count
behind the metric and the reading of the committed HBM-byte summary (no GPU)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _golden():
    vals = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "roofline_bytes.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            key, val = line.split()
            vals[key] = int(val)
    return vals


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_metric_bytes_match_the_roofline_section():
    # weights (144 B per 256 weights) + fp16 x + fp32 y of the metric's shape
    g = _golden()
    fmt, n, k, _ = bench.MAIN
    assert (fmt, n, k) == ("q4k", 4096, 14336)
    want = g["q4k_weight_bytes_4096x14336"] + g["q4k_x_bytes_14336"] + g["q4k_y_bytes_4096"]
    assert bench.algorithmic_bytes(fmt, n, k) == want == 33075200


def test_traffic_only_from_a_summary_of_the_same_build(tmp_path, monkeypatch):
    p = tmp_path / "summary.md"
    p.write_text("# HBM bytes\n\ntraffic_bytes_per_launch: 33417529\ntraffic_build_id: abc123\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(p))
    assert bench.measured_traffic("abc123") == 33417529
    assert bench.measured_traffic("def456") is None
    p.write_text("traffic_build_id: abc123\n")
    assert bench.measured_traffic("abc123") is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("abc123") is None


def test_committed_summary_is_parseable():
    fields = dict(line.split(":", 1) for line in open(bench.TRAFFIC_SUMMARY) if ":" in line)
    bid = fields["traffic_build_id"].strip()
    assert bench.measured_traffic(bid) == int(fields["traffic_bytes_per_launch"])


def test_timed_graph_copies_exceed_the_infinity_cache():
    # every run of up to 16 consecutive launches reads distinct copies; with
    # the 33 MB metric shape that is >= 529 MB, above the 256 MB cache
    assert bench.copies_for(1) == 16 and bench.copies_for(20) == 20 and bench.copies_for(3200) == 32
    per = bench.algorithmic_bytes(*bench.MAIN[:3])
    assert bench.copies_for(20) * per > 2 * 256e6


def test_valu_fields_only_from_a_summary_of_the_same_build(tmp_path, monkeypatch):
    p = tmp_path / "valu.md"
    p.write_text("valu_build_id: abc\nvalu q4k_4096x14336: insts_per_wave=1200 busy_cycles_per_simd=9600\n")
    monkeypatch.setattr(bench, "VALU_SUMMARY", str(p))
    v = bench.valu_estimates("abc")
    f = bench.valu_fields(v, "q4k", 4096, 14336, 8.0)
    # 9600 SIMD-cycles of VALU issue in an 8 us launch at 2.4 GHz = 50%
    assert f == {"valu_insts_per_wave": 1200.0, "est_valu_issue_pct": 50.0}
    assert bench.valu_fields(bench.valu_estimates("other"), "q4k", 4096, 14336, 8.0) == {}
    assert bench.valu_fields(v, "tq1", 14336, 4096, 8.0) == {}


def _counter_csv(path, rows):
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(f'"{c}"' for c in cols) + "\n")
        for did, name, counter, val in rows:
            f.write(f'{did},{did},"Agent 1",1,1,1,1024,1,"{name}",256,0,0,8,0,32,"{counter}",{val},0,1\n')


def test_counter_summary_scales_by_the_copy_and_orders_kernels(tmp_path):
    # two passes of a run over two shapes: FETCH_SIZE reads half of a copy's
    # bytes (scale 2), WRITE_SIZE all of them; kernels in first-dispatch order
    copy = "__amd_rocclr_copyBuffer"
    ka, kb = "void qgemv::q4k_gemv_rows_kernel<7, 2, 8, qgemv::OutF32>(x)", "void qgemv::tq1_gemv_rows_kernel<1>(x)"
    fetch = [(i, copy, "FETCH_SIZE", 32768.0) for i in range(1, 9)]
    fetch += [(20, kb, "FETCH_SIZE", 999.0), (10, ka, "FETCH_SIZE", 16000.0), (11, ka, "FETCH_SIZE", 16400.0),
              (12, ka, "FETCH_SIZE", 16100.0), (13, "void qgemv::read_ceiling_kernel(x)", "FETCH_SIZE", 5.0)]
    write = [(i, copy, "WRITE_SIZE", 65536.0) for i in range(1, 9)]
    write += [(10, ka, "WRITE_SIZE", 16.0), (20, kb, "WRITE_SIZE", 56.0)]
    valu = [(10, ka, "SQ_INSTS_VALU", 2048 * 1200.0), (10, ka, "SQ_WAVES", 2048.0),
            (10, ka, "SQ_ACTIVE_INST_VALU", 2048 * 1200.0), (10, ka, "GRBM_GUI_ACTIVE", 17280.0)]
    _counter_csv(tmp_path / "f" / "h" / "r_counter_collection.csv", fetch)
    _counter_csv(tmp_path / "w" / "h" / "r_counter_collection.csv", write + valu)
    shapes = [("q4k", 4096, 14336, ""), ("tq1", 14336, 4096, "")]
    out = bench.counter_summary([str(tmp_path / "f"), str(tmp_path / "w")], shapes, "bid")
    assert out[0] == "valu_build_id: bid"
    t = [ln for ln in out if ln.startswith("traffic q4k_4096x14336:")]
    assert t == [f"traffic q4k_4096x14336: bytes_per_launch={1024 * (2 * 16100 + 16)} algorithmic=33075200 "
                 f"ratio={1024 * (2 * 16100 + 16) / 33075200:.4f}"]
    assert any(ln.startswith("traffic tq1_14336x4096: bytes_per_launch=" + str(1024 * (2 * 999 + 56))) for ln in out)
    v = [ln for ln in out if ln.startswith("valu q4k_4096x14336:")]
    assert v == ["valu q4k_4096x14336: insts_per_wave=1200.0 busy_cycles_per_simd=9600"]
    # and bench.py reads its own valu lines back
    p = tmp_path / "valu.md"
    p.write_text("\n".join(out) + "\n")
    old = bench.VALU_SUMMARY
    try:
        bench.VALU_SUMMARY = str(p)
        est = bench.valu_estimates("bid")
    finally:
        bench.VALU_SUMMARY = old
    assert est["q4k_4096x14336"]["busy_cycles_per_simd"] == 9600
    f = bench.valu_fields(est, "q4k", 4096, 14336, 8.0)
    assert f == {"valu_insts_per_wave": 1200.0, "est_valu_issue_pct": 50.0}
