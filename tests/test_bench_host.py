"""Host-side checks of the benchmark's bookkeeping (no GPU): algorithmic work of the
dense and grouped calls, roofline classification, and the rocprofv3 csv summaries
(kernel trace, counters) on small synthetic files."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_dense_work_counts_each_operand_once():
    flops, nbytes = bench.algo_work(64, 2112, 7168)
    assert flops == 2.0 * 64 * 2112 * 7168
    kb = 7168 // 128
    assert nbytes == 64 * 7168 + 2112 * 7168 + 64 * 2112 * 2 + 64 * kb * 4 + 17 * kb * 4


def test_grouped_work_live_rows_and_active_groups():
    # 3 active groups, 500 live rows, 640 padded rows
    flops, nbytes, padded = bench.grouped_work(500, 3, 256, 384, m_padded=640)
    assert flops == 2.0 * 500 * 256 * 384 and padded == 2.0 * 640 * 256 * 384
    assert nbytes == 500 * 384 + 3 * 256 * 384 + 500 * 256 * 2 + 500 * 3 * 4 + 3 * 2 * 3 * 4
    f2, b2, p2 = bench.grouped_work(500, 3, 256, 384)
    assert p2 == f2


def test_roofline_classification():
    # the dominant dense shape is matrix-bound, a few-row shape memory-bound
    assert bench.classify(*bench.algo_work(4096, 7168, 16384))[0] == "mfma"
    assert bench.classify(*bench.algo_work(64, 7168, 16384))[0] == "hbm"
    assert bench.classify(*bench.algo_work(4096, 32768, 512))[0] == "hbm"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summaries(tmp_path, capsys):
    shapes = [(64, 256, 512), (128, 512, 1024)]
    rows, d = [], 0
    for rep in range(3):
        for i in range(2):
            d += 1
            rows.append([d, "void fp8gemm::fp8_gemm_kernel<64, 64, 2, 2, 8, false>(fp8gemm::Params)", 1000, 1000 + 1000 * (i + 1)])
            d += 1
            rows.append([d, "void at::native::other_kernel()", 0, 99999])
    _write_csv(str(tmp_path / "t" / "run_kernel_trace.csv"), ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    bench.trace_summary(str(tmp_path / "t"), shapes, steps=1, warmup=0)
    out = [json.loads(l) for l in capsys.readouterr().out.splitlines()]
    assert [o["avg_us"] for o in out] == [1.0, 2.0] and all(o["dispatches"] == 3 for o in out)
    with pytest.raises(SystemExit):  # 6 dispatches cannot come from a run of --steps 2
        bench.trace_summary(str(tmp_path / "t"), shapes, steps=2, warmup=0)

    # grouped: the first GEMM dispatch (the untimed gate+up call) is dropped
    n = len(bench.GROUPED_CASES)
    rows = [[1, "void fp8gemm::fp8_gemm_kernel<128, 256, 2, 4, 3, false>(fp8gemm::Params)", 0, 10 ** 9]]
    for rep in range(2):
        for i in range(n):
            rows.append([2 + rep * n + i, "void fp8gemm::fp8_gemm_kernel<128, 128, 2, 2, 4, true>(fp8gemm::Params)", 0, 1000 * (i + 1)])
    _write_csv(str(tmp_path / "g" / "run_kernel_trace.csv"), ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    bench.trace_summary_grouped(str(tmp_path / "g"), steps=1)
    out = [json.loads(l) for l in capsys.readouterr().out.splitlines()]
    assert len(out) == n and [o["avg_us"] for o in out] == [float(i + 1) for i in range(n)]
    assert [o["timed_avg_us"] for o in out] == [float(i + 1) for i in range(n)]


def test_default_run_dispatch_layout(tmp_path, capsys):
    """A default run's trace: dense shapes step by step, the small case (one checking call,
    then its timed calls), the untimed gate+up call, the grouped cases step by step; the
    event-timed mean covers each case's last `steps` dispatches."""
    shapes = [(64, 256, 512), (128, 512, 1024)]
    steps, warmup = 2, 1
    per = warmup + 2 * steps + 1
    n = len(bench.GROUPED_CASES)
    gemm = "void fp8gemm::fp8_gemm_kernel<64, 64, 2, 2, 8, false>(fp8gemm::Params)"
    rows, d = [], 0

    def add(us):
        nonlocal d
        d += 1
        rows.append([d, gemm, 0, int(us * 1000)])
        d += 1
        rows.append([d, "void at::native::other_kernel()", 0, 99999])

    for rep in range(per):
        for i in range(len(shapes)):
            add(10 * (i + 1) + (5 if rep >= per - steps else 0))
    add(1000)  # the small case's checking call
    for _ in range(bench.N_SMALL * bench.SMALL_REPS):
        add(3)
    add(2000)  # gate+up producing the down GEMM's input
    for rep in range(per):
        for i in range(n):
            add(100 + i)
    _write_csv(str(tmp_path / "t" / "run_kernel_trace.csv"), ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    bench.trace_summary(str(tmp_path / "t"), shapes, steps, warmup)
    out = [json.loads(l) for l in capsys.readouterr().out.splitlines()]
    assert len(out) == len(shapes) + 1 + n
    assert [o["timed_avg_us"] for o in out[:2]] == [15.0, 25.0]
    assert out[0]["avg_us"] == round((10 * per + 5 * steps) / per, 2)
    assert out[2]["avg_us"] == 3.0 and out[2]["dispatches"] == bench.N_SMALL * bench.SMALL_REPS
    assert [o["avg_us"] for o in out[3:]] == [100.0 + i for i in range(n)]
    assert [o["case"] for o in out[3:]] == bench.GROUPED_CASES


def test_packed_scale_bytes():
    f4, b4 = bench.algo_work(64, 2112, 7168)
    f1, b1 = bench.algo_work(64, 2112, 7168, scale_bytes=1.0)
    kb = 7168 // 128
    assert f1 == f4 and b4 - b1 == 3 * (64 * kb + 17 * kb)


def test_counter_summary(tmp_path, capsys):
    shapes = [(64, 256, 512), (128, 512, 1024)]
    rows = []
    for d in range(1, 7):
        rows.append([d, "void fp8gemm::fp8_gemm_kernel<64, 64, 2, 2, 8, false>(fp8gemm::Params)", "GRBM_GUI_ACTIVE", 10 * d])
        rows.append([d, "void fp8gemm::fp8_gemm_kernel<64, 64, 2, 2, 8, false>(fp8gemm::Params)", "SQ_INSTS_LDS", d])
        rows.append([d, "void fp8gemm::fp8_gemm_kernel<64, 64, 2, 2, 8, false>(fp8gemm::Params)", "SQ_INSTS_LDS", d])
    _write_csv(str(tmp_path / "c" / "run_counter_collection.csv"), ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    bench.counter_summary(str(tmp_path / "c"), shapes, steps=1, warmup=0)
    out = [json.loads(l) for l in capsys.readouterr().out.splitlines()]
    # dispatches 1, 3, 5 -> shape 0; 2, 4, 6 -> shape 1; instances of a counter are summed per dispatch
    assert out[0]["GRBM_GUI_ACTIVE"] == 30.0 and out[1]["GRBM_GUI_ACTIVE"] == 40.0
    assert out[0]["SQ_INSTS_LDS"] == 6.0 and out[1]["SQ_INSTS_LDS"] == 8.0


def test_multi_gpu_request_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stdout
