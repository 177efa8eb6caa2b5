"""Host logic of bench.py's counter summaries, on small synthetic
rocprofv3 counter files with values worked out by hand (no GPU)."""
import csv
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow({**{k: 0 for k in FIELDS}, **r})


def _row(disp, name, counter, value, start=0, end=1):
    return {"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value,
            "Start_Timestamp": start, "End_Timestamp": end}


def test_summarize_clock(bench, tmp_path, capsys):
    gemm = "void ragged_gemm_kernel<moe::core::Tile<192, 256, 2, 4, 64, 2, 3>, 1>(moe::RaggedGemm)"
    rows = []
    # two 1 ms dispatches: 8 XCDs x 1.8e6 GUI-active cycles -> 1.8 GHz; the
    # busy counter split over two records of one dispatch (summed)
    for d in (1, 2):
        rows += [_row(d, gemm, "GRBM_GUI_ACTIVE", 8 * 1.8e6, 0, 1_000_000),
                 _row(d, gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1.8e6 * 1024, 0, 1_000_000),
                 _row(d, gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1.8e6 * 1024, 0, 1_000_000)]
    # a short kernel and torch's own kernel are left out
    rows += [_row(3, "topk_gates_kernel", "GRBM_GUI_ACTIVE", 8e6, 0, 10_000),
             _row(3, "topk_gates_kernel", "SQ_VALU_MFMA_BUSY_CYCLES", 0, 0, 10_000),
             _row(4, "void at::native::fill", "GRBM_GUI_ACTIVE", 8e9, 0, 1_000_000),
             _row(4, "void at::native::fill", "SQ_VALU_MFMA_BUSY_CYCLES", 0, 0, 1_000_000)]
    p = tmp_path / "c.csv"
    _write(p, rows)
    bench.summarize_clock(str(p), xcds=8, simds=1024, min_us=400.0)
    out = capsys.readouterr().out.strip().split("\n")
    assert len(out) == 3, out  # header, rule, one kernel
    cells = [c.strip() for c in out[2].strip("|").split("|")]
    assert cells[1] == "2" and cells[2] == "1000.0" and cells[3] == "1.80" and cells[4] == "0.500"
    assert cells[5] == str(round(2500 * 1.8 / 2.4))


def test_summarize_pmc(bench, tmp_path, capsys):
    gemm = "void ragged_gemm_kernel<moe::core::Tile<192, 256, 2, 4, 64, 2, 3>, 1>(moe::RaggedGemm)"
    copy = "__amd_rocclr_copyBuffer"
    mib = 1024 * 1024
    # the 1 GiB calibration copy reads back half its bytes on FETCH_SIZE
    # (scale 2) and all of them on WRITE_SIZE (scale 1); a small copy is not
    # the calibration one
    f = [_row(1, copy, "FETCH_SIZE", 512 * 1024), _row(2, copy, "FETCH_SIZE", 4),
         _row(3, gemm, "FETCH_SIZE", 1000.0), _row(4, gemm, "FETCH_SIZE", 3000.0)]
    w = [_row(1, copy, "WRITE_SIZE", 1024 * 1024), _row(2, copy, "WRITE_SIZE", 8),
         _row(3, gemm, "WRITE_SIZE", 100.0), _row(4, gemm, "WRITE_SIZE", 300.0)]
    fp, wp, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "traffic.json"
    _write(fp, f)
    _write(wp, w)
    bench.summarize_pmc(str(fp), str(wp), "expert_gate_up", "marin_16k", 1024 * mib, str(out), "cmd")
    rec = json.load(open(out))
    assert rec["dispatches"] == [2, 2]
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    # mean 2000 KiB fetched x 2 + mean 200 KiB written x 1
    assert rec["bytes_per_launch"] == pytest.approx((2000 * 2 + 200) * 1024.0)
    assert rec["source_sha256"] == bench.kernel_source_hash("marin_16k")


def test_source_hash_ignores_comments_only(bench, tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text('// header\nint f(int x) { return x + 1; }  /* trailing */\nconst char* s = "// kept";\n')
    b.write_text('/* another header */\nint f(int x) {\n  return x + 1;  // same code\n}\nconst char* s = "// kept";\n')
    c.write_text('// header\nint f(int x) { return x + 2; }\nconst char* s = "// kept";\n')
    assert bench.source_hash([a]) == bench.source_hash([b])
    assert bench.source_hash([a]) != bench.source_hash([c])
    # a comment marker inside a string literal is code
    d = tmp_path / "d.hip"
    d.write_text('// header\nint f(int x) { return x + 1; }\nconst char* s = "// changed";\n')
    assert bench.source_hash([a]) != bench.source_hash([d])
