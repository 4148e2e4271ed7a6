"""bench.py's host-side logic, on the CPU: the summaries of rocprofv3 output
that the committed profiles/ files are made with, the matrix-core and HBM
figures read back from them (and dropped when the kernel sources changed),
and the one-GPU contract of the command line.  Synthetic CSV files in
rocprofv3's column layout, with known answers."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

DECODE = ("void gdn::(anonymous namespace)::decode_kernel<2, 2, 128, 16, 2, 16>"
          "(gdn::(anonymous namespace)::StepArgs)")
ROWS = ("void gdn::(anonymous namespace)::rows_la_kernel<2, 2, 128>"
        "(gdn::(anonymous namespace)::StateArgs)")


def test_short_kernel_names():
    assert bench._short_kernel(DECODE) == "decode_kernel<2, 2, 128, 16, 2, 16>"
    assert bench._short_kernel(ROWS) == "rows_la_kernel<2, 2, 128>"
    assert bench._short_kernel("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    assert bench._short_kernel(
        "void gdn::(anonymous namespace)::stream_kernel<256, 4, true, false>(float4 const*, "
        "float4*, long)") == "stream_kernel<256, 4, true, false>"


def _trace(path, rows):
    cols = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
            "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for i, (name, t0, ns, grid) in enumerate(rows):
            w.writerow(["KERNEL_DISPATCH", i + 1, name, t0, t0 + ns, grid, 1, 1])


def test_trace_summary_splits_by_grid(tmp_path, capsys):
    """Rows per (kernel, grid): the same kernel at two batch sizes stays apart,
    durations from the stamps in ns, shares of the total time."""
    p = str(tmp_path / "t.csv")
    _trace(p, [(DECODE, 0, 45000, 2097152), (DECODE, 10 ** 6, 47000, 2097152),
               (DECODE, 2 * 10 ** 6, 4000, 32768), (ROWS, 3 * 10 ** 6, 104000, 131072)])
    bench.trace_summary(p)
    out = capsys.readouterr().out.splitlines()
    rows = {tuple(c.strip() for c in l.strip("|").split("|")[:2]): l for l in out[2:]}
    big = rows[("decode_kernel<2, 2, 128, 16, 2, 16>", "2097152")]
    assert "| 2 | 46.00 | 46.00 | 45.00 | 47.00 | 46.0% |" in big
    assert "| 1 | 4.00 | 4.00 | 4.00 | 4.00 | 2.0% |" in rows[
        ("decode_kernel<2, 2, 128, 16, 2, 16>", "32768")]
    assert "| 1 | 104.00 |" in rows[("rows_la_kernel<2, 2, 128>", "131072")]
    assert out[2].startswith("| rows_la_kernel")  # largest share first


def _counters(path, rows):
    cols = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name",
            "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for r in rows:
            w.writerow(r)


def test_counter_summary_sums_over_xcds_then_averages(tmp_path, capsys):
    """A dispatch's rows (one per XCD) add up; dispatches then average."""
    p = str(tmp_path / "c.csv")
    rows = []
    for d, per_xcd in ((1, 100.0), (2, 300.0)):
        for x in range(8):
            rows.append([d, d, 2097152, DECODE, "FETCH_SIZE", per_xcd])
    rows.append([3, 3, 512, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 7.0])
    _counters(p, rows)
    bench.counter_summary([p])
    out = capsys.readouterr().out
    assert "decode_kernel<2, 2, 128, 16, 2, 16> grid 2097152:" in out
    assert "FETCH_SIZE 1600 per dispatch (2 dispatches)" in out  # (800 + 2400) / 2
    assert "FETCH_SIZE 7 per dispatch (1 dispatches)" in out


def test_matrix_lines_flops_and_busy(tmp_path, capsys):
    """512 flops per MOPS; busy = MFMA-busy cycles over 1024 SIMDs times the
    GUI-active cycles of one XCD (the counter sums the 8)."""
    p = str(tmp_path / "m.csv")
    vals = {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 1000.0, "SQ_INSTS_VALU_MFMA_MOPS_F16": 0.0,
            "SQ_INSTS_VALU_MFMA_MOPS_F32": 10.0, "SQ_VALU_MFMA_BUSY_CYCLES": 256000.0,
            "GRBM_GUI_ACTIVE": 8000.0}
    _counters(p, [[1, 1, 131072, ROWS, c, v] for c, v in vals.items()])
    bench.matrix_lines([p])
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if l.startswith("matrix.rows_la_kernel")][0]
    assert "bf16_flop=512000 " in line and "f32_flop=5120 " in line
    assert line.endswith("busy=0.2500")  # 256000 / (1024 * 8000 / 8)
    assert out.splitlines()[0] == "scan_source_sha256: %s" % bench.kernel_source_hash(bench.SCAN_SRC)


def test_profile_figures_need_the_current_sources(tmp_path, monkeypatch):
    """The HBM bytes and matrix-core figures come from profiles/ only while the
    summary's source hash matches the kernels being timed."""
    good = bench.kernel_source_hash()
    f = tmp_path / "dec.txt"
    f.write_text("kernel_source_sha256: %s\nhbm_bytes_per_launch: 271697871\n" % good)
    monkeypatch.setattr(bench, "DECODE_COUNTERS", str(f))
    assert bench.read_counters() == 271697871.0
    f.write_text("kernel_source_sha256: 0000000000000000\nhbm_bytes_per_launch: 271697871\n")
    assert bench.read_counters() is None
    monkeypatch.setattr(bench, "DECODE_COUNTERS", str(tmp_path / "missing.txt"))
    assert bench.read_counters() is None

    s = tmp_path / "scan.txt"
    lines = ["scan_source_sha256: %s" % bench.kernel_source_hash(bench.SCAN_SRC)]
    for i, k in enumerate(bench.SCAN_KERNELS[3]):
        lines.append("matrix.%s: bf16_flop=%g f16_flop=0 f32_flop=0 busy=%.4f" % (
            k, 1e9 * (i + 1), 0.5 if i == 0 else 0.1))
    s.write_text("\n".join(lines) + "\n")
    monkeypatch.setattr(bench, "SCAN_COUNTERS", str(s))
    m = bench.scan_matrix_figures(3, 1.0)  # 1 ms per call
    n = len(bench.SCAN_KERNELS[3])
    assert m["main_kernel"] == bench.SCAN_KERNELS[3][0] and m["main_kernel_matrix_busy"] == 0.5
    assert m["bf16_f16_tflops_issued"] == round(1e9 * n * (n + 1) / 2 / 1e-3 / 1e12, 1)
    s.write_text(s.read_text().replace(lines[0], "scan_source_sha256: 0000000000000000"))
    assert bench.scan_matrix_figures(3, 1.0) is None


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, **env))
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
