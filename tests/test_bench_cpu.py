"""Host logic of bench.py that runs without a GPU: the traffic-counter summaries (synthetic
counter files in rocprofv3's CSV shape), the recorded-traffic lookup tied to the source digest,
and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows, 1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def _copies(kib):
    return [("__amd_rocclr_copyBuffer", kib)] * 3


@pytest.fixture
def traffic_file(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    return path


def test_q8_0_summary_groups_dispatches_in_order(tmp_path, traffic_file):
    """Per matrix, per column count, one launch per weight copy: distinct per-count values come
    back under the right keys, scaled by the copy calibration."""
    rows_f, rows_w = _copies(32768.0), _copies(65536.0)
    expect = {}
    for nrows, k, cols, _ in bench.Q8_PROBE_SPECS:
        nc = bench.cold_copies(nrows * synth.row_bytes(synth.Q8_0, k))
        for n in cols:
            nc_pass = 1 << (n - 1).bit_length()
            name = (f"void qmm::gemv_f32_kernel<1, 5, {n}, 512>(x)" if n in bench.fused_cols_of(k, cols) else
                    f"void qmm::gemv_kernel<1, false, {nc_pass}, 5, false, 1, 16, 256>(x)")
            rows_f += [(name, 1000.0 * n + nrows)] * nc
            rows_w += [(name, 10.0 * n)] * nc
            expect[(nrows, k, n)] = round(((1000.0 * n + nrows) * 2.0 + 10.0 * n) * 1024)
    _write(tmp_path / "f.csv", "FETCH_SIZE", rows_f)
    _write(tmp_path / "w.csv", "WRITE_SIZE", rows_w)
    bench.pmc_summary("q8_0", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = json.load(open(traffic_file))
    for (nrows, k, n), b in expect.items():
        r = rec[f"gemv:{synth.Q8_0}:{nrows}x{k}"]
        assert r["bytes_per_launch"][str(n)] == b
        assert r["source_sha256"] == bench.source_digest(r["sources"])
        assert r["fused_columns"] == sorted(bench.fused_cols_of(k, [n for nn, kk, cols, _ in bench.Q8_PROBE_SPECS
                                                                    if (nn, kk) == (nrows, k) for n in cols]))


def test_gemv_summary_and_lookup(tmp_path, traffic_file):
    """The headline GEMV summary keys launches by pass width (fused one-column kernel included);
    the lookup returns the record only while the sources hash the same."""
    rows_f, rows_w = _copies(32768.0), _copies(65536.0)
    for n in bench.PROBE_COLS:   # the fused kernel where the step fuses, the q8_1 GEMV elsewhere
        name = (f"void qmm::gemv_f32_kernel<2, 5, {n}, 512>(x)" if n in bench.FUSED_COLS else
                f"void qmm::gemv_kernel<2, false, {n}, 5, false, 1, 16, 256>(x)")
        rows_f += [(name, 5800.0 + n)] * 4
        rows_w += [(name, 32.0 * n)] * 4
    _write(tmp_path / "f.csv", "FETCH_SIZE", rows_f)
    _write(tmp_path / "w.csv", "WRITE_SIZE", rows_w)
    bench.pmc_summary("gemv", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    key = f"gemv:{synth.IQ4_NL}:8192x2560"
    rec = bench.recorded_traffic(key)
    assert rec is not None
    for n in bench.PROBE_COLS:
        assert rec["bytes_per_launch"][str(n)] == round(((5800.0 + n) * 2.0 + 32.0 * n) * 1024)
    data = json.load(open(traffic_file))
    data[key]["source_sha256"] = "0" * 64
    json.dump(data, open(traffic_file, "w"))
    assert bench.recorded_traffic(key) is None


def test_mmq_summary_sums_each_call(tmp_path, traffic_file):
    """The MMQ-style prefill's launches group into calls ending at the down kernel; the first
    call (cold) is left out of the mean, and each kernel's own bytes are kept beside it."""
    rows_f, rows_w = _copies(32768.0), _copies(65536.0)
    kernels = ("qmm::quantize_planes_kernel(x)", "qmm::schedule_kernel(x)", "qmm::mq_gateup_kernel(MqGuArgs)",
               "qmm::mq_down_kernel(MqDownArgs)")
    for call, scale in ((0, 3.0), (1, 1.0)):
        for j, name in enumerate(kernels):
            rows_f.append((name, scale * 100.0 * (j + 1)))
            rows_w.append((name, 10.0 * (j + 1)))
    _write(tmp_path / "f.csv", "FETCH_SIZE", rows_f)
    _write(tmp_path / "w.csv", "WRITE_SIZE", rows_w)
    bench.pmc_summary("mmq", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = bench.recorded_traffic("mmq")
    assert rec["bytes_per_launch"]["call"] == round((1000.0 * 2.0 + 100.0) * 1024)
    assert rec["mq_down_kernel_bytes"] == round(((1200.0 + 400.0) / 2 * 2.0 + 40.0) * 1024)


def test_dense_and_combine_summaries(tmp_path, traffic_file):
    """Dense projections: two launches per matrix in the probe's order, each matrix under its
    own name; the combine: the mean of its launches."""
    rows_f, rows_w = _copies(32768.0), _copies(65536.0)
    for j in range(4):
        rows_f.append(("qmm::dense_kernel(DenseArgs)", 1000.0 * (j // 2 + 1)))
        rows_w.append(("qmm::dense_kernel(DenseArgs)", 5.0))
    _write(tmp_path / "f.csv", "FETCH_SIZE", rows_f)
    _write(tmp_path / "w.csv", "WRITE_SIZE", rows_w)
    bench.pmc_summary("dense", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = bench.recorded_traffic("dense")
    names = [bench.dense_name(wt, nrows, 2560) for wt, nrows, _ in bench.dense_specs()]
    assert [rec["bytes_per_launch"][n] for n in names] == [round((2000.0 + 5.0) * 1024),
                                                           round((4000.0 + 5.0) * 1024)]
    rows_f, rows_w = _copies(32768.0), _copies(65536.0)
    rows_f += [("void qmm::combine_kernel<3>(x)", v) for v in (300.0, 330.0, 360.0)]
    rows_w += [("void qmm::combine_kernel<3>(x)", 80.0)] * 3
    _write(tmp_path / "f.csv", "FETCH_SIZE", rows_f)
    _write(tmp_path / "w.csv", "WRITE_SIZE", rows_w)
    bench.pmc_summary("combine", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = bench.recorded_traffic("combine")
    assert rec["bytes_per_launch"][bench.COMBINE_SHAPES[0][0]] == round((660.0 + 80.0) * 1024)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
