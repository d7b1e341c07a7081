"""Host logic of bench.py's counter summaries (no GPU): which dispatches count
as the measured steps, the per-step sums and the copy-kernel scaling."""
import csv
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write(folder, counter, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for d, name, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Grid_Size": 256, "Counter_Name": counter,
                        "Counter_Value": v})


def _kv(text):
    out = {}
    for line in text.splitlines():
        if ":" in line and not line.startswith("kernel:"):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def test_traffic_summary_counts_the_steps_only(tmp_path):
    # setup dispatches (inputs, and a library launch while the inputs are
    # made) come before the last non-library dispatch and are left out; the
    # steps' two kernels are summed per step
    a, b = "void qg::k_gate(qg::GemvArgs)", "void qg::k_down(qg::Moe1Args)"
    setup = [(1, "elementwise_kernel", 5.0), (2, a, 999.0), (3, "copyBuffer", 7.0)]
    steps = [(4 + 2 * i, a, 100.0) for i in range(3)] + [(5 + 2 * i, b, 50.0) for i in range(3)]
    _write(str(tmp_path / "f"), "FETCH_SIZE", setup + steps)
    _write(str(tmp_path / "w"), "WRITE_SIZE", [(d, n, v / 10.0) for d, n, v in setup + steps])
    # the copy probe: 1 MiB copied, FETCH reads half of it, WRITE all of it
    _write(str(tmp_path / "cf"), "FETCH_SIZE", [(1, "copyBuffer", 512.0), (2, "copyBuffer", 512.0)])
    _write(str(tmp_path / "cw"), "WRITE_SIZE", [(1, "copyBuffer", 1024.0)])
    text = bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                                 str(tmp_path / "cw"), 1, "moe_test", 300 * 1024, 3)
    kv = _kv(text)
    assert float(kv["fetch_kib_per_step"]) == 150.0
    assert float(kv["write_kib_per_step"]) == 15.0
    # fetch scaled by 2 (the copy's reads read half), write by 1
    assert int(kv["traffic_bytes_per_launch"]) == (150 * 2 + 15) * 1024
    assert abs(float(kv["traffic_over_algorithmic"]) - 315 / 300) < 1e-4
    assert kv["source_sha256"] == bench.source_hash()
    assert "k_gate" in text and "k_down" in text and "999" not in text


def test_load_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    # a summary taken on other kernels than the built ones reads as unmeasured
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    body = "traffic_bytes_per_launch: 12345\nsource_sha256: %s\n"
    (tmp_path / "traffic_k.txt").write_text(body % bench.source_hash())
    assert bench.load_traffic("k") == 12345
    (tmp_path / "traffic_k.txt").write_text(body % ("0" * 64))
    assert bench.load_traffic("k") is None
    assert bench.load_traffic("absent") is None
