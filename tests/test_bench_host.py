"""Host logic of bench.py that needs no GPU: the one-GPU refusal, the HBM
traffic summary of two counter runs, and the source-hash gate on stored
traffic figures."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_summary_scales_by_the_copy_and_is_gated_by_the_source_hash(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "PROFILES", str(tmp_path))
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    ours = "void qg::k_direct_gemm<2, 1, 1, 2, false>(qg::StreamArgs)"
    probe = "qg::k_read_probe(unsigned int __vector(4) const*, unsigned long, unsigned int*)"
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    copy_kib = b.COPY_ELEMS * 4 / 1024
    # the copy reads its 256 MiB but the counter shows half (factor 2), and
    # writes 256 MiB seen whole (factor 1); the read probe is not ours
    _counter_csv(str(tmp_path / "fetch"), [(ours, "FETCH_SIZE", 1000.0), (ours, "FETCH_SIZE", 1002.0),
                                           (probe, "FETCH_SIZE", 9e9), (neg, "FETCH_SIZE", copy_kib / 2)])
    _counter_csv(str(tmp_path / "write"), [(ours, "WRITE_SIZE", 10.0), (neg, "WRITE_SIZE", copy_kib)])
    b.pmc_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), "shape", "cmd-f", "cmd-w")
    d = json.load(open(tmp_path / "traffic.json"))["shape"]
    assert d["fetch_factor"] == pytest.approx(2.0)
    assert d["write_factor"] == pytest.approx(1.0)
    assert d["fetch_bytes"] == 1001 * 1024 * 2
    assert d["write_bytes"] == 10 * 1024
    assert list(d["fetch_kernels"]) == [ours]
    assert (d["fetch_command"], d["write_command"]) == ("cmd-f", "cmd-w")
    assert b.traffic_for("shape") == 1001 * 1024 * 2 + 10 * 1024
    assert b.traffic_for("another shape") is None
    # figures taken on other kernel sources are not reported
    allt = json.load(open(tmp_path / "traffic.json"))
    allt["shape"]["source_hash"] = "0" * 16
    json.dump(allt, open(tmp_path / "traffic.json", "w"))
    assert b.traffic_for("shape") is None


def test_traffic_summary_counts_every_dispatch_of_a_grouped_step(tmp_path, monkeypatch):
    """A MoE-layer step is three grouped calls, each one bucketing and one
    product dispatch: the traffic of a step is every dispatch's counter over
    the number of steps (bucketing dispatches / 3)."""
    b = _bench()
    monkeypatch.setattr(b, "PROFILES", str(tmp_path))
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    bucket = "qg::k_bucket(int const*, int, int, int, int*, float*, int, long, int)"
    grouped = "void qg::k_grouped<2, 2, true, 1, 0, 1, 3>(qg::StreamArgs, int const*, long, long, int, int, long, long, int)"
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    copy_kib = b.COPY_ELEMS * 4 / 1024
    # two steps: gate, up and down products of 100, 200 and 300 KiB, 1 KiB per bucketing
    rows = []
    for _ in range(2):
        for kib in (100.0, 200.0, 300.0):
            rows += [(bucket, "FETCH_SIZE", 1.0), (grouped, "FETCH_SIZE", kib)]
    _counter_csv(str(tmp_path / "fetch"), rows + [(neg, "FETCH_SIZE", copy_kib)])
    _counter_csv(str(tmp_path / "write"), [(bucket, "WRITE_SIZE", 0.0)] * 6 + [(grouped, "WRITE_SIZE", 2.0)] * 6 +
                 [(neg, "WRITE_SIZE", copy_kib)])
    b.pmc_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), "moe_layer", "", "")
    d = json.load(open(tmp_path / "traffic.json"))["moe_layer"]
    assert d["calls_per_step"] == 3
    assert d["fetch_bytes"] == (600 + 3) * 1024
    assert d["write_bytes"] == 6 * 1024


def test_traffic_summary_without_the_copy_is_an_error(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "PROFILES", str(tmp_path))
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    ours = "void qg::k_direct_gemm<2, 1, 1, 2, false>(qg::StreamArgs)"
    _counter_csv(str(tmp_path / "fetch"), [(ours, "FETCH_SIZE", 1000.0)])
    _counter_csv(str(tmp_path / "write"), [(ours, "WRITE_SIZE", 10.0)])
    with pytest.raises(SystemExit):
        b.pmc_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), "shape", "", "")
    assert not (tmp_path / "traffic.json").exists()
