"""bench.py's HBM-traffic bookkeeping on synthetic rocprofv3 output (no GPU).

The calibration factor must come from the copy kernel's own dispatches
only, although torch's other elementwise kernels (the fill that creates the
copy's source, for one) carry the same short name; every template instance
of one of the library's kernels is one kernel; and a record carries the
digest of the machine code the counter runs measured, so that a record
taken on other code is never reported.
"""
import csv
import json
import os

import pytest

import bench

GIB = 1 << 30
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, std::array<char*, 1ul> >(int, at::native::FillFunctor<float>, std::array<char*, 1ul>)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)::{lambda()#1}::operator()() const::{lambda()#8}::operator()() const::{lambda(float)#1}, std::array<char*, 2ul> >(int, at::native::neg_kernel_cuda(at::TensorIteratorBase&)::{lambda()#1}::operator()() const::{lambda()#8}::operator()() const::{lambda(float)#1}, std::array<char*, 2ul>)"
FWD0 = "void rlk::fwd_tiles<false, 0>(rlk::FwdArgs)"
FWD1 = "void rlk::fwd_tiles<false, 1>(rlk::FwdArgs)"


def write_run(d, counter, rows, digests):
    os.makedirs(os.path.join(d, counter.split("_")[0].lower()), exist_ok=True)
    sub = "fetch" if counter == "FETCH_SIZE" else "write"
    with open(os.path.join(d, sub, f"{sub}_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})
    with open(os.path.join(d, f"{sub}.log"), "w") as f:
        f.write("[bench] timing\n" + json.dumps({"metric": "m", "kernel_digests": digests}) + "\n")


@pytest.fixture
def run(tmp_path):
    d = str(tmp_path / "traffic")
    gib_kib = GIB / 1024
    # FETCH_SIZE: the fill reads nothing, the copy half its bytes; fwd_tiles
    # 3 GiB over two instances
    write_run(d, "FETCH_SIZE", [(FILL, 0.0), (NEG, 0.5 * gib_kib), (NEG, 0.5 * gib_kib),
                                (FWD0, 3.0 * gib_kib), (FWD1, 3.0 * gib_kib)], {"fwd_tiles": "abc"})
    write_run(d, "WRITE_SIZE", [(FILL, gib_kib), (NEG, gib_kib), (NEG, gib_kib),
                                (FWD0, 0.25 * gib_kib), (FWD1, 0.25 * gib_kib)], {"fwd_tiles": "abc"})
    return d


def test_calibration_uses_the_copy_dispatches_only(run, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "kernel_digest", lambda k: "abc")
    out = tmp_path / "out"
    out.mkdir()
    rows = bench.traffic_from(run, "cmd", out_dir=str(out))
    assert len(rows) == 1
    rec = json.loads((out / "traffic_fwd_tiles.json").read_text())
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == pytest.approx(6.0 * GIB) and rec["write_bytes"] == pytest.approx(0.25 * GIB)
    assert rec["dispatches"] == 2 and rec["kernel_digest"] == "abc" and rec["command"] == "cmd"


def test_record_keeps_the_measured_digest(run, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "kernel_digest", lambda k: "changed")
    out = tmp_path / "out"
    out.mkdir()
    bench.traffic_from(run, "cmd", out_dir=str(out))
    rec = json.loads((out / "traffic_fwd_tiles.json").read_text())
    assert rec["kernel_digest"] == "abc"


def test_traffic_for_needs_the_current_digest(monkeypatch, tmp_path):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_fwd_tiles.json").write_text(
        json.dumps({"kernel_digest": "abc", "bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "kernel_digest", lambda k: "abc")
    assert bench.traffic_for("fwd_tiles") == 123.0
    monkeypatch.setattr(bench, "kernel_digest", lambda k: "other")
    assert bench.traffic_for("fwd_tiles") is None
