"""Host logic of bench.py: the one-GPU guard, the traffic record's source digest and the
counter summary's copy calibration.  No GPU is touched."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def _fake_tree(tmp_path, phase):
    csrc = tmp_path / "structured_sparse_attention_plan_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES[phase] + bench.COMMON_SOURCES:
        (csrc / f).write_text(f"// {f}\n")
    (tmp_path / "profiles").mkdir()
    return csrc


def test_traffic_record_needs_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = _fake_tree(tmp_path, "fwd")
    assert bench.traffic_from_profile("fwd") is None          # no record
    rec = tmp_path / "profiles" / "traffic_fwd_128k.txt"
    rec.write_text(f"kernel: x\nsource_digest: {bench.source_digest('fwd')}\n"
                   "hbm_bytes_per_launch: 1.234e+09\n")
    assert bench.traffic_from_profile("fwd") == pytest.approx(1.234e9)
    src = csrc / bench.KERNEL_SOURCES["fwd"][0]
    src.write_text(src.read_text() + "// edited\n")            # kernel changed since
    assert bench.traffic_from_profile("fwd") is None


def _write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                           "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_pmc_summary_scales_by_the_copy_probe(tmp_path):
    sym = bench.KERNEL_SYMBOL["fwd"]
    kib = bench.COPY_PROBE_BYTES / 1024

    def kernel_rows(counter, per_dispatch):
        # two dispatches, each value split over two rows (counter instances)
        return [dict(Dispatch_Id=d, Kernel_Name=f"cowa::{sym}(cowa::FwdArgs)", Grid_Size=256,
                     Counter_Name=counter, Counter_Value=per_dispatch / 2)
                for d in (7, 9) for _ in range(2)]

    def copy_rows(counter, big_kib):
        return [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Grid_Size=1 << 20,
                     Counter_Name=counter, Counter_Value=big_kib),
                dict(Dispatch_Id=2, Kernel_Name="__amd_rocclr_copyBuffer", Grid_Size=64,
                     Counter_Name=counter, Counter_Value=3.0),     # small read-back, ignored
                dict(Dispatch_Id=3, Kernel_Name="elementwise_kernel_manual_unroll", Grid_Size=4096,
                     Counter_Name=counter, Counter_Value=big_kib)]

    f, w, cf, cw = (str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    _write_csv(f, kernel_rows("FETCH_SIZE", 1000.0))
    _write_csv(w, kernel_rows("WRITE_SIZE", 300.0))
    _write_csv(cf, copy_rows("FETCH_SIZE", kib / 2))   # the copy's fetch counter reads half
    _write_csv(cw, copy_rows("WRITE_SIZE", kib))
    text = bench.pmc_summary("fwd", f, w, cf, cw, ["cmd"])
    rec = dict(line.split(": ", 1) for line in text.strip().splitlines())
    assert float(rec["fetch_scale"]) == pytest.approx(2.0)
    assert float(rec["write_scale"]) == pytest.approx(1.0)
    assert float(rec["hbm_read_bytes_per_launch"]) == pytest.approx(1000.0 * 1024 * 2, rel=1e-4)
    assert float(rec["hbm_write_bytes_per_launch"]) == pytest.approx(300.0 * 1024, rel=1e-4)
    assert rec["source_digest"] == bench.source_digest("fwd")
