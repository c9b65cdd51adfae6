"""Host-side logic of bench.py (CPU only): the one-GPU rule and the
validity check of the recorded HBM traffic."""
import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        for extra in ([], ["--sweep"]):
            r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n),
                                *extra], capture_output=True, text=True, timeout=120)
            assert r.returncode == 2, r.stderr
            line = json.loads(r.stdout.strip().splitlines()[-1])
            assert line["n_gpus_requested"] == n and "one GPU" in line["error"]


def test_traffic_record_follows_the_gemm_code(tmp_path, monkeypatch):
    """The record is used only for its workload and while the GEMM's code
    (comments and spacing aside) is the one it was measured on."""
    csrc = tmp_path / "scaled_gemm_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("gemm.hip", "device_common.h"):
        shutil.copy(os.path.join(ROOT, "scaled_gemm_amd", "csrc", name), csrc / name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    record = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(record))
    assert bench.measured_traffic("70b_down") is None                 # no record
    record.write_text(json.dumps({"workload": "70b_down", "bytes_per_launch": 123.0,
                                  "gemm_source_sha256_16": bench.gemm_source_hash()}))
    assert bench.measured_traffic("70b_down") == 123.0
    assert bench.measured_traffic("8b_gate_up") is None               # other workload
    gemm = csrc / "gemm.hip"
    text = gemm.read_text()
    gemm.write_text("// a new comment\n" + text.replace("\n", "\n\n", 3) + "/* trailing */\n")
    assert bench.measured_traffic("70b_down") == 123.0                # comments, spacing
    gemm.write_text(text.replace("{", "{ ;", 1))
    assert bench.measured_traffic("70b_down") is None                 # code changed
