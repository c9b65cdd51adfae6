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


def test_traffic_record_follows_the_kernel_code(tmp_path, monkeypatch):
    """A record is used only for its workload and while its kernel's code
    (comments and spacing aside) is the one it was measured on."""
    csrc = tmp_path / "scaled_gemm_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for name in ("gemm.hip", "quant.hip", "device_common.h"):
        shutil.copy(os.path.join(ROOT, "scaled_gemm_amd", "csrc", name), csrc / name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for kind, src in (("gemm_fused", "gemm.hip"), ("quant_act", "quant.hip")):
        record = tmp_path / "profiles" / bench.TRAFFIC[kind]["file"]
        assert bench.measured_traffic("70b_down", kind) is None             # no record
        record.write_text(json.dumps({"workload": "70b_down", "bytes_per_launch": 123.0,
                                      "source_sha256_16": bench.source_hash(kind)}))
        assert bench.measured_traffic("70b_down", kind) == 123.0
        assert bench.measured_traffic("8b_gate_up", kind) is None           # other workload
        f = csrc / src
        text = f.read_text()
        f.write_text("// a new comment\n" + text.replace("\n", "\n\n", 3) + "/* trailing */\n")
        assert bench.measured_traffic("70b_down", kind) == 123.0            # comments, spacing
        f.write_text(text.replace("{", "{ ;", 1))
        assert bench.measured_traffic("70b_down", kind) is None             # code changed
        f.write_text(text)


def test_rotation_exceeds_the_cache():
    """Every rotation holds at least three copies and more than 768 MiB
    between two uses of one copy (up to the cap on copies)."""
    for b in (1 << 10, 1 << 20, 16 << 20, 235 << 20, 470 << 20, 2 << 30):
        n = bench.n_sets(b)
        assert n >= 3
        assert (n - 1) * b > bench.ROTATE_BYTES or n == bench.MAX_SETS
