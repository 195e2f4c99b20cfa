"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic byte counts the
roofline divides by, and the rule that a stored traffic record applies only to the kernel
sources it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import datagen  # noqa: E402
import differentially_private_amd as dp  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout + r.stderr


def test_headline_algorithmic_bytes():
    """Workload 2 (48 fp32 LoRA layers, 16 records x 128 tokens): the norm kernel reads every A
    and G once (305,135,616 bytes) and writes each record's gradient blocks once (16 x 294,912 x 4
    bytes)."""
    w = datagen.workload(2)
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    work = bench.algorithmic_work(w, plan, dp)
    inputs = sum(w.B * w.T * (di + do) * 4 for di, do in w.layers)
    assert inputs == 305_135_616
    assert work["norms"][0] == inputs + w.B * 294_912 * 4 == 324_009_984
    assert all(plan.layer_info(l)[1] == dp.SUM_STORED for l in range(w.n_layers))


@pytest.mark.parametrize("path,names", [("norm_kernel_traffic.json", bench.NORM_KERNEL_SOURCES),
                                        ("int8_gemm_traffic.json", bench.I8_KERNEL_SOURCES)])
def test_traffic_records_follow_the_sources(path, names, tmp_path):
    """A record carries the hash of the sources it was measured on; any edit of them changes the
    hash, so the bench line drops the record instead of reporting stale counters."""
    rec = json.load(open(os.path.join(ROOT, "profiles", path)))
    assert rec["bytes_per_launch"] > 0 and len(rec["src_hash"]) == 16
    h = bench.kernel_src_hash(names)
    assert len(h) == 16
    # the hash reads every listed source: changing one byte of any of them changes it
    import hashlib
    base = hashlib.sha256()
    for n in names:
        base.update(open(os.path.join(ROOT, "differentially_private_amd", "csrc", n), "rb").read())
    assert base.hexdigest()[:16] == h
    altered = hashlib.sha256()
    for i, n in enumerate(names):
        data = open(os.path.join(ROOT, "differentially_private_amd", "csrc", n), "rb").read()
        altered.update(data + (b" " if i == len(names) - 1 else b""))
    assert altered.hexdigest()[:16] != h
