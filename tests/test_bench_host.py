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
    """The default workload is 3 (the largest configuration that fits one GPU): 256 bf16 LoRA
    layers, 256 records x 512 tokens.  The norm kernel's algorithmic bytes are one read of every
    A and G (275,951,648,768 bytes); the per-record gradient blocks of the STORED strategy
    (256 x 16,777,216 x 4 bytes written, as many read back) are reported apart."""
    assert bench.DEFAULT_WORKLOAD == 3
    w = datagen.workload(3)
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    work = bench.algorithmic_work(w, plan, dp)
    inputs = sum(w.B * w.T * (di + do) * 2 for di, do in w.layers)
    assert inputs == 275_951_648_768
    assert work["norms"][0] == inputs
    assert work["stored_write"] == work["stored_read"] == 256 * 16_777_216 * 4
    assert work["clipped_sum"] == [0, 0]          # every layer keeps its blocks
    assert work["noise"][0] == 8 * 16_777_216
    assert bench.norm_launches(w, plan, dp) == 6  # 256 layers, at most 48 a launch
    # the GEMM strategy: the sum re-reads every A and G, 2 B T d_in d_out flops per layer
    g = dp.Plan(w.layers, w.dtype, w.B, w.T, dp.PATH_AUTO, dp.SUM_GEMM)
    wg = bench.algorithmic_work(w, g, dp)
    assert wg["stored_write"] == 0 and wg["norms"][0] == inputs
    assert wg["clipped_sum"] == [inputs + 16_777_216 * 4, 2 * 256 * 512 * 16_777_216]
    assert bench.sum_launches(w, g, dp) == 6      # the tile-engine sums: 256 layers, 48 a launch
    assert bench.sum_launches(w, plan, dp) == 0   # STORED: no GEMM sum


def test_sum_launches_dense_and_lora():
    """The dense clipped sum takes at most 32 layers a launch, the tile engine 48 per MFMA row-block
    group; the GEMM lines report their per-launch figures over these counts."""
    w4 = datagen.workload(4)
    p4 = dp.Plan(w4.layers, w4.dtype, w4.B, w4.T)
    assert bench.sum_launches(w4, p4, dp) == 1    # four 4096 x 4096 bf16 layers
    w2 = datagen.workload(2)
    p2 = dp.Plan(w2.layers, w2.dtype, w2.B, w2.T, dp.PATH_AUTO, dp.SUM_GEMM)
    assert bench.sum_launches(w2, p2, dp) == 1    # 48 fp32 LoRA layers
    layers = tuple([(64, 64)] * 40 + [(64, 8)] * 50)
    p = dp.Plan(layers, dp.DTYPE_BF16, 4, 32, dp.PATH_AUTO, dp.SUM_GEMM)
    w = w4.with_(layers=layers, layer_names=tuple(str(i) for i in range(90)), B=4, T=32)
    assert bench.sum_launches(w, p, dp) == 2 + 2  # 40 dense (32 a launch), 50 tile-engine (48)


def test_workload2_algorithmic_bytes():
    """Workload 2 (48 fp32 LoRA layers, 16 records x 128 tokens): 305,135,616 bytes of inputs read
    once by the norm kernel, in one launch."""
    w = datagen.workload(2)
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    work = bench.algorithmic_work(w, plan, dp)
    assert work["norms"][0] == 305_135_616
    assert work["stored_write"] == w.B * 294_912 * 4
    assert all(plan.layer_info(l)[1] == dp.SUM_STORED for l in range(w.n_layers))
    assert bench.norm_launches(w, plan, dp) == 1


def _traffic_records():
    recs = [(f, bench.PHASE_SOURCES[json.load(open(os.path.join(ROOT, "profiles", f)))["kernel_phase"]])
            for f in sorted(os.listdir(os.path.join(ROOT, "profiles")))
            if f.startswith("traffic_") and f.endswith(".json")]
    return recs + [("int8_gemm_traffic.json", bench.I8_KERNEL_SOURCES)]


@pytest.mark.parametrize("path,names", _traffic_records())
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


@pytest.mark.parametrize("path,names", _traffic_records())
def test_traffic_records_are_current(path, names):
    """The committed counter records were taken on the sources as they stand: an edit of a hashed
    source without new counters would leave the bench lines' `traffic` null."""
    rec = json.load(open(os.path.join(ROOT, "profiles", path)))
    assert rec["src_hash"] == bench.kernel_src_hash(names), \
        f"{path}: its counters predate the current sources; take FETCH_SIZE / WRITE_SIZE again"
