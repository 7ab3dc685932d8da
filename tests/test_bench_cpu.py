"""bench.py host logic (no GPU): the algorithmic byte and FLOP counts behind
the roofline fields, the traffic-summary hash gate, and the single-GPU
contract."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402


@pytest.mark.parametrize("name,mb", [("prefill", 680.525824), ("causal", 1219.493888),
                                     ("decode", 55.738368), ("decode_paged", 55.86944),
                                     ("decode_fp8", 175.14496), ("decode_fp4", 99.647488)])
def test_algorithmic_bytes(name, mb):
    """Unique KV for the shared-cache workloads, every valid slot's row for
    decode, plus Q, out, lse, indices and the block table."""
    assert bench.algorithmic_bytes(workloads.WORKLOADS[name]) == round(mb * 1e6)


def test_flops_per_valid_slot():
    w = workloads.WORKLOADS["prefill"]
    assert w.flops == 2.0 * 64 * (576 + 512) * 4096 * 2048
    c = workloads.WORKLOADS["causal"]
    assert c.flops == 2.0 * 64 * (576 + 512) * sum(min(t + 1, 2048) for t in range(8192))


def test_traffic_summary_applies_only_to_its_kernel_sources(tmp_path, monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "smla_fwd_prefill_traffic.json")))
    got = bench.load_traffic("prefill", 0.0)
    if rec["kernel_hash"] == bench.kernel_hash():
        assert got == rec["hbm_bytes_per_launch"]
    else:
        assert got is None
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0000000000000000")
    assert bench.load_traffic("prefill", 0.0) is None
    assert bench.load_traffic("no_such_workload", 0.0) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,key", [("prefill", "bf16_mall"), ("causal", "bf16_mall"),
                                      ("decode", "bf16_hbm"), ("decode_paged", "bf16_hbm"),
                                      ("decode_fp8", "fp8_hbm"), ("decode_fp4", "fp8_hbm")])
def test_gather_ceiling_regime_of_each_workload(name, key):
    """A shared KV small enough for the MALL is held against the MALL ceiling,
    per-sequence caches against the HBM ceiling of their row size."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "gather_ceiling.json")))
    gbs, regime = bench.gather_ceiling(workloads.WORKLOADS[name])
    assert gbs == rec["ceilings"][key]["gbs"] and regime == rec["ceilings"][key]["regime"]


def test_cpu_description_names_the_blas():
    model, blas = bench.cpu_description()
    assert model and blas and blas != "unknown"
