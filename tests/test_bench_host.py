"""Host-side checks of bench.py's bookkeeping (no GPU): the traffic records in
profiles/ parse, and a record only counts for the sources it was measured on."""

import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from masked_varlen_softmax_amd import build  # noqa: E402

KEYS = {"kernel", "workload", "fetch_kib", "write_kib", "fetch_factor", "write_factor", "source_sha256"}


def _records():
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            out += [json.loads(l.split(":", 1)[1]) for l in f if l.startswith("traffic-record:")]
    return out


def test_traffic_records_are_well_formed():
    recs = _records()
    assert recs, "profiles/ holds no traffic-record line"
    for r in recs:
        assert set(r) == KEYS
        assert r["fetch_kib"] > 0 and r["write_kib"] > 0 and len(r["source_sha256"]) == 64


def test_traffic_only_for_matching_sources(monkeypatch):
    recs = _records()
    wl = recs[0]["workload"]
    monkeypatch.setattr(build, "source_digest", lambda kind=None: recs[0]["source_sha256"])
    r = recs[0]
    want = round(1024 * (r["fetch_kib"] * r["fetch_factor"] + r["write_kib"] * r["write_factor"]))
    assert bench.profiled_traffic(wl) == want
    monkeypatch.setattr(build, "source_digest", lambda kind=None: "0" * 64)
    assert bench.profiled_traffic(wl) is None


def test_source_digest_changes_with_content(tmp_path, monkeypatch):
    (tmp_path / "a.hip").write_text("x")
    monkeypatch.setattr(build, "CSRC", str(tmp_path))
    d1 = build.source_digest()
    (tmp_path / "a.hip").write_text("y")
    assert build.source_digest() != d1


def test_kernel_digest_covers_only_its_sources(tmp_path, monkeypatch):
    for name in {n for v in build.KERNEL_SOURCES.values() for n in v} | {"other.hip"}:
        (tmp_path / name).write_text(name)
    monkeypatch.setattr(build, "CSRC", str(tmp_path))
    pre, dec = build.source_digest("prefill"), build.source_digest("decode")
    (tmp_path / "other.hip").write_text("changed")
    assert build.source_digest("prefill") == pre and build.source_digest("decode") == dec
    (tmp_path / "decode.hip").write_text("changed")
    assert build.source_digest("prefill") == pre and build.source_digest("decode") != dec
    (tmp_path / "kernels.hpp").write_text("changed")
    assert build.source_digest("prefill") != pre


def test_bench_refuses_more_than_one_gpu():
    import subprocess

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_runs_whole_requests_until_the_time_floor(mvs_lib):
    from masked_varlen_softmax_amd import workloads as W

    case = W.make_prefill("tiny", 3, [40, 24], [40, 30], 2, 1, 64, "bf16", causal=True, wl=16)
    pre = {"case": case, "host_table": None, "workload": "tiny"}
    # a floor of zero runs exactly one request; a large floor stops after four passes over the batch
    one = bench.cpu_baseline(pre, min_s=0.0)
    assert one["kind"] == "oracle" and one["value"] > 0 and one["sample"].startswith("1 whole requests of the 2")
    many = bench.cpu_baseline(pre, min_s=1e9)
    assert many["sample"].startswith("8 whole requests of the 2")
    # the sample names the workload's own shape
    assert "24-40 queries x 30-40 keys each, all 2 q heads, head_dim 64" in many["sample"]


def test_layer_record_bound_and_fractions():
    from masked_varlen_softmax_amd import workloads as W

    case = W.make_prefill("tiny", 3, [64], [64], 2, 1, 128, "bf16", causal=True)
    pre = {"case": case, "workload": "c4", "useful_flops": 2.5e15 * 1e-3 / 2, "alg_bytes": 8e12 * 1e-3 / 4,
           "kernel_ms": 1.0, "kernel_ms_min": 1.0, "step_ms": 1.1}
    rec = bench.layer_record(pre)
    # 1.25 TFLOP and 2 GB in 1 ms: half the matrix peak, a quarter of HBM, intensity above the ridge
    assert rec["mfma_frac"] == 0.5 and rec["hbm_frac"] == 0.25 and rec["bound"] == "mfma" and rec["frac"] == 0.5
    pre["alg_bytes"] = 8e12 * 1e-3  # 8 GB: intensity 156 FLOP/B, below the 312 ridge
    rec = bench.layer_record(pre)
    assert rec["bound"] == "hbm" and rec["frac"] == rec["hbm_frac"] == 1.0


def test_algorithmic_bytes_of_the_sliding_layer():
    """Q + K + V + O + table of the 4 x 4096, 16 q / 8 kv heads, D 256 layer (402 784 256 bytes)."""
    from masked_varlen_softmax_amd import workloads as W

    case = W.make_prefill("shape", 3, [1, 1], [1, 1], 16, 8, 256, "bf16")
    case.cu_q = case.cu_k = W._cu([4096] * 4)  # only the sizes matter
    assert bench.algorithmic_bytes(case, True) == 402_784_256
