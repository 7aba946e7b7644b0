"""Host-side logic of bench.py (no GPU): the one-GPU guard and the HBM traffic
summary that scales rocprofv3 byte counters by a plain copy of known size."""

from __future__ import annotations

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


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch):
    b = _bench()
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(out))
    kib = b.COPY_BYTES // 1024
    fwd = "_ZN2fa12_GLOBAL__N_115fwd_mfma_kernelIDF16bLi128ELb1ELb0EEEvNS_4ArgsE"
    # FETCH_SIZE reads half the copy's bytes (factor 2); two rows of one dispatch add up
    _write_counters(tmp_path / "fetch", [
        (1, "neg_kernel<float>", "FETCH_SIZE", kib // 2),
        (2, fwd, "FETCH_SIZE", 600), (2, fwd, "FETCH_SIZE", 400),
        (3, fwd, "FETCH_SIZE", 1200),
        (4, "unrelated_kernel", "FETCH_SIZE", 99999),
    ])
    # WRITE_SIZE reads the copy's bytes exactly (factor 1)
    _write_counters(tmp_path / "write", [
        (1, "neg_kernel<float>", "WRITE_SIZE", kib),
        (2, fwd, "WRITE_SIZE", 100),
        (3, fwd, "WRITE_SIZE", 300),
    ])
    b.summarise_traffic("synthetic", str(tmp_path / "fetch"), str(tmp_path / "write"))
    t = json.loads(out.read_text())
    cal = t["_calibration"]["synthetic"]
    assert cal["fetch_factor"] == pytest.approx(2.0)
    assert cal["write_factor"] == pytest.approx(1.0)
    r = t["synthetic"]["fwd"]
    # per dispatch: fetch (1000 + 1200) / 2 KiB x 2, write (100 + 300) / 2 KiB x 1
    assert r["fetch_bytes"] == 1100 * 1024 * 2
    assert r["write_bytes"] == 200 * 1024
    assert r["bytes_per_launch"] == 1100 * 1024 * 2 + 200 * 1024
    assert r["dispatches"] == [2, 2]
    assert r["source_hash"] == b.source_hash("fwd")
    assert set(t["synthetic"]) == {"fwd"}


def test_traffic_summary_needs_the_copy(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    fwd = "fwd_mfma_kernel"
    _write_counters(tmp_path / "fetch", [(2, fwd, "FETCH_SIZE", 1000)])
    _write_counters(tmp_path / "write", [(2, fwd, "WRITE_SIZE", 100)])
    with pytest.raises(SystemExit):
        b.summarise_traffic("synthetic", str(tmp_path / "fetch"), str(tmp_path / "write"))
    assert not (tmp_path / "traffic.json").exists()


def test_source_hash_follows_the_kernel_sources():
    b = _bench()
    h = {k: b.source_hash(k) for k in b.KERNEL_SOURCES}
    assert all(len(v) == 16 for v in h.values())
    # the pre-pass and dQ kernels share one source file and its dependencies
    assert h["bwd_dsum"] == h["bwd_dq"]
    assert len({h["fwd"], h["bwd_dkdv"], h["bwd_dq"]}) == 3


def test_counter_summary_means_per_dispatch(tmp_path):
    b = _bench()
    d = str(tmp_path / "pmc")
    _write_counters(d, [
        (1, "void fa::(anonymous namespace)::fwd_mfma_kernel<__bf16, 128, true, false, false>(fa::Args)", "MfmaUtil", 40.0),
        (2, "void fa::(anonymous namespace)::fwd_mfma_kernel<__bf16, 128, true, false, false>(fa::Args)", "MfmaUtil", 60.0),
        (3, "void fa::(anonymous namespace)::bwd_dq_kernel<__bf16, 128, true, false, false>(fa::Args)", "LdsUtil", 70.0),
        (4, "neg_kernel", "MfmaUtil", 1.0),
    ])
    out = b.summarise_counters([d])
    assert "| fwd | 2 | — | 50 |" in out.replace("50.0", "50")
    assert "| bwd_dq | 1 | 70 | — |" in out
    assert "neg" not in out


def test_metric_labels_name_their_workload():
    b = _bench()
    sys.path.insert(0, ROOT)
    from exact_io_aware_43_amd.workloads import WORKLOADS

    assert b.metric_label(WORKLOADS["long_causal"], True) == b.METRIC
    for name in ("gpt2m", "gqa", "varlen_alibi", "long_causal_fp16"):
        w = WORKLOADS[name]
        label = b.metric_label(w, bool(w.backward))
        assert label != b.METRIC and f"({name})" in label
        assert ("fwd/bwd" in label) == bool(w.backward)
