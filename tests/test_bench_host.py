"""Host-side logic of bench.py, on the CPU: the comment-blind source hash that
gates the recorded HBM traffic, the scaling of rocprofv3's byte counters by a
plain copy kernel, the one-GPU refusal, and the oracle's CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_code_only_ignores_comments_and_blank_lines_but_not_code():
    a = "int x = 1;  // one\n\n/* block\n   comment */\nint y = 2;\n"
    b = "int x = 1;\n// a different note\nint y = 2;   /* trailing */\n"
    c = "int x = 1;\nint y = 3;\n"
    assert bench._code_only(a) == bench._code_only(b) == "int x = 1;\nint y = 2;"
    assert bench._code_only(c) != bench._code_only(a)


def test_source_hash_covers_each_kernel_and_shares_the_backward_file():
    hs = {k: bench.source_hash(k) for k in bench.KERNEL_SOURCES}
    assert all(h and len(h) == 16 for h in hs.values())
    assert hs["bwd_dkdv"] == hs["bwd_dq"] == hs["bwd_prep"]
    assert len({hs["fwd"], hs["bwd_dkdv"], hs["kv_split"]}) == 3
    assert bench.source_hash("no_such_kernel") is None


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, value) in enumerate(rows):
            f.write(f'{i},"{name}",{counter},{value}\n')


FWD = "void attn::(anonymous namespace)::fwd_kernel<attn::bf16_t, 128, true>(attn::FwdArgs)"
DQ = "void attn::(anonymous namespace)::bwd_dq<attn::bf16_t, 128, true>(attn::BwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def test_record_traffic_scales_counters_by_the_copy_kernel(tmp_path, monkeypatch, capsys):
    traffic = tmp_path / "hbm_traffic.json"
    traffic.write_text(json.dumps({"other_workload": {"fwd": {"bytes_per_launch": 7}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    gib_kib = 1024 * 1024
    # the copy of 1 GiB reads half its bytes per FETCH_SIZE and all per WRITE_SIZE;
    # two dispatches of each kernel are averaged; an unknown kernel is skipped
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(COPY, gib_kib // 2), (COPY, gib_kib // 4), (FWD, 1000), (FWD, 3000), (DQ, 500),
                  ("some_other_kernel", 9)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(COPY, gib_kib), (FWD, 100), (FWD, 300), (DQ, 50), ("some_other_kernel", 9)])
    assert bench.record_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl") == 0
    data = json.loads(traffic.read_text())
    assert data["other_workload"] == {"fwd": {"bytes_per_launch": 7}}
    assert set(data["wl"]) == {"fwd", "bwd_dq"}
    fwd = data["wl"]["fwd"]
    assert fwd["fetch_scale"] == 2.0 and fwd["write_scale"] == 1.0
    assert fwd["bytes_read"] == 2000 * 1024 * 2 and fwd["bytes_written"] == 200 * 1024
    assert fwd["bytes_per_launch"] == fwd["bytes_read"] + fwd["bytes_written"]
    assert fwd["source_hash"] == bench.source_hash("fwd")
    assert data["wl"]["bwd_dq"]["bytes_per_launch"] == 500 * 1024 * 2 + 50 * 1024
    assert "| `fwd_kernel<attn::bf16_t, 128, true>` |" in capsys.readouterr().out


def test_record_traffic_refuses_files_without_the_copy_kernel(tmp_path, monkeypatch):
    traffic = tmp_path / "hbm_traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(FWD, 1000)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(FWD, 100)])
    assert bench.record_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl") == 1
    assert not traffic.exists()


def test_measured_traffic_only_for_the_recorded_source(tmp_path, monkeypatch):
    traffic = tmp_path / "hbm_traffic.json"
    traffic.write_text(json.dumps({"wl": {
        "fwd": {"bytes_per_launch": 123, "source_hash": bench.source_hash("fwd")},
        "bwd_dq": {"bytes_per_launch": 456, "source_hash": "0000000000000000"}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    assert bench.measured_traffic("fwd", "wl") == 123
    assert bench.measured_traffic("bwd_dq", "wl") is None
    assert bench.measured_traffic("fwd", "other") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("fwd", "wl") is None


def test_committed_traffic_records_name_known_kernels():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        data = json.load(f)
    known = set(workloads.WORKLOADS) | set(workloads.KV_WORKLOADS)
    for key, rec in data.items():
        assert key.split("+")[0] in known
        for kernel, r in rec.items():
            assert kernel in bench.KERNEL_SOURCES
            assert r["bytes_per_launch"] == pytest.approx(r["bytes_read"] + r["bytes_written"], abs=1)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_split_summary_percentages_against_the_peak_and_the_clock():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    split = {"fwd_ms_median": 0.6, "bwd_ms_median": 1.9, "clock": {"median_mhz": 1200.0}}
    s = bench.split_summary(w, split)
    tflops = (w.fwd_flops() + w.bwd_flops()) / 2.5e-3 / 1e12
    assert s["tflops"] == pytest.approx(tflops, abs=0.01)
    assert s["pct_of_peak"] == pytest.approx(100 * tflops / bench.PEAK_TFLOPS, abs=0.01)
    assert s["pct_of_peak_at_clock"] == pytest.approx(2 * s["pct_of_peak"], abs=0.02)
    assert s["bwd_tflops"] == pytest.approx(w.bwd_flops() / 1.9e-3 / 1e12, abs=0.01)


def test_kernel_summary_takes_the_kernel_with_the_most_time():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    prof = {"fwd": (10, 6.0), "bwd_prep": (10, 1.8), "bwd_dkdv": (10, 11.0), "bwd_dq": (10, 6.5)}
    kernels, roof = bench.kernel_summary(w, prof, "none", with_traffic=False)
    assert roof["kernel"] == "bwd_dkdv" and roof["traffic"] is None
    assert kernels["bwd_prep"] == {"launches": 10, "avg_ms": 0.18}
    assert roof["achieved"] == pytest.approx(0.8 * w.bwd_flops() / 1.1e-3 / 1e12, abs=0.01)
    assert roof["frac"] == pytest.approx(roof["achieved"] / bench.PEAK_TFLOPS, abs=1e-4)


def test_cpu_baseline_times_whole_heads_of_the_oracle():
    w = workloads.WORKLOADS["causal_b8h16n2048d64"].with_size(B=1, H=3, N=96, d=16)
    x = workloads.make_inputs(w)
    names = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    before = {k: os.environ.get(k) for k in names}
    out = bench.cpu_baseline(w, x, budget_s=30.0, workers=2)
    assert out["kind"] == "oracle" and out["cores"] == 2 and out["unit"] == "TFLOP/s"
    assert out["sample"].startswith(f"3 of 3 heads of {w.name}, fwd+bwd")
    assert out["value"] > 0
    # the pool's one-BLAS-thread setting does not leak into the caller
    assert {k: os.environ.get(k) for k in names} == before
