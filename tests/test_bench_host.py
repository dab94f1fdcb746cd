"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
byte and FLOP-eq models, the percentile summary, the measured-peak fraction,
and the rule that a traffic record applies only to the kernel sources it was
taken on."""
import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from selective_state_space_scan_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_headline():
    w = I.WORKLOADS[2]
    bld, bln = 8 * 4096 * 1024, 8 * 4096 * 16
    # x, delta read and y written (bf16); B, C read (bf16); A_log, D read and h_last written (fp32)
    want = 3 * bld * 2 + 2 * bln * 2 + 1024 * 16 * 4 + 1024 * 4 + 8 * 1024 * 16 * 4
    assert bench.algorithmic_bytes(w, 2) == want == 204017664


def test_algorithmic_bytes_backward_headline():
    w = I.WORKLOADS[2]
    bld, bln, bdn = 8 * 4096 * 1024, 8 * 4096 * 16, 8 * 1024 * 16
    n_chunks = 4096 // 32
    want = (5 * bld * 2 + 2 * bln * 2 + 2 * bln * 4 + (n_chunks - 1) * bdn * 4 + 2 * 1024 * 16 * 4 + 2 * 1024 * 4
            + 2 * bdn * 4)
    assert bench.algorithmic_bytes_bwd(w, 2, 32) == want


def test_flop_model_headline():
    w = I.WORKLOADS[2]
    flops = bench.algorithmic_flops(w, w.batch * w.seqlen)
    upd = w.batch * w.seqlen * w.dim * w.dstate
    assert flops == upd * bench.FLOPEQ_PER_UPDATE + w.batch * w.seqlen * w.dim * bench.FLOPEQ_PER_ROW_STEP
    # 16 per update + 30 per (b, t, d) at N = 16: 17.875 per update
    assert abs(flops / upd - 17.875) < 1e-12


def test_kernel_percentiles():
    p = bench.kernel_percentiles([1.0, 2.0, 3.0, 4.0, 5.0])
    assert p == {"kernel_ms_p10": 1.4, "kernel_ms_p50": 3.0, "kernel_ms_p90": 4.6}


def test_measured_peak_fraction():
    roof = {"bound": "alu", "achieved": 50.0}
    bench.add_measured_peak(roof, {"fp32_fma_tflops": 125.0, "hbm_read_gbps": 6000.0})
    assert roof["peak_measured"] == 125.0 and roof["frac_measured"] == 0.4
    roof = {"bound": "hbm", "achieved": 3000.0}
    bench.add_measured_peak(roof, {"fp32_fma_tflops": 125.0, "hbm_read_gbps": 6000.0})
    assert roof["peak_measured"] == 6000.0 and roof["frac_measured"] == 0.5
    assert "hbm_frac_measured_copy" not in roof  # no copy rate measured
    roof = {"bound": "alu", "achieved": 50.0, "hbm_gbps": 1000.0}
    bench.add_measured_peak(roof, {"fp32_fma_tflops": 125.0, "hbm_read_gbps": 6000.0, "hbm_copy_gbps": 4000.0})
    assert roof["hbm_frac_measured_copy"] == 0.25


def test_traffic_record_needs_matching_sources(tmp_path, monkeypatch):
    w = I.WORKLOADS[2]
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic(w) is None  # no record
    rec = tmp_path / f"traffic_ssm_fwd_kernel_{w.name}.txt"
    rec.write_text("# a record\nkernel_source_sha256: " + bench.kernel_source_hash() + "\n"
                   "hbm_bytes_per_launch: 123456\n")
    assert bench.measured_traffic(w) == 123456
    rec.write_text("kernel_source_sha256: 0000\nhbm_bytes_per_launch: 123456\n")
    assert bench.measured_traffic(w) is None  # taken on other sources
    # the backward's record is keyed to the backward's sources
    rb = tmp_path / f"traffic_ssm_bwd_kernel_{w.name}.txt"
    rb.write_text("kernel_source_sha256: " + bench.kernel_source_hash(bench.BWD_KERNEL_SRCS) + "\n"
                  "hbm_bytes_per_launch: 99\n")
    assert bench.measured_traffic(w, "bwd") == 99


def test_committed_records_parse():
    """The committed traffic records are well formed (whether or not they
    still match the sources)."""
    for kind, (kname, _) in bench.TRAFFIC_RECORDS.items():
        path = os.path.join(bench.PROFILES, f"traffic_{kname}_{I.WORKLOADS[2].name}.txt")
        if not os.path.exists(path):
            pytest.skip(f"no {kind} record")
        keys = {l.split(":", 1)[0].strip() for l in open(path) if ":" in l and not l.startswith("#")}
        assert {"kernel_source_sha256", "hbm_bytes_per_launch"} <= keys


def test_host_cpu_description():
    h = bench.host_cpu()
    assert set(h) == {"cpu_model", "nproc", "usable_cpus"}
    assert isinstance(h["cpu_model"], str) and h["nproc"] >= 1 and 1 <= h["usable_cpus"] <= h["nproc"]
