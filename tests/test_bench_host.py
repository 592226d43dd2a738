"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
flop and byte counts its roofline fractions divide by, the workload names,
and the rule that the committed HBM-traffic figure is reported only for the
GEMM sources it was measured on."""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2",
                        "--steps", "1", "--warmup", "0"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_flop_and_byte_counts():
    # 2*T*L*n multiply-adds of the projection
    assert bench.flops_of(8192) == 2 * 8192 * 1024 * 7168 == 120259084288
    # W window once, the partial once, a read and a write of the out window,
    # the norm weight
    assert bench.bytes_of(1) == 2 * 7168 * 1024 + 2 * 1024 + 4 * 7168 + 2 * 1024 == 14712832
    assert bench.bytes_of(256, n=896, P_=8) == (2 * 896 * 1024 + 2 * 8 * 256 * 1024
                                               + 4 * 256 * 896 + 2 * 1024)
    assert bench.bytes_of(16, norm=False) == bench.bytes_of(16) - 2 * 1024
    # AttnRes zero-block with every switch on: prefix and delta read, prefix,
    # block slot and output written, the weight once
    assert bench.attn_res_bytes(1, 7168) == 10 * 7168 + 2 * 7168 == 86016


def test_workload_names():
    from latent_moe_output_amd import synth

    assert bench.tail_workload("decode16").T == 16
    assert bench.tail_workload("decode1").n == 7168
    assert bench.tail_workload("prefill").T == 8192
    for name in ("shard", "ragged", "ragged_nonorm"):
        assert bench.tail_workload(name) is synth.WORKLOADS[name]
    with pytest.raises(KeyError):
        bench.tail_workload("no_such_workload")


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    srcs = [tmp_path / "k_gemm.hip", tmp_path / "lt_device.h"]
    srcs[0].write_text("kernel source\n")
    srcs[1].write_text("helpers\n")
    sha = hashlib.sha256(b"".join(p.read_bytes() for p in srcs)).hexdigest()
    traffic = tmp_path / "traffic.md"
    traffic.write_text("# summary\n\ntraffic_k_gemm_T8192 bytes=425287680 sources_sha256=%s\n" % sha)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    monkeypatch.setattr(bench, "GEMM_SOURCES", [str(p) for p in srcs])
    assert bench.gemm_traffic_bytes() == 425287680
    srcs[0].write_text("kernel source, changed\n")
    assert bench.gemm_traffic_bytes() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.gemm_traffic_bytes() is None


def test_committed_traffic_figure_matches_the_gemm_sources():
    """The HBM-traffic summary under profiles/ was taken on the GEMM sources
    as committed; a change to them without new counters would turn the
    benchmark's `roofline.traffic` into null."""
    assert bench.gemm_traffic_bytes() is not None
