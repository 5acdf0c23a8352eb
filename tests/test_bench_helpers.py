"""CPU tests of bench.py's bookkeeping: the per-kernel source hashes that
decide whether a committed traffic summary still applies, the traffic it
yields, and the split of a kernel trace by benchmark phase."""
import csv
import json
import os

import pytest

import bench


def _summary(tmp_path, hashes, fetch_kib=1000.0, write_kib=24.0):
    lines = [f"sources {k} {h}" for k, h in hashes.items()]
    lines += ["fetch_factor 2.0000", "write_factor 1.0000",
              f"kernel lq::sign_fp6_kernel<3, 1, 8, 2, false> fetch_kib {fetch_kib} write_kib {write_kib}",
              "kernel lq::wspace_kernel<8, 3, 8> fetch_kib 10.0 write_kib 5.0"]
    p = tmp_path / "traffic.txt"
    p.write_text("\n".join(lines) + "\n")
    return str(p)


def test_traffic_needs_the_kernels_own_hash(tmp_path, monkeypatch):
    good = {k: bench.kernel_sources_hash(k) for k in bench.TRAFFIC_SOURCES}
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", _summary(tmp_path, good))
    # (fetch * factor + write) KiB per launch, in bytes
    assert bench.traffic_from_summary("sign_fp6_kernel") == pytest.approx((1000.0 * 2 + 24.0) * 1024)
    assert bench.traffic_from_summary("wspace_kernel") == pytest.approx((10.0 * 2 + 5.0) * 1024)
    # a kernel with no measured row, or none listed, has no traffic
    assert bench.traffic_from_summary("sign_mfma_large_kernel") is None
    assert bench.traffic_from_summary("not_a_kernel") is None


def test_a_changed_kernel_voids_only_its_own_traffic(tmp_path, monkeypatch):
    hashes = {k: bench.kernel_sources_hash(k) for k in bench.TRAFFIC_SOURCES}
    hashes["wspace_kernel"] = "0" * 16
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", _summary(tmp_path, hashes))
    assert bench.traffic_from_summary("wspace_kernel") is None
    assert bench.traffic_from_summary("sign_fp6_kernel") is not None


def test_source_hash_covers_the_kernel_file_and_headers():
    csrc = os.path.join(bench.ROOT, "bit_matmul_amd", "csrc")
    for k, f in bench.TRAFFIC_SOURCES.items():
        assert os.path.exists(os.path.join(csrc, f)), (k, f)
        assert len(bench.kernel_sources_hash(k)) == 16
    # kernels in different files hash differently
    assert bench.kernel_sources_hash("sign_fp6_kernel") != bench.kernel_sources_hash("wspace_kernel")
    assert bench.kernel_sources_hash("wspace_kernel") == bench.kernel_sources_hash("xpw_kernel")


def test_committed_summary_lists_every_kernel_hash():
    with open(bench.TRAFFIC_SUMMARY) as f:
        listed = {l.split()[1] for l in f if l.startswith("sources ")}
    assert listed == set(bench.TRAFFIC_SOURCES)


def test_trace_split_by_phase(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for dur in (10000, 12000, 20000, 22000):     # two phases of two launches
            w.writerow(["lq::sign_fp6_kernel<3, 1, 8, 2, false>(...)", t, t + dur])
            t += dur + 1000
        w.writerow(["lq::prep_kernel<1, 1, true>(...)", t, t + 3000])
    phases = tmp_path / "phases.json"
    phases.write_text(json.dumps([["first", 2], ["second", 2]]))
    out = bench.summarize_stats(str(d), str(phases))
    assert "first | 2 launches | avg 11.000 us" in out
    assert "second | 2 launches | avg 21.000 us" in out
    assert "lq::prep_kernel<1, 1, true> | 1 | 3.000" in out
