"""Host-side logic of bench.py, no GPU: the FLOP counts against their
definitions, the refusal of more than one GPU, the admitted-key count behind
the CPU baseline's FLOP figure, and the rules that tie recorded HBM counters to
the kernel sources they were taken on."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_forward_flops_follow_the_metric_definition():
    # 4 N_q N_k D H, halved for causal; varlen sums 2 L^2 D H per causal sequence
    w = W.WORKLOADS["dense_n1024_h4_d64_f16"]
    assert bench.fwd_flops(w) == 4 * 1024 * 1024 * 64 * 4
    w = W.WORKLOADS["causal_n4096_h16_d128_bf16"]
    assert bench.fwd_flops(w) == 2 * 4096 * 4096 * 128 * 16
    w = W.WORKLOADS["rect_sq8192_sk2048_h1_d64_f32_fwdbwd"]
    assert bench.fwd_flops(w) == 4 * 8192 * 2048 * 64
    assert bench.bwd_flops(w) == 10 * 8192 * 2048 * 64  # five contractions
    w = W.WORKLOADS["varlen_causal_16k_h8_d64_f16"]
    assert sum(w.lengths) == 16384
    assert bench.fwd_flops(w) == sum(2 * L * L * 64 * 8 for L in w.lengths)


def test_admitted_count_matches_a_brute_force_mask():
    lengths = [5, 0, 3, 1, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    n = int(cu[-1])
    seq = np.repeat(np.arange(len(lengths)), lengths)
    for causal in (False, True):
        w = W.Workload("t", 1, n, n, 64, "f16", causal, 0, lengths=lengths)
        for i in range(n):
            admit = (seq == seq[i]) & ((np.arange(n) <= i) if causal else True)
            assert bench.admitted_count(w, i, cu) == int(admit.sum())
    w = W.Workload("t", 1, 9, 9, 64, "f16", True, 0)
    assert [bench.admitted_count(w, i, None) for i in range(9)] == list(range(1, 10))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hash_ignores_comments_and_layout_only():
    a = "int f(int x) { return x + 1; } // note"
    b = "/* block */ int f(int x)\n{\n    return x + 1;  // other note\n}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only("int f(int x) { return x + 2; }")
    # a comment marker inside a string literal is code
    assert "a//b" in bench._code_only('const char *s = "a//b"; // tail')


def test_recorded_traffic_needs_the_same_workload_kernel_and_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("w", "k") is None  # no records at all
    (tmp_path / "profiles").mkdir()
    rec = {"w": {"kernel": "k", "source_sha": "abc", "traffic_bytes": 123.0}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "abc")
    assert bench.recorded_traffic("w", "k") == 123.0
    assert bench.recorded_traffic("w", "k2") is None
    assert bench.recorded_traffic("w2", "k") is None
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "changed")
    assert bench.recorded_traffic("w", "k") is None


def test_kernel_identifiers_read_mangled_and_demangled_names():
    ids = bench.kernel_identifiers("_ZN6osattn12bwd16_kernelIDF16bLi128ELi1ELb0EEEvNS_9BwdParamsE")
    assert "bwd16_kernel" in ids and "osattn" in ids and "BwdParams" in ids
    ids = bench.kernel_identifiers("void osattn::fwd_wide_kernel<__bf16, 1, false>(osattn::FwdParams)")
    assert "fwd_wide_kernel" in ids


def test_record_traffic_sums_each_kernels_average_and_scales(tmp_path, monkeypatch):
    # Two kernels of one launch, two dispatches each: per kernel the average per
    # dispatch, summed; FETCH_SIZE scaled by the calibration factor, WRITE_SIZE 1x.
    head = '"Kernel_Name","Counter_Name","Counter_Value"\n'
    rows = [("_ZN6osattn16bwd16_pre_kernelIDF16bLi128EEEvNS_9BwdParamsE", 10.0, 14.0),
            ("_ZN6osattn12bwd16_kernelIDF16bLi128ELi1ELb0EEEvNS_9BwdParamsE", 100.0, 300.0),
            ("void at::native::vectorized_elementwise_kernel<4>", 5000.0, 5000.0)]
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    fetch.write_text(head + "".join('"%s","FETCH_SIZE",%f\n"%s","FETCH_SIZE",%f\n' % (n, a, n, b)
                                    for n, a, b in rows))
    write.write_text(head + "".join('"%s","WRITE_SIZE",%f\n"%s","WRITE_SIZE",%f\n' % (n, a, n, b)
                                    for n, a, b in rows))
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "abc")
    rec = bench.record_traffic("w+bwd", "bwd16_pre+bwd16_kernel", str(fetch), str(write))
    assert rec["fetch_kib"] == 12.0 + 200.0 and rec["write_kib"] == 12.0 + 200.0
    assert abs(rec["traffic_bytes"] - (212.0 * bench.FETCH_SCALE + 212.0) * 1024) < 1e-6
    stored = json.loads((tmp_path / "profiles" / "traffic.json").read_text())
    assert stored["w+bwd"]["source_sha"] == "abc"
    assert bench.recorded_traffic("w+bwd", "bwd16_pre+bwd16_kernel") == rec["traffic_bytes"]


def test_counter_per_launch_counts_repeated_and_absent_kernels(tmp_path):
    # Two launches: the reduction runs three times per launch, the schedule
    # kernel not at all; the sum over every dispatch is divided by two.
    head = '"Kernel_Name","Counter_Name","Counter_Value"\n'
    body = ""
    for _ in range(2):
        body += '"_ZN6osattn12bwd16_kernelIDF16_Li64ELi0ELb0EEEvNS_9BwdParamsE","FETCH_SIZE",100\n'
        body += '"_ZN6osattn19bwd16_reduce_kernelIDF16_Li64EEEvNS_12ReduceParamsE","FETCH_SIZE",7\n' * 3
    path = tmp_path / "fetch.csv"
    path.write_text(head + body)
    kib, counts = bench.counter_kib_per_launch(
        str(path), "varlen_schedule_kernel+bwd16_kernel+bwd16_reduce", "FETCH_SIZE")
    assert kib == 100.0 + 21.0
    assert counts == {"varlen_schedule_kernel": 0.0, "bwd16_kernel": 1.0, "bwd16_reduce": 3.0}
    with pytest.raises(SystemExit):
        bench.counter_kib_per_launch(str(path), "fwd16_kernel", "FETCH_SIZE")
