"""CPU checks of the benchmark's host logic: the algorithmic byte counts it
divides by kernel time (against the per-element formulas of the three kernels
and the whole-call totals of the five workloads), the counter calibration that
turns rocprofv3 FETCH_SIZE / WRITE_SIZE into bytes, and the one-GPU guard."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def total(**kw):
    return sum(bench.algorithmic_bytes(**kw).values())


def test_whole_call_bytes_of_the_workloads():
    # N * (P * (b_in + 1.25) + 21.25) per call with compensation
    assert total(P=2, N=2048, b_in=4, compensate=True) == 65_024
    assert total(P=4, N=2048 * 4096, b_in=2, compensate=True) == 287_309_824
    assert total(P=8, N=64 * 4096, b_in=2, compensate=True) == 12_386_304
    assert total(P=4, N=4096 * 4096, b_in=2, compensate=True) == 574_619_648
    assert total(P=8, N=1 << 29, b_in=2, compensate=True) == 25_367_150_592


def test_per_kernel_bytes_of_the_headline_call():
    N, P = 1 << 29, 8
    a = bench.algorithmic_bytes(P, N, 2, True)
    assert a["stage1"] == P * N * (2 + 0.625) == 11_274_289_152
    assert a["owner"] == N * (0.625 * P + 0.625 + 16) == 11_609_833_472
    assert a["decode"] == N * 4.625 == 2_483_027_968


def test_variant_bytes():
    N, P = 1 << 20, 4
    base = bench.algorithmic_bytes(P, N, 2, True)
    # compensation off: the owner neither reads nor writes the two fp32 estimates
    assert bench.algorithmic_bytes(P, N, 2, False)["owner"] == base["owner"] - 16 * N
    # bf16 state: 8 instead of 16 bytes of estimates per element
    assert bench.algorithmic_bytes(P, N, 2, True, state_bf16=True)["owner"] == base["owner"] - 8 * N
    # sender feedback: every rank reads and writes its 4-byte error (2-byte with the bf16 state)
    assert bench.algorithmic_bytes(P, N, 2, True, sender_feedback=True)["stage1"] == base["stage1"] + 8 * P * N
    assert bench.algorithmic_bytes(P, N, 2, True, sender_feedback=True, state_bf16=True)["stage1"] == \
        base["stage1"] + 4 * P * N
    # bf16 output: the decode writes 2 instead of 4 bytes per element
    assert bench.algorithmic_bytes(P, N, 2, True, out_bf16=True)["decode"] == base["decode"] - 2 * N
    # the owners' own shares: P - 1 ranks pass stage 1; the owner reads P - 1 payloads and its partial
    own = bench.algorithmic_bytes(P, N, 2, True, own_exact=True)
    assert own["stage1"] == (P - 1) * N * 2.625
    assert own["owner"] == N * (0.625 * (P - 1) + 2 + 0.625 + 16)
    # larger groups carry fewer scale bytes: 0.5 + 4/group per element of payload
    g128 = bench.algorithmic_bytes(P, N, 2, True, group=128)
    assert g128["stage1"] == P * N * (2 + 0.5 + 4 / 128)


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": "X", "Counter_Value": value})


def test_counter_calibration_scales_by_the_copy_kernel(tmp_path):
    """FETCH_SIZE reading half the copy kernel's known bytes doubles every kernel's
    reads; WRITE_SIZE reading them exactly leaves writes as they are.  Small
    multiplies of the same functor (the input generator's) are not the copy."""
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, " \
           "at::native::binary_internal::MulFunctor<float> > >"
    known_kib = bench.COPY_FLOATS * 4 / 1024
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, [(copy, known_kib / 2), (copy, 3.0), ("echo_quant_pack_k<...>", 100.0),
                         ("echo_quant_pack_k<...>", 120.0), ("echo_quant_pack_k<...>", 110.0),
                         ("echo_owner_k<...>", 50.0), ("echo_unpack_k<...>", 10.0)])
    _counter_csv(write, [(copy, known_kib), ("echo_quant_pack_k<...>", 30.0), ("echo_owner_k<...>", 40.0),
                         ("echo_unpack_k<...>", 80.0)])
    rec = bench.ingest_counters(str(fetch), str(write), workload="w", command="c")
    assert rec["copy_kernel"]["fetch_scale"] == 2.0 and rec["copy_kernel"]["write_scale"] == 1.0
    k = rec["kernels"]
    assert k["stage1"]["read_bytes"] == 110 * 1024 * 2 and k["stage1"]["write_bytes"] == 30 * 1024  # medians
    assert k["owner"]["bytes_per_launch"] == 50 * 1024 * 2 + 40 * 1024
    assert k["decode"]["bytes_per_launch"] == 10 * 1024 * 2 + 80 * 1024
    assert rec["kernel_source_sha"] == bench.kernel_source_hash()


def test_measured_traffic_is_dropped_when_the_kernels_change(tmp_path, monkeypatch):
    import json
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel_source_sha": "not-the-current-sources", "workload": "w",
                             "kernels": {"owner": {"bytes_per_launch": 5}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("owner", "w") is None
    f.write_text(json.dumps({"kernel_source_sha": bench.kernel_source_hash(), "workload": "w",
                             "kernels": {"owner": {"bytes_per_launch": 5}}}))
    assert bench.measured_traffic("owner", "w") == 5
    assert bench.measured_traffic("owner", "another workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
