"""The C ABI used from plain C: the client in tests/c_client (gcc, strict C11,
device memory from the HIP runtime, no Python) runs three calls for each of
two configurations; its outputs must equal the oracle's on the inputs it
wrote, bit for bit."""
import os
import subprocess

import numpy as np
import pytest

from oracle import echo_oracle as eo

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "echo_c_client")
P, N = 4, 32 * 1037


def test_c_client_matches_the_oracle(tmp_path):
    assert os.path.exists(CLIENT), "the C client is not built: run __graft_entry__.build()"
    res = subprocess.run([CLIENT, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr + res.stdout
    bits = np.fromfile(tmp_path / "parts.bin", dtype=np.uint16).reshape(P, N)
    x = eo.bf16_bits_to_f32(bits)
    for c, kw in enumerate(({}, {"state_bf16": True, "out_bf16": True, "own_exact": True})):
        st = eo.OracleState(N)
        for t in range(3):
            o = eo.echo_call(x, st, eo.FWD, **kw)
            if kw.get("out_bf16"):
                got = eo.bf16_bits_to_f32(np.fromfile(tmp_path / f"out{c}_{t}.bin", dtype=np.uint16))
            else:
                got = np.fromfile(tmp_path / f"out{c}_{t}.bin", dtype=np.float32)
            assert np.array_equal(got.view(np.uint32), o["out"].view(np.uint32)), f"config {c} call {t}"


LATENCY = os.path.join(ROOT, "tests", "c_client", "echo_c_latency")


def test_c_latency_program_reports_its_three_figures():
    """The per-call latency program (plain C, eager calls) runs and prints one
    JSON line with positive figures, the round trip of a call and a synchronize
    at least half the back-to-back device time (a loose bound that catches a
    figure scaled by the wrong call count), and refuses bad arguments."""
    import json

    assert os.path.exists(LATENCY), "the latency program is not built: run __graft_entry__.build()"
    res = subprocess.run([LATENCY, "4", str(32 * 1024), "50"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr + res.stdout
    r = json.loads(res.stdout.strip().splitlines()[-1])
    assert (r["P"], r["N"], r["calls"]) == (4, 32 * 1024, 50)
    assert r["device_us"] > 0 and r["enqueue_us"] > 0
    assert r["roundtrip_us"] >= 0.5 * r["device_us"]
    # bad arguments are refused before the GPU is touched
    bad = subprocess.run([LATENCY, "4", "33", "10"], capture_output=True, text=True, timeout=60)
    assert bad.returncode == 2
