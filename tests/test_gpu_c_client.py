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
