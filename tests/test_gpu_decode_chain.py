"""The decode-shaped workload on the GPU: a 128-layer residual chain, P = 8,
[64, 4096] bf16 partials per layer from a pre-norm random map, one forward
compensator state for the whole chain.

Teacher-forced parity: the chain advances with the GPU's outputs, and at every
layer the oracle reduces exactly the bf16 partials the GPU chain produced, with
its own state; every value is compared at the parity bar.  The oracle's
owner-stage sums also give the accumulated owner error D_l = sum_t (B_t - S_t),
which must stay within the compensator's hard bound at every depth (the pages:
with compensation the partial sum of errors stays bounded and does not grow
with depth; rit.work "echo-4-bit-gpu-communication", «Как Echo возвращает
ошибку в следующие вызовы»).
"""
import numpy as np
import pytest

from oracle import echo_oracle as eo
from error_compensated_bit_echo_amd import synth
from parity_helpers import _compare, _fetch, _state, _torch

pytestmark = pytest.mark.gpu


def test_decode_chain_teacher_forced_parity_and_bounded_error(cuda):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    c = synth.DECODE_CHAIN
    P, rows, hd, L = 8, c["rows"], c["hidden"], c["layers"]
    N = rows * hd
    st = _state(P, N, "bf16")
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    h = synth.decode_h0(cuda)
    D = np.zeros(N, np.float64)
    rmax = np.zeros(N, np.float64)
    vmax = 0.0
    worst = 0.0
    for layer in range(1, L + 1):
        parts = synth.decode_partials(h, synth.decode_weight(layer, cuda), P)
        E.echo_reduce(parts, out, st, E.ECHO_FWD)
        host = np.stack([p.float().cpu().numpy() for p in parts])
        o = eo.echo_call(host, so, eo.FWD)
        assert _compare(_fetch(st, out, 0), o, so, 0, True, f"layer {layer}") == 0
        h += out.view(rows, hd)
        # accumulated owner-stage error and the hard bound |D| <= 11 * max_t |r_t|
        # (sum of the compensator's impulse response 1/2 (0.5^n + 0.95^n)), plus
        # the binary32 rounding of V = S + c, at most half an ulp per call
        D += o["B"].astype(np.float64) - o["S"].astype(np.float64)
        rmax = np.maximum(rmax, np.abs(o["r"].astype(np.float64)))
        vmax = max(vmax, float(np.max(np.abs(o["V"]))))
        slack = layer * vmax * 2.0 ** -24
        excess = np.abs(D) - (11.0 * rmax + slack)
        assert np.all(excess <= 0), f"layer {layer}: accumulated error beyond the bound by {excess.max()}"
        worst = max(worst, float(np.max(np.abs(D) / (11.0 * rmax + slack))))
    print(f"decode chain: {L} layers match the oracle; max |D|/bound = {worst:.3f}", flush=True)


def test_decode_chain_with_sender_feedback_keeps_the_end_to_end_error_flat(cuda):
    """The same chain with sender feedback (every rank carries its own stage-1
    error into its next call), teacher-forced against the oracle at every layer,
    and driven against a chain whose all-reduce is exact (float64): its
    end-to-end error stops growing with depth (layers 16 to 128 within 10 %),
    while the chain with owner compensation alone keeps growing."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    c = synth.DECODE_CHAIN
    P, rows, hd, L = 8, c["rows"], c["hidden"], c["layers"]
    N = rows * hd
    sts = {"sfb": _state(P, N, "bf16", sender_feedback=True), "on": _state(P, N, "bf16")}
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    h0 = synth.decode_h0(cuda)
    h = {m: h0.clone() for m in sts}
    hx = h0.double()
    rel = {m: {} for m in sts}
    for layer in range(1, L + 1):
        w = synth.decode_weight(layer, cuda)
        for m, st in sts.items():
            parts = synth.decode_partials(h[m], w, P)
            E.echo_reduce(parts, out, st, E.ECHO_FWD)
            if m == "sfb":
                host = np.stack([p.float().cpu().numpy() for p in parts])
                o = eo.echo_call(host, so, eo.FWD, sender_feedback=True)
                assert _compare(_fetch(st, out, 0), o, so, 0, True, f"layer {layer}") == 0
            h[m] += out.view(rows, hd)
        hx += sum(p.double() for p in synth.decode_partials(hx.float(), w, P)).view(rows, hd)
        scale = hx.pow(2).mean().sqrt().item()
        for m in sts:
            rel[m][layer] = (h[m].double() - hx).pow(2).mean().sqrt().item() / scale
    print(f"decode chain relative error at 16 / 128 layers: sender feedback {rel['sfb'][16]:.4f} / "
          f"{rel['sfb'][128]:.4f}, owner compensation only {rel['on'][16]:.4f} / {rel['on'][128]:.4f}", flush=True)
    assert rel["sfb"][128] <= 1.1 * rel["sfb"][16]
    assert rel["on"][128] >= 1.1 * rel["on"][16]
    assert rel["sfb"][128] < rel["on"][128]
