"""Shared helpers of the GPU parity tests: upload, state creation, fetching the
GPU results through the C ABI's debug views, and the parity bar.

Bar: int4 codes and fp32 scales of both stages bit-exact; out, m_fast and
m_slow within 1e-5 x the group's stage-2 scale (the kernels evaluate the same
sequence of binary32 operations, so they are expected to match exactly, and
the comparison also counts values that are not bit-identical).
"""
import numpy as np

F32 = np.float32
F64 = np.float64
TOL = 1e-5


def _torch():
    import torch
    return torch


def _upload(raw, dtype, device):
    torch = _torch()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw, dtype=F32))
    return [t[r].to(device).contiguous() for r in range(t.shape[0])]


def _state(P, N, dtype, compensate=True, beta=(0.5, 0.95), device="cuda:0", poison=True, group=32,
           sender_feedback=False, state_bf16=False, out_bf16=False, own_exact=False):
    torch = _torch()
    import error_compensated_bit_echo_amd as E
    cfg = E.EchoConfig.make(P, N, dtype, compensate, beta[0], beta[1], group=group,
                            sender_feedback=sender_feedback, state_bf16=state_bf16,
                            out_bf16=out_bf16, own_exact=own_exact)
    ws = torch.full((max(E.echo_workspace_bytes(cfg), 1),), 0xFF if poison else 0,
                    dtype=torch.uint8, device=device)
    return E.echo_init_state(cfg, ws)


def _fetch(state, out, direction, lo=0, hi=None):
    """Host copies of the GPU results for elements [lo, hi)."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    hi = state.numel if hi is None else hi
    v = E.echo_debug_views(state, direction)
    torch.cuda.synchronize()
    G = state.cfg.group
    g0, g1 = lo // G, hi // G
    return {
        "codes1": v["codes1"][:, lo // 2:hi // 2].cpu().numpy(),
        "scales1": v["scales1"][:, g0:g1].cpu().numpy(),
        "codes2": v["codes2"][lo // 2:hi // 2].cpu().numpy(),
        "scales2": v["scales2"][g0:g1].cpu().numpy(),
        "m_fast": v["m_fast"][lo:hi].float().cpu().numpy(),  # bf16 state widens exactly
        "m_slow": v["m_slow"][lo:hi].float().cpu().numpy(),
        "out": out[lo:hi].float().cpu().numpy(),  # a bf16 output widens exactly
        "sender_err": None if v["sender_err"] is None else v["sender_err"][:, lo:hi].float().cpu().numpy(),
    }


def _out_tensor(state, device="cuda:0"):
    torch = _torch()
    dt = torch.bfloat16 if state.cfg.out_bf16 else torch.float32
    return torch.empty(state.numel, dtype=dt, device=device)


def _compare(g, o, st_oracle, direction, compensate, where="", own_exact=False):
    """Assert the parity bar; returns the number of float elements not bit-equal.
    With own_exact, a rank's stage-1 payload over its own segment is never
    written (the owner adds its partial itself) and is left out."""
    if own_exact:
        g = dict(g)
        g["codes1"], g["scales1"] = g["codes1"].copy(), g["scales1"].copy()
        G = o["q2"].size // max(o["scales2"].size, 1)
        for r, (g0, g1) in enumerate(o["segments"]):
            g["codes1"][r, g0 * G // 2:g1 * G // 2] = o["codes1"][r, g0 * G // 2:g1 * G // 2]
            g["scales1"][r, g0:g1] = o["scales1"][r, g0:g1]
    assert np.array_equal(g["codes1"], o["codes1"]), f"stage-1 codes differ {where}"
    assert np.array_equal(g["scales1"].view(np.uint32), o["scales1"].view(np.uint32)), \
        f"stage-1 scales differ {where}"
    assert np.array_equal(g["codes2"], o["codes2"]), f"stage-2 codes differ {where}"
    assert np.array_equal(g["scales2"].view(np.uint32), o["scales2"].view(np.uint32)), \
        f"stage-2 scales differ {where}"
    s2 = np.repeat(o["scales2"].astype(F64), o["q2"].size // max(o["scales2"].size, 1) if o["scales2"].size else 1)
    inexact = 0
    pairs = [("out", o["out"])]
    if compensate:
        pairs += [("m_fast", st_oracle.m_fast[direction]), ("m_slow", st_oracle.m_slow[direction])]
    for key, want in pairs:
        got = g[key]
        d = np.abs(got.astype(F64) - want.astype(F64))
        assert np.all(d <= TOL * s2), f"{key} off by {d.max()} {where}"
        inexact += int(np.count_nonzero(got != want))
    if g.get("sender_err") is not None:
        # the ranks' stage-1 errors (sender-feedback variant), against each rank's scales
        want = st_oracle.sender_err[direction]
        got = g["sender_err"]
        s1 = np.repeat(o["scales1"].astype(F64), got.shape[1] // o["scales1"].shape[1], axis=1)
        d = np.abs(got.astype(F64) - want.astype(F64))
        assert np.all(d <= TOL * s1), f"sender_err off by {d.max()} {where}"
        inexact += int(np.count_nonzero(got != want))
    return inexact


