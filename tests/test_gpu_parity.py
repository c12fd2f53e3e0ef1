"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bar: int4 codes and fp32 scales of both stages bit-exact; out, m_fast and
m_slow within 1e-5 x the group's stage-2 scale (the kernels evaluate the same
sequence of binary32 operations, so they are expected to match exactly, and
the tests also count exact matches).
"""
import numpy as np
import pytest

from oracle import echo_oracle as eo
from error_compensated_bit_echo_amd import synth
from parity_helpers import F32, _compare, _fetch, _out_tensor, _state, _torch, _upload

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# tiny configuration: every call, every value
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("compensate", [True, False])
def test_tiny_config_every_call(cuda, compensate):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    c = synth.WORKLOADS["tiny"]
    P, N = c["P"], synth.numel("tiny")
    st = _state(P, N, "f32", compensate)
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    inexact = 0
    for t in range(c["calls"]):
        raw, vals = synth.host_partials("tiny", 0, t)
        E.echo_reduce(_upload(raw, "f32", cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(vals, so, eo.FWD, compensate=compensate)
        inexact += _compare(_fetch(st, out, 0), o, so, 0, compensate, f"call {t}")
    assert inexact == 0


# ---------------------------------------------------------------------------
# several tiles plus a ragged tail, every P, both dtypes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_multi_tile_ragged(cuda, P, dtype):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    N = 32 * (64 * 3 + 37) * 8 + 32 * 5  # several 2048-element tiles plus a ragged tail
    st = _state(P, N, dtype)
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    for t in range(3):
        raw, vals = synth.host_partials("prefill", 0, t, P=P, n=N, dtype=dtype)
        E.echo_reduce(_upload(raw, dtype, cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(vals, so, eo.FWD)
        assert _compare(_fetch(st, out, 0), o, so, 0, True, f"P={P} {dtype} call {t}") == 0


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("P,dtype", [(1, "bf16"), (3, "f32"), (8, "bf16"), (16, "bf16")])
def test_larger_groups_multi_tile_ragged(cuda, P, dtype, group):
    """The group-size variants: 8 or 16 lanes per group, several tiles and a
    ragged tail, tie-rich and normal data, compensation on."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    N = 2048 * 7 + group * 3
    st = _state(P, N, dtype, group=group)
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    rng = np.random.default_rng(group + P)
    for t in range(4):
        if t % 2:
            vals = (rng.integers(-12, 13, (P, N)) * 0.25).astype(F32)
            raw = vals if dtype == "f32" else synth.f32_to_bf16_bits(vals)
        else:
            raw, vals = synth.host_partials("prefill", 0, t, P=P, n=N, dtype=dtype)
        E.echo_reduce(_upload(raw, dtype, cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(vals, so, eo.FWD, group=group)
        assert _compare(_fetch(st, out, 0), o, so, 0, True, f"G={group} P={P} {dtype} call {t}") == 0


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def _tie_rich(P, N, rng):
    x = (rng.integers(-12, 13, (P, N)) * 0.25).astype(F32)
    return x


def _special_values(P, N, rng):
    x = rng.standard_normal((P, N)).astype(F32)
    g = x.reshape(P, -1, 32)
    ng = g.shape[1]
    g[:, 0] = 0.0                                     # all-zero group
    g[:, 1 % ng] = -0.0                               # negative zeros
    g[:, 2 % ng] *= F32(1e30)                         # huge
    g[:, 3 % ng] *= F32(1e-30)                        # tiny but normal scale
    g[:, 4 % ng] = (rng.integers(-80, 80, (P, 32)) * 2.0 ** -149).astype(F32)  # subnormal
    g[:, 5 % ng] = (rng.integers(-3, 4, (P, 32)) * 2.0 ** -149).astype(F32)    # scale underflows
    g[:, 6 % ng, 1:] = 0.0                            # single nonzero element
    g[:, 7 % ng] = (rng.integers(-127, 128, (P, 32)) * 2.0 ** -133).astype(F32)  # subnormal, exact in bf16
    return g.reshape(P, N)


EDGE_VARIANTS = [{}, {"own_exact": True, "out_bf16": True},
                 {"state_bf16": True, "sender_feedback": True, "group": 64}]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", range(len(EDGE_VARIANTS)))
@pytest.mark.parametrize("case", ["ties", "special", "one_group", "fewer_groups_than_ranks"])
def test_edge_cases(cuda, case, variant, dtype):
    """Partials built to hit the quantizer's special cases, as fp32 and rounded
    to bfloat16 (ties and the special groups stay exact or become other special
    values: zeros, subnormals, single nonzero elements)."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    rng = np.random.default_rng(5)
    if case == "ties":
        P, N, gen = 3, 32 * 300, _tie_rich
    elif case == "special":
        P, N, gen = 4, 32 * 64, _special_values
    elif case == "one_group":
        P, N, gen = 2, 32, lambda P, N, r: r.standard_normal((P, N)).astype(F32)
    else:
        P, N, gen = 16, 32 * 5, lambda P, N, r: r.standard_normal((P, N)).astype(F32)
    kw = EDGE_VARIANTS[variant]
    if N % kw.get("group", 32):
        N = 2 * N if case == "one_group" else N + 32  # whole groups of 64
    st = _state(P, N, dtype, **kw)
    so = eo.OracleState(N)
    out = _out_tensor(st, cuda)
    for t in range(6):
        x = gen(P, N, rng)
        raw = x
        if dtype == "bf16":
            raw = synth.f32_to_bf16_bits(x)
            x = synth.bf16_bits_as_f32(raw)
        E.echo_reduce(_upload(raw, dtype, cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(x, so, eo.FWD, **kw)
        assert _compare(_fetch(st, out, 0), o, so, 0, True, f"{case} {kw} {dtype} call {t}",
                        own_exact=kw.get("own_exact", False)) == 0


def _random_configs(n, seed=2026):
    """n seeded random configurations: rank count, message size (whole groups,
    often ragged against the 2048-element tiles), group, dtype, betas, and every
    switch at random."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        group = int(rng.choice([32, 64, 128]))
        P = int(rng.integers(1, 17))
        N = group * int(rng.integers(1, 2000))
        out.append(dict(P=P, N=N, group=group, dtype=str(rng.choice(["bf16", "f32"])),
                        compensate=bool(rng.random() < 0.8),
                        beta=(float(np.float32(rng.choice([0.0, 0.25, 0.5, 0.75]))),
                              float(np.float32(rng.choice([0.5, 0.9, 0.95, 0.99])))),
                        sender_feedback=bool(rng.random() < 0.4), state_bf16=bool(rng.random() < 0.4),
                        out_bf16=bool(rng.random() < 0.4), own_exact=bool(rng.random() < 0.4)))
    return out


@pytest.mark.parametrize("k", range(24))
def test_random_configurations(cuda, k):
    """Seeded random combinations of rank count, size, group, dtype, betas and
    the variants, both directions interleaved, against the oracle every call."""
    import error_compensated_bit_echo_amd as E
    c = _random_configs(24)[k]
    P, N, G, dt = c["P"], c["N"], c["group"], c["dtype"]
    kw = {key: c[key] for key in ("sender_feedback", "state_bf16", "out_bf16", "own_exact")}
    st = _state(P, N, dt, c["compensate"], beta=c["beta"], group=G, **kw)
    so = eo.OracleState(N)
    out = _out_tensor(st, cuda)
    for t in range(3):
        for d in (0, 1):
            raw, vals = synth.host_partials("training", d, 10 * k + t, P=P, n=N, dtype=dt)
            E.echo_reduce(_upload(raw, dt, cuda), out, st, d)
            o = eo.echo_call(vals, so, d, compensate=c["compensate"], beta_fast=c["beta"][0],
                             beta_slow=c["beta"][1], group=G, **kw)
            assert _compare(_fetch(st, out, d), o, so, d, c["compensate"], f"{c} call {t} dir {d}",
                            own_exact=kw["own_exact"]) == 0


def test_empty_message_is_a_no_op(cuda):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    st = _state(4, 0, "bf16")
    parts = [torch.empty(0, dtype=torch.bfloat16, device=cuda) for _ in range(4)]
    out = torch.empty(0, dtype=torch.float32, device=cuda)
    E.echo_reduce(parts, out, st, E.ECHO_FWD)
    E.echo_reset(st, 3)
    assert E.echo_wire_bytes(st) == eo.wire_bytes(4, 0)
    torch.cuda.synchronize()


def test_beta_zero_error_feedback(cuda):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P, N = 2, 4096
    st = _state(P, N, "bf16", beta=(0.0, 0.0))
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    for t in range(5):
        raw, vals = synth.host_partials("decode", 0, t, P=P, n=N)
        E.echo_reduce(_upload(raw, "bf16", cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(vals, so, eo.FWD, beta_fast=0.0, beta_slow=0.0)
        assert _compare(_fetch(st, out, 0), o, so, 0, True) == 0


# ---------------------------------------------------------------------------
# state lifecycle: directions, reset, checkpoint/restore, determinism
# ---------------------------------------------------------------------------
def test_directions_reset_checkpoint_and_determinism(cuda):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P, N = 4, 32 * 1000
    st = _state(P, N, "bf16")
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    fw = [synth.host_partials("training", 0, t, P=P, n=N) for t in range(6)]
    bw = [synth.host_partials("training", 1, t, P=P, n=N) for t in range(6)]
    snap = None
    for t in range(6):
        E.echo_reduce(_upload(fw[t][0], "bf16", cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(fw[t][1], so, eo.FWD)
        assert _compare(_fetch(st, out, 0), o, so, 0, True, f"fwd {t}") == 0
        E.echo_reduce(_upload(bw[t][0], "bf16", cuda), out, st, E.ECHO_BWD)
        o = eo.echo_call(bw[t][1], so, eo.BWD)
        assert _compare(_fetch(st, out, 1), o, so, 1, True, f"bwd {t}") == 0
        if t == 2:
            v = E.echo_debug_views(st, E.ECHO_FWD)
            snap = (v["m_fast"].clone(), v["m_slow"].clone(), so.copy())
    # restore the forward state of call 2 and replay calls 3..5: bit-identical
    v = E.echo_debug_views(st, E.ECHO_FWD)
    v["m_fast"].copy_(snap[0])
    v["m_slow"].copy_(snap[1])
    so_r = snap[2]
    for t in range(3, 6):
        E.echo_reduce(_upload(fw[t][0], "bf16", cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(fw[t][1], so_r, eo.FWD)
        assert _compare(_fetch(st, out, 0), o, so_r, 0, True, f"replay {t}") == 0
    # reset of the forward direction only
    E.echo_reset(st, 1)
    v = E.echo_debug_views(st, E.ECHO_FWD)
    vb = E.echo_debug_views(st, E.ECHO_BWD)
    torch.cuda.synchronize()
    assert not torch.any(v["m_fast"]) and not torch.any(v["m_slow"])
    assert np.array_equal(vb["m_fast"].cpu().numpy(), so.m_fast[1])
    # determinism: the same call on the same state twice
    parts = _upload(fw[0][0], "bf16", cuda)
    E.echo_reduce(parts, out, st, E.ECHO_FWD)
    a = out.clone()
    E.echo_reset(st, 1)
    E.echo_reduce(parts, out, st, E.ECHO_FWD)
    assert torch.equal(a, out)


def test_stage_entry_points_equal_reduce(cuda):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P, N = 8, 32 * 4096
    raw, _ = synth.host_partials("decode", 0, 0, P=P, n=N)
    parts = _upload(raw, "bf16", cuda)
    s1, s2 = _state(P, N, "bf16"), _state(P, N, "bf16")
    o1 = torch.empty(N, dtype=torch.float32, device=cuda)
    o2 = torch.empty(N, dtype=torch.float32, device=cuda)
    for _ in range(3):
        E.echo_reduce(parts, o1, s1, E.ECHO_FWD)
        E.echo_stage1(parts, s2)
        E.echo_owner(s2, E.ECHO_FWD)
        E.echo_decode(o2, s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(E.echo_debug_views(s1)["m_slow"], E.echo_debug_views(s2)["m_slow"])


def test_graph_capture_replays_match_eager(cuda):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P, N = 8, 64 * 4096
    raw, _ = synth.host_partials("decode", 0, 0, P=P, n=N)
    parts = _upload(raw, "bf16", cuda)
    se, sg = _state(P, N, "bf16"), _state(P, N, "bf16")
    oe = torch.empty(N, dtype=torch.float32, device=cuda)
    og = torch.empty(N, dtype=torch.float32, device=cuda)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        E.echo_reduce(parts, og, sg, E.ECHO_FWD)
    torch.cuda.synchronize()
    E.echo_reset(sg, 3)  # capture does not execute; start from a fresh state
    for k in range(4):
        E.echo_reduce(parts, oe, se, E.ECHO_FWD)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(oe, og), f"replay {k}"
        _ = (oe * 2).sum().item()  # unrelated eager work between replays


@pytest.mark.parametrize("variant", [{"sender_feedback": True, "state_bf16": True},
                                     {"own_exact": True, "out_bf16": True, "group": 64},
                                     {"sender_feedback": True, "compensate": False}])
def test_graph_capture_of_variants_and_resets(cuda, variant):
    """A graph holding a forward call, a backward call and a reset of the
    backward state, replayed 4 times with eager work in between, leaves the same
    outputs and carried state as the same sequence issued eagerly."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    kw = dict(variant)
    comp = kw.pop("compensate", True)
    P, N = 4, 2048 * 9 + 64 * 3
    raw0, _ = synth.host_partials("training", 0, 1, P=P, n=N)
    raw1, _ = synth.host_partials("training", 1, 1, P=P, n=N)
    p0, p1 = _upload(raw0, "bf16", cuda), _upload(raw1, "bf16", cuda)
    se, sg = _state(P, N, "bf16", comp, **kw), _state(P, N, "bf16", comp, **kw)
    oe, og = _out_tensor(se, cuda), _out_tensor(sg, cuda)
    oe1, og1 = _out_tensor(se, cuda), _out_tensor(sg, cuda)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        E.echo_reduce(p0, og, sg, E.ECHO_FWD)
        E.echo_reduce(p1, og1, sg, E.ECHO_BWD)
        E.echo_reset(sg, 2)
    torch.cuda.synchronize()
    E.echo_reset(sg, 3)  # capture does not execute; start from a fresh state
    for k in range(4):
        E.echo_reduce(p0, oe, se, E.ECHO_FWD)
        E.echo_reduce(p1, oe1, se, E.ECHO_BWD)
        E.echo_reset(se, 2)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(oe, og) and torch.equal(oe1, og1), f"replay {k}"
        for d in (0, 1):
            ve, vg = E.echo_debug_views(se, d), E.echo_debug_views(sg, d)
            for key in ("m_fast", "m_slow", "sender_err"):
                if ve[key] is not None:
                    assert torch.equal(ve[key], vg[key]), f"replay {k} dir {d} {key}"
        _ = (oe * 2).sum().item()  # unrelated eager work between replays


# ---------------------------------------------------------------------------
# argument errors are reported and launch nothing
# ---------------------------------------------------------------------------
def test_argument_errors_launch_nothing(cuda):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P, N = 2, 32 * 64
    st = _state(P, N, "bf16")
    raw, _ = synth.host_partials("tiny", 0, 0, P=P, n=N, dtype="bf16")
    parts = _upload(raw, "bf16", cuda)
    out = torch.zeros(N, dtype=torch.float32, device=cuda)
    E.echo_reduce(parts, out, st, E.ECHO_FWD)
    torch.cuda.synchronize()
    before = st.workspace.clone()
    out_before = out.clone()
    lib = E.load_library()
    import ctypes
    arr = (ctypes.c_void_p * P)(*[t.data_ptr() for t in parts])
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    big = torch.zeros(N + 8, dtype=torch.float32, device=cuda)
    from error_compensated_bit_echo_amd import binding as B
    # misaligned output
    assert lib.echo_reduce(arr, ctypes.c_void_p(big.data_ptr() + 4), st.handle, 0, s) == B.ECHO_ERR_ARG
    # output inside the workspace
    assert lib.echo_reduce(arr, ctypes.c_void_p(st.workspace.data_ptr() + 256), st.handle, 0, s) == B.ECHO_ERR_ARG
    # output overlapping a partial
    assert lib.echo_reduce(arr, ctypes.c_void_p(parts[1].data_ptr()), st.handle, 0, s) == B.ECHO_ERR_ARG
    # a null partial, a misaligned partial, a bad direction, a bad reset mask
    bad = (ctypes.c_void_p * P)(parts[0].data_ptr(), None)
    assert lib.echo_reduce(bad, ctypes.c_void_p(out.data_ptr()), st.handle, 0, s) == B.ECHO_ERR_ARG
    bad = (ctypes.c_void_p * P)(parts[0].data_ptr(), parts[1].data_ptr() + 2)
    assert lib.echo_reduce(bad, ctypes.c_void_p(out.data_ptr()), st.handle, 0, s) == B.ECHO_ERR_ARG
    assert lib.echo_reduce(arr, ctypes.c_void_p(out.data_ptr()), st.handle, 2, s) == B.ECHO_ERR_ARG
    assert lib.echo_owner(None, st.handle, 5, s) == B.ECHO_ERR_ARG
    assert lib.echo_reset(st.handle, 0, s) == B.ECHO_ERR_ARG
    assert lib.echo_reset(st.handle, 4, s) == B.ECHO_ERR_ARG
    # binding-level checks: dtype and count
    with pytest.raises(B.EchoError):
        E.echo_reduce([p.float() for p in parts], out, st)
    with pytest.raises(B.EchoError):
        E.echo_reduce(parts[:1], out, st)
    torch.cuda.synchronize()
    assert torch.equal(before, st.workspace)
    assert torch.equal(out_before, out)


def test_wire_bytes_match_the_oracle(cuda):
    import error_compensated_bit_echo_amd as E
    for P, N in ((2, 2048), (4, 2048 * 4096), (8, 64 * 4096), (3, 32 * 7), (16, 32 * 5)):
        st = _state(P, N, "bf16", poison=False)
        assert E.echo_wire_bytes(st) == eo.wire_bytes(P, N)
    for group in (64, 128):
        for P, N in ((8, 64 * 4096), (3, 128 * 7), (16, 128 * 5)):
            st = _state(P, N, "bf16", poison=False, group=group)
            assert E.echo_wire_bytes(st) == eo.wire_bytes(P, N, group)


# ---------------------------------------------------------------------------
# full-size configurations, in the launch configuration the benchmark uses:
# sampled group-aligned windows (the numerics are independent per group and the
# state per element, so a window of the oracle equals that window of the tensor)
# ---------------------------------------------------------------------------
def _windows(N, n_win, width, seed, align=32):
    rng = np.random.default_rng(seed)
    starts = {0, (N - width) // align * align}
    while len(starts) < n_win:
        starts.add(int(rng.integers(0, (N - width) // align)) * align)
    return sorted(starts)


def _window_segments(N, P, group, w, width):
    """The whole message's owner split, restricted to the window [w, w + width)."""
    lo, hi = w // group, (w + width) // group
    return [(min(max(a, lo), hi) - lo, min(max(b, lo), hi) - lo)
            for a, b in eo.owner_segments(N // group, P)]


def _windowed_run(cuda, workload, calls, directions, same_partials=False, n_win=6, width=1 << 14,
                  P=None, N=None, compensate=True, sender_feedback=False, state_bf16=False,
                  out_bf16=False, own_exact=False, extra_windows=(), group=32, threads=1,
                  sequential=False):
    """The configuration's calls at full size; the oracle checks sampled windows.
    P and N override the configuration's rank count and message size (same
    value distribution and dtype); extra_windows adds group-aligned window starts;
    threads > 1 runs the oracle on the windows in parallel (each has its own state).
    With several directions the calls alternate between them, or, with
    sequential, all calls of the first direction come before the second's (a
    forward pass, then a backward pass)."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    c = synth.WORKLOADS[workload]
    P = c["P"] if P is None else P
    N = synth.numel(workload) if N is None else N
    st = _state(P, N, c["dtype"], compensate=compensate, poison=False, sender_feedback=sender_feedback,
                state_bf16=state_bf16, out_bf16=out_bf16, own_exact=own_exact, group=group)
    out = _out_tensor(st, cuda)
    seed = synth.WORKLOADS[workload]["seed_id"]
    wins = sorted(set(_windows(N, n_win, width, seed, align=group)) | set(extra_windows))
    if own_exact:  # add a window on every segment boundary
        per = eo.owner_segments(N // group, P)
        wins = sorted(set(wins) | {max(0, min(N - width, g0 * group - width // 2)) // group * group
                                   for g0, _ in per[1:]})
    so = {w: eo.OracleState(width) for w in wins}
    parts = None
    order = [(t, d) for d in directions for t in range(calls)] if sequential else \
        [(t, d) for t in range(calls) for d in directions]
    for i, (t, d) in enumerate(order):
        if parts is None or not same_partials:
            parts = None
            parts = synth.device_partials(workload, d, t, P=P, n=N, device=cuda)
        E.echo_reduce(parts, out, st, d)
        torch.cuda.synchronize()

        def check(w):
            host = np.stack([p[w:w + width].float().cpu().numpy() for p in parts])
            o = eo.echo_call(host, so[w], d, compensate=compensate, sender_feedback=sender_feedback,
                             state_bf16=state_bf16, out_bf16=out_bf16, own_exact=own_exact, group=group,
                             segments=_window_segments(N, P, group, w, width) if own_exact else None)
            g = _fetch(st, out, d, w, w + width)
            return _compare(g, o, so[w], d, compensate,
                            f"{workload} P={P} N={N} call {t} dir {d} window {w}", own_exact)

        if threads > 1:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(max_workers=threads) as ex:
                assert sum(ex.map(check, wins)) == 0
        else:
            assert sum(check(w) for w in wins) == 0
        if i + 1 == len(order) or order[i + 1][0] != t:
            print(f"{workload} P={P} N={N}: call {t} ok", flush=True)


def test_prefill_config_full_size(cuda):
    """All 72 calls (36 layers, attention and MLP) of the prefill workload on one
    forward state, sampled windows after every call."""
    _windowed_run(cuda, "prefill", synth.WORKLOADS["prefill"]["calls"], (0,))


def test_training_config_full_size(cuda):
    """A training step: the 56 forward calls on the forward state, then the 56
    backward calls on the backward state."""
    _windowed_run(cuda, "training", synth.WORKLOADS["training"]["calls"], (0, 1), sequential=True)


def test_training_config_full_size_interleaved(cuda):
    """The same 56 + 56 calls with the directions alternating call by call."""
    _windowed_run(cuda, "training", synth.WORKLOADS["training"]["calls"], (0, 1))


def test_headline_config_full_size(cuda):
    """All 10 calls of the 1 GiB P = 8 message, 16 group-aligned windows of 2^20
    elements (the first, the last and 14 random ones) checked after every call."""
    calls = synth.WORKLOADS["headline_1GiB"]["calls"]
    _windowed_run(cuda, "headline_1GiB", calls, (0,), same_partials=True, n_win=16, width=1 << 20, threads=16)


def test_headline_config_every_group_of_the_first_two_calls(cuda):
    """1 GiB bf16 per rank, P = 8, the same partials every call: after each of the
    first two calls every group of the message is checked (both payloads, the
    output and both estimates), the oracle running on 16 threads over
    independent windows of 2^23 elements, each with its own state."""
    from concurrent.futures import ThreadPoolExecutor

    import error_compensated_bit_echo_amd as E
    torch = _torch()
    workload = "headline_1GiB"
    c = synth.WORKLOADS[workload]
    P, N = c["P"], synth.numel(workload)
    W = 1 << 23
    st = _state(P, N, c["dtype"], poison=False)
    out = _out_tensor(st, cuda)
    parts = synth.device_partials(workload, 0, 0, device=cuda)
    so = {w: eo.OracleState(W) for w in range(0, N, W)}

    def check(w, t):
        host = np.stack([p[w:w + W].float().cpu().numpy() for p in parts])
        o = eo.echo_call(host, so[w], 0)
        g = _fetch(st, out, 0, w, w + W)
        return _compare(g, o, so[w], 0, True, f"call {t} window {w}")

    for t in range(2):
        E.echo_reduce(parts, out, st, E.ECHO_FWD)
        torch.cuda.synchronize()
        with ThreadPoolExecutor(max_workers=16) as ex:
            inexact = sum(ex.map(lambda w: check(w, t), sorted(so)))
        assert inexact == 0
        print(f"call {t}: all {N // 32} groups ok", flush=True)


def _full_run(cuda, workload, calls, directions, W=1 << 21, **variant):
    """The configuration's first calls at full size, every group checked after each
    call: the oracle runs on 16 threads over the windows of W elements that tile
    the message, each with its own state (given the whole message's owner split
    when the owners keep their own shares)."""
    from concurrent.futures import ThreadPoolExecutor

    import error_compensated_bit_echo_amd as E
    torch = _torch()
    c = synth.WORKLOADS[workload]
    P, N = c["P"], synth.numel(workload)
    assert N % W == 0
    st = _state(P, N, c["dtype"], poison=False, **variant)
    out = _out_tensor(st, cuda)
    so = {w: eo.OracleState(W) for w in range(0, N, W)}
    own = variant.get("own_exact", False)
    group = variant.get("group", 32)
    for t in range(calls):
        for d in directions:
            parts = synth.device_partials(workload, d, t, device=cuda)
            E.echo_reduce(parts, out, st, d)
            torch.cuda.synchronize()

            def check(w):
                host = np.stack([p[w:w + W].float().cpu().numpy() for p in parts])
                o = eo.echo_call(host, so[w], d, segments=_window_segments(N, P, group, w, W) if own else None,
                                 **variant)
                return _compare(_fetch(st, out, d, w, w + W), o, so[w], d, True,
                                f"{workload} call {t} dir {d} window {w}", own)

            with ThreadPoolExecutor(max_workers=16) as ex:
                assert sum(ex.map(check, sorted(so))) == 0
            print(f"{workload} call {t} dir {d}: all {N // group} groups ok", flush=True)


def test_prefill_config_every_group(cuda):
    _full_run(cuda, "prefill", 3, (0,))


def test_training_config_every_group_interleaved(cuda):
    _full_run(cuda, "training", 2, (0, 1))


def test_prefill_config_every_group_with_variants(cuda):
    _full_run(cuda, "prefill", 3, (0,), own_exact=True, out_bf16=True, state_bf16=True)


@pytest.mark.parametrize("P,N", [(4, 14 << 20), (2, 25 << 20), (8, 26 << 20), (8, 29 << 20)])
def test_cache_policy_boundaries(cuda, P, N):
    """Message sizes on both sides of the cache-policy switches at 480 MB and
    1.2 GB per call (466 MB all plain; 695 MB and 1.15 GB with the partials
    streamed in; 1.28 GB streaming), three calls, sampled windows."""
    _windowed_run(cuda, "training", 3, (0,), P=P, N=N, n_win=6, width=1 << 16)


def test_largest_rank_count_large_message(cuda):
    """P = 16 (the most ranks the library takes), 2^27 bf16 elements per rank."""
    _windowed_run(cuda, "headline_1GiB", 3, (0,), P=16, N=1 << 27, n_win=8, width=1 << 14)


def test_fp32_partials_of_2GiB(cuda):
    """fp32 partials of 2^29 elements (2 GiB each, so byte offsets pass 2^31)."""
    _windowed_run(cuda, "tiny", 3, (0,), P=2, N=1 << 29, n_win=8, width=1 << 14)


@pytest.mark.parametrize("group", [64, 128])
def test_larger_groups_full_size(cuda, group):
    """The group-size variants at the prefill size, where every kernel takes its
    two-chunks-per-lane launch (small messages take one)."""
    _windowed_run(cuda, "prefill", 4, (0,), group=group)


def test_full_size_without_compensation(cuda):
    """The plain two-rounding all-reduce (state untouched) at the prefill size."""
    _windowed_run(cuda, "prefill", 4, (0,), compensate=False)


# ---------------------------------------------------------------------------
# sender-side error feedback (a variant): every rank feeds its own stage-1
# rounding error into its next call
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("compensate", [True, False])
def test_sender_feedback_tiny_config_every_call(cuda, compensate):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    c = synth.WORKLOADS["tiny"]
    P, N = c["P"], synth.numel("tiny")
    st = _state(P, N, "f32", compensate, sender_feedback=True)
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    for t in range(c["calls"]):
        raw, vals = synth.host_partials("tiny", 0, t)
        E.echo_reduce(_upload(raw, "f32", cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(vals, so, eo.FWD, compensate=compensate, sender_feedback=True)
        assert _compare(_fetch(st, out, 0), o, so, 0, compensate, f"call {t}") == 0


@pytest.mark.parametrize("P,dtype,group", [(1, "bf16", 32), (3, "f32", 32), (8, "bf16", 32),
                                           (16, "bf16", 64), (4, "bf16", 128)])
def test_sender_feedback_multi_tile_both_directions(cuda, P, dtype, group):
    """Ragged tiles, tie-rich and normal data, forward and backward calls
    interleaved (separate sender errors per direction), a forward reset midway."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    N = 2048 * 5 + group * 3
    st = _state(P, N, dtype, group=group, sender_feedback=True)
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    rng = np.random.default_rng(P * 1000 + group)
    for t in range(6):
        if t == 3:
            E.echo_reset(st, 1)
            so.reset(1)
        for d in (0, 1):
            if (t + d) % 2:
                vals = (rng.integers(-12, 13, (P, N)) * 0.25).astype(F32)
                raw = vals if dtype == "f32" else synth.f32_to_bf16_bits(vals)
            else:
                raw, vals = synth.host_partials("training", d, t, P=P, n=N, dtype=dtype)
            E.echo_reduce(_upload(raw, dtype, cuda), out, st, d)
            o = eo.echo_call(vals, so, d, group=group, sender_feedback=True)
            assert _compare(_fetch(st, out, d), o, so, d, True, f"G={group} P={P} call {t} dir {d}") == 0


def test_sender_feedback_stage_entry_points_equal_reduce(cuda):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P, N = 8, 32 * 4096
    raw, _ = synth.host_partials("decode", 0, 0, P=P, n=N)
    parts = _upload(raw, "bf16", cuda)
    s1 = _state(P, N, "bf16", sender_feedback=True)
    s2 = _state(P, N, "bf16", sender_feedback=True)
    o1 = torch.empty(N, dtype=torch.float32, device=cuda)
    o2 = torch.empty(N, dtype=torch.float32, device=cuda)
    for d in (0, 1, 1, 0):
        E.echo_reduce(parts, o1, s1, d)
        E.echo_stage1(parts, s2, d)
        E.echo_owner(s2, d)
        E.echo_decode(o2, s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for d in (0, 1):
        assert torch.equal(E.echo_debug_views(s1, d)["sender_err"], E.echo_debug_views(s2, d)["sender_err"])


def test_sender_feedback_full_size(cuda):
    _windowed_run(cuda, "prefill", 4, (0,), sender_feedback=True)


# ---------------------------------------------------------------------------
# bf16 compensator state (a variant): every estimate update rounded to bf16
# ---------------------------------------------------------------------------
def test_bf16_state_tiny_config_every_call(cuda):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    c = synth.WORKLOADS["tiny"]
    P, N = c["P"], synth.numel("tiny")
    st = _state(P, N, "f32", state_bf16=True)
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    for t in range(c["calls"]):
        raw, vals = synth.host_partials("tiny", 0, t)
        E.echo_reduce(_upload(raw, "f32", cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(vals, so, eo.FWD, state_bf16=True)
        assert _compare(_fetch(st, out, 0), o, so, 0, True, f"call {t}") == 0


@pytest.mark.parametrize("P,dtype,group,sfb", [(2, "bf16", 32, False), (5, "f32", 32, False),
                                               (8, "bf16", 64, False), (4, "bf16", 32, True),
                                               (16, "bf16", 128, True)])
def test_bf16_state_multi_tile_both_directions(cuda, P, dtype, group, sfb):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    N = 2048 * 5 + group * 3
    st = _state(P, N, dtype, group=group, sender_feedback=sfb, state_bf16=True)
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    rng = np.random.default_rng(P * 100 + group)
    for t in range(5):
        for d in (0, 1):
            if (t + d) % 2:
                vals = (rng.integers(-12, 13, (P, N)) * 0.25).astype(F32)
                raw = vals if dtype == "f32" else synth.f32_to_bf16_bits(vals)
            else:
                raw, vals = synth.host_partials("training", d, t, P=P, n=N, dtype=dtype)
            E.echo_reduce(_upload(raw, dtype, cuda), out, st, d)
            o = eo.echo_call(vals, so, d, group=group, sender_feedback=sfb, state_bf16=True)
            assert _compare(_fetch(st, out, d), o, so, d, True,
                            f"G={group} P={P} sfb={sfb} call {t} dir {d}") == 0


def test_sender_feedback_bf16_state_headline_size(cuda):
    """1 GiB bf16 per rank, P = 8 (streaming cache policy), sender feedback with
    the bf16 state: three calls on the same partials, sampled windows."""
    _windowed_run(cuda, "headline_1GiB", 3, (0,), same_partials=True, n_win=6, width=1 << 16, sender_feedback=True,
                  state_bf16=True, threads=6)


@pytest.mark.parametrize("sfb", [False, True])
def test_bf16_state_full_size(cuda, sfb):
    """Prefill size; with sender feedback the ranks' stage-1 errors are bf16 too."""
    _windowed_run(cuda, "prefill", 6, (0,), state_bf16=True, sender_feedback=sfb)


# ---------------------------------------------------------------------------
# bfloat16 output (a variant): out = bf16(B), the error measured against it
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("compensate", [True, False])
def test_bf16_output_tiny_config_every_call(cuda, compensate):
    import error_compensated_bit_echo_amd as E
    c = synth.WORKLOADS["tiny"]
    P, N = c["P"], synth.numel("tiny")
    st = _state(P, N, "f32", compensate, out_bf16=True)
    so = eo.OracleState(N)
    out = _out_tensor(st, cuda)
    for t in range(c["calls"]):
        raw, vals = synth.host_partials("tiny", 0, t)
        E.echo_reduce(_upload(raw, "f32", cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(vals, so, eo.FWD, compensate=compensate, out_bf16=True)
        assert _compare(_fetch(st, out, 0), o, so, 0, compensate, f"call {t}") == 0


@pytest.mark.parametrize("P,dtype,group,sfb,sb16", [(1, "bf16", 32, False, False), (3, "f32", 32, False, False),
                                                    (8, "bf16", 32, False, False), (16, "bf16", 64, True, False),
                                                    (4, "f32", 128, False, True), (8, "bf16", 32, True, True)])
def test_bf16_output_multi_tile_both_directions(cuda, P, dtype, group, sfb, sb16):
    import error_compensated_bit_echo_amd as E
    N = 2048 * 5 + group * 3
    st = _state(P, N, dtype, group=group, sender_feedback=sfb, state_bf16=sb16, out_bf16=True)
    so = eo.OracleState(N)
    out = _out_tensor(st, cuda)
    rng = np.random.default_rng(P * 10 + group)
    for t in range(5):
        for d in (0, 1):
            if (t + d) % 2:
                vals = (rng.integers(-12, 13, (P, N)) * 0.25).astype(F32)
                raw = vals if dtype == "f32" else synth.f32_to_bf16_bits(vals)
            else:
                raw, vals = synth.host_partials("training", d, t, P=P, n=N, dtype=dtype)
            E.echo_reduce(_upload(raw, dtype, cuda), out, st, d)
            o = eo.echo_call(vals, so, d, group=group, sender_feedback=sfb, state_bf16=sb16, out_bf16=True)
            assert _compare(_fetch(st, out, d), o, so, d, True,
                            f"G={group} P={P} sfb={sfb} sb16={sb16} call {t} dir {d}") == 0


def test_bf16_output_full_size(cuda):
    _windowed_run(cuda, "prefill", 6, (0,), out_bf16=True)


# ---------------------------------------------------------------------------
# the owner adds its own partial exactly (a variant)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("compensate", [True, False])
def test_own_exact_tiny_config_every_call(cuda, compensate):
    import error_compensated_bit_echo_amd as E
    c = synth.WORKLOADS["tiny"]
    P, N = c["P"], synth.numel("tiny")
    st = _state(P, N, "f32", compensate, own_exact=True)
    so = eo.OracleState(N)
    out = _out_tensor(st, cuda)
    for t in range(c["calls"]):
        raw, vals = synth.host_partials("tiny", 0, t)
        E.echo_reduce(_upload(raw, "f32", cuda), out, st, E.ECHO_FWD)
        o = eo.echo_call(vals, so, eo.FWD, compensate=compensate, own_exact=True)
        assert _compare(_fetch(st, out, 0), o, so, 0, compensate, f"call {t}", own_exact=True) == 0


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_own_exact_multi_tile_ragged(cuda, P, dtype):
    """Segment boundaries that fall inside tiles, a ragged tail, both directions."""
    import error_compensated_bit_echo_amd as E
    N = 32 * (64 * 3 + 37) * 8 + 32 * 5
    st = _state(P, N, dtype, own_exact=True)
    so = eo.OracleState(N)
    out = _out_tensor(st, cuda)
    for t in range(3):
        for d in (0, 1):
            raw, vals = synth.host_partials("prefill", d, t, P=P, n=N, dtype=dtype)
            E.echo_reduce(_upload(raw, dtype, cuda), out, st, d)
            o = eo.echo_call(vals, so, d, own_exact=True)
            assert _compare(_fetch(st, out, d), o, so, d, True, f"P={P} {dtype} call {t} dir {d}",
                            own_exact=True) == 0


@pytest.mark.parametrize("P,dtype,group,sfb,comp,sb16,obf", [
    (4, "bf16", 64, False, True, False, False), (3, "f32", 128, False, True, False, False),
    (8, "bf16", 32, True, True, False, False), (16, "f32", 64, True, False, False, False),
    (5, "bf16", 32, False, False, False, True), (8, "bf16", 32, True, True, True, True)])
def test_own_exact_with_other_variants(cuda, P, dtype, group, sfb, comp, sb16, obf):
    import error_compensated_bit_echo_amd as E
    N = 2048 * 5 + group * 3
    st = _state(P, N, dtype, comp, group=group, sender_feedback=sfb, state_bf16=sb16, out_bf16=obf,
                own_exact=True)
    so = eo.OracleState(N)
    out = _out_tensor(st, cuda)
    rng = np.random.default_rng(P * 7 + group)
    for t in range(5):
        for d in (0, 1):
            if (t + d) % 2:
                vals = (rng.integers(-12, 13, (P, N)) * 0.25).astype(F32)
                raw = vals if dtype == "f32" else synth.f32_to_bf16_bits(vals)
            else:
                raw, vals = synth.host_partials("training", d, t, P=P, n=N, dtype=dtype)
            E.echo_reduce(_upload(raw, dtype, cuda), out, st, d)
            o = eo.echo_call(vals, so, d, compensate=comp, group=group, sender_feedback=sfb,
                             state_bf16=sb16, out_bf16=obf, own_exact=True)
            assert _compare(_fetch(st, out, d), o, so, d, comp,
                            f"G={group} P={P} sfb={sfb} comp={comp} call {t} dir {d}", own_exact=True) == 0


@pytest.mark.parametrize("P,N", [(8, 96), (16, 32 * 20), (3, 32), (4, 32 * 5)])
def test_own_exact_fewer_groups_than_owners(cuda, P, N):
    """Owners with empty segments (ceil split): ranks past the last group skip nothing."""
    import error_compensated_bit_echo_amd as E
    st = _state(P, N, "bf16", own_exact=True)
    so = eo.OracleState(N)
    out = _out_tensor(st, cuda)
    for t in range(3):
        raw, vals = synth.host_partials("prefill", 0, t, P=P, n=N)
        E.echo_reduce(_upload(raw, "bf16", cuda), out, st, 0)
        o = eo.echo_call(vals, so, 0, own_exact=True)
        assert _compare(_fetch(st, out, 0), o, so, 0, True, f"P={P} N={N} call {t}", own_exact=True) == 0


def test_own_exact_stage_entry_points_and_graph(cuda):
    """Stage by stage (the owner given the partials) equals echo_reduce; a captured
    graph replays like eager calls; the owner stage needs the partials."""
    import ctypes
    import error_compensated_bit_echo_amd as E
    from error_compensated_bit_echo_amd import binding as B
    torch = _torch()
    P, N = 8, 64 * 4096 + 32 * 3
    raw, _ = synth.host_partials("decode", 0, 0, P=P, n=N)
    parts = _upload(raw, "bf16", cuda)
    kw = dict(own_exact=True, out_bf16=True)
    s1, s2, sg = _state(P, N, "bf16", **kw), _state(P, N, "bf16", **kw), _state(P, N, "bf16", **kw)
    o1, o2, og = _out_tensor(s1, cuda), _out_tensor(s2, cuda), _out_tensor(sg, cuda)
    for d in (0, 1, 1, 0):
        E.echo_reduce(parts, o1, s1, d)
        E.echo_stage1(parts, s2, d)
        E.echo_owner(s2, d, partials=parts)
        E.echo_decode(o2, s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for d in (0, 1):
        assert torch.equal(E.echo_debug_views(s1, d)["m_slow"], E.echo_debug_views(s2, d)["m_slow"])
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert E.load_library().echo_owner(None, s2.handle, 0, s) == B.ECHO_ERR_ARG
    # graph capture
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        E.echo_reduce(parts, og, sg, E.ECHO_FWD)
    torch.cuda.synchronize()
    E.echo_reset(sg, 3)
    E.echo_reset(s1, 3)
    for k in range(3):
        E.echo_reduce(parts, o1, s1, E.ECHO_FWD)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o1, og), f"replay {k}"
        _ = (o1.float() * 2).sum().item()


def test_own_exact_full_size(cuda):
    _windowed_run(cuda, "prefill", 6, (0,), own_exact=True)


def test_own_exact_headline_size(cuda):
    """1 GiB bf16 per rank, P = 8, the same partials every call."""
    _windowed_run(cuda, "headline_1GiB", 4, (0,), same_partials=True, n_win=6, width=1 << 14, own_exact=True)


def test_element_indices_beyond_2_32(cuda):
    """N = 2^32 + 96 elements per rank (P = 2; bf16 state and output and the owners'
    own shares keep the footprint near 65 GB): element, chunk and scale indices
    pass 2^32, 2^29 and 2^27, byte offsets pass 2^33.  Windows at both ends (the
    last one spans element 2^32), on the owner boundary and just below 2^32."""
    N, width = (1 << 32) + 96, 1 << 13
    _windowed_run(cuda, "headline_1GiB", 2, (0,), P=2, N=N, n_win=4, width=width, state_bf16=True,
                  out_bf16=True, own_exact=True, extra_windows=((1 << 32) - 2 * width,))


def test_independent_states_on_two_streams(cuda):
    """Two states with different configurations, driven on two streams at once,
    give exactly what each gives alone: the library keeps no state of its own."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P1, N1, P2, N2 = 8, 32 * 4096 * 3, 3, 64 * 1024 + 192
    raw1, _ = synth.host_partials("decode", 0, 0, P=P1, n=N1)
    raw2, _ = synth.host_partials("prefill", 1, 0, P=P2, n=N2, dtype="f32")
    p1, p2 = _upload(raw1, "bf16", cuda), _upload(raw2, "f32", cuda)
    cfg = [dict(P=P1, N=N1, dtype="bf16", kw=dict(own_exact=True)),
           dict(P=P2, N=N2, dtype="f32", kw=dict(state_bf16=True, out_bf16=True, group=64))]

    def run(streams):
        sts = [_state(c["P"], c["N"], c["dtype"], **c["kw"]) for c in cfg]
        outs = [_out_tensor(st, cuda) for st in sts]
        torch.cuda.synchronize()
        for t in range(4):
            for i, (st, parts) in enumerate(zip(sts, (p1, p2))):
                s = streams[i]
                with torch.cuda.stream(s):
                    E.echo_reduce(parts, outs[i], st, t % 2, stream=s)
        torch.cuda.synchronize()
        return [o.clone() for o in outs], [E.echo_debug_views(st, 0)["m_slow"].clone() for st in sts]

    cur = torch.cuda.current_stream()
    alone = run([cur, cur])
    both = run([torch.cuda.Stream(), torch.cuda.Stream()])
    for a, b in zip(alone[0] + alone[1], both[0] + both[1]):
        assert torch.equal(a, b)


def test_states_driven_from_two_host_threads(cuda):
    """Two host threads, each with its own state and stream, calling the C ABI at
    the same time, give what the same calls give from one thread."""
    import threading

    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P, N = 4, 2048 * 17 + 96
    parts = [_upload(synth.host_partials("training", d, 3, P=P, n=N)[0], "bf16", cuda) for d in (0, 1)]

    def drive(st, out, stream, dirs, log):
        torch.cuda.set_device(cuda)
        with torch.cuda.stream(stream):
            for t in range(20):
                d = dirs[t % len(dirs)]
                E.echo_reduce(parts[d], out, st, d, stream=stream)
                if t % 5 == 4:
                    E.echo_reset(st, 1 << d, stream=stream)
            stream.synchronize()
        log.append(out.clone())

    def run(threaded):
        sts = [_state(P, N, "bf16", sender_feedback=True), _state(P, N, "bf16", state_bf16=True)]
        outs = [_out_tensor(st, cuda) for st in sts]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        logs = [[], []]
        torch.cuda.synchronize()
        args = [(sts[i], outs[i], streams[i], (0, 1) if i == 0 else (1,), logs[i]) for i in range(2)]
        if threaded:
            ths = [threading.Thread(target=drive, args=a) for a in args]
            for th in ths:
                th.start()
            for th in ths:
                th.join()
        else:
            for a in args:
                drive(*a)
        torch.cuda.synchronize()
        views = [[E.echo_debug_views(st, d)[k].clone() for d in (0, 1) for k in ("m_fast", "m_slow")]
                 for st in sts]
        return [lg[0] for lg in logs], views

    seq, par = run(False), run(True)
    for a, b in zip(seq[0], par[0]):
        assert torch.equal(a, b)
    for va, vb in zip(seq[1], par[1]):
        for a, b in zip(va, vb):
            assert torch.equal(a, b)
