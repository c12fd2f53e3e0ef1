"""CPU pins of the oracle: each checks it against something other than itself.

Brute force in exact rationals, hand-worked golden values, closed forms of the
compensator, special cases that reduce to textbook routines, and invariants
that the pages state (at most two roundings per element; a payload of about a
quarter of the 16-bit bytes; an accumulated error that stays bounded with
compensation and grows without it).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import echo_oracle as eo
from oracle import exact as ex
from error_compensated_bit_echo_amd import synth

F32 = np.float32
F64 = np.float64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fr(a):
    return [Fraction(float(t)) for t in np.asarray(a, F32).reshape(-1)]


def _as_f32(frs):
    return np.array([float(t) for t in frs], dtype=F32)


# ---------------------------------------------------------------------------
# binary32 rounding of the exact checker vs the library cast
# ---------------------------------------------------------------------------
def test_exact_rounding_matches_float64_to_float32_cast():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-45, 38, 3000))
    # exact midpoints between neighbouring binary32 values, including subnormals
    for f in [F32(1.0), F32(3.1), F32(1e-39), F32(2.0 ** -149), F32(1e-45) * 5, F32(3e38)]:
        nxt = np.nextafter(f, F32(np.inf))
        vals.append((F64(f) + F64(nxt)) / 2)
        vals.append(-(F64(f) + F64(nxt)) / 2)
    for v in vals:
        v = F64(v)
        want = F32(v)
        if not np.isfinite(want):
            continue
        got = ex.round_to_binary32(Fraction(float(v)))
        assert float(got) == float(want), (v, got, want)


# ---------------------------------------------------------------------------
# P1: the quantizer against brute force in exact rationals
# ---------------------------------------------------------------------------
def _tie_groups(rng, n_groups, group=32):
    """Groups whose scale is exact and whose members are exact half-integer ties."""
    groups = []
    for _ in range(n_groups):
        m = int(rng.integers(1, 2 ** 12)) | 1
        e = int(rng.integers(-20, 20))
        s = F64(m) * 2.0 ** e
        g = np.empty(group, F64)
        g[0] = 7 * s * (1 if rng.random() < 0.5 else -1)
        k = rng.integers(-7, 7, group - 1)
        half = rng.random(group - 1) < 0.7
        g[1:] = (k + np.where(half, 0.5, 0.0)) * s
        g = g.astype(F32)
        assert np.all(g.astype(F64) == np.concatenate([[g[0]], (k + np.where(half, 0.5, 0.0)) * s]))
        groups.append(g)
    return np.concatenate(groups)


@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("kind", ["normal", "tiny", "huge", "ties", "subnormal", "sparse"])
def test_quantizer_matches_brute_force(kind, group):
    rng = np.random.default_rng({"normal": 1, "tiny": 2, "huge": 3, "ties": 4,
                                 "subnormal": 5, "sparse": 6}[kind] + group)
    n = group * 24
    if kind == "normal":
        v = rng.standard_normal(n).astype(F32)
    elif kind == "tiny":
        v = (rng.standard_normal(n) * 1e-30).astype(F32)
    elif kind == "huge":
        v = (rng.standard_normal(n) * 1e30).astype(F32)
    elif kind == "ties":
        v = _tie_groups(rng, 24, group)
    elif kind == "subnormal":
        v = (rng.integers(-80, 80, n) * 2.0 ** -149).astype(F32)
        v[:group] = (rng.integers(-3, 4, group) * 2.0 ** -149).astype(F32)  # s underflows to 0
    else:
        v = rng.standard_normal(n).astype(F32)
        v[rng.random(n) < 0.8] = 0
        v[:group] = 0
        v[group:2 * group] = -0.0
    q, s = eo.quantize_groups(v, group)
    qx, sx = ex.quantize(_fr(v), group)
    assert np.array_equal(q.reshape(-1), np.array(qx, np.int8))
    assert np.array_equal(s, _as_f32(sx))
    # the scale is the binary32 quotient of the group absmax by 7
    a = np.max(np.abs(v.reshape(-1, group)), axis=1)
    assert np.array_equal(s, _as_f32([ex.div(Fraction(float(t)), Fraction(7)) for t in a]))


def test_quantizer_subnormal_saturation_is_nearest_code():
    # a = 10 * 2**-149 gives s = fl(10/7 * 2**-149) = 2**-149, so a/s = 10 > 7.5:
    # the nearest admissible code is 7.
    v = np.zeros(32, F32)
    v[0] = F32(10 * 2.0 ** -149)
    v[1] = -F32(9 * 2.0 ** -149)
    q, s = eo.quantize_groups(v)
    assert s[0] == F32(2.0 ** -149)
    assert q[0, 0] == 7 and q[0, 1] == -7
    qx, _ = ex.quantize(_fr(v))
    assert qx[0] == 7 and qx[1] == -7


# ---------------------------------------------------------------------------
# P2: hand-worked tie table and special cases
# ---------------------------------------------------------------------------
def _load_ties():
    rows = []
    with open(os.path.join(GOLDEN, "quantizer_ties.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((F32(float(a)), int(b)))
    return rows


def test_quantizer_tie_table_golden():
    rows = _load_ties()
    for val, want in rows:
        g = np.zeros(32, F32)
        g[0] = F32(7.0)
        g[1] = val
        q, s = eo.quantize_groups(g)
        assert s[0] == F32(1.0)
        assert q[0, 1] == want, (val, q[0, 1], want)


def test_quantizer_special_cases():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(32 * 64).astype(F32)
    q, s = eo.quantize_groups(v)
    g = v.reshape(-1, 32)
    # the absmax element always maps to +-7
    idx = np.argmax(np.abs(g), axis=1)
    assert np.all(np.abs(q[np.arange(len(idx)), idx]) == 7)
    # every value is within half a step of its code
    err = np.abs(g.astype(F64) - q.astype(F64) * s.astype(F64)[:, None])
    assert np.all(err <= s.astype(F64)[:, None] / 2)
    # a zero group has a zero scale and zero codes
    z, zs = eo.quantize_groups(np.zeros(32, F32))
    assert zs[0] == 0 and not np.any(z)


# ---------------------------------------------------------------------------
# P3: the measured error is exact and bounded
# ---------------------------------------------------------------------------
def test_error_is_exact_and_bounded():
    st = eo.OracleState(2048)
    for t in range(8):
        _, x = synth.host_partials("tiny", 0, t)
        o = eo.echo_call(x, st)
        V, B, r = o["V"].astype(F64), o["B"].astype(F64), o["r"].astype(F64)
        assert np.array_equal(r + B, V)
        s2 = np.repeat(o["scales2"].astype(F64), 32)
        ulpB = np.spacing(np.abs(o["B"])).astype(F64)
        assert np.all(np.abs(r) <= s2 / 2 + ulpB / 2)


# ---------------------------------------------------------------------------
# P4: payload layout and byte counts
# ---------------------------------------------------------------------------
def test_nibble_layout_golden():
    with open(os.path.join(GOLDEN, "nibble_layout.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split("|")
            codes = np.array([int(t) for t in a.split()], np.int8)
            want = bytes.fromhex(b.replace(" ", ""))
            got = eo.pack_nibbles(codes).tobytes()
            assert got == want
            assert np.array_equal(eo.unpack_nibbles(np.frombuffer(want, np.uint8)), codes)


def test_payload_is_about_a_quarter_of_bf16():
    for N in (2048, 4096 * 2048, 536870912):
        assert eo.payload_bytes(N) == N // 2 + N // 8
        assert eo.payload_bytes(N) / (2 * N) == 0.3125
    for P, N in ((2, 2048), (4, 4096 * 2048), (8, 536870912), (8, 262144)):
        w = eo.wire_bytes(P, N)
        assert w["rs_per_rank"] == (P - 1) * eo.payload_bytes(N) // P
        assert w["ag_per_rank"] == (P - 1) * eo.payload_bytes(N) // P
        assert (w["rs_per_rank"] + w["ag_per_rank"]) / w["bf16_allreduce_per_rank"] == 0.3125
    # ragged segments: every group owned exactly once
    for n_g, P in ((1, 8), (7, 3), (100, 16), (64, 2)):
        segs = eo.owner_segments(n_g, P)
        owned = np.zeros(n_g, int)
        for lo, hi in segs:
            owned[lo:hi] += 1
        assert np.all(owned == 1)
    o = eo.echo_call(np.zeros((3, 64), F32), eo.OracleState(64))
    assert o["codes2"].nbytes + o["scales2"].nbytes == eo.payload_bytes(64)
    # larger groups (variants): one fp32 scale per 64 or 128 elements
    for group, ratio in ((64, 0.28125), (128, 0.265625)):
        N = 128 * 1024
        assert eo.payload_bytes(N, group) == N // 2 + 4 * N // group
        assert eo.payload_bytes(N, group) / (2 * N) == ratio
        o = eo.echo_call(np.ones((2, N), F32), eo.OracleState(N), group=group)
        assert o["codes2"].nbytes + o["scales2"].nbytes == eo.payload_bytes(N, group)
        w = eo.wire_bytes(8, N, group)
        assert w["rs_per_rank"] == 7 * eo.payload_bytes(N, group) // 8


# ---------------------------------------------------------------------------
# P5: closed form of the compensator
# ---------------------------------------------------------------------------
def _run(T, compensate, P=2, N=2048, workload="tiny", same=False, beta_fast=0.5, beta_slow=0.95):
    st = eo.OracleState(N)
    outs = []
    for t in range(T):
        _, x = synth.host_partials(workload, 0, 0 if same else t, P=P, n=N)
        outs.append(eo.echo_call(x, st, compensate=compensate,
                                 beta_fast=beta_fast, beta_slow=beta_slow))
    return outs


def test_compensator_closed_form():
    T = 200
    outs = _run(T, True)
    r = np.stack([o["r"].astype(F64) for o in outs])          # [T, N]
    D = np.cumsum(np.stack([o["B"].astype(F64) - o["S"].astype(F64) for o in outs]), 0)
    bf, bs = F64(F32(0.5)), F64(F32(0.95))
    k = 0.5 * (bf ** np.arange(T) + bs ** np.arange(T))
    for Tq in (1, 2, 10, 50, 200):
        pred = -np.sum(k[:Tq, None] * r[Tq - 1::-1], axis=0)
        assert np.max(np.abs(D[Tq - 1] - pred)) < 1e-4 * np.max(np.abs(r))
        assert np.max(np.abs(D[Tq - 1])) <= 11 * np.max(np.abs(r))


def test_error_feedback_special_case_beta_zero():
    # beta = 0 is classic error feedback: the sum of injected errors telescopes
    outs = _run(30, True, beta_fast=0.0, beta_slow=0.0)
    D = sum(o["B"].astype(F64) - o["S"].astype(F64) for o in outs)
    r_last = outs[-1]["r"].astype(F64)
    scale = np.max(np.abs(np.stack([o["S"] for o in outs])))
    assert np.max(np.abs(D + r_last)) < 30 * 2.0 ** -23 * scale


def test_no_compensation_grows_linearly_on_repeated_input():
    off = _run(40, False, same=True)
    e1 = off[0]["B"].astype(F64) - off[0]["S"].astype(F64)
    D = np.zeros_like(e1)
    for t, o in enumerate(off, 1):
        D += o["B"].astype(F64) - o["S"].astype(F64)
        assert np.array_equal(D, t * e1) or np.allclose(D, t * e1, rtol=0, atol=1e-12)
    on = _run(40, True, same=True)
    Don = sum(o["B"].astype(F64) - o["S"].astype(F64) for o in on)
    rmax = max(np.max(np.abs(o["r"])) for o in on)
    assert np.max(np.abs(Don)) <= 11 * rmax
    assert np.sqrt(np.mean(D ** 2)) > 5 * np.sqrt(np.mean(Don ** 2))


def test_single_rank_without_compensation_is_idempotent():
    _, x = synth.host_partials("tiny", 0, 0, P=1, n=4096)
    o = eo.echo_call(x, None, compensate=False)
    assert np.array_equal(o["q1"][0], o["q2"])
    s1, s2 = o["scales1"][0], o["scales2"]
    assert np.all(np.abs(s2.astype(F64) - s1.astype(F64)) <= np.spacing(s1).astype(F64))


# ---------------------------------------------------------------------------
# P7: at most two roundings per element, for every P
# ---------------------------------------------------------------------------
def _lossless_partials(P, n_groups, rng):
    """Integer partials whose stage-1 and stage-2 grids are both exact."""
    b = rng.integers(-4, 5, (n_groups, 32))
    b[:, 0] = 7 * np.where(rng.random(n_groups) < 0.5, 1, -1)
    t = rng.integers(-3, 4, (n_groups, 32))
    t[:, 0] = 0
    # zero-sum signs; for odd P the unsigned rank goes first so that the ring
    # comparator's running sums leave the exact grid
    eps = ([0] if P % 2 else []) + [(1 if r % 2 == 0 else -1) for r in range(P - P % 2)]
    x = np.stack([(b + e * t).reshape(-1) for e in eps]).astype(F32)
    return x, (P * b).reshape(-1).astype(F64)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16])
def test_two_roundings_for_every_P(P):
    rng = np.random.default_rng(P)
    x, exact_sum = _lossless_partials(P, 16, rng)
    o = eo.echo_call(x, None, compensate=False)
    # both quantizations land on exact grid points: nothing else may round
    assert np.array_equal(o["out"].astype(F64), exact_sum)
    # random data: error within one half-step per stage-1 rank plus one stage-2 half-step
    _, xr = synth.host_partials("tiny", 0, 3, P=P, n=4096)
    o = eo.echo_call(xr, None, compensate=False)
    bound = (np.sum(o["scales1"].astype(F64), axis=0) / 2 + o["scales2"].astype(F64) / 2)
    err = np.abs(o["out"].astype(F64) - eo.plain_sum(xr)).reshape(-1, 32).max(axis=1)
    slop = np.repeat(np.abs(xr).sum(0).reshape(-1, 32).max(1), 1) * P * 2.0 ** -22
    assert np.all(err <= bound + slop)
    # contrast: re-quantizing the running sum at every hop of a ring rounds each
    # element P times; its error grows about linearly in P, Echo's about as sqrt(P)
    if P >= 8:
        exact = eo.plain_sum(xr)
        ring = eo.naive_ring_int4(xr).astype(F64)
        rms = lambda e: np.sqrt(np.mean(e ** 2))
        assert rms(ring - exact) > 1.3 * rms(o["out"].astype(F64) - exact)


# ---------------------------------------------------------------------------
# P8: the whole call against the exact-rational implementation
# ---------------------------------------------------------------------------
def _compare_exact(x, T, compensate, beta=(0.5, 0.95), group=32):
    P, N = x[0].shape
    st = eo.OracleState(N)
    mf = [Fraction(0)] * N
    ms = [Fraction(0)] * N
    for t in range(T):
        o = eo.echo_call(x[t], st, compensate=compensate, beta_fast=beta[0], beta_slow=beta[1],
                         group=group)
        e = ex.echo_call([_fr(x[t][r]) for r in range(P)], mf, ms, compensate=compensate,
                         beta_fast=beta[0], beta_slow=beta[1], group=group)
        for r in range(P):
            assert np.array_equal(o["q1"][r], np.array(e["q1"][r], np.int8))
            assert np.array_equal(o["scales1"][r], _as_f32(e["scales1"][r]))
        for key in ("S", "c", "V", "B", "r", "out"):
            assert np.array_equal(o[key], _as_f32(e[key])), (t, key)
        assert np.array_equal(o["q2"], np.array(e["q2"], np.int8))
        assert np.array_equal(o["scales2"], _as_f32(e["scales2"]))
        if compensate:
            assert np.array_equal(st.m_fast[0], _as_f32(mf))
            assert np.array_equal(st.m_slow[0], _as_f32(ms))


@pytest.mark.parametrize("compensate", [True, False])
def test_whole_call_matches_exact_rationals(compensate):
    xs = [synth.host_partials("tiny", 0, t, P=2, n=64)[1] for t in range(16)]
    _compare_exact(xs, 16, compensate)


@pytest.mark.parametrize("group", [64, 128])
def test_whole_call_matches_exact_rationals_larger_groups(group):
    xs = [synth.host_partials("prefill", 0, t, P=3, n=256)[1] for t in range(6)]
    _compare_exact(xs, 6, True, group=group)
    rng = np.random.default_rng(group)
    xs = [(rng.integers(-12, 13, (2, 256)) * 0.25).astype(F32) for _ in range(4)]
    _compare_exact(xs, 4, False, group=group)


def test_whole_call_matches_exact_rationals_tie_rich():
    # dyadic inputs on a coarse grid make stage-2 ties and exact cancellations common
    rng = np.random.default_rng(11)
    xs = [(rng.integers(-12, 13, (3, 64)) * 0.25).astype(F32) for _ in range(10)]
    _compare_exact(xs, 10, True)


def test_whole_call_matches_exact_rationals_bf16_and_small_scales():
    xs = []
    for t in range(6):
        bits, vals = synth.host_partials("prefill", 0, t, P=3, n=64)
        vals = vals.copy()
        vals[:, :32] *= F32(2.0 ** -120)  # scales near the bottom of the normal range
        xs.append(vals)
    _compare_exact(xs, 6, True, beta=(0.5, 0.9))


# ---------------------------------------------------------------------------
# P9: bounded with compensation, growing without it
# ---------------------------------------------------------------------------
def _d_rms(outs):
    D = np.cumsum(np.stack([o["B"].astype(F64) - o["S"].astype(F64) for o in outs]), 0)
    return np.sqrt(np.mean(D ** 2, axis=1))


def test_bounded_accumulated_error_tiny_config():
    T = synth.WORKLOADS["tiny"]["calls"]
    on, off = _run(T, True), _run(T, False)
    d_on, d_off = _d_rms(on), _d_rms(off)
    sig_r = np.sqrt(np.mean(np.stack([o["r"].astype(F64) for o in on]) ** 2))
    assert np.max(d_on) <= 2.5 * sig_r
    assert d_off[-1] / d_on[-1] >= 1.8


def test_bounded_accumulated_error_deep_chain():
    # pre-norm residual chain: h <- h + allreduce(partials of a random linear map)
    P, rows, hid, L = 4, 8, 256, 128
    rng = np.random.default_rng(3)
    h0 = (rng.standard_normal((rows, hid)) * 0.02).astype(F32)
    Ws = [(rng.standard_normal((hid, hid)) / np.sqrt(hid)).astype(F32) for _ in range(L)]
    sl = hid // P
    gamma = F32(0.02 * np.sqrt(P))
    res = {}
    for comp in (True, False):
        h = h0.copy()
        st = eo.OracleState(rows * hid)
        outs = []
        for W in Ws:
            a = (h / np.sqrt(np.mean(h.astype(F64) ** 2))).astype(F32)
            parts = np.stack([(gamma * (a[:, r * sl:(r + 1) * sl] @ W[r * sl:(r + 1) * sl])).reshape(-1)
                              for r in range(P)]).astype(F32)
            o = eo.echo_call(parts, st, compensate=comp)
            outs.append(o)
            h = h + o["out"].reshape(rows, hid)
        res[comp] = outs
    d_on, d_off = _d_rms(res[True]), _d_rms(res[False])
    sig_r = np.sqrt(np.mean(np.stack([o["r"].astype(F64) for o in res[True]]) ** 2))
    assert np.max(d_on) <= 2.5 * sig_r
    assert d_off[-1] / d_on[-1] >= 4.5


# ---------------------------------------------------------------------------
# P10: determinism, windows, directions, reset
# ---------------------------------------------------------------------------
def test_group_aligned_windows_equal_whole_tensor():
    P, N = 3, 32 * 40
    xs = [synth.host_partials("prefill", 0, t, P=P, n=N)[1] for t in range(5)]
    st = eo.OracleState(N)
    whole = [eo.echo_call(x, st) for x in xs]
    for lo, hi in ((0, 32 * 7), (32 * 7, 32 * 8), (32 * 8, N)):
        sw = eo.OracleState(hi - lo)
        for t, x in enumerate(xs):
            o = eo.echo_call(x[:, lo:hi], sw)
            assert np.array_equal(o["out"], whole[t]["out"][lo:hi])
            assert np.array_equal(o["codes2"], whole[t]["codes2"][lo // 2:hi // 2])
        assert np.array_equal(sw.m_fast[0], st.m_fast[0][lo:hi])
        assert np.array_equal(sw.m_slow[0], st.m_slow[0][lo:hi])


def test_directions_are_isolated_and_reset_is_fresh():
    N = 2048
    fw = [synth.host_partials("training", 0, t, P=2, n=N)[1] for t in range(4)]
    bw = [synth.host_partials("training", 1, t, P=2, n=N)[1] for t in range(4)]
    inter = eo.OracleState(N)
    outs_i = []
    for t in range(4):
        outs_i.append(eo.echo_call(fw[t], inter, eo.FWD))
        outs_i.append(eo.echo_call(bw[t], inter, eo.BWD))
    sf, sb = eo.OracleState(N), eo.OracleState(N)
    for t in range(4):
        assert np.array_equal(eo.echo_call(fw[t], sf, eo.FWD)["out"], outs_i[2 * t]["out"])
        assert np.array_equal(eo.echo_call(bw[t], sb, eo.BWD)["out"], outs_i[2 * t + 1]["out"])
    inter.reset(1)
    assert not np.any(inter.m_fast[0]) and np.array_equal(inter.m_fast[1], sb.m_fast[1])
    a = eo.echo_call(fw[0], inter, eo.FWD)["out"]
    assert np.array_equal(a, outs_i[0]["out"])
    again = eo.echo_call(fw[0], eo.OracleState(N), eo.FWD)["out"]
    assert np.array_equal(a, again)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        eo.echo_call(np.zeros((2, 33), F32), None, compensate=False)
    x = np.zeros((2, 64), F32)
    x[0, 3] = np.inf
    with pytest.raises(ValueError):
        eo.echo_call(x, None, compensate=False)


def test_synth_recipe_is_deterministic_and_rounds_to_bf16():
    a = synth.host_partials("prefill", 0, 5, P=2, n=4096)
    b = synth.host_partials("prefill", 0, 5, P=2, n=4096)
    assert np.array_equal(a[0], b[0])
    bits, vals = a
    assert bits.dtype == np.uint16
    raw = np.stack([synth.normal_f32(synth.seed_of("prefill", 0, 5, r), 4096, 0.02, 1e-3, 50.0)
                    for r in range(2)])
    # nearest bfloat16: no representable bf16 value is closer than the chosen one
    err = np.abs(vals.astype(F64) - raw.astype(F64))
    ulp = np.abs(np.spacing(vals.astype(F32))).astype(F64) * 2 ** 16
    assert np.all(err <= ulp / 2)


# ---------------------------------------------------------------------------
# sender-side error feedback (a variant): exact rationals, telescoping,
# bounded end-to-end error
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("compensate", [True, False])
def test_sender_feedback_matches_exact_rationals(compensate):
    P, N, T = 3, 64, 8
    st = eo.OracleState(N)
    mf, ms = [Fraction(0)] * N, [Fraction(0)] * N
    se = [[Fraction(0)] * N for _ in range(P)]
    for t in range(T):
        _, x = synth.host_partials("prefill", 0, t, P=P, n=N)
        o = eo.echo_call(x, st, compensate=compensate, sender_feedback=True)
        e = ex.echo_call([_fr(x[r]) for r in range(P)], mf, ms, compensate=compensate, sender_err=se)
        for r in range(P):
            assert np.array_equal(o["q1"][r], np.array(e["q1"][r], np.int8)), (t, r)
            assert np.array_equal(o["scales1"][r], _as_f32(e["scales1"][r]))
            assert np.array_equal(st.sender_err[0][r], _as_f32(se[r])), (t, r)
        for key in ("S", "V", "B", "out"):
            assert np.array_equal(o[key], _as_f32(e[key])), (t, key)


def test_sender_feedback_telescopes():
    """Sum over calls and ranks of (dequantized stage-1 value - partial) equals
    minus the final sender errors plus the binary32 roundings of x + e, exactly."""
    P, N, T = 2, 64, 12
    st = eo.OracleState(N)
    lhs = [Fraction(0)] * N
    rounding = [Fraction(0)] * N
    for t in range(T):
        _, x = synth.host_partials("tiny", 0, t, P=P, n=N)
        e_before = st.sender_err[0].copy() if st.sender_err[0] is not None else np.zeros((P, N), F32)
        o = eo.echo_call(x, st, sender_feedback=True)
        deq = eo.dequantize_groups(o["q1"].reshape(P, -1), o["scales1"].reshape(-1)).reshape(P, N)
        for r in range(P):
            for i in range(N):
                lhs[i] += Fraction(float(deq[r, i])) - Fraction(float(x[r, i]))
                exact_sum = Fraction(float(x[r, i])) + Fraction(float(e_before[r, i]))
                rounding[i] += Fraction(float(o["x1"][r, i])) - exact_sum
    for i in range(N):
        final = sum(Fraction(float(st.sender_err[0][r, i])) for r in range(P))
        assert lhs[i] == -final + rounding[i]


def test_sender_feedback_bounds_end_to_end_error():
    """With sender feedback and compensation the accumulated end-to-end error
    sum_t (out_t - sum_r x_t,r) stays flat; without sender feedback it grows
    like a random walk (stage-1 roundings are not compensated then)."""
    P, N = 2, 2048

    def run(T, sfb):
        st = eo.OracleState(N)
        acc = np.zeros(N, F64)
        rms = []
        for t in range(T):
            _, x = synth.host_partials("tiny", 0, t, P=P, n=N)
            o = eo.echo_call(x, st, sender_feedback=sfb)
            acc += o["out"].astype(F64) - eo.plain_sum(x)
            rms.append(np.sqrt(np.mean(acc ** 2)))
        return np.array(rms)

    with_fb, without = run(256, True), run(256, False)
    # flat with feedback: no growth between the first 16 and the last 16 calls
    assert with_fb[-16:].mean() < 1.3 * with_fb[:16].mean()
    assert with_fb.max() < 3.0 * with_fb[:16].mean()
    # a random walk without: sqrt(256/16) = 4 times larger at the end
    assert without[-16:].mean() > 2.5 * without[:16].mean()
    assert without[-1] > 3.0 * with_fb[-1]


# ---------------------------------------------------------------------------
# bf16 compensator state (a variant)
# ---------------------------------------------------------------------------
def test_bf16_rounding_matches_exact_rounding():
    rng = np.random.default_rng(31)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(F32)
    x = x[np.isfinite(x) & (np.abs(x) < 3e38)]
    # exact ties: the lower 16 bits are exactly half of a bf16 step
    t = ((rng.integers(0, 2 ** 16, 2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000).view(F32)
    t = t[np.isfinite(t) & (np.abs(t) < 3e38)]
    sub = (rng.integers(-2 ** 20, 2 ** 20, 2000) * 2.0 ** -149).astype(F32)  # subnormals
    for v in (x, t, sub):
        got = eo.round_to_bf16(v)
        want = _as_f32([ex.round_to_bfloat16(Fraction(float(a))) for a in v])
        want = np.where(want == 0, np.copysign(F32(0), v), want).astype(F32)  # IEEE: -0 for negatives
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        # and every result is a bfloat16: the low 16 bits are zero
        assert np.all((got.view(np.uint32) & 0xFFFF) == 0)


@pytest.mark.parametrize("compensate", [True, False])
def test_bf16_state_matches_exact_rationals(compensate):
    P, N, T = 2, 64, 10
    st = eo.OracleState(N)
    mf, ms = [Fraction(0)] * N, [Fraction(0)] * N
    for t in range(T):
        _, x = synth.host_partials("prefill", 0, t, P=P, n=N)
        o = eo.echo_call(x, st, compensate=compensate, state_bf16=True)
        e = ex.echo_call([_fr(x[r]) for r in range(P)], mf, ms, compensate=compensate, state_bf16=True)
        for key in ("S", "V", "B", "out"):
            assert np.array_equal(o[key], _as_f32(e[key])), (t, key)
        assert np.array_equal(st.m_fast[0], _as_f32(mf))
        assert np.array_equal(st.m_slow[0], _as_f32(ms))


# ---------------------------------------------------------------------------
# bfloat16 output (a variant): exact rationals, closed form of the compensator
# with the delivered value, lossless special case
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("compensate", [True, False])
def test_bf16_output_matches_exact_rationals(compensate):
    P, N, T = 3, 64, 10
    st = eo.OracleState(N)
    mf, ms = [Fraction(0)] * N, [Fraction(0)] * N
    for t in range(T):
        _, x = synth.host_partials("prefill", 0, t, P=P, n=N)
        o = eo.echo_call(x, st, compensate=compensate, out_bf16=True)
        e = ex.echo_call([_fr(x[r]) for r in range(P)], mf, ms, compensate=compensate, out_bf16=True)
        for key in ("S", "V", "B", "r", "out"):
            assert np.array_equal(o[key], _as_f32(e[key])), (t, key)
        assert np.array_equal(st.m_fast[0], _as_f32(mf))
        assert np.array_equal(st.m_slow[0], _as_f32(ms))


def test_bf16_output_compensator_closed_form():
    """Unrolling m_f and m_s gives, for the accumulated error of what the ranks
    receive, D_T = sum_t (out_t - S_t) = -sum_{t<T} k_{T-1-t} r_t with
    k_n = (0.5^n + 0.95^n) / 2, provided r is measured against the delivered
    bfloat16 value (an error measured against B would leave the output
    roundings, about 2^-9 relative, out of D's closed form)."""
    P, N, T = 2, 2048, 100
    st = eo.OracleState(N)
    outs = []
    for t in range(T):
        _, x = synth.host_partials("tiny", 0, t, P=P, n=N)
        outs.append(eo.echo_call(x, st, out_bf16=True))
    assert all(np.all((o["out"].view(np.uint32) & 0xFFFF) == 0) for o in outs)
    r = np.stack([o["r"].astype(F64) for o in outs])
    D = np.cumsum(np.stack([o["out"].astype(F64) - o["S"].astype(F64) for o in outs]), 0)
    bf, bs = F64(F32(0.5)), F64(F32(0.95))
    k = 0.5 * (bf ** np.arange(T) + bs ** np.arange(T))
    for Tq in (1, 2, 10, 50, 100):
        pred = -np.sum(k[:Tq, None] * r[Tq - 1::-1], axis=0)
        assert np.max(np.abs(D[Tq - 1] - pred)) < 1e-4 * np.max(np.abs(r))


def test_bf16_output_lossless_partials():
    """Partials on both int4 grids: without compensation the only rounding left
    is the bfloat16 one, so out = bf16(sum) exactly."""
    rng = np.random.default_rng(23)
    x, exact_sum = _lossless_partials(4, 16, rng)
    x = x * F32(1.0 + 2.0 ** -12)  # exact, and the sums are no longer bfloat16 values
    exact_sum = exact_sum * (1.0 + 2.0 ** -12)
    o = eo.echo_call(x, None, compensate=False, out_bf16=True)
    want = _as_f32([ex.round_to_bfloat16(Fraction(float(v))) for v in exact_sum])
    assert np.array_equal(o["out"], want)
    assert not np.array_equal(o["out"].astype(F64), exact_sum)


# ---------------------------------------------------------------------------
# owner adds its own partial exactly (a variant): exact rationals, a hand-worked
# value that fixes the rank order, special cases, error statistics
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("compensate,sfb", [(True, False), (False, False), (True, True)])
def test_own_exact_matches_exact_rationals(compensate, sfb):
    P, N, T = 3, 160, 8   # 5 groups: owners hold 2, 2 and 1 of them
    st = eo.OracleState(N)
    mf, ms = [Fraction(0)] * N, [Fraction(0)] * N
    se = [[Fraction(0)] * N for _ in range(P)] if sfb else None
    for t in range(T):
        _, x = synth.host_partials("prefill", 0, t, P=P, n=N)
        o = eo.echo_call(x, st, compensate=compensate, sender_feedback=sfb, own_exact=True)
        e = ex.echo_call([_fr(x[r]) for r in range(P)], mf, ms, compensate=compensate,
                         sender_err=se, own_exact=True)
        for r in range(P):
            assert np.array_equal(o["q1"][r], np.array(e["q1"][r], np.int8)), (t, r)
            assert np.array_equal(o["scales1"][r], _as_f32(e["scales1"][r]))
            if sfb:
                assert np.array_equal(st.sender_err[0][r], _as_f32(se[r])), (t, r)
        for key in ("S", "V", "B", "r", "out"):
            assert np.array_equal(o[key], _as_f32(e[key])), (t, key)
        if compensate:
            assert np.array_equal(st.m_fast[0], _as_f32(mf))


def test_own_exact_rank_order_golden():
    """P = 3, one group per owner; element 64 lies in rank 2's segment.
    Rank 0 sends [1, 0, ...]: s = fl(1/7), code 7, fl(7 * s) = 1.
    Rank 1 sends [3, 7, 0, ...] * 2^-25: s = 2^-25, codes 3 and 7, so 1.5 * 2^-24.
    Rank 2 holds 2^-24 itself.
    In rank order, 1 + 1.5 * 2^-24 rounds up to 1 + 2^-23, and adding 2^-24 is
    then a tie that goes to the even 1 + 2^-22.  Adding the owner's value first
    would give 1 + 2^-23 instead."""
    x = np.zeros((3, 96), F32)
    x[0, 64] = 1.0
    x[1, 64], x[1, 65] = 3 * 2.0 ** -25, 7 * 2.0 ** -25
    x[2, 64] = 2.0 ** -24
    o = eo.echo_call(x, None, compensate=False, own_exact=True)
    assert o["S"][64] == F32(1 + 2.0 ** -22)
    assert o["S"][65] == F32(7 * 2.0 ** -25)
    assert o["scales1"][1][2] == F32(2.0 ** -25)
    assert o["scales1"][2][2] == 0 and not np.any(o["q1"][2][64:96])


def test_own_exact_single_contributor():
    """Only rank j non-zero: on j's own segment the sum is x_j itself, on the
    other segments it is x_j through one stage-1 rounding."""
    P, N = 4, 32 * 8
    _, base = synth.host_partials("tiny", 0, 5, P=1, n=N)
    segs = eo.owner_segments(N // 32, P)
    for j in range(P):
        x = np.zeros((P, N), F32)
        x[j] = base[0]
        o = eo.echo_call(x, None, compensate=False, own_exact=True)
        q, s = eo.quantize_groups(base[0])
        once = eo.dequantize_groups(q, s).reshape(-1)
        for k, (g0, g1) in enumerate(segs):
            sl = slice(g0 * 32, g1 * 32)
            want = base[0][sl] if k == j else once[sl]
            assert np.array_equal(o["S"][sl], want), (j, k)


def test_own_exact_single_rank_is_one_rounding():
    _, x = synth.host_partials("tiny", 0, 2, P=1, n=4096)
    o = eo.echo_call(x, None, compensate=False, own_exact=True)
    q, s = eo.quantize_groups(x[0])
    assert np.array_equal(o["S"], x[0])
    assert np.array_equal(o["out"], eo.dequantize_groups(q, s).reshape(-1))


def test_own_exact_removes_one_rank_of_stage1_error():
    """Stage-1 errors of independent ranks add in variance; keeping the owner's
    share exact leaves P - 1 of the P, so the owner-sum error shrinks by about
    sqrt((P - 1) / P)."""
    for P in (2, 4):
        _, x = synth.host_partials("tiny", 0, 9, P=P, n=1 << 14)
        exact = eo.plain_sum(x)
        e_all = eo.echo_call(x, None, compensate=False)["S"].astype(F64) - exact
        e_own = eo.echo_call(x, None, compensate=False, own_exact=True)["S"].astype(F64) - exact
        ratio = np.sqrt(np.mean(e_own ** 2) / np.mean(e_all ** 2))
        assert abs(ratio - np.sqrt((P - 1) / P)) < 0.05, (P, ratio)


def test_own_exact_window_with_the_message_split_equals_whole_message():
    """Groups are independent once the owner of each group is fixed: a window
    given the whole message's owner split reproduces the whole call there."""
    P, N, G = 3, 32 * 40, 32
    _, x = synth.host_partials("tiny", 0, 4, P=P, n=N)
    whole = eo.echo_call(x, eo.OracleState(N), own_exact=True)
    segs = eo.owner_segments(N // G, P)
    for g_lo, g_hi in ((0, 40), (5, 19), (13, 14), (12, 33)):
        win = [(min(max(a, g_lo), g_hi) - g_lo, min(max(b, g_lo), g_hi) - g_lo) for a, b in segs]
        o = eo.echo_call(x[:, g_lo * G:g_hi * G], eo.OracleState((g_hi - g_lo) * G), own_exact=True,
                         segments=win)
        for key in ("S", "V", "out", "q2", "scales2"):
            lo, hi = (g_lo, g_hi) if key == "scales2" else (g_lo * G, g_hi * G)
            assert np.array_equal(o[key], whole[key][lo:hi]), (g_lo, g_hi, key)
        assert np.array_equal(o["q1"], whole["q1"][:, g_lo * G:g_hi * G])


def test_reset_clears_the_sender_errors_too():
    """With sender feedback, a reset makes the next call equal a fresh state's:
    output, both estimates and every rank's stage-1 error."""
    P, N = 3, 32 * 20
    st = eo.OracleState(N)
    for t in range(3):
        _, x = synth.host_partials("tiny", 0, t, P=P, n=N)
        eo.echo_call(x, st, sender_feedback=True)
    assert np.any(st.sender_err[0] != 0)
    st.reset(1)
    fresh = eo.OracleState(N)
    _, x = synth.host_partials("tiny", 0, 7, P=P, n=N)
    a = eo.echo_call(x, st, sender_feedback=True)
    b = eo.echo_call(x, fresh, sender_feedback=True)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(st.sender_err[0], fresh.sender_err[0])
    assert np.array_equal(st.m_slow[0], fresh.m_slow[0])


@pytest.mark.parametrize("own", [False, True])
def test_bf16_state_with_sender_feedback_matches_exact_rationals(own):
    """With bf16 state the ranks' stage-1 errors are kept in bfloat16 too."""
    P, N, T = 3, 96, 8
    st = eo.OracleState(N)
    mf, ms = [Fraction(0)] * N, [Fraction(0)] * N
    se = [[Fraction(0)] * N for _ in range(P)]
    for t in range(T):
        _, x = synth.host_partials("prefill", 0, t, P=P, n=N)
        o = eo.echo_call(x, st, sender_feedback=True, state_bf16=True, own_exact=own)
        e = ex.echo_call([_fr(x[r]) for r in range(P)], mf, ms, sender_err=se, state_bf16=True,
                         own_exact=own)
        for r in range(P):
            assert np.array_equal(st.sender_err[0][r], _as_f32(se[r])), (t, r)
            assert np.all((st.sender_err[0][r].view(np.uint32) & 0xFFFF) == 0)
        for key in ("S", "V", "B", "out"):
            assert np.array_equal(o[key], _as_f32(e[key])), (t, key)


def test_bf16_sender_errors_still_bound_the_end_to_end_error():
    """Rounding the carried stage-1 errors to bfloat16 perturbs the telescoping
    sum by far less than the stage-1 step: the accumulated end-to-end error
    still stays flat, close to the fp32-state run."""
    P, N = 2, 2048

    def run(T, sb16):
        st = eo.OracleState(N)
        acc = np.zeros(N, F64)
        rms = []
        for t in range(T):
            _, x = synth.host_partials("tiny", 0, t, P=P, n=N)
            o = eo.echo_call(x, st, sender_feedback=True, state_bf16=sb16)
            acc += o["out"].astype(F64) - eo.plain_sum(x)
            rms.append(np.sqrt(np.mean(acc ** 2)))
        return np.array(rms)

    b16, f32 = run(256, True), run(256, False)
    assert b16[-16:].mean() < 1.3 * b16[:16].mean()
    assert abs(b16[-1] - f32[-1]) < 0.1 * f32[-1]
