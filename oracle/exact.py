"""Exact-rational brute-force checker (TEST INFRASTRUCTURE ONLY).

A second, independent statement of the same call as :mod:`oracle.echo_oracle`,
written with Python ``fractions``: every arithmetic result is computed exactly
and then rounded to the IEEE binary32 grid by :func:`round_to_binary32`, which
is written out here from the definition of the format (24-bit significand,
exponent range -126..127, gradual underflow down to 2**-149, ties to even).
Quantization codes are chosen by brute force over all fifteen codes.  It is
slow and meant for tiny tensors; its job is to pin the numpy oracle.

The method is the one described in prose in the rit.work blog post
"echo-4-bit-gpu-communication", section «Как Echo возвращает ошибку в следующие
вызовы», and in the heraldofai.com article «Come Echo permette ai modelli AI di
grandi dimensioni…», section «Come Echo evita che gli errori si accumulino».
"""
from __future__ import annotations

from fractions import Fraction

GROUP = 32
QMAX = 7

_EMIN = -126          # smallest normal exponent of binary32
_PREC = 24            # significand bits (with the hidden one)
_TINY = Fraction(1, 2 ** 149)   # smallest subnormal step
_OVER = Fraction(2 ** 128)      # first value beyond the largest finite
HALF = Fraction(1, 2)


def _round_half_even_int(y: Fraction) -> int:
    """Nearest integer to ``y`` (y >= 0), ties to the even integer."""
    fl = y.numerator // y.denominator
    rem = y - fl
    if rem > HALF:
        return fl + 1
    if rem < HALF:
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _floor_log2(m: Fraction) -> int:
    e = m.numerator.bit_length() - m.denominator.bit_length()
    # now 2**(e-1) < m < 2**(e+1); settle it
    while Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    return e


def round_to_format(x, prec: int, emin: int = _EMIN, emax: int = 127) -> Fraction:
    """Round an exact rational to the nearest value of a binary format with a
    ``prec``-bit significand (hidden bit included), normal exponents down to
    ``emin`` and gradual underflow below, ties to even."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    m = abs(x)
    e = _floor_log2(m)
    quantum = Fraction(2) ** ((e if e >= emin else emin) - (prec - 1))
    k = _round_half_even_int(m / quantum)
    r = k * quantum
    if r >= Fraction(2) ** (emax + 1):
        raise OverflowError("result exceeds the format's range")
    return sign * r


def round_to_binary32(x) -> Fraction:
    """Round an exact rational to the nearest binary32 value (ties to even)."""
    return round_to_format(x, _PREC)


def round_to_bfloat16(x) -> Fraction:
    """Round an exact rational to the nearest bfloat16 value (8-bit significand,
    binary32's exponent range, subnormals down to 2**-133; ties to even)."""
    return round_to_format(x, 8)


def f32(x) -> Fraction:
    """The binary32 value of a Python float / int / Fraction (rounded)."""
    return round_to_binary32(Fraction(x))


def add(a: Fraction, b: Fraction) -> Fraction:
    return round_to_binary32(a + b)


def sub(a: Fraction, b: Fraction) -> Fraction:
    return round_to_binary32(a - b)


def mul(a: Fraction, b: Fraction) -> Fraction:
    return round_to_binary32(a * b)


def div(a: Fraction, b: Fraction) -> Fraction:
    return round_to_binary32(a / b)


def nearest_code(v: Fraction, s: Fraction) -> int:
    """argmin over k in [-7, 7] of |v - k*s|, exact; ties go to the even k."""
    best_k, best_d = None, None
    for k in range(-QMAX, QMAX + 1):
        d = abs(v - k * s)
        if best_d is None or d < best_d or (d == best_d and k % 2 == 0):
            best_k, best_d = k, d
    return best_k


def quantize_group(v):
    """Q of one group (list of exact binary32 values) -> (codes, scale)."""
    a = max(abs(t) for t in v)
    s = div(a, Fraction(QMAX))
    if s == 0:
        return [0] * len(v), s
    return [nearest_code(t, s) for t in v], s


def quantize(v, group=GROUP):
    codes, scales = [], []
    for g in range(0, len(v), group):
        q, s = quantize_group(v[g:g + group])
        codes.extend(q)
        scales.append(s)
    return codes, scales


def dequantize(codes, scales, group=GROUP):
    return [mul(Fraction(q), scales[i // group]) for i, q in enumerate(codes)]


def echo_call(partials, m_fast, m_slow, compensate=True, beta_fast=0.5,
              beta_slow=0.95, group=GROUP, sender_err=None, state_bf16=False,
              out_bf16=False, own_exact=False):
    """One call on exact binary32 values.

    ``partials`` is a list of P lists of Fractions (each a binary32 value);
    ``m_fast``/``m_slow`` are lists of Fractions, updated in place when
    compensating; ``sender_err``, if given, is the P ranks' stage-1 error
    lists (the sender-feedback variant), updated in place (rounded to bfloat16
    with ``state_bf16``).  ``out_bf16``: the
    ranks receive bf16(B) and the error is measured against it.
    ``own_exact``: the owner of group g (g // ceil(n_groups / P)) adds its own
    input exactly instead of through Q; its own groups are not quantized (codes
    and scales reported as 0) and its sender error there is left alone.
    Returns a dict of lists of Fractions / ints.
    """
    P = len(partials)
    N = len(partials[0])
    n_groups = N // group
    per = (n_groups + P - 1) // P   # groups per owner, the last owner's share shorter

    def owner(i):
        return (i // group) // per

    q1, s1, xin = [], [], []
    for r in range(P):
        # sender feedback (a variant): quantize x + e and keep the new error
        x = partials[r] if sender_err is None else [add(a, b) for a, b in zip(partials[r], sender_err[r])]
        xin.append(x)
        q, s = quantize(x, group)
        if own_exact:
            for i in range(N):
                if owner(i) == r:
                    q[i] = 0
                    s[i // group] = Fraction(0)
        q1.append(q)
        s1.append(s)
        if sender_err is not None:
            deq = dequantize(q, s, group)
            new = [sub(a, b) for a, b in zip(x, deq)]
            if state_bf16:  # variant: the carried state, sender errors included, in bfloat16
                new = [round_to_bfloat16(e) for e in new]
            sender_err[r][:] = [e if (own_exact and owner(i) == r) else n
                                for i, (n, e) in enumerate(zip(new, sender_err[r]))]
    S = []
    for i in range(N):
        acc = None
        for r in range(P):
            if own_exact and owner(i) == r:
                d = xin[r][i]
            else:
                d = mul(Fraction(q1[r][i]), s1[r][i // group])
            acc = d if acc is None else add(acc, d)
        S.append(acc)
    if compensate:
        c = [add(mul(HALF, m_fast[i]), mul(HALF, m_slow[i])) for i in range(N)]
        V = [add(S[i], c[i]) for i in range(N)]
    else:
        c = [Fraction(0)] * N
        V = list(S)
    q2, s2 = quantize(V, group)
    B = dequantize(q2, s2, group)
    out = [round_to_bfloat16(b) for b in B] if out_bf16 else B
    err = [Fraction(0)] * N
    if compensate:
        bf, bs = f32(beta_fast), f32(beta_slow)
        wf, ws = sub(Fraction(1), bf), sub(Fraction(1), bs)
        for i in range(N):
            err[i] = sub(V[i], out[i])
            m_fast[i] = add(mul(bf, m_fast[i]), mul(wf, err[i]))
            m_slow[i] = add(mul(bs, m_slow[i]), mul(ws, err[i]))
            if state_bf16:  # variant: the estimates are stored in bfloat16
                m_fast[i] = round_to_bfloat16(m_fast[i])
                m_slow[i] = round_to_bfloat16(m_slow[i])
    return {"q1": q1, "scales1": s1, "S": S, "c": c, "V": V, "q2": q2,
            "scales2": s2, "B": B, "r": err, "out": out}
