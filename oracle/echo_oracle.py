"""Plain numpy oracle of one Echo all-reduce call (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may use this module; the product path never does.  It imports nothing from the
HIP library's package.

What is computed, step by step, for P rank partials x_0..x_{P-1} of N elements
each, on a direction d ("fwd" = 0, "bwd" = 1) whose compensator state is the
pair (m_fast, m_slow) of fp32 vectors of length N:

  1. Stage 1, on every rank: each group of 32 consecutive elements is mapped to
     4-bit integer codes and one fp32 scale by Q below.  The pages say the ranks
     ship their segments as 4-bit integers
     [rit.work "echo-4-bit-gpu-communication", «Как Echo возвращает ошибку в
     следующие вызовы»].
  2. Exchange: the owner of segment j receives segment j of every rank's
     payload (emulated: the owner reads it in place).
  3. Owner sum: d_r = fl(q_r * s_r), S = (((d_0 + d_1) + d_2) + ...) in fp32,
     in rank order.  The owner restores the codes and adds them in high
     precision [same section; heraldofai.com «Come Echo permette…»,
     «Come Echo evita che gli errori si accumulino»].
  4. Correction: c = fl(fl(0.5*m_fast) + fl(0.5*m_slow)) and V = fl(S + c).
     The correction from earlier calls enters the value that is about to be
     rounded, so it reaches every rank's residual stream through the broadcast
     [rit.work, «Как Echo возвращает ошибку…»].
  5. Stage 2: (q2, s2) = Q(V); B = fl(q2 * s2) is what every rank decodes.
     Each element has therefore passed through Q exactly twice, whatever P is
     [rit.work, «Как Echo возвращает ошибку…»; heraldofai.com,
     «Come Echo evita che gli errori si accumulino»].
  6. Error and compensator: r = fl(V - B) is the error the owner's own rounding
     just introduced; the fast and the slow smoothed estimates are updated as
     m <- fl(fl(beta*m) + fl(omega*r)), omega = fl(1 - beta), with
     beta_fast = 0.5 and beta_slow = fl(0.95); forward and backward keep
     separate pairs [rit.work, «Как Echo возвращает ошибку…»].
  7. Output: out = B in fp32.

Q(v) for one group v of fp32 values (32 consecutive elements by default; the
group sizes 64 and 128 are variants the pages leave open):
  a = max |v_i|;  s = fl(a / 7)  (IEEE binary32 division);
  if s == 0: every code is 0;
  else: q_i = the code k in [-7, 7] nearest to the exact real quotient v_i / s,
        ties to the even k.  (Away from the denormal range this is just the
        round-half-even of v_i / s, which never leaves [-7, 7].)

Readings where the pages are silent (group 32, absmax/7 scale, half-even
ties, nearest-code saturation, correction weights 1/2 + 1/2, beta values,
r = V - B, fp32 output) are fixed in the design notes of this repository.

Every operation below is a single IEEE binary32 operation with round-to-nearest-
even (numpy float32 arithmetic; denormals are kept), except the code choice in
Q, which evaluates v/s in binary64: for binary32 v and s, a quotient that is
not a tie lies at least 2**-26 (relative) away from every half-integer, far
beyond binary64's rounding error, and an exact tie is representable, so the
binary64 quotient always selects the same code as the exact one.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
QMAX = 7
F32 = np.float32
F64 = np.float64

FWD = 0
BWD = 1


# ----------------------------------------------------------------------------
# data conversion
# ----------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly (16-bit shift)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(F32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of every float32 (ties to even), as float32.

    bfloat16 keeps binary32's exponent range with an 8-bit significand: a
    normal value x = m * 2**e (0.5 <= |m| < 1) becomes rint(m * 2**8) * 2**(e-8);
    below 2**-126 the step is fixed at 2**-133 (gradual underflow)."""
    x = np.asarray(x, dtype=F32).astype(F64)
    m, e = np.frexp(x)
    normal = np.abs(x) >= 2.0 ** -126
    r = np.where(normal, np.ldexp(np.rint(np.ldexp(m, 8)), e - 8),
                 np.rint(x * 2.0 ** 133) * 2.0 ** -133)
    return r.astype(F32)


# ----------------------------------------------------------------------------
# the quantizer Q
# ----------------------------------------------------------------------------
def quantize_groups(v: np.ndarray, group: int = GROUP):
    """Q applied to every group of ``group`` consecutive elements of ``v``.

    Returns ``(codes, scales)``: int8 codes in [-7, 7] with the shape of ``v``
    flattened to ``(-1, group)`` and one float32 scale per group.
    """
    v = np.ascontiguousarray(v, dtype=F32).reshape(-1, group)
    a = np.max(np.abs(v), axis=1)
    s = a / F32(QMAX)  # binary32 division, round to nearest even
    codes = np.zeros(v.shape, dtype=np.int8)
    nz = s != F32(0)
    if np.any(nz):
        quot = v[nz].astype(F64) / s[nz].astype(F64)[:, None]
        k = np.rint(quot)  # round half to even
        k = np.clip(k, -QMAX, QMAX)  # nearest admissible code
        codes[nz] = k.astype(np.int8)
    return codes, s.astype(F32)


def dequantize_groups(codes: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """fl(q * s) per element, as float32 of shape ``(-1, group)``."""
    codes = np.asarray(codes, dtype=np.int8).reshape(-1, group)
    scales = np.asarray(scales, dtype=F32).reshape(-1)
    return codes.astype(F32) * scales[:, None]


# ----------------------------------------------------------------------------
# wire format: two's-complement nibbles, element 2k in the low nibble of byte k
# ----------------------------------------------------------------------------
def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int8).reshape(-1)
    u = c.view(np.uint8) & np.uint8(0x0F)
    return (u[0::2] | (u[1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    b = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(b.size * 2, dtype=np.int8)
    lo = (b & np.uint8(0x0F)).astype(np.int16)
    hi = (b >> np.uint8(4)).astype(np.int16)
    out[0::2] = ((lo ^ 8) - 8).astype(np.int8)
    out[1::2] = ((hi ^ 8) - 8).astype(np.int8)
    return out


# ----------------------------------------------------------------------------
# owner segments and wire bytes
# ----------------------------------------------------------------------------
def owner_segments(n_groups: int, P: int):
    """Group ranges [start, end) owned by ranks 0..P-1 (ceil split, last short)."""
    per = -(-n_groups // P) if P > 0 else 0
    segs = []
    for j in range(P):
        lo = min(n_groups, j * per)
        hi = min(n_groups, (j + 1) * per)
        segs.append((lo, hi))
    return segs


def payload_bytes(n_elems: int, group: int = GROUP) -> int:
    """Bytes one int4 payload of ``n_elems`` occupies: codes plus fp32 scales."""
    return n_elems // 2 + 4 * (n_elems // group)


def wire_bytes(P: int, N: int, group: int = GROUP):
    """Bytes each rank would put on the wire for one call.

    rs: largest over ranks of what a rank sends to the other owners;
    ag: largest over owners of what an owner broadcasts to the other ranks;
    bf16: a ring all-reduce of the same message in bfloat16, 2(P-1)/P * 2N.
    """
    segs = owner_segments(N // group, P)
    seg_b = [payload_bytes((hi - lo) * group, group) for lo, hi in segs]
    rs = max((sum(seg_b) - seg_b[r] for r in range(P)), default=0)
    ag = max(((P - 1) * b for b in seg_b), default=0)
    bf16 = (2 * (P - 1) * 2 * N) // P if P > 0 else 0
    return {"rs_per_rank": rs, "ag_per_rank": ag, "bf16_allreduce_per_rank": bf16}


# ----------------------------------------------------------------------------
# compensator state
# ----------------------------------------------------------------------------
class OracleState:
    """(m_fast, m_slow) per direction, fp32, all zero after a reset; with the
    sender-feedback variant also every rank's stage-1 error per direction
    (``sender_err[d]``, [P, N] fp32, created zero on first use)."""

    def __init__(self, N: int):
        self.N = N
        self.m_fast = {FWD: np.zeros(N, F32), BWD: np.zeros(N, F32)}
        self.m_slow = {FWD: np.zeros(N, F32), BWD: np.zeros(N, F32)}
        self.sender_err = {FWD: None, BWD: None}

    def reset(self, mask: int = 3):
        for d in (FWD, BWD):
            if mask & (1 << d):
                self.m_fast[d][:] = 0
                self.m_slow[d][:] = 0
                if self.sender_err[d] is not None:
                    self.sender_err[d][:] = 0

    def copy(self) -> "OracleState":
        o = OracleState(self.N)
        for d in (FWD, BWD):
            o.m_fast[d] = self.m_fast[d].copy()
            o.m_slow[d] = self.m_slow[d].copy()
            o.sender_err[d] = None if self.sender_err[d] is None else self.sender_err[d].copy()
        return o


# ----------------------------------------------------------------------------
# one call
# ----------------------------------------------------------------------------
def echo_call(partials, state: OracleState | None, direction: int = FWD,
              compensate: bool = True, beta_fast: float = 0.5,
              beta_slow: float = 0.95, group: int = GROUP,
              sender_feedback: bool = False, state_bf16: bool = False,
              out_bf16: bool = False, own_exact: bool = False, segments=None):
    """One Echo all-reduce of ``partials`` ([P, N] float32).

    Advances ``state`` (direction ``direction``) in place when compensating and
    returns a dict with every intermediate the GPU path exposes.

    ``sender_feedback`` is a variant the pages leave open: every rank also
    feeds the error of its own stage-1 rounding into its next call (classic
    error feedback): x' = fl(x + e), (q, s) = Q(x'), e <- fl(x' - fl(q * s)),
    the last difference exact.  The stage-1 errors then telescope, so the
    accumulated end-to-end error stays bounded too.

    ``state_bf16`` is another variant: the carried state is stored in
    bfloat16, i.e. every update m <- fl(fl(beta*m) + fl(omega*r)) of the two
    estimates, and with sender feedback every new stage-1 error e, is rounded
    to the nearest bfloat16 before it is kept.

    ``out_bf16`` (a variant): what the ranks receive is the broadcast value
    rounded once more, to the nearest bfloat16, and the owner measures its
    error against that delivered value, r = fl(V - bf16(B)), so the
    compensator also returns the output rounding in later calls.  (The
    difference is exact except when V and bf16(B) straddle a power of two.)

    ``own_exact`` (a variant): the owner of a segment holds its own partial
    and adds it as it is instead of through Q: rank j quantizes and sends
    every segment but its own (its codes and scales there are left zero here,
    and with sender feedback its error there is neither used nor changed), and
    the owner's rank-order sum takes x_j (x_j + e_j with sender feedback) in
    place of fl(q_j * s_j) on segment j.

    ``segments``: the group ranges [g0, g1) owned by ranks 0..P-1; by default
    the ceil split of this message (owner_segments).  Only own_exact depends
    on it: a group-aligned window of a longer message passes that message's
    split restricted to the window.
    """
    x = np.ascontiguousarray(partials, dtype=F32)
    if x.ndim != 2:
        raise ValueError("partials must be [P, N]")
    P, N = x.shape
    if N % group:
        raise ValueError(f"N must be a multiple of the group size {group}")
    if not np.all(np.isfinite(x)):
        raise ValueError("partials must be finite")
    n_g = N // group
    segs = owner_segments(n_g, P) if segments is None else [tuple(sg) for sg in segments]
    if len(segs) != P:
        raise ValueError("one segment per rank")

    # 1. stage 1 on every rank (with sender feedback: on x + e, then the new e)
    q1 = np.empty((P, N), np.int8)
    s1 = np.empty((P, n_g), F32)
    if sender_feedback:
        if state.sender_err[direction] is None or state.sender_err[direction].shape != (P, N):
            state.sender_err[direction] = np.zeros((P, N), F32)
        e1 = state.sender_err[direction]
        xs = x + e1
    else:
        xs = x
    for r in range(P):
        q, s = quantize_groups(xs[r], group)
        sent = np.ones(N, bool)
        if own_exact:  # rank r keeps its own segment: nothing of it is quantized
            g0, g1 = segs[r]
            q[g0:g1] = 0
            s[g0:g1] = 0
            sent[g0 * group:g1 * group] = False
        q1[r] = q.reshape(-1)
        s1[r] = s
        if sender_feedback:
            e_new = xs[r] - dequantize_groups(q, s, group).reshape(-1)
            if state_bf16:
                e_new = round_to_bf16(e_new)
            e1[r] = np.where(sent, e_new, e1[r])

    # 2.-6. each owner works on its own segment of every rank's payload
    S = np.empty(N, F32)
    c = np.zeros(N, F32)
    V = np.empty(N, F32)
    q2 = np.empty(N, np.int8)
    s2 = np.empty(n_g, F32)
    B = np.empty(N, F32)
    err = np.zeros(N, F32)
    if compensate:
        bf, bs = F32(beta_fast), F32(beta_slow)
        wf, ws = F32(1) - bf, F32(1) - bs
        mf = state.m_fast[direction]
        ms = state.m_slow[direction]
    for j, (g0, g1) in enumerate(segs):
        if g1 <= g0:
            continue
        e0, e1 = g0 * group, g1 * group
        # 3. dequantize every rank's contribution and add in rank order
        acc = None
        for r in range(P):
            if own_exact and r == j:
                d = xs[r, e0:e1]
            else:
                d = dequantize_groups(q1[r, e0:e1], s1[r, g0:g1], group).reshape(-1)
            acc = d if acc is None else acc + d
        S[e0:e1] = acc
        # 4. correction from the two smoothed error estimates
        if compensate:
            cc = F32(0.5) * mf[e0:e1] + F32(0.5) * ms[e0:e1]
            c[e0:e1] = cc
            vv = acc + cc
        else:
            vv = acc
        V[e0:e1] = vv
        # 5. stage 2
        qq, ss = quantize_groups(vv, group)
        q2[e0:e1] = qq.reshape(-1)
        s2[g0:g1] = ss
        bb = dequantize_groups(qq, ss, group).reshape(-1)
        B[e0:e1] = bb
        if out_bf16:  # the value the ranks will hold
            bb = round_to_bf16(bb)
        # 6. error of this rounding, then the two estimates
        if compensate:
            rr = vv - bb
            err[e0:e1] = rr
            mf[e0:e1] = bf * mf[e0:e1] + wf * rr
            ms[e0:e1] = bs * ms[e0:e1] + ws * rr
            if state_bf16:
                mf[e0:e1] = round_to_bf16(mf[e0:e1])
                ms[e0:e1] = round_to_bf16(ms[e0:e1])

    # 7. every rank decodes the broadcast payload
    codes2 = pack_nibbles(q2)
    out = dequantize_groups(unpack_nibbles(codes2), s2, group).reshape(-1)
    if out_bf16:
        out = round_to_bf16(out)
    return {
        "codes1": np.stack([pack_nibbles(q1[r]) for r in range(P)]) if P else np.zeros((0, N // 2), np.uint8),
        "scales1": s1,
        "q1": q1,
        "x1": xs,
        "S": S,
        "c": c,
        "V": V,
        "q2": q2,
        "codes2": codes2,
        "scales2": s2,
        "B": B,
        "r": err,
        "out": out,
        "segments": segs,
    }


def plain_sum(partials) -> np.ndarray:
    """Exact-as-possible reference sum, in binary64, of [P, N] partials."""
    return np.sum(np.asarray(partials, dtype=F64), axis=0)


def naive_ring_int4(partials, group: int = GROUP) -> np.ndarray:
    """Comparator: ring reduce that re-quantizes the running sum at every hop.

    Rank 0 quantizes its partial and sends it on; every later rank decodes what
    it received, adds its own partial in fp32 and quantizes again before
    forwarding.  The last rank's payload is what everybody decodes.  An element
    is therefore rounded P times, which is the failure mode the pages contrast
    Echo with [rit.work, «Почему обычное 4-битное суммирование портит модель»].
    """
    x = np.asarray(partials, dtype=F32)
    q, s = quantize_groups(x[0], group)
    acc = dequantize_groups(q, s, group).reshape(-1)
    for r in range(1, x.shape[0]):
        q, s = quantize_groups(acc + x[r], group)
        acc = dequantize_groups(q, s, group).reshape(-1)
    return acc
