"""Stage 1 fused into the producing product (MFMA bf16, fp32 accumulation).

* The product itself: bf16(A_r @ W_r^T) against the exact product of the same
  bf16 inputs (float64 on the host): within half a bf16 ulp plus the fp32
  accumulation bound, and equal to the rounded exact product almost everywhere.
* The fused payload: bit-identical to stage 1 of the unfused bf16 partial, by
  the oracle and by the library's own stage-1 kernel.
* Whole calls: fused stage 1, owner and decode against the oracle fed the
  unfused partials, call after call.
"""
import numpy as np
import pytest

from oracle import echo_oracle as eo
from parity_helpers import _compare, _fetch, _state, _torch

pytestmark = pytest.mark.gpu

# Every tile configuration the launcher picks, each in its steady state: a K
# step issues the loads of step + S - 1 into the slab that step - 1 read, so
# with S slabs each tile runs at least S + 1 steps (and the ring is exercised
# over many turns), plus fewer steps than slabs (the pipeline is never full)
# and, for the grouped tile order, a tile count that is not a multiple of 8 (block
# i then takes tile i of the row-tile-fastest order, without the XCD grouping).
# With n the number of 64 x 128 tiles of the launch (all ranks) and b that of
# 128 x 128 tiles, the launcher takes
#   n <= 128: 64 x 64, 4 slabs, grouped;
#   else, for M an odd multiple of 64: 64 x 128, 4 slabs, grouped;
#   else b <= 128: 64 x 128, 4 slabs, grouped;  b <= 256: 128 x 128, 4 slabs, grouped;
#   b <= 512 with M a multiple of 256: 256 x 128, 3 slabs, grouped;
#   b >= 1024 with M and H multiples of 256: 256 x 256, 2 slabs, grouped;
#   else 128 x 128, 2 slabs, grouped.
SHAPES = [
    (2, 64, 64, 128),        # n = 2: 64 x 64, 4 tiles, 1 K step
    (1, 128, 64, 128),       # n = 2: 64 x 64, 4 tiles, 1 K step
    (4, 128, 192, 2048),     # n = 128: 64 x 64, 256 tiles, 3 steps (the prologue fills every slab but one)
    (2, 128, 64, 4096),      # n = 128: 64 x 64, 256 tiles, 1 step
    (3, 64, 320, 1408),      # n = 33: 64 x 64, 66 tiles (not a multiple of 8), 5 steps
    (2, 256, 512, 384),      # n = 24: 64 x 64, 48 tiles, 8 steps
    (3, 384, 1024, 256),     # n = 36: 64 x 64, 72 tiles, 16 steps
    (8, 128, 3072, 1024),    # n = 128: 64 x 64, 256 tiles, 48 steps
    (8, 64, 512, 4096),      # M = 64, n = 256: 64 x 128, the decode-shaped layer's product (K = 4096 / 8), 8 steps
    (3, 192, 320, 2816),     # M = 192: 64 x 128, 198 tiles (not a multiple of 8), 5 steps
    (4, 320, 1024, 1024),    # M = 320: 64 x 128, 160 tiles, 16 steps
    (4, 128, 128, 4096),     # b = 128: 64 x 128, 256 tiles, 2 steps
    (4, 128, 1024, 4096),    # b = 128: 64 x 128, 16 steps
    (3, 128, 320, 2816),     # b = 66: 64 x 128, 132 tiles (not a multiple of 8), 5 steps
    (16, 128, 128, 2048),    # b = 256: 128 x 128, 4 slabs, 2 steps
    (4, 256, 640, 4096),     # b = 256: 10 steps
    (8, 128, 3072, 4096),    # b = 256: 48 steps: the short product the benchmark times
    (3, 128, 320, 7296),     # b = 171 tiles (not a multiple of 8), 5 steps
    (4, 512, 128, 4096),     # b = 512: 256 x 128, 3 slabs, 256 tiles, 2 steps
    (3, 512, 320, 2816),     # b = 264: 256 x 128, 132 tiles (not a multiple of 8), 5 steps
    (6, 256, 320, 4096),     # b = 384: 256 x 128, 192 tiles, 5 steps
    (8, 256, 3072, 4096),    # b = 512: 256 x 128, 256 tiles, 48 steps
    (2, 2048, 128, 2048),    # b = 512, M = 2048: 256 x 128, 3 slabs, 2 steps
    (2, 2048, 512, 2048),    # b = 512: 256 x 128, 8 steps
    (2, 2176, 192, 2048),    # b = 544: 128 x 128, 2 slabs, 3 steps
    (2, 2176, 512, 2048),    # b = 544: 8 steps
    (3, 128, 320, 11008),    # b = 258 tiles (not a multiple of 8), 5 steps
    (4, 2048, 128, 2048),    # b = 1024: 256 x 256, 2 steps
    (4, 2048, 576, 2048),    # b = 1024: 9 steps (an odd count: the last step reads the other slab)
    (4, 2048, 3072, 4096),   # b = 2048: 48 steps: the product the benchmark times
    (5, 2304, 64, 2304),     # b = 1620: 405 tiles (not a multiple of 8), 1 step
    (16, 384, 192, 1024),    # b = 384: 128 x 128, 2 slabs, 16 ranks, 3 steps
    (16, 1024, 128, 1024),   # b = 1024: 256 x 256, 16 ranks, 2 steps
]
# one shape per tile configuration in its steady state (and the benchmarked
# ones), for the whole-call tests
STEADY = [(8, 64, 512, 4096), (4, 320, 1024, 1024), (2, 256, 512, 384), (8, 128, 3072, 1024), (4, 128, 1024, 4096),
          (4, 256, 640, 4096), (8, 128, 3072, 4096), (2, 2048, 512, 2048), (2, 2176, 512, 2048), (4, 2048, 576, 2048),
          (4, 2048, 3072, 4096)]


def _inputs(P, M, K, H, seed, dev, w=None):
    torch = _torch()
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    A = [torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16) for _ in range(P)]
    if w is None:
        w = [(torch.randn(H, K, generator=g, device=dev) / K ** 0.5).to(torch.bfloat16) for _ in range(P)]
    return A, w


def _unfused(A, W):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    M, H = A[0].shape[0], W[0].shape[0]
    out = [torch.empty(M, H, dtype=torch.bfloat16, device=A[0].device) for _ in A]
    E.echo_gemm_bf16(A, W, out)
    return out


@pytest.mark.parametrize("P,M,K,H", SHAPES)
def test_product_matches_exact_reference(cuda, P, M, K, H):
    A, W = _inputs(P, M, K, H, 1, cuda)
    out = _unfused(A, W)
    for r in range(P):
        a = A[r].float().cpu().numpy().astype(np.float64)
        w = W[r].float().cpu().numpy().astype(np.float64)
        exact = a @ w.T
        mag = np.abs(a) @ np.abs(w).T
        got = out[r].float().cpu().numpy().astype(np.float64)
        bound = np.abs(exact) * 2.0 ** -8 + mag * K * 2.0 ** -24
        assert np.all(np.abs(got - exact) <= bound), f"rank {r}: {np.max(np.abs(got - exact) - bound)}"
        rounded = exact.astype(np.float32)
        rounded_bf16 = (rounded.view(np.uint32) + 0x7FFF + ((rounded.view(np.uint32) >> 16) & 1)) >> 16
        same = np.mean(got.astype(np.float32).view(np.uint32) >> 16 == rounded_bf16)
        assert same > 0.97, f"rank {r}: only {same:.4f} equal to the rounded exact product"


@pytest.mark.parametrize("P,M,K,H", SHAPES)
def test_fused_payload_equals_stage1_of_the_unfused_partial(cuda, P, M, K, H):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    A, W = _inputs(P, M, K, H, 2, cuda)
    N = M * H
    fused = _state(P, N, "bf16")
    E.echo_gemm_stage1(A, W, fused)
    parts = [p.reshape(-1) for p in _unfused(A, W)]
    ref = _state(P, N, "bf16")
    E.echo_stage1(parts, ref)
    vf, vr = E.echo_debug_views(fused), E.echo_debug_views(ref)
    torch.cuda.synchronize()
    assert torch.equal(vf["codes1"], vr["codes1"]) and torch.equal(vf["scales1"], vr["scales1"])
    for r in range(P):
        q, s = eo.quantize_groups(parts[r].float().cpu().numpy())
        assert np.array_equal(vf["codes1"][r].cpu().numpy(), eo.pack_nibbles(q))
        assert np.array_equal(vf["scales1"][r].cpu().numpy().view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("P,M,K,H", [(4, 256, 1024, 512), (8, 128, 512, 1024), (3, 128, 320, 2816),
                                     (3, 128, 320, 7296), (2, 2048, 128, 2048), (2, 2176, 128, 2048),
                                     (3, 128, 320, 11008), (4, 2048, 192, 2048), (16, 1024, 128, 1024)] + STEADY)
def test_fused_whole_calls_match_the_oracle(cuda, P, M, K, H):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    N = M * H
    st = _state(P, N, "bf16")
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    _, W = _inputs(P, M, K, H, 3, cuda)
    for t in range(4):
        A, _ = _inputs(P, M, K, H, 10 + t, cuda, w=W)
        E.echo_gemm_stage1(A, W, st)
        E.echo_owner(st, E.ECHO_FWD)
        E.echo_decode(out, st)
        host = np.stack([p.reshape(-1).float().cpu().numpy() for p in _unfused(A, W)])
        o = eo.echo_call(host, so, eo.FWD)
        assert _compare(_fetch(st, out, 0), o, so, 0, True, f"call {t}") == 0


@pytest.mark.parametrize("P,M,K,H", [(3, 256, 512, 384), (8, 64, 512, 4096), (3, 192, 320, 2816),
                                     (8, 128, 3072, 1024), (4, 256, 640, 4096),
                                     (8, 128, 3072, 4096), (2, 2048, 512, 2048), (2, 2176, 512, 2048),
                                     (4, 2048, 128, 2048), (4, 2048, 576, 2048), (4, 2048, 3072, 4096)])
@pytest.mark.parametrize("sb16", [False, True])
def test_fused_sender_feedback_calls_match_the_oracle(cuda, sb16, P, M, K, H):
    """Sender feedback in the fused epilogue: each rank's carried stage-1 error
    (fp32, or bfloat16 with the bf16 state) is added to its product before the
    quantizer and updated after it, per direction; whole calls in both
    directions, interleaved, against the oracle fed the written-out partials."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    N = M * H
    st = _state(P, N, "bf16", sender_feedback=True, state_bf16=sb16)
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    _, W = _inputs(P, M, K, H, 5, cuda)
    for t in range(4):
        for d in (0, 1):
            A, _ = _inputs(P, M, K, H, 20 + 2 * t + d, cuda, w=W)
            E.echo_gemm_stage1(A, W, st, d)
            E.echo_owner(st, d)
            E.echo_decode(out, st)
            host = np.stack([p.reshape(-1).float().cpu().numpy() for p in _unfused(A, W)])
            o = eo.echo_call(host, so, d, sender_feedback=True, state_bf16=sb16)
            assert _compare(_fetch(st, out, d), o, so, d, True, f"call {t} dir {d}") == 0


def _special_inputs(case, P, M, K, H, seed, dev):
    """Inputs whose products hit the quantizer's special cases: zero rows (whole
    zero groups) and groups with one nonzero column, or every partial scaled
    by a power of two into huge, tiny or subnormal magnitudes."""
    torch = _torch()
    A, W = _inputs(P, M, K, H, seed, dev)
    for r in range(P):
        a, w = A[r].float(), W[r].float()
        if case == "zeros_and_single_columns":
            a[r::3] = 0.0                                   # these output rows are zero
            h = torch.arange(H, device=dev)
            w[((h // 32) % 2 == 0) & (h % 32 != 5 + r)] = 0.0  # every other group: one nonzero column
        elif case == "huge":
            w *= 2.0 ** 100
        elif case == "tiny":
            w *= 2.0 ** -120
        else:  # subnormal partials (and subnormal weights)
            a *= 2.0 ** -6
            w *= 2.0 ** -126
        A[r], W[r] = a.to(torch.bfloat16), w.to(torch.bfloat16)
    return A, W


@pytest.mark.parametrize("sfb", [False, True])
@pytest.mark.parametrize("case", ["zeros_and_single_columns", "huge", "tiny", "subnormal"])
@pytest.mark.parametrize("P,M,K,H", [(2, 256, 128, 256), (2, 64, 128, 2048), (2, 128, 64, 4096), (4, 256, 64, 4096),
                                     (2, 2048, 64, 2048), (4, 2048, 64, 2048)])
def test_fused_special_values_match_the_oracle(cuda, P, M, K, H, case, sfb):
    """The fused epilogue on special values, in every tile configuration, with and
    without sender feedback (bf16 state): whole calls against the oracle fed
    the written-out partials."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    N = M * H
    kw = {"sender_feedback": True, "state_bf16": True} if sfb else {}
    st = _state(P, N, "bf16", **kw)
    so = eo.OracleState(N)
    out = torch.empty(N, dtype=torch.float32, device=cuda)
    for t in range(3):
        A, W = _special_inputs(case, P, M, K, H, 40 + t, cuda)
        E.echo_gemm_stage1(A, W, st, E.ECHO_FWD)
        E.echo_owner(st, E.ECHO_FWD)
        E.echo_decode(out, st)
        host = np.stack([p.reshape(-1).float().cpu().numpy() for p in _unfused(A, W)])
        if case == "zeros_and_single_columns":
            assert np.all(host.reshape(P, M, H)[0, 0::3] == 0)
        if case == "subnormal" and t == 0:
            sub = (host != 0) & (np.abs(host) < np.finfo(np.float32).tiny)
            print(f"subnormal partials: {sub.mean():.3f} of all, {np.mean(host == 0):.3f} zero", flush=True)
            assert sub.any()
        o = eo.echo_call(host, so, eo.FWD, **kw)
        assert _compare(_fetch(st, out, 0), o, so, 0, True, f"{case} call {t}") == 0


@pytest.mark.parametrize("P,M,K,H", [(8, 64, 512, 4096), (8, 128, 256, 1024), (4, 256, 256, 4096),
                                     (4, 2048, 128, 2048)])
def test_fused_calls_in_a_graph_match_eager_calls(cuda, P, M, K, H):
    """A graph holding a fused forward call (product with stage 1 and sender
    feedback, owner step, decode), a fused backward call and the written-out
    product, replayed 4 times on new activations copied into its input tensors
    with eager work in between, leaves the same outputs, partials and carried
    state as the same sequence issued eagerly."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    N = M * H
    kw = {"sender_feedback": True, "state_bf16": True}
    se, sg = _state(P, N, "bf16", **kw), _state(P, N, "bf16", **kw)
    A0, W = _inputs(P, M, K, H, 50, cuda)
    A1, _ = _inputs(P, M, K, H, 51, cuda, w=W)
    oe, og = [torch.empty(N, dtype=torch.float32, device=cuda) for _ in range(2)]
    oe1, og1 = [torch.empty(N, dtype=torch.float32, device=cuda) for _ in range(2)]
    we = [torch.empty(M, H, dtype=torch.bfloat16, device=cuda) for _ in range(P)]
    wg = [torch.empty(M, H, dtype=torch.bfloat16, device=cuda) for _ in range(P)]

    def sequence(A0, A1, st, o, o1, written):
        E.echo_gemm_stage1(A0, W, st, E.ECHO_FWD)
        E.echo_owner(st, E.ECHO_FWD)
        E.echo_decode(o, st)
        E.echo_gemm_stage1(A1, W, st, E.ECHO_BWD)
        E.echo_owner(st, E.ECHO_BWD)
        E.echo_decode(o1, st)
        E.echo_gemm_bf16(A0, W, written)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sequence(A0, A1, sg, og, og1, wg)
    torch.cuda.synchronize()
    E.echo_reset(sg, 3)  # capture does not execute; start from a fresh state
    for k in range(4):
        N0, _ = _inputs(P, M, K, H, 60 + 2 * k, cuda, w=W)
        N1, _ = _inputs(P, M, K, H, 61 + 2 * k, cuda, w=W)
        for dst, src in zip(A0 + A1, N0 + N1):
            dst.copy_(src)
        sequence(N0, N1, se, oe, oe1, we)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(oe, og) and torch.equal(oe1, og1), f"replay {k}"
        assert all(torch.equal(a, b) for a, b in zip(we, wg)), f"replay {k} written-out product"
        for d in (0, 1):
            ve, vg = E.echo_debug_views(se, d), E.echo_debug_views(sg, d)
            for key in ("m_fast", "m_slow", "sender_err"):
                assert torch.equal(ve[key], vg[key]), f"replay {k} dir {d} {key}"
        _ = (oe * 2).sum().item()  # unrelated eager work between replays


def test_largest_row_count(cuda):
    """M = 64 * 65535, the most rows the product accepts: 65535 row blocks of 64
    in the launch grid.  Sampled row blocks (the first, one in the middle and
    the last) of the written-out product against the exact product of the same
    bf16 inputs, and the whole fused payload bit for bit against stage 1 of the
    written-out product."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P, M, K, H = 1, 64 * 65535, 64, 128
    A, W = _inputs(P, M, K, H, 9, cuda)
    out = _unfused(A, W)
    w_host = W[0].float().cpu().numpy().astype(np.float64)
    for r0 in (0, (M // 2) // 64 * 64, M - 64):
        a = A[0][r0:r0 + 64].float().cpu().numpy().astype(np.float64)
        exact = a @ w_host.T
        mag = np.abs(a) @ np.abs(w_host).T
        got = out[0][r0:r0 + 64].float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -8 + mag * K * 2.0 ** -24), f"rows {r0}.."
    N = M * H
    fused = E.echo_init_state(E.EchoConfig.make(P, N, "bf16", compensate=False), device=cuda)
    E.echo_gemm_stage1(A, W, fused)
    ref = E.echo_init_state(E.EchoConfig.make(P, N, "bf16", compensate=False), device=cuda)
    E.echo_stage1([out[0].view(-1)], ref)
    vf, vr = E.echo_debug_views(fused), E.echo_debug_views(ref)
    torch.cuda.synchronize()
    assert torch.equal(vf["codes1"], vr["codes1"]) and torch.equal(vf["scales1"], vr["scales1"])


def test_largest_k(cuda):
    """K = 2^21, the longest product accepted (a 64-row panel then spans 256 MiB
    of 32-bit buffer offsets, the K step's offset reaching 4 MiB): eight sampled
    output columns against the exact product of the same bf16 inputs, and the
    fused payload bit for bit against stage 1 of the written-out product."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    P, M, K, H = 1, 64, 1 << 21, 128
    A, W = _inputs(P, M, K, H, 13, cuda)
    out = _unfused(A, W)
    cols = [0, 1, 31, 32, 63, 64, 100, 127]
    a = A[0].float().cpu().numpy().astype(np.float64)
    w = W[0][cols].float().cpu().numpy().astype(np.float64)
    exact = a @ w.T
    mag = np.abs(a) @ np.abs(w).T
    got = out[0][:, cols].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -8 + mag * K * 2.0 ** -24)
    N = M * H
    fused = E.echo_init_state(E.EchoConfig.make(P, N, "bf16"), device=cuda)
    E.echo_gemm_stage1(A, W, fused)
    ref = E.echo_init_state(E.EchoConfig.make(P, N, "bf16"), device=cuda)
    E.echo_stage1([out[0].view(-1)], ref)
    vf, vr = E.echo_debug_views(fused), E.echo_debug_views(ref)
    torch.cuda.synchronize()
    assert torch.equal(vf["codes1"], vr["codes1"]) and torch.equal(vf["scales1"], vr["scales1"])


def test_argument_errors(cuda):
    import ctypes
    import error_compensated_bit_echo_amd as E
    from error_compensated_bit_echo_amd import binding as B
    torch = _torch()
    P, M, K, H = 2, 128, 64, 128
    A, W = _inputs(P, M, K, H, 4, cuda)
    lib = E.load_library()
    arr = lambda ts: (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = _state(P, M * H, "f32")
    assert lib.echo_gemm_stage1(arr(A), arr(W), M, K, st.handle, 0, s) == B.ECHO_ERR_DTYPE
    st = _state(P, M * H, "bf16", sender_feedback=True)
    assert lib.echo_gemm_stage1(arr(A), arr(W), M, K, st.handle, 2, s) == B.ECHO_ERR_ARG  # bad direction
    st = _state(P, M * H, "bf16", own_exact=True)  # the owner would need the partial itself
    assert lib.echo_gemm_stage1(arr(A), arr(W), M, K, st.handle, 0, s) == B.ECHO_ERR_ARG
    st = _state(P, M * H, "bf16", group=64)
    assert lib.echo_gemm_stage1(arr(A), arr(W), M, K, st.handle, 0, s) == B.ECHO_ERR_SHAPE
    st = _state(P, M * H, "bf16")
    assert lib.echo_gemm_stage1(arr(A), arr(W), 96, K, st.handle, 0, s) == B.ECHO_ERR_SHAPE  # M % 64 != 0
    assert lib.echo_gemm_stage1(arr(A), arr(W), M, 96, st.handle, 0, s) == B.ECHO_ERR_SHAPE
    bad = (ctypes.c_void_p * P)(A[0].data_ptr(), A[1].data_ptr() + 2)
    assert lib.echo_gemm_stage1(bad, arr(W), M, K, st.handle, 0, s) == B.ECHO_ERR_ARG
    # an input inside the workspace the payload is written to (rejected before any launch)
    inside = (ctypes.c_void_p * P)(A[0].data_ptr(), st.workspace.data_ptr())
    assert lib.echo_gemm_stage1(inside, arr(W), M, K, st.handle, 0, s) == B.ECHO_ERR_ARG
    assert lib.echo_gemm_stage1(arr(A), inside, M, K, st.handle, 0, s) == B.ECHO_ERR_ARG
    torch.cuda.synchronize()


def _random_shapes(n, seed):
    """n seeded product shapes: P in 1..16, M = 64 m (m <= 40), K = 64 k (k <= 24), H = 128 h (h <= 32),
    at most 48 Mi output elements over the ranks.  Seed 23 puts at least three shapes on each tile
    configuration of the launcher."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        P = int(rng.integers(1, 17))
        M = 64 * int(rng.integers(1, 41))
        K = 64 * int(rng.integers(1, 25))
        H = 128 * int(rng.integers(1, 33))
        if P * M * H <= 48 * 2 ** 20:
            shapes.append((P, M, K, H))
    return shapes


@pytest.mark.parametrize("P,M,K,H", _random_shapes(48, 23))
def test_random_shapes(cuda, P, M, K, H):
    """Seeded random shapes: sampled rows of every rank's product within the exact bound, and the
    whole fused payload equal to stage 1 of the written-out product."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    A, W = _inputs(P, M, K, H, 5, cuda)
    out = _unfused(A, W)
    rows = np.unique(np.linspace(0, M - 1, 16).astype(np.int64))
    for r in range(P):
        a = A[r][rows].float().cpu().numpy().astype(np.float64)
        w = W[r].float().cpu().numpy().astype(np.float64)
        exact = a @ w.T
        bound = np.abs(exact) * 2.0 ** -8 + (np.abs(a) @ np.abs(w).T) * K * 2.0 ** -24
        got = out[r][rows].float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - exact) <= bound), f"rank {r}"
    fused = _state(P, M * H, "bf16")
    E.echo_gemm_stage1(A, W, fused)
    ref = _state(P, M * H, "bf16")
    E.echo_stage1([o.reshape(-1) for o in out], ref)
    vf, vr = E.echo_debug_views(fused), E.echo_debug_views(ref)
    torch.cuda.synchronize()
    assert torch.equal(vf["codes1"], vr["codes1"]) and torch.equal(vf["scales1"], vr["scales1"])
