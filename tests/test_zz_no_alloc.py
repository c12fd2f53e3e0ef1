"""The all-reduce entry point that allocates nothing (echo_reduce_noalloc)
against echo_reduce, through the C ABI, on the same inputs and carried state.

The payloads it leaves in the library's static scratch are not visible to a
caller, so what is compared is what a caller sees: the output and every
carried vector (both estimates, the ranks' stage-1 errors), bit for bit, since
the same kernels run on the same values.  Calls alternate between a larger and
a smaller message, so every second call runs over a scratch that still holds
the previous call's larger payloads, and each message's second call starts
from the state its first call left.
"""
import pytest

from error_compensated_bit_echo_amd import synth
from parity_helpers import _out_tensor, _state, _torch

pytestmark = pytest.mark.gpu

VARIANTS = {
    "echo": {},
    "no_compensation": {"compensate": False},
    "sender_feedback_bf16_state": {"sender_feedback": True, "state_bf16": True},
    "sender_feedback_own_share_bf16_out": {"sender_feedback": True, "own_exact": True, "out_bf16": True},
    "bf16_state_bf16_out_group_64": {"state_bf16": True, "out_bf16": True, "group": 64},
}


class _Caller:
    """The carried vectors of one message, held as the caller's own tensors."""

    def __init__(self, cfg, device):
        torch = _torch()
        sdt = torch.bfloat16 if cfg.state_bf16 else torch.float32
        N, P = cfg.numel, cfg.P
        self.cfg = cfg
        self.m_fast = torch.zeros(N, dtype=sdt, device=device) if cfg.compensate else None
        self.m_slow = torch.zeros(N, dtype=sdt, device=device) if cfg.compensate else None
        self.sender_err = torch.zeros(P * N, dtype=sdt, device=device) if cfg.sender_feedback else None
        self.out = torch.empty(N, dtype=torch.bfloat16 if cfg.out_bf16 else torch.float32, device=device)

    def call(self, parts, stream=None):
        import error_compensated_bit_echo_amd as E
        E.echo_reduce_noalloc(self.cfg, parts, self.out, self.m_fast, self.m_slow, self.sender_err, stream)


def _assert_same(caller, st, out_ref, where):
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    v = E.echo_debug_views(st, E.ECHO_FWD)
    torch.cuda.synchronize()
    assert torch.equal(caller.out.view(torch.int16 if caller.out.dtype == torch.bfloat16 else torch.int32),
                       out_ref.view(torch.int16 if out_ref.dtype == torch.bfloat16 else torch.int32)), \
        f"output differs {where}"
    if caller.m_fast is not None:
        assert torch.equal(caller.m_fast, v["m_fast"]) and torch.equal(caller.m_slow, v["m_slow"]), \
            f"estimates differ {where}"
    if caller.sender_err is not None:
        assert torch.equal(caller.sender_err.view(st.cfg.P, -1), v["sender_err"]), f"stage-1 errors differ {where}"


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_reduce_on_two_calls_the_second_smaller(cuda, variant, dtype):
    import error_compensated_bit_echo_amd as E
    kw = dict(VARIANTS[variant])
    group = kw.pop("group", 32)
    # several tiles and a ragged tail, then a message of under a tenth of that (another tile count)
    sizes = [(3, 32 * (64 * 40 + 37) * 8 + 32 * 5), (3, 32 * 300 + 32 * 4)]
    run = []
    for P, N in sizes:
        N = N // group * group
        st = _state(P, N, dtype, group=group, **kw)
        caller = _Caller(st.cfg, cuda)
        run.append((P, N, st, caller, _out_tensor(st, cuda)))
    for t in range(2):
        for P, N, st, caller, out_ref in run:
            parts = synth.device_partials("prefill", 0, t, P=P, n=N, device=cuda)
            if dtype == "f32":
                parts = [p.float() for p in parts]
            print(f"no-alloc {variant} {dtype} P={P} N={N} call {t}", flush=True)
            E.echo_reduce(parts, out_ref, st, E.ECHO_FWD)
            caller.call(parts)
            _assert_same(caller, st, out_ref, f"{variant} {dtype} P={P} N={N} call {t}")


@pytest.mark.parametrize("workload,P,N", [("training", 4, 1 << 24), ("headline_1GiB", 8, 1 << 23),
                                          ("decode", 8, 1 << 18)])
def test_noalloc_largest_messages_that_fit(cuda, workload, P, N):
    """Messages whose payloads nearly fill the 64 MiB scratch (the training shape
    at P = 4: 50 MiB; P = 8 with 2^23 elements: 45 MiB), and the decode shape;
    two calls each, the second smaller."""
    import error_compensated_bit_echo_amd as E
    for n in (N, N // 2):
        st = _state(P, n, "bf16", poison=False)
        caller = _Caller(st.cfg, cuda)
        out_ref = _out_tensor(st, cuda)
        for t in range(2):
            parts = synth.device_partials(workload, 0, t, P=P, n=n, device=cuda)
            print(f"no-alloc {workload} P={P} N={n} call {t}", flush=True)
            E.echo_reduce(parts, out_ref, st, E.ECHO_FWD)
            caller.call(parts)
            _assert_same(caller, st, out_ref, f"{workload} P={P} N={n} call {t}")


def test_noalloc_rejects_a_message_beyond_the_scratch(cuda):
    """P = 8 with 2^24 elements needs 90 MiB of payloads: the call fails before
    launching anything, and the output and the estimates keep their values."""
    import error_compensated_bit_echo_amd as E
    from error_compensated_bit_echo_amd import binding as B
    torch = _torch()
    P, N = 8, 1 << 24
    cfg = E.EchoConfig.make(P, N, "bf16")
    caller = _Caller(cfg, cuda)
    caller.out.fill_(3.0)
    caller.m_fast.fill_(1.0)
    parts = synth.device_partials("headline_1GiB", 0, 0, P=P, n=N, device=cuda)
    with pytest.raises(E.EchoError) as err:
        caller.call(parts)
    assert err.value.status == B.ECHO_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((caller.out == 3.0).all()) and bool((caller.m_fast == 1.0).all()) and bool((caller.m_slow == 0).all())


def test_noalloc_in_a_captured_graph(cuda):
    """The use it exists for: calls captured in a HIP graph with no allocation.
    A graph of two calls (a larger and a smaller message) replayed 4 times on new
    partials copied into its inputs, with eager work in between, against the same
    calls through echo_reduce."""
    import error_compensated_bit_echo_amd as E
    torch = _torch()
    sizes = [(4, 32 * 2048 * 9 + 32 * 3), (2, 32 * 70)]
    msgs = []
    for P, N in sizes:
        st = _state(P, N, "bf16", sender_feedback=True)
        caller = _Caller(st.cfg, cuda)
        inputs = [torch.empty(N, dtype=torch.bfloat16, device=cuda) for _ in range(P)]
        msgs.append((P, N, st, caller, inputs, _out_tensor(st, cuda)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call first: the first call on a device looks the scratch up
        for P, N, st, caller, inputs, _ in msgs:
            for x in inputs:
                x.zero_()
            caller.call(inputs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for P, N, st, caller, inputs, _ in msgs:
            caller.call(inputs)
    torch.cuda.synchronize()
    for P, N, st, caller, inputs, _ in msgs:  # capture does not execute: start from zeroed state
        caller.m_fast.zero_()
        caller.m_slow.zero_()
        caller.sender_err.zero_()
    for k in range(4):
        for P, N, st, caller, inputs, out_ref in msgs:
            parts = synth.device_partials("prefill", 0, k, P=P, n=N, device=cuda)
            for dst, src in zip(inputs, parts):
                dst.copy_(src)
            E.echo_reduce(parts, out_ref, st, E.ECHO_FWD)
        print(f"no-alloc graph replay {k}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for P, N, st, caller, inputs, out_ref in msgs:
            _assert_same(caller, st, out_ref, f"graph replay {k} P={P} N={N}")
        _ = (msgs[0][5] * 2).sum().item()  # unrelated eager work between replays
