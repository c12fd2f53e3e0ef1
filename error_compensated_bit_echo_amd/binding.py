"""ctypes binding of libecho (include/echo.h), argument marshalling only.

The names are the C names.  Tensors are torch device tensors; torch provides
device memory and streams, every step of the all-reduce runs in libecho's HIP
kernels.  There is no fallback: if the library cannot be loaded, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))

ECHO_OK = 0
ECHO_ERR_ARG = 1
ECHO_ERR_SHAPE = 2
ECHO_ERR_DTYPE = 3
ECHO_ERR_WORKSPACE = 4
ECHO_ERR_STATE = 5
ECHO_ERR_HIP = 6

ECHO_F32 = 0
ECHO_BF16 = 1
ECHO_FWD = 0
ECHO_BWD = 1
ECHO_GROUP = 32
ECHO_MAX_RANKS = 16


class EchoConfig(ctypes.Structure):
    _fields_ = [
        ("P", ctypes.c_int32),
        ("numel", ctypes.c_int64),
        ("group", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("compensate", ctypes.c_int32),
        ("beta_fast", ctypes.c_float),
        ("beta_slow", ctypes.c_float),
        ("sender_feedback", ctypes.c_int32),
        ("state_bf16", ctypes.c_int32),
        ("out_bf16", ctypes.c_int32),
        ("own_exact", ctypes.c_int32),
    ]

    @classmethod
    def make(cls, P: int, numel: int, dtype: str = "bf16", compensate: bool = True,
             beta_fast: float = 0.5, beta_slow: float = 0.95, group: int = ECHO_GROUP,
             sender_feedback: bool = False, state_bf16: bool = False, out_bf16: bool = False,
             own_exact: bool = False) -> "EchoConfig":
        d = {"f32": ECHO_F32, "float32": ECHO_F32, "bf16": ECHO_BF16, "bfloat16": ECHO_BF16}
        if dtype not in d:
            raise EchoError(ECHO_ERR_DTYPE, f"dtype {dtype!r}")
        return cls(P, numel, group, d[dtype], int(bool(compensate)), beta_fast, beta_slow,
                   int(bool(sender_feedback)), int(bool(state_bf16)), int(bool(out_bf16)),
                   int(bool(own_exact)))


class EchoViews(ctypes.Structure):
    _fields_ = [
        ("stage1_codes", ctypes.c_void_p),
        ("stage1_scales", ctypes.c_void_p),
        ("stage1_codes_stride", ctypes.c_size_t),
        ("stage1_scales_stride", ctypes.c_size_t),
        ("bcast_codes", ctypes.c_void_p),
        ("bcast_scales", ctypes.c_void_p),
        ("m_fast", ctypes.c_void_p),
        ("m_slow", ctypes.c_void_p),
        ("sender_err", ctypes.c_void_p),
        ("sender_err_stride", ctypes.c_size_t),
    ]


class EchoError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = _status_text(status)
        super().__init__(f"{what}: {msg} (status {status})" if what else f"{msg} (status {status})")


_lib = None


def library_path() -> str:
    return os.path.join(_PKG, "libecho.so")


def load_library():
    """Load libecho.so; it is built in-tree first only if it does not exist."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        from . import build
        build.build_library()
    lib = ctypes.CDLL(path)
    vp, sz, i32, u64p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64)
    cfgp = ctypes.POINTER(EchoConfig)
    sig = {
        "echo_workspace_bytes": (sz, [cfgp]),
        "echo_init_state": (i32, [cfgp, vp, sz, vp, ctypes.POINTER(vp)]),
        "echo_reduce": (i32, [ctypes.POINTER(vp), vp, vp, i32, vp]),
        "echo_stage1": (i32, [ctypes.POINTER(vp), vp, i32, vp]),
        "echo_owner": (i32, [ctypes.POINTER(vp), vp, i32, vp]),
        "echo_gemm_stage1": (i32, [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int64, ctypes.c_int64, vp, i32,
                                   vp]),
        "echo_gemm_bf16": (i32, [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int32,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp]),
        "echo_decode": (i32, [vp, vp, vp]),
        "echo_reset": (i32, [vp, i32, vp]),
        "echo_reduce_noalloc": (i32, [cfgp, ctypes.POINTER(vp), vp, vp, vp, vp, vp]),
        "echo_destroy_state": (None, [vp]),
        "echo_wire_bytes": (i32, [vp, u64p, u64p, u64p]),
        "echo_debug_views": (i32, [vp, i32, ctypes.POINTER(EchoViews)]),
        "echo_status_str": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load_library().echo_status_str(status).decode()
    except Exception:  # the library itself failed to load
        return f"status {status}"


def echo_status_str(status: int) -> str:
    return load_library().echo_status_str(status).decode()


def _check(status: int, what: str):
    if status != ECHO_OK:
        raise EchoError(status, what)


_raw_stream = None  # torch's getter of the current stream's raw handle, if it has one


def _stream_handle(stream, device):
    """The hipStream_t of ``stream``, or of torch's current stream on ``device``.
    The current stream is read through torch's raw-handle getter when torch
    provides it (a twentieth of the time of building a Stream object)."""
    global _raw_stream
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    import torch
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream:
        index = device.index if device.index is not None else torch.cuda.current_device()
        return ctypes.c_void_p(_raw_stream(index))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class EchoState:
    """Host handle + the torch workspace tensor it carves (kept alive here)."""

    def __init__(self, handle: ctypes.c_void_p, cfg: EchoConfig, workspace, device):
        self.handle = handle
        self.cfg = cfg
        self.workspace = workspace
        self.device = device
        self.ptr_array_type = ctypes.c_void_p * cfg.P  # the host array of P device pointers

    @property
    def P(self) -> int:
        return self.cfg.P

    @property
    def numel(self) -> int:
        return self.cfg.numel

    def close(self):
        if self.handle is not None and self.handle.value is not None:
            load_library().echo_destroy_state(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def echo_workspace_bytes(cfg: EchoConfig) -> int:
    return int(load_library().echo_workspace_bytes(ctypes.byref(cfg)))


def echo_init_state(cfg: EchoConfig, workspace=None, stream=None, device=None) -> EchoState:
    """Create a state.  ``workspace`` is a uint8 device tensor; allocated if None."""
    import torch
    lib = load_library()
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    need = echo_workspace_bytes(cfg)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    ptr = workspace.data_ptr() if workspace.numel() else None
    h = ctypes.c_void_p()
    with torch.cuda.device(device):
        st = lib.echo_init_state(ctypes.byref(cfg), ptr, workspace.numel(),
                                 _stream_handle(stream, device), ctypes.byref(h))
    _check(st, "echo_init_state")
    return EchoState(h, cfg, workspace, device)


def _partials_array(partials: Sequence, state: EchoState):
    import torch
    cfg = state.cfg
    P, N = cfg.P, cfg.numel
    want = torch.bfloat16 if cfg.dtype == ECHO_BF16 else torch.float32
    if len(partials) != P:
        raise EchoError(ECHO_ERR_ARG, f"expected {P} partials, got {len(partials)}")
    dev = state.device
    for t in partials:
        if t.dtype != want:
            raise EchoError(ECHO_ERR_DTYPE, f"partial dtype {t.dtype}, expected {want}")
        if t.numel() != N or not t.is_contiguous() or t.device != dev:
            raise EchoError(ECHO_ERR_ARG, "partials must be contiguous, numel == N, on the state's device")
    return state.ptr_array_type(*[t.data_ptr() for t in partials])


def _out_ptr(out, state: EchoState):
    import torch
    want = torch.bfloat16 if state.cfg.out_bf16 else torch.float32
    if out.dtype != want or out.numel() != state.cfg.numel or not out.is_contiguous() \
            or out.device != state.device:
        raise EchoError(ECHO_ERR_ARG, f"out must be a contiguous {want} tensor of N elements on the state's device")
    return ctypes.c_void_p(out.data_ptr())


def echo_reduce(partials: Sequence, out, state: EchoState, direction: int = ECHO_FWD, stream=None):
    """One Echo all-reduce of ``partials`` (P device tensors) into ``out`` (fp32, or
    bfloat16 with the out_bf16 variant)."""
    arr = _partials_array(partials, state)
    optr = _out_ptr(out, state)
    _check(load_library().echo_reduce(arr, optr, state.handle, int(direction),
                                      _stream_handle(stream, state.device)), "echo_reduce")
    return out


def echo_stage1(partials: Sequence, state: EchoState, direction: int = ECHO_FWD, stream=None):
    arr = _partials_array(partials, state)
    _check(load_library().echo_stage1(arr, state.handle, int(direction),
                                      _stream_handle(stream, state.device)), "echo_stage1")


def _bf16_matrices(mats, rows, cols, what):
    import torch
    for t in mats:
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (rows, cols) or not t.is_contiguous():
            raise EchoError(ECHO_ERR_ARG, f"{what} must be contiguous bfloat16 [{rows}, {cols}]")
    return (ctypes.c_void_p * len(mats))(*[t.data_ptr() for t in mats])


def echo_gemm_stage1(A: Sequence, W: Sequence, state: EchoState, direction: int = ECHO_FWD, stream=None):
    """Stage 1 fused into the producing product: the payload of bf16(A_r @ W_r.T)
    for every rank (A_r [M, K], W_r [H, K] bfloat16, M*H == N); with sender
    feedback the ranks' stage-1 errors of ``direction`` are used and updated."""
    P = state.cfg.P
    if len(A) != P or len(W) != P:
        raise EchoError(ECHO_ERR_ARG, f"expected {P} A and {P} W matrices")
    M, K = A[0].shape
    H = W[0].shape[0]
    a = _bf16_matrices(A, M, K, "A")
    w = _bf16_matrices(W, H, K, "W")
    _check(load_library().echo_gemm_stage1(a, w, M, K, state.handle, int(direction),
                                           _stream_handle(stream, state.device)), "echo_gemm_stage1")


def echo_gemm_bf16(A: Sequence, W: Sequence, out: Sequence, stream=None):
    """out[r] = bf16(A_r @ W_r.T), the product echo_gemm_stage1 quantizes."""
    P = len(A)
    if P < 1 or len(W) != P or len(out) != P:
        raise EchoError(ECHO_ERR_ARG, "A, W and out must hold the same number (>= 1) of matrices")
    M, K = A[0].shape
    H = W[0].shape[0]
    a = _bf16_matrices(A, M, K, "A")
    w = _bf16_matrices(W, H, K, "W")
    o = _bf16_matrices(out, M, H, "out")
    _check(load_library().echo_gemm_bf16(a, w, o, P, M, K, H, _stream_handle(stream, A[0].device)),
           "echo_gemm_bf16")


def echo_owner(state: EchoState, direction: int = ECHO_FWD, stream=None, partials=None):
    """Owner stage.  ``partials`` (the ones echo_stage1 received) are needed with own_exact."""
    arr = _partials_array(partials, state) if partials is not None else None
    _check(load_library().echo_owner(arr, state.handle, int(direction),
                                      _stream_handle(stream, state.device)), "echo_owner")


def echo_decode(out, state: EchoState, stream=None):
    optr = _out_ptr(out, state)
    _check(load_library().echo_decode(optr, state.handle, _stream_handle(stream, state.device)),
           "echo_decode")
    return out


ECHO_STATIC_SCRATCH_BYTES = 64 << 20


def echo_reduce_noalloc(cfg: EchoConfig, partials: Sequence, out, m_fast=None, m_slow=None, sender_err=None,
                        stream=None):
    """One all-reduce through the entry point that allocates nothing: the
    payloads go to the library's static scratch and the carried state is the
    caller's tensors (m_fast, m_slow: N fp32, or bfloat16 with state_bf16;
    sender_err: [P, N] with sender feedback), advanced in place."""
    import torch
    P, N = cfg.P, cfg.numel
    want = torch.bfloat16 if cfg.dtype == ECHO_BF16 else torch.float32
    if len(partials) != P or any(t.dtype != want or t.numel() != N or not t.is_contiguous() for t in partials):
        raise EchoError(ECHO_ERR_ARG, f"expected {P} contiguous {want} partials of {N} elements")
    sdt = torch.bfloat16 if cfg.state_bf16 else torch.float32
    for name, t, n in (("m_fast", m_fast, N), ("m_slow", m_slow, N), ("sender_err", sender_err, P * N)):
        if t is not None and (t.dtype != sdt or t.numel() != n or not t.is_contiguous()):
            raise EchoError(ECHO_ERR_ARG, f"{name} must be a contiguous {sdt} tensor of {n} elements")
    odt = torch.bfloat16 if cfg.out_bf16 else torch.float32
    if out.dtype != odt or out.numel() != N or not out.is_contiguous():
        raise EchoError(ECHO_ERR_ARG, f"out must be a contiguous {odt} tensor of {N} elements")
    arr = (ctypes.c_void_p * P)(*[t.data_ptr() for t in partials])
    ptr = lambda t: None if t is None else t.data_ptr()
    _check(load_library().echo_reduce_noalloc(ctypes.byref(cfg), arr, out.data_ptr(), ptr(m_fast), ptr(m_slow),
                                              ptr(sender_err), _stream_handle(stream, out.device)),
           "echo_reduce_noalloc")
    return out


def echo_reset(state: EchoState, dir_mask: int = 3, stream=None):
    _check(load_library().echo_reset(state.handle, int(dir_mask),
                                      _stream_handle(stream, state.device)), "echo_reset")


def echo_destroy_state(state: EchoState):
    state.close()


def echo_wire_bytes(state: EchoState) -> dict:
    rs, ag, bf = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(load_library().echo_wire_bytes(state.handle, ctypes.byref(rs), ctypes.byref(ag),
                                          ctypes.byref(bf)), "echo_wire_bytes")
    return {"rs_per_rank": rs.value, "ag_per_rank": ag.value, "bf16_allreduce_per_rank": bf.value}


def echo_debug_views(state: EchoState, direction: int = ECHO_FWD) -> dict:
    """Views (no copies) into the workspace: stage-1 codes [P, N/2] and scales [P, N/group],
    broadcast codes [N/2] and scales [N/group], the m_fast / m_slow vectors of ``direction``
    and, with sender feedback, the ranks' stage-1 errors [P, N] of ``direction``."""
    import torch
    v = EchoViews()
    _check(load_library().echo_debug_views(state.handle, int(direction), ctypes.byref(v)),
           "echo_debug_views")
    ws = state.workspace
    base = ws.data_ptr()
    N, P, G = state.cfg.numel, state.cfg.P, state.cfg.group
    if N == 0:
        e8 = torch.empty(0, dtype=torch.uint8, device=state.device)
        e32 = torch.empty(0, dtype=torch.float32, device=state.device)
        return {"codes1": e8.view(0, 0).expand(P, 0), "scales1": e32.view(0, 0).expand(P, 0),
                "codes2": e8, "scales2": e32, "m_fast": e32, "m_slow": e32, "sender_err": None}

    def sl(ptr, nbytes):
        off = ptr - base
        return ws[off:off + nbytes]

    cs, ss = v.stage1_codes_stride, v.stage1_scales_stride
    sb, sdt = (2, torch.bfloat16) if state.cfg.state_bf16 else (4, torch.float32)
    codes1 = sl(v.stage1_codes, P * cs).view(P, cs)[:, :N // 2]
    scales1 = sl(v.stage1_scales, P * ss).view(torch.float32).view(P, ss // 4)[:, :N // G]
    return {
        "codes1": codes1,
        "scales1": scales1,
        "codes2": sl(v.bcast_codes, N // 2),
        "scales2": sl(v.bcast_scales, 4 * (N // G)).view(torch.float32),
        # bfloat16 vectors with the state_bf16 variant, fp32 otherwise
        "m_fast": sl(v.m_fast, sb * N).view(sdt),
        "m_slow": sl(v.m_slow, sb * N).view(sdt),
        # sender feedback: [P, N] stage-1 errors of the ranks for ``direction``
        # (bfloat16 with the state_bf16 variant)
        "sender_err": None if not v.sender_err else
        sl(v.sender_err, P * v.sender_err_stride).view(sdt)
        .view(P, v.sender_err_stride // sb)[:, :N],
    }
