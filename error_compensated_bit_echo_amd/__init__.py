"""Echo error-compensated int4 all-reduce on AMD MI355X (gfx950).

The compute lives in ``libecho.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/echo.h``).  ``error_compensated_bit_echo_amd.binding``
marshals torch tensors into that ABI; the names it exports are the C names.
Importing the package itself loads nothing; the library is loaded on first use
of a binding name.
"""
_BINDING_NAMES = {
    "EchoConfig", "EchoError", "EchoState", "ECHO_FWD", "ECHO_BWD",
    "echo_workspace_bytes", "echo_init_state", "echo_reduce", "echo_stage1",
    "echo_owner", "echo_decode", "echo_gemm_stage1", "echo_gemm_bf16", "echo_reset", "echo_destroy_state",
    "echo_reduce_noalloc", "ECHO_STATIC_SCRATCH_BYTES",
    "echo_wire_bytes", "echo_debug_views", "echo_status_str", "library_path",
    "load_library",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
