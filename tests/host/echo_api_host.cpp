// The C-ABI host code of libecho as one host-only translation unit, for the
// host-logic check (the kernels are replaced by echo_host_stubs.cpp).
#include "echo_api.hip"
