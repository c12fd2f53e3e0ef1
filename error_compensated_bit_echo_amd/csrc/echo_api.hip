// C-ABI host side of libecho: argument validation, workspace carving and the
// launches of the stage kernels on the caller's stream.  See include/echo.h
// for the contract of every entry point.
#include <new>

#include "echo.h"
#include "echo_internal.h"

namespace echo {
// The library's static scratch of ECHO_STATIC_SCRATCH_BYTES on `device` (which
// must be current): its device address, looked up on the first call per device
// and kept (echo_scratch.hip).
hipError_t static_scratch(int device, void** ptr);
}  // namespace echo

struct echo_state {
  echo_config cfg;
  int device;
  char* ws;
  size_t ws_bytes;
  uint32_t* codes1;             // stage-1 codes of all ranks
  float* scales1;               // stage-1 scales of all ranks
  int64_t codes1_stride_bytes;  // between ranks
  int64_t scales1_stride_bytes;
  uint32_t* codes2;             // broadcast payload
  float* scales2;
  float* m_fast[2];             // per direction
  float* m_slow[2];
  float* state_base;            // both directions, contiguous, then the sender errors
  int64_t vec_words;            // 4-byte words per compensator vector (fp32 or bf16, padded)
  int64_t err_words;            // 4-byte words per sender-error vector (fp32 or bf16, padded)
  float* sender_err[2];         // sender feedback: rank r of direction d at
                                // sender_err[d] + r * err_words; nullptr when off
  echo::CallPolicy policy;      // the cache policy of the calls (echo::call_policy)
};

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
  size_t codes1_stride, scales1_stride;  // bytes per rank
  size_t off_codes1, off_scales1, off_codes2, off_scales2, off_state, off_sender;
  size_t vec_bytes;                      // one compensator vector (fp32 or bf16), aligned
  size_t err_bytes;                      // one rank's sender-error vector (fp32 or bf16), aligned
  size_t total;                          // without the base-alignment slack
};

Layout make_layout(const echo_config& c) {
  const size_t N = static_cast<size_t>(c.numel);
  const size_t P = static_cast<size_t>(c.P);
  Layout L{};
  L.codes1_stride = align_up(N / 2);
  const size_t scale_bytes = 4 * (N / static_cast<size_t>(c.group));
  L.scales1_stride = align_up(scale_bytes);
  L.off_codes1 = 0;
  L.off_scales1 = L.off_codes1 + P * L.codes1_stride;
  L.off_codes2 = L.off_scales1 + P * L.scales1_stride;
  L.off_scales2 = L.off_codes2 + align_up(N / 2);
  L.off_state = L.off_scales2 + align_up(scale_bytes);
  L.vec_bytes = align_up((c.state_bf16 ? 2 : 4) * N);
  L.err_bytes = align_up((c.state_bf16 ? 2 : 4) * N);  // bf16 state: all carried state in bf16
  L.off_sender = L.off_state + 4 * L.vec_bytes;
  // sender feedback: every rank's stage-1 error, per direction, after the state
  L.total = L.off_sender + (c.sender_feedback ? 2 * P * L.err_bytes : 0);
  return L;
}

// The payload regions of a state (stage-1 codes and scales of every rank, the
// broadcast codes and scales) in the layout L, from `base` (256-byte aligned).
void carve_payload(echo_state* st, char* base, const Layout& L) {
  st->codes1 = reinterpret_cast<uint32_t*>(base + L.off_codes1);
  st->scales1 = reinterpret_cast<float*>(base + L.off_scales1);
  st->codes1_stride_bytes = static_cast<int64_t>(L.codes1_stride);
  st->scales1_stride_bytes = static_cast<int64_t>(L.scales1_stride);
  st->codes2 = reinterpret_cast<uint32_t*>(base + L.off_codes2);
  st->scales2 = reinterpret_cast<float*>(base + L.off_scales2);
}

echo_status check_cfg(const echo_config* c) {
  if (c == nullptr) return ECHO_ERR_ARG;
  if (c->P < 1 || c->P > ECHO_MAX_RANKS) return ECHO_ERR_SHAPE;
  if (c->group != 32 && c->group != 64 && c->group != 128) return ECHO_ERR_SHAPE;
  if (c->numel < 0 || c->numel > ECHO_MAX_NUMEL || c->numel % c->group != 0) return ECHO_ERR_SHAPE;
  if (c->dtype != ECHO_F32 && c->dtype != ECHO_BF16) return ECHO_ERR_DTYPE;
  if (c->compensate != 0 && c->compensate != 1) return ECHO_ERR_ARG;
  if (!(c->beta_fast >= 0.0f && c->beta_fast <= 1.0f)) return ECHO_ERR_ARG;  // also rejects NaN
  if (!(c->beta_slow >= 0.0f && c->beta_slow <= 1.0f)) return ECHO_ERR_ARG;
  if (c->sender_feedback != 0 && c->sender_feedback != 1) return ECHO_ERR_ARG;
  if (c->state_bf16 != 0 && c->state_bf16 != 1) return ECHO_ERR_ARG;
  if (c->out_bf16 != 0 && c->out_bf16 != 1) return ECHO_ERR_ARG;
  if (c->own_exact != 0 && c->own_exact != 1) return ECHO_ERR_ARG;
  return ECHO_OK;
}

echo_status check_state(const echo_state* st) {
  if (st == nullptr) return ECHO_ERR_STATE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ECHO_ERR_HIP;
  if (dev != st->device) return ECHO_ERR_STATE;
  return ECHO_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na != 0 && nb != 0 && x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(const echo_config& c) { return c.dtype == ECHO_BF16 ? 2 : 4; }

echo_status check_partials(const void* const* partials, const echo_state* st) {
  if (partials == nullptr) return ECHO_ERR_ARG;
  const size_t nb = static_cast<size_t>(st->cfg.numel) * elem_bytes(st->cfg);
  for (int r = 0; r < st->cfg.P; ++r) {
    if (partials[r] == nullptr || !aligned16(partials[r])) return ECHO_ERR_ARG;
    if (overlaps(partials[r], nb, st->ws, st->ws_bytes)) return ECHO_ERR_ARG;
  }
  return ECHO_OK;
}

echo_status check_out(const void* out, const echo_state* st, const void* const* partials) {
  if (out == nullptr || !aligned16(out)) return ECHO_ERR_ARG;
  const size_t no = static_cast<size_t>(st->cfg.numel) * (st->cfg.out_bf16 ? 2 : 4);
  if (overlaps(out, no, st->ws, st->ws_bytes)) return ECHO_ERR_ARG;
  if (partials != nullptr) {
    const size_t nb = static_cast<size_t>(st->cfg.numel) * elem_bytes(st->cfg);
    for (int r = 0; r < st->cfg.P; ++r)
      if (overlaps(out, no, partials[r], nb)) return ECHO_ERR_ARG;
  }
  return ECHO_OK;
}

// Chunks (8 elements) per owner segment: the ceil(n_groups / P) groups each owner takes.
int64_t segment_chunks(const echo_config& c) {
  const int64_t n_groups = c.numel / c.group;
  return (n_groups + c.P - 1) / c.P * (c.group / echo::kElemsPerLane);
}

echo_status run_stage1(const void* const* partials, echo_state* st, int dir, hipStream_t s) {
  echo::Stage1Args a{};
  for (int r = 0; r < echo::kMaxRanks; ++r) a.src[r] = r < st->cfg.P ? partials[r] : partials[0];
  a.codes = st->codes1;
  a.scales = st->scales1;
  a.codes_stride_words = st->codes1_stride_bytes / 4;
  a.scales_stride = st->scales1_stride_bytes / 4;
  a.nchunk = st->cfg.numel / echo::kElemsPerLane;
  a.err = st->sender_err[dir];
  a.err_stride = st->err_words;
  a.err_bf16 = st->cfg.state_bf16;
  a.own_chunks = st->cfg.own_exact ? segment_chunks(st->cfg) : 0;
  return echo::launch_stage1(a, st->cfg.P, st->cfg.dtype == ECHO_BF16, st->cfg.group, st->policy, s) ==
                 hipSuccess
             ? ECHO_OK
             : ECHO_ERR_HIP;
}

// partials: read only with own_exact (the owners' own shares)
echo_status run_owner(const void* const* partials, echo_state* st, int dir, hipStream_t s) {
  echo::OwnerArgs a{};
  for (int r = 0; r < echo::kMaxRanks; ++r) {
    const int rr = r < st->cfg.P ? r : 0;  // unused slots repeat rank 0
    a.codes1[r] = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(st->codes1) +
                                                    rr * st->codes1_stride_bytes);
    a.scales1[r] = reinterpret_cast<const float*>(reinterpret_cast<const char*>(st->scales1) +
                                                  rr * st->scales1_stride_bytes);
  }
  a.codes2 = st->codes2;
  a.scales2 = st->scales2;
  a.m_fast = st->m_fast[dir];
  a.m_slow = st->m_slow[dir];
  a.nchunk = st->cfg.numel / echo::kElemsPerLane;
  a.beta_fast = st->cfg.beta_fast;
  a.omega_fast = 1.0f - st->cfg.beta_fast;  // fl(1 - beta)
  a.beta_slow = st->cfg.beta_slow;
  a.omega_slow = 1.0f - st->cfg.beta_slow;
  a.out_bf16 = st->cfg.out_bf16;
  a.streaming = st->policy == echo::kCallStreaming ? 1 : 0;
  if (st->cfg.own_exact) {
    a.own_bf16 = st->cfg.dtype == ECHO_BF16;
    a.own_chunks = segment_chunks(st->cfg);
    for (int r = 0; r < echo::kMaxRanks; ++r) a.own_src[r] = partials[r < st->cfg.P ? r : 0];
  }
  return echo::launch_owner(a, st->cfg.P, st->cfg.compensate != 0, st->cfg.group,
                            st->cfg.state_bf16 != 0, st->cfg.own_exact != 0, s) == hipSuccess
             ? ECHO_OK
             : ECHO_ERR_HIP;
}

echo_status run_decode(void* out, const echo_state* st, hipStream_t s) {
  return echo::launch_decode(st->codes2, st->scales2, out, st->cfg.numel, st->cfg.group,
                             st->cfg.out_bf16 != 0, st->policy == echo::kCallStreaming, s) == hipSuccess
             ? ECHO_OK
             : ECHO_ERR_HIP;
}

}  // namespace

extern "C" {

size_t echo_workspace_bytes(const echo_config* cfg) {
  if (check_cfg(cfg) != ECHO_OK || cfg->numel == 0) return 0;
  return make_layout(*cfg).total + kAlign;
}

echo_status echo_init_state(const echo_config* cfg, void* workspace, size_t ws_bytes,
                            echo_stream_t stream, echo_state** out) {
  if (out == nullptr) return ECHO_ERR_ARG;
  *out = nullptr;
  const echo_status cs = check_cfg(cfg);
  if (cs != ECHO_OK) return cs;
  const size_t need = echo_workspace_bytes(cfg);
  if (cfg->numel > 0 && (workspace == nullptr || ws_bytes < need)) return ECHO_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ECHO_ERR_HIP;

  echo_state* st = new (std::nothrow) echo_state();
  if (st == nullptr) return ECHO_ERR_ARG;
  st->cfg = *cfg;
  st->device = dev;
  st->policy = echo::call_policy(cfg->P, cfg->numel, cfg->dtype == ECHO_BF16);
  st->ws = static_cast<char*>(workspace);
  st->ws_bytes = ws_bytes;
  if (cfg->numel > 0) {
    const Layout L = make_layout(*cfg);
    char* base = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(workspace)));
    carve_payload(st, base, L);
    for (int d = 0; d < 2; ++d) {
      st->m_fast[d] = reinterpret_cast<float*>(base + L.off_state + (2 * d) * L.vec_bytes);
      st->m_slow[d] = reinterpret_cast<float*>(base + L.off_state + (2 * d + 1) * L.vec_bytes);
    }
    st->state_base = reinterpret_cast<float*>(base + L.off_state);
    st->vec_words = static_cast<int64_t>(L.vec_bytes / 4);
    st->err_words = static_cast<int64_t>(L.err_bytes / 4);
    const int64_t sender_words = cfg->sender_feedback ? 2 * cfg->P * st->err_words : 0;
    for (int d = 0; d < 2; ++d)
      st->sender_err[d] = cfg->sender_feedback
                              ? reinterpret_cast<float*>(base + L.off_sender) + d * cfg->P * st->err_words
                              : nullptr;
    // the compensator vectors and the sender errors are contiguous: one fill
    // (zero bits are +0 in fp32 and in bf16)
    if (echo::launch_zero(st->state_base, 4 * st->vec_words + sender_words,
                          static_cast<hipStream_t>(stream)) != hipSuccess) {
      delete st;
      return ECHO_ERR_HIP;
    }
  }
  *out = st;
  return ECHO_OK;
}

echo_status echo_stage1(const void* const* partials, echo_state* st, echo_dir dir,
                        echo_stream_t stream) {
  echo_status e = check_state(st);
  if (e != ECHO_OK) return e;
  if (dir != ECHO_FWD && dir != ECHO_BWD) return ECHO_ERR_ARG;
  if (st->cfg.numel == 0) return ECHO_OK;
  if ((e = check_partials(partials, st)) != ECHO_OK) return e;
  return run_stage1(partials, st, static_cast<int>(dir), static_cast<hipStream_t>(stream));
}

namespace {

// The product kernel addresses each block's row panels of A and W (up to 256
// rows of K bf16) through 32-bit buffer offsets: K up to 2^21 keeps a panel
// within 1 GiB.
constexpr int64_t kGemmMaxK = int64_t(1) << 21;

// The product kernel numbers its tiles in 32-bit arithmetic: with at most 2^27
// tiles of 64 x 128 per rank (2^40 elements, far beyond device memory), 16
// ranks stay below 2^31.  The grid's row count, M / 64 at most, stays within
// the 65535 blocks a launch dimension allows.
bool gemm_shape_ok(int64_t M, int64_t K, int64_t H) {
  return M > 0 && K > 0 && H > 0 && M % echo::kGemmRowStep == 0 && H % echo::kGemmTileN == 0 &&
         K % echo::kGemmTileK == 0 && K <= kGemmMaxK && M / echo::kGemmRowStep <= 65535 &&
         H / echo::kGemmTileN <= (int64_t{1} << 26) &&
         (M / echo::kGemmRowStep) * (H / echo::kGemmTileN) <= (int64_t{1} << 27);
}

echo_status gemm_inputs(const void* const* A, const void* const* W, int P, echo::GemmArgs* a) {
  if (A == nullptr || W == nullptr) return ECHO_ERR_ARG;
  for (int r = 0; r < P; ++r)
    if (A[r] == nullptr || W[r] == nullptr || !aligned16(A[r]) || !aligned16(W[r])) return ECHO_ERR_ARG;
  for (int r = 0; r < echo::kMaxRanks; ++r) {
    a->A[r] = static_cast<const uint16_t*>(A[r < P ? r : 0]);
    a->W[r] = static_cast<const uint16_t*>(W[r < P ? r : 0]);
  }
  return ECHO_OK;
}

}  // namespace

echo_status echo_gemm_stage1(const void* const* A, const void* const* W, int64_t M, int64_t K,
                             echo_state* st, echo_dir dir, echo_stream_t stream) {
  echo_status e = check_state(st);
  if (e != ECHO_OK) return e;
  if (dir != ECHO_FWD && dir != ECHO_BWD) return ECHO_ERR_ARG;
  if (st->cfg.dtype != ECHO_BF16) return ECHO_ERR_DTYPE;
  if (st->cfg.own_exact) return ECHO_ERR_ARG;
  if (st->cfg.group != 32 || M <= 0 || st->cfg.numel % M != 0) return ECHO_ERR_SHAPE;
  const int64_t H = st->cfg.numel / M;
  if (!gemm_shape_ok(M, K, H)) return ECHO_ERR_SHAPE;
  echo::GemmArgs a{};
  if ((e = gemm_inputs(A, W, st->cfg.P, &a)) != ECHO_OK) return e;
  // the inputs are read while the payload is written: they must not overlap the workspace
  const size_t na = static_cast<size_t>(M) * static_cast<size_t>(K) * 2;
  const size_t nw = static_cast<size_t>(H) * static_cast<size_t>(K) * 2;
  for (int r = 0; r < st->cfg.P; ++r)
    if (overlaps(A[r], na, st->ws, st->ws_bytes) || overlaps(W[r], nw, st->ws, st->ws_bytes))
      return ECHO_ERR_ARG;
  a.codes = st->codes1;
  a.scales = st->scales1;
  a.codes_stride_words = st->codes1_stride_bytes / 4;
  a.scales_stride = st->scales1_stride_bytes / 4;
  a.M = M;
  a.K = K;
  a.H = H;
  a.err = st->sender_err[dir];  // sender feedback: the ranks' stage-1 errors of `dir`
  a.err_stride = st->err_words;
  a.err_bf16 = st->cfg.state_bf16;
  return echo::launch_gemm(a, st->cfg.P, true, static_cast<hipStream_t>(stream)) == hipSuccess
             ? ECHO_OK
             : ECHO_ERR_HIP;
}

echo_status echo_gemm_bf16(const void* const* A, const void* const* W, void* const* out, int32_t P,
                           int64_t M, int64_t K, int64_t H, echo_stream_t stream) {
  if (P < 1 || P > ECHO_MAX_RANKS || !gemm_shape_ok(M, K, H)) return ECHO_ERR_SHAPE;
  if (out == nullptr) return ECHO_ERR_ARG;
  echo::GemmArgs a{};
  echo_status e = gemm_inputs(A, W, P, &a);
  if (e != ECHO_OK) return e;
  const size_t nout = static_cast<size_t>(M) * static_cast<size_t>(H) * 2;
  const size_t na = static_cast<size_t>(M) * static_cast<size_t>(K) * 2;
  const size_t nw = static_cast<size_t>(H) * static_cast<size_t>(K) * 2;
  for (int r = 0; r < P; ++r) {
    if (out[r] == nullptr || !aligned16(out[r])) return ECHO_ERR_ARG;
    for (int q = 0; q < P; ++q)
      if (overlaps(out[r], nout, A[q], na) || overlaps(out[r], nout, W[q], nw) ||
          (q != r && overlaps(out[r], nout, out[q], nout)))
        return ECHO_ERR_ARG;
  }
  for (int r = 0; r < echo::kMaxRanks; ++r) a.out[r] = static_cast<uint16_t*>(out[r < P ? r : 0]);
  a.M = M;
  a.K = K;
  a.H = H;
  return echo::launch_gemm(a, P, false, static_cast<hipStream_t>(stream)) == hipSuccess ? ECHO_OK
                                                                                      : ECHO_ERR_HIP;
}

echo_status echo_owner(const void* const* partials, echo_state* st, echo_dir dir,
                       echo_stream_t stream) {
  echo_status e = check_state(st);
  if (e != ECHO_OK) return e;
  if (dir != ECHO_FWD && dir != ECHO_BWD) return ECHO_ERR_ARG;
  if (st->cfg.numel == 0) return ECHO_OK;
  if (st->cfg.own_exact && (e = check_partials(partials, st)) != ECHO_OK) return e;
  return run_owner(partials, st, static_cast<int>(dir), static_cast<hipStream_t>(stream));
}

echo_status echo_decode(void* out, const echo_state* st, echo_stream_t stream) {
  echo_status e = check_state(st);
  if (e != ECHO_OK) return e;
  if (st->cfg.numel == 0) return ECHO_OK;
  if ((e = check_out(out, st, nullptr)) != ECHO_OK) return e;
  return run_decode(out, st, static_cast<hipStream_t>(stream));
}

echo_status echo_reduce(const void* const* partials, void* out, echo_state* st, echo_dir dir,
                        echo_stream_t stream) {
  echo_status e = check_state(st);
  if (e != ECHO_OK) return e;
  if (dir != ECHO_FWD && dir != ECHO_BWD) return ECHO_ERR_ARG;
  if (st->cfg.numel == 0) return ECHO_OK;
  if ((e = check_partials(partials, st)) != ECHO_OK) return e;
  if ((e = check_out(out, st, partials)) != ECHO_OK) return e;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((e = run_stage1(partials, st, static_cast<int>(dir), s)) != ECHO_OK) return e;
  if ((e = run_owner(partials, st, static_cast<int>(dir), s)) != ECHO_OK) return e;
  return run_decode(out, st, s);
}

echo_status echo_reduce_noalloc(const echo_config* cfg, const void* const* partials, void* out, void* m_fast,
                                void* m_slow, void* sender_err, echo_stream_t stream) {
  echo_status e = check_cfg(cfg);
  if (e != ECHO_OK) return e;
  if (cfg->numel == 0) return ECHO_OK;
  // the payloads go to the static scratch: only messages whose payloads fit
  const Layout L = make_layout(*cfg);
  if (L.off_state > ECHO_STATIC_SCRATCH_BYTES) return ECHO_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ECHO_ERR_HIP;
  void* scratch = nullptr;
  if (echo::static_scratch(dev, &scratch) != hipSuccess || scratch == nullptr) return ECHO_ERR_HIP;

  // a state on the stack over the scratch, with the caller's carried vectors
  // standing in for both directions' (nothing is allocated)
  echo_state st{};
  st.cfg = *cfg;
  st.device = dev;
  st.policy = echo::call_policy(cfg->P, cfg->numel, cfg->dtype == ECHO_BF16);
  st.ws = static_cast<char*>(scratch);
  st.ws_bytes = L.off_state;
  carve_payload(&st, st.ws, L);
  const size_t N = static_cast<size_t>(cfg->numel);
  const size_t vb = (cfg->state_bf16 ? 2 : 4) * N;  // one carried vector
  const size_t eb = static_cast<size_t>(cfg->P) * vb;  // the ranks' stage-1 errors
  if (cfg->compensate) {
    if (m_fast == nullptr || m_slow == nullptr || !aligned16(m_fast) || !aligned16(m_slow)) return ECHO_ERR_ARG;
    if (overlaps(m_fast, vb, m_slow, vb)) return ECHO_ERR_ARG;
  } else {
    m_fast = m_slow = nullptr;  // not touched without compensation
  }
  if (cfg->sender_feedback) {
    if (sender_err == nullptr || !aligned16(sender_err)) return ECHO_ERR_ARG;
    if (overlaps(sender_err, eb, m_fast, m_fast ? vb : 0) || overlaps(sender_err, eb, m_slow, m_slow ? vb : 0))
      return ECHO_ERR_ARG;
  } else if (sender_err != nullptr) {
    return ECHO_ERR_ARG;
  }
  for (int d = 0; d < 2; ++d) {
    st.m_fast[d] = static_cast<float*>(m_fast);
    st.m_slow[d] = static_cast<float*>(m_slow);
    st.sender_err[d] = static_cast<float*>(sender_err);
  }
  st.err_words = static_cast<int64_t>(vb / 4);  // rank r's errors at sender_err + r * N elements
  if ((e = check_partials(partials, &st)) != ECHO_OK) return e;
  if ((e = check_out(out, &st, partials)) != ECHO_OK) return e;
  // the carried vectors overlap neither the partials nor the output
  const size_t pb = N * elem_bytes(*cfg), ob = N * (cfg->out_bf16 ? 2 : 4);
  const void* carried[3] = {m_fast, m_slow, sender_err};
  const size_t cb[3] = {vb, vb, eb};
  for (int k = 0; k < 3; ++k) {
    if (carried[k] == nullptr) continue;
    if (overlaps(carried[k], cb[k], out, ob) || overlaps(carried[k], cb[k], st.ws, st.ws_bytes)) return ECHO_ERR_ARG;
    for (int r = 0; r < cfg->P; ++r)
      if (overlaps(carried[k], cb[k], partials[r], pb)) return ECHO_ERR_ARG;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((e = run_stage1(partials, &st, 0, s)) != ECHO_OK) return e;
  if ((e = run_owner(partials, &st, 0, s)) != ECHO_OK) return e;
  return run_decode(out, &st, s);
}

echo_status echo_reset(echo_state* st, int dir_mask, echo_stream_t stream) {
  echo_status e = check_state(st);
  if (e != ECHO_OK) return e;
  if (dir_mask < 1 || dir_mask > 3) return ECHO_ERR_ARG;
  if (st->cfg.numel == 0) return ECHO_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int d = 0; d < 2; ++d) {
    if (!(dir_mask & (1 << d))) continue;
    // m_fast[d] and m_slow[d] are adjacent: one fill covers both
    if (echo::launch_zero(st->m_fast[d], 2 * st->vec_words, s) != hipSuccess) return ECHO_ERR_HIP;
    if (st->sender_err[d] != nullptr &&
        echo::launch_zero(st->sender_err[d], st->cfg.P * st->err_words, s) != hipSuccess)
      return ECHO_ERR_HIP;
  }
  return ECHO_OK;
}

void echo_destroy_state(echo_state* st) { delete st; }

echo_status echo_wire_bytes(const echo_state* st, uint64_t* rs_per_rank, uint64_t* ag_per_rank,
                            uint64_t* bf16_allreduce_per_rank) {
  if (st == nullptr) return ECHO_ERR_STATE;
  if (rs_per_rank == nullptr || ag_per_rank == nullptr || bf16_allreduce_per_rank == nullptr)
    return ECHO_ERR_ARG;
  const uint64_t P = static_cast<uint64_t>(st->cfg.P);
  const uint64_t N = static_cast<uint64_t>(st->cfg.numel);
  const uint64_t G = static_cast<uint64_t>(st->cfg.group);
  const uint64_t n_g = N / G;
  const uint64_t per = (n_g + P - 1) / P;
  const uint64_t bytes_per_group = G / 2 + 4;  // codes + one fp32 scale
  uint64_t total = 0, smallest = UINT64_MAX, largest = 0;
  for (uint64_t j = 0; j < P; ++j) {
    const uint64_t lo = j * per < n_g ? j * per : n_g;
    const uint64_t hi = (j + 1) * per < n_g ? (j + 1) * per : n_g;
    const uint64_t b = (hi - lo) * bytes_per_group;
    total += b;
    smallest = b < smallest ? b : smallest;
    largest = b > largest ? b : largest;
  }
  *rs_per_rank = total - smallest;  // a rank keeps its own segment
  *ag_per_rank = (P - 1) * largest;
  *bf16_allreduce_per_rank = (2 * (P - 1) * 2 * N) / P;
  return ECHO_OK;
}

echo_status echo_debug_views(const echo_state* st, echo_dir dir, echo_views* out) {
  if (st == nullptr) return ECHO_ERR_STATE;
  if (out == nullptr || (dir != ECHO_FWD && dir != ECHO_BWD)) return ECHO_ERR_ARG;
  out->stage1_codes = st->codes1;
  out->stage1_scales = st->scales1;
  out->stage1_codes_stride = static_cast<size_t>(st->codes1_stride_bytes);
  out->stage1_scales_stride = static_cast<size_t>(st->scales1_stride_bytes);
  out->bcast_codes = st->codes2;
  out->bcast_scales = st->scales2;
  out->m_fast = st->m_fast[dir];
  out->m_slow = st->m_slow[dir];
  out->sender_err = st->sender_err[dir];
  out->sender_err_stride = st->sender_err[dir] != nullptr ? static_cast<size_t>(4 * st->err_words) : 0;
  return ECHO_OK;
}

const char* echo_status_str(echo_status s) {
  switch (s) {
    case ECHO_OK: return "ok";
    case ECHO_ERR_ARG: return "invalid argument (null, misaligned or overlapping pointer, bad enum)";
    case ECHO_ERR_SHAPE:
      return "invalid shape (P outside [1,16], group not 32/64/128, numel not a multiple of the group or too large)";
    case ECHO_ERR_DTYPE: return "invalid dtype";
    case ECHO_ERR_WORKSPACE:
      return "workspace missing or too small (echo_reduce_noalloc: the payloads exceed the static scratch)";
    case ECHO_ERR_STATE: return "null state, or another device is current";
    case ECHO_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
