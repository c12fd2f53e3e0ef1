// Host-logic check of libecho's C ABI on a machine without a GPU.  The host
// code (include/echo.h; csrc/echo_api.hip) runs against the recording
// stand-ins of echo_host_stubs.cpp: workspaces and tensors are fake device
// addresses that the host code only does arithmetic on, so messages up to the
// largest the ABI accepts can be carved.  For every configuration it checks
// that
//   * the regions the state carves (stage-1 payload of every rank, broadcast
//     payload, both compensator vectors of both directions, the ranks'
//     sender errors) lie inside the workspace, start 256-byte aligned and do
//     not overlap, and the debug views point at them;
//   * every launch of echo_init_state, echo_reduce, the stage entry points,
//     echo_reset and echo_gemm_stage1 receives exactly those regions, with
//     extents (what the kernels address for the launch's chunk count) inside
//     them, and the configuration's coefficients;
//   * bad arguments launch nothing and leave the state as it was;
//   * echo_wire_bytes matches a direct count of the owner segments.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_logic_cpu.py; prints "ok" and exits 0 when every check holds.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "echo.h"
#include "echo_host_stubs.h"

namespace {

int g_failures = 0;
int g_checks = 0;

#define CHECK(cond, ...)                                          \
  do {                                                            \
    ++g_checks;                                                   \
    if (!(cond)) {                                                \
      if (++g_failures <= 40) {                                   \
        std::fprintf(stderr, "FAIL line %d [%s]: ", __LINE__, g_ctx.c_str()); \
        std::fprintf(stderr, __VA_ARGS__);                        \
        std::fprintf(stderr, "\n");                               \
      }                                                           \
    }                                                             \
  } while (0)

std::string g_ctx;

typedef unsigned long long u64;

struct Region {
  std::string what;
  u64 lo, hi;  // [lo, hi)
};

u64 addr(const void* p) { return static_cast<u64>(reinterpret_cast<uintptr_t>(p)); }
void* fake(u64 a) { return reinterpret_cast<void*>(static_cast<uintptr_t>(a)); }

bool inside(const Region& inner, const Region& outer) {
  return inner.lo >= outer.lo && inner.hi <= outer.hi && inner.lo <= inner.hi;
}

struct Case {
  int P;
  int64_t N;
  int group;
  echo_dtype dtype;
  int compensate, sfb, sb16, obf, own;
};

echo_config make_cfg(const Case& c) {
  echo_config cfg;
  std::memset(&cfg, 0, sizeof(cfg));
  cfg.P = c.P;
  cfg.numel = c.N;
  cfg.group = c.group;
  cfg.dtype = c.dtype;
  cfg.compensate = c.compensate;
  cfg.beta_fast = 0.5f;
  cfg.beta_slow = 0.95f;
  cfg.sender_feedback = c.sfb;
  cfg.state_bf16 = c.sb16;
  cfg.out_bf16 = c.obf;
  cfg.own_exact = c.own;
  return cfg;
}

// The state's regions, from its debug views, with the sizes the header states.
std::vector<Region> regions(echo_state* st, const Case& c) {
  std::vector<Region> rs;
  const u64 N = static_cast<u64>(c.N), G = static_cast<u64>(c.group);
  const u64 sv = c.sb16 ? 2 : 4;  // bytes per element of the carried state
  for (int d = 0; d < 2; ++d) {
    echo_views v;
    CHECK(echo_debug_views(st, static_cast<echo_dir>(d), &v) == ECHO_OK, "views");
    if (d == 0) {
      for (int r = 0; r < c.P; ++r) {
        rs.push_back({"codes1[" + std::to_string(r) + "]", addr(v.stage1_codes) + r * v.stage1_codes_stride,
                      addr(v.stage1_codes) + r * v.stage1_codes_stride + N / 2});
        rs.push_back({"scales1[" + std::to_string(r) + "]", addr(v.stage1_scales) + r * v.stage1_scales_stride,
                      addr(v.stage1_scales) + r * v.stage1_scales_stride + 4 * (N / G)});
      }
      CHECK(v.stage1_codes_stride >= N / 2 && v.stage1_scales_stride >= 4 * (N / G), "strides");
      rs.push_back({"codes2", addr(v.bcast_codes), addr(v.bcast_codes) + N / 2});
      rs.push_back({"scales2", addr(v.bcast_scales), addr(v.bcast_scales) + 4 * (N / G)});
    }
    const std::string dn = d ? "bwd" : "fwd";
    rs.push_back({"m_fast " + dn, addr(v.m_fast), addr(v.m_fast) + sv * N});
    rs.push_back({"m_slow " + dn, addr(v.m_slow), addr(v.m_slow) + sv * N});
    if (c.sfb) {
      CHECK(v.sender_err != nullptr && v.sender_err_stride >= sv * N, "sender views");
      for (int r = 0; r < c.P; ++r)
        rs.push_back({"sender_err " + dn + "[" + std::to_string(r) + "]",
                      addr(v.sender_err) + r * v.sender_err_stride,
                      addr(v.sender_err) + r * v.sender_err_stride + sv * N});
    } else {
      CHECK(v.sender_err == nullptr && v.sender_err_stride == 0, "no sender errors without sender feedback");
    }
  }
  return rs;
}

const Region* find(const std::vector<Region>& rs, const std::string& what) {
  for (const Region& r : rs)
    if (r.what == what) return &r;
  return nullptr;
}

void check_stage1(const HostLaunch& l, const Case& c, const std::vector<Region>& rs, const void* const* parts,
                  int dir, const Region& ws) {
  const echo::Stage1Args& a = l.stage1;
  const u64 N = static_cast<u64>(c.N);
  CHECK(l.P == c.P && l.group == c.group && l.flag == (c.dtype == ECHO_BF16), "stage-1 launch shape");
  CHECK(a.nchunk == c.N / 8, "stage-1 chunks");
  for (int r = 0; r < echo::kMaxRanks; ++r)
    CHECK(a.src[r] == parts[r < c.P ? r : 0], "stage-1 source of rank %d", r);
  const int lpg = c.group / 8;
  for (int r = 0; r < c.P; ++r) {
    // what the kernel addresses: code words [0, nchunk), scales [0, nchunk / lpg)
    const Region codes{"", addr(a.codes) + 4ull * r * a.codes_stride_words,
                       addr(a.codes) + 4ull * r * a.codes_stride_words + 4ull * a.nchunk};
    const Region scales{"", addr(a.scales) + 4ull * r * a.scales_stride,
                        addr(a.scales) + 4ull * r * a.scales_stride + 4ull * (a.nchunk / lpg)};
    const Region* rc = find(rs, "codes1[" + std::to_string(r) + "]");
    const Region* rsc = find(rs, "scales1[" + std::to_string(r) + "]");
    CHECK(rc && codes.lo == rc->lo && inside(codes, *rc), "stage-1 codes of rank %d", r);
    CHECK(rsc && scales.lo == rsc->lo && inside(scales, *rsc), "stage-1 scales of rank %d", r);
    if (c.sfb) {
      const u64 per = c.sb16 ? 16 : 32;  // bytes of error per chunk
      const Region err{"", addr(a.err) + 4ull * r * a.err_stride, addr(a.err) + 4ull * r * a.err_stride + per * a.nchunk};
      const Region* re = find(rs, std::string("sender_err ") + (dir ? "bwd" : "fwd") + "[" + std::to_string(r) + "]");
      CHECK(re && err.lo == re->lo && inside(err, *re) && inside(err, ws), "stage-1 sender errors of rank %d", r);
    }
  }
  CHECK(c.sfb ? a.err != nullptr : a.err == nullptr, "stage-1 error pointer");
  CHECK(c.sfb == 0 || a.err_bf16 == c.sb16, "stage-1 error dtype");
  const int64_t n_g = c.N / c.group, per = (n_g + c.P - 1) / c.P;
  CHECK(a.own_chunks == (c.own ? per * (c.group / 8) : 0), "stage-1 own chunks %lld", (long long)a.own_chunks);
  (void)N;
}

void check_owner(const HostLaunch& l, const Case& c, const std::vector<Region>& rs, const void* const* parts, int dir) {
  const echo::OwnerArgs& a = l.owner;
  const u64 N = static_cast<u64>(c.N);
  CHECK(l.P == c.P && l.group == c.group && l.flag == (c.compensate != 0) && l.state_bf16 == (c.sb16 != 0) &&
            l.own_exact == (c.own != 0),
        "owner launch shape");
  CHECK(a.nchunk == c.N / 8, "owner chunks");
  for (int r = 0; r < echo::kMaxRanks; ++r) {
    const int rr = r < c.P ? r : 0;
    const Region* rc = find(rs, "codes1[" + std::to_string(rr) + "]");
    const Region* rsc = find(rs, "scales1[" + std::to_string(rr) + "]");
    CHECK(rc && addr(a.codes1[r]) == rc->lo, "owner codes of rank %d", r);
    CHECK(rsc && addr(a.scales1[r]) == rsc->lo, "owner scales of rank %d", r);
    if (c.own) CHECK(a.own_src[r] == parts[rr], "owner's own partial %d", r);
  }
  const Region* c2 = find(rs, "codes2");
  const Region* s2 = find(rs, "scales2");
  CHECK(c2 && addr(a.codes2) == c2->lo && s2 && addr(a.scales2) == s2->lo, "owner broadcast payload");
  const std::string dn = dir ? "bwd" : "fwd";
  const Region* mf = find(rs, "m_fast " + dn);
  const Region* ms = find(rs, "m_slow " + dn);
  CHECK(mf && addr(a.m_fast) == mf->lo && ms && addr(a.m_slow) == ms->lo, "owner estimates of %s", dn.c_str());
  CHECK(mf && (c.sb16 ? 16ull : 32ull) * a.nchunk == mf->hi - mf->lo, "estimate extent");
  CHECK(a.beta_fast == 0.5f && a.beta_slow == 0.95f, "betas");
  CHECK(a.omega_fast == 1.0f - 0.5f && a.omega_slow == 1.0f - 0.95f, "omegas");
  CHECK(a.out_bf16 == c.obf, "owner output dtype");
  const int64_t n_g = c.N / c.group, per = (n_g + c.P - 1) / c.P;
  CHECK(a.own_chunks == (c.own ? per * (c.group / 8) : 0), "owner own chunks");
  CHECK(!c.own || a.own_bf16 == (c.dtype == ECHO_BF16), "owner own dtype");
  (void)N;
}

void check_decode(const HostLaunch& l, const Case& c, const std::vector<Region>& rs, void* out) {
  const Region* c2 = find(rs, "codes2");
  const Region* s2 = find(rs, "scales2");
  CHECK(c2 && addr(l.codes) == c2->lo && s2 && addr(l.scales) == s2->lo, "decode payload");
  CHECK(l.out == out && l.n == c.N && l.group == c.group && l.flag == (c.obf != 0), "decode launch");
}

// A fill of n floats at p covers each of `want` and stays inside the workspace.
void check_zero_covers(const HostLaunch& l, const std::vector<const Region*>& want, const Region& ws) {
  const Region z{"", addr(l.out), addr(l.out) + 4ull * static_cast<u64>(l.n)};
  CHECK(inside(z, ws), "fill outside the workspace");
  for (const Region* w : want) CHECK(w && inside(*w, z), "fill misses %s", w ? w->what.c_str() : "?");
}

// echo_reduce_noalloc: the same three launches as echo_reduce, with the
// payloads carved from the static scratch exactly as a state carves them from
// its workspace, and the caller's carried vectors in place of the state's.
void check_noalloc(const Case& c, const std::vector<Region>& rs, const void* const* parts, void* out) {
  const echo_config cfg = make_cfg(c);
  const u64 N = static_cast<u64>(c.N), G = static_cast<u64>(c.group), P = static_cast<u64>(c.P);
  auto al = [](u64 x) { return (x + 255) / 256 * 256; };
  const u64 payload = P * (al(N / 2) + al(4 * (N / G))) + al(N / 2) + al(4 * (N / G));
  const u64 sv = c.sb16 ? 2 : 4;
  const u64 mf = 1ull << 51, ms = mf + al(sv * N) + 4096, se = ms + al(sv * N) + 4096;
  void* m_fast = fake(mf);
  void* m_slow = fake(ms);
  void* serr = c.sfb ? fake(se) : nullptr;
  g_launches.clear();
  const echo_status got = echo_reduce_noalloc(&cfg, parts, out, m_fast, m_slow, serr, nullptr);
  if (payload > ECHO_STATIC_SCRATCH_BYTES) {
    CHECK(got == ECHO_ERR_WORKSPACE && g_launches.empty(), "no-alloc call beyond the scratch (%llu B)", payload);
    return;
  }
  CHECK(got == ECHO_OK, "no-alloc call");
  // the expected regions: the state's payload layout moved to the scratch, the caller's vectors
  const Region* base = find(rs, "codes1[0]");
  std::vector<Region> nr;
  for (const Region& r : rs)
    if (r.what.rfind("codes", 0) == 0 || r.what.rfind("scales", 0) == 0)
      nr.push_back({r.what, r.lo - base->lo + kFakeScratch, r.hi - base->lo + kFakeScratch});
  const Region scratch{"scratch", kFakeScratch, kFakeScratch + payload};
  for (const Region& r : nr) CHECK(inside(r, scratch), "%s outside the scratch's payload bytes", r.what.c_str());
  for (const char* dn : {"fwd", "bwd"}) {
    const u64 f = c.compensate ? mf : 0, sl = c.compensate ? ms : 0;  // not passed without compensation
    nr.push_back({std::string("m_fast ") + dn, f, f + sv * N});
    nr.push_back({std::string("m_slow ") + dn, sl, sl + sv * N});
    for (u64 r = 0; c.sfb && r < P; ++r)
      nr.push_back({std::string("sender_err ") + dn + "[" + std::to_string(r) + "]", se + r * sv * N,
                    se + (r + 1) * sv * N});
  }
  const Region anywhere{"", 0, ~0ull};
  CHECK(g_launches.size() == 3, "no-alloc call launches three kernels (%zu)", g_launches.size());
  if (g_launches.size() == 3) {
    CHECK(g_launches[0].kind == HostLaunch::kStage1 && g_launches[1].kind == HostLaunch::kOwner &&
              g_launches[2].kind == HostLaunch::kDecode,
          "no-alloc launch order");
    check_stage1(g_launches[0], c, nr, parts, 0, anywhere);
    check_owner(g_launches[1], c, nr, parts, 0);
    check_decode(g_launches[2], c, nr, out);
  }
  // a failing launch stops the call there
  for (int k = 0; k < 3; ++k) {
    g_launches.clear();
    g_attempts = 0;
    g_fail_at = k;
    CHECK(echo_reduce_noalloc(&cfg, parts, out, m_fast, m_slow, serr, nullptr) == ECHO_ERR_HIP &&
              static_cast<int>(g_launches.size()) == k,
          "no-alloc call with launch %d failing", k);
  }
  g_fail_at = -1;
  // bad arguments launch nothing
  g_launches.clear();
  const void* part_in_scratch[echo::kMaxRanks];
  std::memcpy(part_in_scratch, parts, sizeof(part_in_scratch));
  part_in_scratch[0] = fake(kFakeScratch + 256);
  CHECK(echo_reduce_noalloc(&cfg, part_in_scratch, out, m_fast, m_slow, serr, nullptr) == ECHO_ERR_ARG,
        "partial in the scratch");
  CHECK(echo_reduce_noalloc(&cfg, parts, fake(kFakeScratch), m_fast, m_slow, serr, nullptr) == ECHO_ERR_ARG,
        "output in the scratch");
  CHECK(echo_reduce_noalloc(&cfg, parts, out, m_fast, m_slow, c.sfb ? nullptr : fake(se), nullptr) == ECHO_ERR_ARG,
        "sender errors given exactly when sender feedback is off");
  if (c.compensate) {
    CHECK(echo_reduce_noalloc(&cfg, parts, out, nullptr, m_slow, serr, nullptr) == ECHO_ERR_ARG, "null m_fast");
    CHECK(echo_reduce_noalloc(&cfg, parts, out, fake(mf + 8), m_slow, serr, nullptr) == ECHO_ERR_ARG,
          "misaligned m_fast");
    CHECK(echo_reduce_noalloc(&cfg, parts, out, m_fast, fake(mf + 16), serr, nullptr) == ECHO_ERR_ARG,
          "m_slow over m_fast");
    CHECK(echo_reduce_noalloc(&cfg, parts, out, m_fast, const_cast<void*>(parts[c.P - 1]), serr, nullptr) ==
              ECHO_ERR_ARG,
          "m_slow over a partial");
    CHECK(echo_reduce_noalloc(&cfg, parts, out, out, m_slow, serr, nullptr) == ECHO_ERR_ARG, "m_fast over the output");
    CHECK(echo_reduce_noalloc(&cfg, parts, out, fake(kFakeScratch + 512), m_slow, serr, nullptr) == ECHO_ERR_ARG,
          "m_fast in the scratch");
  }
  if (c.sfb) {
    CHECK(echo_reduce_noalloc(&cfg, parts, out, m_fast, m_slow, fake(se + 2), nullptr) == ECHO_ERR_ARG,
          "misaligned sender errors");
    if (c.compensate)
      CHECK(echo_reduce_noalloc(&cfg, parts, out, m_fast, m_slow, fake(ms + 16), nullptr) == ECHO_ERR_ARG,
            "sender errors over m_slow");
  }
  CHECK(echo_reduce_noalloc(nullptr, parts, out, m_fast, m_slow, serr, nullptr) == ECHO_ERR_ARG, "null config");
  CHECK(g_launches.empty(), "bad no-alloc arguments launched %zu kernels", g_launches.size());
}

void run_case(const Case& c, u64 ws_offset) {
  char buf[200];
  std::snprintf(buf, sizeof(buf), "P=%d N=%lld G=%d %s comp=%d sfb=%d sb16=%d obf=%d own=%d off=%llu", c.P,
                (long long)c.N, c.group, c.dtype == ECHO_BF16 ? "bf16" : "f32", c.compensate, c.sfb, c.sb16, c.obf,
                c.own, ws_offset);
  g_ctx = buf;
  const echo_config cfg = make_cfg(c);
  const size_t need = echo_workspace_bytes(&cfg);
  const u64 N = static_cast<u64>(c.N);
  if (c.N == 0) {
    CHECK(need == 0, "empty message needs no workspace");
    echo_state* st = nullptr;
    g_launches.clear();
    CHECK(echo_init_state(&cfg, nullptr, 0, nullptr, &st) == ECHO_OK && st != nullptr, "empty init");
    CHECK(g_launches.empty(), "empty init launches nothing");
    echo_destroy_state(st);
    return;
  }
  const u64 ws_base = (1ull << 44) + ws_offset;
  const Region ws{"workspace", ws_base, ws_base + need};

  // too small a workspace is rejected before anything is launched
  echo_state* st = nullptr;
  g_launches.clear();
  CHECK(echo_init_state(&cfg, fake(ws_base), need - 1, nullptr, &st) == ECHO_ERR_WORKSPACE && st == nullptr,
        "short workspace");
  CHECK(g_launches.empty(), "short workspace launches nothing");

  CHECK(echo_init_state(&cfg, fake(ws_base), need, nullptr, &st) == ECHO_OK && st != nullptr, "init");
  if (st == nullptr) return;
  const std::vector<Region> rs = regions(st, c);
  for (size_t i = 0; i < rs.size(); ++i) {
    CHECK(inside(rs[i], ws), "%s [%llx, %llx) outside the workspace [%llx, %llx)", rs[i].what.c_str(), rs[i].lo,
          rs[i].hi, ws.lo, ws.hi);
    CHECK(rs[i].lo % 256 == 0, "%s not 256-byte aligned", rs[i].what.c_str());
    for (size_t j = 0; j < i; ++j)
      CHECK(rs[i].hi <= rs[j].lo || rs[j].hi <= rs[i].lo, "%s overlaps %s", rs[i].what.c_str(), rs[j].what.c_str());
  }
  // init zeroes every piece of carried state of both directions in one fill
  CHECK(g_launches.size() == 1 && g_launches[0].kind == HostLaunch::kZero, "init fills the state once");
  if (g_launches.size() == 1) {
    std::vector<const Region*> st_regions;
    for (const Region& r : rs)
      if (r.what.rfind("m_", 0) == 0 || r.what.rfind("sender_err", 0) == 0) st_regions.push_back(&r);
    check_zero_covers(g_launches[0], st_regions, ws);
  }

  // partials and output: fake device tensors far above the workspace
  const u64 eb = c.dtype == ECHO_BF16 ? 2 : 4;
  const u64 part_base = 1ull << 52, part_stride = ((eb * N + 4095) / 4096) * 4096 + 4096;
  const void* parts[echo::kMaxRanks];
  for (int r = 0; r < echo::kMaxRanks; ++r) parts[r] = fake(part_base + r * part_stride);
  void* out = fake((1ull << 53) + 256);

  for (int dir = 0; dir < 2; ++dir) {
    g_launches.clear();
    CHECK(echo_reduce(parts, out, st, static_cast<echo_dir>(dir), nullptr) == ECHO_OK, "reduce");
    CHECK(g_launches.size() == 3, "reduce launches three kernels (%zu)", g_launches.size());
    if (g_launches.size() == 3) {
      CHECK(g_launches[0].kind == HostLaunch::kStage1 && g_launches[1].kind == HostLaunch::kOwner &&
                g_launches[2].kind == HostLaunch::kDecode,
            "reduce launch order");
      check_stage1(g_launches[0], c, rs, parts, dir, ws);
      check_owner(g_launches[1], c, rs, parts, dir);
      check_decode(g_launches[2], c, rs, out);
    }
    // the stage entry points launch the same kernels with the same arguments
    g_launches.clear();
    CHECK(echo_stage1(parts, st, static_cast<echo_dir>(dir), nullptr) == ECHO_OK &&
              echo_owner(c.own ? parts : nullptr, st, static_cast<echo_dir>(dir), nullptr) == ECHO_OK &&
              echo_decode(out, st, nullptr) == ECHO_OK,
          "stage entry points");
    if (g_launches.size() == 3) {
      check_stage1(g_launches[0], c, rs, parts, dir, ws);
      check_owner(g_launches[1], c, rs, parts, dir);
      check_decode(g_launches[2], c, rs, out);
    } else {
      CHECK(false, "stage entry points launch one kernel each");
    }
  }

  // a launch that fails stops the call there: ECHO_ERR_HIP, the launches before
  // it were made (and stay enqueued), none after it
  for (int k = 0; k < 3; ++k) {
    g_launches.clear();
    g_attempts = 0;
    g_fail_at = k;
    CHECK(echo_reduce(parts, out, st, ECHO_BWD, nullptr) == ECHO_ERR_HIP, "reduce with launch %d failing", k);
    CHECK(static_cast<int>(g_launches.size()) == k && g_attempts == k + 1,
          "launch %d failing: %zu launches made, %d attempted", k, g_launches.size(), g_attempts);
    g_launches.clear();
    g_attempts = 0;
    CHECK(echo_reset(st, 3, nullptr) == (k < (c.sfb ? 4 : 2) ? ECHO_ERR_HIP : ECHO_OK), "reset with fill %d failing", k);
    CHECK(static_cast<int>(g_launches.size()) == std::min(k, c.sfb ? 4 : 2), "reset with fill %d failing: %zu fills", k,
          g_launches.size());
  }
  g_fail_at = -1;

  // reset of one direction fills exactly that direction's carried state
  for (int mask = 1; mask <= 3; ++mask) {
    g_launches.clear();
    CHECK(echo_reset(st, mask, nullptr) == ECHO_OK, "reset %d", mask);
    std::vector<const Region*> want;
    for (int d = 0; d < 2; ++d) {
      if (!(mask & (1 << d))) continue;
      const std::string dn = d ? "bwd" : "fwd";
      for (const Region& r : rs)
        if (r.what == "m_fast " + dn || r.what == "m_slow " + dn || r.what.rfind("sender_err " + dn, 0) == 0)
          want.push_back(&r);
    }
    std::vector<bool> covered(want.size(), false);
    for (const HostLaunch& l : g_launches) {
      CHECK(l.kind == HostLaunch::kZero, "reset launches fills only");
      const Region z{"", addr(l.out), addr(l.out) + 4ull * static_cast<u64>(l.n)};
      CHECK(inside(z, ws), "reset fill outside the workspace");
      // no fill touches the other direction's state or the payloads
      for (const Region& r : rs) {
        bool wanted = false;
        for (const Region* w : want) wanted = wanted || w == &r;
        if (!wanted) CHECK(z.hi <= r.lo || r.hi <= z.lo, "reset %d fills %s", mask, r.what.c_str());
      }
      for (size_t i = 0; i < want.size(); ++i) covered[i] = covered[i] || inside(*want[i], z);
    }
    for (size_t i = 0; i < want.size(); ++i) CHECK(covered[i], "reset %d misses %s", mask, want[i]->what.c_str());
  }

  // bad arguments launch nothing
  g_launches.clear();
  const void* bad[echo::kMaxRanks];
  std::memcpy(bad, parts, sizeof(bad));
  bad[c.P - 1] = fake(ws_base + need / 2);  // inside the workspace
  CHECK(echo_reduce(bad, out, st, ECHO_FWD, nullptr) == ECHO_ERR_ARG, "partial in the workspace");
  bad[c.P - 1] = fake(addr(parts[c.P - 1]) + 2);  // misaligned
  CHECK(echo_reduce(bad, out, st, ECHO_FWD, nullptr) == ECHO_ERR_ARG, "misaligned partial");
  CHECK(echo_reduce(parts, fake(ws_base + 256), st, ECHO_FWD, nullptr) == ECHO_ERR_ARG, "output in the workspace");
  CHECK(echo_reduce(parts, const_cast<void*>(parts[0]), st, ECHO_FWD, nullptr) == ECHO_ERR_ARG,
        "output over a partial");
  CHECK(echo_reduce(nullptr, out, st, ECHO_FWD, nullptr) == ECHO_ERR_ARG, "null partials");
  CHECK(echo_reduce(parts, out, st, static_cast<echo_dir>(2), nullptr) == ECHO_ERR_ARG, "bad direction");
  CHECK(echo_reset(st, 0, nullptr) == ECHO_ERR_ARG && echo_reset(st, 4, nullptr) == ECHO_ERR_ARG, "bad mask");
  g_device = 1;
  CHECK(echo_reduce(parts, out, st, ECHO_FWD, nullptr) == ECHO_ERR_STATE, "another device current");
  g_device = 0;
  if (c.own) CHECK(echo_owner(nullptr, st, ECHO_FWD, nullptr) == ECHO_ERR_ARG, "own_exact needs the partials");
  CHECK(g_launches.empty(), "bad arguments launched %zu kernels", g_launches.size());

  // wire bytes against a direct count of the owner segments
  uint64_t rs_b = 0, ag_b = 0, bf_b = 0;
  CHECK(echo_wire_bytes(st, &rs_b, &ag_b, &bf_b) == ECHO_OK, "wire bytes");
  {
    const u64 n_g = N / c.group, per = (n_g + c.P - 1) / c.P, gb = c.group / 2 + 4;
    u64 largest_send = 0, largest_seg = 0;
    for (int j = 0; j < c.P; ++j) {  // rank j sends every segment but its own
      u64 send = 0;
      for (int k = 0; k < c.P; ++k) {
        const u64 lo = std::min<u64>(k * per, n_g), hi = std::min<u64>((k + 1) * per, n_g);
        if (k != j) send += (hi - lo) * gb;
        if (k == j) largest_seg = std::max(largest_seg, (hi - lo) * gb);
      }
      largest_send = std::max(largest_send, send);
    }
    CHECK(rs_b == largest_send && ag_b == (c.P - 1) * largest_seg && bf_b == (2 * (c.P - 1) * 2 * N) / c.P,
          "wire bytes %llu %llu %llu", (u64)rs_b, (u64)ag_b, (u64)bf_b);
  }

  check_noalloc(c, rs, parts, out);

  // the fused product writes the same stage-1 regions
  if (c.dtype == ECHO_BF16 && c.group == 32 && !c.own && N % (128 * 128) == 0) {
    const int64_t M = 128, K = 256, H = c.N / M;
    g_launches.clear();
    CHECK(echo_gemm_stage1(parts, parts, M, K, st, ECHO_BWD, nullptr) == ECHO_OK, "fused product");
    if (g_launches.size() == 1 && g_launches[0].kind == HostLaunch::kGemm) {
      const echo::GemmArgs& a = g_launches[0].gemm;
      CHECK(a.M == M && a.K == K && a.H == H && g_launches[0].flag && g_launches[0].P == c.P, "gemm shape");
      for (int r = 0; r < c.P; ++r) {
        const Region* rc = find(rs, "codes1[" + std::to_string(r) + "]");
        const Region* rsc = find(rs, "scales1[" + std::to_string(r) + "]");
        CHECK(rc && addr(a.codes) + 4ull * r * a.codes_stride_words == rc->lo, "gemm codes of rank %d", r);
        CHECK(rsc && addr(a.scales) + 4ull * r * a.scales_stride == rsc->lo, "gemm scales of rank %d", r);
        if (c.sfb) {  // the backward direction's errors, whole-message extent
          const Region* re = find(rs, "sender_err bwd[" + std::to_string(r) + "]");
          const u64 lo = addr(a.err) + 4ull * r * a.err_stride;
          CHECK(re && lo == re->lo && lo + (c.sb16 ? 2 : 4) * N <= re->hi, "gemm errors of rank %d", r);
        }
      }
      CHECK(c.sfb ? (a.err != nullptr && a.err_bf16 == c.sb16) : a.err == nullptr, "gemm error pointer");
    } else {
      CHECK(false, "fused product launches one kernel");
    }
    g_launches.clear();
    CHECK(echo_gemm_stage1(parts, parts, M, K, st, static_cast<echo_dir>(2), nullptr) == ECHO_ERR_ARG &&
              g_launches.empty(),
          "fused product with a bad direction");
  }
  echo_destroy_state(st);
}

}  // namespace

int main() {
  std::vector<Case> cases;
  const int64_t sizes[] = {32, 96, 128 * 5 + 32 * 3, 4096 + 96, 1 << 14, 128 * 128 * 3, (int64_t(1) << 20) + 128,
                           int64_t(1) << 29, ECHO_MAX_NUMEL};
  const int ranks[] = {1, 2, 3, 5, 8, 16};
  for (int64_t N : sizes)
    for (int P : ranks)
      for (int G : {32, 64, 128}) {
        if (N % G) continue;
        for (int v = 0; v < 7; ++v) {
          // (comp, sfb, sb16, obf, own) combinations
          static const int V[7][5] = {{1, 0, 0, 0, 0}, {0, 0, 0, 0, 0}, {1, 1, 0, 0, 0}, {1, 0, 1, 0, 0},
                                      {1, 1, 1, 1, 0}, {1, 0, 0, 1, 1}, {1, 1, 1, 0, 1}};
          for (echo_dtype dt : {ECHO_BF16, ECHO_F32})
            cases.push_back({P, N, G, dt, V[v][0], V[v][1], V[v][2], V[v][3], V[v][4]});
        }
      }
  cases.push_back({4, 0, 32, ECHO_BF16, 1, 0, 0, 0, 0});
  cases.push_back({16, 0, 128, ECHO_F32, 1, 1, 1, 1, 1});
  u64 k = 0;
  for (const Case& c : cases) run_case(c, (k++ * 37) % 256);  // any workspace alignment
  if (g_failures) {
    std::fprintf(stderr, "%d of %d checks failed\n", g_failures, g_checks);
    return 1;
  }
  std::printf("ok: %zu configurations, %d checks\n", cases.size(), g_checks);
  return 0;
}
