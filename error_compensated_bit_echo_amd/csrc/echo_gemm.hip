// The producing product with stage 1 in its epilogue (gfx950, MFMA).
//
// In a tensor-parallel layer each rank's partial sum is the output of a
// row-parallel product, partial_r = A_r * W_r^T (A_r: [M, K] activations,
// W_r: [H, K] weights, bf16, fp32 accumulation), which the rank then rounds
// to bf16 and sends to the all-reduce.  Here the stage-1 quantization (rit.work
// blog post "echo-4-bit-gpu-communication", «Как Echo возвращает ошибку в
// следующие вызовы»: ranks send their segments as 4-bit integers) runs in the
// product's epilogue: the bf16 partial never leaves the registers, and the
// same quantizer as the stage-1 kernel turns it into the rank's payload.
// The payload is therefore bit-identical to stage 1 applied to the unfused
// bf16 partial, which the same kernel writes when asked to.
//
// Tiling: a block computes a 256 x 256 tile of one rank's [M, H] partial with 8
// wavefronts, each a 64 x 128 sub-tile of 2 x 4 v_mfma_f32_32x32x16_bf16 tiles,
// where the product is large enough; 128 x 128 with 8 wavefronts (32 x 64 each)
// for mid-sized and short products; 256 x 128 with 8 wavefronts (64 x 64 each)
// for products of one to two 128 x 128 tiles per CU; 64 x 128 with 4 wavefronts
// for the shortest and where M is an odd multiple of 64; 64 x 64 with 4
// wavefronts (one 32 x 32 MFMA tile each) where even 64 x 128 tiles would leave
// CUs idle.  The 256 x 256 tiles issue each K step's weight loads a quarter per
// 16-deep sub-step rather than in one burst.
// K advances 64 at a time through a ring of LDS slabs: while the matrix cores
// work on one slab, the next ones stream from global memory straight into the
// others (buffer_load_dwordx4 ... lds through a buffer resource over the block's
// row panel: each wavefront instruction fills 1 KiB of LDS, eight 128-byte rows,
// with no register staging), so each K step needs one barrier.  Within a K step
// the fragments of the four 16-deep sub-steps are double-buffered in registers.
// The slabs are unpadded; within a row the 16-byte chunk c of row r sits in slot
// c ^ ((r / 2) % 8), which spreads the 32 rows a fragment read touches over all
// LDS banks.  (Measured at P = 4, M = 2048, K = 3072, H = 4096: 11 % faster than
// staging through registers into padded rows; 128 x 64 tiles were slower.)
// Lane layout of the 32x32x16 bf16 product (checked on the device): lane l
// supplies A[l % 32][8 (l / 32) + i] and B[8 (l / 32) + i][l % 32], i < 8, and
// accumulator v of lane l is C[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
#pragma clang fp contract(off)

#include <type_traits>

#include "echo_device.h"

namespace echo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Two fp32 values rounded to bfloat16 (nearest, ties to even: the hardware
// conversion v_cvt_pk_bf16_f32), x in the low and y in the high half.
__device__ __forceinline__ uint32_t bf16x2_rne(float x, float y) {
  return __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(x), static_cast<__bf16>(y)});
}

// The value lane l ^ 32 holds (one v_permlane32_swap, which exchanges the two
// 32-lane halves, and a select).
__device__ __forceinline__ uint32_t xor32(uint32_t x, int half) {
  const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return half ? sw[0] : sw[1];
}

constexpr int kTileK = 64;
static_assert(kTileK == 64, "the slab loads assume 64-element (128-byte) rows");

// Fourth word of a raw buffer resource: 32-bit data format (any nonzero format
// does for these loads; a zero format would make every load return zero).
constexpr int kBufferWord3 = 0x00020000;

// The non-temporal (nt) bit of the cache-policy operand: the lines are kept in
// the caches as streaming data, evicted first.
constexpr int kNonTemporal = 2;

// A raw buffer resource over `bytes` bytes from `base`, and one 16-byte-per-lane
// load through it straight into LDS (lane l's 16 bytes land at lds + 16 l bytes;
// an offset at or past `bytes` reads zeros).  The slab loads use these rather
// than global_load_lds: the compiler counts a global (FLAT-encoded) load into
// LDS as pending LDS traffic too, so every wait for fragment reads in the K loop
// also waited for the next slab's loads (measured 4-5 % slower).  The builtins
// exist only for the device; the host pass, which also compiles the kernel
// bodies, gets stand-ins it never runs.
struct BufRsrc {
  __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ BufRsrc buffer_rsrc(const void* base, int32_t bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  return BufRsrc{__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferWord3)};
#else
  (void)base;
  (void)bytes;
  return BufRsrc{};
#endif
}
// POLICY: the cache-policy operand of the load (0, or kNonTemporal).
template <int POLICY>
__device__ __forceinline__ void buffer_load_lds16(BufRsrc r, uint16_t* lds, uint32_t voffset, uint32_t soffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.r, (__attribute__((address_space(3))) void*)lds, 16, voffset,
                                           soffset, 0, POLICY);
#else
  (void)r;
  (void)lds;
  (void)voffset;
  (void)soffset;
#endif
}

// s_waitcnt immediate that waits for every outstanding LDS access of this
// wavefront (lgkmcnt 0) and not for vector-memory operations or exports.
constexpr int kLdsDrained = 0xC07F;

// Element offset of (row, 16-byte chunk c) in a swizzled slab of 64-element rows.
__device__ __forceinline__ int slab_at(int row, int c) { return row * kTileK + 8 * (c ^ ((row >> 1) & 7)); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wavefront are outstanding (lgkm and export counts not waited on):
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 7, lgkmcnt 15.
constexpr int vmcnt_at_most(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// The same, and every outstanding LDS access too (lgkmcnt 0).
constexpr int vmcnt_at_most_lds_drained(int n) { return vmcnt_at_most(n) & ~(15 << 8); }

// Workgroup barrier for the slab pipeline.  __syncthreads() would also make
// every wavefront wait for all its outstanding global loads (its release fence
// covers the loads that write LDS), which would drain the loads of the later
// slabs at every step; here each wavefront first waits, with vmcnt_at_most,
// for the loads of the slab about to be read only.  The empty asm statements
// keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void slab_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// BM x TN: the block tile; NW: wavefronts, laid out (NW/2) x 2 over the
// tile, each computing (2 BM / NW) rows x TN/2 columns; S: LDS slabs in the
// pipeline (S - 1 K steps of loads in flight while one is multiplied).
//   256 x 256, 8 wavefronts, 2 slabs and a third W slab (160 KiB): one block
//     per CU, the fewest slab bytes per multiply-add;
//   128 x 128, 8 wavefronts, 2 slabs and a third W slab (80 KiB): two blocks per CU;
//   128 x 128, 8 wavefronts, 4 slabs (128 KiB): one block per CU with three K
//     steps of loads in flight, for products of at most one tile per CU, which
//     stream their weights and are bound by memory rather than matrix work;
//   64 x 128, 4 wavefronts, 4 slabs (96 KiB): the same for products of at most
//     half a tile per CU, in twice as many blocks, and for M an odd multiple of 64;
//   64 x 64, 4 wavefronts, 4 slabs (64 KiB): the same where 64 x 128 tiles would
//     number at most 128, half the CUs;
//   256 x 128, 8 wavefronts, 3 slabs (144 KiB): one block per CU for products of
//     one to two 128 x 128 tiles per CU, each weight panel read once per block.
// SFB (fused only): 0 no sender feedback; 1 the rank's stage-1 errors are fp32;
// 2 they are bfloat16 (each new error rounded to nearest even before it is kept).
// XG: the tile order.  The hardware hands the blocks of a launch to the eight
// XCDs in turn (block i to XCD i % 8), and each XCD has its own L2.  With XG,
// the tiles are ordered row tile fastest, then column panel, then rank, and
// block i takes tile (i % 8) T/8 + i / 8 of them when the T tiles are a
// multiple of 8 (else tile i), so that each XCD works through one contiguous
// run of them: the row tiles of a column panel share an XCD (its weights come
// from memory once), and so do as few ranks as the run spans (each rank's
// activations come from memory once per XCD that needs them; at P = 8 with 32
// panels of 128 columns, one rank per XCD instead of all eight on every XCD).
// Without XG, tile (x, y, r) is block x + gx (y + gy r), column panel fastest.
// WNT: the weight loads are non-temporal, for the short products (at most two
// 128 x 128 tiles per CU), where the few blocks that read a weight panel run at
// the same time on one XCD and nothing reads it later.
// WAHEAD (with S = 2): the weights are loaded a K step further ahead than the
// activations, through a ring of three W slabs beside the two A slabs.
template <int BM, int TN, int NW, int S, bool FUSED, int SFB, bool XG, bool WNT, bool WAHEAD>
__global__ __launch_bounds__(64 * NW) void echo_gemm_k(const GemmArgs a) {
  static_assert(FUSED || SFB == 0, "sender feedback only in the fused epilogue");
  constexpr int kThreads = 64 * NW;
  constexpr int RW = 2 * BM / NW;                  // rows per wavefront
  constexpr int MI = RW / 32;                      // 32-row MFMA tiles per wavefront
  constexpr int CW = TN / 2;                       // columns per wavefront
  constexpr int NJ = CW / 32;                      // 32-column MFMA tiles per wavefront
  static_assert(MI == 1 || MI == 2, "one or two 32-row MFMA tiles per wavefront");
  static_assert(TN == 64 || TN == 128 || TN == 256, "64-, 128- or 256-column block tiles");
  constexpr int JA = BM / (8 * NW), JW = TN / (8 * NW);  // 1 KiB slab blocks per wavefront
  static_assert(JA * 8 * NW == BM && JW * 8 * NW == TN, "slab blocks split evenly");
  constexpr int kLoads = JA + JW;                  // global loads per wavefront per slab
  constexpr int kSlabA = BM * kTileK;              // bf16 of one A slab
  constexpr int kSlab = (BM + TN) * kTileK;        // bf16 of one A + W slab
  constexpr int kLdsN = TN + 8;                    // bf16 per LDS row of the written-out tile (padded)
  static_assert(!WAHEAD || S == 2, "weights a step further ahead only with two activation slabs");
  constexpr int kSlabW = TN * kTileK;              // bf16 of one W slab
  constexpr int kRing = WAHEAD ? S * kSlabA + (S + 1) * kSlabW : S * kSlab;
  constexpr int kLdsTotal = (!FUSED && BM * kLdsN > kRing) ? BM * kLdsN : kRing;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsTotal];  // the written-out tile reuses the slabs
  unsigned bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if constexpr (XG) {
    const unsigned gx = gridDim.x, gy = gridDim.y, T = gx * gy * gridDim.z;
    unsigned i = bx + gx * (by + gy * bz);
    if (T % 8 == 0) i = (i % 8) * (T / 8) + i / 8;
    by = i % gy;
    bx = (i / gy) % gx;
    bz = i / (gx * gy);
  }
  const int r = static_cast<int>(bz);
  const uint16_t* A = a.A[0];
  const uint16_t* W = a.W[0];
#pragma unroll
  for (int i = 1; i < kMaxRanks; ++i)
    if (r == i) {
      A = a.A[i];
      W = a.W[i];
    }
  const int64_t K = a.K, H = a.H;
  const int64_t m0 = static_cast<int64_t>(by) * BM;
  const int64_t n0 = static_cast<int64_t>(bx) * TN;
  const int t = threadIdx.x, lane = t & 63, wm = (t >> 6) >> 1, wn = (t >> 6) & 1;

  // global -> LDS slab `buf`: wavefront w fills 1 KiB blocks JA w ... of the A
  // slab and JW w ... of the W slab; in block i lane l writes slot l, i.e. row
  // 8i + l/8, slot l % 8, which holds chunk (l % 8) ^ ((row / 2) % 8) of that row.
  // The loads go through buffer resources over the block's row panels of A and
  // W (BM or TN rows of K elements; under 2^31 bytes for the K the launcher
  // accepts): a lane's byte offset within the panel is fixed, the K step's is
  // a scalar offset.
  const int wave = t >> 6;
  const BufRsrc rA = buffer_rsrc(A + m0 * K, static_cast<int32_t>(BM * K * 2));
  const BufRsrc rW = buffer_rsrc(W + n0 * K, static_cast<int32_t>(TN * K * 2));
  uint32_t offA[JA], offW[JW];
  {
    const int sub = lane & 7;
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int row = 8 * (JA * wave + j) + (lane >> 3);
      offA[j] = static_cast<uint32_t>((row * K + 8 * (sub ^ ((row >> 1) & 7))) * 2);
    }
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const int row = 8 * (JW * wave + j) + (lane >> 3);
      offW[j] = static_cast<uint32_t>((row * K + 8 * (sub ^ ((row >> 1) & 7))) * 2);
    }
  }
  auto issue = [&](int buf, int64_t k0) {
    uint16_t* As = lds + buf * kSlab;
    uint16_t* Ws = As + kSlabA;
    const uint32_t kb = static_cast<uint32_t>(k0 * 2);
#pragma unroll
    for (int j = 0; j < JA; ++j) buffer_load_lds16<0>(rA, As + 512 * (JA * wave + j), offA[j], kb);
#pragma unroll
    for (int j = 0; j < JW; ++j)
      buffer_load_lds16<WNT ? kNonTemporal : 0>(rW, Ws + 512 * (JW * wave + j), offW[j], kb);
  };
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // The slab rings.  Without WAHEAD, S slabs each hold a K step's A and W
  // tiles: K step `it` multiplies slab it % S, and the loads of step
  // it + S - 1 are issued at its start into the slab step it - 1 used.  With
  // WAHEAD, two slabs of A tiles and, after them, three of W tiles: step it
  // multiplies A slot it % 2 and W slot it % 3 and issues the loads of A for
  // step it + 1 and of W for step it + 2, so the weights, which come from HBM
  // when cold while the activations are usually cached, have two steps to
  // arrive.  Either way a load goes into a slot that step it - 1 read and every
  // wavefront has finished reading: each waits for its own LDS reads before
  // the barrier that ends a step.  The fragments of a step's four 16-deep
  // sub-steps are double-buffered in registers: the reads of sub-step k + 1 go
  // out before the MFMAs of sub-step k, and the reads of the next slab's first
  // sub-step right after the barrier, before the last sub-step's MFMAs.  (The
  // compiler's own wait before a sub-step's MFMAs would be for every
  // outstanding LDS read, the new ones included; each sub-step therefore first
  // drains the reads issued a sub-step earlier, which have had the MFMAs
  // between to land, and its MFMAs need no wait.)
  const int64_t steps = K / kTileK;
  bf16x8 af[2][MI], bf[2][NJ];
  auto read_frags = [&](auto buf, const uint16_t* As, const uint16_t* Ws, int ks) {
    const int c = 2 * ks + (lane >> 5);  // lane supplies k = 8c .. 8c + 7
#pragma unroll
    for (int i = 0; i < MI; ++i)
      af[buf][i] = *reinterpret_cast<const bf16x8*>(As + slab_at(RW * wm + 32 * i + (lane & 31), c));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      bf[buf][j] = *reinterpret_cast<const bf16x8*>(Ws + slab_at(CW * wn + 32 * j + (lane & 31), c));
  };
  auto mfmas = [&](auto buf) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[buf][j], af[buf][i], acc[i][j], 0, 0, 0);  // C^T tile
  };
  // a sub-step: drain the reads of its own fragments, issue the next sub-step's
  // reads, then its MFMAs, in that order
  auto sub_step = [&](auto cur, auto next, const uint16_t* As, const uint16_t* Ws, int ks_next) {
    __builtin_amdgcn_s_waitcnt(kLdsDrained);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(next, As, Ws, ks_next);
    mfmas(cur);
    __builtin_amdgcn_sched_group_barrier(0x100, MI + NJ, 0);  // the LDS reads first
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NJ, 0);  // then the MFMAs
  };
  constexpr std::integral_constant<int, 0> B0{};
  constexpr std::integral_constant<int, 1> B1{};
  static_assert(kTileK / 16 == 4, "four sub-steps per K step");
  if constexpr (!WAHEAD) {
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < steps) issue(s, static_cast<int64_t>(s) * kTileK);
    if (steps >= S - 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_at_most((S - 2) * kLoads));  // step 0's slab has landed
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
    slab_barrier();
    // one K step; the last one issues no loads and needs no barrier before its
    // MFMAs (but one after its reads when the written-out epilogue reuses the slabs)
    auto step = [&](int64_t it, auto last) {
      const int cur = static_cast<int>(it % S);
      const bool more = it + S - 1 < steps;
      if constexpr (!decltype(last)::value) {
        if (more) issue(static_cast<int>((it + S - 1) % S), (it + S - 1) * kTileK);  // in flight below
      }
      const uint16_t* As = lds + cur * kSlab;
      const uint16_t* Ws = As + kSlabA;
      sub_step(B0, B1, As, Ws, 1);
      sub_step(B1, B0, As, Ws, 2);
      sub_step(B0, B1, As, Ws, 3);
      if constexpr (!decltype(last)::value) {
        // step it + 1's slab has landed (the S - 2 later steps' loads may still fly)
        // and this wavefront's reads of slab `cur` are done
        if (more)
          __builtin_amdgcn_s_waitcnt(vmcnt_at_most_lds_drained((S - 2) * kLoads));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_at_most_lds_drained(0));
        slab_barrier();
        const uint16_t* An = lds + static_cast<int>((it + 1) % S) * kSlab;
        read_frags(B0, An, An + kSlabA, 0);
      } else {
        __builtin_amdgcn_s_waitcnt(kLdsDrained);
        // the written-out epilogue reuses the slabs for its tile: every
        // wavefront's reads of them are done before any wavefront writes it
        if constexpr (!FUSED) slab_barrier();
      }
      mfmas(B1);
    };
    read_frags(B0, lds, lds + kSlabA, 0);
    for (int64_t it = 0; it + 1 < steps; ++it) step(it, std::false_type{});
    step(steps - 1, std::true_type{});
  } else {
    // Loads go out in the order A(0), W(0), W(1), then A(it + 1), W(it + 2) at
    // step it, and complete in that order: at the end of step it A(it + 1) and
    // W(it + 1) must have landed, and only W(it + 2), issued after A(it + 1), may
    // still be in flight.  The slots are tracked incrementally (a 64-bit
    // remainder by 3 each step cost several per cent).
    uint16_t* const abase = lds;
    uint16_t* const wbase = lds + S * kSlabA;
    auto issue_a_to = [&](uint16_t* As, int64_t st) {
      const uint32_t kb = static_cast<uint32_t>(st * kTileK * 2);
#pragma unroll
      for (int j = 0; j < JA; ++j) buffer_load_lds16<0>(rA, As + 512 * (JA * wave + j), offA[j], kb);
    };
    auto issue_w_to = [&](uint16_t* Ws, int64_t st) {
      const uint32_t kb = static_cast<uint32_t>(st * kTileK * 2);
#pragma unroll
      for (int j = 0; j < JW; ++j)
        buffer_load_lds16<WNT ? kNonTemporal : 0>(rW, Ws + 512 * (JW * wave + j), offW[j], kb);
    };
    int sa = 0, sw = 0;  // slots of the current step's A and W slabs
    auto next3 = [](int x) { return x == 2 ? 0 : x + 1; };
    issue_a_to(abase, 0);
    issue_w_to(wbase, 0);
    if (steps > 1) issue_w_to(wbase + kSlabW, 1);
    if (steps > 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_at_most(JW));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
    slab_barrier();
    // The 256-column tiles issue W(it + 2) a quarter at a time, one share at the
    // step's start after A(it + 1) and one after the MFMAs of each of the first
    // three sub-steps, rather than in one burst with A(it + 1); A(it + 1) still
    // goes out first, so the end-of-step wait is unchanged.  (Measured with the weights cold: at P = 4, M = 2048,
    // K = 3072, H = 4096 176.2 against 181.8 us, at P = 8 345.3 against 358.7;
    // no faster on the 128 x 128 tiles, nor with A spread over the first two
    // sub-steps as well.)
    constexpr bool kSpreadW = TN == 256;
    static_assert(!kSpreadW || JW % 4 == 0, "weight loads split evenly over the four sub-steps");
    auto step = [&](int64_t it, auto last) {
      const bool w_more = it + 2 < steps;
      const int sa1 = sa ^ 1, sw1 = next3(sw), sw2 = next3(sw1);
      constexpr bool kSpread = kSpreadW && !decltype(last)::value;
      auto issue_w_share = [&](int q) {  // share q of W(it + 2): loads q JW/4 .. (q + 1) JW/4 - 1
        const uint32_t kb = static_cast<uint32_t>((it + 2) * kTileK * 2);
        uint16_t* const Ws2 = wbase + sw2 * kSlabW;
#pragma unroll
        for (int j = q * (JW / 4); j < (q + 1) * (JW / 4); ++j)
          buffer_load_lds16<WNT ? kNonTemporal : 0>(rW, Ws2 + 512 * (JW * wave + j), offW[j], kb);
      };
      if constexpr (!decltype(last)::value) {
        issue_a_to(abase + sa1 * kSlabA, it + 1);
        if constexpr (kSpread) {
          if (w_more) issue_w_share(0);
        } else {
          if (w_more) issue_w_to(wbase + sw2 * kSlabW, it + 2);
        }
      }
      const uint16_t* As = abase + sa * kSlabA;
      const uint16_t* Ws = wbase + sw * kSlabW;
      sub_step(B0, B1, As, Ws, 1);
      if constexpr (kSpread) if (w_more) issue_w_share(1);
      sub_step(B1, B0, As, Ws, 2);
      if constexpr (kSpread) if (w_more) issue_w_share(2);
      sub_step(B0, B1, As, Ws, 3);
      if constexpr (kSpread) if (w_more) issue_w_share(3);
      if constexpr (!decltype(last)::value) {
        if (w_more)
          __builtin_amdgcn_s_waitcnt(vmcnt_at_most_lds_drained(JW));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_at_most_lds_drained(0));
        slab_barrier();
        read_frags(B0, abase + sa1 * kSlabA, wbase + sw1 * kSlabW, 0);
      } else {
        __builtin_amdgcn_s_waitcnt(kLdsDrained);
        if constexpr (!FUSED) slab_barrier();
      }
      mfmas(B1);
      sa = sa1;
      sw = sw1;
    };
    read_frags(B0, abase, wbase, 0);
    for (int64_t it = 0; it + 1 < steps; ++it) step(it, std::false_type{});
    step(steps - 1, std::true_type{});
  }

  // Epilogue straight from the accumulators (no LDS round trip).  The product
  // is computed transposed, C^T = W * A^T, so lane l of tile (i, j) holds
  // output row m = (BM/2) wm + 32 i + l % 32 and the 16 columns
  // h = (TN/2) wn + 32 j + 8 (v / 4) + 4 (l / 32) + v % 4: a group of 32 columns of
  // one row lives in lanes l and l ^ 32 (16 values each), and each run of 4
  // consecutive columns in one lane.
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t m = m0 + RW * wm + 32 * i + (lane & 31);
      const int64_t e = m * H + n0 + CW * wn + 32 * j;  // first element of the row's group
      // the bf16-rounded partial: pk[q] holds columns 2q and 2q + 1 of the lane's
      // 16 (in accumulator order), v the same values widened to fp32
      uint32_t pk[8];
      float v[16];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        pk[q] = bf16x2_rne(acc[i][j][2 * q], acc[i][j][2 * q + 1]);
        v[2 * q] = __uint_as_float(pk[q] << 16);
        v[2 * q + 1] = __uint_as_float(pk[q] & 0xFFFF0000u);
      }
      if constexpr (!FUSED) {
        // into the row-major LDS tile, 4 columns (8 bytes) per store; written out below
        const int row = RW * wm + 32 * i + (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // columns 8q + 4 half .. + 3
          const uint32_t lo = pk[2 * q], hi = pk[2 * q + 1];
          *reinterpret_cast<uint2*>(lds + row * kLdsN + CW * wn + 32 * j + 8 * q + 4 * half) = make_uint2(lo, hi);
        }
      } else {
        // sender feedback: x' = fl(x + e) with the rank's carried stage-1 error of
        // these 16 elements (runs of 4 at columns 8q + 4 half, q < 4)
        [[maybe_unused]] float* err = nullptr;
        if constexpr (SFB != 0) {
          err = a.err + static_cast<int64_t>(r) * a.err_stride;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t at = e + 8 * q + 4 * half;  // element index of the run
            float ev[4];
            if constexpr (SFB == 2) {
              const uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(err) + at);
              ev[0] = __uint_as_float(b.x << 16);
              ev[1] = __uint_as_float(b.x & 0xFFFF0000u);
              ev[2] = __uint_as_float(b.y << 16);
              ev[3] = __uint_as_float(b.y & 0xFFFF0000u);
            } else {
              const f32x4 f = *reinterpret_cast<const f32x4*>(err + at);
#pragma unroll
              for (int k = 0; k < 4; ++k) ev[k] = f[k];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) v[4 * q + k] = v[4 * q + k] + ev[k];
          }
        }
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) amax = fmaxf(amax, __builtin_fabsf(v[k]));
        amax = fmaxf(amax, __uint_as_float(xor32(__float_as_uint(amax), half)));
        const float s = echo_div7(amax);
        float v0[8], v1[8], kf[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v0[k] = v[k];
          v1[k] = v[8 + k];
        }
        // w0: columns 4 half + {0..3} (low half-word) and 8 + 4 half + {0..3} (high);
        // w1: the same plus 16
        float kf1[8];
        const uint32_t w0 = quantize8(v0, s, kf);
        const uint32_t w1 = quantize8(v1, s, kf1);
        if constexpr (SFB != 0) {
          // e <- x' - fl(q * s), exact; written back where it was read
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t at = e + 8 * q + 4 * half;
            float en[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int i = 4 * q + k;
              en[k] = i < 8 ? v0[i] - kf[i] * s : v1[i - 8] - kf1[i - 8] * s;
            }
            if constexpr (SFB == 2) {
              const uint32_t lo = __builtin_amdgcn_perm(bf16_rne_carry(en[1]), bf16_rne_carry(en[0]), 0x07060302u);
              const uint32_t hi = __builtin_amdgcn_perm(bf16_rne_carry(en[3]), bf16_rne_carry(en[2]), 0x07060302u);
              *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(err) + at) = make_uint2(lo, hi);
            } else {
              *reinterpret_cast<f32x4*>(err + at) = f32x4{en[0], en[1], en[2], en[3]};
            }
          }
        }
        // code word q of the group holds columns 8q .. 8q + 7, its low half-word from
        // the lower lane; the lower lane writes words 0 and 1, the upper 2 and 3
        const uint32_t got = xor32(half ? w0 : w1, half);
        uint2 words;
        if (half == 0)
          words = make_uint2((w0 & 0xFFFFu) | (got << 16), (w0 >> 16) | (got & 0xFFFF0000u));
        else
          words = make_uint2((got & 0xFFFFu) | (w1 << 16), (got >> 16) | (w1 & 0xFFFF0000u));
        uint32_t* codes = a.codes + static_cast<int64_t>(r) * a.codes_stride_words;
        *reinterpret_cast<uint2*>(codes + (e >> 3) + 2 * half) = words;
        if (half == 0) a.scales[static_cast<int64_t>(r) * a.scales_stride + (e >> 5)] = s;
      }
    }
  if constexpr (!FUSED) {
    // the bf16 tile from LDS to the rank's partial: TN / 8 lanes per row, 16 bytes each
    __syncthreads();
    uint16_t* out = a.out[0];
#pragma unroll
    for (int q = 1; q < kMaxRanks; ++q)
      if (r == q) out = a.out[q];
#pragma unroll
    for (int u = 0; u < BM * TN / 8 / kThreads; ++u) {
      const int chunk = t + kThreads * u;
      const int row = chunk / (TN / 8), cc = (chunk % (TN / 8)) * 8;
      *reinterpret_cast<u32x4*>(out + (m0 + row) * H + n0 + cc) =
          *reinterpret_cast<const u32x4*>(lds + row * kLdsN + cc);
    }
  }
}

}  // namespace

namespace {

template <int BM, int TN, int NW, int S, bool XG, bool WNT, bool WAHEAD>
hipError_t gemm_cfg(const GemmArgs& a, int P, bool fused, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.H / TN), static_cast<unsigned>(a.M / BM),
                  static_cast<unsigned>(P));
  if (!fused)
    hipLaunchKernelGGL((echo_gemm_k<BM, TN, NW, S, false, 0, XG, WNT, WAHEAD>), grid, dim3(64 * NW), 0, s, a);
  else if (a.err == nullptr)
    hipLaunchKernelGGL((echo_gemm_k<BM, TN, NW, S, true, 0, XG, WNT, WAHEAD>), grid, dim3(64 * NW), 0, s, a);
  else if (a.err_bf16)
    hipLaunchKernelGGL((echo_gemm_k<BM, TN, NW, S, true, 2, XG, WNT, WAHEAD>), grid, dim3(64 * NW), 0, s, a);
  else
    hipLaunchKernelGGL((echo_gemm_k<BM, TN, NW, S, true, 1, XG, WNT, WAHEAD>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Where the launch has at most 128 tiles of 64 x 128 (all ranks), 64 x 64 tiles,
// 4 slabs, grouped, weights non-temporal: one block per CU instead of one per two
// CUs.  Measured cold (as below), us: P = 2, M = 128, K = 3072, H = 4096: 19.3
// against 27.5 for 64 x 128 tiles; P = 4, M = 64, same K and H: 21.8 against
// 30.2; P = 1, M = 128, K = 4096, H = 8192: 24.1 against 32.4; P = 2, M = 128,
// K = 512, H = 4096: 7.5 against 8.6.  With 256 tiles of 64 x 128 they were no
// faster (P = 8, M = 64, K = 512, H = 4096: 11.5 against 11.5) or slower (P = 4,
// M = 128, K = 3072, H = 4096: 35.6 against 30.3), and 6 or 8 slabs no faster.
// Otherwise, for M a multiple of 128, by the number b of 128 x 128 tiles of the whole launch:
//   b <= 128: 64 x 128, 4 slabs, grouped, weights non-temporal;
//   b <= 256: 128 x 128, 8 wavefronts, 4 slabs, grouped, weights non-temporal;
//   b <= 512 with M a multiple of 256: 256 x 128, 8 wavefronts, 3 slabs, grouped,
//     weights non-temporal (cold, us: P = 8, M = 256, K = 3072, H = 4096 61.5
//     against 68.1 for 128 x 128 tiles with 2 slabs and weights ahead; P = 6,
//     same M, K and H, 53.9 against 64.1; P = 4, M = 512, 55.4 against 60.7;
//     P = 16, M = 256, H = 2048, 60.9 against 68.8; P = 1, M = 2048, 55.9 against
//     56.4; with the weights in the Infinity Cache 4-12 % slower, e.g. 61.5
//     against 54.6 at the first shape);
//   b >= 1024 with M and H multiples of 256: 256 x 256, grouped, weights ahead;
//   else 128 x 128, 8 wavefronts, 2 slabs, grouped, weights ahead.
// Measured with the weights cold (each call's weights last touched more than
// 256 MB of traffic earlier, as in a model whose layers each bring their own):
// fused product with stage 1, median of 5 x 40 calls, against the same shapes
// in other tile configurations, each comparison from one run, us:
//   P = 2, M = 256, K = 1024, H = 1024: 11.3 against 12.9 for 64 x 128 tiles with 2 slabs;
//   P = 4, M = 128, K = 3072, H = 4096: 29.9 against 46.5 (64 x 128, 2 slabs) and
//     37.1 (128 x 128, 4 slabs);
//   P = 8, M = 128, same K and H: 43.4 against 59.1 (64 x 128, 2 slabs) and 45.0
//     (the same tiles with cached weight loads; 35.2 against 41.6 when the
//     weights are still in the Infinity Cache);
//   P = 4, M = 2048, K = 3072, H = 4096: 178.9 against 190.2 without the third W
//     slab (175.2 against 171.2 with the weights in the Infinity Cache), 205.0 in
//     the column-panel-fastest order and 244.2 for 128 x 128 tiles with 2 slabs;
//     at K = 12288, 678 against 726;
//   P = 4, M = 2048, K = 3072, H = 2176: 127.8 against 149.8 without the third W
//     slab and 185.5 for 256 x 128 tiles;
//   P = 2, M = 2176, K = 3072, H = 4096: 127.0 against 144.8 without the third W
//     slab and 149.2 for 128 x 128 tiles of 4 wavefronts;
//   P = 8, M = 256, K = 3072, H = 4096: 67.5 against 72.2 without the third W
//     slab, 74.7 for 128 x 128 tiles with 4 slabs and 78.2 for 256 x 128.
hipError_t launch_gemm(const GemmArgs& a, int P, bool fused, hipStream_t s) {
  // at most 128 tiles of 64 x 128 over all ranks: 64 x 64 tiles
  if ((a.M / kGemmRowStep) * (a.H / kGemmTileN) * P <= 128)
    return gemm_cfg<64, 64, 4, 4, true, true, false>(a, P, fused, s);
  // M a multiple of 64 but not of 128: 64 x 128 tiles, 4 slabs, grouped; the
  // weight loads non-temporal for M = 64, where each weight panel has one reader
  if (a.M % kGemmTileM != 0)
    return a.M == kGemmRowStep ? gemm_cfg<64, 128, 4, 4, true, true, false>(a, P, fused, s)
                               : gemm_cfg<64, 128, 4, 4, true, false, false>(a, P, fused, s);
  const int64_t b = (a.M / kGemmTileM) * (a.H / kGemmTileN) * P;
  if (b <= 128) return gemm_cfg<64, 128, 4, 4, true, true, false>(a, P, fused, s);
  if (b <= 256) return gemm_cfg<128, 128, 8, 4, true, true, false>(a, P, fused, s);
  if (b <= 512 && a.M % 256 == 0) return gemm_cfg<256, 128, 8, 3, true, true, false>(a, P, fused, s);
  if (b >= 1024 && a.M % 256 == 0 && a.H % 256 == 0) return gemm_cfg<256, 256, 8, 2, true, false, true>(a, P, fused, s);
  return gemm_cfg<128, 128, 8, 2, true, false, true>(a, P, fused, s);
}

}  // namespace echo
