/*
 * echo.h -- C ABI of libecho: the Echo error-compensated int4 all-reduce on
 * one AMD MI355X (gfx950), with the P tensor-parallel ranks emulated as P
 * partial buffers in the GPU's HBM and the int4 payload buffers standing in
 * for the wire.
 *
 * The method is described in prose, with no code or formulas, on two pages,
 * cited below as
 *   Page R: the rit.work blog post "echo-4-bit-gpu-communication";
 *   Page H: the heraldofai.com article «Come Echo permette ai modelli AI di
 *           grandi dimensioni di allenarsi più velocemente usando dati
 *           ultra-leggeri a 4 bit».
 * In short (Page R, «Почему обычное 4-битное суммирование портит модель» and
 * «Как Echo возвращает ошибку в следующие вызовы»; Page H, «Come Echo evita
 * che gli errori si accumulino»):
 *   - every rank cuts its partial sum into owner segments and sends them as
 *     4-bit integers (here: groups of 32 elements, one fp32 scale per group;
 *     groups of 64 or 128 are a configurable variant);
 *   - the owner of a segment decodes the P contributions, adds them in fp32,
 *     adds a correction built from two smoothed estimates (fast, slow) of the
 *     rounding error of its earlier calls, re-quantizes the sum to int4 and
 *     broadcasts it, so an element is rounded at most twice whatever P is;
 *   - from the fp32 sum the owner knows the error its own rounding just made
 *     and folds it into the estimates; forward and backward keep separate
 *     estimates.
 *
 * Arithmetic of one call, per element i of group g (fl = binary32 rounding):
 *   stage 1 (every rank r):  a = max|x_r| over the group, s = fl(a/7),
 *                            q = nearest code in [-7,7] to the exact x/s,
 *                            ties to even (s == 0: all codes 0);
 *   owner sum:               S = (((d_0 + d_1) + d_2) + ...), d_r = fl(q_r*s_r);
 *   correction:              V = fl(S + fl(fl(0.5*m_fast) + fl(0.5*m_slow)));
 *   stage 2:                 (q2, s2) = Q(V),  B = fl(q2*s2);
 *   compensator:             e = fl(V - B),
 *                            m <- fl(fl(beta*m) + fl((1-beta)*e)) for both;
 *   output:                  out = B (fp32; no third rounding).
 * With compensate == 0 the correction is zero and the state is not touched.
 * Four variants change this chain: out_bf16 delivers bf16(B) and measures
 * e = fl(V - bf16(B)); own_exact lets the owner of a segment add its own
 * partial x_j in place of d_j (rank j quantizes every segment but its own);
 * sender_feedback has every rank quantize x + e_r and keep its own stage-1
 * error e_r <- fl(x + e_r - fl(q*s)) for its next call; state_bf16 keeps all
 * carried state (both estimates and the ranks' errors) in bfloat16.
 *
 * Conventions for every entry point
 *   - Device pointers point to the memory of the device that was current when
 *     the state was created; that device must be current at every call.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and is asynchronous; nothing synchronises the host.
 *   - Every argument is validated before anything is enqueued: on every
 *     error but ECHO_ERR_HIP nothing is launched and the state is unchanged.
 *     ECHO_ERR_HIP reports a failed HIP call.  An entry point that launches
 *     several kernels (echo_reduce: stage 1, owner, decode; echo_reset: one
 *     fill per region) stops at the first failed launch, and the launches
 *     before it stay enqueued and run: after a failed owner launch the
 *     stage-1 payload and, with sender_feedback, the ranks' stage-1 errors of
 *     the direction have advanced; after a failed decode the compensator has
 *     too and `out` is not written.  Reset the direction before using it
 *     again.  No exception crosses the ABI; the library allocates no device
 *     memory and keeps no global mutable state, apart from the static
 *     scratch of echo_reduce_noalloc.
 *   - A state may be used by one stream at a time (not re-entrant).
 *   - Inputs must be finite; for NaN or Inf the results are unspecified.
 */
#ifndef ECHO_H
#define ECHO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ECHO_OK = 0,
  ECHO_ERR_ARG = 1,       /* null / misaligned / overlapping pointer, bad enum   */
  ECHO_ERR_SHAPE = 2,     /* P outside [1,16], group not 32/64/128, numel % group != 0 or too large */
  ECHO_ERR_DTYPE = 3,     /* unknown dtype                                        */
  ECHO_ERR_WORKSPACE = 4, /* workspace missing or smaller than echo_workspace_bytes */
  ECHO_ERR_STATE = 5,     /* null state, or called with another device current   */
  ECHO_ERR_HIP = 6        /* a HIP runtime call or a kernel launch failed         */
} echo_status;

typedef enum { ECHO_F32 = 0, ECHO_BF16 = 1 } echo_dtype;
typedef enum { ECHO_FWD = 0, ECHO_BWD = 1 } echo_dir;

#define ECHO_MAX_RANKS 16
#define ECHO_GROUP 32
#define ECHO_MAX_NUMEL (((int64_t)1) << 36)

typedef struct {
  int32_t P;          /* emulated ranks, 1..ECHO_MAX_RANKS                        */
  int64_t numel;      /* N, elements per rank partial; 0 <= N <= ECHO_MAX_NUMEL,  */
                      /* N % group == 0 (N == 0 makes every call a no-op)         */
  int32_t group;      /* elements per scale: ECHO_GROUP (32), or 64 / 128 (variants) */
  echo_dtype dtype;   /* element type of every partial (fp32 or bfloat16)         */
  int32_t compensate; /* 1 = Echo with error compensation, 0 = plain 2-rounding   */
  float beta_fast;    /* smoothing of the fast estimate, in [0,1]; default 0.5    */
  float beta_slow;    /* smoothing of the slow estimate, in [0,1]; default 0.95   */
  int32_t sender_feedback; /* 1 = variant: every rank also feeds its own stage-1 */
                      /* rounding error into its next call (x' = x + e, e <- x' - */
                      /* fl(q*s), per rank and direction); 0 = off (default)       */
  int32_t state_bf16; /* 1 = variant: m_fast / m_slow (and, with sender_feedback, */
                      /* the ranks' stage-1 errors) stored in bfloat16, each fp32 */
                      /* update rounded to nearest, ties to even; 0 = fp32        */
  int32_t out_bf16;   /* 1 = variant: the output is bfloat16, bf16(B) rounded to  */
                      /* nearest even, and the owner's error is measured against */
                      /* it, e = fl(V - bf16(B)), so later calls compensate the  */
                      /* output rounding too; 0 = fp32 output B (default)         */
  int32_t own_exact;  /* 1 = variant: the owner of segment j adds its own partial */
                      /* x_j as it is (x_j + e_j with sender feedback) in rank    */
                      /* order instead of fl(q_j*s_j); rank j neither quantizes  */
                      /* nor sends segment j (its stage-1 codes, scales and error */
                      /* there are left untouched); 0 = off (default)             */
} echo_config;

typedef struct echo_state echo_state; /* opaque host handle */

typedef void* echo_stream_t; /* a hipStream_t */

/* Source: Page R «Как Echo возвращает ошибку в следующие вызовы» (ranks send
 * their segments as 4-bit integers; the owner keeps fast and slow error
 * estimates, separately for the forward and the backward pass).
 * Bytes of device workspace a state needs: stage-1 payloads of the P ranks
 * (codes N/2 B + scales 4N/group B each), the broadcast payload, the two
 * compensator vectors of both directions (2 x 2 x 4N B, or 2 x 2 x 2N B with
 * state_bf16) and, with
 * sender_feedback, every rank's stage-1 error for both directions
 * (2 x P x 4N B, or 2 x P x 2N B with state_bf16), plus alignment slack.  Returns 0 for an invalid configuration and for N == 0. */
size_t echo_workspace_bytes(const echo_config* cfg);

/* Source: Page R «Как Echo возвращает ошибку в следующие вызовы» (the
 * compensator's two smoothed estimates, one pair per pass direction, start
 * from nothing).
 * Create a state over a caller-owned device workspace of `ws_bytes` bytes
 * (at least echo_workspace_bytes(cfg); any alignment) and zero the
 * compensator of both directions on `stream`.  The workspace must outlive
 * the state; the library only carves it.  On success *out receives a host
 * handle to free with echo_destroy_state.  Errors: ECHO_ERR_ARG (null cfg or
 * out, bad compensate/beta), ECHO_ERR_SHAPE, ECHO_ERR_DTYPE,
 * ECHO_ERR_WORKSPACE, ECHO_ERR_HIP. */
echo_status echo_init_state(const echo_config* cfg, void* workspace, size_t ws_bytes,
                            echo_stream_t stream, echo_state** out);

/* Source: Page R «Почему обычное 4-битное суммирование портит модель» (the
 * all-reduce that adds the ranks' partial results of a tensor-parallel layer
 * and hands every rank the total) with the arithmetic of «Как Echo возвращает
 * ошибку в следующие вызовы»; Page H «Come Echo evita che gli errori si
 * accumulino» (4-bit transfer, high-precision sum, at most two roundings).
 * `dir` selects the forward or backward estimates, which Page R «Как Echo
 * возвращает ошибку в следующие вызовы» keeps apart for the two passes.
 * One whole all-reduce: echo_stage1, then echo_owner on direction `dir`,
 * then echo_decode.  partials: host array of P device pointers, each to N
 * contiguous elements of cfg.dtype, 16-byte aligned, read-only for the call.
 * out: device pointer to N fp32 (N bfloat16 with out_bf16), 16-byte aligned,
 * overlapping neither the partials nor the workspace; it receives the reduced
 * tensor every rank would hold.  The state of `dir` advances in place.
 * Deterministic: identical inputs and state give bit-identical results. */
echo_status echo_reduce(const void* const* partials, void* out, echo_state* st,
                        echo_dir dir, echo_stream_t stream);

/* Source: Page R «Как Echo возвращает ошибку в следующие вызовы» (every GPU
 * sends its segments as 4-bit integers).
 * Stage 1 on every rank: quantize each rank's partial to int4 codes and fp32
 * group scales in the state's stage-1 payload buffers (the "wire").  `dir`
 * selects the ranks' stage-1 errors when sender_feedback is on (otherwise it
 * is only validated). */
echo_status echo_stage1(const void* const* partials, echo_state* st, echo_dir dir,
                        echo_stream_t stream);

/* Source: Page R «Как Echo возвращает ошибку в следующие вызовы» (the authors
 * fuse compensation, quantization and exchange into their kernels) and
 * «Почему обычное 4-битное суммирование портит модель» (each GPU computes its
 * part of a layer's product, which the all-reduce then adds).
 * Stage 1 fused into the producing product (the step before the all-reduce in
 * a tensor-parallel layer: each rank's partial is the output of its slice of a
 * row-parallel product).  For every rank r the partial is
 * bf16(A_r * W_r^T), A_r [M, K] and W_r [H, K] bfloat16 row-major (W_r's rows
 * are output features), accumulated in fp32 on the matrix cores and rounded to
 * nearest-even; N = M*H.  Each rank's stage-1 payload is written into the
 * state exactly as echo_stage1 would write it from that bf16 partial, which
 * itself never reaches memory; with sender_feedback the ranks' stage-1 errors
 * of direction `dir` are added and updated as echo_stage1 does (otherwise
 * `dir` is only validated).  Follow with echo_owner and echo_decode on `dir`.
 * A, W: host arrays of P device pointers, 16-byte aligned, read-only.
 * Requires a bf16 state with group 32 and no own_exact (the owner would need
 * the partial itself), M a multiple of 64 (M/64 <= 65535), H a multiple of
 * 128 ((M/64)*(H/128) <= 2^27), K a multiple of 64 and at most 2^21.  Errors: ECHO_ERR_ARG (null or misaligned pointer, A or W
 * overlapping the workspace, own_exact on, bad dir), ECHO_ERR_SHAPE (sizes,
 * M*H != N, group != 32), ECHO_ERR_DTYPE (state not bf16), ECHO_ERR_STATE,
 * ECHO_ERR_HIP. */
echo_status echo_gemm_stage1(const void* const* A, const void* const* W, int64_t M, int64_t K,
                             echo_state* st, echo_dir dir, echo_stream_t stream);

/* Source: Page R «Почему обычное 4-битное суммирование портит модель» (each
 * GPU computes its own part of the layer's result).
 * The same product written out, for comparison: out[r] = bf16(A_r * W_r^T),
 * [M, H] bfloat16 row-major, for r < P (1..16).  Same shape rules; out[r] must
 * not overlap A or W.  Errors: ECHO_ERR_ARG, ECHO_ERR_SHAPE, ECHO_ERR_HIP. */
echo_status echo_gemm_bf16(const void* const* A, const void* const* W, void* const* out, int32_t P,
                           int64_t M, int64_t K, int64_t H, echo_stream_t stream);

/* Source: Page R «Как Echo возвращает ошибку в следующие вызовы» (the owner of
 * a segment restores the 4-bit values, adds them in high precision, measures
 * the error its rounding just made and folds it into the fast and slow
 * estimates); Page H «Come Echo evita che gli errori si accumulino».
 * Owner stage for all segments: decode the P stage-1 payloads, sum in fp32,
 * apply the correction of direction `dir`, re-quantize into the broadcast
 * payload and update the compensator of `dir`.  partials: with own_exact, the
 * same P device pointers the preceding echo_stage1 received (the owners read
 * their own shares from them; ECHO_ERR_ARG if NULL); otherwise ignored and
 * may be NULL. */
echo_status echo_owner(const void* const* partials, echo_state* st, echo_dir dir,
                       echo_stream_t stream);

/* Source: Page R «Как Echo возвращает ошибку в следующие вызовы» (the
 * compressed total is sent to the other GPUs, which restore it).
 * Every rank's decode of the broadcast payload into `out` (N fp32, or N
 * bfloat16 with out_bf16; 16-byte aligned, not in the workspace). */
echo_status echo_decode(void* out, const echo_state* st, echo_stream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * One whole all-reduce, the same kernels and results as echo_reduce on a
 * state whose carried vectors held what m_fast, m_slow and sender_err hold,
 * but with no state handle and no workspace.  The stage-1 payloads of the P
 * ranks and the broadcast payload go to a scratch buffer the library holds on
 * each device: a static device array of ECHO_STATIC_SCRATCH_BYTES, kept from
 * the first call on a device until the process ends.  The call allocates
 * nothing, on the device or on the host.
 *   cfg: as for echo_init_state.  The payloads take
 *     P * (A(N/2) + A(4N/group)) + A(N/2) + A(4N/group) bytes, A(x) = x
 *     rounded up to a multiple of 256; a larger message returns
 *     ECHO_ERR_WORKSPACE before anything is launched.  (64 MiB holds, e.g.,
 *     P = 4 with N = 2^24 elements, or P = 8 with N = 2^23.)
 *   partials, out: as for echo_reduce.
 *   m_fast, m_slow: the carried estimates of the direction the call belongs
 *     to, N fp32 each (N bfloat16 with state_bf16), read and advanced in
 *     place; ignored (may be NULL) when cfg->compensate is 0.  A direction
 *     starts from zeroed vectors: zero them (e.g. with a fill kernel) to reset.
 *   sender_err: with sender_feedback, the P ranks' carried stage-1 errors of
 *     that direction, rank r at element offset r*N (fp32, or bfloat16 with
 *     state_bf16), read and advanced in place; NULL otherwise.
 * Every device pointer 16-byte aligned and on the current device; no two of
 * out, m_fast, m_slow, sender_err and the partials overlap.  No part of the
 * scratch needs to start at zero (every call writes each payload before it
 * reads it); it keeps the last call's payloads.  All calls on one device
 * share it: calls that overlap in time on one device (two streams, two host
 * threads) race and must be serialised by the caller.  Errors as for
 * echo_reduce, plus ECHO_ERR_WORKSPACE for a message beyond the scratch. */
#define ECHO_STATIC_SCRATCH_BYTES (((size_t)64) << 20)
echo_status echo_reduce_noalloc(const echo_config* cfg, const void* const* partials, void* out,
                                void* m_fast, void* m_slow, void* sender_err, echo_stream_t stream);

/* Source: Page R «Как Echo возвращает ошибку в следующие вызовы» (separate
 * estimates for the forward and the backward pass; each pass over the layer
 * stack starts its own).
 * Zero the compensator (and, with sender_feedback, the ranks' stage-1 errors)
 * of the directions in dir_mask (1 = fwd, 2 = bwd, 3 = both), e.g. at the
 * start of every pass over the layer stack.
 * Uses a fill kernel (no memset node), so it may be captured in a graph. */
echo_status echo_reset(echo_state* st, int dir_mask, echo_stream_t stream);

/* Source: none on the pages (host bookkeeping of the state above).
 * Free the host handle (not the workspace).  NULL is accepted. */
void echo_destroy_state(echo_state* st);

/* Source: Page H «I fatti principali» (4-bit transfer at about a quarter of
 * the 16-bit cost); Page R «Почему обычное 4-битное суммирование портит
 * модель» (almost four times less data than 16-bit values).
 * Bytes one rank would send per call over a real interconnect: rs = the
 * largest stage-1 payload share a rank sends to the other owners, ag = the
 * largest broadcast an owner sends to the other ranks, bf16 = a ring
 * all-reduce of the same message in bfloat16 (2(P-1)/P * 2N). */
echo_status echo_wire_bytes(const echo_state* st, uint64_t* rs_per_rank, uint64_t* ag_per_rank,
                            uint64_t* bf16_allreduce_per_rank);

/* Source: Page R «Как Echo возвращает ошибку в следующие вызовы» (the
 * payloads on the wire and the two smoothed estimates the owner keeps).
 * Device pointers into the workspace, for inspection, checkpoint and restore
 * of the state (copy m_fast/m_slow out and back). */
typedef struct {
  const void* stage1_codes;    /* rank r: stage1_codes + r*stage1_codes_stride bytes, N/2 B  */
  const float* stage1_scales;  /* rank r: (char*)stage1_scales + r*stage1_scales_stride, N/group */
  size_t stage1_codes_stride;  /* bytes between ranks                                      */
  size_t stage1_scales_stride; /* bytes between ranks                                      */
  const void* bcast_codes;     /* N/2 B: two's-complement nibbles, element 2k low nibble   */
  const float* bcast_scales;   /* N/group fp32                                             */
  void* m_fast;                /* N fp32 (N bf16 with state_bf16), compensator of the dir  */
  void* m_slow;                /* N fp32 (N bf16 with state_bf16)                          */
  void* sender_err;            /* rank r: (char*)sender_err + r*sender_err_stride, N fp32 */
                               /* (N bf16 with state_bf16), the requested direction;     */
  size_t sender_err_stride;    /* NULL without sender_feedback                            */
} echo_views;

echo_status echo_debug_views(const echo_state* st, echo_dir dir, echo_views* out);

/* Source: none on the pages (error reporting of this library).
 * Static description of a status code. */
const char* echo_status_str(echo_status s);

#ifdef __cplusplus
}
#endif

#endif /* ECHO_H */
