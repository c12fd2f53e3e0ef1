/*
 * Per-call latency of echo_reduce called eagerly through the C ABI from plain C
 * (no Python, no torch, no graph), for the small messages where a call is
 * bound by launches rather than by memory.  Used by `bench.py --config decode`.
 *
 * usage: echo_c_latency P N CALLS
 *   P ranks of N bfloat16 elements each (N a multiple of 32), fp32 output,
 *   compensation on, the default stream.  After 200 warm-up calls it prints one
 *   JSON line with, per call:
 *   device_us      HIP events around CALLS back-to-back calls (no host waits);
 *   enqueue_us     host time of the same loop (argument checks and 3 launches);
 *   roundtrip_us   host time of CALLS calls each followed by a stream synchronize.
 * Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include <hip/hip_runtime_api.h>

#include "echo.h"

#define MAX_P 16

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static double now_us(void) {
  struct timespec t;
  clock_gettime(CLOCK_MONOTONIC, &t);
  return (double)t.tv_sec * 1e6 + (double)t.tv_nsec * 1e-3;
}

/* bfloat16 bit pattern of a deterministic pseudo-random value in about [-4, 4) */
static uint16_t sample(uint32_t i, uint32_t r) {
  uint32_t h = i * 2654435761u ^ (r + 1u) * 0x9E3779B9u;
  h ^= h >> 15;
  h *= 0x2c1b3c6du;
  h ^= h >> 12;
  const float x = ((float)(h & 0xFFFFu) - 32768.0f) / 8192.0f;
  uint32_t bits;
  memcpy(&bits, &x, 4);
  return (uint16_t)(bits >> 16);
}

int main(int argc, char** argv) {
  if (argc != 4) {
    fprintf(stderr, "usage: %s P N CALLS\n", argv[0]);
    return 2;
  }
  const int P = atoi(argv[1]);
  const long long N = atoll(argv[2]);
  const int calls = atoi(argv[3]);
  if (P < 1 || P > MAX_P || N < 32 || N % 32 != 0 || calls < 1) {
    fprintf(stderr, "bad arguments\n");
    return 2;
  }
  uint16_t* host = malloc(sizeof(uint16_t) * (size_t)N);
  if (host == NULL) return 1;
  void* parts[MAX_P];
  for (int r = 0; r < P; ++r) {
    for (long long i = 0; i < N; ++i) host[i] = sample((uint32_t)i, (uint32_t)r);
    if (!hip_ok(hipMalloc(&parts[r], sizeof(uint16_t) * (size_t)N), "hipMalloc partial")) return 1;
    if (!hip_ok(hipMemcpy(parts[r], host, sizeof(uint16_t) * (size_t)N, hipMemcpyHostToDevice), "hipMemcpy"))
      return 1;
  }
  free(host);
  void* out = NULL;
  if (!hip_ok(hipMalloc(&out, sizeof(float) * (size_t)N), "hipMalloc out")) return 1;

  echo_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.P = P;
  cfg.numel = N;
  cfg.group = ECHO_GROUP;
  cfg.dtype = ECHO_BF16;
  cfg.compensate = 1;
  cfg.beta_fast = 0.5f;
  cfg.beta_slow = 0.95f;
  const size_t ws_bytes = echo_workspace_bytes(&cfg);
  void* ws = NULL;
  echo_state* st = NULL;
  if (ws_bytes == 0 || !hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc workspace")) return 1;
  if (echo_init_state(&cfg, ws, ws_bytes, NULL, &st) != ECHO_OK) return 1;

  const void* const* pp = (const void* const*)parts;
  for (int i = 0; i < 200; ++i)
    if (echo_reduce(pp, out, st, ECHO_FWD, NULL) != ECHO_OK) return 1;
  if (!hip_ok(hipDeviceSynchronize(), "warm-up")) return 1;

  hipEvent_t e0, e1;
  if (!hip_ok(hipEventCreate(&e0), "event") || !hip_ok(hipEventCreate(&e1), "event")) return 1;
  if (!hip_ok(hipEventRecord(e0, NULL), "record")) return 1;
  const double h0 = now_us();
  for (int i = 0; i < calls; ++i)
    if (echo_reduce(pp, out, st, ECHO_FWD, NULL) != ECHO_OK) return 1;
  const double h1 = now_us();
  if (!hip_ok(hipEventRecord(e1, NULL), "record") || !hip_ok(hipEventSynchronize(e1), "sync")) return 1;
  float ms = 0.0f;
  if (!hip_ok(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;

  const double r0 = now_us();
  for (int i = 0; i < calls; ++i) {
    if (echo_reduce(pp, out, st, ECHO_FWD, NULL) != ECHO_OK) return 1;
    if (!hip_ok(hipStreamSynchronize(NULL), "sync")) return 1;
  }
  const double r1 = now_us();

  printf("{\"P\": %d, \"N\": %lld, \"calls\": %d, \"device_us\": %.3f, \"enqueue_us\": %.3f, "
         "\"roundtrip_us\": %.3f}\n",
         P, N, calls, 1e3 * (double)ms / calls, (h1 - h0) / calls, (r1 - r0) / calls);
  echo_destroy_state(st);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  hipFree(ws);
  hipFree(out);
  for (int r = 0; r < P; ++r) hipFree(parts[r]);
  return 0;
}
