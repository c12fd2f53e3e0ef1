/*
 * A plain C client of libecho (include/echo.h): device memory from the HIP
 * runtime, no Python and no torch.  Used by tests/test_gpu_c_client.py.
 *
 * For two configurations (the default: bf16 partials, fp32 output; and one
 * with bf16 state, bf16 output and the owners adding their own partials) it
 * creates a state, runs three forward all-reduces of the same partials and
 * writes, into the directory given as the only argument:
 *   parts.bin      P x N bfloat16 partials (uint16 bit patterns, rank-major)
 *   out<c>_<t>.bin the output of call t of configuration c (fp32 or bf16)
 * It also checks that an invalid call is rejected.  Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "echo.h"

#define RANKS 4
#define NUMEL (32 * 1037)

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static int echo_ok(echo_status s, const char* what) {
  if (s != ECHO_OK) {
    fprintf(stderr, "%s: %s\n", what, echo_status_str(s));
    return 0;
  }
  return 1;
}

/* bfloat16 bit pattern of a deterministic pseudo-random value (the top half of a float) */
static uint16_t sample(uint32_t i, uint32_t r) {
  uint32_t h = i * 2654435761u ^ (r + 1u) * 0x9E3779B9u;
  h ^= h >> 15;
  h *= 0x2c1b3c6du;
  h ^= h >> 12;
  float x = ((float)(h & 0xFFFFu) - 32768.0f) / 8192.0f;
  if ((h >> 16) % 997u == 0u) x *= 64.0f; /* a few outliers */
  uint32_t bits;
  memcpy(&bits, &x, 4);
  return (uint16_t)(bits >> 16);
}

static int write_file(const char* dir, const char* name, const void* p, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (f == NULL) return 0;
  const size_t w = fwrite(p, 1, n, f);
  fclose(f);
  return w == n;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s <output directory>\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  uint16_t* host = malloc(sizeof(uint16_t) * RANKS * NUMEL);
  float* hout = malloc(sizeof(float) * NUMEL);
  if (host == NULL || hout == NULL) return 1;
  for (uint32_t r = 0; r < RANKS; ++r)
    for (uint32_t i = 0; i < NUMEL; ++i) host[r * NUMEL + i] = sample(i, r);
  if (!write_file(dir, "parts.bin", host, sizeof(uint16_t) * RANKS * NUMEL)) return 1;

  void* parts[RANKS];
  for (int r = 0; r < RANKS; ++r) {
    if (!hip_ok(hipMalloc(&parts[r], sizeof(uint16_t) * NUMEL), "hipMalloc partial")) return 1;
    if (!hip_ok(hipMemcpy(parts[r], host + (size_t)r * NUMEL, sizeof(uint16_t) * NUMEL, hipMemcpyHostToDevice),
                "hipMemcpy partial"))
      return 1;
  }
  void* out = NULL;
  if (!hip_ok(hipMalloc(&out, sizeof(float) * NUMEL), "hipMalloc out")) return 1;

  for (int c = 0; c < 2; ++c) {
    echo_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.P = RANKS;
    cfg.numel = NUMEL;
    cfg.group = ECHO_GROUP;
    cfg.dtype = ECHO_BF16;
    cfg.compensate = 1;
    cfg.beta_fast = 0.5f;
    cfg.beta_slow = 0.95f;
    if (c == 1) {
      cfg.state_bf16 = 1;
      cfg.out_bf16 = 1;
      cfg.own_exact = 1;
    }
    const size_t ws_bytes = echo_workspace_bytes(&cfg);
    void* ws = NULL;
    echo_state* st = NULL;
    if (ws_bytes == 0 || !hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc workspace")) return 1;
    if (!echo_ok(echo_init_state(&cfg, ws, ws_bytes, NULL, &st), "echo_init_state")) return 1;
    /* an invalid call is rejected and launches nothing */
    if (echo_reduce(NULL, out, st, ECHO_FWD, NULL) != ECHO_ERR_ARG) {
      fprintf(stderr, "echo_reduce accepted a null partial array\n");
      return 1;
    }
    const size_t out_bytes = (cfg.out_bf16 ? 2 : 4) * (size_t)NUMEL;
    for (int t = 0; t < 3; ++t) {
      if (!echo_ok(echo_reduce((const void* const*)parts, out, st, ECHO_FWD, NULL), "echo_reduce")) return 1;
      if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) return 1;
      if (!hip_ok(hipMemcpy(hout, out, out_bytes, hipMemcpyDeviceToHost), "hipMemcpy out")) return 1;
      char name[64];
      snprintf(name, sizeof name, "out%d_%d.bin", c, t);
      if (!write_file(dir, name, hout, out_bytes)) return 1;
    }
    echo_destroy_state(st);
    if (!hip_ok(hipFree(ws), "hipFree workspace")) return 1;
  }
  for (int r = 0; r < RANKS; ++r) hipFree(parts[r]);
  hipFree(out);
  free(host);
  free(hout);
  printf("c client ok: P=%d N=%d, 2 configurations x 3 calls\n", RANKS, NUMEL);
  return 0;
}
