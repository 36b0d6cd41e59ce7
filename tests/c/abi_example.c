/* A plain C user of the C ABI (include/lowbit.h): packs ternary codes, runs
 * one low-bit linear on the current GPU and prints the FP32 outputs, one per
 * line, for a test to compare with the CPU oracle. Device memory and copies
 * come from the HIP runtime's C API; nothing here knows about Python.
 *
 * usage: abi_example M N K   (inputs are made here from a fixed LCG; the
 * test recreates the same inputs from the same recipe) */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "lowbit.h"

/* the few HIP runtime entry points used, declared by hand to stay plain C */
typedef int hipError_t;
hipError_t hipMalloc(void** ptr, size_t size);
hipError_t hipFree(void* ptr);
hipError_t hipMemcpy(void* dst, const void* src, size_t size, int kind);
hipError_t hipDeviceSynchronize(void);
enum { H2D = 1, D2H = 2 };

static uint32_t lcg = 12345u;
static uint32_t next(void) { lcg = lcg * 1664525u + 1013904223u; return lcg >> 8; }

#define CHECK(x) do { int s_ = (x); if (s_) { fprintf(stderr, "%s failed: %d\n", #x, s_); return 1; } } while (0)

int main(int argc, char** argv) {
  if (argc != 4) { fprintf(stderr, "usage: %s M N K\n", argv[0]); return 2; }
  const int64_t M = atoll(argv[1]), N = atoll(argv[2]), K = atoll(argv[3]);
  int8_t* t = malloc((size_t)(N * K));
  uint16_t* x = malloc((size_t)(M * K) * 2);
  uint16_t* s = malloc((size_t)(N * K / LOWBIT_GROUP) * 2);
  float* y = malloc((size_t)(M * N) * 4);
  /* codes in {-1, 0, 1}; activations: bf16 of small integers / 8 (exact);
     scales: fp16 powers of two 2^-3 .. 2^0 (exact) */
  for (int64_t i = 0; i < N * K; ++i) t[i] = (int8_t)((int)(next() % 3) - 1);
  for (int64_t i = 0; i < M * K; ++i) {
    const int v = (int)(next() % 17) - 8;                 /* -8 .. 8 */
    const float f = (float)v / 8.0f;
    union { float f; uint32_t u; } c = {f};
    x[i] = (uint16_t)(c.u >> 16);                         /* exact in bf16 */
  }
  for (int64_t i = 0; i < N * K / LOWBIT_GROUP; ++i) s[i] = (uint16_t)(0x3000 + 0x400 * (next() % 4));
  void *dt, *dp, *dx, *ds, *dy;
  const int64_t pb = lowbit_packed_bytes(LOWBIT_TERNARY_INT2, N, K);
  CHECK(pb < 0);
  CHECK(hipMalloc(&dt, (size_t)(N * K)));
  CHECK(hipMalloc(&dp, (size_t)pb));
  CHECK(hipMalloc(&dx, (size_t)(M * K) * 2));
  CHECK(hipMalloc(&ds, (size_t)(N * K / LOWBIT_GROUP) * 2));
  CHECK(hipMalloc(&dy, (size_t)(M * N) * 4));
  CHECK(hipMemcpy(dt, t, (size_t)(N * K), H2D));
  CHECK(hipMemcpy(dx, x, (size_t)(M * K) * 2, H2D));
  CHECK(hipMemcpy(ds, s, (size_t)(N * K / LOWBIT_GROUP) * 2, H2D));
  CHECK(lowbit_init());
  CHECK(pack_ternary(dt, N, K, dp, NULL, NULL));
  const size_t wsb = lowbit_gemm_workspace_bytes(LOWBIT_TERNARY_INT2, M, N, K);
  void* dws = NULL;
  if (wsb) {
    CHECK(hipMalloc(&dws, wsb));
    uint8_t* zero = calloc(wsb, 1);
    CHECK(hipMemcpy(dws, zero, wsb, H2D));
    free(zero);
  }
  CHECK(lowbit_gemm(LOWBIT_TERNARY_INT2, dx, LOWBIT_BF16, M, K, K, dp, ds, LOWBIT_GROUP, N, NULL, LOWBIT_NONE,
                    dy, LOWBIT_F32, N, LOWBIT_ACT_NONE, dws, wsb, NULL));
  CHECK(hipDeviceSynchronize());
  CHECK(hipMemcpy(y, dy, (size_t)(M * N) * 4, D2H));
  for (int64_t i = 0; i < M * N; ++i) printf("%.9g\n", y[i]);
  hipFree(dt); hipFree(dp); hipFree(dx); hipFree(ds); hipFree(dy);
  if (dws) hipFree(dws);
  free(t); free(x); free(s); free(y);
  return 0;
}
