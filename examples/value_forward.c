/* The MoVA value projection called from C through the library's C ABI.
 *
 * Builds a small synthetic layer on the host (bf16 tokens, router and
 * expert weights from a fixed-seed generator), copies it to the current
 * GPU, queries the workspace size, runs mova_value_forward on the default
 * stream and prints a checksum of the bf16 output [T, n_kv_heads,
 * head_dim] and the routing.  With a file argument it also writes the
 * shapes, inputs and results there (raw little-endian arrays, in argument
 * order), so that a test can recompute them another way.
 *
 * Build (mixture_value_projection_amd/build.py does this):
 *   clang -O2 -D__HIP_PLATFORM_AMD__ -I include -I /opt/rocm/include \
 *     examples/value_forward.c -L <lib dir> -lmova -L /opt/rocm/lib -lamdhip64
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mova.h"

/* fp32 -> bf16, round to nearest even (finite inputs). */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float bf16_to_float(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Uniform in [-1, 1) from a 32-bit linear congruential generator. */
static float uniform(uint32_t* s) {
  *s = *s * 1664525u + 1013904223u;
  return (float)(*s >> 8) / 8388608.0f - 1.0f;
}

#define CHECK(call)                                                        \
  do {                                                                     \
    hipError_t e_ = (call);                                                \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));           \
      return 1;                                                            \
    }                                                                      \
  } while (0)

int main(int argc, char** argv) {
  const int T = 64, d = 256, E = 8, k = 2, H = 2, D = 64, N = H * D;
  const float scale = 2.5f;
  const size_t nx = (size_t)T * d, nr = (size_t)E * d, nw = (size_t)E * N * d, no = (size_t)T * N;

  uint16_t* x = malloc(nx * 2);
  uint16_t* rw = malloc(nr * 2);
  float* rb = malloc(E * sizeof(float));
  uint16_t* ew = malloc(nw * 2);
  uint16_t* out = malloc(no * 2);
  int32_t* idx = malloc((size_t)T * k * sizeof(int32_t));
  float* w = malloc((size_t)T * k * sizeof(float));
  if (!x || !rw || !rb || !ew || !out || !idx || !w) return 1;
  uint32_t s = 12345u;
  for (size_t i = 0; i < nx; ++i) x[i] = to_bf16(uniform(&s));
  for (size_t i = 0; i < nr; ++i) rw[i] = to_bf16(0.05f * uniform(&s));
  for (int i = 0; i < E; ++i) rb[i] = 0.01f * uniform(&s);
  for (size_t i = 0; i < nw; ++i) ew[i] = to_bf16(uniform(&s) / sqrtf((float)d));

  void *dx, *drw, *drb, *dew, *dout, *didx, *dw, *dws = NULL;
  CHECK(hipMalloc(&dx, nx * 2));
  CHECK(hipMalloc(&drw, nr * 2));
  CHECK(hipMalloc(&drb, E * sizeof(float)));
  CHECK(hipMalloc(&dew, nw * 2));
  CHECK(hipMalloc(&dout, no * 2));
  CHECK(hipMalloc(&didx, (size_t)T * k * sizeof(int32_t)));
  CHECK(hipMalloc(&dw, (size_t)T * k * sizeof(float)));
  CHECK(hipMemcpy(dx, x, nx * 2, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(drw, rw, nr * 2, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(drb, rb, E * sizeof(float), hipMemcpyHostToDevice));
  CHECK(hipMemcpy(dew, ew, nw * 2, hipMemcpyHostToDevice));

  const size_t ws_bytes = mova_workspace_bytes(T, d, E, k, H, D);
  if (ws_bytes == (size_t)-1) {
    fprintf(stderr, "shape outside the supported domain\n");
    return 1;
  }
  if (ws_bytes > 0) CHECK(hipMalloc(&dws, ws_bytes));  /* 256-byte aligned */

  const int rc = mova_value_forward(dx, drw, (const float*)drb, dew, T, d, E, k, scale, H, D, dout,
                                    (int32_t*)didx, (float*)dw, dws, ws_bytes, NULL);
  if (rc != MOVA_OK) {
    fprintf(stderr, "mova_value_forward: %s\n", mova_status_str(rc));
    return 1;
  }
  CHECK(hipDeviceSynchronize());
  CHECK(hipMemcpy(out, dout, no * 2, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(idx, didx, (size_t)T * k * sizeof(int32_t), hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(w, dw, (size_t)T * k * sizeof(float), hipMemcpyDeviceToHost));

  double sum = 0.0;
  for (size_t i = 0; i < no; ++i) sum += bf16_to_float(out[i]);
  printf("mova %d: T=%d d=%d E=%d k=%d out[%d,%d,%d] sum %.6f, token 0 -> experts %d %d\n",
         mova_version(), T, d, E, k, T, H, D, sum, idx[0], idx[1]);

  if (argc > 1) {
    FILE* f = fopen(argv[1], "wb");
    if (!f) return 1;
    const int32_t shapes[6] = {T, d, E, k, H, D};
    fwrite(shapes, sizeof shapes, 1, f);
    fwrite(x, 2, nx, f);
    fwrite(rw, 2, nr, f);
    fwrite(rb, sizeof(float), E, f);
    fwrite(ew, 2, nw, f);
    fwrite(out, 2, no, f);
    fwrite(idx, sizeof(int32_t), (size_t)T * k, f);
    fwrite(w, sizeof(float), (size_t)T * k, f);
    fclose(f);
  }
  hipFree(dx);
  hipFree(drw);
  hipFree(drb);
  hipFree(dew);
  hipFree(dout);
  hipFree(didx);
  hipFree(dw);
  if (dws) hipFree(dws);
  free(x);
  free(rw);
  free(rb);
  free(ew);
  free(out);
  free(idx);
  free(w);
  return 0;
}
