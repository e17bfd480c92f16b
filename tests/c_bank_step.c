/* A plain C consumer of libanvil.so on the GPU: reads a gradient stack from a file, runs one
 * anvil_bank_step through the C ABI with memory from the HIP runtime API (no torch, no Python),
 * and writes the bf16 update and the rails to files.
 *
 *   c_bank_step g m n momentum fast_beta fast_weight grad.f32 out.bf16 velocity.f32
 *
 * Exit status 0 on success; otherwise it prints the failing call and its status. */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "anvil.h"

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    printf("%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

int main(int argc, char** argv) {
  if (argc != 10) {
    printf("usage: c_bank_step g m n momentum fast_beta fast_weight grad out velocity\n");
    return 2;
  }
  const int64_t g = atoll(argv[1]), m = atoll(argv[2]), n = atoll(argv[3]);
  const float mu = (float)atof(argv[4]), fb = (float)atof(argv[5]), fw = (float)atof(argv[6]);
  const size_t cnt = (size_t)(g * m * n);
  float* grad_h = malloc(cnt * sizeof(float));
  uint16_t* out_h = malloc(cnt * sizeof(uint16_t));
  float* vel_h = malloc(2 * cnt * sizeof(float));
  if (!grad_h || !out_h || !vel_h) return 3;
  FILE* f = fopen(argv[7], "rb");
  if (!f || fread(grad_h, sizeof(float), cnt, f) != cnt) return 4;
  fclose(f);

  float *grad = NULL, *vel = NULL;
  uint16_t* out = NULL;
  void* ws = NULL;
  const size_t ws_bytes = anvil_workspace_bytes(g, m, n);
  if (ws_bytes == 0) return 5;
  if (!hip_ok(hipMalloc((void**)&grad, cnt * sizeof(float)), "hipMalloc grad") ||
      !hip_ok(hipMalloc((void**)&vel, 2 * cnt * sizeof(float)), "hipMalloc velocity") ||
      !hip_ok(hipMalloc((void**)&out, cnt * sizeof(uint16_t)), "hipMalloc out") ||
      !hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc workspace") ||
      !hip_ok(hipMemcpy(grad, grad_h, cnt * sizeof(float), hipMemcpyHostToDevice), "copy grad") ||
      !hip_ok(hipMemset(vel, 0, 2 * cnt * sizeof(float)), "clear velocity"))
    return 6;

  const int st = anvil_bank_step_ws(grad, vel, mu, fb, fw, out, g, m, n, ws, ws_bytes, NULL);
  if (st != ANVIL_OK) {
    printf("anvil_bank_step_ws: %s\n", anvil_status_string(st));
    return 7;
  }
  if (!hip_ok(hipDeviceSynchronize(), "synchronize") ||
      !hip_ok(hipMemcpy(out_h, out, cnt * sizeof(uint16_t), hipMemcpyDeviceToHost), "copy out") ||
      !hip_ok(hipMemcpy(vel_h, vel, 2 * cnt * sizeof(float), hipMemcpyDeviceToHost), "copy vel"))
    return 8;
  f = fopen(argv[8], "wb");
  if (!f || fwrite(out_h, sizeof(uint16_t), cnt, f) != cnt) return 9;
  fclose(f);
  f = fopen(argv[9], "wb");
  if (!f || fwrite(vel_h, sizeof(float), 2 * cnt, f) != 2 * cnt) return 10;
  fclose(f);
  hipFree(grad);
  hipFree(vel);
  hipFree(out);
  hipFree(ws);
  free(grad_h);
  free(out_h);
  free(vel_h);
  printf("ok\n");
  return 0;
}
