// Frobenius normalisation of the cascade input.
//
// Source: modded-nanogpt anvil.py, `anvil_cascade`, the normalisation step after the first Gram.
// The sum of a Gram matrix's diagonal is the squared Frobenius norm of X, so one Gram of the
// unscaled X yields both the scale d = sqrt(trace) * 1.05 + 1e-6 and, divided by d^2, the Gram of
// the scaled X that the first map needs.
//
// The trace arrives as per-diagonal-tile partial sums written by the map-0 Gram; each workgroup
// sums them in slot order (deterministic), forms d in fp32, and rewrites its share of X and A in
// place: x <- bf16(x / d), a <- bf16(a / (d*d)), with correctly rounded fp32 division.  The square
// root is taken in fp64 and rounded to fp32, which gives the correctly rounded fp32 square root
// (53 >= 2*24 + 2 bits, so the double rounding is innocuous).  HBM-bound: 4 bytes per element.
#include "device_common.h"
#include "launchers.h"

namespace anvil {

namespace {

__device__ __forceinline__ uint32_t div_pair(uint32_t w, float d) {
  const float lo = bf16_to_f32(w & 0xFFFFu) / d;
  const float hi = bf16_to_f32(w >> 16) / d;
  return pack_bf16x2(lo, hi);
}

__global__ __launch_bounds__(256) void normalize_kernel(u32x4_t* __restrict__ x, int64_t x_chunks,
                                                        u32x4_t* __restrict__ a, int64_t a_chunks,
                                                        const float* __restrict__ partials,
                                                        int slots, float* __restrict__ d_out) {
  const int64_t b = blockIdx.y;
  float tr = 0.0f;
  for (int s = 0; s < slots; ++s) tr += partials[b * slots + s];
  const float root = static_cast<float>(__builtin_sqrt(static_cast<double>(tr)));
  const float scaled = root * 1.05f;
  const float d = scaled + 1e-6f;
  const float dd = d * d;
  if (d_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) d_out[b] = d;

  u32x4_t* xb = x + b * x_chunks;
  u32x4_t* ab = a + b * a_chunks;
  const int64_t total = x_chunks + a_chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    u32x4_t* ptr = i < x_chunks ? xb + i : ab + (i - x_chunks);
    const float div = i < x_chunks ? d : dd;
    u32x4_t v = *ptr;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = div_pair(v[e], div);
    *ptr = v;
  }
}

}  // namespace

hipError_t launch_normalize(uint16_t* x, uint16_t* a, const float* trace_partials, float* d,
                            const Shape& sh, hipStream_t stream) {
  const int s = sh.s();
  const int64_t x_chunks = (int64_t)sh.m * sh.n / 8;
  const int64_t a_chunks = (int64_t)s * s / 8;
  int64_t blocks = (x_chunks + a_chunks + 1023) / 1024;   // about 4 chunks per thread
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(normalize_kernel, dim3((unsigned)blocks, (unsigned)sh.g), dim3(256), 0,
                     stream, reinterpret_cast<u32x4_t*>(x), x_chunks,
                     reinterpret_cast<u32x4_t*>(a), a_chunks, trace_partials,
                     gram_trace_slots(sh), d);
  return hipGetLastError();
}

}  // namespace anvil
