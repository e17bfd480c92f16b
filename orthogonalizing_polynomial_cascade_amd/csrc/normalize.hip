// Frobenius normalisation of the cascade input.
//
// Source: modded-nanogpt anvil.py, `anvil_cascade`, the normalisation step after the first Gram.
// The sum of a Gram matrix's diagonal is the squared Frobenius norm of X, so one Gram of the
// unscaled X yields both the scale d = sqrt(trace) * 1.05 + 1e-6 and, divided by d^2, the Gram of
// the scaled X that the first map needs.
//
// The trace arrives as per-diagonal-tile partial sums written by the map-0 Gram; each workgroup
// sums them in slot order (deterministic), forms d in fp32, and rewrites its share of X and A in
// place: x <- bf16(x / d), a <- bf16(a / (d*d)), each quotient the correctly rounded fp32 one.  The
// square root is taken in fp64 and rounded to fp32, which gives the correctly rounded fp32 square
// root (53 >= 2*24 + 2 bits, so the double rounding is innocuous).
//
// HBM-bound (4 bytes per element), but a full-precision fp32 division per element would make the
// pass as VALU-bound as it is memory-bound.  Since the divisor is one value per matrix, each
// quotient comes instead from the correctly rounded reciprocal r = 1/d: q = x*r, its exact
// remainder x - q*d (one fused multiply-add) and one correction q + remainder*r (another), which
// is the correctly rounded quotient whenever x and q lie in [2^-100, 2^100] (no remainder falls
// below the normal range; checked against the correctly rounded division for every bf16 x and
// thousands of divisors).  Chunks holding any value outside that range, zeros, infinities or NaN
// use the division itself.  Each thread moves 4 chunks of 16 bytes per iteration, loads first.
#include "device_common.h"
#include "launchers.h"

namespace anvil {

namespace {

struct Divisor {
  float d, r;   // the divisor and its correctly rounded reciprocal
};

__device__ __forceinline__ bool fast_ok(float x, float q) {
  const float ax = fabsf(x), aq = fabsf(q);
  return ax >= 0x1p-100f && ax <= 0x1p100f && aq >= 0x1p-100f && aq <= 0x1p100f;
}

// bf16(x / d) for the 8 bf16 values of one 16-byte chunk.
__device__ __forceinline__ u32x4_t div_chunk(u32x4_t v, Divisor dv) {
  float x[8], q[8];
  bool ok = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = bf16_to_f32((e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xFFFFu));
    q[e] = x[e] * dv.r;
    ok = ok && fast_ok(x[e], q[e]);
  }
  if (ok) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float rem = __builtin_fmaf(-q[e], dv.d, x[e]);
      q[e] = __builtin_fmaf(rem, dv.r, q[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = x[e] / dv.d;
  }
  u32x4_t out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(q[2 * e], q[2 * e + 1]);
  return out;
}

constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void normalize_kernel(u32x4_t* __restrict__ x, int64_t x_chunks,
                                                        u32x4_t* __restrict__ a, int64_t a_chunks,
                                                        const float* __restrict__ partials,
                                                        int slots, float* __restrict__ d_out) {
  const int64_t b = blockIdx.y;
  u32x4_t* xb = x + b * x_chunks;
  u32x4_t* ab = a + b * a_chunks;
  const int64_t total = x_chunks + a_chunks;
  const int64_t chunk = (int64_t)kUnroll * blockDim.x;
  const int64_t stride = chunk * gridDim.x;
  auto load = [&](u32x4_t* v, int64_t base) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * blockDim.x;
      if (i < total) v[u] = i < x_chunks ? xb[i] : ab[i - x_chunks];
    }
  };
  // the first chunks are requested before the trace partials, so both latencies overlap
  int64_t base = (int64_t)blockIdx.x * chunk + threadIdx.x;
  u32x4_t v[kUnroll];
  if (base < total) load(v, base);

  float tr = 0.0f;
  for (int s = 0; s < slots; ++s) tr += partials[b * slots + s];
  const float root = static_cast<float>(__builtin_sqrt(static_cast<double>(tr)));
  const float scaled = root * 1.05f;
  const float d = scaled + 1e-6f;
  const float dd = d * d;
  if (d_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) d_out[b] = d;
  // correctly rounded reciprocals (fp64 quotient rounded once to fp32: 53 >= 2*24 + 2)
  const Divisor dx{d, static_cast<float>(1.0 / static_cast<double>(d))};
  const Divisor da{dd, static_cast<float>(1.0 / static_cast<double>(dd))};

  for (; base < total; base += stride) {
    if (base != (int64_t)blockIdx.x * chunk + threadIdx.x) load(v, base);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * blockDim.x;
      if (i >= total) continue;
      if (i < x_chunks) {
        xb[i] = div_chunk(v[u], dx);
      } else {
        ab[i - x_chunks] = div_chunk(v[u], da);
      }
    }
  }
}

}  // namespace

hipError_t launch_normalize(uint16_t* x, uint16_t* a, const float* trace_partials, float* d,
                            const Shape& sh, hipStream_t stream) {
  const int s = sh.s();
  const int64_t x_chunks = (int64_t)sh.m * sh.n / 8;
  const int64_t a_chunks = (int64_t)s * s / 8;
  int64_t blocks = (x_chunks + a_chunks + 256 * kUnroll - 1) / (256 * kUnroll);
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(normalize_kernel, dim3((unsigned)blocks, (unsigned)sh.g), dim3(256), 0,
                     stream, reinterpret_cast<u32x4_t*>(x), x_chunks,
                     reinterpret_cast<u32x4_t*>(a), a_chunks, trace_partials,
                     gram_trace_slots(sh), d);
  return hipGetLastError();
}

}  // namespace anvil
