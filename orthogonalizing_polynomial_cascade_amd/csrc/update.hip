// The rest of the bank update after the cascade: the per-lane energy equalizer and the
// sign-aligned decay of a bf16 parameter with a 16-bit mantissa.
//
// Source: modded-nanogpt anvil.py, `_rail_equalizer`, `_sign_aligned_decay_update` and
// `anvil_bank_update`.
//
// Lanes: one per row when rows >= cols (the equalizer reduces over the columns), else one per
// column (reducing over the rows) -- the page's code, whose docstring calls the reduced axis the
// longer one.  Per matrix, in fp32:
//   power[l] = mean over the lane of u^2             pre  = sqrt(sum_l power[l] * len)
//   e[l]     = lerp(e[l], power[l], 1 - beta2)        gain = 1 / sqrt(max(e[l], 1e-10))
//   post     = sqrt(sum_l (power[l] * len) * gain^2)
//   scale[l] = bf16(gain * (pre / max(post, 1e-10)))
//   u       <- bf16(u * scale[lane])
// then, per element, with the fp32 master m = (param bits << 16) | mantissa:
//   m <- (m - ((m * [gate * m >= 0]) * wd) * lr[matrix]) - u * lr[matrix]
//   param bits = high half of m (truncation), mantissa = low half.
//
// lerp is torch's, which the page calls (`lerp_`): d = end - start, then one fused multiply-add
// about the nearer end point, fma(w, d, start) for |w| < 1/2, else fma(w - 1, d, end).
//
// Three kernels: lane powers (deterministic fixed-order reductions), one workgroup per matrix for
// the scales and the energy EMA, and one fused elementwise pass that rescales the update, writes
// it back and applies the decay (HBM-bound: 16 bytes per element with the decay).
#include <algorithm>

#include "device_common.h"
#include "launchers.h"

namespace anvil {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float sqrt_rn(float x) {
  // correctly rounded fp32 square root (fp64 root, then one rounding; 53 >= 2*24 + 2)
  return static_cast<float>(__builtin_sqrt(static_cast<double>(x)));
}

__device__ __forceinline__ float rsqrt_rn(float x) {
  // fp32 of 1/sqrt(x), from fp64
  return static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(x)));
}

// Row lanes (rows >= cols): one wave per row, 8 elements per lane per step, butterfly sum.  The
// grid's x extent is capped (a dispatch counts its work-items in 32 bits); waves then take every
// (gridDim.x * 4)-th row, each row still summed by one wave in the same order.
constexpr int kMaxRowBlocks = 1 << 20;
__global__ __launch_bounds__(kThreads) void lane_power_rows(const uint16_t* __restrict__ u,
                                                            float* __restrict__ power, int m,
                                                            int n) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t b = blockIdx.y;
  const int row_step = gridDim.x * (kThreads / 64);
  for (int row = blockIdx.x * (kThreads / 64) + wave; row < m; row += row_step) {
    const uint16_t* r = u + (b * m + row) * (int64_t)n;
    float s = 0.0f;
    for (int c = lane * 8; c < n; c += 64 * 8) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(r + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_to_f32(v[e] & 0xFFFFu);
        const float hi = bf16_to_f32(v[e] >> 16);
        const float slo = lo * lo;
        const float shi = hi * hi;
        s += slo;
        s += shi;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) power[b * m + row] = s / static_cast<float>(n);
  }
}

// Column lanes (rows < cols): a block covers 64 columns (8 chunks of 8) and 32 row groups; each
// thread sums every 32nd row of its chunk (eight lanes read one row's 128 bytes), then the row
// groups are added in order through LDS.  Small blocks so that even a few wide matrices give
// thousands of workgroups.
constexpr int kColChunks = 8;
constexpr int kRowGroups = kThreads / kColChunks;
__global__ __launch_bounds__(kThreads) void lane_power_cols(const uint16_t* __restrict__ u,
                                                            float* __restrict__ power, int m,
                                                            int n) {
  __shared__ float part[kRowGroups][kColChunks * 8 + 1];
  const int chunk = threadIdx.x % kColChunks;
  const int rg = threadIdx.x / kColChunks;
  const int col0 = blockIdx.x * (kColChunks * 8) + chunk * 8;
  const int64_t b = blockIdx.y;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col0 < n) {
    const uint16_t* base = u + b * (int64_t)m * n + col0;
#pragma unroll 4
    for (int row = rg; row < m; row += kRowGroups) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(base + (int64_t)row * n);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_to_f32(v[e] & 0xFFFFu);
        const float hi = bf16_to_f32(v[e] >> 16);
        const float slo = lo * lo;
        const float shi = hi * hi;
        s[2 * e] += slo;
        s[2 * e + 1] += shi;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][chunk * 8 + e] = s[e];
  __syncthreads();
  if (threadIdx.x < kColChunks * 8) {
    const int col = blockIdx.x * (kColChunks * 8) + threadIdx.x;
    if (col < n) {
      float t = 0.0f;
      for (int g = 0; g < kRowGroups; ++g) t += part[g][threadIdx.x];
      power[b * n + col] = t / static_cast<float>(m);
    }
  }
}

// One workgroup per matrix for the per-lane terms: 1024 threads, a few lanes each.
constexpr int kScaleThreads = 1024;

// Fixed-order block sum of one value per thread (kScaleThreads threads): butterfly within each
// wave, then the wave sums in wave order.
__device__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < kScaleThreads / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// One workgroup per matrix: pre and post norms, the energy EMA, the bf16 lane scales.
__global__ __launch_bounds__(kScaleThreads) void lane_scales(const float* __restrict__ power,
                                                             float* __restrict__ energy,
                                                             float* __restrict__ scale, int lanes,
                                                             int len, float w_coef,
                                                             bool w_from_end) {
  __shared__ float red[kScaleThreads / 64];
  const int64_t b = blockIdx.x;
  const float* pw = power + b * lanes;
  float* en = energy + b * lanes;
  float* sc = scale + b * lanes;
  const float flen = static_cast<float>(len);

  float ps = 0.0f;
  for (int l = threadIdx.x; l < lanes; l += kScaleThreads) ps += pw[l];
  const float psum = block_sum(ps, red);
  const float pre = sqrt_rn(psum * flen);

  float qs = 0.0f;
  for (int l = threadIdx.x; l < lanes; l += kScaleThreads) {
    const float p = pw[l];
    const float e0 = en[l];
    const float e = __builtin_fmaf(w_coef, p - e0, w_from_end ? p : e0);
    en[l] = e;
    const float gain = rsqrt_rn(fmaxf(e, 1e-10f));
    const float pl = p * flen;
    const float g2 = gain * gain;
    qs += pl * g2;
    sc[l] = gain;   // the gain for now; the scale once the post norm is known
  }
  const float post = sqrt_rn(block_sum(qs, red));
  const float ratio = pre / fmaxf(post, 1e-10f);
  for (int l = threadIdx.x; l < lanes; l += kScaleThreads) {
    sc[l] = bf16_to_f32(f32_to_bf16(sc[l] * ratio));
  }
}

struct DecayArgs {
  uint16_t* param;        // nullptr: no decay
  uint16_t* mantissa;
  const float* gate;      // the slow rail
  const float* lr;        // per matrix
  float wd;
  const float* wd_dev;    // when not null, wd is read from here when the kernel runs
};

// Elementwise: u <- bf16(u * scale[lane]) (if scale), write u back (if write_u), then the decay
// (if d.param).  8 elements per thread per step.  Column lanes read their 8 scales with two
// 16-byte loads when the scale array is 16-byte aligned (vec_scale).
__global__ __launch_bounds__(kThreads) void scale_decay(uint16_t* __restrict__ u,
                                                        const float* __restrict__ scale,
                                                        bool vec_scale, bool write_u, DecayArgs d,
                                                        int m, int n, bool row_lanes,
                                                        int64_t chunks_per_matrix, int64_t g) {
  const int64_t total = chunks_per_matrix * g;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
    const int64_t b = c / chunks_per_matrix;
    const int64_t within = (c - b * chunks_per_matrix) * 8;
    const int row = static_cast<int>(within / n);
    const int col = static_cast<int>(within - (int64_t)row * n);
    const int64_t off = c * 8;
    u32x4_t uv = *reinterpret_cast<const u32x4_t*>(u + off);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_to_f32(uv[e] & 0xFFFFu);
      x[2 * e + 1] = bf16_to_f32(uv[e] >> 16);
    }
    if (scale != nullptr) {
      const float* sb = scale + b * (row_lanes ? m : n);
      float sv[8];
      if (row_lanes) {
        const float s = sb[row];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = s;
      } else if (vec_scale) {
        const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(sb + col);
        const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(sb + col + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[e] = s0[e];
          sv[e + 4] = s1[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = sb[col + e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(f32_to_bf16(x[e] * sv[e]));
      if (write_u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) uv[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
        *reinterpret_cast<u32x4_t*>(u + off) = uv;
      }
    }
    if (d.param != nullptr) {
      const float wd = d.wd_dev != nullptr ? *d.wd_dev : d.wd;
      // param, mantissa and gate are touched once per step: stream them past the caches
      const u32x4_t pv =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(d.param + off));
      const u32x4_t mv =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(d.mantissa + off));
      const f32x4_t g0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(d.gate + off));
      const f32x4_t g1 =
          __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(d.gate + off + 4));
      const float gate[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
      const float lr = d.lr[b];
      u32x4_t po, mo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t pb = (e & 1) ? (pv[e >> 1] >> 16) : (pv[e >> 1] & 0xFFFFu);
        const uint32_t mb = (e & 1) ? (mv[e >> 1] >> 16) : (mv[e >> 1] & 0xFFFFu);
        const float master = __uint_as_float((pb << 16) | mb);
        const float aligned = (gate[e] * master >= 0.0f) ? 1.0f : 0.0f;
        const float t1 = ((master * aligned) * wd) * lr;
        const float t2 = x[e] * lr;
        const uint32_t raw = __float_as_uint((master - t1) - t2);
        const uint32_t hi = raw >> 16;
        const uint32_t lo = raw & 0xFFFFu;
        if (e & 1) {
          po[e >> 1] |= hi << 16;
          mo[e >> 1] |= lo << 16;
        } else {
          po[e >> 1] = hi;
          mo[e >> 1] = lo;
        }
      }
      __builtin_nontemporal_store(po, reinterpret_cast<u32x4_t*>(d.param + off));
      __builtin_nontemporal_store(mo, reinterpret_cast<u32x4_t*>(d.mantissa + off));
    }
  }
}

int64_t elementwise_blocks(int64_t chunks) {
  int64_t blocks = (chunks + kThreads - 1) / kThreads;
  const int64_t cap = 256 * 32;   // workgroups per CU: measured on MI355X
  return blocks < 1 ? 1 : (blocks > cap ? cap : blocks);
}

}  // namespace

int equalizer_lanes(const Shape& sh) { return sh.m >= sh.n ? sh.m : sh.n; }

hipError_t launch_equalize(uint16_t* u, float* lane_energy, double beta2, float* scratch,
                           const Shape& sh, hipStream_t stream, uint16_t* param,
                           uint16_t* mantissa, const float* gate, const float* lr, float wd,
                           const float* wd_dev) {
  const bool rows = sh.m >= sh.n;
  const int lanes = equalizer_lanes(sh);
  const int len = rows ? sh.n : sh.m;
  float* power = scratch;
  float* scale = scratch + sh.g * lanes;
  if (rows) {
    const int row_blocks = std::min((sh.m + 3) / 4, kMaxRowBlocks);
    hipLaunchKernelGGL(lane_power_rows, dim3((unsigned)row_blocks, (unsigned)sh.g),
                       dim3(kThreads), 0, stream, u, power, sh.m, sh.n);
  } else {
    hipLaunchKernelGGL(lane_power_cols,
                       dim3((unsigned)((sh.n + kColChunks * 8 - 1) / (kColChunks * 8)),
                            (unsigned)sh.g),
                       dim3(kThreads), 0, stream, u, power, sh.m, sh.n);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 1 - beta2 formed in double and taken as fp32, as the page's lerp weight; the lerp starts
  // from the nearer end point
  const float w_ema = static_cast<float>(1.0 - beta2);
  const bool w_from_end = !(w_ema > -0.5f && w_ema < 0.5f);
  hipLaunchKernelGGL(lane_scales, dim3((unsigned)sh.g), dim3(kScaleThreads), 0, stream, power,
                     lane_energy, scale, lanes, len, w_from_end ? w_ema - 1.0f : w_ema,
                     w_from_end);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  DecayArgs d{param, mantissa, gate, lr, wd, wd_dev};
  const int64_t cpm = (int64_t)sh.m * sh.n / 8;
  // the scale rows start at multiples of 8 floats from `scale`: 16-byte loads need only its base
  const bool vec = (reinterpret_cast<uintptr_t>(scale) & 15u) == 0;
  hipLaunchKernelGGL(scale_decay, dim3((unsigned)elementwise_blocks(cpm * sh.g)), dim3(kThreads),
                     0, stream, u, scale, vec, true, d, sh.m, sh.n, rows, cpm, sh.g);
  return hipGetLastError();
}

hipError_t launch_decay(uint16_t* param, uint16_t* mantissa, const uint16_t* u, float wd,
                        const float* lr, const float* gate, const Shape& sh, hipStream_t stream) {
  DecayArgs d{param, mantissa, gate, lr, wd, nullptr};
  const int64_t cpm = (int64_t)sh.m * sh.n / 8;
  hipLaunchKernelGGL(scale_decay, dim3((unsigned)elementwise_blocks(cpm * sh.g)), dim3(kThreads),
                     0, stream, const_cast<uint16_t*>(u), nullptr, false, false, d, sh.m, sh.n,
                     sh.m >= sh.n, cpm, sh.g);
  return hipGetLastError();
}

}  // namespace anvil
