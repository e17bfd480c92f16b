// Kernel 1: fused twin-rail momentum and bf16 cast.
//
// Source: modded-nanogpt anvil.py, `anvil_cascade`, momentum block.  Per element, in fp32:
//   v0 <- lerp(v0, g, wf)               wf = 1.0f - fast_beta
//   v1 <- lerp(v1, g, ws)               ws = (float)(1 - 0.98)
//   blend = w * v0 + (1 - w) * v1       w = fast_weight; three separately rounded operations
//   y = lerp(g, blend, mu)              mu = momentum
//   x = bf16(y)                         round to nearest even
// where lerp is torch's (the page calls `lerp_`): d = end - start, then one fused multiply-add
// about the nearer end, fma(w, d, start) for |w| < 1/2, else fma(w - 1, d, end).  The file is
// built with -ffp-contract=off, so the fused operations are exactly the explicit fmaf calls.
//
// HBM-bound: each element reads grad (4 B, or 2 B for a bf16 gradient, which the page widens to
// fp32 exactly before the lerps) and both rails (8 B) and writes both rails (8 B) and x (2 B) —
// 22 (20) bytes, touched once.  Each thread moves groups of 4 elements with 16-byte loads and
// stores (8-byte for x and a bf16 grad), several groups per iteration with all loads issued
// first; grad and the rails stream through with non-temporal accesses, x stays cacheable for the
// Gram after it.  The rail scalars come by value, or from a device array read when the kernel
// runs (so a captured graph picks up their current values).
#include "device_common.h"
#include "launchers.h"

namespace anvil {

namespace {

// One lerp weight as torch forms it: the multiplier of end - start and which end point the fused
// multiply-add starts from (the nearer one).
struct LerpWeight {
  float coef;
  bool from_end;
};

__host__ __device__ __forceinline__ LerpWeight lerp_weight(float w) {
  const bool big = !(w > -0.5f && w < 0.5f);
  return LerpWeight{big ? w - 1.0f : w, big};
}

__device__ __forceinline__ float lerp_torch(float start, float end, LerpWeight lw) {
  const float d = end - start;
  return __builtin_fmaf(lw.coef, d, lw.from_end ? end : start);
}

struct RailWeights {
  LerpWeight wf, ws, mu;
  float w, omw;
};

// The rail weights from the fp32 scalars (momentum, fast_beta, fast_weight): 1 - fast_beta and
// 1 - fast_weight are fp32 subtractions; the slow weight is the host double 1 - 0.98 taken as
// fp32 (0.02f).
__host__ __device__ __forceinline__ RailWeights rail_weights(float momentum, float fast_beta,
                                                             float fast_weight) {
  RailWeights rw;
  rw.wf = lerp_weight(1.0f - fast_beta);
  rw.ws = lerp_weight(static_cast<float>(1.0 - 0.98));
  rw.w = fast_weight;
  rw.omw = 1.0f - fast_weight;
  rw.mu = lerp_weight(momentum);
  return rw;
}

// Groups of 4 elements per thread per iteration, and workgroups per CU of the grid (grid-stride
// beyond); chosen by measurement on MI355X (about 6.7 TB/s on the 24x2816x768 bank, against 5.2
// with 16 workgroups per CU and cacheable rail loads).  Banks of at most 2^24 elements take one
// group per thread (more, shorter threads: qk 24.9 -> 22.6 us, vo 54.2 -> 51.6 us); on the
// larger banks that costs 4-11%.
constexpr int kUnroll = 4;
constexpr int kSmallUnroll = 1;
constexpr int64_t kSmallCount = int64_t(1) << 24;
constexpr int kBlocksPerCu = 64;

// 4 gradient values as fp32: a 16-byte fp32 load, or an 8-byte bf16 load widened exactly.
__device__ __forceinline__ f32x4_t load_grad4(const float* grad, int64_t i) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(grad) + i);
}
__device__ __forceinline__ f32x4_t load_grad4(const uint16_t* grad, int64_t i) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(grad) + i);
  return f32x4_t{bf16_to_f32(v[0] & 0xFFFFu), bf16_to_f32(v[0] >> 16),
                 bf16_to_f32(v[1] & 0xFFFFu), bf16_to_f32(v[1] >> 16)};
}

// Each thread moves UNROLL groups of 4 elements per iteration: all loads first (3*UNROLL
// loads in flight), then the arithmetic, then the stores.  A block covers UNROLL*256
// consecutive groups, so every load and store instruction stays coalesced.  `scalars`, when not
// null, holds (momentum, fast_beta, fast_weight) on the device and replaces `rw`.
template <int UNROLL, typename GradT>
__global__ __launch_bounds__(256) void momentum_kernel(const GradT* __restrict__ grad,
                                                       f32x4_t* __restrict__ v0,
                                                       f32x4_t* __restrict__ v1,
                                                       u32x2_t* __restrict__ x, int64_t n4,
                                                       RailWeights rw,
                                                       const float* __restrict__ scalars) {
  if (scalars != nullptr) rw = rail_weights(scalars[0], scalars[1], scalars[2]);
  const int64_t chunk = (int64_t)UNROLL * blockDim.x;
  const int64_t stride = chunk * gridDim.x;
  for (int64_t base = (int64_t)blockIdx.x * chunk + threadIdx.x; base < n4; base += stride) {
    f32x4_t g[UNROLL], a[UNROLL], c[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * blockDim.x;
      if (i < n4) {
        g[u] = load_grad4(grad, i);
        a[u] = __builtin_nontemporal_load(v0 + i);
        c[u] = __builtin_nontemporal_load(v1 + i);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * blockDim.x;
      if (i >= n4) continue;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[u][e] = lerp_torch(a[u][e], g[u][e], rw.wf);
        c[u][e] = lerp_torch(c[u][e], g[u][e], rw.ws);
        const float blend = rw.w * a[u][e] + rw.omw * c[u][e];
        y[e] = lerp_torch(g[u][e], blend, rw.mu);
      }
      // the rails are next read one step later: stream them past the caches
      __builtin_nontemporal_store(a[u], v0 + i);
      __builtin_nontemporal_store(c[u], v1 + i);
      u32x2_t packed;
      packed[0] = pack_bf16x2(y[0], y[1]);
      packed[1] = pack_bf16x2(y[2], y[3]);
      x[i] = packed;   // read right away by the first Gram: keep it cacheable
    }
  }
}

template <int UNROLL, typename GradT>
hipError_t launch_momentum_u(const GradT* grad, float* v0, float* v1, uint16_t* x, int64_t count,
                             RailWeights rw, const float* scalars, hipStream_t stream) {
  const int64_t n4 = count / 4;
  const int threads = 256;
  int64_t blocks = (n4 + threads * UNROLL - 1) / (threads * UNROLL);
  const int64_t max_blocks = 256 * kBlocksPerCu;
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((momentum_kernel<UNROLL, GradT>), dim3((unsigned)blocks), dim3(threads), 0,
                     stream, grad, reinterpret_cast<f32x4_t*>(v0), reinterpret_cast<f32x4_t*>(v1),
                     reinterpret_cast<u32x2_t*>(x), n4, rw, scalars);
  return hipGetLastError();
}

template <typename GradT>
hipError_t launch_momentum_t(const GradT* grad, float* v0, float* v1, uint16_t* x, int64_t count,
                             RailWeights rw, const float* scalars, hipStream_t stream) {
  if (count <= kSmallCount)
    return launch_momentum_u<kSmallUnroll>(grad, v0, v1, x, count, rw, scalars, stream);
  return launch_momentum_u<kUnroll>(grad, v0, v1, x, count, rw, scalars, stream);
}

}  // namespace

hipError_t launch_momentum(const float* grad, float* v0, float* v1, uint16_t* x, int64_t count,
                           float momentum, float fast_beta, float fast_weight,
                           hipStream_t stream) {
  return launch_momentum_t(grad, v0, v1, x, count, rail_weights(momentum, fast_beta, fast_weight),
                           nullptr, stream);
}

hipError_t launch_momentum_dev(const void* grad, bool grad_bf16, float* v0, float* v1,
                               uint16_t* x, int64_t count, const float* scalars,
                               hipStream_t stream) {
  const RailWeights unused = rail_weights(0.0f, 0.0f, 0.0f);
  if (grad_bf16)
    return launch_momentum_t(static_cast<const uint16_t*>(grad), v0, v1, x, count, unused,
                             scalars, stream);
  return launch_momentum_t(static_cast<const float*>(grad), v0, v1, x, count, unused, scalars,
                           stream);
}

}  // namespace anvil
