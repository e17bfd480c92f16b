// Kernels 2-4: the Gram, polynomial and apply products of the ANVIL cascade on bf16 MFMA.
//
// Source: modded-nanogpt anvil.py, `anvil_cascade` (tall and wide branches).  Every product in the
// cascade is one of three batched contractions over a stack of matrices, all written here as
//
//     C[i][j] = sum_k P(i, k) * Q(j, k)          (fp32 accumulation on v_mfma_f32_32x32x16_bf16)
//
// with a fused fp32 epilogue and a single bf16 rounding at the page's storage points:
//
//   Gram   A = X^T X (tall: P = Q = X read down its columns, "K-strided")
//          A = X X^T (wide: P = Q = X read along its rows, "K-contiguous")
//          epilogue bf16(acc); optional trace partials of the bf16 diagonal.
//   poly   B = b A + c A A   (A symmetric, so A A = A A^T: P = Q = A, K-contiguous)
//          epilogue bf16(b * A[i][j] + c * acc).
//   apply  tall: C = a X + X B   (P = X, Q = B rows; B symmetric so B[k][j] = B[j][k])
//          wide: C = a X + B X   (P = B, Q(j, k) = X[k][j]: K-strided)
//          epilogue bf16(a * X[i][j] + acc), or with split rounding
//          bf16(bf16(acc) + a * X[i][j]) (the page's two-kernel form for banks of > 1024 rows).
//
// The Gram and the polynomial are symmetric, so only tiles on or above the diagonal are computed;
// each is stored twice (C[i][j] and C[j][i]) from the same fp32 value, which keeps the stored
// matrices exactly symmetric.  Inside a diagonal tile only entries with i <= j are stored.
//
// Tiling: 256 threads (4 waves of 64) per 128x128 output tile, waves in a 2x2 grid, each wave a
// 64x64 block of 2x2 MFMA 32x32 fragments.  K advances in steps of 64 through double-buffered
// LDS; the next K-slab is fetched into registers while the current one feeds the MFMAs, so one
// barrier per slab suffices.  LDS rows hold one operand row with K contiguous (plus 8 bf16 of
// padding), so each MFMA operand is one 16-byte LDS read per lane.  K-strided operands (X read
// down its columns) are transposed on the way into LDS: a thread fetches a 4(k) x 8(i) block as
// four 16-byte row segments and rewrites it as eight 4-element K-runs.
//
// Shapes: M, N, K are multiples of 8; partial tiles at the M, N and K edges are zero-filled on
// load and masked on store.
#include "device_common.h"
#include "launchers.h"

namespace anvil {

namespace {

enum { OP_GRAM = 0, OP_POLY = 1, OP_APPLY = 2 };

constexpr int kThreads = 256;
constexpr int kBM = 128;          // output tile rows
constexpr int kBN = 128;          // output tile cols
constexpr int kBK = 64;           // K per LDS slab
constexpr int kPad = 8;           // bf16 padding per LDS row
constexpr int kLds = kBK + kPad;  // LDS row pitch in bf16

struct GemmParams {
  const uint16_t* P;
  const uint16_t* Q;
  int64_t strideP, strideQ;   // elements between consecutive matrices of the stack
  int ldp, ldq;               // row pitch (elements) of the stored P and Q
  int M, N, K;
  uint16_t* C;
  int64_t strideC;
  int ldc;
  const uint16_t* E;          // epilogue operand: A (poly) or X (apply)
  int64_t strideE;
  int lde;
  float alpha;                // poly: b; apply: a
  float beta;                 // poly: c
  float* trace;               // Gram: per-matrix diagonal partials, or nullptr
  int trace_slots;
  int tiles_m, tiles_n;
  int split;
};

// Fetch one operand slab (R rows x kBK) from global memory into registers, then write it to LDS
// as [row][k] with k contiguous.
template <bool KSTRIDED, int R>
struct SlabLoader;

// K-contiguous operand: element (row, k) at base[row * ld + k].  16-byte chunks of 8 k's.
template <int R>
struct SlabLoader<false, R> {
  static constexpr int kChunksPerRow = kBK / 8;
  static constexpr int kPerThread = R * kChunksPerRow / kThreads;
  u32x4_t reg[kPerThread];

  __device__ __forceinline__ void load(const uint16_t* base, int ld, int row0, int rows, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / kChunksPerRow;
      const int kc = c % kChunksPerRow;
      const int gr = row0 + row;
      const int gk = k0 + kc * 8;
      if (gr < rows && gk < K) {
        reg[r] = *reinterpret_cast<const u32x4_t*>(base + (int64_t)gr * ld + gk);
      } else {
        reg[r] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / kChunksPerRow;
      const int kc = c % kChunksPerRow;
      *reinterpret_cast<u32x4_t*>(lds + row * kLds + kc * 8) = reg[r];
    }
  }
};

// K-strided operand: element (row, k) at base[k * ld + row].  A thread fetches 4 consecutive k
// of 8 consecutive rows (four 16-byte segments) and transposes them in registers.
template <int R>
struct SlabLoader<true, R> {
  static constexpr int kRowChunks = R / 8;
  static constexpr int kBlocks = kRowChunks * (kBK / 4);
  static constexpr int kPerThread = kBlocks / kThreads;
  static_assert(kPerThread * kThreads == kBlocks, "slab must split evenly over the threads");
  u32x4_t reg[kPerThread][4];

  __device__ __forceinline__ void load(const uint16_t* base, int ld, int row0, int rows, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int bidx = tid + kThreads * r;
      const int ic = bidx % kRowChunks;
      const int kq = bidx / kRowChunks;
      const int gr = row0 + ic * 8;
      const int gk = k0 + kq * 4;
      const bool ok = gr < rows && gk < K;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (ok) {
          reg[r][kk] = *reinterpret_cast<const u32x4_t*>(base + (int64_t)(gk + kk) * ld + gr);
        } else {
          reg[r][kk] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int bidx = tid + kThreads * r;
      const int ic = bidx % kRowChunks;
      const int kq = bidx / kRowChunks;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // dword j of each k-row holds rows 2j (low half) and 2j+1 (high half)
        const uint32_t k0w = reg[r][0][j], k1w = reg[r][1][j];
        const uint32_t k2w = reg[r][2][j], k3w = reg[r][3][j];
        u32x2_t even, odd;
        even[0] = (k0w & 0xFFFFu) | (k1w << 16);
        even[1] = (k2w & 0xFFFFu) | (k3w << 16);
        odd[0] = (k0w >> 16) | (k1w & 0xFFFF0000u);
        odd[1] = (k2w >> 16) | (k3w & 0xFFFF0000u);
        *reinterpret_cast<u32x2_t*>(lds + (ic * 8 + 2 * j) * kLds + kq * 4) = even;
        *reinterpret_cast<u32x2_t*>(lds + (ic * 8 + 2 * j + 1) * kLds + kq * 4) = odd;
      }
    }
  }
};

// Upper-triangle tile (ti <= tj) of linear index t, row by row.
__device__ __forceinline__ void upper_tile(int t, int tiles, int* ti, int* tj) {
  int i = 0;
  int len = tiles;
  while (t >= len) {
    t -= len;
    ++i;
    --len;
  }
  *ti = i;
  *tj = i + t;
}

template <int OP, bool PT, bool QT>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sP[2][kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][kBN * kLds];
  __shared__ float sRed[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int64_t b = blockIdx.y;

  int ti, tj;
  if constexpr (OP == OP_APPLY) {
    ti = blockIdx.x / p.tiles_n;
    tj = blockIdx.x % p.tiles_n;
  } else {
    upper_tile(blockIdx.x, p.tiles_m, &ti, &tj);
  }
  const int i0 = ti * kBM;
  const int j0 = tj * kBN;

  const uint16_t* Pb = p.P + b * p.strideP;
  const uint16_t* Qb = p.Q + b * p.strideQ;

  SlabLoader<PT, kBM> lp;
  SlabLoader<QT, kBN> lq;

  f32x16_t acc[2][2];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.0f;

  const int KT = (p.K + kBK - 1) / kBK;
  lp.load(Pb, p.ldp, i0, p.M, 0, p.K, tid);
  lq.load(Qb, p.ldq, j0, p.N, 0, p.K, tid);
  lp.store(sP[0], tid);
  lq.store(sQ[0], tid);
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      lp.load(Pb, p.ldp, i0, p.M, (kt + 1) * kBK, p.K, tid);
      lq.load(Qb, p.ldq, j0, p.N, (kt + 1) * kBK, p.K, tid);
    }
    const uint16_t* cp = sP[cur];
    const uint16_t* cq = sQ[cur];
    // Each slab accumulates into fresh registers and is then added to the running sums with IEEE
    // fp32 adds: the MFMA's own addition into a large running accumulator is measurably less
    // accurate (about twice the drift from an fp64 reference on low-rank-dominated inputs).
    f32x16_t slab[2][2];
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) slab[tm][tn][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
        fa[tm] = *reinterpret_cast<const bf16x8_t*>(
            cp + (wm * 64 + tm * 32 + frag_row) * kLds + ks * 16 + frag_k);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        fb[tn] = *reinterpret_cast<const bf16x8_t*>(
            cq + (wn * 64 + tn * 32 + frag_row) * kLds + ks * 16 + frag_k);
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
          slab[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], slab[tm][tn], 0, 0, 0);
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) acc[tm][tn] += slab[tm][tn];
    if (more) {
      lp.store(sP[cur ^ 1], tid);
      lq.store(sQ[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  uint16_t* Cb = p.C + b * p.strideC;
  const uint16_t* Eb = p.E ? p.E + b * p.strideE : nullptr;
  float tsum = 0.0f;
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // accumulator layout of the 32x32 MFMA: register r of lane l holds
        // row 8*(r/4) + 4*(l/32) + r%4, column l%32
        const int gi = i0 + wm * 64 + tm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int gj = j0 + wn * 64 + tn * 32 + (lane & 31);
        if (gi >= p.M || gj >= p.N) continue;
        const float v = acc[tm][tn][r];
        if constexpr (OP == OP_APPLY) {
          const float ax = p.alpha * bf16_to_f32(Eb[(int64_t)gi * p.lde + gj]);
          uint32_t o;
          if (p.split) {
            o = f32_to_bf16(bf16_to_f32(f32_to_bf16(v)) + ax);
          } else {
            o = f32_to_bf16(ax + v);
          }
          Cb[(int64_t)gi * p.ldc + gj] = static_cast<uint16_t>(o);
        } else {
          if (ti == tj && gi > gj) continue;
          float w = v;
          if constexpr (OP == OP_POLY) {
            const float ba = p.alpha * bf16_to_f32(Eb[(int64_t)gi * p.lde + gj]);
            const float cq = p.beta * v;
            w = ba + cq;
          }
          const uint32_t o = f32_to_bf16(w);
          Cb[(int64_t)gi * p.ldc + gj] = static_cast<uint16_t>(o);
          Cb[(int64_t)gj * p.ldc + gi] = static_cast<uint16_t>(o);
          if constexpr (OP == OP_GRAM) {
            if (gi == gj) tsum += bf16_to_f32(o);
          }
        }
      }
    }
  }

  if constexpr (OP == OP_GRAM) {
    if (p.trace != nullptr && ti == tj) {
      // fixed-order reduction: butterfly within each wave, then waves 0..3 in order
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) tsum += __shfl_xor(tsum, off, 64);
      if (lane == 0) sRed[wave] = tsum;
      __syncthreads();
      if (tid == 0) {
        float t = 0.0f;
        for (int w = 0; w < kThreads / 64; ++w) t += sRed[w];
        p.trace[b * p.trace_slots + ti] = t;
      }
    }
  }
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int OP, bool PT, bool QT>
hipError_t launch(const GemmParams& p, int64_t g, int tiles, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_kernel<OP, PT, QT>), dim3((unsigned)tiles, (unsigned)g), dim3(kThreads),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace

int gram_trace_slots(int s) { return ceil_div(s, kBM); }

hipError_t launch_gram(const uint16_t* x, uint16_t* a, float* trace_partials, const Shape& sh,
                       hipStream_t stream) {
  const int s = sh.s();
  GemmParams p{};
  p.P = x;
  p.Q = x;
  p.strideP = p.strideQ = (int64_t)sh.m * sh.n;
  p.ldp = p.ldq = sh.n;
  p.M = p.N = s;
  p.K = sh.L();
  p.C = a;
  p.strideC = (int64_t)s * s;
  p.ldc = s;
  p.trace = trace_partials;
  p.trace_slots = gram_trace_slots(s);
  p.tiles_m = p.tiles_n = ceil_div(s, kBM);
  const int tiles = p.tiles_m * (p.tiles_m + 1) / 2;
  if (sh.tall()) return launch<OP_GRAM, true, true>(p, sh.g, tiles, stream);
  return launch<OP_GRAM, false, false>(p, sh.g, tiles, stream);
}

hipError_t launch_poly(const uint16_t* a, uint16_t* bout, float coef_b, float coef_c, int64_t g,
                       int s, hipStream_t stream) {
  GemmParams p{};
  p.P = a;
  p.Q = a;
  p.strideP = p.strideQ = (int64_t)s * s;
  p.ldp = p.ldq = s;
  p.M = p.N = p.K = s;
  p.C = bout;
  p.strideC = (int64_t)s * s;
  p.ldc = s;
  p.E = a;
  p.strideE = (int64_t)s * s;
  p.lde = s;
  p.alpha = coef_b;
  p.beta = coef_c;
  p.tiles_m = p.tiles_n = ceil_div(s, kBM);
  const int tiles = p.tiles_m * (p.tiles_m + 1) / 2;
  return launch<OP_POLY, false, false>(p, g, tiles, stream);
}

hipError_t launch_apply(const uint16_t* x, const uint16_t* bm, uint16_t* c, float coef_a,
                        bool split, const Shape& sh, hipStream_t stream) {
  const int s = sh.s();
  GemmParams p{};
  p.M = sh.m;
  p.N = sh.n;
  p.C = c;
  p.strideC = (int64_t)sh.m * sh.n;
  p.ldc = sh.n;
  p.E = x;
  p.strideE = (int64_t)sh.m * sh.n;
  p.lde = sh.n;
  p.alpha = coef_a;
  p.split = split ? 1 : 0;
  p.tiles_m = ceil_div(sh.m, kBM);
  p.tiles_n = ceil_div(sh.n, kBN);
  const int tiles = p.tiles_m * p.tiles_n;
  if (sh.tall()) {
    // C = a X + X B: P = X rows (K = n contiguous), Q = rows of symmetric B
    p.P = x;
    p.strideP = (int64_t)sh.m * sh.n;
    p.ldp = sh.n;
    p.Q = bm;
    p.strideQ = (int64_t)s * s;
    p.ldq = s;
    p.K = sh.n;
    return launch<OP_APPLY, false, false>(p, sh.g, tiles, stream);
  }
  // C = a X + B X: P = rows of B (K = m contiguous), Q(j, k) = X[k][j] (K-strided)
  p.P = bm;
  p.strideP = (int64_t)s * s;
  p.ldp = s;
  p.Q = x;
  p.strideQ = (int64_t)sh.m * sh.n;
  p.ldq = sh.n;
  p.K = sh.m;
  return launch<OP_APPLY, false, true>(p, sh.g, tiles, stream);
}

}  // namespace anvil
