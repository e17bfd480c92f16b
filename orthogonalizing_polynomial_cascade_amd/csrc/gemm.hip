// Kernels 2-4: the Gram, polynomial and apply products of the ANVIL cascade on bf16 MFMA.
//
// Source: modded-nanogpt anvil.py, `anvil_cascade` (tall and wide branches).  Every product in the
// cascade is one of three batched contractions over a stack of matrices, all written here as
//
//     C[i][j] = sum_k P(i, k) * Q(j, k)          (fp32 accumulation on v_mfma_f32_32x32x16_bf16)
//
// with a fused fp32 epilogue and a single bf16 rounding at the page's storage points:
//
//   Gram   A = X^T X (tall: P = Q = X read down its columns, "K-major")
//          A = X X^T (wide: P = Q = X read along its rows, "K-contiguous")
//          epilogue bf16(acc); optional trace partials of the bf16 diagonal.
//   poly   B = b A + c A A   (A symmetric, so A A = A A^T: P = Q = A, K-contiguous)
//          epilogue bf16(b * A[i][j] + c * acc).
//   apply  tall: C = a X + X B   (P = X; Q(j, k) = B[k][j], K-major: B is symmetric, and its
//                                 rows k give whole row pieces where B[j][k] gives half lines)
//          wide: C = a X + B X   (P = B, Q(j, k) = X[k][j]: K-major)
//          epilogue bf16(a * X[i][j] + acc), or with split rounding
//          bf16(bf16(acc) + a * X[i][j]) (the page's two-kernel form for banks of > 1024 rows).
//
// No epilogue reads its operand from memory: the polynomial's A[i][j] and the tall apply's
// X[i][j] are their P operand at k = j, the wide apply's X[i][j] its Q operand at k = i, and each
// wave keeps the MFMA fragments that hold them for its block as the k loop passes them.
//
// The Gram and the polynomial are symmetric: only tiles on or above the diagonal are computed,
// and each is stored twice (C[i][j] and C[j][i]) from the same fp32 value, so the stored matrices
// are exactly symmetric.  Inside a diagonal tile every entry is still stored once, in 16-byte
// pieces of 8 columns: pieces on or above the diagonal and the 8x8 blocks the diagonal crosses
// directly (an entry below the diagonal in such a block takes the value of its mirrored
// position), pieces wholly below it by the mirror.  A diagonal tile has the same rows in both
// operands: it copies them once, and its waves whose block lies wholly below the diagonal skip
// their multiplies.
//
// For stacks of small wide matrices (s <= 256) whose tiles fit one round on the CUs,
// poly_apply_kernel runs a map's polynomial and apply as one launch, each workgroup forming the
// rows of B its tile needs (same bits as the two kernels).
//
// Pipeline (CDNA4 / gfx950):
//  * Operand slabs (rows x BK k, BK = 32, 64 or 128) travel HBM -> LDS with
//    buffer_load_dwordx4 ... lds (16 bytes per lane straight into LDS, no register staging)
//    through a ring of STAGES LDS buffers; the loads for slab k+STAGES-1 are in flight while
//    slab k feeds the MFMAs.  Lanes outside the matrix (ragged M, N or K edges) get an offset
//    past the buffer's range, which loads zeros.
//  * K-contiguous slabs are stored [row][BK k] with 16-byte slots XOR-swizzled by row, so that
//    an MFMA operand (32 rows x 8 k) is one ds_read_b128 per lane without bank conflicts.
//  * K-major slabs (X read down its columns, B by its rows k) are stored [BK k][rows] as they
//    arrive, slots swizzled by k; an MFMA operand is two ds_read_b64_tr_b16, the LDS transpose
//    read: within a 16-lane group, lanes 4j..4j+3 point at 16 consecutive rows of k-row j and
//    lane r receives the 4 k-values of row r.  No VALU transposes.
//  * Each wave owns a (BM/WM) x (BN/WN) block of 32x32 MFMA fragments.  In the Gram, each group
//    of 512 k (256 k for s <= 256) is accumulated into fresh registers and then added to the
//    running sums with IEEE fp32 adds (one MFMA accumulation chain over thousands of k drifts
//    from an fp64 reference noticeably more than sgemm on low-rank-dominated inputs); small
//    Grams may give the groups of a tile to separate sets of waves and add their sums in group
//    order, which is the same arithmetic.  The polynomial and the apply (K = the short side)
//    accumulate directly.
//  * Tiles are ordered so that consecutive tiles of one matrix land on the same XCD (hardware
//    dispatches workgroups round-robin over the 8 XCDs, each with its own L2); a Gram launch of
//    one to two rounds puts its diagonal tiles on the CUs that hold two workgroups.
//  * The epilogue goes through LDS, 32 rows at a time per wave: rows leave as 16-byte stores, and
//    the mirror of a symmetric tile is read down the LDS columns and leaves as 16-byte stores,
//    four lanes per mirrored row.
//
// Shapes: M, N, K are multiples of 8 (16-byte rows).
#include <algorithm>
#include <atomic>
#include <cstdint>

#include "device_common.h"
#include "launchers.h"

// m0 is written by the DMA inline assembly; the kernel has no other use of it (no indirect
// register indexing), which is what the compiler's reserved-register warning is about.
#pragma clang diagnostic ignored "-Winline-asm"

namespace anvil {

namespace {

// OP_APPLY: the wide apply (C = a X + B X), whose epilogue operand X[i][j] is its Q operand at
// k = i.  OP_APPLY_XT: the tall apply (C = a X + X B), whose epilogue operand is its P operand at
// k = j.  Both keep it from the k loop (see gemm_kernel).
enum { OP_GRAM = 0, OP_POLY = 1, OP_APPLY = 2, OP_APPLY_XT = 3 };


constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past any range: the load returns 0
constexpr int kCus = 256;                // compute units of the MI355X (8 XCDs of 32)
constexpr int kFullRound = 512;          // two workgroups per CU

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

struct GemmParams {
  const uint16_t* P;
  const uint16_t* Q;
  int64_t strideP, strideQ;   // elements between consecutive matrices of the stack
  int ldp, ldq;               // row pitch (elements) of the stored P and Q
  uint32_t bytesP, bytesQ;    // bytes of one matrix of P and of Q (buffer range)
  int M, N, K;
  uint16_t* C;
  int64_t strideC;
  int ldc;
  float alpha;                // poly: b; apply: a
  float beta;                 // poly: c
  float* trace;               // Gram: per-matrix diagonal partials, or nullptr
  int trace_slots;
  int tiles_m, tiles_n;       // tile grid of one matrix
  int tiles;                  // tiles per matrix (upper triangle for Gram and poly)
  int total;                  // tiles * g
  int split;
  int pair_diagonals;         // symmetric product of one to two rounds: see diagonal_first
};

// ---------------------------------------------------------------------------------------------
// LDS slab layouts
// ---------------------------------------------------------------------------------------------

// [ROWS][BK] bf16: a row is BK*2 bytes = BK/8 slots of 16 bytes (8 k each), and 256 bytes of LDS
// (one pass over the 64 banks) hold 16/(BK/8) rows, or one row spans BK/128 such passes.
// Logical slot c of row r sits at slot c ^ ((r / rows_per_256B) % min(slots, 16)): 16
// consecutive rows read at one logical slot hit 16 distinct 16-byte bank groups.
template <int ROWS, int BK>
struct KContig {
  static constexpr int kSlots = BK / 8;
  static constexpr int kRowsPer256 = kSlots >= 16 ? 1 : 16 / kSlots;
  static constexpr int kSwizzle = kSlots >= 16 ? 16 : kSlots;
  __device__ static __forceinline__ int swz(int row) { return (row / kRowsPer256) % kSwizzle; }
  __device__ static __forceinline__ int offset(int row, int c) {
    return row * (BK * 2) + ((c ^ swz(row)) << 4);
  }
};

// [BK][ROWS] bf16: a k-row is ROWS*2 bytes = ROWS/8 slots.  Logical slot c of k-row kr sits at
// slot c ^ (4 * (kr & 3)).
template <int ROWS>
struct KMajor {
  static_assert(ROWS >= 128, "K-major slabs need at least 16 slots per k-row");
  __device__ static __forceinline__ int offset(int kr, int c) {
    return kr * (ROWS * 2) + ((c ^ ((kr & 3) << 2)) << 4);
  }
};

// Raw buffer resource (stride 0, flags word of the gfx9 family) over `bytes` bytes at `base`.
// All four words are wave-uniform and live in SGPRs.
__device__ __forceinline__ i32x4_t make_rsrc(const uint16_t* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}

// 32-bit LDS address of a pointer into dynamic shared memory (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const char* ptr) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_ptr)(ptr))));
}

// One wave-instruction of DMA: lane L's 16 bytes at `voff` of the buffer land in LDS at
// lds + 16*L.  Issued as inline assembly so that the compiler neither reorders it nor inserts its
// own (conservative) waits on it; completion is tracked with wait_vmcnt below.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// The DMA of one operand's slabs (rows row0.., k0..k0+BK-1) into LDS.  A slab is ROWS*BK/512
// wave-instructions of 1 KB; instruction u lands at dst + u*1024, lane L's 16 bytes at
// dst + u*1024 + 16*L, and this wave issues instructions u = wave, wave + NW, ...  The per-lane
// source offsets of k0 = 0 are computed once per tile; a slab then costs one add per instruction
// (all destination arithmetic is scalar).  Lanes past the matrix edge get an offset past the
// buffer's range, which loads zeros.
template <bool KMAJOR, int ROWS, int BK, int NW>
struct SlabCopy {
  static constexpr int kInsts = ROWS * BK / 512 / NW;
  static_assert(ROWS * BK / 512 % NW == 0, "slab instructions must split evenly over the waves");
  // K-major: a wave's instructions i = 0, 1, .. cover k-rows kStepRows apart; when that keeps the
  // slot swizzle (k-row & 3), every instruction reads the same columns, so its offset is the
  // first one's plus i * kStepRows rows (past-the-edge lanes stay past the range), one register.
  static constexpr int kStepRows = KMAJOR ? NW * (512 / ROWS) : 0;
  static constexpr bool kOneBase = KMAJOR && kStepRows % 4 == 0;
  uint32_t vbase[kOneBase ? 1 : kInsts];   // byte offset at k0 = 0, or kOOB past the edge
  uint32_t kbytes;                         // bytes per unit of k0

  // Row (K-contiguous: row of the slab; K-major: k-row) and 16-byte slot of lane `lane`'s piece
  // in instruction i.
  __device__ static __forceinline__ void piece(int i, int wave, int lane, int* row, int* c) {
    const int u = wave + i * NW;
    if constexpr (!KMAJOR) {
      constexpr int kSlots = BK / 8;
      constexpr int kRowsPerInst = 64 / kSlots;
      *row = kRowsPerInst * u + lane / kSlots;
      *c = (lane % kSlots) ^ KContig<ROWS, BK>::swz(*row);
    } else {
      constexpr int kSlots = ROWS / 8;
      constexpr int kRowsPerKb = 64 / kSlots;
      *row = u * kRowsPerKb + lane / kSlots;
      *c = (lane % kSlots) ^ ((*row & 3) << 2);
    }
  }

  SlabCopy() = default;
  __device__ __forceinline__ SlabCopy(int ld, int row0, int rows, int wave, int lane) {
    kbytes = KMAJOR ? 2u * (uint32_t)ld : 2u;
#pragma unroll
    for (int i = 0; i < (kOneBase ? 1 : kInsts); ++i) {
      int row, c;
      piece(i, wave, lane, &row, &c);
      if constexpr (!KMAJOR) {
        const int gr = row0 + row;
        vbase[i] = gr < rows ? (uint32_t)(gr * ld + c * 8) * 2u : kOOB;
      } else {
        const int gr = row0 + c * 8;
        vbase[i] = gr < rows ? (uint32_t)(row * ld + gr) * 2u : kOOB;
      }
    }
  }

  // Issue this wave's instructions of the slab at k0 into LDS at byte address `dst` (uniform).
  // The lane's k offset inside a ragged last slab is recomputed there (not kept in registers).
  __device__ __forceinline__ void issue(i32x4_t rsrc, uint32_t dst, int k0, int K, int wave) const {
    const uint32_t koff = (uint32_t)k0 * kbytes;
    auto base = [&](int i) {
      return kOneBase ? vbase[0] + (uint32_t)(i * kStepRows) * kbytes : vbase[kOneBase ? 0 : i];
    };
    if (k0 + BK <= K) {
#pragma unroll
      for (int i = 0; i < kInsts; ++i)
        dma16(rsrc, dst + (uint32_t)(wave + i * NW) * 1024u, base(i) + koff);
    } else {
      const int lane = __lane_id();
#pragma unroll
      for (int i = 0; i < kInsts; ++i) {
        int row, c;
        piece(i, wave, lane, &row, &c);
        const int kin = KMAJOR ? row : c * 8;
        dma16(rsrc, dst + (uint32_t)(wave + i * NW) * 1024u,
              k0 + kin < K ? base(i) + koff : kOOB);
      }
    }
  }
};

// MFMA operand of a 32-row fragment (rows R0..R0+31) at k-step ks (k = 16ks .. 16ks+15):
// lane l holds row R0 + l%32, k = 16ks + 8(l/32) + 0..7.
template <bool KMAJOR, int ROWS, int BK>
__device__ __forceinline__ bf16x8_t read_frag(const char* tile, int R0, int ks, int lane) {
  if constexpr (!KMAJOR) {
    const int row = R0 + (lane & 31);
    const int c = 2 * ks + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(tile + KContig<ROWS, BK>::offset(row, c));
  } else {
    const int grp = lane >> 4;
    const int r = lane & 15;
    const int i = R0 + 16 * (grp & 1) + 4 * (r & 3);
    const int kr = 16 * ks + 8 * (grp >> 1) + (r >> 2);
    const int c = i >> 3;
    const int half = ((i >> 2) & 1) * 8;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_ptr)(tile + KMajor<ROWS>::offset(kr, c) + half));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_ptr)(tile + KMajor<ROWS>::offset(kr + 4, c) + half));
    const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Wait for this wave's LDS operations (lgkmcnt(0)).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup id -> logical tile id such that each XCD gets a contiguous run of logical ids.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd;
  const int r = total % kXcd;
  const int x = id % kXcd;
  const int local = id / kXcd;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

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

// Diagonal tiles of an upper-triangle tile grid (tiles_m tiles per side, tiles_m(tiles_m+1)/2 per
// matrix, row by row): the diagonal tile of row i sits at t = i*tiles_m - i(i-1)/2.
__device__ __forceinline__ int diag_pos(int i, int tiles_m) {
  return i * tiles_m - i * (i - 1) / 2;
}

// Number of diagonal tiles with logical id below L (matrices one after the other).
__device__ __forceinline__ int diagonals_before(int L, int tiles, int tiles_m) {
  const int t = L % tiles;
  int i = 0;
  while (i < tiles_m && diag_pos(i, tiles_m) < t) ++i;
  return (L / tiles) * tiles_m + i;
}

// Gram launches with one to two rounds of workgroups: the first round puts one workgroup on every
// CU of an XCD (32 per XCD) and each later workgroup of the XCD shares a CU with one of the first
// (observed: workgroup 32+k of an XCD joins the CU of workgroup k).  A CU holding two workgroups
// sets the launch's time, so those slots take the XCD's cheaper diagonal tiles (one operand copy,
// a wave fewer multiplying) first: workgroup `local` of an XCD whose logical range is
// [start, start + count) gets the rank-th tile of the range in diagonal-first order, where the
// shared slots (0..p-1 and 32..count-1, p = count - 32) come first.  The result is a permutation
// of the range; which tile a workgroup takes changes no arithmetic.
__device__ __forceinline__ int diagonal_first(int start, int count, int local, int tiles,
                                              int tiles_m) {
  constexpr int kCusPerXcd = 32;
  const int p = count > kCusPerXcd ? count - kCusPerXcd : 0;
  const int rank = local < p ? local
                   : local >= kCusPerXcd ? p + (local - kCusPerXcd)
                                         : 2 * p + (local - p);
  const int d0 = diagonals_before(start, tiles, tiles_m);
  const int nd = diagonals_before(start + count, tiles, tiles_m) - d0;
  if (rank < nd) {
    const int gd = d0 + rank;
    return (gd / tiles_m) * tiles + diag_pos(gd % tiles_m, tiles_m);
  }
  const int offs = tiles - tiles_m;   // off-diagonal tiles per matrix (> 0 here)
  const int go = (start - d0) + (rank - nd);
  int k = go % offs;
  int i = 0;
  while (k >= tiles_m - 1 - i) {
    k -= tiles_m - 1 - i;
    ++i;
  }
  return (go / offs) * tiles + diag_pos(i, tiles_m) + 1 + k;
}

template <int BM, int BN, int WM, int WN, int STAGES, int BK>
struct Cfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kWTM = BM / WM;   // wave tile rows
  static constexpr int kWTN = BN / WN;   // wave tile cols
  static constexpr int kFM = kWTM / 32;
  static constexpr int kFN = kWTN / 32;
  static constexpr int kStageBytes = (BM + BN) * BK * 2;
  static constexpr int kQOffset = BM * BK * 2;
  static constexpr int kEpiPitch = kWTN + 4;                  // fp32 per LDS epilogue row
  static constexpr int kEpiBytes = kWaves * 32 * kEpiPitch * 4;
  static constexpr int kLdsBytes =
      (STAGES * kStageBytes > kEpiBytes ? STAGES * kStageBytes : kEpiBytes);
  static_assert(kWTN % 8 == 0 && 64 % (kWTN / 8) == 0, "epilogue moves 8 columns per lane");
  static constexpr int kLoadsPerSlab = (BM + BN) * BK / 512 / kWaves;
  static_assert(BK == 32 || BK == 64 || BK == 128, "slab depth");
  static_assert(kWTM % 32 == 0 && kWTN % 32 == 0, "wave tile must be whole 32x32 fragments");
  static_assert(STAGES >= 2, "at least double buffering");
  static_assert(kLoadsPerSlab * (STAGES - 2) < 64, "vmcnt range");
};

// The four-wave Gram tiles run two workgroups per CU, two waves per SIMD: they may take up to 256
// registers per lane, which their read-ahead of a whole slab's fragments needs.
// The eight-wave applies and polynomial keep four waves per SIMD (two workgroups per CU) with
// their kept operand fragments: at most 128 registers.
template <int OP, int WAVES, int KSPLIT>
constexpr int kMinWavesPerEu = OP == OP_GRAM && WAVES == 4 && KSPLIT == 1 ? 2
                               : OP != OP_GRAM && WAVES == 8         ? 4
                                                                      : 1;

// KSPLIT > 1 (Gram tiles with slab groups only): the tile's KSPLIT slab groups go to KSPLIT sets
// of WM x WN waves, each set with its own ring, which accumulate one group each from zero; the
// group sums are then added to the first set's in group order, which is exactly the unsplit
// kernel's running sum (0 + G0 = G0, then + G1, + G2, ...), and the first set runs the epilogue.
// With several waves per set every wave runs SLAB iterations (skipping slabs past its k range),
// so that all waves meet every barrier; such a tile writes one trace partial per 32-row diagonal
// wave block, the partials of 32x32 tiles.
template <int OP, bool PT, bool QT, int BM, int BN, int WM, int WN, int STAGES, int BK, int SLAB,
          int KSPLIT = 1>
__global__ __launch_bounds__(WM * WN * KSPLIT * 64)
__attribute__((amdgpu_waves_per_eu(kMinWavesPerEu<OP, WM * WN, KSPLIT>)))
void gemm_kernel(GemmParams p) {
  using C = Cfg<BM, BN, WM, WN, STAGES, BK>;
  constexpr bool kApply = OP == OP_APPLY || OP == OP_APPLY_XT;
  static_assert(KSPLIT == 1 || (OP == OP_GRAM && SLAB > 0 && STAGES == 2),
                "k groups over waves: Gram tiles with slab groups and two stages");
  static_assert(KSPLIT == 1 || C::kWaves == 1 || (WM == WN && C::kWTM == 32 && C::kWTN == 32),
                "a split tile of several waves has 32x32 wave blocks on its diagonal");
  extern __shared__ __attribute__((aligned(1024))) char smem_all[];
  __shared__ float sRed[C::kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = KSPLIT > 1 ? wave_all / C::kWaves : 0;                     // k group
  const bool computes = kg == 0;                                           // runs the epilogue
  char* smem = smem_all + kg * C::kLdsBytes;                               // this group's ring
  const int wave = KSPLIT > 1 ? wave_all % C::kWaves : wave_all;
  const int wm = wave / WN;
  const int wn = wave % WN;

  int logical = xcd_remap(blockIdx.x, p.total);
  if (OP == OP_GRAM && p.pair_diagonals) {
    constexpr int kXcd = 8;
    const int x = blockIdx.x % kXcd;
    const int q = p.total / kXcd, r = p.total % kXcd;
    const int start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    logical = diagonal_first(start, q + (x < r ? 1 : 0), blockIdx.x / kXcd, p.tiles, p.tiles_m);
  }
  const int64_t b = logical / p.tiles;
  const int t = logical % p.tiles;
  int ti, tj;
  if constexpr (kApply) {
    ti = t / p.tiles_n;
    tj = t % p.tiles_n;
  } else {
    upper_tile(t, p.tiles_m, &ti, &tj);
  }
  const int i0 = ti * BM;
  const int j0 = tj * BN;

  const i32x4_t rP = make_rsrc(p.P + b * p.strideP, p.bytesP);
  const i32x4_t rQ = make_rsrc(p.Q + b * p.strideQ, p.bytesQ);
  const SlabCopy<PT, BM, BK, C::kWaves> copyP(p.ldp, i0, p.M, wave, lane);
  const SlabCopy<QT, BN, BK, C::kWaves> copyQ(p.ldq, j0, p.N, wave, lane);
  const uint32_t smem_lds = lds_addr(smem);
  // A diagonal tile of a symmetric product has the same rows in both operands: it copies them once
  // and reads both operands' fragments from that slab (with two stages every slab iteration waits
  // for all of this wave's copies, so the copy count does not enter the waits).
  const bool same_pq = STAGES == 2 && PT == QT && BM == BN && !kApply && ti == tj;

  f32x16_t acc[C::kFM][C::kFN];
#pragma unroll
  for (int fm = 0; fm < C::kFM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::kFN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;

  const int KT_all = (p.K + BK - 1) / BK;
  const int kt0 = KSPLIT > 1 ? kg * SLAB : 0;                        // this wave's slabs
  const int KT = KSPLIT > 1 ? min(KT_all, kt0 + SLAB) : KT_all;

  // prologue: slabs kt0 .. kt0+STAGES-2 in flight (stage of slab kt: (kt - kt0) % STAGES)
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    if (kt0 + s < KT) {
      const uint32_t st = smem_lds + (uint32_t)(s * C::kStageBytes);
      copyP.issue(rP, st, (kt0 + s) * BK, p.K, wave);
      if (!same_pq) copyQ.issue(rQ, st + (uint32_t)C::kQOffset, (kt0 + s) * BK, p.K, wave);
    }
  }

  // Epilogue operand (X for the apply, A for the polynomial).  Tall apply and polynomial: the
  // operand (X[i][j], A[i][j]) of this wave's block is its P operand at k = j, and it passes
  // through the wave's registers as MFMA fragments while the k loop crosses the wave's columns
  // (k-steps xs0 .. xs0 + kXsKs - 1).  The wide apply (C = a X + B X) finds X[i][j] in its Q
  // operand at k = i, over the k-steps of the wave's rows, transposed (lane l: column j = l%32 of
  // a 32-column fragment, rows 8(l/32) .. +7 of the k-step).  Those fragments are kept (32
  // registers for a 64x64 wave block), and the epilogue takes the operand from them instead of
  // reading it again from memory (for the apply X has left L2 by then: one mlp apply re-read
  // ~90 MB of it from HBM).
  constexpr int kLanesPerRow = C::kWTN / 8;     // epilogue passes: 8 consecutive columns a lane
  constexpr int kRowsPerPass = 64 / kLanesPerRow;
  constexpr int kPasses = 32 / kRowsPerPass;
  constexpr bool kKeep = OP != OP_GRAM;
  constexpr bool kXsQ = OP == OP_APPLY;
  constexpr int kXsKs = kXsQ ? C::kWTM / 16 : C::kWTN / 16;   // k-steps kept
  constexpr int kXsF = kXsQ ? C::kFN : C::kFM;                 // fragments kept per k-step
  const int xs0 = kXsQ ? (i0 + wm * C::kWTM) / 16 : (j0 + wn * C::kWTN) / 16;
  bf16x8_t xs[kKeep ? kXsKs : 1][kKeep ? kXsF : 1];
  if constexpr (kKeep) {
#pragma unroll
    for (int q = 0; q < kXsKs; ++q)
#pragma unroll
      for (int f = 0; f < kXsF; ++f) xs[q][f] = bf16x8_t{};
  }

  // On a diagonal tile of a symmetric product, a wave whose block lies wholly below the diagonal
  // stores nothing (those entries come from the mirror of the block above it): it takes its share
  // of the copies and every barrier, but skips its fragment reads and multiplies.
  const bool idle = !kApply && ti == tj && wm * C::kWTM >= (wn + 1) * C::kWTN;

  f32x16_t slab[SLAB > 0 ? C::kFM : 1][SLAB > 0 ? C::kFN : 1];
  constexpr bool kPadded = KSPLIT > 1 && C::kWaves > 1;   // uniform trip count: shared barriers
  const int kt_last = kPadded ? kt0 + SLAB : KT;
  for (int kt = kt0; kt < kt_last; ++kt) {
    // slab kt has landed once at most STAGES-2 younger slabs of this wave are still in flight
    if (KT - 1 - kt >= STAGES - 2) {
      wait_vmcnt<C::kLoadsPerSlab * (STAGES - 2)>();
    } else {
      wait_vmcnt<0>();
    }
    // every wave's part of slab kt is in LDS; slab kt-1's buffer is free (a wave of a split tile
    // reads only the slabs it copied itself)
    if constexpr (KSPLIT == 1 || C::kWaves > 1) {
      __syncthreads();
    } else {
      __builtin_amdgcn_wave_barrier();
    }
    {
      const int kn = kt + STAGES - 1;
      if (kn < KT) {
        const uint32_t st = smem_lds + (uint32_t)(((kn - kt0) % STAGES) * C::kStageBytes);
        copyP.issue(rP, st, kn * BK, p.K, wave);
        if (!same_pq) copyQ.issue(rQ, st + (uint32_t)C::kQOffset, kn * BK, p.K, wave);
      }
    }
    if (kPadded && kt >= KT) continue;
    if (idle) continue;
    const char* tp = smem + ((kt - kt0) % STAGES) * C::kStageBytes;
    const char* tq = same_pq ? tp : tp + C::kQOffset;

    // SLAB > 0: groups of SLAB consecutive slabs accumulate into fresh registers, which are then
    // added to the running sums (IEEE fp32 adds); SLAB == 0: the MFMAs accumulate into the
    // running sums directly.
    const bool group_start = SLAB > 0 && kt % (SLAB > 0 ? SLAB : 1) == 0;
    const bool group_end = SLAB > 0 && (kt % (SLAB > 0 ? SLAB : 1) == (SLAB > 0 ? SLAB : 1) - 1 ||
                                        kt == KT - 1);
    if constexpr (SLAB > 0) {
      if (group_start) {
#pragma unroll
        for (int fm = 0; fm < C::kFM; ++fm)
#pragma unroll
          for (int fn = 0; fn < C::kFN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) slab[fm][fn][r] = 0.0f;
      }
    }
    // Fragments of the whole slab are read before its multiplies when a wave holds at most two
    // fragments (its MFMAs then form one or two dependent chains, and reading per k-step would
    // put an LDS round trip in front of every MFMA), and in the Gram, whose four waves per
    // workgroup leave room for them (mlp Gram 63.5 -> 60.5 us).  The apply's and polynomial's
    // larger wave tiles read per k-step, which keeps their registers within four waves per SIMD
    // (reading ahead there made the 128x256 apply 140 registers and the mlp step 25% slower).
    constexpr bool kHoist = C::kFM * C::kFN <= 2 || OP == OP_GRAM;
    constexpr int kKs = BK / 16;
    bf16x8_t fa[kKs][C::kFM], fb[kKs][C::kFN];
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      if (ks == 0 || !kHoist) {
#pragma unroll
        for (int kr = ks; kr < (kHoist ? kKs : ks + 1); ++kr) {
#pragma unroll
          for (int fm = 0; fm < C::kFM; ++fm)
            fa[kr][fm] = read_frag<PT, BM, BK>(tp, wm * C::kWTM + fm * 32, kr, lane);
#pragma unroll
          for (int fn = 0; fn < C::kFN; ++fn)
            fb[kr][fn] = read_frag<QT, BN, BK>(tq, wn * C::kWTN + fn * 32, kr, lane);
        }
        // keep the reads ahead of the multiplies (the scheduler would sink each to its use)
        if constexpr (kHoist) __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kKeep) {
        const int aks = kt * kKs + ks;
#pragma unroll
        for (int q = 0; q < kXsKs; ++q)
          if (aks == xs0 + q) {
            // a real branch (taken on a few slabs): keeps the copies out of the other slabs
            asm volatile("" ::: "memory");
#pragma unroll
            for (int f = 0; f < kXsF; ++f) {
              if constexpr (kXsQ) {
                xs[q][f] = fb[ks][f];
              } else {
                xs[q][f] = fa[ks][f];
              }
            }
          }
      }
#pragma unroll
      for (int fm = 0; fm < C::kFM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::kFN; ++fn) {
          if constexpr (SLAB > 0) {
            slab[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][fn], fa[ks][fm],
                                                                   slab[fm][fn], 0, 0, 0);
          } else {
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][fn], fa[ks][fm],
                                                                  acc[fm][fn], 0, 0, 0);
          }
        }
    }
    if constexpr (SLAB > 0) {
      if (group_end) {
#pragma unroll
        for (int fm = 0; fm < C::kFM; ++fm)
#pragma unroll
          for (int fn = 0; fn < C::kFN; ++fn) acc[fm][fn] += slab[fm][fn];
      }
    }
  }
  __syncthreads();   // every wave is done with the operand ring; reuse it for the epilogue
  if constexpr (KSPLIT > 1) {
    // group sums of the later sets (in their own ring space, per wave and lane) added to the
    // first set's in group order
    constexpr int kFrags = C::kFM * C::kFN;
    static_assert(C::kWaves * kFrags * 16 * 64 * 4 <= C::kLdsBytes, "group sums fit the ring");
    if (!computes) {
      float* red = reinterpret_cast<float*>(smem) + (wave * 64 + lane) * kFrags * 16;
#pragma unroll
      for (int fm = 0; fm < C::kFM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::kFN; ++fn)
#pragma unroll
          for (int r = 0; r < 16; r += 4)
            *reinterpret_cast<f32x4_t*>(red + (fm * C::kFN + fn) * 16 + r) =
                f32x4_t{acc[fm][fn][r], acc[fm][fn][r + 1], acc[fm][fn][r + 2], acc[fm][fn][r + 3]};
    }
    __syncthreads();
    if (computes) {
#pragma unroll
      for (int w = 1; w < KSPLIT; ++w) {
        const float* red = reinterpret_cast<const float*>(smem_all + w * C::kLdsBytes) +
                           (wave * 64 + lane) * kFrags * 16;
#pragma unroll
        for (int fm = 0; fm < C::kFM; ++fm)
#pragma unroll
          for (int fn = 0; fn < C::kFN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
              const f32x4_t v =
                  *reinterpret_cast<const f32x4_t*>(red + (fm * C::kFN + fn) * 16 + r);
              acc[fm][fn][r] += v[0];
              acc[fm][fn][r + 1] += v[1];
              acc[fm][fn][r + 2] += v[2];
              acc[fm][fn][r + 3] += v[3];
            }
      }
    }
  }

  // ---------------- epilogue: per wave, 32 rows at a time through LDS ----------------
  // With the MFMA operands as (Q, P) the fragment holds C transposed: register r of lane l is
  // C[i][j] with i = l%32 and j = 8(r/4) + 4(l/32) + r%4, i.e. runs of 4 consecutive columns of
  // one row, which go to LDS as one 16-byte write.  The rows then leave LDS 8 columns per lane
  // and go to memory as coalesced 16-byte stores; the mirror of a symmetric tile is read down the
  // LDS columns and leaves as 16-byte stores too, four lanes covering 64 contiguous bytes of a
  // mirrored row (16 rows per store instruction).  Rows 16..31 of the block are stored with their
  // columns XOR 16: with the 68-word row pitch, the four 8-row groups read by one mirror
  // instruction (16 columns each) then cover 64 distinct banks of 64, or every bank of 32 twice.
  float* epi = reinterpret_cast<float*>(smem) + wave * 32 * C::kEpiPitch;
  auto ep = [&](int row, int col) {
    return epi + row * C::kEpiPitch + (col ^ (row & 16));
  };
  uint16_t* Cb = p.C + b * p.strideC;
  const bool diag_tile = !kApply && ti == tj;
  float tsum = 0.0f;

#pragma unroll
  for (int fm = 0; fm < C::kFM; ++fm) {
    if (!computes) break;
    // The kept operand of this block in the accumulators' layout: lane l needs entries
    // (row l%32, columns 8q' + 4(l/32) + 0..3) of every 32-column fragment fn, as two dwords
    // xw[fn][q'].
    u32x2_t xw[kKeep ? C::kFN : 1][4];
    if constexpr (kKeep && !kXsQ) {
      // P fragments: lane l holds row l%32 at k = 16q + 8(l/32) + 0..7 of k-step q.  Swapping
      // dwords 2, 3 of the lower 32 lanes with dwords 0, 1 of the upper 32 leaves every lane
      // with its own columns: dwords 0, 1 of k-step 2fn + q'/2 for even q', dwords 2, 3 for odd.
#pragma unroll
      for (int q = 0; q < kXsKs; ++q) {
        const u32x4_t w = __builtin_bit_cast(u32x4_t, xs[q][fm]);
        const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
        xw[q / 2][2 * (q % 2)] = u32x2_t{s02[0], s13[0]};
        xw[q / 2][2 * (q % 2) + 1] = u32x2_t{s02[1], s13[1]};
      }
    } else if constexpr (kXsQ) {
      // Q fragments (wide apply): lane l holds column 32fn + l%32 at rows 16q + 8(l/32) + 0..7
      // of k-step q.  The block's two k-steps go to LDS as rows of 32 bf16 per column (column
      // c at byte c * kXP), and transposing reads bring back rows: in each 16-lane group g,
      // lane 4a + b points at columns 8q' + 4(g/2) + a, rows 16(g%2) + 4b .. +3, and lane r
      // receives those four columns of row 16(g%2) + r (a 96-byte pitch spreads both the
      // 16-byte writes and the 8-byte reads evenly over the banks).
      constexpr int kXP = 96;
      static_assert(C::kWTN * kXP <= 32 * C::kEpiPitch * 4, "transpose fits the wave's area");
      char* xt = reinterpret_cast<char*>(epi);
#pragma unroll
      for (int fn = 0; fn < C::kFN; ++fn)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *reinterpret_cast<u32x4_t*>(xt + (fn * 32 + (lane & 31)) * kXP +
                                      (16 * h + 8 * (lane >> 5)) * 2) =
              __builtin_bit_cast(u32x4_t, xs[2 * fm + h][fn]);
      wait_lds();
      __builtin_amdgcn_wave_barrier();
      const int g = lane >> 4;
      const int r = lane & 15;
#pragma unroll
      for (int fn = 0; fn < C::kFN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xw[fn][q] = __builtin_bit_cast(
              u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(
                           xt + (fn * 32 + 8 * q + 4 * (g >> 1) + (r >> 2)) * kXP +
                           (16 * (g & 1) + 4 * (r & 3)) * 2)));
      wait_lds();   // the staging below overwrites the area
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int fn = 0; fn < C::kFN; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = lane & 31;
        const int col = fn * 32 + 8 * q + 4 * (lane >> 5);
        float v[4] = {acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                      acc[fm][fn][4 * q + 3]};
        if constexpr (kKeep) {
          // the epilogue expression in fp32: b A + c (A A) for the polynomial; a X + P, or
          // bf16(P) + a X with split rounding, for the apply
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t d = xw[fn][q][e / 2];
            const float ax = p.alpha * bf16_to_f32((e % 2) ? (d >> 16) : (d & 0xFFFFu));
            if constexpr (OP == OP_POLY) {
              const float cq = p.beta * v[e];
              v[e] = ax + cq;
            } else {
              v[e] = p.split ? bf16_to_f32(f32_to_bf16(v[e])) + ax : ax + v[e];
            }
          }
        }
        *reinterpret_cast<f32x4_t*>(ep(row, col)) = f32x4_t{v[0], v[1], v[2], v[3]};
      }
    wait_lds();
    __builtin_amdgcn_wave_barrier();

    const int gi0 = i0 + wm * C::kWTM + fm * 32;   // first global row of this block
    const int gj0 = j0 + wn * C::kWTN;             // first global col of this wave

    // direct rows: each lane takes 8 consecutive columns of one row
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int row = pass * kRowsPerPass + lane / kLanesPerRow;
      const int col = (lane % kLanesPerRow) * 8;
      const int gi = gi0 + row;
      const int gj = gj0 + col;
      if (gi >= p.M || gj >= p.N) continue;
      const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(ep(row, col));
      const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(ep(row, col + 4));
      float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      u32x4_t out;
      if constexpr (kApply) {
        // already a·X + P (or its split form) in fp32
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        *reinterpret_cast<u32x4_t*>(Cb + (int64_t)gi * p.ldc + gj) = out;
      } else {
        if (diag_tile) {
          // below the diagonal of a diagonal tile: pieces wholly below are the mirror's; a piece
          // that straddles it (gi - gj = d in 1..7) takes its entries e < d from the mirrored
          // position (gj + e, gi), which this block holds d - e rows up and d columns right, so
          // that the whole piece leaves as one 16-byte store.  Every lane reads seven words (its
          // own position where it needs none) so that the reads go out together.
          if (gi >= gj + 8) continue;
          const int d = gi - gj;
          const bool straddle = d > 0;
          const int tr = straddle ? row - d : row;
          const int tc = straddle ? col + d : col;
          const int tmax = straddle ? d - 1 : 0;
          float t[7];
#pragma unroll
          for (int e = 0; e < 7; ++e) t[e] = *ep(tr + min(e, tmax), tc);
#pragma unroll
          for (int e = 0; e < 7; ++e)
            if (e < d) v[e] = t[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        *reinterpret_cast<u32x4_t*>(Cb + (int64_t)gi * p.ldc + gj) = out;
        if (diag_tile) {
          if constexpr (OP == OP_GRAM) {
            if (gi >= gj && gi < gj + 8) {
              const uint32_t w = out[(gi - gj) >> 1];
              tsum += bf16_to_f32(((gi - gj) & 1) ? (w >> 16) : (w & 0xFFFFu));
            }
          }
        }
      }
    }

    if constexpr (!kApply) {
      wait_lds();
      __builtin_amdgcn_wave_barrier();
      // mirror: C[gj][gi .. gi+7] from LDS column gj, rows gi .. gi+7 (8-row groups); lanes
      // 4c .. 4c+3 of a pass take the four groups of one column
#pragma unroll
      for (int pass = 0; pass < (C::kWTN * 4) / 64; ++pass) {
        const int item = pass * 64 + lane;
        const int col = item / 4;
        const int rq = item % 4;
        const int gj = gj0 + col;
        const int gi = gi0 + rq * 8;
        if (gj >= p.N || gi >= p.M) continue;
        // a diagonal tile mirrors only pieces wholly below its diagonal (the direct pass wrote
        // the pieces on and above it, and the 8x8 blocks the diagonal crosses)
        if (diag_tile && gj < gi + 8) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = *ep(rq * 8 + e, col);
        u32x4_t out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        *reinterpret_cast<u32x4_t*>(Cb + (int64_t)gj * p.ldc + gi) = out;
      }
    }
    wait_lds();
    __builtin_amdgcn_wave_barrier();
  }

  if constexpr (OP == OP_GRAM) {
    if (p.trace != nullptr && diag_tile) {
      // fixed-order reduction: butterfly within each wave, then waves in index order
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) tsum += __shfl_xor(tsum, off, 64);
      if constexpr (KSPLIT > 1 && C::kWaves > 1) {
        // one partial per diagonal 32x32 wave block, as a 32x32 tile writes it
        if (lane == 0 && computes && wm == wn && i0 + wm * 32 < p.M)
          p.trace[b * p.trace_slots + ti * WM + wm] = tsum;
      } else {
        if (lane == 0 && computes) sRed[wave] = tsum;
        __syncthreads();
        if (tid == 0) {
          float s = 0.0f;
          for (int w = 0; w < C::kWaves; ++w) s += sRed[w];
          p.trace[b * p.trace_slots + ti] = s;
        }
      }
    }
  }
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int OP, bool PT, bool QT, int BM, int BN, int WM, int WN, int STAGES, int BK, int SLAB,
          int KSPLIT = 1>
hipError_t launch(GemmParams p, int64_t g, hipStream_t stream) {
  using C = Cfg<BM, BN, WM, WN, STAGES, BK>;
  auto kern = gemm_kernel<OP, PT, QT, BM, BN, WM, WN, STAGES, BK, SLAB, KSPLIT>;
  constexpr int kThreads = C::kThreads * KSPLIT;
  constexpr int kLdsBytes = C::kLdsBytes * KSPLIT;
  // raise the dynamic LDS limit once per instantiation and device (bit d of the mask: device d;
  // devices past 63 set it on every launch)
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit == 0 || !(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_release);
  }
  // A dispatch counts its work-items in 32 bits: a stack whose tiles need more goes out as
  // consecutive sub-stacks (every matrix keeps its own tiles, so nothing in its arithmetic moves).
  const int64_t per_launch =
      std::max<int64_t>(1, int64_t(UINT32_MAX) / ((int64_t)p.tiles * kThreads));
  for (int64_t b0 = 0; b0 < g; b0 += per_launch) {
    const int64_t gb = std::min(per_launch, g - b0);
    GemmParams q = p;
    q.P += b0 * p.strideP;
    q.Q += b0 * p.strideQ;
    q.C += b0 * p.strideC;
    if (q.trace) q.trace += b0 * p.trace_slots;
    q.total = (int)(p.tiles * gb);
    // Gram launches of one to two rounds whose diagonal tiles can fill every shared CU (the Vs
    // and Us Grams: 320 tiles, 128 of them diagonal, 9% / 5% shorter); the polynomial's diagonal
    // tiles are not the cheaper ones (their epilogue costs twice an off-diagonal one's at K = s),
    // and there pairing them was 8-12% slower
    q.pair_diagonals = OP == OP_GRAM && q.total > kCus && q.total <= kFullRound &&
                       gb * p.tiles_m >= 2 * (q.total - kCus);
    hipLaunchKernelGGL(kern, dim3((unsigned)q.total), dim3(kThreads), kLdsBytes, stream, q);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Tile configurations (measured on MI355X over the five bank shapes):
//  * Gram: 128x128 tiles, 2x2 waves of 64x64, 64-deep slabs, two LDS stages (64 KB), so two
//    workgroups share a CU; it sums groups of 8 slabs (long K).
//  * Polynomial: the same tiles and ring with 2x4 waves of 64x32 (eight waves, four per SIMD over
//    the two workgroups: more waves to cover each other's waits); accumulates directly (K = s).
//  * Apply: 128x256 tiles, 2x4 waves of 64x64, 32-deep slabs, two stages (48 KB; two workgroups
//    per CU, 16 waves) when the stack fills at least half a round of 512 workgroups; otherwise
//    128x128 tiles (2x4 waves of 64x32, 64-deep slabs, two stages), which keep more CUs busy on
//    small stacks.  The wave layout and ring depth change no arithmetic: an element's MFMA chain
//    over k and its epilogue are the same in every configuration.
constexpr int kSymTile = 128;
// Small Grams and polynomials (at most 256 rows) take 32x32 tiles, one wave each: such launches
// have few tiles (three per 256x768 matrix at 128x128) and each workgroup streams its operands at
// a limited rate, so smaller tiles that spread the same work over more workgroups finish sooner.
// Their slabs are 128 deep (32 KB of LDS): a slab iteration costs about the same whatever its
// depth, and deeper slabs halve the iterations (256-deep ones cost the qk bank occupancy).
// The Gram of a tall matrix reads X down its columns (K-major slabs of at least 128 rows) and
// keeps 128x128.
constexpr int kSmallSym = 256;
int gram_tile(const Shape& sh) { return (!sh.tall() && sh.s() <= kSmallSym) ? 32 : kSymTile; }
int poly_tile(int s) { return s <= kSmallSym ? 32 : kSymTile; }
constexpr int kSmallBK = 128;
// The small Gram (k up to a few thousand) sums groups of 256 k, which its k-split launch spreads
// over waves; the larger Grams sum groups of 512 k (kGramSlabGroup).
constexpr int kSmallGroupK = 256;
// The Gram (K = the long side, up to thousands) sums each group of 8 slabs (512 k) in fresh
// registers and adds the group sums to the running sums: on low-rank-dominated inputs one long
// MFMA accumulation chain drifts from an fp64 reference noticeably more than fp32 sgemm does,
// while groups of 1 to 8 slabs all match sgemm's drift (measured on the warmed mlp bank); 8
// keeps the extra adds to one per 512 k.
#ifndef ANVIL_SLAB_GROUP
#define ANVIL_SLAB_GROUP 8
#endif
constexpr int kGramSlabGroup = ANVIL_SLAB_GROUP;   // in 64-deep slabs: 512 k


// ---------------------------------------------------------------------------------------------
// Fused polynomial and apply for small wide matrices (s = m <= 256 rows, m <= n): one launch per
// map instead of two.  Each workgroup owns a 32 x 128 tile of C = a X + B X.  It first forms the
// 32 rows of B = b A + c (A A) that the tile needs (all s columns; A is symmetric, so A A = A Aᵀ
// with both operands read along their rows) in LDS, with the polynomial kernel's arithmetic for
// every element: the same MFMA chain over k, the same epilogue expression and rounding (an entry
// below the diagonal is the sum of the same products in the same order as its mirror, so it has
// the same bits).  Then it multiplies those rows by the X slabs as the apply kernel does.  The
// row block of B is formed once per column tile (n / 128 times), which costs little at these
// sizes and saves the polynomial's launch.
//
// LDS: the 32 rows of A (later overwritten by the 32 rows of B) stay resident as one [32][256]
// K-contiguous block, loaded once; the ring holds only the slabs of all rows of A (phase 1), then
// the X slabs (phase 2); the accumulators are staged in the ring's space between the phases.
// ---------------------------------------------------------------------------------------------

struct PolyApplyParams {
  const uint16_t* A;          // [g][s][s]
  const uint16_t* X;          // [g][s][n]
  uint16_t* C;                // [g][s][n]
  int s, n;
  float a, b, c;
  int tiles_n;                // column tiles per matrix
  int tiles;                  // tiles per matrix
  int total;                  // tiles * g
};

constexpr int kPaRows = 32;         // tile rows (rows of B and of C)
constexpr int kPaChunk = 128;       // columns of C per chunk; a tile is NC chunks
constexpr int kPaMaxS = 256;
constexpr int kPaBK = 64;
constexpr int kPaBsBytes = kPaRows * kPaMaxS * 2;                       // 16 KB: A, then B, rows
constexpr int kPaStage1 = kPaMaxS * kPaBK * 2;                          // 32 KB: all rows of A
constexpr int kPaEpi2Pitch = 32 + 4;                                    // fp32 per staged row

// A tile of NC chunks of 128 columns, W = 4 or 8 waves: wave w owns columns 32(w % 4) .. +31 of
// chunks w / 4, w / 4 + W / 4, ... (every chunk with four waves, every other one with eight).
// In phase 1 wave w forms columns (256 / W) w .. of the 32 rows of B.  The X slabs of the chunks
// sit side by side in a stage (64 deep, or 32 deep for more than three chunks, so that two
// stages fit beside the rows of B and the phase-1 staging).
template <int NC, int W>
struct PaCfg {
  static_assert(W == 4 || W == 8, "four or eight waves");
  static_assert(NC % (W / 4) == 0, "whole chunks per wave");
  static constexpr int kWaves = W;
  static constexpr int kChunkStep = W / 4;          // chunks between a wave's chunks
  static constexpr int kOwn = NC / kChunkStep;      // chunks per wave
  static constexpr int kCols = kPaChunk * NC;
  static constexpr int kBK2 = NC <= 3 ? 64 : 32;
  static constexpr int kChunkBytes = kPaChunk * kBK2 * 2;
  static constexpr int kStage2 = NC * kChunkBytes;
  static constexpr int kEpi1Pitch = kPaMaxS / W + 4;                       // fp32 per staged row
  static constexpr int kEpi1Bytes = W * kPaRows * kEpi1Pitch * 4;          // 34.8 / 36.9 KB
  static constexpr int kRing2 = kPaBsBytes + kEpi1Bytes;                   // phase-2 ring offset
  static constexpr int kLdsBytes =
      kPaBsBytes + (2 * kPaStage1 > kEpi1Bytes + 2 * kStage2 ? 2 * kPaStage1
                                                             : kEpi1Bytes + 2 * kStage2);
  static_assert(kRing2 % 16 == 0, "16-byte aligned phase-2 ring");
  static_assert(kPaBsBytes + W * kPaRows * kPaEpi2Pitch * 4 <= kRing2,
                "phase-2 staging below the phase-2 ring");
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one CU");
};

template <int NC, int W>
__global__ __launch_bounds__(W * 64) void poly_apply_kernel(PolyApplyParams p) {
  using PC = PaCfg<NC, W>;
  constexpr int kWaves = W;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int logical = xcd_remap(blockIdx.x, p.total);
  const int64_t b = logical / p.tiles;
  const int t = logical % p.tiles;
  const int i0 = (t / p.tiles_n) * kPaRows;
  const int j0 = (t % p.tiles_n) * PC::kCols;
  const int s = p.s;

  const uint16_t* Ab = p.A + b * (int64_t)s * s;
  const uint16_t* Xb = p.X + b * (int64_t)s * p.n;
  uint16_t* Cb = p.C + b * (int64_t)s * p.n;
  const i32x4_t rA = make_rsrc(Ab, (uint32_t)((int64_t)s * s * 2));
  const i32x4_t rX = make_rsrc(Xb, (uint32_t)((int64_t)s * p.n * 2));
  char* Bs = smem;                 // [32][256] bf16, KContig<32, 256>: rows i0.. of A, then of B
  using BsLayout = KContig<kPaRows, kPaMaxS>;
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t ring1 = lds0 + kPaBsBytes;
  const uint32_t ring2 = lds0 + PC::kRing2;

  // rows i0..i0+31 of A into Bs: instruction u (1 KB) holds rows 2u, 2u+1, lane L row 2u + L/32,
  // physical slot L%32 = logical slot (L%32) ^ swizzle(row); zeros past s
#pragma unroll
  for (int q = 0; q < kPaRows / 2 / kWaves; ++q) {
    const int u = wave + q * kWaves;
    const int row = 2 * u + (lane >> 5);
    const int c = (lane & 31) ^ BsLayout::swz(row);
    const int gr = i0 + row;
    const uint32_t voff = (gr < s && c * 8 < s) ? (uint32_t)(gr * s + c * 8) * 2u : kOOB;
    dma16(rA, lds0 + (uint32_t)u * 1024u, voff);
  }
  // phase 1: the slabs of all rows of A (K-contiguous, 64 deep)
  const SlabCopy<false, kPaMaxS, kPaBK, kWaves> copyQ1(s, 0, s, wave, lane);
  constexpr int kFn1 = kPaMaxS / kWaves / 32;                 // 2 fragments per wave (1 of 8)
  const int KT = (s + kPaBK - 1) / kPaBK;
  copyQ1.issue(rA, ring1, 0, s, wave);

  // the X values of this wave's part of the final epilogue, fetched now (8 columns per lane)
  constexpr int kLanesPerRow2 = 32 / 8;                      // 4
  constexpr int kRowsPerPass2 = 64 / kLanesPerRow2;         // 16
  constexpr int kPasses2 = kPaRows / kRowsPerPass2;         // 2
  const int cg = wave % 4;                                   // column group inside a chunk
  const int c0 = wave / 4;                                   // this wave's first chunk
  u32x4_t xe[PC::kOwn][kPasses2];
#pragma unroll
  for (int o = 0; o < PC::kOwn; ++o)
#pragma unroll
    for (int pass = 0; pass < kPasses2; ++pass) {
      const int ch = c0 + o * PC::kChunkStep;
      const int gi = i0 + pass * kRowsPerPass2 + lane / kLanesPerRow2;
      const int gj = j0 + ch * kPaChunk + cg * 32 + (lane % kLanesPerRow2) * 8;
      xe[o][pass] = (gi < s && gj < p.n)
                        ? *reinterpret_cast<const u32x4_t*>(Xb + (int64_t)gi * p.n + gj)
                        : u32x4_t{0u, 0u, 0u, 0u};
    }

  f32x16_t acc1[kFn1];
#pragma unroll
  for (int f = 0; f < kFn1; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc1[f][r] = 0.0f;
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmcnt<0>();
    __syncthreads();
    if (kt + 1 < KT)
      copyQ1.issue(rA, ring1 + (uint32_t)(((kt + 1) & 1) * kPaStage1), (kt + 1) * kPaBK, s, wave);
    const char* tq = smem + kPaBsBytes + (kt & 1) * kPaStage1;
#pragma unroll
    for (int ks = 0; ks < kPaBK / 16; ++ks) {
      const bf16x8_t fa = read_frag<false, kPaRows, kPaMaxS>(Bs, 0, kt * (kPaBK / 16) + ks, lane);
#pragma unroll
      for (int f = 0; f < kFn1; ++f) {
        const bf16x8_t fb =
            read_frag<false, kPaMaxS, kPaBK>(tq, wave * (kPaMaxS / kWaves) + f * 32, ks, lane);
        acc1[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc1[f], 0, 0, 0);
      }
    }
  }
  __syncthreads();   // the ring and the A rows are read: stage the accumulators, load X

  // the X slabs of the chunks (chunk ch at ch * kChunkBytes of a stage)
  using Copy2 = SlabCopy<true, kPaChunk, PC::kBK2, kWaves>;
  Copy2 copyQ2[NC];
#pragma unroll
  for (int ch = 0; ch < NC; ++ch) copyQ2[ch] = Copy2(p.n, j0 + ch * kPaChunk, p.n, wave, lane);
  auto issue2 = [&](uint32_t dst, int k0) {
#pragma unroll
    for (int ch = 0; ch < NC; ++ch)
      copyQ2[ch].issue(rX, dst + (uint32_t)(ch * PC::kChunkBytes), k0, s, wave);
  };
  issue2(ring2, 0);

  // phase-1 epilogue: B = b*A + c*(A*A), rounded to bf16, in place of A in Bs (each lane reads
  // the A piece it then overwrites; zeros past column s)
  {
    float* epi = reinterpret_cast<float*>(smem + kPaBsBytes) + wave * kPaRows * PC::kEpi1Pitch;
    auto ep = [&](int row, int col) { return epi + row * PC::kEpi1Pitch + (col ^ (row & 16)); };
#pragma unroll
    for (int f = 0; f < kFn1; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = lane & 31;
        const int col = f * 32 + 8 * q + 4 * (lane >> 5);
        *reinterpret_cast<f32x4_t*>(ep(row, col)) =
            f32x4_t{acc1[f][4 * q], acc1[f][4 * q + 1], acc1[f][4 * q + 2], acc1[f][4 * q + 3]};
      }
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    constexpr int kLanesPerRow = (kPaMaxS / kWaves) / 8;   // 8 (four waves), 4 (eight)
    constexpr int kRowsPerPass = 64 / kLanesPerRow;           // 8
#pragma unroll
    for (int pass = 0; pass < kPaRows / kRowsPerPass; ++pass) {
      const int row = pass * kRowsPerPass + lane / kLanesPerRow;
      const int col = (lane % kLanesPerRow) * 8;
      const int j = wave * (kPaMaxS / kWaves) + col;       // column of B (k of phase 2)
      u32x4_t* piece = reinterpret_cast<u32x4_t*>(Bs + BsLayout::offset(row, j / 8));
      const u32x4_t ae = *piece;
      const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(ep(row, col));
      const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(ep(row, col + 4));
      const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      u32x4_t out = {0u, 0u, 0u, 0u};
      if (j < s && i0 + row < s) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ba0 = p.b * bf16_to_f32(ae[e] & 0xFFFFu);
          const float ba1 = p.b * bf16_to_f32(ae[e] >> 16);
          const float cq0 = p.c * v[2 * e];
          const float cq1 = p.c * v[2 * e + 1];
          out[e] = pack_bf16x2(ba0 + cq0, ba1 + cq1);
        }
      }
      *piece = out;
    }
  }
  __syncthreads();   // Bs holds B; the staging area is free

  // ---- phase 2: C = a X + B X on the chunks' columns (wave w: 32w .. 32w+31 of each), K = s ----
  constexpr int kKs2 = PC::kBK2 / 16;
  const int KT2 = (s + PC::kBK2 - 1) / PC::kBK2;
  f32x16_t acc2[PC::kOwn];
#pragma unroll
  for (int o = 0; o < PC::kOwn; ++o)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc2[o][r] = 0.0f;
  for (int kt = 0; kt < KT2; ++kt) {
    wait_vmcnt<0>();
    __syncthreads();
    if (kt + 1 < KT2) issue2(ring2 + (uint32_t)(((kt + 1) & 1) * PC::kStage2), (kt + 1) * PC::kBK2);
    const char* tq = smem + PC::kRing2 + (kt & 1) * PC::kStage2;
#pragma unroll
    for (int ks = 0; ks < kKs2; ++ks) {
      const bf16x8_t fa = read_frag<false, kPaRows, kPaMaxS>(Bs, 0, kt * kKs2 + ks, lane);
#pragma unroll
      for (int o = 0; o < PC::kOwn; ++o) {
        const int ch = c0 + o * PC::kChunkStep;
        const bf16x8_t fb = read_frag<true, kPaChunk, PC::kBK2>(tq + ch * PC::kChunkBytes,
                                                                cg * 32, ks, lane);
        acc2[o] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc2[o], 0, 0, 0);
      }
    }
  }

  // phase-2 epilogue: C = bf16(a*X + B X), as the apply's fused form, one chunk at a time
  float* epi = reinterpret_cast<float*>(smem + kPaBsBytes) + wave * kPaRows * kPaEpi2Pitch;
  auto ep = [&](int row, int col) { return epi + row * kPaEpi2Pitch + (col ^ (row & 16)); };
#pragma unroll
  for (int o = 0; o < PC::kOwn; ++o) {
    const int ch = c0 + o * PC::kChunkStep;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = lane & 31;
      const int col = 8 * q + 4 * (lane >> 5);
      *reinterpret_cast<f32x4_t*>(ep(row, col)) =
          f32x4_t{acc2[o][4 * q], acc2[o][4 * q + 1], acc2[o][4 * q + 2], acc2[o][4 * q + 3]};
    }
    wait_lds();
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int pass = 0; pass < kPasses2; ++pass) {
      const int row = pass * kRowsPerPass2 + lane / kLanesPerRow2;
      const int col = (lane % kLanesPerRow2) * 8;
      const int gi = i0 + row;
      const int gj = j0 + ch * kPaChunk + cg * 32 + col;
      if (gi >= s || gj >= p.n) continue;
      const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(ep(row, col));
      const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(ep(row, col + 4));
      const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      u32x4_t out;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ax0 = p.a * bf16_to_f32(xe[o][pass][e] & 0xFFFFu);
        const float ax1 = p.a * bf16_to_f32(xe[o][pass][e] >> 16);
        out[e] = pack_bf16x2(ax0 + v[2 * e], ax1 + v[2 * e + 1]);
      }
      *reinterpret_cast<u32x4_t*>(Cb + (int64_t)gi * p.n + gj) = out;
    }
    // the next chunk reuses this wave's staging rows
    wait_lds();
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

int gram_trace_slots(const Shape& sh) { return ceil_div(sh.s(), gram_tile(sh)); }

hipError_t launch_gram(const uint16_t* x, uint16_t* a, float* trace_partials, const Shape& sh,
                       hipStream_t stream) {
  const int s = sh.s();
  GemmParams p{};
  p.P = x;
  p.Q = x;
  p.strideP = p.strideQ = (int64_t)sh.m * sh.n;
  p.bytesP = p.bytesQ = (uint32_t)((int64_t)sh.m * sh.n * 2);
  p.ldp = p.ldq = sh.n;
  p.M = p.N = s;
  p.K = sh.L();
  p.C = a;
  p.strideC = (int64_t)s * s;
  p.ldc = s;
  p.trace = trace_partials;
  p.trace_slots = gram_trace_slots(sh);
  p.tiles_m = p.tiles_n = ceil_div(s, gram_tile(sh));
  p.tiles = p.tiles_m * (p.tiles_m + 1) / 2;
  if (gram_tile(sh) == 32) {
    // A launch whose one-wave tiles fit one round on the CUs gives each 256-k group of a tile to
    // a wave of its own (KSPLIT); the sums and their order are those of the one-wave tile.
    constexpr int kSlab = kSmallGroupK / kSmallBK;
    const int groups = ceil_div(ceil_div(p.K, kSmallBK), kSlab);
    if ((int64_t)p.tiles * sh.g <= kCus) {
      if (groups == 2)
        return launch<OP_GRAM, false, false, 32, 32, 1, 1, 2, kSmallBK, kSlab, 2>(p, sh.g, stream);
      if (groups == 3)
        return launch<OP_GRAM, false, false, 32, 32, 1, 1, 2, kSmallBK, kSlab, 3>(p, sh.g, stream);
      if (groups == 4)
        return launch<OP_GRAM, false, false, 32, 32, 1, 1, 2, kSmallBK, kSlab, 4>(p, sh.g, stream);
    }
    // Too many one-wave tiles for one round: 64x64 tiles of 2x2 such blocks (64-deep slabs, the
    // same 256-k groups) when those fit one round, each group on its own four waves.
    constexpr int kSlab64 = kSmallGroupK / 64;
    const int tiles_m64 = ceil_div(s, 64);
    const int tiles64 = tiles_m64 * (tiles_m64 + 1) / 2;
    if ((int64_t)p.tiles * sh.g > kCus && (int64_t)tiles64 * sh.g <= kCus && groups >= 2 &&
        groups <= 4) {
      p.tiles_m = p.tiles_n = tiles_m64;
      p.tiles = tiles64;
      if (groups == 2)
        return launch<OP_GRAM, false, false, 64, 64, 2, 2, 2, 64, kSlab64, 2>(p, sh.g, stream);
      if (groups == 3)
        return launch<OP_GRAM, false, false, 64, 64, 2, 2, 2, 64, kSlab64, 3>(p, sh.g, stream);
      return launch<OP_GRAM, false, false, 64, 64, 2, 2, 2, 64, kSlab64, 4>(p, sh.g, stream);
    }
    return launch<OP_GRAM, false, false, 32, 32, 1, 1, 2, kSmallBK, kSlab>(p, sh.g, stream);
  }
  if (sh.tall())
    return launch<OP_GRAM, true, true, 128, 128, 2, 2, 2, 64, kGramSlabGroup>(p, sh.g, stream);
  return launch<OP_GRAM, false, false, 128, 128, 2, 2, 2, 64, kGramSlabGroup>(p, sh.g, stream);
}

hipError_t launch_poly(const uint16_t* a, uint16_t* bout, float coef_b, float coef_c, int64_t g,
                       int s, hipStream_t stream) {
  GemmParams p{};
  p.P = a;
  p.Q = a;
  p.strideP = p.strideQ = (int64_t)s * s;
  p.bytesP = p.bytesQ = (uint32_t)((int64_t)s * s * 2);
  p.ldp = p.ldq = s;
  p.M = p.N = p.K = s;
  p.C = bout;
  p.strideC = (int64_t)s * s;
  p.ldc = s;
  p.alpha = coef_b;
  p.beta = coef_c;
  p.tiles_m = p.tiles_n = ceil_div(s, poly_tile(s));
  p.tiles = p.tiles_m * (p.tiles_m + 1) / 2;
  if (poly_tile(s) == 32) {
    if ((int64_t)p.tiles * g <= kCus)
      return launch<OP_POLY, false, false, 32, 32, 1, 1, 2, kSmallBK, 0>(p, g, stream);
    // more one-wave tiles than CUs: 64x64 tiles of four such waves (a quarter of the workgroups,
    // each copying its operand rows once for four blocks); 3-9% shorter steps from 32 matrices of
    // 256x768 up, the same below
    p.tiles_m = p.tiles_n = ceil_div(s, 64);
    p.tiles = p.tiles_m * (p.tiles_m + 1) / 2;
    return launch<OP_POLY, false, false, 64, 64, 2, 2, 2, kSmallBK, 0>(p, g, stream);
  }
  return launch<OP_POLY, false, false, 128, 128, 2, 4, 2, 64, 0>(p, g, stream);
}

// Tall apply, C = a X + X B: P = X rows (K = n contiguous); Q(j, k) = B[k][j] (K-major: B is
// symmetric, and a slab of its rows k is 2*BN contiguous bytes per row where the K-contiguous form
// would fetch 2*BK-byte pieces, half a cache line at BK = 32; measured 1.3% faster per mlp step).
template <int BM, int BN, int WM, int WN, int STAGES, int BK>
hipError_t launch_apply_tall(const uint16_t* x, const uint16_t* bm, uint16_t* c, float coef_a,
                             bool split, const Shape& sh, hipStream_t stream) {
  const int s = sh.s();
  GemmParams p{};
  p.M = sh.m;
  p.N = sh.n;
  p.K = sh.n;
  p.P = x;
  p.strideP = (int64_t)sh.m * sh.n;
  p.bytesP = (uint32_t)((int64_t)sh.m * sh.n * 2);
  p.ldp = sh.n;
  p.Q = bm;
  p.strideQ = (int64_t)s * s;
  p.bytesQ = (uint32_t)((int64_t)s * s * 2);
  p.ldq = s;
  p.C = c;
  p.strideC = (int64_t)sh.m * sh.n;
  p.ldc = sh.n;
  p.alpha = coef_a;
  p.split = split ? 1 : 0;
  p.tiles_m = ceil_div(p.M, BM);
  p.tiles_n = ceil_div(p.N, BN);
  p.tiles = p.tiles_m * p.tiles_n;
  return launch<OP_APPLY_XT, false, true, BM, BN, WM, WN, STAGES, BK, 0>(p, sh.g, stream);
}

// Wide (and square) apply, C = a X + B X: P = rows of B (K = m contiguous), Q(j, k) = X[k][j]
// (K-major); the epilogue takes X[i][j] from the Q fragments its waves keep.
template <int BM, int BN, int WM, int WN, int STAGES, int BK>
hipError_t launch_apply_wide(const uint16_t* x, const uint16_t* bm, uint16_t* c, float coef_a,
                             bool split, const Shape& sh, hipStream_t stream) {
  const int s = sh.s();
  GemmParams p{};
  p.M = sh.m;
  p.N = sh.n;
  p.K = sh.m;
  p.P = bm;
  p.strideP = (int64_t)s * s;
  p.bytesP = (uint32_t)((int64_t)s * s * 2);
  p.ldp = s;
  p.Q = x;
  p.strideQ = (int64_t)sh.m * sh.n;
  p.bytesQ = (uint32_t)((int64_t)sh.m * sh.n * 2);
  p.ldq = sh.n;
  p.C = c;
  p.strideC = (int64_t)sh.m * sh.n;
  p.ldc = sh.n;
  p.alpha = coef_a;
  p.split = split ? 1 : 0;
  p.tiles_m = ceil_div(p.M, BM);
  p.tiles_n = ceil_div(p.N, BN);
  p.tiles = p.tiles_m * p.tiles_n;
  return launch<OP_APPLY, false, true, BM, BN, WM, WN, STAGES, BK, 0>(p, sh.g, stream);
}

namespace {

enum ApplyTiles { kApply128x256, kApply32x128, kApply128x128 };

ApplyTiles apply_tiles(const Shape& sh) {
  const int64_t wide_tiles = (int64_t)ceil_div(sh.m, 128) * ceil_div(sh.n, 256) * sh.g;
  if (2 * wide_tiles >= kFullRound) return kApply128x256;
  // launches with no more 128x128 tiles than CUs: 32x128 tiles, four times the workgroups
  if ((int64_t)ceil_div(sh.m, 128) * ceil_div(sh.n, 128) * sh.g <= kCus) return kApply32x128;
  return kApply128x128;
}

}  // namespace

hipError_t launch_apply(const uint16_t* x, const uint16_t* bm, uint16_t* c, float coef_a,
                        bool split, const Shape& sh, hipStream_t stream) {
  if (sh.tall()) {
    switch (apply_tiles(sh)) {
      case kApply128x256:
        return launch_apply_tall<128, 256, 2, 4, 2, 32>(x, bm, c, coef_a, split, sh, stream);
      case kApply32x128:
        return launch_apply_tall<32, 128, 1, 2, 2, 64>(x, bm, c, coef_a, split, sh, stream);
      default:
        return launch_apply_tall<128, 128, 2, 4, 2, 64>(x, bm, c, coef_a, split, sh, stream);
    }
  }
  switch (apply_tiles(sh)) {
    case kApply128x256:
      return launch_apply_wide<128, 256, 2, 4, 2, 32>(x, bm, c, coef_a, split, sh, stream);
    case kApply32x128:
      return launch_apply_wide<32, 128, 1, 2, 2, 64>(x, bm, c, coef_a, split, sh, stream);
    default:
      return launch_apply_wide<128, 128, 2, 4, 2, 64>(x, bm, c, coef_a, split, sh, stream);
  }
}

// The fused launch forms each 32-row block of B once per column tile, so it pays only while its
// workgroups fit one round on the CUs: the column tile is the narrowest of 1, 2, 3 or 6 chunks
// of 128 columns with which they do (one chunk: 82 KB of LDS; more: up to 149 KB, one workgroup
// per CU).  Measured on 256x768 with one chunk it beats the two launches up to 4 matrices (94.6
// against 109.1 us alone) and loses from 8 on, where it would form each block of B six times.
// Tiles of an even number of chunks run eight waves (two waves per SIMD; each wave owns every
// other chunk), which took the step from 100.9 to 96.1 us at 8 matrices (2 chunks) and from 204.1
// to 194.3 us at 32 (6 chunks); with four waves six chunks lost to the two launches at 24
// matrices (165.8 against 159.4 us), with eight they win (152.1).
static int poly_apply_chunks(const Shape& sh) {
  if (sh.tall() || sh.s() > kPaMaxS) return 0;
  for (int nc : {1, 2, 3, 6})
    if ((int64_t)ceil_div(sh.m, kPaRows) * ceil_div(sh.n, kPaChunk * nc) * sh.g <= kCus) return nc;
  return 0;
}

bool poly_apply_fused(const Shape& sh) { return poly_apply_chunks(sh) > 0; }

namespace {

template <int NC, int W = 4>
hipError_t launch_poly_apply_nc(const PolyApplyParams& p0, int64_t g, int m, int n,
                                hipStream_t stream) {
  using PC = PaCfg<NC, W>;
  auto kern = poly_apply_kernel<NC, W>;
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit == 0 || !(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, PC::kLdsBytes);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_release);
  }
  PolyApplyParams p = p0;
  p.tiles_n = ceil_div(n, PC::kCols);
  p.tiles = ceil_div(m, kPaRows) * p.tiles_n;
  // the tiles of the whole stack fit one round on the CUs, so the grid fits one launch
  p.total = (int)(p.tiles * g);
  hipLaunchKernelGGL(kern, dim3((unsigned)p.total), dim3(W * 64), PC::kLdsBytes, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_poly_apply(const uint16_t* a, const uint16_t* x, uint16_t* c, float coef_a,
                             float coef_b, float coef_c, const Shape& sh, hipStream_t stream) {
  const int nc = poly_apply_chunks(sh);
  PolyApplyParams p{};
  p.A = a;
  p.X = x;
  p.C = c;
  p.s = sh.m;
  p.n = sh.n;
  p.a = coef_a;
  p.b = coef_b;
  p.c = coef_c;
  switch (nc) {
    case 1:
      return launch_poly_apply_nc<1>(p, sh.g, sh.m, sh.n, stream);
    case 2:
      return launch_poly_apply_nc<2, 8>(p, sh.g, sh.m, sh.n, stream);
    case 3:
      return launch_poly_apply_nc<3>(p, sh.g, sh.m, sh.n, stream);
    case 6:
      return launch_poly_apply_nc<6, 8>(p, sh.g, sh.m, sh.n, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace anvil
