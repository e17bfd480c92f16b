// C ABI of libanvil.so: argument checks, workspace management and the launch sequence of one
// ANVIL bank step (modded-nanogpt anvil.py, `anvil_cascade`).
#include <hip/hip_runtime.h>

#include <atomic>
#include <initializer_list>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/anvil.h"
#include "launchers.h"

namespace {

using anvil::Shape;

// The six quintic maps (a, b, c) in application order (anvil.py, the table of maps); the kernels
// take them as fp32 values of these doubles.
const double kMaps[6][3] = {
    {3.923798038567, -6.095026865488, 3.905234618423},
    {3.278126713798, -3.328923386476, 0.989127286973},
    {3.505298394150, -5.137358782410, 1.968325560615},
    {2.815058591845, -3.685181239622, 1.417196497642},
    {2.245503932403, -2.443826979899, 0.963091710461},
    {2.256537145403, -2.166840097229, 0.929501253245},
};
struct MapTable {
  float v[6][3];
  MapTable() {
    for (int k = 0; k < 6; ++k)
      for (int j = 0; j < 3; ++j) v[k][j] = static_cast<float>(kMaps[k][j]);
  }
};
const MapTable kAnvilMaps;
constexpr int kMaxMaps = 16;

// Banks with more rows than this use the split (two-rounding) apply (anvil.py).
constexpr int64_t kSplitMinRows = 1024;

thread_local int t_last_hip = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ANVIL_OK;
  t_last_hip = static_cast<int>(e);
  return ANVIL_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

// Shape checks shared by every entry point.  Returns ANVIL_OK with *empty set for a zero-size
// stack.
int check_shape(int64_t g, int64_t m, int64_t n, Shape* sh, bool* empty) {
  if (g < 0 || m < 0 || n < 0) return ANVIL_ERR_INVALID_ARG;
  *empty = (g == 0 || m == 0 || n == 0);
  if (*empty) return ANVIL_OK;
  if (m % 8 != 0 || n % 8 != 0) return ANVIL_ERR_UNSUPPORTED;
  if (g > 65535) return ANVIL_ERR_UNSUPPORTED;
  // one bf16 matrix at most 2 GiB: every buffer offset (and the past-the-end offset that loads
  // zeros at ragged edges) stays below 2^32
  if (m * n > (int64_t(1) << 30)) return ANVIL_ERR_UNSUPPORTED;
  // a whole stack at most 2^35 elements (already 384 GiB of gradient and rails, more than one
  // GPU holds): every launch grid stays far below 2^31 workgroups
  if (g * m * n > (int64_t(1) << 35)) return ANVIL_ERR_UNSUPPORTED;
  sh->g = g;
  sh->m = static_cast<int>(m);
  sh->n = static_cast<int>(n);
  return ANVIL_OK;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace regions: ping-pong X (bf16 [g,m,n]), A and B (bf16 [g,s,s]), trace partials
// (fp32 [g, slots]) and d (fp32 [g]).
struct Layout {
  size_t ping, a, b, partials, d, lanes, total;
};

Layout layout_for(const Shape& sh) {
  const size_t g = static_cast<size_t>(sh.g);
  const size_t s = static_cast<size_t>(sh.s());
  Layout l;
  size_t off = 0;
  l.ping = off;
  off += round_up(g * sh.m * sh.n * 2);
  l.a = off;
  off += round_up(g * s * s * 2);
  l.b = off;
  off += round_up(g * s * s * 2);
  l.partials = off;
  off += round_up(g * anvil::gram_trace_slots(sh) * 4);
  l.d = off;
  off += round_up(g * 4);
  l.lanes = off;   // equalizer scratch: lane powers and lane scales
  off += round_up(2 * g * anvil::equalizer_lanes(sh) * 4);
  l.total = off;
  return l;
}

// A caller buffer: its address and the bytes the call touches.
struct Buf {
  const void* p;
  size_t bytes;
};

// ANVIL_ERR_ALIAS if any two of the (non-null) buffers overlap.
int check_disjoint(std::initializer_list<Buf> bufs) {
  for (auto i = bufs.begin(); i != bufs.end(); ++i)
    for (auto j = i + 1; j != bufs.end(); ++j)
      if (i->p && j->p && overlap(i->p, i->bytes, j->p, j->bytes)) return ANVIL_ERR_ALIAS;
  return ANVIL_OK;
}

// The step's buffers: grad (fp32 or bf16: grad_bytes per element), velocity, out.
int check_step_args(const void* grad, size_t grad_bytes, float* velocity, uint16_t* out,
                    const Shape& sh) {
  if (!grad || !velocity || !out) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(grad, 16) || !aligned(velocity, 16) || !aligned(out, 16))
    return ANVIL_ERR_MISALIGNED;
  const size_t cnt = static_cast<size_t>(sh.g) * sh.m * sh.n;
  return check_disjoint({{grad, cnt * grad_bytes}, {velocity, cnt * 8}, {out, cnt * 2}});
}

// The launch sequence: momentum, Gram 0 with trace, normalise, then per map (Gram, poly, apply).
// The apply ping-pongs between `out` and the workspace copy; X starts in `out` for an even number
// of maps and in the workspace copy for an odd number, so that the last apply writes `out`.
// The momentum inputs: an fp32 or bf16 gradient and the rail scalars by value or on the device.
struct MomentumIn {
  const void* grad;
  bool grad_bf16;
  const float* scalars;   // device (momentum, fast_beta, fast_weight), or null: use the values
  float momentum, fast_beta, fast_weight;
};

int run_step(const MomentumIn& mi, float* velocity, uint16_t* out, const Shape& sh, char* ws,
             hipStream_t stream, const float (*maps)[3] = kAnvilMaps.v, int steps = 6) {
  const Layout l = layout_for(sh);
  uint16_t* ping = reinterpret_cast<uint16_t*>(ws + l.ping);
  uint16_t* A = reinterpret_cast<uint16_t*>(ws + l.a);
  uint16_t* B = reinterpret_cast<uint16_t*>(ws + l.b);
  float* partials = reinterpret_cast<float*>(ws + l.partials);
  float* d = reinterpret_cast<float*>(ws + l.d);
  const int64_t count = sh.g * sh.m * sh.n;
  const bool split = sh.m > kSplitMinRows;

  uint16_t* X = (steps % 2 == 0) ? out : ping;
  uint16_t* Y = (steps % 2 == 0) ? ping : out;
  hipError_t e =
      mi.scalars != nullptr
          ? anvil::launch_momentum_dev(mi.grad, mi.grad_bf16, velocity, velocity + count, X, count,
                                       mi.scalars, stream)
          : anvil::launch_momentum(static_cast<const float*>(mi.grad), velocity, velocity + count,
                                   X, count, mi.momentum, mi.fast_beta, mi.fast_weight, stream);
  if (e != hipSuccess) return hip_status(e);
  e = anvil::launch_gram(X, A, partials, sh, stream);
  if (e != hipSuccess) return hip_status(e);
  e = anvil::launch_normalize(X, A, partials, d, sh, stream);
  if (e != hipSuccess) return hip_status(e);
  // small wide shapes (s <= 256, few matrices) form B inside the apply's launch
  const bool fused = anvil::poly_apply_fused(sh);
  for (int k = 0; k < steps; ++k) {
    if (k > 0) {
      e = anvil::launch_gram(X, A, nullptr, sh, stream);
      if (e != hipSuccess) return hip_status(e);
    }
    if (fused) {
      e = anvil::launch_poly_apply(A, X, Y, maps[k][0], maps[k][1], maps[k][2], sh, stream);
      if (e != hipSuccess) return hip_status(e);
    } else {
      e = anvil::launch_poly(A, B, maps[k][1], maps[k][2], sh.g, sh.s(), stream);
      if (e != hipSuccess) return hip_status(e);
      e = anvil::launch_apply(X, B, Y, maps[k][0], split, sh, stream);
      if (e != hipSuccess) return hip_status(e);
    }
    std::swap(X, Y);
  }
  return ANVIL_OK;
}

// The update's buffers on top of the step's; scalars (device fp32 [4]) may be null.
int check_update_args(const void* grad, size_t grad_bytes, const float* velocity,
                      const uint16_t* update, const float* lane_energy, const uint16_t* param,
                      const uint16_t* mantissa, const float* eff_lr, const float* scalars,
                      const Shape& sh) {
  if (!lane_energy || !param || !mantissa || !eff_lr) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(param, 16) || !aligned(mantissa, 16) || !aligned(lane_energy, 4) ||
      !aligned(eff_lr, 4) || !aligned(scalars, 4))
    return ANVIL_ERR_MISALIGNED;
  const size_t cnt = static_cast<size_t>(sh.g) * sh.m * sh.n;
  const size_t lb = static_cast<size_t>(sh.g) * anvil::equalizer_lanes(sh) * 4;
  return check_disjoint({{grad, cnt * grad_bytes}, {velocity, cnt * 8}, {update, cnt * 2},
                         {param, cnt * 2}, {mantissa, cnt * 2}, {lane_energy, lb},
                         {eff_lr, static_cast<size_t>(sh.g) * 4}, {scalars, 16}});
}

// The parameter side of the update: the equalizer state and the decay's inputs.
struct UpdateIn {
  float* lane_energy;
  double beta2;
  uint16_t* param;
  uint16_t* mantissa;
  float eff_wd;
  const float* wd_dev;   // device eff_wd, or null: use the value
  const float* eff_lr;
};

// The whole bank update: the step (into `update`), then the equalizer and the decay, gated on the
// slow rail the step has just written.
int run_update(const MomentumIn& mi, float* velocity, uint16_t* update, const UpdateIn& ui,
               const Shape& sh, char* ws, hipStream_t stream) {
  int st = run_step(mi, velocity, update, sh, ws, stream);
  if (st != ANVIL_OK) return st;
  const Layout l = layout_for(sh);
  const int64_t count = sh.g * sh.m * sh.n;
  return hip_status(anvil::launch_equalize(update, ui.lane_energy, ui.beta2,
                                           reinterpret_cast<float*>(ws + l.lanes), sh, stream,
                                           ui.param, ui.mantissa, velocity + count, ui.eff_lr,
                                           ui.eff_wd, ui.wd_dev));
}

// Workspace cache of the allocating entry point, one grow-only buffer per (device, stream).
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, std::pair<void*, size_t>> g_ws;

// The cached workspace of at least `need` bytes for the current device and `stream`.  `lock`
// keeps the cache locked until the caller has enqueued its work with the buffer: a call on the
// same stream from another thread that has to grow it waits until then, and its stream
// synchronisation before the free then covers that work.
int cached_workspace(size_t need, hipStream_t hs, char** out, std::unique_lock<std::mutex>* lock) {
  // the cache may allocate, synchronise and free: none of that may happen under stream capture,
  // and a captured graph would keep using a buffer the cache frees later
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(hs, &cs);
  if (e != hipSuccess) return hip_status(e);
  if (cs != hipStreamCaptureStatusNone) return ANVIL_ERR_CAPTURING;
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  *lock = std::unique_lock<std::mutex>(g_ws_mutex);
  auto& slot = g_ws[{dev, hs}];
  if (slot.second < need) {
    if (slot.first) {
      // the old buffer may still be in use by work queued on this stream
      e = hipStreamSynchronize(hs);
      if (e != hipSuccess) return hip_status(e);
      e = hipFree(slot.first);
      slot = {nullptr, 0};
      if (e != hipSuccess) return hip_status(e);
    }
    void* p = nullptr;
    if (hipMalloc(&p, need) != hipSuccess || !p) {
      (void)hipGetLastError();
      return ANVIL_ERR_OOM;
    }
    slot = {p, need};
  }
  *out = static_cast<char*>(slot.first);
  return ANVIL_OK;
}

// Checks of a caller-owned workspace: size, alignment, and no overlap with the call's buffers.
int check_workspace(const void* workspace, size_t workspace_bytes, const Shape& sh,
                    std::initializer_list<Buf> bufs) {
  if (!workspace) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(workspace, kAlign)) return ANVIL_ERR_MISALIGNED;
  const Layout l = layout_for(sh);
  if (workspace_bytes < l.total) return ANVIL_ERR_UNSUPPORTED;
  for (const Buf& b : bufs)
    if (b.p && overlap(workspace, l.total, b.p, b.bytes)) return ANVIL_ERR_ALIAS;
  return ANVIL_OK;
}

// The workspace to use: the caller's (checked against `bufs`) or, when null, the cached one.
int pick_workspace(void* workspace, size_t workspace_bytes, const Shape& sh, hipStream_t hs,
                   std::initializer_list<Buf> bufs, char** ws, std::unique_lock<std::mutex>* lock) {
  if (workspace) {
    const int st = check_workspace(workspace, workspace_bytes, sh, bufs);
    if (st != ANVIL_OK) return st;
    *ws = static_cast<char*>(workspace);
    return ANVIL_OK;
  }
  return cached_workspace(layout_for(sh).total, hs, ws, lock);
}

// Scratch of anvil_bank_step_noalloc: the whole workspace of one bank step in a file-scope device
// array, so that a call allocates nothing.  Each device the library runs on holds its own copy
// (ANVIL_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, once per device, and every launch
// uses that address.
static __device__ __align__(256) char scratch[ANVIL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<char*> g_scratch_addr[kMaxScratchDevices];

// The current device's address of `scratch` (looked up on the first call on that device).
int scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return ANVIL_ERR_UNSUPPORTED;
  char* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (addr == nullptr) return ANVIL_ERR_HIP;
    p = static_cast<char*>(addr);
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return ANVIL_OK;
}

MomentumIn by_value(const float* grad, float momentum, float fast_beta, float fast_weight) {
  return MomentumIn{grad, false, nullptr, momentum, fast_beta, fast_weight};
}

size_t grad_elem_bytes(int grad_dtype) { return grad_dtype == ANVIL_GRAD_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

const char* anvil_status_string(int status) {
  switch (status) {
    case ANVIL_OK: return "ok";
    case ANVIL_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or bad flag)";
    case ANVIL_ERR_UNSUPPORTED:
      return "unsupported shape (m and n must be multiples of 8, m*n <= 2^30, g <= 65535, "
             "g*m*n <= 2^35) or workspace too small";
    case ANVIL_ERR_MISALIGNED: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case ANVIL_ERR_ALIAS: return "an output overlaps an input";
    case ANVIL_ERR_OOM: return "workspace allocation failed";
    case ANVIL_ERR_HIP: return "HIP runtime or launch error (see anvil_last_hip_error)";
    case ANVIL_ERR_TOO_LARGE:
      return "the bank step needs more scratch than anvil_bank_step_noalloc holds "
             "(anvil_workspace_bytes(g, m, n) > ANVIL_NOALLOC_SCRATCH_BYTES)";
    case ANVIL_ERR_CAPTURING:
      return "the stream is being captured: pass a caller workspace (the cached workspace may "
             "allocate and synchronise)";
    default: return "unknown status";
  }
}

int anvil_last_hip_error(void) { return t_last_hip; }

int anvil_version(void) { return 100; }

size_t anvil_workspace_bytes(int64_t g, int64_t m, int64_t n) {
  Shape sh;
  bool empty = false;
  if (check_shape(g, m, n, &sh, &empty) != ANVIL_OK || empty) return 0;
  return layout_for(sh).total;
}

int anvil_bank_step_ws(const float* grad, float* velocity, float momentum, float fast_beta,
                       float fast_weight, uint16_t* out, int64_t g, int64_t m, int64_t n,
                       void* workspace, size_t workspace_bytes, void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  st = check_step_args(grad, 4, velocity, out, sh);
  if (st != ANVIL_OK) return st;
  if (!workspace) return ANVIL_ERR_INVALID_ARG;
  const size_t cnt = static_cast<size_t>(sh.g) * sh.m * sh.n;
  char* ws = nullptr;
  std::unique_lock<std::mutex> lock;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = pick_workspace(workspace, workspace_bytes, sh, hs,
                      {{grad, cnt * 4}, {velocity, cnt * 8}, {out, cnt * 2}}, &ws, &lock);
  if (st != ANVIL_OK) return st;
  return run_step(by_value(grad, momentum, fast_beta, fast_weight), velocity, out, sh, ws, hs);
}

int anvil_bank_step(const float* grad, float* velocity, float momentum, float fast_beta,
                    float fast_weight, uint16_t* out, int64_t g, int64_t m, int64_t n,
                    void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  st = check_step_args(grad, 4, velocity, out, sh);
  if (st != ANVIL_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  std::unique_lock<std::mutex> lock;
  st = cached_workspace(layout_for(sh).total, hs, &ws, &lock);
  if (st != ANVIL_OK) return st;
  return run_step(by_value(grad, momentum, fast_beta, fast_weight), velocity, out, sh, ws, hs);
}

int anvil_bank_step_noalloc(const float* grad, float* velocity, float momentum, float fast_beta,
                            float fast_weight, uint16_t* out, int64_t g, int64_t m, int64_t n,
                            void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  st = check_step_args(grad, 4, velocity, out, sh);
  if (st != ANVIL_OK) return st;
  if (layout_for(sh).total > ANVIL_NOALLOC_SCRATCH_BYTES) return ANVIL_ERR_TOO_LARGE;
  char* ws = nullptr;
  st = scratch_address(&ws);
  if (st != ANVIL_OK) return st;
  // every scratch region the step reads is written earlier in the same step (ping-pong copy,
  // A, B, trace partials, d), so the array needs no clearing between calls
  return run_step(by_value(grad, momentum, fast_beta, fast_weight), velocity, out, sh, ws,
                  static_cast<hipStream_t>(stream));
}

int anvil_bank_step_maps(const float* grad, float* velocity, float momentum, float fast_beta,
                         float fast_weight, const float* maps, int steps, uint16_t* out,
                         int64_t g, int64_t m, int64_t n, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (steps < 1 || steps > kMaxMaps) return ANVIL_ERR_INVALID_ARG;
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  if (!maps) return ANVIL_ERR_INVALID_ARG;
  st = check_step_args(grad, 4, velocity, out, sh);
  if (st != ANVIL_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const size_t cnt = static_cast<size_t>(sh.g) * sh.m * sh.n;
  char* ws = nullptr;
  std::unique_lock<std::mutex> lock;
  st = pick_workspace(workspace, workspace_bytes, sh, hs,
                      {{grad, cnt * 4}, {velocity, cnt * 8}, {out, cnt * 2}}, &ws, &lock);
  if (st != ANVIL_OK) return st;
  float table[kMaxMaps][3];
  for (int k = 0; k < steps; ++k)
    for (int j = 0; j < 3; ++j) table[k][j] = maps[3 * k + j];
  return run_step(by_value(grad, momentum, fast_beta, fast_weight), velocity, out, sh, ws, hs,
                  table, steps);
}

int anvil_bank_step_dev(const void* grad, int grad_dtype, float* velocity, const float* scalars,
                        uint16_t* out, int64_t g, int64_t m, int64_t n, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (grad_dtype != ANVIL_GRAD_F32 && grad_dtype != ANVIL_GRAD_BF16) return ANVIL_ERR_INVALID_ARG;
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  const size_t gb = grad_elem_bytes(grad_dtype);
  st = check_step_args(grad, gb, velocity, out, sh);
  if (st != ANVIL_OK) return st;
  if (!scalars || !workspace) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(scalars, 4)) return ANVIL_ERR_MISALIGNED;
  const size_t cnt = static_cast<size_t>(sh.g) * sh.m * sh.n;
  st = check_disjoint({{scalars, 12}, {velocity, cnt * 8}, {out, cnt * 2}});
  if (st != ANVIL_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  std::unique_lock<std::mutex> lock;
  st = pick_workspace(workspace, workspace_bytes, sh, hs,
                      {{grad, cnt * gb}, {velocity, cnt * 8}, {out, cnt * 2}, {scalars, 12}}, &ws,
                      &lock);
  if (st != ANVIL_OK) return st;
  const MomentumIn mi{grad, grad_dtype == ANVIL_GRAD_BF16, scalars, 0.0f, 0.0f, 0.0f};
  return run_step(mi, velocity, out, sh, ws, hs);
}

int anvil_bank_update(const float* grad, float* velocity, float momentum, float fast_beta,
                      float fast_weight, uint16_t* update, float* lane_energy, double beta2,
                      uint16_t* param, uint16_t* mantissa, float eff_wd, const float* eff_lr,
                      int64_t g, int64_t m, int64_t n, void* stream) {
  return anvil_bank_update_ws(grad, velocity, momentum, fast_beta, fast_weight, update,
                              lane_energy, beta2, param, mantissa, eff_wd, eff_lr, g, m, n,
                              nullptr, 0, stream);
}

int anvil_bank_update_ws(const float* grad, float* velocity, float momentum, float fast_beta,
                         float fast_weight, uint16_t* update, float* lane_energy, double beta2,
                         uint16_t* param, uint16_t* mantissa, float eff_wd, const float* eff_lr,
                         int64_t g, int64_t m, int64_t n, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  st = check_step_args(grad, 4, velocity, update, sh);
  if (st != ANVIL_OK) return st;
  st = check_update_args(grad, 4, velocity, update, lane_energy, param, mantissa, eff_lr, nullptr,
                         sh);
  if (st != ANVIL_OK) return st;
  const size_t cnt = static_cast<size_t>(sh.g) * sh.m * sh.n;
  const size_t lb = static_cast<size_t>(sh.g) * anvil::equalizer_lanes(sh) * 4;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  std::unique_lock<std::mutex> lock;
  st = pick_workspace(workspace, workspace_bytes, sh, hs,
                      {{grad, cnt * 4}, {velocity, cnt * 8}, {update, cnt * 2}, {param, cnt * 2},
                       {mantissa, cnt * 2}, {lane_energy, lb},
                       {eff_lr, static_cast<size_t>(sh.g) * 4}},
                      &ws, &lock);
  if (st != ANVIL_OK) return st;
  const UpdateIn ui{lane_energy, beta2, param, mantissa, eff_wd, nullptr, eff_lr};
  return run_update(by_value(grad, momentum, fast_beta, fast_weight), velocity, update, ui, sh, ws,
                    hs);
}

int anvil_bank_update_dev(const void* grad, int grad_dtype, float* velocity,
                          const float* scalars, uint16_t* update, float* lane_energy,
                          double beta2, uint16_t* param, uint16_t* mantissa,
                          const float* eff_lr, int64_t g, int64_t m, int64_t n, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (grad_dtype != ANVIL_GRAD_F32 && grad_dtype != ANVIL_GRAD_BF16) return ANVIL_ERR_INVALID_ARG;
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  const size_t gb = grad_elem_bytes(grad_dtype);
  st = check_step_args(grad, gb, velocity, update, sh);
  if (st != ANVIL_OK) return st;
  if (!scalars || !workspace) return ANVIL_ERR_INVALID_ARG;
  st = check_update_args(grad, gb, velocity, update, lane_energy, param, mantissa, eff_lr, scalars,
                         sh);
  if (st != ANVIL_OK) return st;
  const size_t cnt = static_cast<size_t>(sh.g) * sh.m * sh.n;
  const size_t lb = static_cast<size_t>(sh.g) * anvil::equalizer_lanes(sh) * 4;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  std::unique_lock<std::mutex> lock;
  st = pick_workspace(workspace, workspace_bytes, sh, hs,
                      {{grad, cnt * gb}, {velocity, cnt * 8}, {update, cnt * 2}, {param, cnt * 2},
                       {mantissa, cnt * 2}, {lane_energy, lb},
                       {eff_lr, static_cast<size_t>(sh.g) * 4}, {scalars, 16}},
                      &ws, &lock);
  if (st != ANVIL_OK) return st;
  const MomentumIn mi{grad, grad_dtype == ANVIL_GRAD_BF16, scalars, 0.0f, 0.0f, 0.0f};
  const UpdateIn ui{lane_energy, beta2, param, mantissa, 0.0f, scalars + 3, eff_lr};
  return run_update(mi, velocity, update, ui, sh, ws, hs);
}

int64_t anvil_equalizer_lanes(int64_t m, int64_t n) {
  Shape sh;
  bool empty = false;
  if (check_shape(1, m, n, &sh, &empty) != ANVIL_OK || empty) return 0;
  return anvil::equalizer_lanes(sh);
}

int anvil_equalize(uint16_t* update, float* lane_energy, double beta2, float* lane_scratch,
                   int64_t g, int64_t m, int64_t n, void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  if (!update || !lane_energy || !lane_scratch) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(update, 16) || !aligned(lane_energy, 4) || !aligned(lane_scratch, 4))
    return ANVIL_ERR_MISALIGNED;
  const size_t cnt = static_cast<size_t>(sh.g) * sh.m * sh.n;
  const size_t lb = static_cast<size_t>(sh.g) * anvil::equalizer_lanes(sh) * 4;
  if (overlap(update, cnt * 2, lane_energy, lb) || overlap(update, cnt * 2, lane_scratch, 2 * lb) ||
      overlap(lane_energy, lb, lane_scratch, 2 * lb))
    return ANVIL_ERR_ALIAS;
  return hip_status(anvil::launch_equalize(update, lane_energy, beta2, lane_scratch, sh,
                                           static_cast<hipStream_t>(stream), nullptr, nullptr,
                                           nullptr, nullptr, 0.0f));
}

int anvil_decay_update(uint16_t* param, uint16_t* mantissa, const uint16_t* update, float eff_wd,
                       const float* eff_lr, const float* gate, int64_t g, int64_t m, int64_t n,
                       void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  if (!param || !mantissa || !update || !eff_lr || !gate) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(param, 16) || !aligned(mantissa, 16) || !aligned(update, 16) || !aligned(gate, 16) ||
      !aligned(eff_lr, 4))
    return ANVIL_ERR_MISALIGNED;
  const size_t cnt = static_cast<size_t>(sh.g) * sh.m * sh.n;
  const void* bufs[4] = {param, mantissa, update, gate};
  const size_t sizes[4] = {cnt * 2, cnt * 2, cnt * 2, cnt * 4};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(bufs[i], sizes[i], bufs[j], sizes[j])) return ANVIL_ERR_ALIAS;
  if (overlap(eff_lr, sh.g * 4, param, cnt * 2) || overlap(eff_lr, sh.g * 4, mantissa, cnt * 2))
    return ANVIL_ERR_ALIAS;
  return hip_status(anvil::launch_decay(param, mantissa, update, eff_wd, eff_lr, gate, sh,
                                        static_cast<hipStream_t>(stream)));
}

int anvil_release_workspaces(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int st = ANVIL_OK;
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_ws) {
    if (!kv.second.first) continue;
    hipError_t e = hipSetDevice(kv.first.first);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipFree(kv.second.first);
    if (e != hipSuccess) st = hip_status(e);
  }
  g_ws.clear();
  if (have_cur) (void)hipSetDevice(cur);
  return st;
}

int anvil_momentum(const float* grad, float* velocity, float momentum, float fast_beta,
                   float fast_weight, uint16_t* x_out, int64_t g, int64_t m, int64_t n,
                   void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  st = check_step_args(grad, 4, velocity, x_out, sh);
  if (st != ANVIL_OK) return st;
  const int64_t count = sh.g * sh.m * sh.n;
  return hip_status(anvil::launch_momentum(grad, velocity, velocity + count, x_out, count,
                                           momentum, fast_beta, fast_weight,
                                           static_cast<hipStream_t>(stream)));
}

int64_t anvil_trace_slots(int64_t m, int64_t n) {
  Shape sh;
  bool empty = false;
  if (check_shape(1, m, n, &sh, &empty) != ANVIL_OK || empty) return 0;
  return anvil::gram_trace_slots(sh);
}

int anvil_gram(const uint16_t* x, uint16_t* a_out, float* trace_partials, int64_t g, int64_t m,
               int64_t n, void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  if (!x || !a_out) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(a_out, 16) || (trace_partials && !aligned(trace_partials, 16)))
    return ANVIL_ERR_MISALIGNED;
  const size_t s = sh.s();
  const size_t xb = static_cast<size_t>(sh.g) * sh.m * sh.n * 2, ab = sh.g * s * s * 2;
  const size_t tb = static_cast<size_t>(sh.g) * anvil::gram_trace_slots(sh) * 4;
  if (overlap(a_out, ab, x, xb) || (trace_partials && (overlap(trace_partials, tb, x, xb) ||
                                                       overlap(trace_partials, tb, a_out, ab))))
    return ANVIL_ERR_ALIAS;
  return hip_status(anvil::launch_gram(x, a_out, trace_partials, sh,
                                       static_cast<hipStream_t>(stream)));
}

int anvil_normalize(uint16_t* x, uint16_t* a, const float* trace_partials, float* d_out,
                    int64_t g, int64_t m, int64_t n, void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  if (!x || !a || !trace_partials) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(a, 16) || !aligned(trace_partials, 4) ||
      (d_out && !aligned(d_out, 4)))
    return ANVIL_ERR_MISALIGNED;
  const size_t s = sh.s();
  const size_t xb = static_cast<size_t>(sh.g) * sh.m * sh.n * 2, ab = sh.g * s * s * 2;
  const size_t tb = static_cast<size_t>(sh.g) * anvil::gram_trace_slots(sh) * 4;
  if (overlap(x, xb, a, ab) || overlap(x, xb, trace_partials, tb) ||
      overlap(a, ab, trace_partials, tb) ||
      (d_out && (overlap(d_out, sh.g * 4, x, xb) || overlap(d_out, sh.g * 4, a, ab) ||
                 overlap(d_out, sh.g * 4, trace_partials, tb))))
    return ANVIL_ERR_ALIAS;
  return hip_status(anvil::launch_normalize(x, a, trace_partials, d_out, sh,
                                            static_cast<hipStream_t>(stream)));
}

int anvil_poly(const uint16_t* a, uint16_t* b_out, float coef_b, float coef_c, int64_t g,
               int64_t s, void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, s, s, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  if (!a || !b_out) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(a, 16) || !aligned(b_out, 16)) return ANVIL_ERR_MISALIGNED;
  const size_t bytes = static_cast<size_t>(sh.g) * s * s * 2;
  if (overlap(a, bytes, b_out, bytes)) return ANVIL_ERR_ALIAS;
  return hip_status(anvil::launch_poly(a, b_out, coef_b, coef_c, sh.g, sh.m,
                                       static_cast<hipStream_t>(stream)));
}

int anvil_apply(const uint16_t* x, const uint16_t* b, uint16_t* c_out, float coef_a, int split,
                int64_t g, int64_t m, int64_t n, void* stream) {
  Shape sh;
  bool empty = false;
  int st = check_shape(g, m, n, &sh, &empty);
  if (st != ANVIL_OK || empty) return st;
  if (!x || !b || !c_out || (split != 0 && split != 1)) return ANVIL_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(b, 16) || !aligned(c_out, 16)) return ANVIL_ERR_MISALIGNED;
  const size_t s = sh.s();
  const size_t xb = static_cast<size_t>(sh.g) * sh.m * sh.n * 2, bb = sh.g * s * s * 2;
  if (overlap(c_out, xb, x, xb) || overlap(c_out, xb, b, bb)) return ANVIL_ERR_ALIAS;
  return hip_status(anvil::launch_apply(x, b, c_out, coef_a, split != 0, sh,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
