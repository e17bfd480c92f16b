// Host-side launchers of the ANVIL kernels (internal to libanvil.so).  Arguments are checked by
// the C ABI layer before these are called; each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace anvil {

// Fused twin-rail momentum + bf16 cast over `count` elements (count % 8 == 0).
hipError_t launch_momentum(const float* grad, float* v0, float* v1, uint16_t* x, int64_t count,
                           float momentum, float fast_beta, float fast_weight, hipStream_t stream);

// The same with the gradient fp32 or bf16 and (momentum, fast_beta, fast_weight) read from a
// device array when the kernel runs.
hipError_t launch_momentum_dev(const void* grad, bool grad_bf16, float* v0, float* v1,
                               uint16_t* x, int64_t count, const float* scalars,
                               hipStream_t stream);

// Geometry of one bank: stack g of m x n matrices.
struct Shape {
  int64_t g;
  int m, n;
  bool tall() const { return m > n; }
  int s() const { return m > n ? n : m; }
  int L() const { return m > n ? m : n; }
};

// Trace partials per matrix that launch_gram writes: one per 32-row diagonal block for wide or
// square shapes with s <= 256, else one per 128-row diagonal tile.
int gram_trace_slots(const Shape& sh);

hipError_t launch_gram(const uint16_t* x, uint16_t* a, float* trace_partials, const Shape& sh,
                       hipStream_t stream);
hipError_t launch_normalize(uint16_t* x, uint16_t* a, const float* trace_partials, float* d,
                            const Shape& sh, hipStream_t stream);
hipError_t launch_poly(const uint16_t* a, uint16_t* b, float coef_b, float coef_c, int64_t g,
                       int s, hipStream_t stream);
hipError_t launch_apply(const uint16_t* x, const uint16_t* b, uint16_t* c, float coef_a,
                        bool split, const Shape& sh, hipStream_t stream);
// Polynomial and apply of one map in a single launch (C = a X + B X with B = b A + c A·A formed
// per tile), for wide or square shapes with s <= 256 whose tiles of 32 rows by 1, 2, 3 or 6
// chunks of 128 columns fit one round on the CUs; the same arithmetic as launch_poly followed by
// launch_apply, element for element.
bool poly_apply_fused(const Shape& sh);
hipError_t launch_poly_apply(const uint16_t* a, const uint16_t* x, uint16_t* c, float coef_a,
                             float coef_b, float coef_c, const Shape& sh, hipStream_t stream);

// Equalizer lanes of an m x n matrix: rows when m >= n, else columns.
int equalizer_lanes(const Shape& sh);

// Equalizer on u (in place) with lane energies updated in place; scratch holds 2*g*lanes fp32.
// If param is not null, the same elementwise pass applies the sign-aligned decay to
// (param, mantissa) with the rescaled u, gate (the slow rail), per-matrix lr and wd (or wd read
// from the device at *wd_dev when that is not null).
hipError_t launch_equalize(uint16_t* u, float* lane_energy, double beta2, float* scratch,
                           const Shape& sh, hipStream_t stream, uint16_t* param,
                           uint16_t* mantissa, const float* gate, const float* lr, float wd,
                           const float* wd_dev = nullptr);

// The sign-aligned decay alone, with u as given.
hipError_t launch_decay(uint16_t* param, uint16_t* mantissa, const uint16_t* u, float wd,
                        const float* lr, const float* gate, const Shape& sh, hipStream_t stream);

}  // namespace anvil
