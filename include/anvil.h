/*
 * anvil.h — C ABI of the MI355X (gfx950) ANVIL bank-step library, libanvil.so.
 *
 * The ANVIL bank step (modded-nanogpt, track_1_short/optim/anvil.py, function `anvil_cascade`)
 * turns the gradient of a stack of same-shape projection matrices into an orthogonalised update:
 *
 *   1. twin-rail momentum in fp32: the fast rail lerps toward the gradient with weight
 *      1 - fast_beta, the slow rail with weight 1 - 0.98; the rails are blended as
 *      w * fast + (1 - w) * slow (w = fast_weight), and the gradient is lerped toward the blend
 *      with weight `momentum` (a Nesterov lookahead).  Every lerp is torch's, which the page
 *      calls: the difference of the end points, then one fused multiply-add about the nearer
 *      end point (fma(w, end - start, start) for |w| < 1/2, else fma(w - 1, end - start, end));
 *   2. the lookahead is rounded to bf16, X;
 *   3. the Gram A = X^T X (rows > cols, "tall") or X X^T (otherwise) is formed in bf16; the trace
 *      of its bf16 diagonal is ||X||_F^2, giving d = sqrt(trace) * 1.05 + 1e-6; X and A are
 *      replaced by bf16(X / d) and bf16(A / d^2);
 *   4. six quintic maps (a_k, b_k, c_k) follow: B = b A + c A A, then X <- a X + X B (tall) or
 *      a X + B X (wide); every map after the first recomputes A from the current X.  Banks with
 *      more than 1024 rows round X B (or B X) to bf16 before adding a X (the page's two-kernel
 *      form); the others round once.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers to contiguous row-major data on the current HIP device.
 *     bf16 tensors are passed as their uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue work and return;
 *     kernel faults surface at the caller's next synchronisation.  The exception is the cached
 *     workspace of the entry points that take no workspace (anvil_bank_step, anvil_bank_update,
 *     and anvil_bank_step_maps / anvil_bank_update_ws with a NULL workspace): the first call for
 *     a shape larger than the cached buffer allocates (hipMalloc) and, when it replaces an older
 *     buffer, synchronises the stream before freeing it.  Those calls therefore cannot be
 *     captured into a HIP graph: on a capturing stream they return ANVIL_ERR_CAPTURING without
 *     enqueueing anything.  Every entry point that takes a caller workspace allocates nothing,
 *     never synchronises and may be captured.
 *   - g, m, n: stack size and matrix shape.  Any of them 0 means an empty stack: the call returns
 *     ANVIL_OK without touching memory (pointers may then be NULL).  Negative sizes are
 *     ANVIL_ERR_INVALID_ARG.  m and n must be multiples of 8 (16-byte rows), m*n <= 2^30,
 *     g <= 65535 and g*m*n <= 2^35, else ANVIL_ERR_UNSUPPORTED.
 *   - Pointers must be 16-byte aligned (ANVIL_ERR_MISALIGNED).  Outputs may not overlap inputs
 *     (ANVIL_ERR_ALIAS), except where an argument is documented as in-place.
 *   - The caller owns every buffer.  The library owns only the workspaces cached by
 *     anvil_bank_step (released by anvil_release_workspaces).
 *   - No exception crosses the ABI.  NaN and Inf in the data propagate; nothing checks them.
 *   - Thread safety: calls are safe from several threads; the cached workspace is per
 *     (device, stream), so calls on different streams do not share scratch memory, and calls that
 *     use the cache hold its lock while they enqueue (their enqueues take turns).
 */
#ifndef ANVIL_H_
#define ANVIL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum anvil_status {
  ANVIL_OK = 0,
  ANVIL_ERR_INVALID_ARG = 1, /* NULL pointer for a non-empty call, negative size, bad flag */
  ANVIL_ERR_UNSUPPORTED = 2, /* shape outside the supported set, or workspace too small */
  ANVIL_ERR_MISALIGNED = 3,  /* a pointer is not 16-byte aligned */
  ANVIL_ERR_ALIAS = 4,       /* an output overlaps an input it may not overlap */
  ANVIL_ERR_OOM = 5,         /* the workspace allocation failed */
  ANVIL_ERR_HIP = 6,         /* a HIP API or launch error; see anvil_last_hip_error() */
  ANVIL_ERR_CAPTURING = 7,   /* a cached-workspace call on a stream that is being captured */
  ANVIL_ERR_TOO_LARGE = 8    /* anvil_bank_step_noalloc: the step needs more than its scratch */
};

/* Gradient element types of the device-scalar entry points. */
enum anvil_grad_dtype {
  ANVIL_GRAD_F32 = 0,  /* fp32 [g, m, n] */
  ANVIL_GRAD_BF16 = 1  /* bf16 bits [g, m, n]; widened to fp32 exactly before the rail lerps */
};

/* Static, NUL-terminated description of a status code. */
const char* anvil_status_string(int status);

/* The hipError_t of the most recent ANVIL_ERR_HIP returned on the calling thread (0 if none). */
int anvil_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int anvil_version(void);

/*
 * One ANVIL bank step (anvil.py, `anvil_cascade`, momentum block plus tall or wide branch).
 *
 *   grad        fp32 [g, m, n], read only.
 *   velocity    fp32 [2, g, m, n], updated in place: rail 0 (fast) at offset 0, rail 1 (slow) at
 *               offset g*m*n.
 *   momentum    Nesterov weight of the lookahead (0.95 in the source's schedule).
 *   fast_beta   the fast rail's beta (0.85); its lerp weight is the fp32 value 1.0f - fast_beta.
 *   fast_weight the fast rail's share of the blend (1.0 before the engage step, 0.4385 after).
 *   out         bf16 [g, m, n]: receives the orthogonalised update.  It also serves as one of the
 *               two ping-pong buffers of the cascade, so it may not overlap grad or velocity.
 *
 * Uses a workspace of anvil_workspace_bytes(g, m, n) bytes cached per (device, stream); the first
 * call for a larger shape allocates it (ANVIL_ERR_OOM if that fails).
 */
int anvil_bank_step(const float* grad, float* velocity, float momentum, float fast_beta,
                    float fast_weight, uint16_t* out, int64_t g, int64_t m, int64_t n,
                    void* stream);

/* As anvil_bank_step, with a caller-owned device workspace of at least
 * anvil_workspace_bytes(g, m, n) bytes, 256-byte aligned (ANVIL_ERR_UNSUPPORTED if smaller,
 * ANVIL_ERR_MISALIGNED if not aligned).  No allocation happens.  The workspace may not overlap
 * any other argument; two calls in flight at once need two workspaces. */
int anvil_bank_step_ws(const float* grad, float* velocity, float momentum, float fast_beta,
                       float fast_weight, uint16_t* out, int64_t g, int64_t m, int64_t n,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch that anvil_bank_step_noalloc holds per device (192 MiB: every bank of
 * the qk, vo, mlp, Vs and Us shapes fits, the largest, 32 x 4096 x 512, needs 161 MiB). */
#define ANVIL_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)

/* As anvil_bank_step, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The workspace is a device
 * array of ANVIL_NOALLOC_SCRATCH_BYTES compiled into the library, one per device, held until the
 * process ends; the call allocates nothing and never synchronises.  A bank whose
 * anvil_workspace_bytes(g, m, n) exceeds ANVIL_NOALLOC_SCRATCH_BYTES is refused with
 * ANVIL_ERR_TOO_LARGE before anything is enqueued.  Every call on a device shares that device's
 * scratch: calls that may overlap in time on one device (other streams, other threads) race and
 * must be ordered by the caller.  The first call on a device looks up the scratch's address
 * (hipGetSymbolAddress), so make it outside graph capture. */
int anvil_bank_step_noalloc(const float* grad, float* velocity, float momentum, float fast_beta,
                            float fast_weight, uint16_t* out, int64_t g, int64_t m, int64_t n,
                            void* stream);

/* The bank step with a caller-chosen table of quintic maps (the page's cascade loop with another
 * coefficient list and step count, e.g. a plain quintic Newton-Schulz iteration).
 *   maps        HOST array of `steps` triples (a, b, c), fp32, applied in order exactly as the
 *               six ANVIL maps are: B = b A + c A A, then X <- a X + X B (tall) or a X + B X.
 *   steps       1 .. 16 (else ANVIL_ERR_INVALID_ARG).
 *   workspace   a caller workspace as for anvil_bank_step_ws, or NULL for the cached one.
 * With the ANVIL table and steps = 6 the result is identical to anvil_bank_step. */
int anvil_bank_step_maps(const float* grad, float* velocity, float momentum, float fast_beta,
                         float fast_weight, const float* maps, int steps, uint16_t* out,
                         int64_t g, int64_t m, int64_t n, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Workspace bytes for a [g, m, n] bank step or bank update (0 for an empty stack, or for
 * unsupported sizes). */
size_t anvil_workspace_bytes(int64_t g, int64_t m, int64_t n);

/* Frees every cached workspace on every device.  Synchronises each device first. */
int anvil_release_workspaces(void);

/* ------------------------------------------------------------------------------------------
 * Stage entry points.  They launch the same kernels anvil_bank_step launches, one stage at a
 * time, for per-stage parity tests and per-kernel profiles.  s = min(m, n) is the Gram size;
 * "tall" means m > n.
 * ------------------------------------------------------------------------------------------ */

/* Momentum and bf16 cast (step 1-2 above).  grad fp32 [g,m,n] read only; velocity fp32
 * [2,g,m,n] in place; x_out bf16 [g,m,n]. */
int anvil_momentum(const float* grad, float* velocity, float momentum, float fast_beta,
                   float fast_weight, uint16_t* x_out, int64_t g, int64_t m, int64_t n,
                   void* stream);

/* Number of fp32 trace partials per matrix that anvil_gram writes for shape m x n: one per
 * 32-row block of the Gram's diagonal when min(m, n) <= 256 and m <= n, else one per 128-row
 * block (0 for an unsupported shape). */
int64_t anvil_trace_slots(int64_t m, int64_t n);

/* Gram (step 3): a_out bf16 [g,s,s] = bf16(X^T X) if tall else bf16(X X^T), fp32 accumulation,
 * stored exactly symmetric.  If trace_partials is not NULL (fp32 [g, anvil_trace_slots(m,n)]),
 * it receives partial sums of the bf16-rounded diagonal; their sum in slot order is the trace. */
int anvil_gram(const uint16_t* x, uint16_t* a_out, float* trace_partials, int64_t g, int64_t m,
               int64_t n, void* stream);

/* Frobenius normalisation (step 3): from the trace partials, d = sqrt(trace) * 1.05f + 1e-6f
 * (fp32; written to d_out fp32 [g] when d_out is not NULL), then x <- bf16(x / d) and
 * a <- bf16(a / (d*d)), both IN PLACE.  x bf16 [g,m,n], a bf16 [g,s,s]. */
int anvil_normalize(uint16_t* x, uint16_t* a, const float* trace_partials, float* d_out,
                    int64_t g, int64_t m, int64_t n, void* stream);

/* Polynomial (step 4): b_out bf16 [g,s,s] = bf16(coef_b * A + coef_c * (A A)), the product in
 * fp32; A must be symmetric (as anvil_gram stores it).  b_out is stored exactly symmetric. */
int anvil_poly(const uint16_t* a, uint16_t* b_out, float coef_b, float coef_c, int64_t g,
               int64_t s, void* stream);

/* Apply (step 4): c_out bf16 [g,m,n] = coef_a X + X B (tall) or coef_a X + B X (wide), with
 * B bf16 [g,s,s] symmetric.  split = 0: one rounding of the fp32 sum; split = 1: the product is
 * rounded to bf16 first and coef_a X is added to it in fp32.  c_out may not overlap x or b. */
int anvil_apply(const uint16_t* x, const uint16_t* b, uint16_t* c_out, float coef_a, int split,
                int64_t g, int64_t m, int64_t n, void* stream);

/* ------------------------------------------------------------------------------------------
 * The rest of the bank update (anvil.py, `_rail_equalizer`, `_sign_aligned_decay_update`,
 * `anvil_bank_update`).
 *
 * Equalizer lanes: one per row when m >= n (the equalizer reduces over the columns), else one
 * per column (reducing over the rows); lanes = anvil_equalizer_lanes(m, n), lane length = the
 * other dimension.  Per matrix, in fp32: power = mean over the lane of u^2; pre = sqrt(sum of
 * power * length); energy += (1 - beta2) * (power - energy) (1 - beta2 formed in double, then
 * taken as fp32); gain = 1/sqrt(max(energy, 1e-10)); post = sqrt(sum of (power * length) *
 * gain^2); scale = bf16(gain * (pre / max(post, 1e-10))); u <- bf16(u * scale).
 *
 * Decay: the fp32 master is (param bits << 16) | mantissa; where gate * master >= 0 (gate: the
 * slow rail) it decays: master <- (master - ((master * aligned) * eff_wd) * eff_lr[matrix]) -
 * u * eff_lr[matrix]; the new param bits are its high half (truncation), the mantissa its low
 * half.
 * ------------------------------------------------------------------------------------------ */

/* One whole bank update: anvil_bank_step into `update`, then the equalizer (update rewritten in
 * place with the equalized values, lane_energy updated in place), then the decay of
 * (param, mantissa) gated on the slow rail this call has just written.
 *   update       bf16 [g,m,n] out (also the cascade's ping-pong buffer)
 *   lane_energy  fp32 [g, lanes] in/out (the page's [g,m,1] or [g,1,n])
 *   beta2        the energy EMA's decay, a double (a Python float on the page); the lerp
 *                weight is fp32(1 - beta2) with the subtraction in double
 *   param        bf16 bits [g,m,n] in/out; mantissa uint16 [g,m,n] in/out
 *   eff_wd       decay factor (wd_mul * weight_decay * lr on the page); eff_lr fp32 [g] device
 * No two of grad, velocity, update, lane_energy, param, mantissa, eff_lr may overlap.  Uses the
 * cached workspace (anvil_workspace_bytes covers it). */
int anvil_bank_update(const float* grad, float* velocity, float momentum, float fast_beta,
                      float fast_weight, uint16_t* update, float* lane_energy, double beta2,
                      uint16_t* param, uint16_t* mantissa, float eff_wd, const float* eff_lr,
                      int64_t g, int64_t m, int64_t n, void* stream);

/* As anvil_bank_update with a caller-owned workspace (anvil_workspace_bytes(g, m, n) bytes,
 * 256-byte aligned); allocates nothing. */
int anvil_bank_update_ws(const float* grad, float* velocity, float momentum, float fast_beta,
                         float fast_weight, uint16_t* update, float* lane_energy, double beta2,
                         uint16_t* param, uint16_t* mantissa, float eff_wd, const float* eff_lr,
                         int64_t g, int64_t m, int64_t n, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Equalizer lanes per matrix for shape m x n (0 for unsupported shapes). */
int64_t anvil_equalizer_lanes(int64_t m, int64_t n);

/* The equalizer alone: update bf16 [g,m,n] rescaled IN PLACE, lane_energy fp32 [g, lanes]
 * updated in place; lane_scratch fp32 [2*g*lanes] is overwritten (lane powers and scales). */
int anvil_equalize(uint16_t* update, float* lane_energy, double beta2, float* lane_scratch,
                   int64_t g, int64_t m, int64_t n, void* stream);

/* The decay alone: (param, mantissa) updated in place from update bf16 [g,m,n] read only, gate
 * fp32 [g,m,n] read only, eff_lr fp32 [g]. */
int anvil_decay_update(uint16_t* param, uint16_t* mantissa, const uint16_t* update, float eff_wd,
                       const float* eff_lr, const float* gate, int64_t g, int64_t m, int64_t n,
                       void* stream);

/* ------------------------------------------------------------------------------------------
 * The page's bank contract (anvil.py, `AnvilBank` and `anvil_bank_update`): a bf16 (or fp32)
 * gradient, the per-step scalars as device values read when the kernels run, fixed caller
 * buffers and a caller workspace.  These calls allocate nothing, never synchronise and read no
 * device value on the host, so a sequence of them can be captured into a HIP graph and replayed
 * with new gradients and scalars written into the same buffers between replays.  The first call
 * for a given shape must run outside capture (it sets kernel attributes once).
 *
 *   grad        fp32 or bf16 [g, m, n] per grad_dtype (enum anvil_grad_dtype), read only.
 *   scalars     DEVICE fp32 array: [0] momentum, [1] fast_beta, [2] fast_weight, and for the
 *               update [3] eff_wd; the caller refreshes it (one host-to-device copy per step).
 *   workspace   required (anvil_workspace_bytes(g, m, n) bytes, 256-byte aligned).
 * Everything else as in anvil_bank_step / anvil_bank_update.
 * ------------------------------------------------------------------------------------------ */
int anvil_bank_step_dev(const void* grad, int grad_dtype, float* velocity, const float* scalars,
                        uint16_t* out, int64_t g, int64_t m, int64_t n, void* workspace,
                        size_t workspace_bytes, void* stream);

int anvil_bank_update_dev(const void* grad, int grad_dtype, float* velocity,
                          const float* scalars, uint16_t* update, float* lane_energy,
                          double beta2, uint16_t* param, uint16_t* mantissa,
                          const float* eff_lr, int64_t g, int64_t m, int64_t n, void* workspace,
                          size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ANVIL_H_ */
