/*
 * linattn.h - C ABI of the MI355X (gfx950) causal kernelized linear attention library.
 *
 * The operation (learn.pranaymahendrakar.com page, Researcher level, "Derivation";
 * aicassindra.com page, "The quadratic wall, and the kernel that removes it"):
 *
 *     phi(x) = elu(x) + 1                     (alpha = 1, applied to q and k, never to v)
 *     S_i = S_{i-1} + phi(k_i) v_i^T,  z_i = z_{i-1} + phi(k_i)
 *     o_i = phi(q_i)^T S_i / max(phi(q_i)^T z_i, eps)
 *
 * computed in the chunked parallel form (aiwiki.thehackersbrain.dev page, the
 * chunked listing and its closing paragraph): a causally masked quadratic product
 * inside each chunk of `chunk` tokens, and the state (S, z) carried across chunks.
 * There is no 1/sqrt(D) scaling.  The denominator is clamped to eps, as the chunked
 * listing on that page does.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer is DEVICE memory owned by the caller.  The library never
 *    allocates or frees device memory and keeps no pointer after it returns.
 *  - Tensors are contiguous and row-major.  Base pointers must be 16-byte aligned.
 *  - q, k, v, o hold `dtype` elements (LINATTN_F32: float, LINATTN_BF16: bfloat16
 *    bit patterns).  States (S, z, s0, z0, s_out, z_out) and gates are always float.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null stream).
 *    Results are valid once the stream has synchronised.
 *  - Arguments are checked before anything is launched: a return other than
 *    LINATTN_OK guarantees that no device memory was written.
 *  - B*H*N == 0 (or B*H == 0 for decode) is LINATTN_OK and does nothing.
 *  - NaN or Inf in the inputs propagate to the outputs; they are not trapped.
 *  - Results are bitwise reproducible for identical inputs and shapes (no float atomics).
 *  - Nothing aborts and no C++ exception crosses this interface.
 *
 * Supported shapes on the GPU: D and Dv in {64, 128}; chunk in {32, 64, 128, 256}
 * when the chunk's on-chip tiles fit the 160 KiB LDS of a compute unit.  When the
 * full-width tiles do not fit but 64-column ones do (Dv = 128), the forward walks the
 * value columns as two parts of 64, each with its own workgroups.  That leaves:
 *   bf16: every chunk;
 *   f32:  chunk <= 128 when D = 64, <= 64 when D = 128.
 * Other shapes return LINATTN_ERR_UNSUPPORTED.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LINATTN_OK = 0,
    LINATTN_ERR_INVALID_ARGUMENT = 1,  /* null pointer, negative size, eps <= 0, misalignment */
    LINATTN_ERR_UNSUPPORTED = 2,       /* valid but not built: D/Dv/chunk/dtype combination */
    LINATTN_ERR_WORKSPACE = 3,         /* workspace missing or smaller than linattn_fwd_workspace_size */
    LINATTN_ERR_HIP = 4,               /* no usable device, or a launch failed */
    LINATTN_ERR_SCRATCH_LIMIT = 5      /* linattn_fwd_ex_noalloc: more scratch than its fixed array */
} linattn_status_t;

typedef enum {
    LINATTN_F32 = 0,
    LINATTN_BF16 = 1
} linattn_dtype_t;

/*
 * What o holds (linattn_fwd_ex, linattn_decode_step_ex).  The normaliser-free mode is
 * the output of retention, which drops the phi(q)^T z denominator and leaves the scale
 * to a normalisation layer after the attention (aicassindra.com page, "RetNet and gated
 * linear attention"; learn.pranaymahendrakar.com page, "Implementation reality").
 */
typedef enum {
    LINATTN_OUT_NORMALIZED = 0,   /* o = phi(q)^T S / max(phi(q)^T z, eps) */
    LINATTN_OUT_NUMERATOR = 1     /* o = phi(q)^T S; eps is not used */
} linattn_output_t;

/*
 * Bytes of device scratch the chunked and gated forwards need for these sizes
 * (per-segment state totals and prefixes, float).  0 when B*H*N == 0 or a size is
 * not positive.  The same value serves both forwards.  Its contents are undefined
 * after a call; it must not be shared by calls that may run concurrently.
 */
size_t linattn_fwd_workspace_size(int B, int H, int N, int D, int Dv, int chunk);

/*
 * Chunked forward of causal kernelized linear attention.
 *
 *  q, k   [B,H,N,D]   dtype         input, read-only
 *  v      [B,H,N,Dv]  dtype         input, read-only
 *  o      [B,H,N,Dv]  dtype         output; must not overlap any input, s0 or z0
 *  s0     [B,H,D,Dv]  float or NULL initial state S (NULL: zeros)
 *  z0     [B,H,D]     float or NULL initial normaliser z (NULL: zeros)
 *  s_out  [B,H,D,Dv]  float or NULL final state S_N (NULL: not written); may equal s0
 *  z_out  [B,H,D]     float or NULL final normaliser z_N (NULL: not written); may equal z0
 *                     (s_out and z_out may share memory with s0 and z0, which are read
 *                     before the final state is written, but not with q, k, v, g, o or
 *                     each other: LINATTN_ERR_INVALID_ARGUMENT)
 *  chunk               tokens per chunk (the last chunk of a sequence may be shorter)
 *  eps > 0             denominator clamp: o = num / max(den, eps)
 *  workspace           device scratch of at least linattn_fwd_workspace_size(...) bytes,
 *                      16-byte aligned (NULL allowed only when that size is 0)
 *
 * Resuming: fwd(N1) then fwd(N2) with s0/z0 = the first call's s_out/z_out equals
 * fwd(N1 + N2) up to rounding (aiwiki.thehackersbrain.dev page, "It is a linear RNN":
 * the state is a fixed-size summary of everything seen).
 */
linattn_status_t linattn_fwd_chunked(
    const void* q, const void* k, const void* v, void* o,
    const float* s0, const float* z0, float* s_out, float* z_out,
    int B, int H, int N, int D, int Dv, int chunk, linattn_dtype_t dtype, float eps,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Scalar-gated chunked forward: S_t = g_t S_{t-1} + phi(k_t) v_t^T and
 * z_t = g_t z_{t-1} + phi(k_t), o_t = phi(q_t)^T S_t / max(phi(q_t)^T z_t, eps)
 * (the decay term of the aiwiki.thehackersbrain.dev page, "What is actually lost",
 * with a scalar gate per head and token; the aicassindra.com page, "RetNet and gated
 * linear attention").
 *
 *  g [B,H,N] float, device, read-only.  Precondition (not checked on the device):
 *  0 < g <= 1.  Every other argument is as for linattn_fwd_chunked.
 */
linattn_status_t linattn_fwd_gated(
    const void* q, const void* k, const void* v, const float* g, void* o,
    const float* s0, const float* z0, float* s_out, float* z_out,
    int B, int H, int N, int D, int Dv, int chunk, linattn_dtype_t dtype, float eps,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The general forward: linattn_fwd_chunked when g is NULL, linattn_fwd_gated otherwise,
 * with the output chosen by `out` (LINATTN_OUT_NORMALIZED gives exactly those two calls).
 * In the numerator mode the state recurrence is unchanged: s_out and z_out receive the
 * same S_N and z_N, so a sequence may be resumed in either mode.  An `out` outside the
 * enum is LINATTN_ERR_INVALID_ARGUMENT.  Every other argument is as for
 * linattn_fwd_gated, g [B,H,N] being optional.
 */
linattn_status_t linattn_fwd_ex(
    const void* q, const void* k, const void* v, const float* g, void* o,
    const float* s0, const float* z0, float* s_out, float* z_out,
    int B, int H, int N, int D, int Dv, int chunk, linattn_dtype_t dtype, float eps,
    linattn_output_t out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): linattn_fwd_ex without a workspace.
 * Every argument is as for linattn_fwd_ex, and so are the results, bit for bit (the same
 * kernels on the same plan).  The call allocates and frees nothing.  Its scratch is a
 * fixed array of LINATTN_NOALLOC_SCRATCH_BYTES in device memory, one per device, placed
 * when the library's device code loads on that device and held until the process ends;
 * the first call on a device looks up its address there.
 *  - Shapes whose scratch would exceed the array return LINATTN_ERR_SCRATCH_LIMIT before
 *    anything is launched (linattn_fwd_workspace_size(...) <= LINATTN_NOALLOC_SCRATCH_BYTES
 *    is sufficient for a shape to fit).
 *  - Every call on one device shares that device's array, which keeps the last call's
 *    contents (nothing in it needs to start at zero: a call writes every part it reads).
 *    Calls that may overlap in time on one device (on different streams, or from
 *    different host threads without ordering) race on it; calls on one stream are
 *    ordered and safe.
 *  - Under HIP graph capture: let one call of the same element type, D, Dv, gating and
 *    chunk run on the device first (it looks up the array's address and sets the kernels'
 *    LDS limits, which are not stream work); the captured launches then replay with the
 *    pointers and sizes of the captured call.
 */
#define LINATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

linattn_status_t linattn_fwd_ex_noalloc(
    const void* q, const void* k, const void* v, const float* g, void* o,
    const float* s0, const float* z0, float* s_out, float* z_out,
    int B, int H, int N, int D, int Dv, int chunk, linattn_dtype_t dtype, float eps,
    linattn_output_t out, void* stream);

/*
 * Per-dimension decay (gated linear attention):
 *
 *     S_t = Diag(a_t) S_{t-1} + phi(k_t) v_t^T,   z_t = a_t * z_{t-1} + phi(k_t),
 *     o_t = S_t^T phi(q_t) / max(phi(q_t) . z_t, eps)   (or the numerator, `out`)
 *
 * (aicassindra.com page, "RetNet and gated linear attention": S_i = Diag(alpha_i) S_{i-1}
 * + k_i v_i^T; aiwiki.thehackersbrain.dev page, "What is actually lost": an elementwise
 * decay G_t of S_{t-1}, here G_t[d, e] = a_t[d]; z decays alike).
 *
 *  a  [B,H,N,D] float, device, read-only.  Precondition (not checked on the device):
 *     2^-8 <= a <= 1 (within a 16-token block the rescaled operands of the chunk products
 *     stay below 2^64).
 *  Every other argument is as for linattn_fwd_ex; the workspace is sized by
 *  linattn_fwd_vdecay_workspace_size (room for the state after every 64-token chunk).
 *  Supported shapes: D, Dv in {64, 128}; bf16 at every pair, f32 unless D = Dv = 128
 *  (LINATTN_ERR_UNSUPPORTED).
 */
size_t linattn_fwd_vdecay_workspace_size(int B, int H, int N, int D, int Dv);

linattn_status_t linattn_fwd_vdecay(
    const void* q, const void* k, const void* v, const float* a, void* o,
    const float* s0, const float* z0, float* s_out, float* z_out,
    int B, int H, int N, int D, int Dv, linattn_dtype_t dtype, float eps, linattn_output_t out,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step under the per-dimension decay: S <- Diag(a) S + phi(k) v^T,
 * z <- a * z + phi(k), then o as chosen by `out`; a [B,H,D] float is this token's decay,
 * 0 < a <= 1, and must not overlap S, z or o.  Every other argument is as for
 * linattn_decode_step_ex (z may be NULL without the denominator).
 */
linattn_status_t linattn_decode_step_vdecay(
    const void* q, const void* k, const void* v, const float* a, float* S, float* z, void* o,
    int B, int H, int D, int Dv, linattn_dtype_t dtype, float eps, linattn_output_t out, void* stream);

/*
 * Feature maps other than elu + 1 (the forward of linattn_fwd_ex with phi replaced):
 *   LINATTN_FEATURE_RELU   phi(x) = max(x, 0) + shift, M = D (the "F.relu(x) + eps"
 *                          alternative of the anandmoghan-problems page, "Key Functions
 *                          & Tricks"); W must be NULL
 *   LINATTN_FEATURE_FAVOR  phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(M) for the M rows of
 *                          W [H][M][D] float (one set of random features per head, drawn
 *                          by the caller), Performer's positive random features
 *                          (aicassindra.com page, "Performer: unbiased softmax by
 *                          positive random features"); shift is not used
 * The state then has M rows: s0, s_out [B,H,M,Dv], z0, z_out [B,H,M].  The features are
 * computed in a pass of their own into the workspace (linattn_fwd_features_workspace_size),
 * then the chunked walk runs over them.  Supported: D, M, Dv in {64, 128}; chunk 64 or
 * 128 (where the walk's tiles fit the LDS).  Every other argument is as for linattn_fwd_ex.
 * A decode step under these maps is this call over one token (N = 1) with s_out = s0 and
 * z_out = z0: the state is updated in place.
 */
typedef enum {
    LINATTN_FEATURE_RELU = 1,
    LINATTN_FEATURE_FAVOR = 2
} linattn_feature_t;

size_t linattn_fwd_features_workspace_size(int B, int H, int N, int D, int Dv, int chunk, int M,
                                           linattn_dtype_t dtype);

linattn_status_t linattn_fwd_features(
    const void* q, const void* k, const void* v, const float* g, void* o,
    const float* s0, const float* z0, float* s_out, float* z_out,
    int B, int H, int N, int D, int Dv, int chunk, linattn_dtype_t dtype, float eps, linattn_output_t out,
    linattn_feature_t feature, float shift, const float* W, int M,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device scratch linattn_bwd needs for these sizes and dtype (room for the
 * state in front of every run of 64-token chunks and its adjoint, float, at any run
 * length, plus per-token intermediates).
 * 0 when B*H*N == 0 or a size is not positive.  Contents are undefined after a call; it
 * must not be shared by calls that may run concurrently.
 */
size_t linattn_bwd_workspace_size(int B, int H, int N, int D, int Dv, linattn_dtype_t dtype);

/*
 * Gradients of the forward (linattn_fwd_ex with the same g, s0, z0, eps and `out`) for
 * the loss sum(dout * o): the reverse-mode derivative of the recurrence
 * S_t = g_t S_{t-1} + phi(k_t) v_t^T, z alike, o_t as chosen by `out` (learn.pranaymahendrakar.com
 * page, "Derivation" and "Try it yourself"; the chunked form is the training path, as
 * the aiwiki.thehackersbrain.dev page's chunked listing and the learn page's
 * "Implementation reality" say).  The clamp max(den, eps) passes no gradient where
 * den < eps.  The chunking is the library's own (64 tokens); results do not depend on
 * the forward's chunk.
 *
 *  q, k [B,H,N,D], v [B,H,N,Dv], dout [B,H,N,Dv]   dtype, read-only
 *  g    [B,H,N] float or NULL                      as for the forward
 *  s0   [B,H,D,Dv], z0 [B,H,D] float or NULL       the forward's initial state
 *  dq, dk [B,H,N,D], dv [B,H,N,Dv]                 dtype, written; must not alias any input
 *  dg   [B,H,N] float or NULL                      written when g is given (NULL: skipped)
 *  ds0  [B,H,D,Dv], dz0 [B,H,D] float or NULL      gradients of the initial state (NULL: skipped)
 *  run                                             chunks per run, >= 0: the passes walk runs of
 *                                                  this many chunks and carry the states through
 *                                                  them; 0 lets the library choose from the
 *                                                  device's size (values past the chunk count
 *                                                  act as the chunk count).  The results differ
 *                                                  between choices only by rounding.
 *  workspace                                       at least linattn_bwd_workspace_size bytes
 *
 * Supported shapes: D, Dv in {64, 128}; bf16 at every pair, f32 unless D = Dv = 128
 * (LINATTN_ERR_UNSUPPORTED).  Every other convention is the forward's.
 */
linattn_status_t linattn_bwd(
    const void* q, const void* k, const void* v, const float* g, const void* dout,
    const float* s0, const float* z0, void* dq, void* dk, void* dv, float* dg, float* ds0, float* dz0,
    int B, int H, int N, int D, int Dv, linattn_dtype_t dtype, float eps, linattn_output_t out,
    int run, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step for B*H independent heads (aiwiki.thehackersbrain.dev page,
 * "It is a linear RNN": O(D*Dv) work per token, no cache that grows):
 *
 *     S <- S + phi(k) v^T,  z <- z + phi(k),  o = phi(q)^T S / max(phi(q)^T z, eps)
 *
 * The token is added before it is read (mlblogg.com page, "The causal recurrence").
 *
 *  q, k  [B,H,D]     dtype   read-only
 *  v     [B,H,Dv]    dtype   read-only
 *  S     [B,H,D,Dv]  float   updated in place
 *  z     [B,H,D]     float   updated in place
 *  o     [B,H,Dv]    dtype   output; must not alias any other argument
 */
linattn_status_t linattn_decode_step(
    const void* q, const void* k, const void* v, float* S, float* z, void* o,
    int B, int H, int D, int Dv, linattn_dtype_t dtype, float eps, void* stream);

/*
 * The general decode step: the gated recurrence of linattn_fwd_gated for one token,
 *
 *     S <- g S + phi(k) v^T,  z <- g z + phi(k),  then o as chosen by `out`,
 *
 * the recurrent form of the gated forward (aicassindra.com page, "Linear Transformer:
 * elu+1 and the RNN in disguise": the parallel form for training, the recurrence for
 * generation; "RetNet and gated linear attention": S_i = gamma S_{i-1} + k_i v_i^T).
 *
 *  g  [B,H]  float or NULL  this token's gate per head, 0 < g <= 1 (not checked on the
 *                           device); NULL means 1 and gives exactly linattn_decode_step
 *  z  [B,H,D] float         updated in place; may be NULL only with LINATTN_OUT_NUMERATOR,
 *                           and is then neither read nor written
 *  out                      LINATTN_OUT_NORMALIZED or LINATTN_OUT_NUMERATOR
 * Every other argument is as for linattn_decode_step; g must not overlap S, z or o.
 */
linattn_status_t linattn_decode_step_ex(
    const void* q, const void* k, const void* v, const float* g, float* S, float* z, void* o,
    int B, int H, int D, int Dv, linattn_dtype_t dtype, float eps, linattn_output_t out, void* stream);

/*
 * Measurement hook, not part of the computation.  Arms the NEXT linattn_fwd_chunked or
 * linattn_fwd_gated call on this process to record caller-created hipEvent_t handles on
 * its stream: ev0 before the segment-totals walk, ev1 after it, ev2 after the scan over
 * segments, ev3 after the output walk and, when s_out or z_out is given, the final-state
 * copy (a step that a shape does not need is skipped, so its two events bracket
 * nothing).  NULL handles are not recorded; every event recorded sits between dependent
 * launches and delays the next one by a few microseconds.  The first forward whose
 * arguments pass validation consumes (and disarms) the hook; four NULLs disarm it.
 * Always returns LINATTN_OK.
 */
linattn_status_t linattn_set_profile_events(void* ev0, void* ev1, void* ev2, void* ev3);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* linattn_status_string(linattn_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
