/*
 * ob.h — C ABI of the 1-bit Adam compression-phase step on one AMD Instinct
 * MI355X (gfx950).
 *
 * The method: the nubint.ai review of "1-bit Adam: Communication Efficient
 * Large-Scale Training with Adam's Convergence Speed" (Tang, Gan et al.),
 * called "the 1-bit Adam review" in the Source line of each declaration.
 * After a full-precision Adam warmup, Adam's variance is frozen and used as a
 * fixed preconditioner (Abstract; Proposed method, bullet 2), and training
 * continues as momentum SGD whose momentum is exchanged with 1-bit
 * error-compensated compression (One-line summary; Proposed method, bullets
 * 1 and 3).  The review's system exchanges the compressed messages with
 * custom collectives (Proposed method, bullet 4).  Here all W workers'
 * buffers live in one GPU's HBM and the exchange is a local reduction over
 * the W packed messages.  Declared below with their sources as well: the
 * warmup phase and the switch to compression, a partitioned server, a
 * layer-wise trust ratio, and ScaleCom's cyclic local top-k codec.
 *
 * Arithmetic (the pages give no formulas; these are the readings taken):
 *   c1 = fp32(beta1), c2 = fp32(1 - beta1) (complement in double, rounded once)
 *   worker w, element i of tensor t (every fp32 operation rounded once, no FMA):
 *     x        = (c1*m[i] + c2*g_w[i]) + e_w[i]
 *     bit      = x >= 0            (+0 and -0 give 1, NaN gives 0)
 *     s_w,t    = fp32( sqrt( fl64(sum over tensor t of x^2) / n_t ) )
 *     e_w[i]   = bit ? x - s_w,t : x + s_w,t
 *   server:
 *     y        = (sum over w = 0..W-1, ascending, from +0, of (bit_w ? s_w,t : -s_w,t)) / W
 *     z        = y + e_s[i];  bit_s = z >= 0;  s_s,t as above over z
 *     e_s[i]   = bit_s ? z - s_s,t : z + s_s,t
 *   update:
 *     m[i]     = bit_s ? s_s,t : -s_s,t
 *     p[i]     = p[i] - lr * (m[i] / (sqrt(v[i]) + eps))   (correctly rounded sqrt and /)
 *   A tensor holding a non-finite x (or z) gets a NaN scale.
 *
 * Layout.  T tensors with n_t >= 1 elements.  Every flat buffer uses the same
 * padded layout: tensor t occupies elements [off[t], off[t] + n_t) with
 * off[0] = 0 and off[t+1] = off[t] + 64*ceil(n_t/64); N = off[T].  Elements in
 * [off[t] + n_t, off[t+1]) are padding: never read, never written.
 * Per-worker buffers are [W][N] with row stride N.  A packed sign message is
 * uint64 words, Nw = N/64 per worker: word j, bit k holds element 64*j + k;
 * each tensor starts on a word; bits past a tensor's end are written as 0.
 * Scales are fp32: scale_w is [W][T] (row stride T), scale_s is [S]: one
 * per tensor (S = T) unless the server is partitioned (ob_set_server_chunks).
 *
 * Ownership.  The caller owns every buffer passed in: device memory (HBM)
 * pointers, each aligned to 16 bytes.  The library owns only the context and
 * its scratch: a tile table, server-piece tables and partial sums per tile
 * and, for the residual worker pass, per 1024-element chunk (allocated in
 * ob_init), and the CLT-k codec's
 * histograms, candidate lists, masks and per-tile counts (allocated in
 * ob_cltk_configure); ob_destroy frees both.
 *
 * Streams.  Every device call enqueues its kernels on the given stream (a
 * hipStream_t; NULL means the null stream) and returns without waiting.  A
 * context's scratch lives on the device that was current at ob_init: later
 * calls must pass buffers and a stream of that device, with it current.
 * Results are visible to later work on that stream.  Concurrent calls on one
 * context from several host threads, or on several streams at once, race on
 * the context's scratch and are not allowed.
 *
 * Errors.  Calls return OB_OK or an ob_status code.  Argument errors are
 * detected before anything is enqueued.  A failed launch returns
 * OB_ERR_DEVICE; faults inside a kernel surface at the caller's next
 * synchronization with the stream.
 */
#ifndef OB_H
#define OB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ob_ctx ob_ctx;

typedef enum {
  OB_OK = 0,
  OB_ERR_INVALID = 1,   /* null pointer, bad count, bad range, non-finite hyper-parameter */
  OB_ERR_ALIGN = 2,     /* a device pointer not aligned to 16 bytes */
  OB_ERR_NOMEM = 3,     /* device or host allocation failed */
  OB_ERR_DEVICE = 4,    /* a HIP runtime call or kernel launch failed */
  OB_ERR_SCRATCH = 5    /* the list needs more than ob_step_residual_noalloc's static scratch */
} ob_status;

typedef enum {
  OB_GRAD_F32 = 0,      /* gradients are IEEE binary32 */
  OB_GRAD_BF16 = 1      /* gradients are bfloat16 (widened exactly to fp32) */
} ob_grad_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char *ob_status_string(int status);

/* Host only (no device access).  Fills elem_off[0..T] with the padded layout
 * described above for numel[0..T-1].  Returns OB_ERR_INVALID if T < 1, a
 * pointer is NULL or some numel[t] is < 1 or > 2^40. */
int ob_layout(int32_t num_tensors, const int64_t *numel, int64_t *elem_off);

/* Source: the 1-bit Adam review, Proposed method, bullets 1 and 2: after the
 * Adam warmup the optimizer is momentum SGD (momentum coefficient beta1)
 * preconditioned by the frozen variance (eps in the denominator).  The flat
 * tensor list and its layout are this library's.
 *
 * Creates a context for T tensors of numel[] elements (host array, copied),
 * 1 <= W <= 4096 simulated workers, gradients of grad_dtype, and the fixed
 * hyper-parameters beta1 (momentum, in [0, 1)) and eps (> 0 also once rounded
 * to fp32, the precision the kernels use it in).  Allocates the
 * context's device scratch on the current HIP device and uploads its tables
 * with synchronous copies.  OB_ERR_INVALID also when a launch over the list
 * would exceed the device's grid limit (2^32 - 1 work-items, i.e. 16,777,215
 * workgroups of 256): the (worker group, tile) grid of 8192-element tiles,
 * the 1024-element chunks of the residual worker pass, or one workgroup per
 * (worker, tensor) for the scales.  OB_ERR_NOMEM when the
 * scratch cannot be allocated.  Blocking calls of this library: ob_init,
 * ob_destroy, ob_set_server_chunks, ob_cltk_configure and ob_profile_read;
 * every other call only enqueues work on the given stream. */
int ob_init(ob_ctx **out, int32_t num_tensors, const int64_t *numel, int32_t num_workers,
            int32_t grad_dtype, double beta1, double eps);

/* Frees the context and its scratch (waits for the device as hipFree does).
 * NULL is ignored. */
void ob_destroy(ob_ctx *ctx);

/* Source: the 1-bit Adam review, Proposed method, bullet 3 (error-compensated
 * compression applied to the momentum, not the gradient), Abstract (error
 * compensation keeps convergence robust under 1-bit compression) and One-line
 * summary (1-bit compression).  The scale ||x||_2/sqrt(n) and the bit layout
 * are readings: the pages give no formula.
 *
 * Workers [w_begin, w_end) ⊆ [0, W): momentum, error feedback, 1-bit
 * compression and the new worker error.
 *   grads    [W][N] grad_dtype, read (rows w_begin..w_end-1)
 *   m        [N]    fp32, read (the shared momentum)
 *   err_w    [W][N] fp32, read and overwritten with the new errors
 *   packed_w [W][Nw] uint64, written (the messages)
 *   scale_w  [W][T] fp32, written */
int ob_compress_worker(ob_ctx *ctx, int32_t w_begin, int32_t w_end, const void *grads,
                       const float *m, float *err_w, uint64_t *packed_w, float *scale_w,
                       void *stream);

/* Source: the 1-bit Adam review, Proposed method, bullet 4 (the compressed
 * messages are exchanged through custom collectives).  The pages describe the
 * collective only in prose; a server that averages the W decompressed messages
 * and re-compresses the average with its own error buffer is the reading
 * taken, and here the exchange is a local reduction in one GPU's memory.
 *
 * Server: decompress and average all W messages, add the server error,
 * re-compress, store the new server error.
 *   packed_w [W][Nw], scale_w [W][T] read; err_s [N] read and overwritten;
 *   packed_s [Nw] and scale_s [S] written (the server message; S = T unless the
 *   server is partitioned, see ob_set_server_chunks). */
int ob_server_reduce(ob_ctx *ctx, const uint64_t *packed_w, const float *scale_w,
                     float *err_s, uint64_t *packed_s, float *scale_s, void *stream);

/* Source: the 1-bit Adam review, Abstract (the variance, stable after warmup,
 * is a fixed preconditioner for the rest of training), Proposed method, bullet
 * 2, and One-line summary (preconditioned momentum SGD).  No bias correction,
 * eps outside the root.
 *
 * Update from the server message with the frozen variance:
 *   packed_s [Nw], scale_s [S], v [N] read; m [N] written; params [N] read and
 *   overwritten.  lr must be finite. */
int ob_apply_update(ob_ctx *ctx, const uint64_t *packed_s, const float *scale_s,
                    const float *v, float *m, float *params, double lr, void *stream);

/* Source: the 1-bit Adam review, One-line summary and Proposed method, bullets
 * 1 to 4: one step of the compression phase (compressed momentum, exchange,
 * preconditioned update).
 *
 * One whole compression-phase step: ob_compress_worker over all W workers,
 * ob_server_reduce and ob_apply_update, with the server's second pass and the
 * update fused into one kernel.  Same buffers and results as the three calls
 * in sequence. */
int ob_step(ob_ctx *ctx, const void *grads, float *m, const float *v, float *params,
            float *err_w, float *err_s, uint64_t *packed_w, float *scale_w,
            uint64_t *packed_s, float *scale_s, double lr, void *stream);

/* Source: as ob_step (the 1-bit Adam review, One-line summary and Proposed
 * method, bullets 1 to 4).  The residual form of the state between steps is
 * this library's: the pages say nothing of what is stored between steps.
 *
 * The same step with the error and momentum state kept in residual form,
 * one pass per phase instead of two.
 *
 * Residual form: err_w[w] holds x_w, the value worker w compressed in the
 * last step, and scale_w its scales; err_s holds z, the value the server
 * compressed, and scale_s / packed_s its scales and message.  The state of
 * the strict form is an exact function of it (see ob_materialize):
 *   e_w = x_w - s_w,t*sign(x_w),  e_s = z - s_s,t*sign(z),  m = s_s,t*sign(z),
 * the same fp32 operations the strict form performs, so both forms follow
 * bit-identical trajectories (the momentum of this phase is the server's
 * 1-bit message, so it needs no separate buffer).
 *
 *   first != 0: err_w, err_s and m hold strict-form errors and momentum (for
 *               example zeros at the start of the compression phase);
 *               packed_s and scale_s are only written.
 *   first == 0: the buffers hold the residual form left by the previous call;
 *               m is not read and may be NULL.
 * On return err_w, err_s, packed_w, scale_w, packed_s and scale_s hold this
 * step's residual form and messages, params is updated, m is untouched. */
int ob_step_residual(ob_ctx *ctx, int32_t first, const void *grads, const float *m,
                     const float *v, float *params, float *err_w, float *err_s,
                     uint64_t *packed_w, float *scale_w, uint64_t *packed_s, float *scale_s,
                     double lr, void *stream);

/* For callers that cannot allocate device memory when they step: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same step as ob_step_residual (same arguments, buffers and results),
 * with every per-step scratch buffer -- the per-tile and per-chunk partial
 * sums of squares and the trust ratios -- in one static device array of this
 * library (64 MiB per GPU, held from the library's first use on that GPU
 * until the process ends) instead of the context's scratch.  It allocates
 * nothing: no hipMalloc, hipFree, event creation or allocating library call
 * (so its launches are not timed by ob_profile_*); its device address is
 * looked up once per GPU by ob_init.  A list needs (W+1)*tiles*16 +
 * W*tiles*128 + T*4 bytes of it (tiles = its 8192-element tiles; each of the
 * three sections rounded up to 256 bytes): 48 MB for the BERT-Large-shaped
 * list at W = 8.  A list needing more than 64 MiB returns OB_ERR_SCRATCH
 * before anything is enqueued; OB_ERR_DEVICE if ob_init could not look the
 * array up.  Every context and call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (two streams, two host threads) race on it.  Each
 * call writes every scratch entry before reading it, so nothing is cleared
 * between calls. */
int ob_step_residual_noalloc(ob_ctx *ctx, int32_t first, const void *grads, const float *m,
                             const float *v, float *params, float *err_w, float *err_s,
                             uint64_t *packed_w, float *scale_w, uint64_t *packed_s,
                             float *scale_s, double lr, void *stream);

/* Source: the 1-bit Adam review, Proposed method, bullet 3: the error left by
 * compressing x is x minus its 1-bit reconstruction.
 *
 * Writes the strict-form state of a residual-form state:
 *   err_w [W][N] = x_w - s_w,t*sign(x_w),  err_s [N] = z - s_s,t*sign(z),
 *   m [N] = s_s,t*sign(z).
 * x_w [W][N], scale_w [W][T], z [N], scale_s [S] are read.  Outputs may be
 * the same buffers as the inputs (in place). */
int ob_materialize(ob_ctx *ctx, const float *x_w, const float *scale_w, const float *z,
                   const float *scale_s, float *err_w, float *err_s, float *m, void *stream);

/* Source: the 1-bit Adam review, Proposed method, bullet 1 (full-precision
 * Adam for about the first 20% of steps).
 *
 * Warmup phase: one uncompressed Adam step on the workers' average gradient,
 * the first phase of the method (the review of "1-bit Adam ...", Proposed
 * method, bullet 1: full-precision Adam for about the first 20% of steps,
 * whose variance the compression phase then keeps fixed, bullet 2):
 *   gbar = (sum over w = 0..W-1, ascending, from +0, of g_w[i]) / W
 *   m[i] = c1*m[i] + c2*gbar
 *   v[i] = fp32(beta2)*v[i] + fp32(1 - beta2)*(gbar*gbar)
 *   p[i] = p[i] - lr * (m[i] / (sqrt(v[i]) + eps))      (no bias correction)
 * grads [W][N] read; m, v, params [N] read and overwritten.  beta2 in [0, 1),
 * lr finite. */
int ob_warmup_step(ob_ctx *ctx, const void *grads, float *m, float *v, float *params,
                   double beta2, double lr, void *stream);

/* Source: the 1-bit Adam review, Proposed method, bullets 1 and 2 (the switch
 * to compressed momentum SGD, with the variance kept fixed from then on).
 *
 * The switch from warmup to compression: v is kept as it is from now on
 * (frozen) and the error buffers start from zero.  Writes 0 to every tensor
 * element of err_w [W][N] and err_s [N] (padding untouched).  The next step
 * is ob_step, or ob_step_residual with first != 0. */
int ob_begin_compression(ob_ctx *ctx, float *err_w, float *err_s, void *stream);

/* Source: the 1-bit Adam review, Proposed method, bullet 4 (the custom
 * collective).  One scale per server chunk is the reading for a server role
 * split across ranks; the pages do not say.
 *
 * Partitioned server: when the server role is split C ways, rank j holds
 * chunk j of every tensor and compresses it with its own scale.  Chunk j of
 * an n-element tensor covers elements [j*S_t, min((j+1)*S_t, n)) with
 * S_t = 8192*ceil(ceil(n/8192)/C) (whole 8192-element blocks, so a chunk
 * boundary never splits a sign word); a tensor has ceil(n/S_t) <= C chunks.
 * After this call every server scale (scale_s, the server message) is per
 * chunk, in tensor order then chunk order; ob_server_scale_count gives their
 * number S.  C = 1 (the default) is one scale per tensor; any C at or above
 * a tensor's tile count gives that tensor one scale per 8192-element block.
 * Synchronous: waits for the stream of this context's latest launch (which
 * must still exist), then uploads small tables; if an upload fails it
 * restores the previous setting's tables and returns OB_ERR_DEVICE.  Changes
 * of C between steps also change what scale_s holds, so use it before the
 * first step. */
int ob_set_server_chunks(ob_ctx *ctx, int32_t chunks);
int32_t ob_server_scale_count(const ob_ctx *ctx);

/* Source: the fugumt page on "1-bit LAMB: Communication Efficient Large-Scale
 * Large-Batch Training with LAMB's Convergence Speed", Abstract (LAMB's layer-
 * wise adaptive learning rates kept under 1-bit compression).
 *
 * Layer-wise trust ratio (the fugumt page on "1-bit LAMB": LAMB's layer-wise
 * adaptive learning rates kept under compressed communication; the page gives
 * no formula, this is the plainest reading).  With enable != 0 every update of
 * this context (ob_step, ob_step_residual, ob_apply_update) becomes, per
 * tensor t:
 *   u[i] = m[i] / (sqrt(v[i]) + eps)   (+ fp32(weight_decay) * p[i] if > 0)
 *   r_t  = fp32( sqrt(fl64(sum p^2)) / sqrt(fl64(sum u^2)) ), 1 if a sum is 0
 *   p[i] = p[i] - lr * (r_t * u[i])
 * with the sums exact up to one rounding, as for the scales.  It costs two
 * more launches per step (the ratio needs the whole tensor's update) and one
 * more read of v and params.  weight_decay >= 0 and finite. */
int ob_set_trust_ratio(ob_ctx *ctx, int32_t enable, double weight_decay);

/* Source: the nubint.ai review of "ScaleCom: Scalable Sparsified Gradient
 * Compression for Communication-Efficient Distributed Training", Proposed
 * method, bullet 1 (a cyclically chosen leader's top-k indices shared by all
 * workers) and Main results, bullet 3.
 *
 * Cyclic local top-k (CLT-k), an alternative codec for the exchange: the
 * commutative compressor of the review of "ScaleCom: Scalable Sparsified
 * Gradient Compression for Communication-Efficient Distributed Training"
 * (Proposed method, bullet 1; Main results, bullet 3).  Per tensor t with
 * k_t = max(1, ceil(density * n_t)) entries kept:
 *   x_w     = memory_w + g_w                              (fp32, every worker)
 *   index   = the k_t positions of largest |x_leader|, leader = step mod W,
 *             ties to the lower position, listed in ascending order
 *   values_w = x_w at index;  memory_w = x_w with those positions set to 0
 *   average = (sum over w ascending, from +0, of values_w) / W
 * The page names a low-pass filter on the memory without its form; none is
 * applied.  Inputs must be finite.
 *
 * ob_cltk_configure allocates the codec's scratch for the given density
 * (0 < density <= 1; every n_t at most INT32_MAX, else OB_ERR_INVALID;
 * synchronous: waits for the stream of this context's latest launch, then
 * allocates and uploads) and returns K = sum of k_t; ob_cltk_layout writes the host
 * array k_off[0..T] (tensor t's entries are k_off[t] .. k_off[t+1]-1).
 * ob_cltk_step: grads [W][N] read; memory [W][N] fp32 read and overwritten;
 * index [K] int32 (position within the tensor), values [W][K] fp32 and
 * average [K] fp32 written. */
int ob_cltk_configure(ob_ctx *ctx, double density, int64_t *k_total);
int ob_cltk_layout(const ob_ctx *ctx, int64_t *k_off);
int ob_cltk_step(ob_ctx *ctx, int64_t step, const void *grads, float *memory, int32_t *index,
                 float *values, float *average, void *stream);

/* Kernel timing for measurement.  With profiling on, every kernel the context
 * launches is bracketed by HIP events on its stream.  ob_profile_read waits for
 * the recorded events, writes per kernel kind the summed milliseconds and the
 * launch count (arrays of ob_profile_kinds() entries), and with reset != 0
 * forgets them.  ob_profile_kind_name names kind k (NULL when out of range). */
int ob_profile_enable(ob_ctx *ctx, int32_t enable);
int32_t ob_profile_kinds(void);
const char *ob_profile_kind_name(int32_t kind);
int ob_profile_read(ob_ctx *ctx, double *total_ms, int64_t *launches, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* OB_H */
