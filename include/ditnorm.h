/*
 * ditnorm -- fused adaLN row normalisation for diffusion transformers on
 * AMD Instinct MI355X (gfx950).  C ABI of libditnorm.so.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer owned by the caller.
 *   The library never allocates, frees or keeps any of them.  bf16 tensors
 *   are passed as `void*` (2-byte bfloat16 bit patterns); fp32 tensors as
 *   `float*`.  Every tensor pointer must be 16-byte aligned.
 *
 * Layout.  Activations are dense row-major [rows, cols] (row stride == cols
 *   elements).  For a [B, S, D] activation, rows = B*S and cols = D.
 *   Modulation rows (scale, shift, gate) are [B, cols] with a row stride of
 *   `mod_batch_stride` elements (>= cols; a multiple of 8 when B > 1), so a
 *   chunk view of a [B, k*D] adaLN embedding can be passed directly.
 *   Activation row r uses modulation row r / rows_per_batch; B is
 *   rows / rows_per_batch.  The caller picks the (scale, shift) order of its
 *   embedding's chunks by passing the right pointers.
 *
 * Streams.  Calls are asynchronous: the work is enqueued on `stream` (a
 *   hipStream_t passed as void*; NULL = the null stream) and the call
 *   returns.  Outputs are valid once the stream has been synchronised.
 *
 * Status.  Every entry point returns an int:
 *   DITNORM_OK (0)
 *   DITNORM_INVALID_ARGUMENT (1): a required pointer is NULL, a size is
 *       negative or zero where it must be positive, rows is not a multiple of
 *       rows_per_batch, mod_batch_stride < cols, eps is negative or not finite,
 *       or an optional group is given half-way (see each entry point).
 *   DITNORM_UNSUPPORTED (2): the arguments are valid but outside what the
 *       kernels implement: cols not a multiple of 8 or above the stated
 *       maximum, more than DITNORM_MAX_ROWS rows (rows_q + rows_k for
 *       qk_layernorm), more than DITNORM_MAX_VECTORS 16-byte vectors in an
 *       activation of the elementwise entry points, head_dim over 128 or
 *       not a multiple of 8, a pointer not 16-byte aligned, a modulation row stride that breaks
 *       16-byte alignment or exceeds DITNORM_MAX_MOD_STRIDE, or an output
 *       that overlaps an input other than in the exact in-place forms
 *       allowed.
 *   DITNORM_DEVICE_ERROR (3): the current device is not gfx950, or a HIP call
 *       or kernel launch failed (ditnorm_last_hip_error() keeps the code).
 *   DITNORM_SCRATCH_EXCEEDED (4): ln_modulate_backward_noalloc only: the call
 *       needs more partial-sum memory than the library's fixed scratch array
 *       holds (DITNORM_NOALLOC_SCRATCH_BYTES).
 *   All argument checks run on the host before any HIP call; a call that
 *   fails them has no effect.  rows == 0 is a valid no-op.  No exception
 *   crosses the ABI and nothing falls back to another implementation.
 *
 * Aliasing.  `out == x` (exactly the same pointer) is allowed: every row is
 *   read completely before any of it is written.  `residual_out == residual`
 *   is allowed likewise.  Any other overlap of an output with an input or
 *   with another output returns DITNORM_UNSUPPORTED.
 *
 * Optional outputs.  mean_out / rstd_out (fp32, one value per row), y_out
 *   (bf16, the normalised value before modulation) and xb_out (bf16, the
 *   biased input) expose intermediate stages for verification; pass NULL in
 *   production.  They cost one extra write each.
 *
 * Numerics.  Statistics are fp32 values: mean = fp32(sum(x)/N),
 *   rstd = fp32(1/sqrt(var + eps)) with the biased variance, the sums
 *   accumulated in binary64 so that they are exact or within 1e-16 of exact.
 *   Every elementwise stage keeps the eager chain's bf16 round-to-nearest-even
 *   at each op boundary, with no fused multiply-add.
 *
 * Thread safety.  Entry points may be called concurrently from several host
 *   threads; the library keeps only per-device read-only state and the last
 *   HIP error code (thread-local).  The one exception is
 *   ln_modulate_backward_noalloc, whose calls on one device share that
 *   device's scratch array (see there).
 */
#ifndef DITNORM_H
#define DITNORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DITNORM_OK 0
#define DITNORM_INVALID_ARGUMENT 1
#define DITNORM_UNSUPPORTED 2
#define DITNORM_DEVICE_ERROR 3
#define DITNORM_SCRATCH_EXCEEDED 4

/* Storage types of the standalone elementwise entry points and of the
 * conv-bias epilogue (fp32 only there). */
#define DITNORM_DTYPE_BF16 0
#define DITNORM_DTYPE_F16 1
#define DITNORM_DTYPE_F32 2

/* Largest row width of the row kernels (ln_modulate, gated_ln_modulate,
 * rms_modulate) and the largest channel count of the channels_last kernels. */
#define DITNORM_MAX_COLS 16384
#define DITNORM_MAX_CHANNELS 4096
/* Largest row width of ln_modulate_backward (bf16; fp32 rows up to
 * DITNORM_MAX_BACKWARD_F32_COLS). */
#define DITNORM_MAX_BACKWARD_COLS 4096
#define DITNORM_MAX_BACKWARD_F32_COLS 3072
/* Bytes of the per-device scratch array of ln_modulate_backward_noalloc
 * (32 MiB). */
#define DITNORM_NOALLOC_SCRATCH_BYTES 33554432LL
/* Most rows of one call (a row has up to one 64-lane wavefront, so at this
 * limit a launch of 4-row workgroups holds 2^31 work-items, within the 32-bit
 * grid size; every kernel indexes in 64 bits), and most 16-byte vectors in
 * one activation of modulate_scale_shift, residual_gate_add and
 * conv_bias_epilogue (one work-item per vector). */
#define DITNORM_MAX_ROWS 33554431LL
#define DITNORM_MAX_VECTORS 2147483647LL
/* Largest modulation row stride, in elements (far beyond any real tensor; it
 * keeps every byte-span computation of the argument checks inside int64). */
#define DITNORM_MAX_MOD_STRIDE 68719476736LL

/* Human-readable name of a status code (static storage, never NULL). */
const char *ditnorm_status_string(int status);

/* hipError_t of the last failing HIP call on this host thread (0 if none). */
int ditnorm_last_hip_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int ditnorm_version(void);

/*
 * ln_modulate -- affine-free LayerNorm of each row, then the adaLN modulate.
 *
 * Defined on the GLM-Image page ("[diffusion] GLM-Image bit-exact fused aten
 * LayerNorm+modulate / qk-LN", Motivation and "What rounding-faithful means
 * here") and on the FLUX.1 page (fused adaLN modulate, Commit 2):
 *     y   = bf16( rstd * (x - mean) )                    per row, fp32 stats
 *     out = bf16( bf16( y * bf16(1 + scale) ) + shift )  per element
 * x, out: bf16 [rows, cols].  scale, shift: bf16 [B, cols], row stride
 * mod_batch_stride.  eps: fp32 (1e-6 on the pages' adaLN sites).
 * cols: multiple of 8, at most DITNORM_MAX_COLS.  out == x allowed.
 * mean_out, rstd_out (fp32 [rows]) and y_out (bf16 [rows, cols]) optional.
 */
int ln_modulate(const void *x, const void *scale, const void *shift, void *out,
                int64_t rows, int64_t cols, int64_t rows_per_batch,
                int64_t mod_batch_stride, float eps, float *mean_out, float *rstd_out,
                void *y_out, void *stream);

/*
 * ln_modulate_folded -- the lossy one-pass form of ln_modulate: the modulate
 * folded into the LayerNorm's elementwise affine.
 *
 * FLUX.1 page ("[diffusion] FLUX.1 fused adaLN modulate (bit-exact) + RoPE
 * cache hoist, LN-affine folding behind quality=high", Commit 3): LayerNorm
 * with weight = bf16(1 + scale) (the [D] row keeps its eager rounding) and
 * bias = shift, so scale and shift act in fp32 on the unrounded normalised
 * value and the result is rounded once:
 *     t   = rstd * (x - mean)                           fp32, not rounded
 *     out = bf16( (t * bf16(1 + scale)) + shift )      fp32 ops, no FMA
 * Not bit-exact with ln_modulate (the pages report a max abs difference of
 * about 0.05 on FLUX.1 shapes); for callers that accept that, as the pages'
 * quality tier does.  Statistics as for ln_modulate (mean_out, rstd_out
 * optional).  Arguments, layout, batching and aliasing as for ln_modulate;
 * unlike the pages' per-call guard, B > 1 modulation rows are supported.
 */
int ln_modulate_folded(const void *x, const void *scale, const void *shift, void *out,
                       int64_t rows, int64_t cols, int64_t rows_per_batch,
                       int64_t mod_batch_stride, float eps, float *mean_out, float *rstd_out,
                       void *stream);

/*
 * gated_ln_modulate -- the pre-norm gated residual, then ln_modulate on it.
 *
 * The residual-gate half of the adaLN block (GLM-Image page, ff gate
 * "hidden + ff_out * gate"; ERNIE-Image page "[diffusion] ERNIE-Image
 * bit-exact fused RMSNorm+scale/shift", second kernel, which also returns the
 * residual stream):
 *     h   = bf16( residual + bf16( gate * update ) )     -> residual_out
 *     out = ln_modulate(h, scale, shift)
 * update (x), residual, residual_out, out: bf16 [rows, cols].
 * gate, scale, shift: bf16 [B, cols], row stride mod_batch_stride.
 * residual_out == residual allowed; out must not alias anything.
 * mean_out, rstd_out, y_out optional, as for ln_modulate (statistics of h).
 */
int gated_ln_modulate(const void *x, const void *residual, const void *gate,
                      const void *scale, const void *shift, void *residual_out, void *out,
                      int64_t rows, int64_t cols, int64_t rows_per_batch,
                      int64_t mod_batch_stride, float eps, float *mean_out,
                      float *rstd_out, void *y_out, void *stream);

/*
 * rms_modulate -- weighted RMSNorm of each row, then the adaLN modulate;
 * optionally preceded by the gated residual.
 *
 * ERNIE-Image page ("[diffusion] ERNIE-Image bit-exact fused
 * RMSNorm+scale/shift", "What rounding-faithful means here" and
 * Modifications):
 *     rstd = fp32( 1 / sqrt( sum(x^2)/cols + eps ) )
 *     y    = bf16( (x * rstd) * weight )           two fp32 products, left to right
 *     out  = bf16( bf16( y * bf16(1 + scale) ) + shift )
 * Gated site (residual, gate and residual_out all non-NULL; all NULL for the
 * plain site -- anything else is DITNORM_INVALID_ARGUMENT):
 *     h = bf16( residual + bf16( gate * x ) ) -> residual_out, and the norm
 *     runs on h.
 * x, out, residual, residual_out: bf16 [rows, cols]; weight: bf16 [cols];
 * scale, shift, gate: bf16 [B, cols], row stride mod_batch_stride.
 * out == x allowed on the plain site; residual_out == residual allowed.
 * rstd_out (fp32 [rows]) and y_out optional.
 */
int rms_modulate(const void *x, const void *weight, const void *scale, const void *shift,
                 void *out, const void *residual, const void *gate, void *residual_out,
                 int64_t rows, int64_t cols, int64_t rows_per_batch,
                 int64_t mod_batch_stride, float eps, float *rstd_out, void *y_out,
                 void *stream);

/*
 * qk_layernorm -- per-head affine-free LayerNorm of q and k in one launch.
 *
 * GLM-Image page, Motivation (nn.LayerNorm(128) per head on (1, S, 32, 128))
 * and "What rounding-faithful means here" (q and k in one launch; the page's
 * kernel serves head dims up to 128):
 *     for every head_dim-wide row of q, then of k:
 *     out = bf16( rstd * (x - mean) ),  fp32 stats, eps (1e-5 on the page's model)
 * q, q_out: bf16 [rows_q, head_dim]; k, k_out: bf16 [rows_k, head_dim] (a
 * (B, S, H, head_dim) tensor is rows = B*S*H).  head_dim: a multiple of 8, at
 * most 128 (else UNSUPPORTED); 128 is the tuned case.  k and k_out may be NULL
 * only when rows_k == 0.  q_out == q and k_out == k allowed.
 * mean_out, rstd_out: optional fp32 [rows_q + rows_k], q rows first.
 */
int qk_layernorm(const void *q, const void *k, void *q_out, void *k_out, int64_t rows_q,
                 int64_t rows_k, int64_t head_dim, float eps, float *mean_out,
                 float *rstd_out, void *stream);

/*
 * rmsnorm_silu_bias -- channels_last RMSNorm over the channels of each pixel,
 * times gamma, then SiLU, with the deferred conv bias folded in first.
 *
 * Wan VAE page ("[Diffusion] Fuse the Wan VAE conv bias epilogue and tile the
 * RMSNorm+SiLU kernel", Modifications, Quality-gated: the [ROWS, C] tiled
 * kernel and its conv_bias= fold, applied exactly like aten's add_):
 *     xb   = bf16( x + bf16(bias) )        (xb = x when bias is NULL)
 *     rstd = fp32( 1 / sqrt( sum(xb^2)/C + eps ) )
 *     t    = (xb * rstd) * gamma           fp32
 *     out  = bf16( SiLU(t) )               one rounding, within 1 bf16 ulp
 * x, out: bf16 channels_last [N, C, D, H, W] = [rows = N*D*H*W, C] dense rows
 * of C channels.  bias: fp32 [C] or NULL; gamma: fp32 [C].
 * channels: multiple of 8, at most DITNORM_MAX_CHANNELS.  out == x allowed.
 * rstd_out (fp32 [rows]) and xb_out (bf16 [rows, C]) optional.
 */
int rmsnorm_silu_bias(const void *x, const float *bias, const float *gamma, void *out,
                      int64_t rows, int64_t channels, float eps, float *rstd_out,
                      void *xb_out, void *stream);

/*
 * conv_bias_epilogue -- the channels_last conv-bias add, optionally fused
 * with the residual add that follows the conv.
 *
 * Wan VAE page (same title), Modifications, the lossless epilogue kernel:
 * the arithmetic of aten's add_ (the sum formed in fp32, rounded once to the
 * activation's type); an fp32 bias on a half-precision activation is cast to
 * the activation's type first, as autocast does before the conv; the
 * residual form rounds twice, once after the bias and once after adding h,
 * as the eager conv output plus h does.  With rnd the rounding to dtype
 * (nearest even; the identity for fp32):
 *     out = rnd( x + rnd(bias) )                       (h == NULL)
 *     out = rnd( rnd( x + rnd(bias) ) + h )            (h != NULL)
 * dtype: DITNORM_DTYPE_BF16, _F16 or _F32, the type of x, h and out
 * ([rows, channels], channels_last pixels).  bias: [C] of bias_dtype,
 * DITNORM_DTYPE_F32 or dtype itself (UNSUPPORTED otherwise).  channels:
 * multiple of 8, at most DITNORM_MAX_CHANNELS; at most DITNORM_MAX_VECTORS
 * 16-byte vectors in x.  out == x allowed.
 */
int conv_bias_epilogue(const void *x, const void *bias, const void *h, void *out,
                       int64_t rows, int64_t channels, int dtype, int bias_dtype,
                       void *stream);

/*
 * modulate_scale_shift -- the adaLN modulate alone, for sites whose norm is
 * not fused into it.
 *
 * FLUX.1 page ("[diffusion] FLUX.1 fused adaLN modulate (bit-exact) + RoPE
 * cache hoist, LN-affine folding behind quality=high", Commit 2): the three
 * results of the eager chain each rounded to the storage type where the
 * eager kernels round them; bf16 or fp16 storage, one modulation row per
 * batch, chunked embedding views:
 *     out = rnd( rnd( x * rnd(1 + scale) ) + shift )
 * dtype: DITNORM_DTYPE_BF16 or DITNORM_DTYPE_F16 -- x, scale, shift and out
 * all of that type, rnd rounding to it nearest-even.  x, out: [rows, cols];
 * scale, shift: [B, cols], row stride mod_batch_stride.  cols: multiple of 8,
 * at most DITNORM_MAX_COLS.  out == x allowed.
 */
int modulate_scale_shift(const void *x, const void *scale, const void *shift, void *out,
                         int64_t rows, int64_t cols, int64_t rows_per_batch,
                         int64_t mod_batch_stride, int dtype, void *stream);

/*
 * residual_gate_add -- the gated residual alone.
 *
 * GLM-Image page (the ff gate reuses the residual-gate-add kernel) and
 * ERNIE-Image page ("What rounding-faithful means here": the residual
 * variant's eager pair round(gate*update), round(residual+...)):
 *     out = rnd( residual + rnd( gate * update ) )
 * dtype as for modulate_scale_shift.  update, residual, out: [rows, cols];
 * gate: [B, cols], row stride mod_batch_stride.  out == residual allowed.
 */
int residual_gate_add(const void *update, const void *residual, const void *gate, void *out,
                      int64_t rows, int64_t cols, int64_t rows_per_batch,
                      int64_t mod_batch_stride, int dtype, void *stream);

/*
 * ln_modulate_backward -- gradients of out = LN(x) * (1 + scale) + shift.
 *
 * Qwen-Image page ("[WS1][Qwen-Image][CUDA] Final AdaLN output
 * (final_adaln_out)", What): the forward and backward of the final adaLN
 * output, the LayerNorm (no affine, fp32 statistics) run in fp32 on widened
 * inputs, the modulation-parameter gradients as token sums reduced by fixed
 * fp32 balanced trees that depend only on the token count:
 *     x_hat   = (x - mean) * rstd,   g = d_out * (1 + scale)   (1 + scale in fp32)
 *     d_x     = bf16( rstd * (g - mean_row(g) - x_hat * mean_row(g * x_hat)) )
 *               (evaluated in binary64, one rounding to bf16)
 *     d_shift = sum over the batch's tokens of d_out
 *     d_scale = sum over the batch's tokens of d_out * x_hat   (terms in fp32,
 *               x_hat = rstd * (x - mean) in fp32)
 * The token sums: adjacent pairs within groups of 32 consecutive tokens, then
 * the group sums again in groups of 32, until one value remains; a short
 * group is padded with +0.  The result for a batch depends only on its own
 * rows and its token count (bitwise batch-invariant).
 * dtype: DITNORM_DTYPE_BF16, or DITNORM_DTYPE_F32 for the page's fp32
 * stream (d_x then the binary64 value rounded once to fp32).  x, d_out, d_x:
 * dtype [rows, cols]; scale: dtype [B, cols], row stride mod_batch_stride;
 * d_scale, d_shift: fp32 [B, cols] dense.  cols: multiple of 8, at most
 * DITNORM_MAX_BACKWARD_COLS (bf16) or DITNORM_MAX_BACKWARD_F32_COLS (fp32).
 * B times rows_per_batch, rounded up to a multiple of the kernel's tokens
 * per workgroup, at most DITNORM_MAX_ROWS; that count is 8 for bf16 when
 * cols <= 3072 and either rows_per_batch is 5-8 or the batches fill more
 * than 128 eight-token workgroups, else 4 (always 4 for fp32).  No output
 * may overlap an input or another output.
 * workspace: device memory of at least
 * ln_modulate_backward_workspace_bytes(rows, cols, rows_per_batch, dtype) bytes,
 * 256-byte aligned, owned by the caller, clobbered by the call (it holds the
 * partial tree sums); when that size is 0 (batches of at most 8 tokens, 4
 * for rows over 3072 columns) workspace may be NULL.  mean_out, rstd_out
 * (fp32 [rows]) optional.  The work is one kernel launch on `stream` when the
 * workspace size is 0, else one more per level of the token tree: two for
 * batches of up to 1024 tokens, three up to 32768, four up to 2^20.
 */
int ln_modulate_backward(const void *x, const void *scale, const void *d_out, void *d_x,
                         float *d_scale, float *d_shift, int64_t rows, int64_t cols,
                         int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                         void *workspace, int64_t workspace_bytes, float *mean_out,
                         float *rstd_out, int dtype, void *stream);

/*
 * ln_modulate_backward_noalloc -- ln_modulate_backward without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results, kernels and launches as ln_modulate_backward,
 * bitwise the same outputs; the partial tree sums go to a scratch array of
 * DITNORM_NOALLOC_SCRATCH_BYTES that the library holds on every device it
 * runs on (loaded with the library, kept until the process ends).  The call
 * makes no allocation of any kind (no hipMalloc, no hipFree).  A call whose
 * ln_modulate_backward_workspace_bytes(rows, cols, rows_per_batch, dtype) exceeds
 * DITNORM_NOALLOC_SCRATCH_BYTES returns DITNORM_SCRATCH_EXCEEDED and enqueues
 * nothing.  The partial sums take about one byte per element of x when the
 * kernel runs 8 tokens per workgroup and two when it runs 4 (see
 * ln_modulate_backward), nothing for batches of at most 8 tokens (4 over 3072
 * columns): 6889 tokens of 3072 columns need 21.4 MB.  The scratch needs no
 * clearing between calls: every
 * value a call reads there was written earlier in the same call.  Calls on
 * one device share its array: two calls whose work overlaps in time on one
 * device (different streams, or host threads racing on one stream's order)
 * race on it and give wrong results; order them on one stream or with
 * events.  The first call on a device looks the array's address up there
 * (hipGetSymbolAddress; DITNORM_DEVICE_ERROR if that fails).
 */
int ln_modulate_backward_noalloc(const void *x, const void *scale, const void *d_out, void *d_x,
                                 float *d_scale, float *d_shift, int64_t rows, int64_t cols,
                                 int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                                 float *mean_out, float *rstd_out, int dtype, void *stream);

/* Workspace bytes ln_modulate_backward needs (0 for rows == 0; -1 for invalid
 * sizes or storage type and for rows above DITNORM_MAX_ROWS or cols above
 * the type's maximum, which the call rejects).  Host-only, never touches the
 * GPU. */
int64_t ln_modulate_backward_workspace_bytes(int64_t rows, int64_t cols,
                                             int64_t rows_per_batch, int dtype);

/*
 * *_supported -- 1 if the same call would pass every argument check (it may
 * still fail with DITNORM_DEVICE_ERROR), else 0.  Never fails, never touches
 * the GPU, never enqueues work.
 */
int ln_modulate_supported(const void *x, const void *scale, const void *shift,
                          const void *out, int64_t rows, int64_t cols,
                          int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                          const float *mean_out, const float *rstd_out, const void *y_out);
int ln_modulate_folded_supported(const void *x, const void *scale, const void *shift,
                                 const void *out, int64_t rows, int64_t cols,
                                 int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                                 const float *mean_out, const float *rstd_out);
int gated_ln_modulate_supported(const void *x, const void *residual, const void *gate,
                                const void *scale, const void *shift,
                                const void *residual_out, const void *out, int64_t rows,
                                int64_t cols, int64_t rows_per_batch,
                                int64_t mod_batch_stride, float eps, const float *mean_out,
                                const float *rstd_out, const void *y_out);
int rms_modulate_supported(const void *x, const void *weight, const void *scale,
                           const void *shift, const void *out, const void *residual,
                           const void *gate, const void *residual_out, int64_t rows,
                           int64_t cols, int64_t rows_per_batch, int64_t mod_batch_stride,
                           float eps, const float *rstd_out, const void *y_out);
int qk_layernorm_supported(const void *q, const void *k, const void *q_out,
                           const void *k_out, int64_t rows_q, int64_t rows_k,
                           int64_t head_dim, float eps, const float *mean_out,
                           const float *rstd_out);
int rmsnorm_silu_bias_supported(const void *x, const float *bias, const float *gamma,
                                const void *out, int64_t rows, int64_t channels, float eps,
                                const float *rstd_out, const void *xb_out);
int conv_bias_epilogue_supported(const void *x, const void *bias, const void *h,
                                 const void *out, int64_t rows, int64_t channels, int dtype,
                                 int bias_dtype);
int ln_modulate_backward_supported(const void *x, const void *scale, const void *d_out,
                                   const void *d_x, const float *d_scale, const float *d_shift,
                                   int64_t rows, int64_t cols, int64_t rows_per_batch,
                                   int64_t mod_batch_stride, float eps, const void *workspace,
                                   int64_t workspace_bytes, const float *mean_out,
                                   const float *rstd_out, int dtype);
int modulate_scale_shift_supported(const void *x, const void *scale, const void *shift,
                                   const void *out, int64_t rows, int64_t cols,
                                   int64_t rows_per_batch, int64_t mod_batch_stride, int dtype);
int residual_gate_add_supported(const void *update, const void *residual, const void *gate,
                                const void *out, int64_t rows, int64_t cols,
                                int64_t rows_per_batch, int64_t mod_batch_stride, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* DITNORM_H */
