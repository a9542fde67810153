/*
 * ditnorm oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU definition of what the fused adaLN
 * row-normalisation kernels compute.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load or call this library; the
 * product path (the HIP library and its Python binding) never does, and this
 * file shares no code, header, table or helper with it.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math (x86-64 SSE2).
 * Every `float` operation below is therefore one IEEE binary32 operation
 * rounded to nearest-even, every `double` one IEEE binary64 operation, and
 * no multiply-add is ever contracted into an FMA.
 *
 * What is computed, and where it comes from (page titles are the pull
 * requests the method is described in):
 *
 *  - bf16 storage.  Activations, modulation rows and outputs are bfloat16;
 *    every bf16 value widens exactly to binary32, and every op boundary of
 *    the eager chain rounds back with round-to-nearest-even ("GLM-Image
 *    bit-exact fused aten LayerNorm+modulate / qk-LN", section "What
 *    rounding-faithful means here": the bitcast RNE helper).
 *
 *  - LayerNorm statistics (affine-free LN, same page): the row mean and the
 *    biased variance (divide by N).  The pages fix these as fp32 values; the
 *    eager kernel reaches them through one particular fp32 accumulation
 *    order.  The plain definition is taken here: the exact mean and variance
 *    (accumulated in binary64, which is exact or within 1e-16 for bf16 rows),
 *    rounded once to binary32 where the eager chain holds a binary32 value:
 *        mean_f = fp32(S / N),   rstd_f = fp32(1 / sqrt(var + eps)).
 *
 *  - LN normalise: y = bf16( rstd_f * (x - mean_f) ), subtract then multiply,
 *    two fp32 ops, no FMA (same page and section).
 *
 *  - adaLN modulate (same section; the ERNIE-Image RMSNorm+scale/shift page;
 *    the FLUX.1 fused-modulate page, "Commit 2"): three eager kernels, each
 *    rounding to bf16:  s1 = bf16(1 + scale);  p = bf16(y * s1);
 *    out = bf16(p + shift).
 *
 *  - Weighted RMSNorm ("ERNIE-Image bit-exact fused RMSNorm+scale/shift",
 *    section "What rounding-faithful means here"): mean of squares over the
 *    H columns (no mean subtraction), rstd = 1/sqrt(ms + eps) in fp32, and one
 *    rounding of the product x * rstd * w evaluated left to right in binary32
 *    ((x * rstd) * w; x * (rstd * w) differs on rare elements).
 *
 *  - fp16 storage of the standalone modulate and residual-gate add (FLUX.1
 *    page, Commit 2: bf16 and fp16): the same binary32 operations, each
 *    result rounded to IEEE half precision, nearest-even, overflow to
 *    infinity, subnormals kept.
 *
 *  - LN-affine folding, the lossy one-pass form ("FLUX.1 fused adaLN
 *    modulate (bit-exact) + RoPE cache hoist, LN-affine folding behind
 *    quality=high", Commit 3): the modulate becomes the LayerNorm's affine,
 *    weight = bf16(1 + scale) (the [D] row keeps its eager rounding) and
 *    bias = shift, applied in fp32 to the unrounded normalised value and
 *    rounded once: out = bf16((rstd * (x - mean)) * w + shift).  The page
 *    leaves the fp32 order of the affine open; the order written here (the
 *    normalise's subtract-then-multiply, then the weight, then the bias, no
 *    FMA) is the plain reading.
 *
 *  - Backward of LN (no affine) + modulate ("[WS1][Qwen-Image][CUDA] Final
 *    AdaLN output (final_adaln_out)", What): the forward
 *    out = LN(x) * (1 + scale) + shift executed in fp32 on widened inputs,
 *    with fp32 statistics kept from the forward.  With x_hat the normalised
 *    value and g = d_out * (1 + scale):
 *      d_x     = rstd * (g - mean_row(g) - x_hat * mean_row(g * x_hat)),
 *                evaluated here in binary64 and rounded once to the storage
 *                type (the execution-dtype store): bf16, or binary32 for the
 *                page's fp32 stream, where x, scale and d_out are binary32
 *                too and 1 + scale is their binary32 sum;
 *      d_shift = sum over a batch's tokens of d_out,
 *      d_scale = sum over a batch's tokens of d_out * x_hat,
 *    the two token sums in fp32 by the page's fixed balanced trees: adjacent
 *    pairs within groups of 32 consecutive values (5 levels), the group sums
 *    again in groups of 32, until one value remains; a short group is padded
 *    with +0.  The tree depends only on the batch's token count.  The fp32
 *    terms are d_out (exact) and d_out * x_hat with x_hat = rstd * (x - mean)
 *    in fp32 (the normalise's subtract-then-multiply, unrounded).
 *
 *  - Gated residual (pre-norm; same ERNIE page, second kernel, and the GLM
 *    page's ff-gate):  h = bf16(residual + bf16(gate * update)); the norm
 *    then runs on h, and h is returned as the residual stream.
 *
 *  - Per-head qk LayerNorm (GLM page, Motivation and "What rounding-faithful
 *    means here"): the LN statistics + normalise over every head_dim-wide
 *    row of q and of k, no affine, no modulate.
 *
 *  - channels_last RMSNorm + SiLU with the conv bias folded in ("Fuse the Wan
 *    VAE conv bias epilogue and tile the RMSNorm+SiLU kernel", Modifications):
 *    the deferred conv bias is applied exactly like aten's add_ with an fp32
 *    bias cast to the activation dtype first, xb = bf16(x + bf16(bias)); the
 *    RMS statistics run on xb over the C channels of each pixel; then one fp32
 *    pass t = (xb * rstd) * gamma and a single rounding of SiLU(t).  SiLU is
 *    evaluated in binary64 and rounded once, directly, to bf16.
 *
 *  - Conv-bias epilogue (same Wan page, "New kernel"; its tests cover bf16,
 *    fp16 and fp32 activations with an fp32 or same-type bias): x.dtype(x +
 *    bias) with the bias cast to the activation dtype first, optionally
 *    followed by the residual add as a second rounding, e.g. for bf16
 *    bf16(bf16(x + bf16(bias)) + h); each addition one binary32 operation,
 *    rounded to the storage type (the identity for fp32).
 *
 * Every function takes host pointers; bf16 tensors are passed as uint16_t bit
 * patterns.  Functions return 0 on success and 1 on an invalid argument.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#define OR_OK 0
#define OR_INVALID 1

/* ------------------------------------------------------------------------- */
/* bf16 <-> binary32                                                         */
/* ------------------------------------------------------------------------- */

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 value to bf16, nearest-even.  NaN maps to the canonical
 * quiet NaN 0x7FC0 (sign dropped), as torch's CPU conversion does. */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    /* Adding 0x7FFF plus the lsb of the kept half rounds to nearest, ties to
     * even; a carry out of the mantissa correctly bumps the exponent (and
     * turns the largest values into infinity). */
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/* Round a binary64 value to bf16 with a single rounding (nearest-even).
 * Rounding through binary32 first is only wrong when the binary32 result
 * lands exactly on a bf16 halfway point while the double does not; that case
 * is resolved toward the side the double lies on. */
static uint16_t f64_to_bf16(double d)
{
    if (isnan(d))
        return 0x7FC0u;
    float f = (float)d;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0xFFFFu) == 0x8000u && (double)f != d && !isinf(f)) {
        if (fabs(d) > fabs((double)f))
            u += 0x8000u; /* the larger-magnitude neighbour */
        else
            u -= 0x8000u; /* the smaller-magnitude neighbour */
        return (uint16_t)(u >> 16);
    }
    return f32_to_bf16(f);
}

/* binary16 (fp16) storage, for the standalone elementwise sites (the FLUX.1
 * page's fused modulate is checked on bf16 and fp16). */
static float f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    float f;
    if (e == 0x1Fu) {
        uint32_t u = sign | 0x7F800000u | (m << 13);
        memcpy(&f, &u, sizeof f);
        return f;
    }
    if (e == 0) {
        f = ldexpf((float)m, -24); /* subnormal (or zero): m * 2^-24, exact */
        return sign ? -f : f;
    }
    uint32_t u = sign | ((e + 112u) << 23) | (m << 13);
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 value to binary16, nearest-even; NaN -> 0x7E00 | sign. */
static uint16_t f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return sign | 0x7E00u;
    if (a >= 0x477FF000u) /* >= 65520: rounds to infinity */
        return sign | 0x7C00u;
    int e = (int)(a >> 23) - 127; /* unbiased binary32 exponent */
    uint32_t sig = (a & 0x7FFFFFu) | (a ? 0x800000u : 0u);
    if (a < 0x00800000u)
        return sign; /* binary32 subnormals are far below half the least fp16 step */
    int shift = e >= -14 ? 13 : 13 + (-14 - e); /* bits dropped from the 24-bit significand */
    if (shift > 31)
        return sign;
    uint32_t q = sig >> shift, rem = sig & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;
    if (e >= -14) /* normal: q holds the implicit bit; rebase the exponent */
        return sign | (uint16_t)((((uint32_t)(e + 15)) << 10) + (q - 0x400u));
    return sign | (uint16_t)q; /* subnormal (q may carry into the least normal) */
}

/* The storage type of an elementwise stage: 0 = bf16, 1 = fp16. */
static float st_to_f32(uint16_t v, int dtype) { return dtype ? f16_to_f32(v) : bf16_to_f32(v); }
static uint16_t f32_to_st(float f, int dtype) { return dtype ? f32_to_f16(f) : f32_to_bf16(f); }

/* ------------------------------------------------------------------------- */
/* Row statistics: the plain definitions                                     */
/* ------------------------------------------------------------------------- */

/* LayerNorm: mean and biased variance of one row, rounded once to fp32. */
static void ln_stats(const float *x, int64_t n, float eps, float *mean_f, float *rstd_f)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += (double)x[i];
    double mean = s / (double)n;
    double m2 = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double d = (double)x[i] - mean;
        m2 += d * d;
    }
    double var = m2 / (double)n;
    *mean_f = (float)mean;
    *rstd_f = (float)(1.0 / sqrt(var + (double)eps));
}

/* RMSNorm: mean of squares of one row (no mean subtraction), rounded once. */
static void rms_stats(const float *x, int64_t n, float eps, float *rstd_f)
{
    double s2 = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)x[i];
        s2 += v * v;
    }
    double ms = s2 / (double)n;
    *rstd_f = (float)(1.0 / sqrt(ms + (double)eps));
}

/* ------------------------------------------------------------------------- */
/* Elementwise stages                                                        */
/* ------------------------------------------------------------------------- */

static uint16_t ln_normalize(float x, float mean, float rstd)
{
    float centred = x - mean;
    return f32_to_bf16(rstd * centred);
}

static uint16_t rms_normalize(float x, float rstd, float w)
{
    float t = x * rstd;
    return f32_to_bf16(t * w);
}

static uint16_t modulate(uint16_t y, uint16_t scale, uint16_t shift)
{
    uint16_t s1 = f32_to_bf16(1.0f + bf16_to_f32(scale));
    uint16_t p = f32_to_bf16(bf16_to_f32(y) * bf16_to_f32(s1));
    return f32_to_bf16(bf16_to_f32(p) + bf16_to_f32(shift));
}

static uint16_t ln_modulate_folded(float x, float mean, float rstd, uint16_t scale,
                                   uint16_t shift)
{
    float t = rstd * (x - mean);
    float w = bf16_to_f32(f32_to_bf16(1.0f + bf16_to_f32(scale)));
    float p = t * w;
    return f32_to_bf16(p + bf16_to_f32(shift));
}

static uint16_t gate_residual(uint16_t residual, uint16_t gate, uint16_t update)
{
    uint16_t g = f32_to_bf16(bf16_to_f32(gate) * bf16_to_f32(update));
    return f32_to_bf16(bf16_to_f32(residual) + bf16_to_f32(g));
}

static uint16_t bias_add(uint16_t x, float bias)
{
    uint16_t b = f32_to_bf16(bias);
    return f32_to_bf16(bf16_to_f32(x) + bf16_to_f32(b));
}

static double silu64(double t)
{
    return t / (1.0 + exp(-t));
}

static uint16_t silu_bf16(float t)
{
    return f64_to_bf16(silu64((double)t));
}

/* ------------------------------------------------------------------------- */
/* Argument checks shared by the composites                                  */
/* ------------------------------------------------------------------------- */

static int mod_args_ok(int64_t rows, int64_t cols, int64_t rows_per_batch,
                       int64_t mod_batch_stride)
{
    if (rows < 0 || cols <= 0 || rows_per_batch <= 0)
        return 0;
    if (rows % rows_per_batch != 0)
        return 0;
    if (mod_batch_stride < cols)
        return 0;
    return 1;
}

/* ------------------------------------------------------------------------- */
/* Exported: conversions (for pinning the rounding helpers)                  */
/* ------------------------------------------------------------------------- */

void oracle_round_f32_to_f16(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_f16(in[i]);
}

void oracle_widen_f16(const uint16_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f16_to_f32(in[i]);
}

void oracle_round_f32_to_bf16(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16(in[i]);
}

void oracle_round_f64_to_bf16(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f64_to_bf16(in[i]);
}

void oracle_silu_bf16(const float *t, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = silu_bf16(t[i]);
}

/* ------------------------------------------------------------------------- */
/* Exported: stages (each applied given its inputs, so a GPU result can be   */
/* checked stage by stage)                                                    */
/* ------------------------------------------------------------------------- */

/* Widen one bf16 row into a binary32 buffer (exact). */
#define OR_MAX_COLS 65536
static _Thread_local float row_buf[OR_MAX_COLS];

static const float *widen_row(const uint16_t *xr, int64_t n)
{
    for (int64_t c = 0; c < n; ++c)
        row_buf[c] = bf16_to_f32(xr[c]);
    return row_buf;
}

/* Per-row LN statistics of bf16 rows. */
int oracle_ln_stats(const uint16_t *x, int64_t rows, int64_t cols, float eps,
                    float *mean_out, float *rstd_out)
{
    if (rows < 0 || cols <= 0 || cols > OR_MAX_COLS)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r)
        ln_stats(widen_row(x + r * cols, cols), cols, eps, &mean_out[r], &rstd_out[r]);
    return OR_OK;
}

/* Per-row RMS statistics of bf16 rows. */
int oracle_rms_stats(const uint16_t *x, int64_t rows, int64_t cols, float eps,
                     float *rstd_out)
{
    if (rows < 0 || cols <= 0 || cols > OR_MAX_COLS)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r)
        rms_stats(widen_row(x + r * cols, cols), cols, eps, &rstd_out[r]);
    return OR_OK;
}

/* y = bf16(rstd * (x - mean)) given per-row fp32 statistics. */
int oracle_ln_normalize(const uint16_t *x, const float *mean, const float *rstd,
                        uint16_t *y, int64_t rows, int64_t cols)
{
    if (rows < 0 || cols <= 0)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            y[r * cols + c] = ln_normalize(bf16_to_f32(x[r * cols + c]), mean[r], rstd[r]);
    return OR_OK;
}

/* y = bf16((x * rstd) * w) given per-row fp32 rstd and a bf16 weight row. */
int oracle_rms_normalize(const uint16_t *x, const float *rstd, const uint16_t *w,
                         uint16_t *y, int64_t rows, int64_t cols)
{
    if (rows < 0 || cols <= 0)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            y[r * cols + c] = rms_normalize(bf16_to_f32(x[r * cols + c]), rstd[r],
                                            bf16_to_f32(w[c]));
    return OR_OK;
}

/* out = bf16(bf16(y * bf16(1 + scale)) + shift); modulation row r / rows_per_batch. */
int oracle_modulate(const uint16_t *y, const uint16_t *scale, const uint16_t *shift,
                    uint16_t *out, int64_t rows, int64_t cols, int64_t rows_per_batch,
                    int64_t mod_batch_stride)
{
    if (!mod_args_ok(rows, cols, rows_per_batch, mod_batch_stride))
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / rows_per_batch;
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = modulate(y[r * cols + c], scale[b * mod_batch_stride + c],
                                         shift[b * mod_batch_stride + c]);
    }
    return OR_OK;
}

/* Standalone modulate in the storage type `dtype` (0 bf16, 1 fp16):
 * out = rnd(rnd(x * rnd(1 + scale)) + shift), every op one binary32 op. */
int oracle_modulate_dt(const uint16_t *x, const uint16_t *scale, const uint16_t *shift,
                       uint16_t *out, int64_t rows, int64_t cols, int64_t rows_per_batch,
                       int64_t mod_batch_stride, int dtype)
{
    if (!mod_args_ok(rows, cols, rows_per_batch, mod_batch_stride) || (dtype != 0 && dtype != 1))
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / rows_per_batch;
        for (int64_t c = 0; c < cols; ++c) {
            float s1 = st_to_f32(f32_to_st(1.0f + st_to_f32(scale[b * mod_batch_stride + c], dtype), dtype), dtype);
            float p = st_to_f32(f32_to_st(st_to_f32(x[r * cols + c], dtype) * s1, dtype), dtype);
            out[r * cols + c] = f32_to_st(p + st_to_f32(shift[b * mod_batch_stride + c], dtype), dtype);
        }
    }
    return OR_OK;
}

/* Standalone residual-gate add in `dtype`: out = rnd(residual + rnd(gate * update)). */
int oracle_gate_residual_dt(const uint16_t *update, const uint16_t *residual,
                            const uint16_t *gate, uint16_t *out, int64_t rows, int64_t cols,
                            int64_t rows_per_batch, int64_t mod_batch_stride, int dtype)
{
    if (!mod_args_ok(rows, cols, rows_per_batch, mod_batch_stride) || (dtype != 0 && dtype != 1))
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / rows_per_batch;
        for (int64_t c = 0; c < cols; ++c) {
            float g = st_to_f32(f32_to_st(st_to_f32(gate[b * mod_batch_stride + c], dtype) *
                                              st_to_f32(update[r * cols + c], dtype), dtype), dtype);
            out[r * cols + c] = f32_to_st(st_to_f32(residual[r * cols + c], dtype) + g, dtype);
        }
    }
    return OR_OK;
}

/* h = bf16(residual + bf16(gate * update)). */
int oracle_gate_residual(const uint16_t *update, const uint16_t *residual,
                         const uint16_t *gate, uint16_t *h, int64_t rows, int64_t cols,
                         int64_t rows_per_batch, int64_t mod_batch_stride)
{
    if (!mod_args_ok(rows, cols, rows_per_batch, mod_batch_stride))
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / rows_per_batch;
        for (int64_t c = 0; c < cols; ++c)
            h[r * cols + c] = gate_residual(residual[r * cols + c],
                                            gate[b * mod_batch_stride + c],
                                            update[r * cols + c]);
    }
    return OR_OK;
}

/* xb = bf16(x + bf16(bias[c])) over [rows, channels]. */
int oracle_bias_add(const uint16_t *x, const float *bias, uint16_t *xb, int64_t rows,
                    int64_t channels)
{
    if (rows < 0 || channels <= 0)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < channels; ++c)
            xb[r * channels + c] = bias_add(x[r * channels + c], bias[c]);
    return OR_OK;
}

/* out = bf16(SiLU((xb * rstd) * gamma)) given per-row fp32 rstd. */
int oracle_silu_normalize(const uint16_t *xb, const float *rstd, const float *gamma,
                          uint16_t *out, int64_t rows, int64_t channels)
{
    if (rows < 0 || channels <= 0)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < channels; ++c) {
            float t = bf16_to_f32(xb[r * channels + c]) * rstd[r];
            t = t * gamma[c];
            out[r * channels + c] = silu_bf16(t);
        }
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* Exported: the composites, one per library entry point                     */
/* ------------------------------------------------------------------------- */

/* LN (no affine) + modulate.  mean_out / rstd_out / y_out may be NULL. */
int oracle_ln_modulate(const uint16_t *x, const uint16_t *scale, const uint16_t *shift,
                       uint16_t *out, int64_t rows, int64_t cols, int64_t rows_per_batch,
                       int64_t mod_batch_stride, float eps, float *mean_out,
                       float *rstd_out, uint16_t *y_out)
{
    if (!mod_args_ok(rows, cols, rows_per_batch, mod_batch_stride))
        return OR_INVALID;
    if (cols > OR_MAX_COLS)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = widen_row(x + r * cols, cols);
        int64_t b = r / rows_per_batch;
        float mean, rstd;
        ln_stats(xr, cols, eps, &mean, &rstd);
        if (mean_out)
            mean_out[r] = mean;
        if (rstd_out)
            rstd_out[r] = rstd;
        for (int64_t c = 0; c < cols; ++c) {
            uint16_t y = ln_normalize(xr[c], mean, rstd);
            if (y_out)
                y_out[r * cols + c] = y;
            out[r * cols + c] = modulate(y, scale[b * mod_batch_stride + c],
                                         shift[b * mod_batch_stride + c]);
        }
    }
    return OR_OK;
}

/* LN with the modulate folded into its affine (lossy form).  mean_out /
 * rstd_out may be NULL. */
int oracle_ln_modulate_folded(const uint16_t *x, const uint16_t *scale, const uint16_t *shift,
                              uint16_t *out, int64_t rows, int64_t cols, int64_t rows_per_batch,
                              int64_t mod_batch_stride, float eps, float *mean_out,
                              float *rstd_out)
{
    if (!mod_args_ok(rows, cols, rows_per_batch, mod_batch_stride))
        return OR_INVALID;
    if (cols > OR_MAX_COLS)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = widen_row(x + r * cols, cols);
        int64_t b = r / rows_per_batch;
        float mean, rstd;
        ln_stats(xr, cols, eps, &mean, &rstd);
        if (mean_out)
            mean_out[r] = mean;
        if (rstd_out)
            rstd_out[r] = rstd;
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = ln_modulate_folded(xr[c], mean, rstd,
                                                   scale[b * mod_batch_stride + c],
                                                   shift[b * mod_batch_stride + c]);
    }
    return OR_OK;
}

/* The fixed fp32 token-sum tree: v[0..n-1] is reduced in place by adjacent
 * pairs within groups of 32 (a short group padded with +0), group by group,
 * level after level, until one value remains.  n == 0 gives +0. */
static float tree32_sum(float *v, int64_t n)
{
    if (n == 0)
        return 0.0f;
    while (n > 1) {
        int64_t groups = (n + 31) / 32;
        for (int64_t g = 0; g < groups; ++g) {
            float t[32];
            for (int i = 0; i < 32; ++i) {
                int64_t k = g * 32 + i;
                t[i] = k < n ? v[k] : 0.0f;
            }
            for (int width = 16; width >= 1; width /= 2)
                for (int i = 0; i < width; ++i)
                    t[i] = t[2 * i] + t[2 * i + 1];
            v[g] = t[0];
        }
        n = groups;
    }
    return v[0];
}

/* Exposed for the tests: the fixed tree over n fp32 values (v is clobbered). */
float oracle_tree32_sum(float *v, int64_t n)
{
    return tree32_sum(v, n);
}

/* Backward of LN (no affine) + modulate.  x, d_out: [rows, cols] bf16;
 * scale: [B, cols] bf16 at row stride mod_batch_stride; d_x: bf16 [rows,
 * cols]; d_scale, d_shift: fp32 [B, cols] (dense).  mean_out / rstd_out may be
 * NULL. */
/* One value of a backward operand: dtype 0 bf16 (uint16 bit patterns), 2 fp32. */
static float bwd_ld(const void *p, int64_t i, int dtype)
{
    return dtype == 2 ? ((const float *)p)[i] : bf16_to_f32(((const uint16_t *)p)[i]);
}

/* The backward over a storage type (0 bf16, 2 fp32); d_x is the binary64
 * value rounded once to that type. */
static int ln_modulate_backward_dt(const void *x, const void *scale, const void *d_out,
                                   int64_t rows, int64_t cols, int64_t rows_per_batch,
                                   int64_t mod_batch_stride, float eps, void *d_x,
                                   float *d_scale, float *d_shift, float *mean_out,
                                   float *rstd_out, int dtype)
{
    if (!mod_args_ok(rows, cols, rows_per_batch, mod_batch_stride))
        return OR_INVALID;
    if (cols > OR_MAX_COLS)
        return OR_INVALID;
    int64_t nb = rows / rows_per_batch;
    float *mean = (float *)malloc(sizeof(float) * (size_t)(rows > 0 ? rows : 1));
    float *rstd = (float *)malloc(sizeof(float) * (size_t)(rows > 0 ? rows : 1));
    float *xr = (float *)malloc(sizeof(float) * (size_t)cols);
    float *ts = (float *)malloc(sizeof(float) * (size_t)(rows_per_batch > 0 ? rows_per_batch : 1));
    float *tc = (float *)malloc(sizeof(float) * (size_t)(rows_per_batch > 0 ? rows_per_batch : 1));
    if (!mean || !rstd || !xr || !ts || !tc) {
        free(mean); free(rstd); free(xr); free(ts); free(tc);
        return OR_INVALID;
    }
    /* per row: statistics and d_x */
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c)
            xr[c] = bwd_ld(x, r * cols + c, dtype);
        int64_t so = (r / rows_per_batch) * mod_batch_stride;
        ln_stats(xr, cols, eps, &mean[r], &rstd[r]);
        if (mean_out)
            mean_out[r] = mean[r];
        if (rstd_out)
            rstd_out[r] = rstd[r];
        double m = (double)mean[r], rs = (double)rstd[r];
        double c1 = 0.0, c2 = 0.0;
        for (int64_t c = 0; c < cols; ++c) {
            double xh = ((double)xr[c] - m) * rs;
            double g = (double)bwd_ld(d_out, r * cols + c, dtype) *
                       (double)(1.0f + bwd_ld(scale, so + c, dtype));
            c1 += g;
            c2 += g * xh;
        }
        c1 /= (double)cols;
        c2 /= (double)cols;
        for (int64_t c = 0; c < cols; ++c) {
            double xh = ((double)xr[c] - m) * rs;
            double g = (double)bwd_ld(d_out, r * cols + c, dtype) *
                       (double)(1.0f + bwd_ld(scale, so + c, dtype));
            double v = rs * (g - c1 - xh * c2);
            if (dtype == 2)
                ((float *)d_x)[r * cols + c] = (float)v;
            else
                ((uint16_t *)d_x)[r * cols + c] = f64_to_bf16(v);
        }
    }
    /* per batch and column: the two token sums */
    for (int64_t b = 0; b < nb; ++b) {
        for (int64_t c = 0; c < cols; ++c) {
            for (int64_t s = 0; s < rows_per_batch; ++s) {
                int64_t r = b * rows_per_batch + s;
                float dout = bwd_ld(d_out, r * cols + c, dtype);
                float xh = rstd[r] * (bwd_ld(x, r * cols + c, dtype) - mean[r]);
                ts[s] = dout;
                tc[s] = dout * xh;
            }
            d_shift[b * cols + c] = tree32_sum(ts, rows_per_batch);
            d_scale[b * cols + c] = tree32_sum(tc, rows_per_batch);
        }
    }
    free(mean); free(rstd); free(xr); free(ts); free(tc);
    return OR_OK;
}

int oracle_ln_modulate_backward(const uint16_t *x, const uint16_t *scale, const uint16_t *d_out,
                                int64_t rows, int64_t cols, int64_t rows_per_batch,
                                int64_t mod_batch_stride, float eps, uint16_t *d_x,
                                float *d_scale, float *d_shift, float *mean_out,
                                float *rstd_out)
{
    return ln_modulate_backward_dt(x, scale, d_out, rows, cols, rows_per_batch, mod_batch_stride,
                                   eps, d_x, d_scale, d_shift, mean_out, rstd_out, 0);
}

/* The fp32 stream ("[WS1][Qwen-Image][CUDA] Final AdaLN output
 * (final_adaln_out)", the FP32 column of its forward + backward table and
 * its BF16/FP32 accuracy gates): the same computation on fp32 x, scale and
 * d_out, d_x rounded once from binary64 to fp32. */
int oracle_ln_modulate_backward_f32(const float *x, const float *scale, const float *d_out,
                                    int64_t rows, int64_t cols, int64_t rows_per_batch,
                                    int64_t mod_batch_stride, float eps, float *d_x,
                                    float *d_scale, float *d_shift, float *mean_out,
                                    float *rstd_out)
{
    return ln_modulate_backward_dt(x, scale, d_out, rows, cols, rows_per_batch, mod_batch_stride,
                                   eps, d_x, d_scale, d_shift, mean_out, rstd_out, 2);
}

/* Gated residual, then LN (no affine) + modulate on h.  Writes h and out. */
int oracle_gated_ln_modulate(const uint16_t *update, const uint16_t *residual,
                             const uint16_t *gate, const uint16_t *scale,
                             const uint16_t *shift, uint16_t *residual_out, uint16_t *out,
                             int64_t rows, int64_t cols, int64_t rows_per_batch,
                             int64_t mod_batch_stride, float eps, float *mean_out,
                             float *rstd_out, uint16_t *y_out)
{
    if (!mod_args_ok(rows, cols, rows_per_batch, mod_batch_stride))
        return OR_INVALID;
    int rc = oracle_gate_residual(update, residual, gate, residual_out, rows, cols,
                                  rows_per_batch, mod_batch_stride);
    if (rc != OR_OK)
        return rc;
    return oracle_ln_modulate(residual_out, scale, shift, out, rows, cols, rows_per_batch,
                              mod_batch_stride, eps, mean_out, rstd_out, y_out);
}

/* [gated residual], weighted RMSNorm + modulate.  residual/gate/residual_out
 * are all NULL (plain site) or all non-NULL (gated site). */
int oracle_rms_modulate(const uint16_t *x, const uint16_t *weight, const uint16_t *scale,
                        const uint16_t *shift, uint16_t *out, const uint16_t *residual,
                        const uint16_t *gate, uint16_t *residual_out, int64_t rows,
                        int64_t cols, int64_t rows_per_batch, int64_t mod_batch_stride,
                        float eps, float *rstd_out, uint16_t *y_out)
{
    if (!mod_args_ok(rows, cols, rows_per_batch, mod_batch_stride) || cols > OR_MAX_COLS)
        return OR_INVALID;
    int gated = residual != NULL;
    if (gated != (gate != NULL) || gated != (residual_out != NULL))
        return OR_INVALID;
    const uint16_t *src = x;
    if (gated) {
        int rc = oracle_gate_residual(x, residual, gate, residual_out, rows, cols,
                                      rows_per_batch, mod_batch_stride);
        if (rc != OR_OK)
            return rc;
        src = residual_out;
    }
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = widen_row(src + r * cols, cols);
        int64_t b = r / rows_per_batch;
        float rstd;
        rms_stats(xr, cols, eps, &rstd);
        if (rstd_out)
            rstd_out[r] = rstd;
        for (int64_t c = 0; c < cols; ++c) {
            uint16_t y = rms_normalize(xr[c], rstd, bf16_to_f32(weight[c]));
            if (y_out)
                y_out[r * cols + c] = y;
            out[r * cols + c] = modulate(y, scale[b * mod_batch_stride + c],
                                         shift[b * mod_batch_stride + c]);
        }
    }
    return OR_OK;
}

/* Per-head LN of q rows then k rows.  mean_out / rstd_out: [rows_q + rows_k]. */
int oracle_qk_layernorm(const uint16_t *q, const uint16_t *k, uint16_t *q_out,
                        uint16_t *k_out, int64_t rows_q, int64_t rows_k, int64_t head_dim,
                        float eps, float *mean_out, float *rstd_out)
{
    if (rows_q < 0 || rows_k < 0 || head_dim <= 0 || head_dim > OR_MAX_COLS)
        return OR_INVALID;
    for (int pass = 0; pass < 2; ++pass) {
        const uint16_t *src = pass == 0 ? q : k;
        uint16_t *dst = pass == 0 ? q_out : k_out;
        int64_t rows = pass == 0 ? rows_q : rows_k;
        int64_t base = pass == 0 ? 0 : rows_q;
        for (int64_t r = 0; r < rows; ++r) {
            const float *xr = widen_row(src + r * head_dim, head_dim);
            float mean, rstd;
            ln_stats(xr, head_dim, eps, &mean, &rstd);
            if (mean_out)
                mean_out[base + r] = mean;
            if (rstd_out)
                rstd_out[base + r] = rstd;
            for (int64_t c = 0; c < head_dim; ++c)
                dst[r * head_dim + c] = ln_normalize(xr[c], mean, rstd);
        }
    }
    return OR_OK;
}

/* channels_last [rows = N*D*H*W, C]: [bias], RMS over C, * gamma, SiLU. */
int oracle_rmsnorm_silu_bias(const uint16_t *x, const float *bias, const float *gamma,
                             uint16_t *out, int64_t rows, int64_t channels, float eps,
                             float *rstd_out, uint16_t *xb_out)
{
    if (rows < 0 || channels <= 0 || channels > OR_MAX_COLS)
        return OR_INVALID;
    float *row = row_buf;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * channels;
        for (int64_t c = 0; c < channels; ++c) {
            uint16_t xb = bias ? bias_add(xr[c], bias[c]) : xr[c];
            if (xb_out)
                xb_out[r * channels + c] = xb;
            row[c] = bf16_to_f32(xb);
        }
        float rstd;
        rms_stats(row, channels, eps, &rstd);
        if (rstd_out)
            rstd_out[r] = rstd;
        for (int64_t c = 0; c < channels; ++c) {
            float t = row[c] * rstd;
            t = t * gamma[c];
            out[r * channels + c] = silu_bf16(t);
        }
    }
    return OR_OK;
}

/* Conv-bias epilogue over a storage type ("[Diffusion] Fuse the Wan VAE conv
 * bias epilogue and tile the RMSNorm+SiLU kernel", Modifications and Tests /
 * docs): aten's add_ forms x + bias in fp32 and rounds once to x's type; an
 * fp32 bias on a half-precision x is cast to x's type first; the residual form
 * then adds h the same way.  dtype: 0 bf16, 1 fp16 (x, h, out as uint16 bit
 * patterns), 2 fp32 (as float); bias_dtype: 2 (fp32) or dtype.  With rnd the
 * rounding to dtype (the identity for fp32):
 *     out = rnd(x + rnd(bias)),   then   out = rnd(out + h). */
int oracle_conv_bias_epilogue_dt(const void *x, const void *bias, const void *h, void *out,
                                 int64_t rows, int64_t channels, int dtype, int bias_dtype)
{
    if (rows < 0 || channels <= 0 || dtype < 0 || dtype > 2)
        return OR_INVALID;
    if (bias_dtype != 2 && bias_dtype != dtype)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < channels; ++c) {
            const int64_t i = r * channels + c;
            if (dtype == 2) {
                float v = ((const float *)x)[i] + ((const float *)bias)[c];
                if (h)
                    v = v + ((const float *)h)[i];
                ((float *)out)[i] = v;
                continue;
            }
            /* the bias in x's type: cast from fp32, or as given */
            uint16_t b = bias_dtype == 2 ? f32_to_st(((const float *)bias)[c], dtype)
                                         : ((const uint16_t *)bias)[c];
            float sum = st_to_f32(((const uint16_t *)x)[i], dtype) + st_to_f32(b, dtype);
            uint16_t v = f32_to_st(sum, dtype);
            if (h)
                v = f32_to_st(st_to_f32(v, dtype) + st_to_f32(((const uint16_t *)h)[i], dtype),
                              dtype);
            ((uint16_t *)out)[i] = v;
        }
    return OR_OK;
}

/* Standalone conv-bias epilogue: out = bf16(x + bf16(bias[c])), then, when h
 * is given, out = bf16(out + h). */
int oracle_conv_bias_epilogue(const uint16_t *x, const float *bias, const uint16_t *h,
                              uint16_t *out, int64_t rows, int64_t channels)
{
    if (rows < 0 || channels <= 0)
        return OR_INVALID;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < channels; ++c) {
            uint16_t v = bias_add(x[r * channels + c], bias[c]);
            if (h)
                v = f32_to_bf16(bf16_to_f32(v) + bf16_to_f32(h[r * channels + c]));
            out[r * channels + c] = v;
        }
    return OR_OK;
}
