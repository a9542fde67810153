// Row kernels: per-row LayerNorm (no affine) or weighted RMSNorm, fused with
// the adaLN modulate, with an optional gated-residual stage in front.
//
// What is computed (per row of `cols` bf16 values):
//   gated:  h = bf16(residual + bf16(gate * update)), stored, and used as x
//           (ERNIE-Image fused RMSNorm+scale/shift page, second kernel; the
//           GLM-Image page's ff gate)
//   LN:     mean = fp32(S1/N), rstd = fp32(1/sqrt(M2/N + eps)),
//           y = bf16(rstd * (x - mean))          (GLM-Image page, "What
//           rounding-faithful means here": subtract, multiply, no FMA)
//   RMS:    rstd = fp32(1/sqrt(S2/N + eps)), y = bf16((x * rstd) * w)
//           (ERNIE-Image page, "What rounding-faithful means here")
//   out = bf16(bf16(y * bf16(1 + scale)) + shift)   (the eager modulate's
//           three rounded kernels; FLUX.1 page, Commit 2)
//   FOLD (LN only, the lossy affine-folded form of the FLUX.1 page, Commit 3):
//           out = bf16((rstd * (x - mean)) * bf16(1 + scale) + shift), every
//           op in fp32 on the unrounded normalised value, one rounding
//
// Layout of the work on gfx950.  One workgroup of NT threads (NT/64
// wavefronts) owns one row at a time; thread t holds the 16-byte vectors
// t, t+NT, ..., t+(NV-1)*NT of the row in registers, so the row is read from
// HBM once and both statistics passes run from VGPRs.  Each wavefront reduces
// with DPP (binary64), the NT/64 wave partials combine through LDS in a fixed
// order.  The grid is persistent: a workgroup walks rows b, b+G, b+2G, ...,
// keeps the modulation rows (already rounded to 1+scale) in VGPRs for as long
// as the batch index does not change, and issues the loads of its next row
// before reducing the current one.
#include "device_common.hpp"
#include "launch.hpp"

namespace ditnorm {

template <int NT, int NV, bool RMS, bool GATED, bool FOLD = false>
__global__ __launch_bounds__(NT) void row_kernel(const RowArgs a) {
  constexpr int NW = NT / 64;
  __shared__ double red[2][2][NW];  // [row parity][pass][wave]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int cols = a.cols;
  const int nvec = cols >> 3;
  const double inv_n_exact = (double)cols;  // divisor (exact in binary64)

  int vcol[NV];
  bool ok[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    vcol[k] = (tid + k * NT) * 8;
    ok[k] = (tid + k * NT) < nvec;
  }

  int64_t row = blockIdx.x;
  if (row >= a.rows) return;

  // Modulation rows for the current batch index, as fp32 values that are
  // already bf16-rounded where the eager chain rounds them.
  float s1[NV][8], sh[NV][8], wt[RMS ? NV : 1][8], gt[GATED ? NV : 1][8];
  if constexpr (RMS) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const uint4 zero = {0, 0, 0, 0};
      unpack8(ok[k] ? ld16(a.weight + vcol[k]) : zero, wt[k]);
    }
  }
  int64_t cur_b = -1;

  uint4 nx[NV], nr[GATED ? NV : 1];
  auto load_row = [&](int64_t r) {
    const uint16_t *xp = a.x + r * (int64_t)cols;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const uint4 zero = {0, 0, 0, 0};
      nx[k] = ok[k] ? ld16(xp + vcol[k]) : zero;
    }
    if constexpr (GATED) {
      const uint16_t *rp = a.residual + r * (int64_t)cols;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const uint4 zero = {0, 0, 0, 0};
        nr[k] = ok[k] ? ld16(rp + vcol[k]) : zero;
      }
    }
  };
  load_row(row);

  int parity = 0;
  for (; row < a.rows; row += gridDim.x, parity ^= 1) {
    uint4 cx[NV], cr[GATED ? NV : 1];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      cx[k] = nx[k];
      if constexpr (GATED) cr[k] = nr[k];
    }
    const int64_t next = row + gridDim.x;
    if (next < a.rows) load_row(next);

    const int64_t b = row / a.rows_per_batch;
    if (b != cur_b) {
      cur_b = b;
      const int64_t mo = b * a.mod_stride;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const uint4 zero = {0, 0, 0, 0};
        unpack8(ok[k] ? ld16(a.scale + mo + vcol[k]) : zero, s1[k]);
        unpack8(ok[k] ? ld16(a.shift + mo + vcol[k]) : zero, sh[k]);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          s1[k][e] = 1.0f + s1[k][e];
          s1[k][e + 1] = 1.0f + s1[k][e + 1];
          round2(s1[k][e], s1[k][e + 1]);
        }
        if constexpr (GATED) unpack8(ok[k] ? ld16(a.gate + mo + vcol[k]) : zero, gt[k]);
      }
    }

    // ---- gated residual: h = bf16(residual + bf16(gate * update)) -------
    float v[NV][8];
#pragma unroll
    for (int k = 0; k < NV; ++k) unpack8(cx[k], v[k]);
    if constexpr (GATED) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        float r8[8];
        unpack8(cr[k], r8);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float g0 = gt[k][e] * v[k][e], g1 = gt[k][e + 1] * v[k][e + 1];
          round2(g0, g1);
          float h0 = r8[e] + g0, h1 = r8[e + 1] + g1;
          round2(h0, h1);
          v[k][e] = h0;
          v[k][e + 1] = h1;
        }
        if (ok[k]) st16(a.residual_out + row * (int64_t)cols + vcol[k], pack8(v[k]));
      }
    }

    // ---- statistics (binary64 accumulation, fp32 results) ---------------
    float mean_f = 0.0f, rstd_f;
    if constexpr (RMS) {
      double s2 = 0.0;
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double d = (double)v[k][e];
          s2 = __builtin_fma(d, d, s2);  // padding lanes hold 0
        }
      s2 = sum64(s2);
      if constexpr (NW > 1) {
        if (lane == 0) red[parity][0][wid] = s2;
        lds_barrier();
        s2 = red[parity][0][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) s2 += red[parity][0][w];
      }
      rstd_f = rstd_from(s2 / inv_n_exact + (double)a.eps);
    } else {
      double s1d = 0.0;
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) s1d += (double)v[k][e];
      s1d = sum64(s1d);
      if constexpr (NW > 1) {
        if (lane == 0) red[parity][0][wid] = s1d;
        lds_barrier();
        s1d = red[parity][0][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) s1d += red[parity][0][w];
      }
      const double mean_d = s1d / inv_n_exact;
      double m2 = 0.0;
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double d = (double)v[k][e] - mean_d;
          m2 = ok[k] ? __builtin_fma(d, d, m2) : m2;
        }
      m2 = sum64(m2);
      if constexpr (NW > 1) {
        if (lane == 0) red[parity][1][wid] = m2;
        lds_barrier();
        m2 = red[parity][1][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) m2 += red[parity][1][w];
      }
      mean_f = (float)mean_d;
      rstd_f = rstd_from(m2 / inv_n_exact + (double)a.eps);
    }
    if (tid == 0) {
      if (a.mean_out) a.mean_out[row] = mean_f;
      if (a.rstd_out) a.rstd_out[row] = rstd_f;
    }

    // ---- normalise, modulate, store --------------------------------------
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float y[8], o[8];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float y0, y1;
        if constexpr (FOLD) {
          const float t0 = rstd_f * (v[k][e] - mean_f), t1 = rstd_f * (v[k][e + 1] - mean_f);
          const float p0 = t0 * s1[k][e], p1 = t1 * s1[k][e + 1];
          o[e] = p0 + sh[k][e];
          o[e + 1] = p1 + sh[k][e + 1];
          continue;
        }
        if constexpr (RMS) {
          y0 = (v[k][e] * rstd_f) * wt[k][e];
          y1 = (v[k][e + 1] * rstd_f) * wt[k][e + 1];
        } else {
          y0 = rstd_f * (v[k][e] - mean_f);
          y1 = rstd_f * (v[k][e + 1] - mean_f);
        }
        round2(y0, y1);
        y[e] = y0;
        y[e + 1] = y1;
        float p0 = y0 * s1[k][e], p1 = y1 * s1[k][e + 1];
        round2(p0, p1);
        o[e] = p0 + sh[k][e];
        o[e + 1] = p1 + sh[k][e + 1];
      }
      if (ok[k]) {
        const int64_t off = row * (int64_t)cols + vcol[k];
        st16(a.out + off, pack8(o));
        if (!FOLD && a.y_out) st16(a.y_out + off, pack8(y));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One wavefront per row (rows of up to 4096 columns)
// ---------------------------------------------------------------------------
//
// A workgroup of four wavefronts owns four consecutive rows, one per
// wavefront.  Lane l holds the row's 16-byte vectors l, l+64, ...,
// l+64*(NV-1) as packed bf16 (NV*4 VGPRs).  The statistics are one pass of
// binary64 moments (sum and sum of squares, exact for bf16 rows) reduced
// across the wavefront with DPP, so a row needs no LDS traffic and no
// barrier of its own.  The grid is one-shot -- rows/4 workgroups -- and the
// register and LDS budgets are kept low enough that every row of a launch
// the size of the pages' workloads is resident at once: all loads are issued
// at the start and the launch streams at the rate HBM delivers.
//
// The modulation rows are converted once per workgroup: s1 = bf16(1 + scale)
// goes to LDS as fp32, laid out so that the 64 lanes of a wavefront read 64
// consecutive 16-byte words (no bank conflicts); the shift likewise (fp32)
// for LN and as its bf16 bits for RMS, whose weight is staged as bf16 too --
// 16-byte words, one per lane, again consecutive.  A row whose batch index
// differs from the workgroup's first row (batched modulation with a batch
// boundary inside the workgroup) reads its modulation row directly.

// fp32 slot of element half h (0: elements 0-3, 1: 4-7) of vector j.
__device__ __forceinline__ int mod_slot(int j, int h) {
  return (((j >> 6) * 2 + h) * 64 + (j & 63)) * 4;
}

// A compile-time bool as a type: run-time choices dispatched to generic
// lambdas, so that they are taken once outside the unrolled loops.
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};
template <int N>
struct IntC {
  static constexpr int value = N;
};

// How a row kernel obtains its modulation operands (s1 = bf16(1+scale),
// shift, the RMS weight; the gate always per vector from the caches).
enum ModMode : int {
  MOD_SERIAL = 0,  // per 16-byte vector, from the caches, as each is needed
  MOD_LDS = 1,     // staged once per workgroup in LDS (see above)
};

template <int NV, bool FULL, bool RMS, bool GATED, int MODE = MOD_LDS, bool FOLD = false>
__global__ __launch_bounds__(256) void row_wave_kernel(const RowArgs a) {
  constexpr int WPB = 4;  // wavefronts (rows) per workgroup
  constexpr int NT = 64 * WPB;
  constexpr bool MODLDS = MODE == MOD_LDS;
  constexpr bool WLDS = MODLDS && RMS;  // RMS: the shift and the weight staged as bf16
  // gated rows: every gate load ahead of the residual stores in the LN forms
  // whose register footprint it leaves alone (measured: the RMS forms and
  // the masked LN forms of 5-8 vectors per lane lost a wavefront per SIMD or
  // ran slower with it)
  constexpr bool GFIRST = !RMS && (FULL || NV <= 4);
  __shared__ float4 lds_s1[MODLDS ? NV * 128 : 1], lds_sh[(MODLDS && !RMS) ? NV * 128 : 1];
  __shared__ uint4 lds_sh16[WLDS ? NV * 64 : 1], lds_w[WLDS ? NV * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int cols = a.cols;
  const int nvec = cols >> 3;
  const int64_t row0 = (int64_t)blockIdx.x * WPB;
  const int64_t row = row0 + wave_id();
  const bool live = row < a.rows;
  const int64_t base = row * (int64_t)cols;
  const uint4 zero = {0, 0, 0, 0};
  auto ok = [&](int k) { return FULL || lane + 64 * k < nvec; };
  auto col = [&](int k) { return (lane + 64 * k) * 8; };

  // Modulation rows of the workgroup's first batch (cache-resident), issued
  // before the row loads.  The loads sit under branches (rows past the end,
  // vectors past the row), so the compiler's wait before the LDS staging
  // covers the whole row too, and the workgroup's wavefronts pass the staging
  // barrier together once their rows have arrived.  Unconditional loads at
  // clamped addresses, which let the staging and the barrier overlap the row
  // still in flight, measured slower (FLUX LN 11.0 -> 11.9 us, 4096 rows of
  // 4096 12.6 -> 13.7 us).
  constexpr int FILL = MODLDS ? (NV * 64 + NT - 1) / NT : 0;
  const int64_t b0 = row0 / a.rows_per_batch;
  uint4 fsc[FILL > 0 ? FILL : 1], fsh[FILL > 0 ? FILL : 1], fw[WLDS ? FILL : 1];
#pragma unroll
  for (int i = 0; i < FILL; ++i) {
    const int j = threadIdx.x + NT * i;
    const bool in = j < nvec;
    fsc[i] = in ? ld16(a.scale + b0 * a.mod_stride + j * 8) : zero;
    fsh[i] = in ? ld16(a.shift + b0 * a.mod_stride + j * 8) : zero;
    if constexpr (WLDS) fw[i] = in ? ld16(a.weight + j * 8) : zero;
  }

  // this wavefront's row
  uint4 xv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) xv[k] = (live && ok(k)) ? ld16s(a.x + base + col(k)) : zero;
  uint4 rv[GATED ? NV : 1];
  if constexpr (GATED) {
#pragma unroll
    for (int k = 0; k < NV; ++k)
      rv[k] = (live && ok(k)) ? ld16s(a.residual + base + col(k)) : zero;
  }
  const int64_t mo = (row / a.rows_per_batch) * a.mod_stride;

  // stage s1 = bf16(1 + scale) in LDS as fp32, the shift as fp32 (LN) or as
  // bf16 with the weight (RMS)
#pragma unroll
  for (int i = 0; i < FILL; ++i) {
    const int j = threadIdx.x + NT * i;
    if (j >= NV * 64) break;
    float sc[8];
    unpack8(fsc[i], sc);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      sc[e] = 1.0f + sc[e];
      sc[e + 1] = 1.0f + sc[e + 1];
      round2(sc[e], sc[e + 1]);
    }
    lds_s1[mod_slot(j, 0) / 4] = make_float4(sc[0], sc[1], sc[2], sc[3]);
    lds_s1[mod_slot(j, 1) / 4] = make_float4(sc[4], sc[5], sc[6], sc[7]);
    if constexpr (WLDS) {
      lds_sh16[j] = fsh[i];
      lds_w[j] = fw[i];
    } else {
      float sh[8];
      unpack8(fsh[i], sh);
      lds_sh[mod_slot(j, 0) / 4] = make_float4(sh[0], sh[1], sh[2], sh[3]);
      lds_sh[mod_slot(j, 1) / 4] = make_float4(sh[4], sh[5], sh[6], sh[7]);
    }
  }
  if constexpr (MODLDS) lds_barrier();
  if (!live) return;  // whole wavefront; no barrier follows
  const bool mod_in_lds = MODLDS && (mo == b0 * a.mod_stride);

  // gated residual: h = bf16(residual + bf16(gate * update)), stored
  if constexpr (GATED) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float u[8], r[8], g[8];
      unpack8(xv[k], u);
      unpack8(rv[k], r);
      unpack8(ok(k) ? ld16(a.gate + mo + col(k)) : zero, g);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float g0 = g[e] * u[e], g1 = g[e + 1] * u[e + 1];
        round2(g0, g1);
        u[e] = r[e] + g0;
        u[e + 1] = r[e + 1] + g1;
      }
      xv[k] = pack8(u);
      if (!GFIRST && ok(k)) st16s(a.residual_out + base + col(k), xv[k]);
    }
    // GFIRST: stored after every gate load has been issued (a store between
    // them orders each load behind it, a cache round trip per vector)
    if constexpr (GFIRST) {
#pragma unroll
      for (int k = 0; k < NV; ++k)
        if (ok(k)) st16s(a.residual_out + base + col(k), xv[k]);
    }
  }

  // statistics: one pass of binary64 moments (padding vectors hold zeros).
  // The widened row stays in registers for the normalise pass.
  Moments m = {0.0, 0.0};
  float xf[NV][8];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    unpack8(xv[k], xf[k]);
#pragma unroll
    for (int e = 0; e < 8; ++e) accumulate(m, xf[k][e]);
  }
  const double n_d = (double)cols;
  const double s2 = sum64(m.s2);
  float mean_f = 0.0f, rstd_f;
  if constexpr (RMS) {
    rstd_f = rstd_from(s2 / n_d + (double)a.eps);
  } else {
    const double s1 = sum64(m.s1);
    const double mean_d = s1 / n_d;
    const double var_d = clamp_var(__builtin_fma(-s1, mean_d, s2) / n_d);
    mean_f = (float)mean_d;
    rstd_f = rstd_from(var_d + (double)a.eps);
  }
  if (lane == 0) {
    if (a.mean_out) a.mean_out[row] = mean_f;
    if (a.rstd_out) a.rstd_out[row] = rstd_f;
  }

  // normalise, modulate, store.  The two run-time choices (debug output,
  // modulation source) are taken once, outside the loop, so the unrolled
  // loop is one basic block the scheduler can interleave freely.
  auto normalise = [&](auto with_y, auto from_lds) {
    constexpr bool WY = decltype(with_y)::value, FROM_LDS = decltype(from_lds)::value;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!ok(k)) continue;
      float s1v[8], shv[8], y[8], o[8];
      const float *v = xf[k];
      if constexpr (FROM_LDS) {
        const int j = lane + 64 * k;
        const float4 a0 = lds_s1[mod_slot(j, 0) / 4], a1 = lds_s1[mod_slot(j, 1) / 4];
        s1v[0] = a0.x; s1v[1] = a0.y; s1v[2] = a0.z; s1v[3] = a0.w;
        s1v[4] = a1.x; s1v[5] = a1.y; s1v[6] = a1.z; s1v[7] = a1.w;
        if constexpr (WLDS) {
          unpack8(lds_sh16[j], shv);
        } else {
          const float4 c0 = lds_sh[mod_slot(j, 0) / 4], c1 = lds_sh[mod_slot(j, 1) / 4];
          shv[0] = c0.x; shv[1] = c0.y; shv[2] = c0.z; shv[3] = c0.w;
          shv[4] = c1.x; shv[5] = c1.y; shv[6] = c1.z; shv[7] = c1.w;
        }
      } else {
        unpack8(ld16(a.scale + mo + col(k)), s1v);
        unpack8(ld16(a.shift + mo + col(k)), shv);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          s1v[e] = 1.0f + s1v[e];
          s1v[e + 1] = 1.0f + s1v[e + 1];
          round2(s1v[e], s1v[e + 1]);
        }
      }
      if constexpr (FOLD) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = rstd_f * (v[e] - mean_f);
          const float p = t * s1v[e];
          o[e] = p + shv[e];
        }
        st16s(a.out + base + col(k), pack8(o));
        continue;
      }
      if constexpr (RMS) {
        float w[8];
        if constexpr (WLDS) {
          unpack8(lds_w[lane + 64 * k], w);
        } else {
          unpack8(ld16(a.weight + col(k)), w);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (v[e] * rstd_f) * w[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = rstd_f * (v[e] - mean_f);
      }
      uint4 yq;  // y as stored bf16
      if constexpr (WY) {
        yq = pack8(y);
        unpack8(yq, y);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = round1(y[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float p0 = y[e] * s1v[e], p1 = y[e + 1] * s1v[e + 1];
        round2(p0, p1);
        o[e] = p0 + shv[e];
        o[e + 1] = p1 + shv[e + 1];
      }
      st16s(a.out + base + col(k), pack8(o));
      if constexpr (WY) st16(a.y_out + base + col(k), yq);
    }
  };
  using T = BoolC<true>;
  using F = BoolC<false>;
  if (a.y_out) {
    if (mod_in_lds) normalise(T{}, T{});
    else normalise(T{}, F{});
  } else {
    if (mod_in_lds) normalise(F{}, T{});
    else normalise(F{}, F{});
  }
}

// ---------------------------------------------------------------------------
// Balanced variant: whole rows for whole rounds, split rows for the remainder
// ---------------------------------------------------------------------------
//
// A launch lasts as long as its busiest SIMD.  With one wavefront per row,
// 4608 rows put 5 rows on half of the 1024 SIMDs and 4 on the rest, and the
// launch takes as long as 5120 rows would (measured: 4096 rows of 3072 in
// 9.7 us, 4608 and 5120 rows both 13.5 us).  Here the first rows go one per
// wavefront in whole rounds (full_blocks workgroups of 4 rows) and the
// remaining rows are split into P segments, one wavefront each: halves (P =
// 2, a workgroup of 4 wavefronts taking 2 rows), so 4608 rows are 4 whole
// rows plus one half row per SIMD; or, when the remainder is at most a
// quarter round, quarters (P = 4, a workgroup per row), so 4216 rows of 4096
// are 4 whole rows plus a quarter row on 480 SIMDs instead of a half row on
// 240.  A launch with no whole round (at most a quarter or half a round of
// rows in all) splits every row.  The segments' binary64 moments meet through
// LDS; the sums are exact, so the statistics carry the same bits either way.
// Everything else is the wavefront-per-row kernel's MOD_LDS path (rows of
// NV * 512 columns).
template <int NVW, int NV, bool RMS, bool GATED, int WPB, bool GFIRST, bool FOLD = false,
          int TP = 0>
__device__ __forceinline__ void row_segment(const RowArgs &a, float4 *lds_s1, float4 *lds_sh,
                                            uint4 *lds_sh16, uint4 *lds_w, float4 *lds_w32,
                                            uint4 *lds_s116,
                                            double (*red)[2], int64_t row0, int64_t row, int seg,
                                            int64_t trow0 = -1) {
  constexpr bool SPLIT = NVW != NV;
  // TP > 0 (whole rows, plain forms): the workgroup also owns the WPB / TP
  // remainder rows from trow0 on (none if trow0 is negative), a 1/TP part
  // per wavefront, loaded ahead of the whole row and finished after it
  static_assert(TP == 0 || (!SPLIT && !GATED && !FOLD && WPB % TP == 0 && NV % TP == 0),
                "tail: whole plain rows");
  constexpr int TPD = TP > 0 ? TP : 1;
  constexpr int NVT = NV / TPD;
  constexpr int NT = 64 * WPB;
  // RMS with 8-wavefront workgroups: the shift and the weight staged as fp32
  constexpr bool F32W = RMS && WPB == 8;
  // rows over 4096 columns: s1, the shift and the weight staged as bf16
  // vectors (s1 is already a bf16 value), half the LDS of fp32 copies, so
  // that four or five workgroups fit a compute unit instead of three
  constexpr bool B16 = NV > 8;
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int cols = a.cols;
  const bool live = row < a.rows;
  const int64_t base = (live ? row : row0) * (int64_t)cols;
  const uint4 zero = {0, 0, 0, 0};
  auto vid = [&](int k) { return seg * (NVW * 64) + lane + 64 * k; };
  auto col = [&](int k) { return vid(k) * 8; };
  const int tpart = w % TPD;                   // this wavefront's part of its tail row
  const int64_t trow = trow0 + w / TPD;
  const bool tail = TP > 0 && trow0 >= 0 && trow < a.rows;  // uniform over the part's wavefronts
  const int64_t tbase = (tail ? trow : (live ? row : row0)) * (int64_t)cols;
  uint4 tv[NVT];
  if constexpr (TP > 0) {  // unconditional (a wavefront without a tail reads its own row)
#pragma unroll
    for (int k = 0; k < NVT; ++k)
      tv[k] = ld16s(a.x + tbase + (tpart * (NVT * 64) + lane + 64 * k) * 8);
  }

  // modulation rows of the workgroup's first batch, then this segment
  constexpr int FILL = (NV * 64 + NT - 1) / NT;
  const int64_t b0 = row0 / a.rows_per_batch;
  uint4 fsc[FILL], fsh[FILL], fw[RMS ? FILL : 1];
#pragma unroll
  for (int i = 0; i < FILL; ++i) {
    const int j = threadIdx.x + NT * i;
    const bool in = j < NV * 64;
    fsc[i] = in ? ld16(a.scale + b0 * a.mod_stride + j * 8) : zero;
    fsh[i] = in ? ld16(a.shift + b0 * a.mod_stride + j * 8) : zero;
    if constexpr (RMS) fw[i] = in ? ld16(a.weight + j * 8) : zero;
  }
  uint4 xv[NVW], rv[GATED ? NVW : 1];
#pragma unroll
  for (int k = 0; k < NVW; ++k) xv[k] = live ? ld16s(a.x + base + col(k)) : zero;
  if constexpr (GATED) {
#pragma unroll
    for (int k = 0; k < NVW; ++k) rv[k] = live ? ld16s(a.residual + base + col(k)) : zero;
  }
  const int64_t mo = ((live ? row : row0) / a.rows_per_batch) * a.mod_stride;
#pragma unroll
  for (int i = 0; i < FILL; ++i) {
    const int j = threadIdx.x + NT * i;
    if (j >= NV * 64) break;
    float sc[8];
    unpack8(fsc[i], sc);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      sc[e] = 1.0f + sc[e];
      sc[e + 1] = 1.0f + sc[e + 1];
      round2(sc[e], sc[e + 1]);
    }
    if constexpr (B16) {
      lds_s116[j] = pack8(sc);  // exact: sc holds bf16 values
      lds_sh16[j] = fsh[i];
      if constexpr (RMS) lds_w[j] = fw[i];
      continue;
    }
    lds_s1[mod_slot(j, 0) / 4] = make_float4(sc[0], sc[1], sc[2], sc[3]);
    lds_s1[mod_slot(j, 1) / 4] = make_float4(sc[4], sc[5], sc[6], sc[7]);
    if constexpr (F32W) {
      float sh[8], wt[8];
      unpack8(fsh[i], sh);
      unpack8(fw[i], wt);
      lds_sh[mod_slot(j, 0) / 4] = make_float4(sh[0], sh[1], sh[2], sh[3]);
      lds_sh[mod_slot(j, 1) / 4] = make_float4(sh[4], sh[5], sh[6], sh[7]);
      lds_w32[mod_slot(j, 0) / 4] = make_float4(wt[0], wt[1], wt[2], wt[3]);
      lds_w32[mod_slot(j, 1) / 4] = make_float4(wt[4], wt[5], wt[6], wt[7]);
    } else if constexpr (RMS) {
      // shift and weight as bf16, widened where they are used: with the
      // weight staged too, fp32 copies would cost a workgroup of occupancy
      lds_sh16[j] = fsh[i];
      lds_w[j] = fw[i];
    } else {
      float sh[8];
      unpack8(fsh[i], sh);
      lds_sh[mod_slot(j, 0) / 4] = make_float4(sh[0], sh[1], sh[2], sh[3]);
      lds_sh[mod_slot(j, 1) / 4] = make_float4(sh[4], sh[5], sh[6], sh[7]);
    }
  }
  if constexpr (TP > 0) {  // the tail part's moments, exchanged with the staging barrier
    if (tail) {
      Moments mt = {0.0, 0.0};
#pragma unroll
      for (int k = 0; k < NVT; ++k) {
        float tf[8];
        unpack8(tv[k], tf);
#pragma unroll
        for (int e = 0; e < 8; ++e) accumulate(mt, tf[e]);
      }
      const double t2 = sum64(mt.s2), t1 = RMS ? 0.0 : sum64(mt.s1);
      if (lane == 0) {
        red[w][0] = t1;
        red[w][1] = t2;
      }
    }
  }
  // normalise, modulate, store (the run-time choices taken outside the loop)
  auto normalise = [&](auto with_y, auto from_lds, auto nvc, const float (*xs)[8], int sg,
                       int64_t bs, float mean_v, float rstd_v, int64_t mov) {
    constexpr bool WY = decltype(with_y)::value, FROM_LDS = decltype(from_lds)::value;
    constexpr int NC = decltype(nvc)::value;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      float s1v[8], shv[8], y[8], o[8];
      const float *v = xs[k];
      const int j = sg * (NC * 64) + lane + 64 * k;
      const int64_t cj = (int64_t)j * 8;
      if constexpr (FROM_LDS && B16) {
        unpack8(lds_s116[j], s1v);
        unpack8(lds_sh16[j], shv);
      } else if constexpr (FROM_LDS) {
        const float4 a0 = lds_s1[mod_slot(j, 0) / 4], a1 = lds_s1[mod_slot(j, 1) / 4];
        s1v[0] = a0.x; s1v[1] = a0.y; s1v[2] = a0.z; s1v[3] = a0.w;
        s1v[4] = a1.x; s1v[5] = a1.y; s1v[6] = a1.z; s1v[7] = a1.w;
        if constexpr (RMS && !F32W) {
          unpack8(lds_sh16[j], shv);
        } else {
          const float4 c0 = lds_sh[mod_slot(j, 0) / 4], c1 = lds_sh[mod_slot(j, 1) / 4];
          shv[0] = c0.x; shv[1] = c0.y; shv[2] = c0.z; shv[3] = c0.w;
          shv[4] = c1.x; shv[5] = c1.y; shv[6] = c1.z; shv[7] = c1.w;
        }
      } else {
        unpack8(ld16(a.scale + mov + cj), s1v);
        unpack8(ld16(a.shift + mov + cj), shv);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          s1v[e] = 1.0f + s1v[e];
          s1v[e + 1] = 1.0f + s1v[e + 1];
          round2(s1v[e], s1v[e + 1]);
        }
      }
      if constexpr (RMS) {
        float wt[8];
        if constexpr (F32W) {
          const float4 w0 = lds_w32[mod_slot(j, 0) / 4], w1 = lds_w32[mod_slot(j, 1) / 4];
          wt[0] = w0.x; wt[1] = w0.y; wt[2] = w0.z; wt[3] = w0.w;
          wt[4] = w1.x; wt[5] = w1.y; wt[6] = w1.z; wt[7] = w1.w;
        } else {
          unpack8(lds_w[j], wt);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (v[e] * rstd_v) * wt[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = rstd_v * (v[e] - mean_v);
      }
      if constexpr (FOLD) {  // the folded affine: one fp32 chain, one rounding
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = y[e] * s1v[e];
          o[e] = p + shv[e];
        }
        st16s(a.out + bs + cj, pack8(o));
        continue;
      }
      uint4 yq;  // y as stored bf16
      if constexpr (WY) {
        yq = pack8(y);
        unpack8(yq, y);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = round1(y[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float q0 = y[e] * s1v[e], q1 = y[e + 1] * s1v[e + 1];
        round2(q0, q1);
        o[e] = q0 + shv[e];
        o[e + 1] = q1 + shv[e + 1];
      }
      st16s(a.out + bs + cj, pack8(o));
      if constexpr (WY) st16(a.y_out + bs + cj, yq);
    }
  };
  using T = BoolC<true>;
  using F = BoolC<false>;
  if constexpr (!SPLIT) {
    lds_barrier();
    if constexpr (TP > 0) {  // the tail part, finished while the whole row's loads are in flight
      if (tail) {
        const int pw = w - tpart;
        double t1, t2;
        if constexpr (TP == 2) {
          t1 = red[pw][0] + red[pw + 1][0];
          t2 = red[pw][1] + red[pw + 1][1];
        } else if constexpr (TP == 4) {
          t1 = (red[pw][0] + red[pw + 1][0]) + (red[pw + 2][0] + red[pw + 3][0]);
          t2 = (red[pw][1] + red[pw + 1][1]) + (red[pw + 2][1] + red[pw + 3][1]);
        } else {
          static_assert(TP == 8, "tail parts: 2, 4 or 8");
          t1 = ((red[0][0] + red[1][0]) + (red[2][0] + red[3][0])) +
               ((red[4][0] + red[5][0]) + (red[6][0] + red[7][0]));
          t2 = ((red[0][1] + red[1][1]) + (red[2][1] + red[3][1])) +
               ((red[4][1] + red[5][1]) + (red[6][1] + red[7][1]));
        }
        float tmean = 0.0f, trstd;
        if constexpr (RMS) {
          trstd = rstd_from(t2 / (double)cols + (double)a.eps);
        } else {
          const double tm = t1 / (double)cols;
          tmean = (float)tm;
          trstd = rstd_from(clamp_var(__builtin_fma(-t1, tm, t2) / (double)cols) + (double)a.eps);
        }
        if (lane == 0 && tpart == 0) {
          if (a.mean_out) a.mean_out[trow] = tmean;
          if (a.rstd_out) a.rstd_out[trow] = trstd;
        }
        float tf[NVT][8];
#pragma unroll
        for (int k = 0; k < NVT; ++k) unpack8(tv[k], tf[k]);
        const int64_t tmo = (trow / a.rows_per_batch) * a.mod_stride;
        const IntC<NVT> nt;
        if (a.y_out) {
          if (tmo == b0 * a.mod_stride) normalise(T{}, T{}, nt, tf, tpart, tbase, tmean, trstd, tmo);
          else normalise(T{}, F{}, nt, tf, tpart, tbase, tmean, trstd, tmo);
        } else {
          if (tmo == b0 * a.mod_stride) normalise(F{}, T{}, nt, tf, tpart, tbase, tmean, trstd, tmo);
          else normalise(F{}, F{}, nt, tf, tpart, tbase, tmean, trstd, tmo);
        }
      }
    }
    if (!live) return;  // whole wavefront; no barrier follows
  }

  // gated residual: h = bf16(residual + bf16(gate * update)), stored
  if constexpr (GATED) {
#pragma unroll
    for (int k = 0; k < NVW; ++k) {
      float u[8], r[8], g[8];
      unpack8(xv[k], u);
      unpack8(rv[k], r);
      unpack8(ld16(a.gate + mo + col(k)), g);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float g0 = g[e] * u[e], g1 = g[e + 1] * u[e + 1];
        round2(g0, g1);
        u[e] = r[e] + g0;
        u[e + 1] = r[e + 1] + g1;
      }
      xv[k] = pack8(u);
      if (!GFIRST && live) st16s(a.residual_out + base + col(k), xv[k]);
    }
    // GFIRST: stored after every gate load has been issued (a store between
    // them orders each load behind it, a cache round trip per vector)
    if (GFIRST && live) {
#pragma unroll
      for (int k = 0; k < NVW; ++k) st16s(a.residual_out + base + col(k), xv[k]);
    }
  }

  // binary64 moments of the segment; the widened segment stays in registers
  Moments m = {0.0, 0.0};
  float xf[NVW][8];
#pragma unroll
  for (int k = 0; k < NVW; ++k) {
    unpack8(xv[k], xf[k]);
#pragma unroll
    for (int e = 0; e < 8; ++e) accumulate(m, xf[k][e]);
  }
  double s2 = sum64(m.s2);
  double s1 = RMS ? 0.0 : sum64(m.s1);
  if constexpr (SPLIT) {
    if (lane == 0) {
      red[w][0] = s1;
      red[w][1] = s2;
    }
    lds_barrier();  // the staged modulation rows and every segment's moments
    if (!live) return;  // whole wavefront; no barrier follows
    constexpr int P = NV / NVW;  // segments per row: 2, 4 or 8
    const int pw = w & ~(P - 1);
    if constexpr (P == 2) {
      s1 = red[pw][0] + red[pw + 1][0];
      s2 = red[pw][1] + red[pw + 1][1];
    } else if constexpr (P == 4) {
      s1 = (red[pw][0] + red[pw + 1][0]) + (red[pw + 2][0] + red[pw + 3][0]);
      s2 = (red[pw][1] + red[pw + 1][1]) + (red[pw + 2][1] + red[pw + 3][1]);
    } else {
      s1 = ((red[pw][0] + red[pw + 1][0]) + (red[pw + 2][0] + red[pw + 3][0])) +
           ((red[pw + 4][0] + red[pw + 5][0]) + (red[pw + 6][0] + red[pw + 7][0]));
      s2 = ((red[pw][1] + red[pw + 1][1]) + (red[pw + 2][1] + red[pw + 3][1])) +
           ((red[pw + 4][1] + red[pw + 5][1]) + (red[pw + 6][1] + red[pw + 7][1]));
    }
  }
  const double n_d = (double)cols;
  float mean_f = 0.0f, rstd_f;
  if constexpr (RMS) {
    rstd_f = rstd_from(s2 / n_d + (double)a.eps);
  } else {
    const double mean_d = s1 / n_d;
    const double var_d = clamp_var(__builtin_fma(-s1, mean_d, s2) / n_d);
    mean_f = (float)mean_d;
    rstd_f = rstd_from(var_d + (double)a.eps);
  }
  if (lane == 0 && seg == 0) {
    if (a.mean_out) a.mean_out[row] = mean_f;
    if (a.rstd_out) a.rstd_out[row] = rstd_f;
  }
  const bool mod_in_lds = mo == b0 * a.mod_stride;

  const IntC<NVW> nw;
  if (a.y_out) {
    if (mod_in_lds) normalise(T{}, T{}, nw, xf, seg, base, mean_f, rstd_f, mo);
    else normalise(T{}, F{}, nw, xf, seg, base, mean_f, rstd_f, mo);
  } else {
    if (mod_in_lds) normalise(F{}, T{}, nw, xf, seg, base, mean_f, rstd_f, mo);
    else normalise(F{}, F{}, nw, xf, seg, base, mean_f, rstd_f, mo);
  }
}

template <int NV, bool RMS, bool GATED, int P, int WPB = 4, bool REMFIRST = false,
          bool FOLD = false, bool TAIL = false>
__global__ __launch_bounds__(64 * WPB) void row_mixed_kernel(const RowArgs a) {
  constexpr bool F32W = RMS && WPB == 8;
  // gated rows: every gate load ahead of the residual stores, except in the
  // remainder-first launches and the 2048-column LN form (measured faster in
  // the vector-by-vector order there)
  constexpr bool GFIRST = !REMFIRST && !(NV == 4 && !RMS);
  constexpr bool B16 = NV > 8;  // modulation rows staged as bf16 (see row_segment)
  __shared__ float4 lds_s1[B16 ? 1 : NV * 128], lds_sh[(RMS && !F32W) || B16 ? 1 : NV * 128];
  __shared__ uint4 lds_sh16[(RMS && !F32W) || B16 ? NV * 64 : 1];
  __shared__ uint4 lds_w[(RMS && !F32W) || (B16 && RMS) ? NV * 64 : 1];
  __shared__ uint4 lds_s116[B16 ? NV * 64 : 1];
  __shared__ float4 lds_w32[F32W ? NV * 128 : 1];
  __shared__ double red[WPB][2];
  const int w = wave_id();
  int64_t g = blockIdx.x;
  if constexpr (REMFIRST) {  // the remainder's workgroups first in the grid
    const int64_t nrem = (int64_t)gridDim.x - a.full_blocks;
    g = g < nrem ? a.full_blocks + g : g - nrem;
  }
  // (rows over 4096 columns come only in halves: no whole-row path to hold
  // their registers)
  if constexpr (TAIL) {  // whole rows; the first workgroups take WPB / P remainder rows each
    const int64_t row0 = g * WPB;
    const int64_t tr0 = a.full_blocks * WPB + g * (WPB / P);
    row_segment<NV, NV, RMS, GATED, WPB, GFIRST, FOLD, P>(a, lds_s1, lds_sh, lds_sh16, lds_w, lds_w32,
                                                     lds_s116, red, row0, row0 + w, 0,
                                                     tr0 < a.rows ? tr0 : -1);
  } else if (NV <= 8 && g < a.full_blocks) {
    const int64_t row0 = g * WPB;
    if constexpr (NV <= 8)
      row_segment<NV, NV, RMS, GATED, WPB, GFIRST, FOLD>(a, lds_s1, lds_sh, lds_sh16, lds_w, lds_w32,
                                                   lds_s116, red, row0, row0 + w, 0);
  } else if constexpr (P == 2) {  // WPB / 2 rows per workgroup, a half per wavefront
    const int64_t row0 = a.full_blocks * WPB + (g - a.full_blocks) * (WPB / 2);
    row_segment<NV / 2, NV, RMS, GATED, WPB, GFIRST, FOLD>(a, lds_s1, lds_sh, lds_sh16, lds_w, lds_w32,
                                                     lds_s116, red, row0, row0 + (w >> 1), w & 1);
  } else if constexpr (P == 4) {  // WPB / 4 rows per workgroup, a quarter per wavefront
    const int64_t row0 = a.full_blocks * WPB + (g - a.full_blocks) * (WPB / 4);
    row_segment<NV / 4, NV, RMS, GATED, WPB, GFIRST, FOLD>(a, lds_s1, lds_sh, lds_sh16, lds_w, lds_w32,
                                                     lds_s116, red, row0, row0 + (w >> 2), w & 3);
  } else {  // (8-wavefront workgroups) a row per workgroup, an eighth per wavefront
    static_assert(P == 8 && WPB == 8, "eighths: one row per 8-wavefront workgroup");
    const int64_t row0 = a.full_blocks * WPB + (g - a.full_blocks);
    row_segment<NV / 8, NV, RMS, GATED, WPB, GFIRST, FOLD>(a, lds_s1, lds_sh, lds_sh16, lds_w, lds_w32,
                                                     lds_s116, red, row0, row0, w);
  }
}

// Whole rounds of rows (one row per wavefront, one wavefront per SIMD per
// round) and the remainder in eighths when it is at most an eighth of a round
// (the 8-wavefront plain RMS form: a row per workgroup, or with exactly four
// whole rounds a remainder row per whole-row workgroup, see below; ERNIE's
// 120 extra rows of 4096 14.27 -> 14.04 us in their own workgroups, 1-3% at
// other such remainders, bitwise unchanged), in quarters when it is at most
// a quarter round (rows of 2048 or
// 4096 columns), in halves when it is at most half a round;
// else every row whole.  A launch of fewer rows than that (no whole round)
// splits every row the same way, so that it spreads over the SIMDs instead
// of leaving most of them idle.
// The remainder's workgroups go first in the grid for the gated forms at
// 4096 columns with a quarter-round remainder of at least 64 rows.  There four
// whole-row workgroups fill a compute unit, so a remainder dispatched last
// waits for free slots and adds its whole latency as a tail; dispatched first,
// it overlaps the whole rows and only displaces as many of them: gated RMS at
// 4216 rows 26.10 -> 24.55 us, gated LN 26.16 -> 23.99 us, 4160 rows 25.25 ->
// 24.79 / 25.60 -> 24.20 us.  With fewer remainder rows (4112, 4128: 1-5%
// slower), for the plain forms (the displaced whole rows cost more than the
// tail: up to 5% slower) and at other widths (room for the remainder beside
// the whole rows) the remainder stays last.
template <int NV, int WPB, bool R, bool G>
static void launch_mixed_kind(const RowArgs &a, int P, bool remfirst, bool tail, dim3 grid,
                              hipStream_t stream) {
  constexpr int P4 = NV % 4 == 0 ? 4 : 2;
  const dim3 block(64 * WPB);
  if constexpr (WPB == 8 && NV % 8 == 0 && !G) {
    if (tail) {  // (the grid holds the whole-row workgroups only)
      if (P == 8)
        hipLaunchKernelGGL((row_mixed_kernel<NV, R, G, 8, 8, false, false, true>), grid, block, 0,
                           stream, a);
      else
        hipLaunchKernelGGL((row_mixed_kernel<NV, R, G, 4, 8, false, false, true>), grid, block, 0,
                           stream, a);
      return;
    }
  }
  if constexpr (NV == 8 && WPB == 4 && G) {
    if (P == 4 && remfirst) {
      hipLaunchKernelGGL((row_mixed_kernel<NV, R, G, 4, 4, true>), grid, block, 0, stream, a);
      return;
    }
  }
  if constexpr (WPB == 8 && NV % 8 == 0) {
    if (P == 8) {
      hipLaunchKernelGGL((row_mixed_kernel<NV, R, G, 8, 8>), grid, block, 0, stream, a);
      return;
    }
  }
  if (P == 4)
    hipLaunchKernelGGL((row_mixed_kernel<NV, R, G, P4, WPB>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((row_mixed_kernel<NV, R, G, 2, WPB>), grid, block, 0, stream, a);
}

template <int NV, int WPB>
static hipError_t launch_mixed_w(const RowArgs &a0, bool rms, bool gated, const DeviceInfo &dev,
                                 hipStream_t stream, int split = 0) {
  RowArgs a = a0;
  const int64_t simds = (int64_t)dev.num_cu * 4;
  const int64_t whole = split ? 0 : a.rows / simds * simds;
  const int64_t rem = a.rows - whole;
  int64_t blocks;
  int P = 2;
  if (split) {  // every row in `split` segments, whatever the row count
    a.full_blocks = 0;
    P = split;
    blocks = (a.rows + WPB / P - 1) / (WPB / P);
  } else if (WPB == 8 && whole > 0 && rem > 0 && 8 * rem <= simds && NV % 8 == 0) {
    a.full_blocks = whole / WPB;
    blocks = a.full_blocks + rem;  // a row per workgroup, an eighth per wavefront
    P = 8;
  } else if (whole > 0 && rem > 0 && 4 * rem <= simds && NV % 4 == 0) {
    a.full_blocks = whole / WPB;
    blocks = a.full_blocks + (rem + WPB / 4 - 1) / (WPB / 4);
    P = 4;
  } else if (whole > 0 && rem > 0 && 2 * rem <= simds) {
    a.full_blocks = whole / WPB;
    blocks = a.full_blocks + (rem + WPB / 2 - 1) / (WPB / 2);
  } else if (whole == 0 && 4 * rem <= simds && NV % 4 == 0) {
    a.full_blocks = 0;  // fewer rows than a quarter round: every row in quarters
    blocks = (rem + WPB / 4 - 1) / (WPB / 4);
    P = 4;
  } else if (whole == 0 && 2 * rem <= simds) {
    a.full_blocks = 0;  // fewer rows than half a round: every row in halves
    blocks = (rem + WPB / 2 - 1) / (WPB / 2);
  } else {
    a.full_blocks = (a.rows + WPB - 1) / WPB;
    blocks = a.full_blocks;
  }
  const bool remfirst = gated && P == 4 && whole > 0 && rem >= 64;
  // The plain RMS form in 8-wavefront workgroups with exactly four whole
  // rounds -- every SIMD's four resident wavefronts -- and a remainder of at
  // most a quarter round: the remainder rows go to the first whole-row
  // workgroups (WPB / P rows each, a part per wavefront, loaded with the
  // whole row), not to workgroups of their own.  Those had to wait for whole
  // rows to finish, and each staged the 48 KB of modulation rows for a single
  // row: 4100 rows of 4096 13.45 -> 12.61 us, 4160 13.74 -> 12.65, 4216
  // (eighths) 14.01 -> 12.62, 4225 14.37 -> 13.76, 4350 (quarters) 14.85 ->
  // 13.98, bitwise the same.  Halves (4500: 15.13 -> 16.33 us), more whole
  // rounds (5220, 7288, 8292 rows: 2-4% slower) and the 4-wavefront forms
  // (FLUX LN 11.0 -> 11.9 us, where the remainder's workgroups fit beside the
  // whole rows) keep the remainder's own workgroups.
  const bool tail = WPB == 8 && !gated && !split && whole == 4 * simds && rem > 0 &&
                    4 * rem <= simds;
  if (tail) blocks = a.full_blocks;
  const dim3 grid((unsigned)blocks), block(64 * WPB);
  if constexpr (WPB == 8) {  // the plain RMS form only
    launch_mixed_kind<NV, 8, true, false>(a, P, false, tail, grid, stream);
  } else {
    if (!rms && !gated) launch_mixed_kind<NV, 4, false, false>(a, P, remfirst, tail, grid, stream);
    else if (!rms && gated) launch_mixed_kind<NV, 4, false, true>(a, P, remfirst, false, grid, stream);
    else if (rms && !gated) launch_mixed_kind<NV, 4, true, false>(a, P, remfirst, tail, grid, stream);
    else launch_mixed_kind<NV, 4, true, true>(a, P, remfirst, false, grid, stream);
  }
  return hipGetLastError();
}

// The plain RMS form at 4096 columns with at least four whole rounds (the
// chip's resident capacity of 4096-column rows) runs in 8-wavefront
// workgroups, whose 48 KB of fp32 modulation rows and weight spare the two
// bf16 widenings per element: 4096 rows 13.65 -> 12.61 us, 4216 rows 14.56 ->
// 14.30 us, 4608 rows 16.14 -> 15.49 us (bitwise the same).  Smaller launches
// keep 4-wavefront workgroups (1024 rows: 6.60 against 5.84 us, half of the
// compute units would idle); so do the gated forms, which measured 2-3%
// slower in 8-wavefront workgroups.
template <int NV>
static hipError_t launch_mixed(const RowArgs &a, bool rms, bool gated, const DeviceInfo &dev,
                               hipStream_t stream) {
  if constexpr (NV == 8) {
    if (rms && !gated && a.rows >= 4 * (int64_t)dev.num_cu * 4)
      return launch_mixed_w<NV, 8>(a, rms, gated, dev, stream);
  }
  return launch_mixed_w<NV, 4>(a, rms, gated, dev, stream);
}

template <int NV, bool FULL>
hipError_t launch_wave(const RowArgs &a, bool rms, bool gated, bool fold, hipStream_t stream) {
  const dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
#define DITNORM_WAVE(R, G, F) \
  hipLaunchKernelGGL((row_wave_kernel<NV, FULL, R, G, MOD_LDS, F>), grid, block, 0, stream, a)
  if (fold) DITNORM_WAVE(false, false, true);  // LN only
  else if (!rms && !gated) DITNORM_WAVE(false, false, false);
  else if (!rms && gated) DITNORM_WAVE(false, true, false);
  else if (rms && !gated) DITNORM_WAVE(true, false, false);
  else DITNORM_WAVE(true, true, false);
#undef DITNORM_WAVE
  return hipGetLastError();
}

// The folded form at 1024-4096 columns (multiples of 1024): one wavefront per
// row, modulation rows read per row.  A launch of at most half a round of
// rows (fewer rows than SIMDs) splits every row over the balanced kernel
// instead, in quarters (at most a quarter round, 2048 or 4096 columns) or
// halves, so that it spreads over the SIMDs (512 rows of 3072: 4.75 -> 4.13 us,
// bitwise the same).
template <int NV>
hipError_t launch_folded(const RowArgs &a0, const DeviceInfo &dev, hipStream_t stream) {
  const int64_t simds = (int64_t)dev.num_cu * 4;
  if (2 * a0.rows <= simds) {
    RowArgs a = a0;
    a.full_blocks = 0;
    const dim3 block(256);
    if constexpr (NV % 4 == 0) {
      if (4 * a.rows <= simds) {
        hipLaunchKernelGGL((row_mixed_kernel<NV, false, false, 4, 4, false, true>),
                           dim3((unsigned)a.rows), block, 0, stream, a);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((row_mixed_kernel<NV, false, false, 2, 4, false, true>),
                       dim3((unsigned)((a.rows + 1) / 2)), block, 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a0.rows + 3) / 4)), block(256);
  hipLaunchKernelGGL((row_wave_kernel<NV, true, false, false, MOD_SERIAL, true>), grid, block, 0,
                     stream, a0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------

template <int NT, int NV>
static hipError_t launch_cfg(const RowArgs &a, bool rms, bool gated, bool fold,
                             const DeviceInfo &dev, hipStream_t stream) {
  const void *kfn;
#define DITNORM_PICK(R, G) \
  if (rms == R && gated == G) kfn = (const void *)row_kernel<NT, NV, R, G>;
  kfn = nullptr;
  DITNORM_PICK(false, false)
  DITNORM_PICK(false, true)
  DITNORM_PICK(true, false)
  DITNORM_PICK(true, true)
#undef DITNORM_PICK
  if (fold) kfn = (const void *)row_kernel<NT, NV, false, false, true>;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, NT, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int64_t grid = (int64_t)dev.num_cu * per_cu;
  if (grid > a.rows) grid = a.rows;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(kfn, dim3((unsigned)grid), dim3(NT), args, 0, stream);
}

hipError_t launch_row(const RowArgs &a, bool rms, bool gated, bool fold, const DeviceInfo &dev,
                      hipStream_t stream) {
  const int nvec = a.cols / 8;
  // Rows of 1024-4096 columns (multiples of 1024): the balanced kernel, the
  // modulation rows (and the RMS weight) staged in LDS once per workgroup --
  // except for the folded form, whose lighter chain measured faster reading
  // them per row.  Other widths up to 4096: one wavefront per row.
  if (fold) {
    switch (nvec) {
      case 128: return launch_folded<2>(a, dev, stream);
      case 256: return launch_folded<4>(a, dev, stream);
      case 384: return launch_folded<6>(a, dev, stream);
      case 512: return launch_folded<8>(a, dev, stream);
      default: break;
    }
  }
  switch (nvec) {
    case 128: return launch_mixed<2>(a, rms, gated, dev, stream);
    case 256: return launch_mixed<4>(a, rms, gated, dev, stream);
    case 384: return launch_mixed<6>(a, rms, gated, dev, stream);
    case 512: return launch_mixed<8>(a, rms, gated, dev, stream);
    default: break;
  }
  // (as many 16-byte vectors per lane as the row needs, multiples of 512
  // columns without masks: 1152 x 16384 LN 16.7 -> 16.0 us, RMS 1536 x 10000
  // 13.8 -> 13.1 us, the other widths within 2%; the balanced kernel with
  // whole rows only was no faster at 1536, 2560 and 3584 columns)
  switch (nvec) {
    case 192: return launch_wave<3, true>(a, rms, gated, fold, stream);
    case 320: return launch_wave<5, true>(a, rms, gated, fold, stream);
    case 448: return launch_wave<7, true>(a, rms, gated, fold, stream);
    default: break;
  }
  if (nvec <= 64) return launch_wave<1, false>(a, rms, gated, fold, stream);
  if (nvec <= 128) return launch_wave<2, false>(a, rms, gated, fold, stream);
  if (nvec <= 192) return launch_wave<3, false>(a, rms, gated, fold, stream);
  if (nvec <= 256) return launch_wave<4, false>(a, rms, gated, fold, stream);
  if (nvec <= 320) return launch_wave<5, false>(a, rms, gated, fold, stream);
  if (nvec <= 384) return launch_wave<6, false>(a, rms, gated, fold, stream);
  if (nvec <= 448) return launch_wave<7, false>(a, rms, gated, fold, stream);
  if (nvec <= 512) return launch_wave<8, false>(a, rms, gated, fold, stream);
  // 5120-8192 columns (multiples of 1024): every row in two halves, one
  // wavefront each, the halves' binary64 moments meeting through LDS -- the
  // balanced kernel's half-row path, its modulation rows staged as bf16.
  // Against a workgroup per row (below): LN 5120 x 4096 24.2 -> 17.6 us,
  // 8192 x 2048 18.8 -> 14.4 us, 7168 x 1000 12.8 -> 7.9 us, gated LN 6144 x
  // 2048 24.1 -> 19.4 us, 8192 x 2048 30.2 -> 24.3 us; RMS 5120 x 4096 20.2
  // -> 18.7 us, 6144 x 2048 13.8 -> 12.5 us (gated 23.1 -> 20.3), but at 8192
  // x 2048 15.9 -> 18.0 us (its weight too in LDS: three workgroups per
  // compute unit), so RMS rows over 6144 columns keep the workgroup per row.
  // Quarter rows measured slower than halves (6144 x 2048 LN 13.2 against
  // 11.0 us).
  if (!fold) {
    switch (nvec) {
      case 640: return launch_mixed_w<10, 4>(a, rms, gated, dev, stream, 2);
      case 768: return launch_mixed_w<12, 4>(a, rms, gated, dev, stream, 2);
      case 896:
        if (!rms) return launch_mixed_w<14, 4>(a, rms, gated, dev, stream, 2);
        break;
      case 1024:
        if (!rms) return launch_mixed_w<16, 4>(a, rms, gated, dev, stream, 2);
        break;
      default: break;
    }
  }
  // the other rows over 4096 columns (to 16384) and the folded form there:
  // one workgroup per row, (threads, vectors per thread) such that NT*NV
  // vectors hold the row with 3-4 vectors (24-32 values) per thread
  if (nvec <= 768) return launch_cfg<256, 3>(a, rms, gated, fold, dev, stream);
  if (nvec <= 1024) return launch_cfg<256, 4>(a, rms, gated, fold, dev, stream);
  return launch_cfg<512, 4>(a, rms, gated, fold, dev, stream);  // up to 16384 columns
}

}  // namespace ditnorm
