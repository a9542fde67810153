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

template <int NT, int NV, bool RMS, bool GATED>
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
        if (a.y_out) st16(a.y_out + off, pack8(y));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------

template <int NT, int NV>
static hipError_t launch_cfg(const RowArgs &a, bool rms, bool gated, const DeviceInfo &dev,
                             hipStream_t stream) {
  const void *kfn;
#define DITNORM_PICK(R, G) \
  if (rms == R && gated == G) kfn = (const void *)row_kernel<NT, NV, R, G>;
  kfn = nullptr;
  DITNORM_PICK(false, false)
  DITNORM_PICK(false, true)
  DITNORM_PICK(true, false)
  DITNORM_PICK(true, true)
#undef DITNORM_PICK
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, NT, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int64_t grid = (int64_t)dev.num_cu * per_cu;
  if (grid > a.rows) grid = a.rows;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(kfn, dim3((unsigned)grid), dim3(NT), args, 0, stream);
}

hipError_t launch_row(const RowArgs &a, bool rms, bool gated, const DeviceInfo &dev,
                      hipStream_t stream) {
  const int nvec = a.cols / 8;
  // (threads, vectors per thread): the row must fit NT*NV vectors; prefer
  // exact fits and 2-4 vectors (16-32 values) per thread.
  if (nvec <= 64) return launch_cfg<64, 1>(a, rms, gated, dev, stream);
  if (nvec <= 128) return launch_cfg<64, 2>(a, rms, gated, dev, stream);
  if (nvec <= 192) return launch_cfg<64, 3>(a, rms, gated, dev, stream);
  if (nvec <= 256) return launch_cfg<128, 2>(a, rms, gated, dev, stream);
  if (nvec <= 384) return launch_cfg<128, 3>(a, rms, gated, dev, stream);
  if (nvec <= 512) return launch_cfg<128, 4>(a, rms, gated, dev, stream);
  if (nvec <= 768) return launch_cfg<256, 3>(a, rms, gated, dev, stream);
  if (nvec <= 1024) return launch_cfg<256, 4>(a, rms, gated, dev, stream);
  return launch_cfg<512, 4>(a, rms, gated, dev, stream);  // up to 16384 columns
}

}  // namespace ditnorm
