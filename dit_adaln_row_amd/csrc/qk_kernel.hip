// Per-head LayerNorm (no affine) over the 128-wide head rows of q and of k in
// one launch (GLM-Image page, Motivation: nn.LayerNorm(128) per head on
// (1, S, 32, 128); "What rounding-faithful means here": q and k handled by one
// launch).  Per row: mean = fp32(S1/128), rstd = fp32(1/sqrt(M2/128 + eps)),
// out = bf16(rstd * (x - mean)).
//
// The eager kernel spends a 128-thread block on each 128-element row (one
// warp busy, three idle).  Here a 128-element row is 256 bytes = 16 lanes x
// one 16-byte vector, so one wavefront instruction covers 4 rows and every
// lane does useful work.  The reduction over a row is a 16-lane DPP
// butterfly in binary64 (no LDS, no barrier).  Each wavefront keeps G row
// groups (4G rows) in flight and issues the loads of its next 4G rows before
// it reduces the current ones.  Rows are numbered q first, then k; a row
// group may straddle the q/k boundary.
#include "device_common.hpp"
#include "launch.hpp"

namespace ditnorm {

constexpr int QK_HEAD = 128;
constexpr int QK_BLOCK = 256;

template <int G>
__global__ __launch_bounds__(QK_BLOCK) void qk_kernel(const QkArgs a) {
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4;            // row within a group of 4
  const int col = (lane & 15) * 8;      // first element of this lane's vector
  const int64_t total = a.rows_q + a.rows_k;
  const int64_t waves = (int64_t)gridDim.x * (QK_BLOCK / 64);
  const int64_t wave = (int64_t)blockIdx.x * (QK_BLOCK / 64) + (threadIdx.x >> 6);
  const int64_t step = waves * 4 * G;

  auto src = [&](int64_t r) -> const uint16_t * {
    return r < a.rows_q ? a.q + r * QK_HEAD : a.k + (r - a.rows_q) * QK_HEAD;
  };
  auto dst = [&](int64_t r) -> uint16_t * {
    return r < a.rows_q ? a.q_out + r * QK_HEAD : a.k_out + (r - a.rows_q) * QK_HEAD;
  };

  int64_t base = wave * 4 * G;
  if (base >= total) return;

  uint4 nx[G];
  auto load = [&](int64_t b0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t r = b0 + 4 * g + sub;
      const uint4 zero = {0, 0, 0, 0};
      nx[g] = r < total ? ld16(src(r) + col) : zero;
    }
  };
  load(base);

  const double eps = (double)a.eps;
  for (; base < total; base += step) {
    uint4 cx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) cx[g] = nx[g];
    if (base + step < total) load(base + step);

#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t r = base + 4 * g + sub;
      float v[8];
      unpack8(cx[g], v);
      double s = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (double)v[e];
      s = sum16(s);
      const double mean_d = s * (1.0 / QK_HEAD);  // exact: 128 is a power of two
      double m2 = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double d = (double)v[e] - mean_d;
        m2 = __builtin_fma(d, d, m2);
      }
      m2 = sum16(m2);
      const float mean_f = (float)mean_d;
      const float rstd_f = rstd_from(m2 * (1.0 / QK_HEAD) + eps);
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = rstd_f * (v[e] - mean_f);
      if (r < total) {
        st16(dst(r) + col, pack8(y));
        if ((lane & 15) == 0) {
          if (a.mean_out) a.mean_out[r] = mean_f;
          if (a.rstd_out) a.rstd_out[r] = rstd_f;
        }
      }
    }
  }
}

hipError_t launch_qk(const QkArgs &a, const DeviceInfo &dev, hipStream_t stream) {
  constexpr int G = 4;
  const int64_t total = a.rows_q + a.rows_k;
  const int64_t groups = (total + 4 * G - 1) / (4 * G);          // wave-iterations
  const int64_t blocks = (groups + QK_BLOCK / 64 - 1) / (QK_BLOCK / 64);
  const int64_t grid = persistent_grid(qk_kernel<G>, QK_BLOCK, blocks, dev);
  hipLaunchKernelGGL(qk_kernel<G>, dim3((unsigned)grid), dim3(QK_BLOCK), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ditnorm
