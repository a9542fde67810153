// Per-head LayerNorm (no affine) over the head rows of q and of k in one
// launch (GLM-Image page, Motivation: the q and k tensors of shape
// (1, S, 32, 128) normalised head by head over their 128 values; "What
// rounding-faithful means here": q and k handled by one launch; its kernel
// takes head dims up to 128).  Per row of d = head_dim
// values: mean = fp32(S1/d), rstd = fp32(1/sqrt(M2/d + eps)),
// out = bf16(rstd * (x - mean)).
//
// The eager kernel spends a 128-thread block on each 128-element row (one
// warp busy, three idle).  Here a 128-element row (256 bytes) is spread over
// L lanes holding 16/L 16-byte vectors each (lane p of a row: vectors p,
// p+L, ...), so one wavefront instruction covers 64/L rows and the per-row
// finalisation (one binary64 square root and division) is shared by them.
// L = 8 is used: every load instruction then reads whole 128-byte lines (with
// L = 4 each instruction reads half lines, and the streaming hint lets the
// other half be evicted before its turn), the row reduction is three DPP
// steps.  Statistics are one pass of binary64 moments.  The grid is one-shot:
// each wavefront owns G groups of 64/L consecutive rows and issues all their
// loads before it reduces them.  Rows are numbered q first, then k; a group
// may straddle the q/k boundary.
//
// Other head dims (multiples of 8 up to 128) take the same layout with the
// head dim read at run time: 4 lanes per row up to 32 values, else 8, and as
// many vectors per lane as the row needs, the vectors past the row's end
// masked.
#include "device_common.hpp"
#include "launch.hpp"

namespace ditnorm {

constexpr int QK_HEAD = 128;
constexpr int QK_BLOCK = 256;

// HEAD: the head dim, or 0 for a.head_dim (then VPL vectors per lane, masked)
//
// The first waves_q wavefronts take q's rows, the rest k's, so no
// wavefront's rows straddle the two tensors: each wavefront reads and
// writes through buffer resources at its first row (wavefront-uniform),
// with 32-bit per-lane offsets -- no 64-bit address arithmetic per lane --
// and its stores write through the L2 (about 1% faster).
template <int L, int G, bool NTL, int HEAD = QK_HEAD, int VPL = HEAD / 8 / L>
__global__ __launch_bounds__(QK_BLOCK) void qk_kernel(const QkArgs a, int64_t waves_q) {
  constexpr int RPW = 64 / L;   // rows per wavefront instruction
  const int head = HEAD > 0 ? HEAD : a.head_dim;
  const int nvec = head >> 3;   // 16-byte vectors per row
  const int lane = threadIdx.x & 63;
  const int sub = lane / L;     // row within a group of RPW
  const int part = lane % L;    // lane within the row
  const int64_t wave = (int64_t)blockIdx.x * (QK_BLOCK / 64) + wave_id();
  const bool on_k = wave >= waves_q;
  const int64_t nrows = on_k ? a.rows_k : a.rows_q;
  const int64_t base = (on_k ? wave - waves_q : wave) * RPW * G;  // first row, within q or k
  if (base >= nrows) return;
  const int64_t gbase = on_k ? a.rows_q + base : base;  // ... counted over q then k
  const uint16_t *src = (on_k ? a.k : a.q) + base * head;
  uint16_t *dst = (on_k ? a.k_out : a.q_out) + base * head;
  const __amdgpu_buffer_rsrc_t in_r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(src), (short)0, -1, 0x00020000);
  const auto out_r = wt_rsrc(dst);
  const int last = (int)((nrows - base < RPW * G ? nrows - base : RPW * G) - 1);
  auto ok = [&](int k) { return HEAD > 0 || part + L * k < nvec; };
  constexpr int kNt = 2;  // cache policy: the streaming hint

  // Every load unconditional, at a valid address: a load under a branch was
  // waited for inside it, so a lane's loads went out one latency apart.  A
  // row past the end reads the last row (its statistics are its own, and it
  // is not stored); a vector past a head row's end (run-time head dims) reads
  // the row's first vector and is zeroed.
  uint4 xv[G][VPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int lr = RPW * g + sub;  // row within the wavefront's rows
    const uint32_t rb = (uint32_t)((lr < last ? lr : last) * head * 2);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const uint4 zero = {0, 0, 0, 0};
      const uint32_t vo = rb + (uint32_t)((ok(k) ? part + L * k : 0) * 16);
      uint4 v;
      if constexpr (NTL) {
        const u32x4 q = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      in_r, (int)vo, 0, kNt));
        v.x = q.x; v.y = q.y; v.z = q.z; v.w = q.w;
      } else {
        v = ld16(src + vo / 2);
      }
      xv[g][k] = ok(k) ? v : zero;
    }
  }

  const double eps = (double)a.eps;
  float mean_f[G], rstd_f[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Moments m = {0.0, 0.0};
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      float v[8];
      unpack8(xv[g][k], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) accumulate(m, v[e]);
    }
    const double s1 = group_sum<L>(m.s1), s2 = group_sum<L>(m.s2);
    double mean_d, var_d;
    if constexpr (HEAD == QK_HEAD) {  // exact: 128 is a power of two
      mean_d = s1 * (1.0 / QK_HEAD);
      var_d = clamp_var(__builtin_fma(-s1, mean_d, s2) * (1.0 / QK_HEAD));
    } else {
      const double n_d = (double)head;
      mean_d = s1 / n_d;
      var_d = clamp_var(__builtin_fma(-s1, mean_d, s2) / n_d);
    }
    mean_f[g] = (float)mean_d;
    rstd_f[g] = rstd_from(var_d + eps);
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int k = 0; k < VPL; ++k) launder(xv[g][k]);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int lr = RPW * g + sub;
    if (lr > last) continue;
    const uint32_t rb = (uint32_t)(lr * head * 2);  // the row's byte offset
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      if (!ok(k)) continue;
      float v[8], y[8];
      unpack8(xv[g][k], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = rstd_f[g] * (v[e] - mean_f[g]);
      st16w(out_r, rb + (uint32_t)((part + L * k) * 16), pack8(y));
    }
    if (part == 0) {
      if (a.mean_out) a.mean_out[gbase + lr] = mean_f[g];
      if (a.rstd_out) a.rstd_out[gbase + lr] = rstd_f[g];
    }
  }
}

template <int L, int G, bool NTL, int HEAD = QK_HEAD, int VPL = HEAD / 8 / L>
hipError_t launch_qk_cfg(const QkArgs &a, hipStream_t stream) {
  const int64_t rows_per_wave = (64 / L) * G;
  const int64_t waves_q = (a.rows_q + rows_per_wave - 1) / rows_per_wave;
  const int64_t waves = waves_q + (a.rows_k + rows_per_wave - 1) / rows_per_wave;
  const int64_t grid = (waves + QK_BLOCK / 64 - 1) / (QK_BLOCK / 64);
  hipLaunchKernelGGL((qk_kernel<L, G, NTL, HEAD, VPL>), dim3((unsigned)grid), dim3(QK_BLOCK), 0,
                     stream, a, waves_q);
  return hipGetLastError();
}

hipError_t launch_qk(const QkArgs &a, const DeviceInfo &dev, hipStream_t stream) {
  (void)dev;
  // 8 lanes per row: each load instruction reads whole 128-byte lines
  if (a.head_dim == QK_HEAD) return launch_qk_cfg<8, 1, true>(a, stream);
  const int nvec = a.head_dim >> 3;
  if (nvec <= 4) return launch_qk_cfg<4, 1, true, 0, 1>(a, stream);
  if (nvec <= 8) return launch_qk_cfg<8, 1, true, 0, 1>(a, stream);
  return launch_qk_cfg<8, 1, true, 0, 2>(a, stream);
}

}  // namespace ditnorm
