// Backward of the adaLN LayerNorm + modulate ("[WS1][Qwen-Image][CUDA] Final
// AdaLN output (final_adaln_out)", What: forward and backward of
// out = LN(x) * (1 + scale) + shift, LN in fp32 on widened inputs, the
// modulation-parameter gradients as token sums over fixed fp32 balanced
// trees that depend only on the token count).
//
// Three kernels, all on the caller's stream:
//
//  bwd_row_kernel     one wavefront per row (as the forward): one pass of
//                     binary64 sums over the raw row (sum x, sum x^2, sum g,
//                     sum g x with g = d_out * (1 + scale)) gives the fp32
//                     statistics and both row means the gradient needs, so
//                       d_x = rstd * (g - mean(g) - x_hat * mean(g * x_hat))
//                     becomes A g + B x + C with per-row binary64 constants,
//                     rounded once to bf16 (round to odd into binary32, then
//                     nearest-even into bf16: a single correct rounding); the
//                     row's mean and rstd go to the workspace for the next
//                     kernel.
//  bwd_token_kernel   the first level of the token trees: a wavefront owns 32
//                     consecutive tokens of one batch and 256 columns; each
//                     lane walks the 32 rows of its 4 columns, 8 rows at a
//                     time, and folds the fp32 terms d_out and d_out * x_hat
//                     (x_hat in fp32: rstd * (x - mean)) by adjacent pairs --
//                     the balanced tree of the 32 values, 8 at a time; rows
//                     past the batch contribute +0 (the tree's padding).
//  bwd_tree_kernel    every further level: groups of 32 partial sums folded
//                     the same way, until one value per batch and column.
//
// The result depends only on the batch's token count: no atomics, no order
// chosen at run time, bitwise equal for any batch size or batch position.
#include "device_common.hpp"
#include "launch.hpp"

namespace ditnorm {

// ---------------------------------------------------------------------------
// binary64 -> bf16 with one rounding: round to odd into binary32 (24 >= 2*8+2
// bits, so the second rounding is innocuous), then nearest-even into bf16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float f64_round_odd_f32(double d) {
  float f = (float)d;  // nearest-even
  const double back = (double)f;
  if (back != d) {
    uint32_t u = __float_as_uint(f);
    // step toward zero if nearest-even went away from it, then mark inexact
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1;
    u |= 1u;
    f = __uint_as_float(u);
  }
  return f;
}

// ---------------------------------------------------------------------------
// kernel A: statistics and d_x, one wavefront per row
// ---------------------------------------------------------------------------
template <int NV, bool FULL>
__global__ __launch_bounds__(256) void bwd_row_kernel(const BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= a.rows) return;  // whole wavefront; the kernel has no barrier
  const int cols = a.cols;
  const int nvec = cols >> 3;
  const int64_t base = row * (int64_t)cols;
  const int64_t mo = (row / a.rows_per_batch) * a.mod_stride;
  const uint4 zero = {0, 0, 0, 0};
  auto ok = [&](int k) { return FULL || lane + 64 * k < nvec; };
  auto col = [&](int k) { return (lane + 64 * k) * 8; };

  uint4 xv[NV], dv[NV], sv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) xv[k] = ok(k) ? ld16s(a.x + base + col(k)) : zero;
#pragma unroll
  for (int k = 0; k < NV; ++k) dv[k] = ok(k) ? ld16s(a.d_out + base + col(k)) : zero;
#pragma unroll
  for (int k = 0; k < NV; ++k) sv[k] = ok(k) ? ld16(a.scale + mo + col(k)) : zero;

  // one pass of binary64 sums over the raw inputs (padding contributes
  // zeros): S1 = sum x, S2 = sum x^2 (the statistics), G = sum g and
  // GX = sum g x with g = d_out * (1 + scale)
  Moments m = {0.0, 0.0};
  double sg = 0.0, sgx = 0.0;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float v[8], d[8], sc[8];
    unpack8(xv[k], v);
    unpack8(dv[k], d);
    unpack8(sv[k], sc);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double xd = (double)v[e];
      m.s1 += xd;
      m.s2 = __builtin_fma(xd, xd, m.s2);
      const double g = (double)d[e] * (double)(1.0f + sc[e]);
      sg += g;
      sgx = __builtin_fma(g, xd, sgx);
    }
  }
  const double n_d = (double)cols;
  const double s1 = sum64(m.s1), s2 = sum64(m.s2);
  const double mean_d = s1 / n_d;
  const double var_d = __builtin_fmax(__builtin_fma(-s1, mean_d, s2) / n_d, 0.0);
  const float mean_f = (float)mean_d;
  const float rstd_f = rstd_from(var_d + (double)a.eps);
  const double mu = (double)mean_f, rs = (double)rstd_f;
  // with x_hat = (x - mu) rs:  c1 = mean(g),  c2 = mean(g x_hat) = rs (GX - mu G) / N,
  // and d_x = rs (g - c1 - x_hat c2) = A g + B x + C for per-row constants
  const double G = sum64(sg), GX = sum64(sgx);
  const double c1 = G / n_d;
  const double c2 = rs * __builtin_fma(-mu, G, GX) / n_d;
  const double A = rs;
  const double B = -rs * rs * c2;
  const double C = __builtin_fma(rs * rs * c2, mu, -rs * c1);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    launder(xv[k]);
    launder(dv[k]);
    launder(sv[k]);
  }

  // d_x, one rounding to bf16
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (!ok(k)) continue;
    float v[8], d[8], sc[8], o[8];
    unpack8(xv[k], v);
    unpack8(dv[k], d);
    unpack8(sv[k], sc);
    // Nearest-even into binary32 and then into bf16 rounds once, correctly,
    // unless the binary32 value is inexact and lands exactly on a bf16
    // halfway point (low 16 bits 0x8000): only then, and only for the
    // wavefront that meets one, the rounding goes through round-to-odd.
    double t[8];
    bool tie = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double g = (double)d[e] * (double)(1.0f + sc[e]);
      t[e] = __builtin_fma(B, (double)v[e], __builtin_fma(A, g, C));
      o[e] = (float)t[e];
      tie |= (__float_as_uint(o[e]) & 0xFFFFu) == 0x8000u;
    }
    if (__builtin_amdgcn_ballot_w64(tie) != 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f64_round_odd_f32(t[e]);
    }
    st16s(a.d_x + base + col(k), pack8(o));
  }
  if (lane == 0) {
    a.ws_mean[row] = mean_f;
    a.ws_rstd[row] = rstd_f;
    if (a.mean_out) a.mean_out[row] = mean_f;
    if (a.rstd_out) a.rstd_out[row] = rstd_f;
  }
}

// ---------------------------------------------------------------------------
// The balanced fold of 32 values, in 4 chunks of 8: a chunk's 8 values are
// folded by adjacent pairs (3 levels, in registers), and the chunk sums
// o0..o3 combine as (o0 + o1) + (o2 + o3) -- together the adjacent-pairs tree
// of the 32 values.  W floats per lane.
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ void fold8(float (&t)[8][W], float (&o)[W]) {
#pragma unroll
  for (int e = 0; e < W; ++e) {
    const float p0 = t[0][e] + t[1][e], p1 = t[2][e] + t[3][e];
    const float p2 = t[4][e] + t[5][e], p3 = t[6][e] + t[7][e];
    o[e] = (p0 + p1) + (p2 + p3);
  }
}

// chunk c's sum o enters the fold: chunk 0 and 2 wait as left operands,
// chunk 1 forms (o0 + o1), chunk 3 forms (o2 + o3) and the group sum.
template <int W>
__device__ __forceinline__ void fold_chunk(int c, float (&o)[W], float (&left)[W],
                                           float (&half)[W], float (&out)[W]) {
#pragma unroll
  for (int e = 0; e < W; ++e) {
    if ((c & 1) == 0) {
      left[e] = o[e];
    } else {
      const float pair = left[e] + o[e];
      if (c == 1) half[e] = pair;
      else out[e] = half[e] + pair;
    }
  }
}

// ---------------------------------------------------------------------------
// kernel B: first tree level over tokens.  grid.x: batch * groups-per-batch,
// grid.y: column blocks of 256 columns (one wavefront, 4 columns = 8 bytes per
// lane, so each row access is 512 contiguous bytes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint2 ld8s(const uint16_t *p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  return make_uint2(v.x, v.y);
}

__global__ __launch_bounds__(64) void bwd_token_kernel(const BwdArgs a, int64_t groups,
                                                       float *out_shift, float *out_scale) {
  const int nq = a.cols >> 2;
  const int q = blockIdx.y * 64 + threadIdx.x;  // column quad
  const int64_t bg = blockIdx.x;
  const int64_t b = bg / groups, g = bg - b * groups;
  const int64_t first = g * 32;                           // token index within the batch
  const int64_t left_tokens = a.rows_per_batch - first;
  const int n = (int)(left_tokens < 32 ? left_tokens : 32);  // tokens in this group
  const int64_t r0 = b * a.rows_per_batch + first;
  const bool live = q < nq;
  const int qc = live ? q : nq - 1;  // clamped: every load is valid

  float ls[4], hs[4], os[4], lc[4], hc[4], oc[4];
#pragma unroll 1
  for (int c = 0; c < 4; ++c) {
    if (c * 8 >= n) {  // a chunk wholly past the group folds to +0
      float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      fold_chunk(c, z, ls, hs, os);
      fold_chunk(c, z, lc, hc, oc);
      continue;
    }
    // this chunk's 8 rows: loads with clamped rows, then +0 for rows past
    // the group (the tree's padding)
    uint2 xq[8], dq[8];
    float mu[8], rs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = c * 8 + i;
      const int64_t r = r0 + (s < n ? s : n - 1);
      xq[i] = ld8s(a.x + r * a.cols + qc * 4);
      dq[i] = ld8s(a.d_out + r * a.cols + qc * 4);
      mu[i] = a.ws_mean[r];
      rs[i] = a.ws_rstd[r];
    }
    float ts[8][4], tc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = c * 8 + i < n;
      const float v[4] = {bf_lo(xq[i].x), bf_hi(xq[i].x), bf_lo(xq[i].y), bf_hi(xq[i].y)};
      const float d[4] = {bf_lo(dq[i].x), bf_hi(dq[i].x), bf_lo(dq[i].y), bf_hi(dq[i].y)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = d[e] * (rs[i] * (v[e] - mu[i]));
        ts[i][e] = in ? d[e] : 0.0f;
        tc[i][e] = in ? t : 0.0f;
      }
    }
    float o[4];
    fold8(ts, o);
    fold_chunk(c, o, ls, hs, os);
    fold8(tc, o);
    fold_chunk(c, o, lc, hc, oc);
  }
  if (!live) return;
  const int64_t o = bg * a.cols + q * 4;
  *reinterpret_cast<float4 *>(out_shift + o) = make_float4(os[0], os[1], os[2], os[3]);
  *reinterpret_cast<float4 *>(out_scale + o) = make_float4(oc[0], oc[1], oc[2], oc[3]);
}

// ---------------------------------------------------------------------------
// kernel C: one further tree level.  in: [B * n_in, cols] (both sums), out:
// [B * n_out, cols], n_out = ceil(n_in / 32).  A lane folds one column (the
// data is small and latency-bound: more lanes, more loads in flight);
// grid.x: batch * n_out, grid.y: column blocks of 64.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void bwd_tree_kernel(const float *in_shift, const float *in_scale,
                                                      float *out_shift, float *out_scale,
                                                      int64_t n_in, int64_t n_out, int32_t cols) {
  const int cidx = blockIdx.y * 64 + threadIdx.x;  // column
  const int64_t bo = blockIdx.x;
  const int64_t b = bo / n_out, go = bo - b * n_out;
  const int64_t first = go * 32;
  const int64_t left_vals = n_in - first;
  const int n = (int)(left_vals < 32 ? left_vals : 32);
  const bool live = cidx < cols;
  const int cc = live ? cidx : cols - 1;  // clamped: every load is valid

  float ls[1], hs[1], os[1], lc[1], hc[1], oc[1];
#pragma unroll 1
  for (int c = 0; c < 4; ++c) {
    if (c * 8 >= n) {  // a chunk wholly past the last value folds to +0
      float z[1] = {0.0f};
      fold_chunk(c, z, ls, hs, os);
      fold_chunk(c, z, lc, hc, oc);
      continue;
    }
    float ts[8][1], tc[8][1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = c * 8 + i;
      const int64_t off = (b * n_in + first + (s < n ? s : n - 1)) * cols + cc;
      const float vs = in_shift[off], vc = in_scale[off];
      const bool in = s < n;  // +0 padding past the last value
      ts[i][0] = in ? vs : 0.0f;
      tc[i][0] = in ? vc : 0.0f;
    }
    float o[1];
    fold8(ts, o);
    fold_chunk(c, o, ls, hs, os);
    fold8(tc, o);
    fold_chunk(c, o, lc, hc, oc);
  }
  if (!live) return;
  out_shift[bo * cols + cidx] = os[0];
  out_scale[bo * cols + cidx] = oc[0];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

BwdLayout bwd_layout(int64_t rows, int64_t cols, int64_t rows_per_batch) {
  BwdLayout L{};
  const int64_t nb = rows / rows_per_batch;
  const int64_t g = (rows_per_batch + 31) / 32;
  const int64_t g1 = (g + 31) / 32;
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  L.groups = g;
  L.mean_off = 0;
  L.rstd_off = up(rows * 4);
  L.part0_off = L.rstd_off + up(rows * 4);
  L.part0_floats = nb * g * cols;                        // per sum
  L.part1_off = L.part0_off + up(2 * L.part0_floats * 4);
  L.part1_floats = g > 1 ? nb * g1 * cols : 0;
  L.bytes = L.part1_off + up(2 * L.part1_floats * 4);
  return L;
}

template <int NV, bool FULL>
static void launch_bwd_row(const BwdArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_row_kernel<NV, FULL>), dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0,
                     stream, a);
}

hipError_t launch_backward(const BwdArgs &a, float *part0, float *part1, int64_t groups,
                           hipStream_t stream) {
  const int nvec = a.cols >> 3;
  switch (nvec) {
    case 128: launch_bwd_row<2, true>(a, stream); break;
    case 256: launch_bwd_row<4, true>(a, stream); break;
    case 384: launch_bwd_row<6, true>(a, stream); break;
    case 512: launch_bwd_row<8, true>(a, stream); break;
    default:
      if (nvec <= 64) launch_bwd_row<1, false>(a, stream);
      else if (nvec <= 128) launch_bwd_row<2, false>(a, stream);
      else if (nvec <= 256) launch_bwd_row<4, false>(a, stream);
      else if (nvec <= 384) launch_bwd_row<6, false>(a, stream);
      else launch_bwd_row<8, false>(a, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int64_t nb = a.rows / a.rows_per_batch;
  const int64_t pf = nb * groups * a.cols;  // floats per sum in part0
  float *s_out = groups == 1 ? a.d_shift : part0;
  float *c_out = groups == 1 ? a.d_scale : part0 + pf;
  const int quads = a.cols / 4;
  hipLaunchKernelGGL(bwd_token_kernel, dim3((unsigned)(nb * groups), (unsigned)((quads + 63) / 64)),
                     dim3(64), 0, stream, a, groups, s_out, c_out);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // further levels, ping-ponging between the two partial regions
  int64_t n = groups;
  float *src = part0, *dst = part1;
  int64_t src_f = pf;
  while (n > 1) {
    const int64_t n_out = (n + 31) / 32;
    const int64_t dst_f = nb * n_out * a.cols;
    float *os = n_out == 1 ? a.d_shift : dst;
    float *oc = n_out == 1 ? a.d_scale : dst + dst_f;
    hipLaunchKernelGGL(bwd_tree_kernel, dim3((unsigned)(nb * n_out), (unsigned)((a.cols + 63) / 64)),
                       dim3(64), 0, stream, src, src + src_f, os, oc, n, n_out, a.cols);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    n = n_out;
    float *t = src;
    src = dst;
    dst = t;
    src_f = dst_f;
  }
  return hipSuccess;
}

}  // namespace ditnorm
