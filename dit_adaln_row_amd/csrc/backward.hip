// Backward of the adaLN LayerNorm + modulate ("[WS1][Qwen-Image][CUDA] Final
// AdaLN output (final_adaln_out)", What: forward and backward of
// out = LN(x) * (1 + scale) + shift, LN in fp32 on widened inputs, the
// modulation-parameter gradients as token sums over fixed fp32 balanced
// trees that depend only on the token count).
//
// The token trees fold groups of 32 consecutive tokens by adjacent pairs, then
// the group sums in groups of 32 again, +0 padding a short group.  Every
// aligned run of 8 (or 4) tokens inside a group is a complete subtree of it,
// and the 32 * (32 / R) runs of R tokens in 32 consecutive groups are the
// leaves of one value of the second level; the kernels follow those subtrees:
//
//  bwd_fused_kernel  a workgroup of R wavefronts owns R consecutive tokens of
//                    one batch (R = 8; 4 for batches of at most 4 tokens, for
//                    rows over 3072 columns and for small launches -- see
//                    bwd_layout), one row per wavefront.  One
//                    pass of binary64 sums over the raw row (sum x, sum x^2,
//                    sum g, sum g x with g = d_out * (1 + scale)) gives the
//                    fp32 statistics and
//                    both row means the gradient needs, so
//                      d_x = rstd * (g - mean(g) - x_hat * mean(g * x_hat))
//                    becomes A g + B x + C with per-row binary64 constants,
//                    rounded once to bf16.  Then the rows' raw x and d_out
//                    pass through LDS, column-major: each thread takes two
//                    columns and folds the fp32 terms d_out and
//                    d_out * x_hat (x_hat = rstd * (x - mean) in fp32) of the
//                    R rows by adjacent pairs -- the subtree of those R
//                    tokens.  x and d_out are read from HBM once.
//  bwd_tree_kernel   one or more levels at once: out = the balanced fold of
//                    L consecutive partial sums (L = 4, 8, 32, 128 or 256), T
//                    wavefronts folding 4, 8 or 16 each, their sums combined
//                    through LDS.
//
// The result depends only on the batch's token count: no atomics, no order
// chosen at run time, bitwise equal for any batch size or batch position.
//
// Storage types (DT): bf16 (0) and the page's fp32 stream (2).  A 16-byte
// vector holds 8 bf16 or 4 fp32 values, so a lane keeps the same 48 values of
// a 3072-column row either way; in fp32 those take twice the registers, so
// 1 + scale is not kept per lane but staged once per workgroup in LDS (the
// workgroup's tokens share one batch), the workgroups hold 4 tokens, and d_x
// is the binary64 value rounded once to fp32.
#include "../../include/ditnorm.h"
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

// Address of element `elem` of a DT array, as the 16-bit pointer the vector
// load and store helpers take.
template <int DT>
__device__ __forceinline__ const uint16_t *at(const void *base, int64_t elem) {
  if constexpr (DT == 2) return (const uint16_t *)((const float *)base + elem);
  else return (const uint16_t *)base + elem;
}

// A 16-byte vector of DT values widened to fp32 (8 bf16 or 4 fp32 values).
template <int DT>
__device__ __forceinline__ void widen_vec(const uint4 v, float f[8]) {
  if constexpr (DT == 2) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  } else {
    unpack8(v, f);
  }
}

// The balanced fold of N values by adjacent pairs (N a power of two).
template <int N>
__device__ __forceinline__ float tree_fold(const float *v) {
  if constexpr (N == 1) {
    return v[0];
  } else {
    return tree_fold<N / 2>(v) + tree_fold<N / 2>(v + N / 2);
  }
}

// ---------------------------------------------------------------------------
// one row: statistics and d_x.  xv / dv keep the raw row for the token sums.
// ---------------------------------------------------------------------------
template <int NV, bool FULL, int DT>
__device__ __forceinline__ void bwd_row(const BwdArgs &a, int64_t row, int64_t mo, int lane,
                                        uint4 (&xv)[NV], uint4 (&dv)[NV], float &mean_f,
                                        float &rstd_f, const float *s1_lds) {
  constexpr int VE = DT == 2 ? 4 : 8;  // values per 16-byte vector
  const int cols = a.cols;
  const int nvec = cols / VE;
  const int64_t base = row * (int64_t)cols;
  const uint4 zero = {0, 0, 0, 0};
  auto ok = [&](int k) { return FULL || lane + 64 * k < nvec; };
  auto col = [&](int k) { return (lane + 64 * k) * VE; };
  // fp32: 1 + scale of the vector's 4 columns from the workgroup's LDS copy
  auto scale1 = [&](const uint4 &, int k, float s1[8]) {
    const float4 q = *reinterpret_cast<const float4 *>(s1_lds + col(k));
    s1[0] = q.x; s1[1] = q.y; s1[2] = q.z; s1[3] = q.w;
  };

  // Every load unconditional (a vector past the row's end reads the row's
  // first vector and is zeroed): a load under a branch was waited for inside
  // it, so a lane's loads went out one latency apart.
  auto lc = [&](int k) { return ok(k) ? col(k) : 0; };
  uint4 sv[DT == 2 ? 1 : NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const uint4 v = ld16s(at<DT>(a.x, base + lc(k)));
    xv[k] = ok(k) ? v : zero;
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const uint4 v = ld16s(at<DT>(a.d_out, base + lc(k)));
    dv[k] = ok(k) ? v : zero;
  }
  if constexpr (DT != 2) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const uint4 v = ld16(at<DT>(a.scale, mo + lc(k)));
      sv[k] = ok(k) ? v : zero;
    }
  }

  // one pass of binary64 sums over the raw inputs (padding contributes
  // zeros): S1 = sum x, S2 = sum x^2 (the statistics), G = sum g and
  // GX = sum g x with g = d_out * (1 + scale)
  Moments m = {0.0, 0.0};
  double sg = 0.0, sgx = 0.0;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float v[8], d[8], sc[8];
    widen_vec<DT>(xv[k], v);
    widen_vec<DT>(dv[k], d);
    if constexpr (DT == 2) {
      if (!ok(k)) continue;  // (the LDS copy ends at cols)
      scale1(sv[0], k, sc);  // 1 + scale
    } else {
      unpack8(sv[k], sc);  // scale
    }
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const double xd = (double)v[e];
      m.s1 += xd;
      m.s2 = __builtin_fma(xd, xd, m.s2);
      const double g = DT == 2 ? (double)d[e] * (double)sc[e]
                               : (double)d[e] * (double)(1.0f + sc[e]);
      sg += g;
      sgx = __builtin_fma(g, xd, sgx);
    }
  }
  const double n_d = (double)cols;
  const double s1 = sum64(m.s1), s2 = sum64(m.s2);
  const double mean_d = s1 / n_d;
  const double var_d = clamp_var(__builtin_fma(-s1, mean_d, s2) / n_d);
  mean_f = (float)mean_d;
  rstd_f = rstd_from(var_d + (double)a.eps);
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
    if constexpr (DT != 2) launder(sv[k]);
  }

  // d_x, one rounding to the storage type, written through the L2 from a
  // buffer resource at the row (about 1% faster than streaming stores)
  const auto dx_r = wt_rsrc(at<DT>(a.d_x, base));
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (!ok(k)) continue;
    float v[8], d[8], sc[8], o[8];
    widen_vec<DT>(xv[k], v);
    widen_vec<DT>(dv[k], d);
    if constexpr (DT == 2) {  // binary64 -> fp32: one correctly rounded conversion
      scale1(sv[0], k, sc);  // 1 + scale
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double g = (double)d[e] * (double)sc[e];
        o[e] = (float)__builtin_fma(B, (double)v[e], __builtin_fma(A, g, C));
      }
      uint4 q;
      q.x = __float_as_uint(o[0]); q.y = __float_as_uint(o[1]);
      q.z = __float_as_uint(o[2]); q.w = __float_as_uint(o[3]);
      st16w(dx_r, col(k) * 4, q);
      continue;
    } else {
      // Nearest-even into binary32 and then into bf16 rounds once, correctly,
      // unless the binary32 value is inexact and lands exactly on a bf16
      // halfway point (low 16 bits 0x8000): only then, and only for the
      // wavefront that meets one, the rounding goes through round-to-odd.
      // (one ballot per element, the wave masks OR-ed in scalar registers)
      unpack8(sv[k], sc);  // scale
      double t[8];
      uint64_t tie = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double g = (double)d[e] * (double)(1.0f + sc[e]);
        t[e] = __builtin_fma(B, (double)v[e], __builtin_fma(A, g, C));
        o[e] = (float)t[e];
        tie |= __builtin_amdgcn_ballot_w64((__float_as_uint(o[e]) & 0xFFFFu) == 0x8000u);
      }
      if (tie != 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = f64_round_odd_f32(t[e]);
      }
      st16w(dx_r, col(k) * 2, pack8(o));
    }
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    launder(xv[k]);
    launder(dv[k]);
  }
}

// ---------------------------------------------------------------------------
// the fused kernel.  grid.x: batch * chunks (chunk = R consecutive tokens of a
// batch); block: R wavefronts.  out_*: [B * chunks, cols] per sum, the chunk
// subtree sums; with a single chunk per batch they are the final sums, and
// the +0 padding of the rest of the 32-token group is added here.
// ---------------------------------------------------------------------------
template <int NV, bool FULL, int R, int DT>
__global__ __launch_bounds__(64 * R) void bwd_fused_kernel(const BwdArgs a, int64_t chunks,
                                                           float *out_shift, float *out_scale,
                                                           int final_level) {
  // a step moves VS 16-byte vectors per lane through LDS (VS * 256 dwords:
  // 512 bf16 or 256 fp32 columns), and every thread folds one dword column
  // of them (2 bf16 columns or 1 fp32 column)
  constexpr int VS = R / 4;
  constexpr int STEPS = (NV + VS - 1) / VS;
  constexpr int CPD = DT == 2 ? 1 : 2;  // columns per dword
  __shared__ float stat[R][2];
  __shared__ __attribute__((aligned(16))) uint32_t tile[2][R][2][VS * 256];  // [buffer][row][x | d_out][dword]
  __shared__ __attribute__((aligned(16))) float s1_lds[DT == 2 ? DITNORM_MAX_BACKWARD_F32_COLS : 1];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int64_t b = blockIdx.x / chunks, j = blockIdx.x - b * chunks;
  const int64_t left = a.rows_per_batch - j * R;
  const int nrow = (int)(left < R ? left : R);  // tokens of this chunk
  const int64_t row = b * a.rows_per_batch + j * R + w;
  const int nvec = a.cols / (DT == 2 ? 4 : 8);

  if constexpr (DT == 2) {  // 1 + scale of the chunk's batch, once per workgroup
    const float *sc = (const float *)a.scale + b * a.mod_stride;
    for (int i = threadIdx.x; i < a.cols; i += 64 * R) s1_lds[i] = 1.0f + sc[i];
    lds_barrier();
  }

  // A wavefront past the chunk's last token stands for the tree's +0
  // padding: it puts a zero row and zero statistics (mean 0, rstd 0) into
  // LDS, whose terms d_out = +0 and d_out * (rstd * (x - mean)) = +0 are
  // exactly the padding, so the token step needs no per-row selects.
  uint4 xv[NV], dv[NV];
  if (w < nrow) {
    float mean_f, rstd_f;
    bwd_row<NV, FULL, DT>(a, row, b * a.mod_stride, lane, xv, dv, mean_f, rstd_f, s1_lds);
    if (lane == 0) {
      stat[w][0] = mean_f;
      stat[w][1] = rstd_f;
      if (a.mean_out) a.mean_out[row] = mean_f;
      if (a.rstd_out) a.rstd_out[row] = rstd_f;
    }
  } else {
#pragma unroll
    for (int k = 0; k < NV; ++k) xv[k] = dv[k] = uint4{0, 0, 0, 0};
    if (lane == 0) stat[w][0] = stat[w][1] = 0.0f;
  }

  // token sums of the chunk
  const int vk = (int)(threadIdx.x >> 8);  // vector of the step this thread folds
  const int pr = (int)(threadIdx.x & 255);  // its dword within that vector
  float mu[R], rs[R];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int buf = s & 1;
#pragma unroll
    for (int v = 0; v < VS; ++v) {
      const int k = s * VS + v;
      if (k < NV && (FULL || lane + 64 * k < nvec)) {
        *reinterpret_cast<uint4 *>(&tile[buf][w][0][v * 256 + lane * 4]) = xv[k];
        *reinterpret_cast<uint4 *>(&tile[buf][w][1][v * 256 + lane * 4]) = dv[k];
      }
    }
    lds_barrier();
    if (s == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        mu[i] = stat[i][0];
        rs[i] = stat[i][1];
      }
    }
    const int k = s * VS + vk;
    const int c = (k * 256 + pr) * CPD;
    if (k < NV && (FULL || c < a.cols)) {
      // Every row's words are read before any is used: a use between the
      // reads would wait out each row's LDS latency in turn.
      uint32_t xwv[R], dwv[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        xwv[i] = tile[buf][i][0][vk * 256 + pr];
        dwv[i] = tile[buf][i][1][vk * 256 + pr];
      }
      asm volatile("" ::: "memory");  // (all the reads issued before any use)
      float s0[R], s1[R], c0[R], c1[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const uint32_t xw = xwv[i], dw = dwv[i];
        if constexpr (DT == 2) {
          const float x0 = __uint_as_float(xw), d0 = __uint_as_float(dw);
          s0[i] = d0;
          c0[i] = d0 * (rs[i] * (x0 - mu[i]));
        } else {
          const float x0 = bf_lo(xw), x1 = bf_hi(xw), d0 = bf_lo(dw), d1 = bf_hi(dw);
          s0[i] = d0;
          s1[i] = d1;
          c0[i] = d0 * (rs[i] * (x0 - mu[i]));
          c1[i] = d1 * (rs[i] * (x1 - mu[i]));
        }
      }
      const int64_t o = (int64_t)blockIdx.x * a.cols + c;
      if constexpr (DT == 2) {
        float hs = tree_fold<R>(s0), hc = tree_fold<R>(c0);
        if (final_level) {  // the rest of the 32-token group is +0
          hs += 0.0f;
          hc += 0.0f;
        }
        out_shift[o] = hs;
        out_scale[o] = hc;
      } else {
        float2 hs = make_float2(tree_fold<R>(s0), tree_fold<R>(s1));
        float2 hc = make_float2(tree_fold<R>(c0), tree_fold<R>(c1));
        if (final_level) {  // the rest of the 32-token group is +0
          hs.x += 0.0f;
          hs.y += 0.0f;
          hc.x += 0.0f;
          hc.y += 0.0f;
        }
        *reinterpret_cast<float2 *>(out_shift + o) = hs;
        *reinterpret_cast<float2 *>(out_scale + o) = hc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// tree levels.  in: [B * n_in, cols] per sum, out: [B * n_out, cols],
// n_out = ceil(n_in / L), L = CH * T.  Wavefront p folds values
// [o L + p CH, o L + (p + 1) CH) of 64 columns (+0 past n_in); wavefront 0
// folds the T chunk sums.  grid.x: batch * n_out, grid.y: column blocks of 64.
// ---------------------------------------------------------------------------
template <int CH, int T>
__global__ __launch_bounds__(64 * T) void bwd_tree_kernel(const float *in_shift,
                                                          const float *in_scale, float *out_shift,
                                                          float *out_scale, int64_t n_in,
                                                          int64_t n_out, int32_t cols) {
  const int lane = threadIdx.x & 63;
  const int p = T == 1 ? 0 : wave_id();
  const int cidx = blockIdx.y * 64 + lane;  // column
  const int64_t bo = blockIdx.x;
  const int64_t b = bo / n_out, go = bo - b * n_out;
  const int64_t first = go * (CH * T) + p * CH;
  const bool live = cidx < cols;
  const int cc = live ? cidx : cols - 1;  // clamped: every load is valid

  float vs[CH], vc[CH];
  if (first < n_in) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t s = first + i;
      const int64_t off = (b * n_in + (s < n_in ? s : n_in - 1)) * cols + cc;
      const float ls = in_shift[off], lc = in_scale[off];
      vs[i] = s < n_in ? ls : 0.0f;  // +0 padding past the last value
      vc[i] = s < n_in ? lc : 0.0f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < CH; ++i) vs[i] = vc[i] = 0.0f;
  }
  float hs = tree_fold<CH>(vs), hc = tree_fold<CH>(vc);
  if constexpr (T > 1) {
    __shared__ float red[T][2][64];
    red[p][0][lane] = hs;
    red[p][1][lane] = hc;
    lds_barrier();
    if (p != 0) return;
    float ts[T], tc[T];
#pragma unroll
    for (int q = 0; q < T; ++q) {
      ts[q] = red[q][0][lane];
      tc[q] = red[q][1][lane];
    }
    hs = tree_fold<T>(ts);
    hc = tree_fold<T>(tc);
  }
  if (!live) return;
  out_shift[bo * cols + cidx] = hs;
  out_scale[bo * cols + cidx] = hc;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Leaves per value of the first tree level after the fused kernel: the rest
// of a 32-token group (32 / R chunk sums), and with more than one group per
// batch, the 32 groups of the next level too.
static int64_t first_fanin(int64_t rows_per_batch, int rows_per_chunk) {
  const int64_t per_group = 32 / rows_per_chunk;
  return rows_per_batch <= 32 ? per_group : 32 * per_group;
}

BwdLayout bwd_layout(int64_t rows, int64_t cols, int64_t rows_per_batch, int dtype) {
  BwdLayout L{};
  const int64_t nb = rows / rows_per_batch;
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  // 8 tokens per workgroup; 4 for batches of at most 4 tokens, for rows over
  // 3072 columns (whose register footprint leaves room for one 8-wavefront
  // workgroup per compute unit but three of 4), and for batches of more than
  // 8 tokens that 8-token workgroups would spread over at most 128 of them
  // (half the 256 compute units): there each workgroup's serial chain of rows
  // sets the time, and 4-row workgroups halve it (measured 2-15% faster up to
  // 128 eight-token workgroups, slower from 138 on, where the doubled run
  // sums cost more).  Batches of 5-8 tokens keep one 8-row workgroup and one
  // launch.
  const int64_t wg8 = nb * ((rows_per_batch + 7) / 8);
  // (fp32: 4 tokens, whose rows already take the registers 8 bf16 rows do)
  L.rows_per_chunk = (dtype == 2 || rows_per_batch <= 4 || cols > 3072 ||
                      (rows_per_batch > 8 && wg8 <= 128))
                         ? 4
                         : 8;
  L.chunks = (rows_per_batch + L.rows_per_chunk - 1) / L.rows_per_chunk;
  int64_t n1 = 1;
  if (L.chunks > 1) {
    const int64_t f = first_fanin(rows_per_batch, L.rows_per_chunk);
    n1 = (L.chunks + f - 1) / f;
  }
  L.part0_off = 0;
  L.part0_floats = L.chunks > 1 ? nb * L.chunks * cols : 0;  // per sum
  L.part1_off = up(2 * L.part0_floats * 4);
  L.part1_floats = n1 > 1 ? nb * n1 * cols : 0;
  L.bytes = L.part1_off + up(2 * L.part1_floats * 4);
  return L;
}

template <int NV, bool FULL, int R, int DT>
static void launch_fused(const BwdArgs &a, int64_t nb, int64_t chunks, float *os, float *oc,
                         hipStream_t stream) {
  hipLaunchKernelGGL((bwd_fused_kernel<NV, FULL, R, DT>), dim3((unsigned)(nb * chunks)),
                     dim3(64 * R), 0, stream, a, chunks, os, oc, chunks == 1 ? 1 : 0);
}

template <int R>
static void launch_fused_r(const BwdArgs &a, int64_t nb, int64_t chunks, float *os, float *oc,
                           hipStream_t stream) {
  switch (a.cols >> 3) {
    case 128: launch_fused<2, true, R, 0>(a, nb, chunks, os, oc, stream); return;
    case 256: launch_fused<4, true, R, 0>(a, nb, chunks, os, oc, stream); return;
    case 384: launch_fused<6, true, R, 0>(a, nb, chunks, os, oc, stream); return;
    case 512: launch_fused<8, true, R, 0>(a, nb, chunks, os, oc, stream); return;
    default: break;
  }
  const int nvec = a.cols >> 3;
  if (nvec <= 64) launch_fused<1, false, R, 0>(a, nb, chunks, os, oc, stream);
  else if (nvec <= 128) launch_fused<2, false, R, 0>(a, nb, chunks, os, oc, stream);
  else if (nvec <= 256) launch_fused<4, false, R, 0>(a, nb, chunks, os, oc, stream);
  else if (nvec <= 384) launch_fused<6, false, R, 0>(a, nb, chunks, os, oc, stream);
  else launch_fused<8, false, R, 0>(a, nb, chunks, os, oc, stream);
}

// fp32 rows (4 values per vector, up to DITNORM_MAX_BACKWARD_F32_COLS columns)
static void launch_fused_f32(const BwdArgs &a, int64_t nb, int64_t chunks, float *os, float *oc,
                             hipStream_t stream) {
  switch (a.cols >> 2) {
    case 256: launch_fused<4, true, 4, 2>(a, nb, chunks, os, oc, stream); return;
    case 512: launch_fused<8, true, 4, 2>(a, nb, chunks, os, oc, stream); return;
    case 768: launch_fused<12, true, 4, 2>(a, nb, chunks, os, oc, stream); return;
    default: break;
  }
  const int nvec = a.cols >> 2;
  if (nvec <= 64) launch_fused<1, false, 4, 2>(a, nb, chunks, os, oc, stream);
  else if (nvec <= 128) launch_fused<2, false, 4, 2>(a, nb, chunks, os, oc, stream);
  else if (nvec <= 256) launch_fused<4, false, 4, 2>(a, nb, chunks, os, oc, stream);
  else if (nvec <= 512) launch_fused<8, false, 4, 2>(a, nb, chunks, os, oc, stream);
  else launch_fused<12, false, 4, 2>(a, nb, chunks, os, oc, stream);
}

hipError_t launch_backward(const BwdArgs &a, const BwdLayout &L, float *part0, float *part1,
                           hipStream_t stream) {
  const int64_t nb = a.rows / a.rows_per_batch;
  const int64_t pf = L.part0_floats;
  float *s_out = L.chunks == 1 ? a.d_shift : part0;
  float *c_out = L.chunks == 1 ? a.d_scale : part0 + pf;
  if (nb * L.chunks * 64 * L.rows_per_chunk > (int64_t)INT32_MAX) return hipErrorInvalidConfiguration;
  if (a.dtype == 2) launch_fused_f32(a, nb, L.chunks, s_out, c_out, stream);
  else if (L.rows_per_chunk == 4) launch_fused_r<4>(a, nb, L.chunks, s_out, c_out, stream);
  else launch_fused_r<8>(a, nb, L.chunks, s_out, c_out, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  int64_t n = L.chunks, f = first_fanin(a.rows_per_batch, L.rows_per_chunk);

  // tree levels, ping-ponging between the two partial regions
  float *src = part0, *dst = part1;
  int64_t src_f = pf;
  const unsigned cblocks = (unsigned)((a.cols + 63) / 64);
  while (n > 1) {
    const int64_t n_out = (n + f - 1) / f;
    const int64_t dst_f = nb * n_out * a.cols;
    float *os = n_out == 1 ? a.d_shift : dst;
    float *oc = n_out == 1 ? a.d_scale : dst + dst_f;
    const dim3 grid((unsigned)(nb * n_out), cblocks);
    const float *is = src, *ic = src + src_f;
    switch (f) {
      case 4:
        hipLaunchKernelGGL((bwd_tree_kernel<4, 1>), grid, dim3(64), 0, stream, is, ic, os, oc, n,
                           n_out, a.cols);
        break;
      case 8:
        hipLaunchKernelGGL((bwd_tree_kernel<8, 1>), grid, dim3(64), 0, stream, is, ic, os, oc, n,
                           n_out, a.cols);
        break;
      case 32:
        hipLaunchKernelGGL((bwd_tree_kernel<8, 4>), grid, dim3(256), 0, stream, is, ic, os, oc, n,
                           n_out, a.cols);
        break;
      case 128:
        hipLaunchKernelGGL((bwd_tree_kernel<8, 16>), grid, dim3(1024), 0, stream, is, ic, os, oc,
                           n, n_out, a.cols);
        break;
      default:  // 256
        hipLaunchKernelGGL((bwd_tree_kernel<16, 16>), grid, dim3(1024), 0, stream, is, ic, os, oc,
                           n, n_out, a.cols);
        break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    n = n_out;
    f = 32;
    float *t = src;
    src = dst;
    dst = t;
    src_f = dst_f;
  }
  return hipSuccess;
}

}  // namespace ditnorm
