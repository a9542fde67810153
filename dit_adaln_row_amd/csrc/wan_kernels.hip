// channels_last kernels of the Wan VAE decoder ("[Diffusion] Fuse the Wan VAE
// conv bias epilogue and tile the RMSNorm+SiLU kernel").
//
// rmsnorm_silu_bias (Modifications, Quality-gated): per pixel, over its C
// contiguous channels,
//     xb   = bf16(x + bf16(bias))          the deferred conv bias, like add_
//     rstd = fp32(1/sqrt(sum(xb^2)/C + eps))
//     out  = bf16(SiLU((xb * rstd) * gamma))
// conv_bias_epilogue (Modifications, New kernel): out = bf16(x + bf16(bias)),
// optionally followed by the residual add bf16(out + h).
//
// Work layout for rmsnorm_silu_bias: a pixel row of C channels is split over
// L lanes of a wavefront, each lane holding VPL 16-byte vectors (vectors
// l, l+L, ...), so one wavefront instruction covers 64/L pixels and the load
// of a group of pixels is one contiguous stretch of memory.  C = 96 uses
// L = 4 (16 pixels per instruction), C = 384 uses L = 16 (4 pixels); other
// widths use a whole wavefront per pixel.  The channel-indexed bias (already
// rounded to bf16) and gamma stay in VGPRs for the whole kernel, the sum of
// squares is a DPP butterfly over the L lanes in binary64, and each
// wavefront prefetches its next pixel group while it computes the current one.
//
// SiLU(t) = t * sigmoid(t) with sigmoid from e = exp(-|t|) (never overflows):
// sigmoid = 1/(1+e) for t >= 0 and e/(1+e) for t < 0, using the hardware
// exp2 and reciprocal.  Its relative error (a few 1e-7) is far below half a
// bf16 ulp (2^-9), so the rounded result is within one bf16 ulp of the
// correctly rounded SiLU.
#include "device_common.hpp"
#include "launch.hpp"

namespace ditnorm {

constexpr int WAN_BLOCK = 256;

__device__ __forceinline__ float silu_f32(float t) {
  const float e = __builtin_exp2f(-__builtin_fabsf(t) * 1.4426950408889634f);
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  const float s = t >= 0.0f ? r : e * r;
  return t * s;
}

template <int L, int VPL, bool BIAS, bool EXACT>
__global__ __launch_bounds__(WAN_BLOCK) void wan_kernel(const WanArgs a) {
  constexpr int RPW = 64 / L;  // pixels per wavefront instruction
  constexpr int G = (RPW >= 16) ? 1 : 2;  // pixel groups in flight per wavefront
  const int lane = threadIdx.x & 63;
  const int sub = lane / L;
  const int part = lane % L;
  const int C = a.channels;
  const int nvec = C >> 3;

  int vch[VPL];
  bool ok[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    vch[k] = (part + k * L) * 8;
    ok[k] = EXACT || (part + k * L) < nvec;
  }

  // per-lane channel constants
  float bq[BIAS ? VPL : 1][8], gm[VPL][8];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      const float4 zero = {0.f, 0.f, 0.f, 0.f};
      const float4 gv = ok[k] ? ld16f(a.gamma + vch[k] + e) : zero;
      gm[k][e] = gv.x; gm[k][e + 1] = gv.y; gm[k][e + 2] = gv.z; gm[k][e + 3] = gv.w;
      if constexpr (BIAS) {
        const float4 bv = ok[k] ? ld16f(a.bias + vch[k] + e) : zero;
        bq[k][e] = bv.x; bq[k][e + 1] = bv.y; bq[k][e + 2] = bv.z; bq[k][e + 3] = bv.w;
        round2(bq[k][e], bq[k][e + 1]);
        round2(bq[k][e + 2], bq[k][e + 3]);
      }
    }
  }

  const int64_t waves = (int64_t)gridDim.x * (WAN_BLOCK / 64);
  const int64_t wave = (int64_t)blockIdx.x * (WAN_BLOCK / 64) + (threadIdx.x >> 6);
  const int64_t per_iter = (int64_t)RPW * G;
  const int64_t step = waves * per_iter;
  int64_t base = wave * per_iter;
  if (base >= a.rows) return;

  uint4 nx[G][VPL];
  auto load = [&](int64_t b0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t r = b0 + g * RPW + sub;
      const uint16_t *p = a.x + r * (int64_t)C;
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        const uint4 zero = {0, 0, 0, 0};
        nx[g][k] = (r < a.rows && ok[k]) ? ld16(p + vch[k]) : zero;
      }
    }
  };
  load(base);

  const double n_d = (double)C;
  const double eps = (double)a.eps;
  for (; base < a.rows; base += step) {
    uint4 cx[G][VPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int k = 0; k < VPL; ++k) cx[g][k] = nx[g][k];
    if (base + step < a.rows) load(base + step);

#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t r = base + g * RPW + sub;
      const bool live = r < a.rows;
      float v[VPL][8];
      double s2 = 0.0;
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        unpack8(cx[g][k], v[k]);
        if constexpr (BIAS) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float b0 = v[k][e] + bq[k][e], b1 = v[k][e + 1] + bq[k][e + 1];
            round2(b0, b1);
            v[k][e] = b0;
            v[k][e + 1] = b1;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double d = (double)v[k][e];
          s2 = ok[k] ? __builtin_fma(d, d, s2) : s2;
        }
      }
      s2 = group_sum<L>(s2);
      const float rstd_f = rstd_from(s2 / n_d + eps);
      const int64_t off = r * (int64_t)C;
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float t = v[k][e] * rstd_f;
          t = t * gm[k][e];
          o[e] = silu_f32(t);
        }
        if (live && ok[k]) {
          st16(a.out + off + vch[k], pack8(o));
          if (a.xb_out) st16(a.xb_out + off + vch[k], pack8(v[k]));
        }
      }
      if (live && part == 0 && a.rstd_out) a.rstd_out[r] = rstd_f;
    }
  }
}

template <int L, int VPL, bool EXACT>
static hipError_t launch_wan_cfg(const WanArgs &a, const DeviceInfo &dev, hipStream_t stream) {
  constexpr int RPW = 64 / L;
  constexpr int G = (RPW >= 16) ? 1 : 2;
  const int64_t iters = (a.rows + RPW * G - 1) / (RPW * G);
  const int64_t blocks = (iters + WAN_BLOCK / 64 - 1) / (WAN_BLOCK / 64);
  if (a.bias) {
    const int64_t grid = persistent_grid(wan_kernel<L, VPL, true, EXACT>, WAN_BLOCK, blocks, dev);
    hipLaunchKernelGGL((wan_kernel<L, VPL, true, EXACT>), dim3((unsigned)grid), dim3(WAN_BLOCK),
                       0, stream, a);
  } else {
    const int64_t grid = persistent_grid(wan_kernel<L, VPL, false, EXACT>, WAN_BLOCK, blocks, dev);
    hipLaunchKernelGGL((wan_kernel<L, VPL, false, EXACT>), dim3((unsigned)grid), dim3(WAN_BLOCK),
                       0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_wan(const WanArgs &a, const DeviceInfo &dev, hipStream_t stream) {
  switch (a.channels) {
    case 96: return launch_wan_cfg<4, 3, true>(a, dev, stream);
    case 128: return launch_wan_cfg<16, 1, true>(a, dev, stream);
    case 192: return launch_wan_cfg<8, 3, true>(a, dev, stream);
    case 256: return launch_wan_cfg<16, 2, true>(a, dev, stream);
    case 384: return launch_wan_cfg<16, 3, true>(a, dev, stream);
    case 512: return launch_wan_cfg<16, 4, true>(a, dev, stream);
    default: return launch_wan_cfg<64, 8, false>(a, dev, stream);  // any C <= 4096
  }
}

// ---------------------------------------------------------------------------
// conv-bias epilogue: out = bf16(x + bf16(bias)) [then bf16(out + h)]
// ---------------------------------------------------------------------------
//
// Thread t of a grid of T threads (T a multiple of C/8) always handles vector
// column t % (C/8), so its 8 bias values stay in registers; consecutive
// threads still touch consecutive 16-byte vectors of the row-major tensor.

template <bool RES>
__global__ __launch_bounds__(WAN_BLOCK) void epilogue_kernel(const EpilogueArgs a,
                                                             int64_t active_threads) {
  const int64_t t = (int64_t)blockIdx.x * WAN_BLOCK + threadIdx.x;
  if (t >= active_threads) return;
  const int nvec = a.channels >> 3;
  const int col = (int)(t % nvec) * 8;
  float bq[8];
#pragma unroll
  for (int e = 0; e < 8; e += 4) {
    const float4 bv = ld16f(a.bias + col + e);
    bq[e] = bv.x; bq[e + 1] = bv.y; bq[e + 2] = bv.z; bq[e + 3] = bv.w;
    round2(bq[e], bq[e + 1]);
    round2(bq[e + 2], bq[e + 3]);
  }
  const int64_t total = a.rows * (int64_t)nvec;  // vectors
  for (int64_t i = t; i < total; i += active_threads) {
    float v[8];
    unpack8(ld16(a.x + i * 8), v);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float s0 = v[e] + bq[e], s1 = v[e + 1] + bq[e + 1];
      round2(s0, s1);
      v[e] = s0;
      v[e + 1] = s1;
    }
    if constexpr (RES) {
      float h[8];
      unpack8(ld16(a.h + i * 8), h);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] + h[e];
    }
    st16(a.out + i * 8, pack8(v));
  }
}

hipError_t launch_epilogue(const EpilogueArgs &a, const DeviceInfo &dev, hipStream_t stream) {
  const int nvec = a.channels >> 3;
  const int64_t total = a.rows * (int64_t)nvec;
  int per_cu = 0;
  const void *k = a.h ? (const void *)epilogue_kernel<true> : (const void *)epilogue_kernel<false>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, WAN_BLOCK, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int64_t threads = (int64_t)dev.num_cu * per_cu * WAN_BLOCK;
  if (threads > total) threads = total;
  threads = threads / nvec * nvec;  // a multiple of the vectors per row
  if (threads < nvec) threads = nvec;
  const int64_t grid = (threads + WAN_BLOCK - 1) / WAN_BLOCK;
  if (a.h)
    hipLaunchKernelGGL(epilogue_kernel<true>, dim3((unsigned)grid), dim3(WAN_BLOCK), 0, stream,
                       a, threads);
  else
    hipLaunchKernelGGL(epilogue_kernel<false>, dim3((unsigned)grid), dim3(WAN_BLOCK), 0, stream,
                       a, threads);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// plain 16-byte copy (measurement utility)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(WAN_BLOCK) void copy_kernel(const uint4 *src, uint4 *dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * WAN_BLOCK;
  for (int64_t i = (int64_t)blockIdx.x * WAN_BLOCK + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

hipError_t launch_copy(const void *src, void *dst, int64_t bytes, const DeviceInfo &dev,
                       hipStream_t stream) {
  const int64_t n = bytes / 16;
  const int64_t blocks = (n + WAN_BLOCK - 1) / WAN_BLOCK;
  const int64_t grid = persistent_grid(copy_kernel, WAN_BLOCK, blocks, dev);
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(WAN_BLOCK), 0, stream,
                     (const uint4 *)src, (uint4 *)dst, n);
  return hipGetLastError();
}

}  // namespace ditnorm
