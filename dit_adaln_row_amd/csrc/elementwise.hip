// Standalone elementwise adaLN stages, for sites whose norm is not fused.
//
// modulate_scale_shift (FLUX.1 page, Commit 2: the modulate in one kernel,
// each of the eager chain's three results rounded to the storage type where
// the eager kernels round it; bf16 or fp16 storage, one modulation row per
// batch, chunked embedding views):
//     out = rnd(rnd(x * rnd(1 + scale)) + shift)
// residual_gate_add (GLM-Image page, the ff gate reusing residual_gate_add;
// ERNIE-Image page, the residual variant):
//     out = rnd(residual + rnd(gate * update))
// rnd rounds to the storage type (bf16 or fp16) nearest-even; each operation
// is one binary32 operation on exactly widened operands.  For fp16 the
// compiler may fuse a widen / operate / round triple into one fp16
// instruction: a binary32 intermediate has at least 2p+2 significand bits for
// p = 11, so the correctly rounded fp16 result is the same either way.
//
// Work layout: thread t owns the 16-byte column slot t % (cols/8) of U
// consecutive rows, so its modulation vector (already rounded 1 + scale, and
// shift; or the gate) is loaded once and reused; consecutive threads touch
// consecutive 16-byte vectors of a row, and each of the U row accesses is a
// separate fully coalesced instruction.  One-shot grid.
#include "device_common.hpp"
#include "launch.hpp"

namespace ditnorm {

constexpr int EW_BLOCK = 256;
constexpr int EW_ROWS = 2;  // rows per thread (2 measured best on MI355X; 1, 4, 8 within 7%)

// OP 0: modulate (x, scale, shift); OP 1: gate add (update, residual, gate)
template <int OP, int DT, int U>
__global__ __launch_bounds__(EW_BLOCK) void elementwise_kernel(const ElementwiseArgs a) {
  const int nvec = a.cols >> 3;
  const int64_t t = (int64_t)blockIdx.x * EW_BLOCK + threadIdx.x;
  const int64_t rg = t / nvec;
  const int c8 = (int)(t - rg * nvec) * 8;
  const int64_t r0 = rg * U;
  if (r0 >= a.rows) return;
  const int nr = (int)(a.rows - r0 < U ? a.rows - r0 : U);

  // the rows first
  uint4 in0[U], in1[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= nr) break;
    const int64_t off = (r0 + u) * (int64_t)a.cols + c8;
    in0[u] = ld16s(a.a + off);
    if constexpr (OP == 1) in1[u] = ld16s(a.b + off);
  }

  int64_t cur_b = -1;
  float m0[8], m1[8];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= nr) break;
    const int64_t r = r0 + u;
    const int64_t b = r / a.rows_per_batch;
    if (b != cur_b) {  // the first row, and batch boundaries
      cur_b = b;
      const int64_t mo = b * a.mod_stride + c8;
      widen8<DT>(ld16(a.m0 + mo), m0);
      if constexpr (OP == 0) {
        widen8<DT>(ld16(a.m1 + mo), m1);
#pragma unroll
        for (int e = 0; e < 8; ++e) m0[e] = 1.0f + m0[e];
        round8<DT>(m0);  // s1 = rnd(1 + scale)
      }
    }
    float v[8], w[8], o[8];
    widen8<DT>(in0[u], v);
    if constexpr (OP == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = v[e] * m0[e];
      round8<DT>(w);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = w[e] + m1[e];
    } else {
      float res[8];
      widen8<DT>(in1[u], res);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = m0[e] * v[e];
      round8<DT>(w);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = res[e] + w[e];
    }
    st16s(a.out + r * (int64_t)a.cols + c8, narrow8<DT>(o));
  }
}

template <int U>
hipError_t launch_elementwise_u(const ElementwiseArgs &a, int op, int dtype, hipStream_t stream) {
  const int64_t nvec = a.cols >> 3;
  const int64_t threads = nvec * ((a.rows + U - 1) / U);
  if (threads > (int64_t)INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((threads + EW_BLOCK - 1) / EW_BLOCK)), block(EW_BLOCK);
  if (op == 0 && dtype == 0) hipLaunchKernelGGL((elementwise_kernel<0, 0, U>), grid, block, 0, stream, a);
  if (op == 0 && dtype == 1) hipLaunchKernelGGL((elementwise_kernel<0, 1, U>), grid, block, 0, stream, a);
  if (op == 1 && dtype == 0) hipLaunchKernelGGL((elementwise_kernel<1, 0, U>), grid, block, 0, stream, a);
  if (op == 1 && dtype == 1) hipLaunchKernelGGL((elementwise_kernel<1, 1, U>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_elementwise(const ElementwiseArgs &a, int op, int dtype, hipStream_t stream) {
  return launch_elementwise_u<EW_ROWS>(a, op, dtype, stream);
}

}  // namespace ditnorm
