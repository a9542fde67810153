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
// rnd rounds to the storage type (bf16 or fp16) nearest-even.  bf16: each
// operation is one binary32 operation on exactly widened operands, rounded.
// fp16: each operation is one packed fp16 instruction on a pair of values
// (v_pk_mul_f16 / v_pk_add_f16, IEEE nearest-even with subnormals kept):
// a binary32 intermediate has at least 2p+2 significand bits for p = 11, so
// the binary32 operation rounded to fp16 and the direct fp16 operation give
// the same bits, and the packed form takes one instruction per two values
// where the widened chain took about ten.
//
// Work layout: thread t owns the 16-byte column slot t % (cols/8) of U
// consecutive rows, so its modulation vector (already rounded 1 + scale, and
// shift; or the gate) is loaded once and reused; consecutive threads touch
// consecutive 16-byte vectors of a row, and each of the U row accesses is a
// separate fully coalesced instruction.  One-shot grid.
//
// U is chosen per launch so that every wavefront is resident at once and the
// busiest SIMD carries as few row vectors as the launch allows: a launch
// lasts as long as its busiest SIMD.  4608 x 3072 at U = 2 puts 14
// wavefronts (28 vectors per lane) on some SIMDs and streams in rounds; at
// U = 9 it is 3 wavefronts of 9 rows on every SIMD (27, the minimum).
// Measured on 4096 x 3072: U = 8 (3 wavefronts per SIMD) 9.65 us, U = 4 (6)
// 11.13 us, U = 2 10.91 us, against 9.98 us for a plain copy of the bytes;
// 4608 x 3072 at U = 9 11.10 us against 11.92 at U = 2.  Launches too large
// for that (more than 12 rows per thread) keep U = 2.  The fp16 forms, in
// packed fp16 arithmetic, take the same choice: 4608 x 3072 modulate 11.77
// (U = 2, widened chain) -> 10.14 us, gate add 16.11 -> 15.41 us.  The bf16
// gate add, with two input rows per vector, measured 6-10% slower with it
// (17.12 us against 15.57) and keeps U = 2.
#include <atomic>
#include <utility>

#include "device_common.hpp"
#include "launch.hpp"

namespace ditnorm {

constexpr int EW_BLOCK = 256;
constexpr int EW_MAX_ROWS = 12;  // rows per thread, at most
constexpr int EW_MAX_WAVES = 4;  // resident wavefronts per SIMD the choice may use

// OP 0: modulate (x, scale, shift); OP 1: gate add (update, residual, gate)
template <int OP, int DT, int U>
__global__ __launch_bounds__(EW_BLOCK) void elementwise_kernel(const ElementwiseArgs a) {
  // Index arithmetic in 32 bits (the call's limits: rows < 2^25, cols <=
  // 16384, under 2^31 threads) and the batch of each row found by stepping
  // from the first row's: one division per thread instead of a 64-bit
  // division per row, which had been a third of the instructions.
  const uint32_t nvec = (uint32_t)a.cols >> 3;
  const uint32_t t = blockIdx.x * EW_BLOCK + threadIdx.x;
  const uint32_t rg = t / nvec;
  const int c8 = (int)(t - rg * nvec) * 8;
  const uint64_t r0w = (uint64_t)rg * U;
  if (r0w >= (uint64_t)a.rows) return;
  const uint32_t r0 = (uint32_t)r0w;
  const int nr = (int)((uint32_t)a.rows - r0 < (uint32_t)U ? (uint32_t)a.rows - r0 : U);
  const uint32_t rpb = (uint32_t)a.rows_per_batch;
  const int64_t base = (int64_t)r0 * a.cols + c8;  // element offset of row r0

  // the rows first
  uint4 in0[U], in1[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= nr) continue;  // (continue, not break: the loops stay fully unrolled)
    const int64_t off = base + (int64_t)u * a.cols;
    in0[u] = ld16s(a.a + off);
    if constexpr (OP == 1) in1[u] = ld16s(a.b + off);
  }

  // batch b of the current row; rows from `next` on belong to batch b + 1
  uint32_t b = r0 / rpb;
  uint32_t next = (b + 1) * rpb;

  if constexpr (DT == 1) {
    // fp16: each eager op is one packed fp16 operation on a pair (IEEE
    // nearest-even, subnormals kept): the binary32 operation rounded to fp16
    // gives the same bits, since binary32 holds 2 * 11 + 2 significand bits
    f16x2 h0[4], h1[4];
    auto load_mod = [&]() {
      const int64_t mo = (int64_t)b * a.mod_stride + c8;
      as_f16x2(ld16(a.m0 + mo), h0);
      if constexpr (OP == 0) {
        as_f16x2(ld16(a.m1 + mo), h1);
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) h0[i] = one + h0[i];  // s1 = rnd(1 + scale)
      }
    };
    load_mod();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u >= nr) continue;
      if (u > 0 && r0 + u >= next) {  // a batch boundary
        ++b;
        next += rpb;
        load_mod();
      }
      f16x2 v[4], o[4];
      as_f16x2(in0[u], v);
      if constexpr (OP == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f16x2 w = v[i] * h0[i];  // rnd(x * s1)
          o[i] = w + h1[i];              // rnd(. + shift)
        }
      } else {
        f16x2 res[4];
        as_f16x2(in1[u], res);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f16x2 w = h0[i] * v[i];  // rnd(gate * update)
          o[i] = res[i] + w;             // rnd(residual + .)
        }
      }
      st16s(a.out + base + (int64_t)u * a.cols, from_f16x2(o));
    }
    return;
  }

  float m0[8], m1[8];
  auto load_mod = [&]() {
    const int64_t mo = (int64_t)b * a.mod_stride + c8;
    widen8<DT>(ld16(a.m0 + mo), m0);
    if constexpr (OP == 0) {
      widen8<DT>(ld16(a.m1 + mo), m1);
#pragma unroll
      for (int e = 0; e < 8; ++e) m0[e] = 1.0f + m0[e];
      round8<DT>(m0);  // s1 = rnd(1 + scale)
    }
  };
  load_mod();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= nr) continue;
    if (u > 0 && r0 + u >= next) {  // a batch boundary
      ++b;
      next += rpb;
      load_mod();
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
    st16s(a.out + base + (int64_t)u * a.cols, narrow8<DT>(o));
  }
}

template <int OP, int DT, int U>
static hipError_t launch_u(const ElementwiseArgs &a, hipStream_t stream) {
  const int64_t nvec = a.cols >> 3;
  const int64_t threads = nvec * ((a.rows + U - 1) / U);
  if (threads > (int64_t)INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((threads + EW_BLOCK - 1) / EW_BLOCK)), block(EW_BLOCK);
  hipLaunchKernelGGL((elementwise_kernel<OP, DT, U>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// Workgroups of an instantiation resident per compute unit (= its
// wavefronts per SIMD: a workgroup is 4 wavefronts on 4 SIMDs), cached per
// process.
template <int OP, int DT, int U>
static int resident_u() {
  static std::atomic<int> cache;
  int r = cache.load(std::memory_order_relaxed);
  if (r > 0) return r;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &r, (const void *)elementwise_kernel<OP, DT, U>, EW_BLOCK, 0) != hipSuccess ||
      r < 1)
    r = 1;
  cache.store(r, std::memory_order_relaxed);
  return r;
}

template <int OP, int DT, int... Us>
static int resident(int u, std::integer_sequence<int, Us...>) {
  int r = 1;
  ((u == Us + 1 ? (r = resident_u<OP, DT, Us + 1>(), 0) : 0), ...);
  return r;
}

// Rows per thread: every wavefront resident at once (at most EW_MAX_WAVES
// per SIMD, and no more than the instantiation's registers allow) and the
// fewest row vectors on the busiest SIMD; of equal choices the larger U
// (fewer wavefronts).  0 if no U fits.
template <int OP, int DT>
static int rows_per_thread(int64_t rows, int64_t nvec, int num_cu) {
  const int64_t simds = 4LL * num_cu;
  int best = 0;
  int64_t best_cost = 0;
  for (int u = 1; u <= EW_MAX_ROWS; ++u) {
    const int64_t waves = ((rows + u - 1) / u * nvec + 63) / 64;
    const int64_t per_simd = (waves + simds - 1) / simds;
    if (per_simd > EW_MAX_WAVES ||
        per_simd > resident<OP, DT>(u, std::make_integer_sequence<int, EW_MAX_ROWS>{}))
      continue;
    const int64_t cost = per_simd * u;
    if (best == 0 || cost <= best_cost) {
      best = u;
      best_cost = cost;
    }
  }
  return best;
}

template <int OP, int DT, int... Us>
static hipError_t launch_rows(int u, const ElementwiseArgs &a, hipStream_t stream,
                              std::integer_sequence<int, Us...>) {
  hipError_t e = hipErrorInvalidValue;
  ((u == Us + 1 ? (e = launch_u<OP, DT, Us + 1>(a, stream), 0) : 0), ...);
  return e;
}

template <int OP, int DT>
static hipError_t launch_balanced(const ElementwiseArgs &a, const DeviceInfo &dev,
                                  hipStream_t stream) {
  const int u = rows_per_thread<OP, DT>(a.rows, a.cols >> 3, dev.num_cu);
  if (u == 0) return launch_u<OP, DT, 2>(a, stream);  // streams in rounds
  return launch_rows<OP, DT>(u, a, stream, std::make_integer_sequence<int, EW_MAX_ROWS>{});
}

// The bf16 gate add keeps two rows per thread (the balanced choice measured
// 6-10% slower for it); the modulate in both types and the fp16 gate add
// take the balanced choice.
hipError_t launch_elementwise(const ElementwiseArgs &a, int op, int dtype, const DeviceInfo &dev,
                              hipStream_t stream) {
  if (op == 1) {
    if (dtype == 0) return launch_u<1, 0, 2>(a, stream);
    return launch_balanced<1, 1>(a, dev, stream);
  }
  if (dtype == 1) return launch_balanced<0, 1>(a, dev, stream);
  return launch_balanced<0, 0>(a, dev, stream);
}

}  // namespace ditnorm
